"""The allocation-free linear forward (convrot_linear_forward_noalloc) against
the workspace forward it shares its kernels with: bit for bit on two calls in
a row, the second with a smaller input (the static scratch keeps the first
call's contents), on both output types, and the host-side rejection of a
shape whose workspace exceeds the scratch."""
import numpy as np
import pytest
import torch

from w8a8_int8_rotated_amd import workloads as wl
from gpu_util import announce, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cr():
    from w8a8_int8_rotated_amd import convrot
    convrot.library()
    return convrot


def _bits(y):
    return y.view(torch.int16 if y.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def test_noalloc_matches_workspace_forward(cr):
    big = wl.WORKLOADS["linear_4096"]                                     # 22 MB of scratch
    small = wl.Workload("s", "linear", M=300, K=1024, N=272, block=64, out="f32",
                        x_dist="student_t4", bias_std=0.5, seed=7)
    for w in (big, small):
        announce(f"no-alloc forward {w.M}x{w.K}x{w.N} b={w.block} out={w.out}")
        pw = cr.convrot_linear_prepare_weights(to_dev(w.weight()), w.block)
        X = to_dev_bf16(w.activations())
        bias = to_dev(w.bias())
        dt = torch.bfloat16 if w.out == "bf16" else torch.float32
        need = cr.convrot_linear_workspace_bytes(w.M, w.K, w.N, w.block)
        assert 0 < need <= 32 << 20
        out = torch.full((w.M, w.N), float("nan"), dtype=dt, device="cuda")
        cr.convrot_linear_forward_noalloc(X, pw, bias=bias, out=out)
        want = cr.convrot_linear_forward(X, pw, bias=bias, out_dtype=dt)
        torch.cuda.synchronize()
        diff = int(np.count_nonzero(_bits(out) != _bits(want)))
        print(f"[parity] no-alloc vs workspace forward: {diff} of {out.numel()} differ",
              flush=True)
        assert diff == 0


def test_noalloc_rejects_beyond_scratch(cr):
    announce("no-alloc forward: shape beyond the static scratch")
    w = wl.scaled("linear_4096", M=16, K=5376, N=512)
    pw = cr.convrot_linear_prepare_weights(to_dev(w.weight()), w.block)
    M = 8192                                          # 44 MB of codes at K = 5376
    assert cr.convrot_linear_workspace_bytes(M, w.K, w.N, w.block) > 32 << 20
    X = torch.zeros((M, w.K), dtype=torch.bfloat16, device="cuda")
    Y = torch.full((M, w.N), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(cr.ConvRotError) as e:
        cr.convrot_linear_forward_noalloc(X, pw, out=Y)
    assert e.value.status == cr.EWORKSPACE
    torch.cuda.synchronize()
    assert bool((Y == 3.0).all())                      # nothing was launched
