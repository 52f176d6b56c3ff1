"""The allocation-free weight-gradient call (partials in the library's
device array) against the workspace call, through the C ABI: bit for bit on
two calls in a row, the second with a smaller input (the array keeps the
first call's contents), and against the oracle."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_convolution_pruned_amd import ops, workloads as wl
from tests.gpu_util import assert_close, dev, host, tdtype

pytestmark = pytest.mark.gpu


def both(L, N, K=3, accumulate=False, seed_dw=None):
    dt = tdtype(L.dtype)
    X, dY, Nd = dev(L.X, dt), dev(L.dY, dt), dev(N)
    taps, Ci, Co = K * K, L.X.shape[1], L.dY.shape[1]
    outs = []
    for noalloc in (False, True):
        dW = torch.zeros((taps, Ci, Co), dtype=torch.float32, device="cuda")
        db = torch.zeros((Co,), dtype=torch.float32, device="cuda")
        if seed_dw is not None:
            dW.copy_(seed_dw[0])
            db.copy_(seed_dw[1])
        if noalloc:
            ops.sv_sparseconv2d_bwd_dw_noalloc_k(X, Nd, dY, dW, db, accumulate)
        else:
            ops.sv_sparseconv2d_bwd_dw_k(X, Nd, dY, dW, db, accumulate)
        outs.append((dW, db))
    torch.cuda.synchronize()
    (dW0, db0), (dW1, db1) = outs
    assert torch.equal(dW0.view(torch.int32), dW1.view(torch.int32)), "dW differs from the workspace call"
    assert torch.equal(db0.view(torch.int32), db1.view(torch.int32)), "db differs from the workspace call"
    return host(dW1), host(db1)


def test_two_calls_second_smaller():
    # first: a c5-sized layer (split-K partials ~38 MB), then a small one
    L1 = wl.make_random_case(61, 160, 16, 16, 0.6, 256, 256, "bf16")
    L2 = wl.make_random_case(62, 7, 16, 16, 0.4, 256, 256, "bf16")
    assert L2.n < L1.n
    for L in (L1, L2):
        print(f"n={L.n} dW workspace {ops.sv_workspace_bytes(ops.SV_OP_DW, L.n, 256, 256, torch.bfloat16)} B",
              flush=True)
        assert 0 < ops.sv_workspace_bytes(ops.SV_OP_DW, L.n, 256, 256, torch.bfloat16) <= ops.SV_NOALLOC_SCRATCH_BYTES
        _, N, _ = O.build_index(L.coords, L.frame_offsets, L.T, L.H, L.W)
        dW, db = both(L, N)
        assert_close(dW, O.bwd_dw(L.X, N, L.dY), "bf16", f"noalloc dW n={L.n}")
        assert_close(db, O.bwd_db(L.dY), "bf16", f"noalloc db n={L.n}")


def test_fp32_kxk_and_accumulate():
    L = wl.make_random_case(63, 3, 9, 11, 0.5, 48, 40, "f32", ksize=5)
    _, N, _ = O.build_index(L.coords, L.frame_offsets, L.T, L.H, L.W, K=5)
    base = (torch.randn(25, 48, 40, device="cuda"), torch.randn(40, device="cuda"))
    dW, db = both(L, N, K=5, accumulate=True, seed_dw=base)
    assert_close(dW - host(base[0]), O.bwd_dw(L.X, N, L.dY), "f32", "noalloc 5x5 accumulated dW")
    assert_close(db - host(base[1]), O.bwd_db(L.dY), "f32", "noalloc accumulated db")


def test_rejects_beyond_the_array():
    # a 5 x 5 layer with 2M tokens: partials of several rounds of slices
    n = 2_000_000
    lib = ops.load()
    need = lib.sv_workspace_bytes_k(ops.SV_OP_DW, n, 5, 512, 512, ops.SV_BF16)
    assert need > ops.SV_NOALLOC_SCRATCH_BYTES
    st = lib.sv_sparseconv2d_bwd_dw_noalloc_k(1 << 12, 1 << 12, 1 << 12, 1 << 12, None, n, 5, 512, 512,
                                              ops.SV_BF16, 0, None)
    assert st == ops.SV_ERR_WORKSPACE
