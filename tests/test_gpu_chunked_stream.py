"""The device chunk driver with its weight gradients on a second stream
(`dw_stream` in the descriptor) against the same driver on one stream: the
same kernels run on the same chunks and dW accumulates in the same chunk
order, so Y, dX, dW and db must match bit for bit.  Chunk sizes of 1-3
frames exercise the reuse of the two N tables (chunk c + 2 rebuilds the
table chunk c's dW reads); empty frames and K = 5 are covered too.  The
one-stream driver itself is checked against the oracle in
test_gpu_configs."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_convolution_pruned_amd import ops, workloads as wl
from tests.gpu_util import assert_close, dev, host

pytestmark = pytest.mark.gpu

ALL = ops.SV_PASS_FWD | ops.SV_PASS_DX | ops.SV_PASS_DW


def run(L, chunk_frames, passes, dw_stream, dt=torch.bfloat16, kernel="auto", ksize=3, host_offsets=True):
    n, Ci, Co = L.n, L.X.shape[1], L.Wt.shape[2]
    Wt, b = dev(L.Wt, dt), dev(L.b, dt)
    coords, offs = dev(L.coords), dev(L.frame_offsets)
    X, dY = dev(L.X, dt), dev(L.dY, dt)
    Y = torch.zeros((n, Co), dtype=dt, device="cuda")
    dX = torch.zeros((n, Ci), dtype=dt, device="cuda")
    dW = torch.full((ksize * ksize, Ci, Co), 7.0, dtype=torch.float32, device="cuda")
    db = torch.full((Co,), 7.0, dtype=torch.float32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    offs_h = torch.from_numpy(L.frame_offsets.copy()) if host_offsets else None
    d = ops.make_chunked_desc(L.T, L.H, L.W, coords, offs, offs_h, Ci, Co, dt, chunk_frames, X=X, Wt=Wt,
                              bias=b, Y=Y, dY=dY, dX=dX, dW=dW, db=db, err_flag=flag, kernel=kernel,
                              ksize=ksize, dw_stream=dw_stream)
    ws = torch.empty(max(256, ops.sv_chunked_workspace_bytes(d, passes)), dtype=torch.uint8, device="cuda")
    ops.sv_sparseconv2d_chunked(d, passes, ws)
    # the call's stream alone orders the results: no wait on dw_stream here
    out = [t.cpu() for t in (Y, dX, dW, db)]
    assert int(flag.item()) == 0
    return out


def check(L, chunk_frames, passes=ALL, **kw):
    print(f"n={L.n} T={L.T} chunk_frames={chunk_frames} passes={passes} {kw}", flush=True)
    side = torch.cuda.Stream()
    a = run(L, chunk_frames, passes, None, **kw)
    b = run(L, chunk_frames, passes, side, **kw)
    for name, u, v in zip(("Y", "dX", "dW", "db"), a, b):
        assert torch.equal(u, v), f"{name} differs with the dW stream"


def test_c4_dw_stream():
    check(wl.make_layer("c4"), 256)


@pytest.mark.parametrize("chunk_frames", [1, 2, 3])
def test_small_chunks_and_empty_frames(chunk_frames):
    L = wl.make_random_case(81, 7, 16, 16, [90, 0, 130, 256, 0, 40, 200], 128, 128, "bf16")
    check(L, chunk_frames)


@pytest.mark.parametrize("passes", [ops.SV_PASS_FWD | ops.SV_PASS_DW, ops.SV_PASS_DX | ops.SV_PASS_DW,
                                    ops.SV_PASS_DW])
def test_pass_subsets(passes):
    L = wl.make_random_case(82, 5, 14, 14, 0.5, 128, 256, "bf16")
    check(L, 2, passes)


def test_kxk_and_valu():
    L = wl.make_random_case(83, 6, 16, 16, 0.4, 128, 128, "bf16", ksize=5)
    check(L, 2, ksize=5)
    L = wl.make_random_case(84, 6, 14, 14, 0.5, 48, 40, "f32")
    check(L, 2, dt=torch.float32)


@pytest.mark.parametrize("dw_side", [False, True])
def test_without_host_offsets(dw_side):
    """No host copy of the frame offsets: the workspace is sized for full
    frames and the call reads the offsets from the device itself; the
    results equal the call with the host copy bit for bit."""
    L = wl.make_random_case(83, 9, 14, 14, [30, 0, 196, 80, 5, 0, 150, 99, 61], 256, 256, "bf16")
    print(f"n={L.n} dw_side={dw_side}", flush=True)
    side = torch.cuda.Stream() if dw_side else None
    a = run(L, 2, ALL, side)
    b = run(L, 2, ALL, side, host_offsets=False)
    for name, u, v in zip(("Y", "dX", "dW", "db"), a, b):
        assert torch.equal(u, v), f"{name} differs without the host offsets"


@pytest.mark.parametrize("Ci,Co,ksize", [(128, 256, 3), (256, 128, 3), (512, 512, 1)])
def test_paired_fragment_launch(Ci, Co, ksize):
    """Chunks whose forward and input gradient both fit the fragment kernel
    run them as one paired launch: Y and dX equal the unchunked calls bit for
    bit (same summation order whatever the tile shape) and the oracle."""
    L = wl.make_random_case(85, 6, 14, 14, [150, 0, 196, 33, 120, 90], Ci, Co, "bf16", ksize=ksize)
    print(f"n={L.n} Ci={Ci} Co={Co} K={ksize}", flush=True)
    Y, dX, _, _ = run(L, 2, ALL, torch.cuda.Stream(), ksize=ksize)
    _, N, _ = O.build_index(L.coords, L.frame_offsets, L.T, L.H, L.W, K=ksize)
    dt = torch.bfloat16
    X, Wt, b, dY, Nd = dev(L.X, dt), dev(L.Wt, dt), dev(L.b, dt), dev(L.dY, dt), dev(N)
    Y1 = torch.empty((L.n, Co), dtype=dt, device="cuda")
    dX1 = torch.empty((L.n, Ci), dtype=dt, device="cuda")
    ops.sv_sparseconv2d_fwd_k(X, Nd, Wt, b, Y1, "mfma")
    ops.sv_sparseconv2d_bwd_dx_k(dY, Nd, Wt, dX1, "mfma")
    torch.cuda.synchronize()
    assert torch.equal(Y, Y1.cpu()), "Y differs from the unchunked call"
    assert torch.equal(dX, dX1.cpu()), "dX differs from the unchunked call"
    assert_close(host(Y1), O.fwd(L.X, N, L.Wt, L.b), "bf16", "paired Y")
    assert_close(host(dX1), O.bwd_dx(L.dY, N, L.Wt), "bf16", "paired dX")
