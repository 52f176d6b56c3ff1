"""The host-streamed chunk driver (per-token tensors in pinned host memory,
double-buffered through the device on two copy streams) against the device
chunk driver: the same kernels run on the same chunks in the same order, so
Y, dX, dW and db must match bit for bit.  Config 4 is also compared with the
oracle directly, every element."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_convolution_pruned_amd import ops, workloads as wl
from tests.gpu_util import assert_close, dev, host

pytestmark = pytest.mark.gpu

ALL = ops.SV_PASS_FWD | ops.SV_PASS_DX | ops.SV_PASS_DW


def pinned(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.pin_memory()


def run_both(L, chunk_frames, passes, dt=torch.bfloat16, kernel="auto", ksize=3):
    n, Ci, Co = L.n, L.X.shape[1], L.Wt.shape[2]
    Wt, b = dev(L.Wt, dt), dev(L.b, dt)
    # device driver
    coords, offs = dev(L.coords), dev(L.frame_offsets)
    X, dY = dev(L.X, dt), dev(L.dY, dt)
    Y = torch.zeros((n, Co), dtype=dt, device="cuda")
    dX = torch.zeros((n, Ci), dtype=dt, device="cuda")
    dW = torch.zeros((ksize * ksize, Ci, Co), dtype=torch.float32, device="cuda")
    db = torch.zeros((Co,), dtype=torch.float32, device="cuda")
    offs_h = torch.from_numpy(L.frame_offsets.copy())
    d = ops.make_chunked_desc(L.T, L.H, L.W, coords, offs, offs_h, Ci, Co, dt, chunk_frames, X=X, Wt=Wt,
                              bias=b, Y=Y, dY=dY, dX=dX, dW=dW, db=db, kernel=kernel, ksize=ksize)
    ws = torch.empty(max(256, ops.sv_chunked_workspace_bytes(d, passes)), dtype=torch.uint8, device="cuda")
    ops.sv_sparseconv2d_chunked(d, passes, ws)
    # host-streamed driver
    Xh, dYh = pinned(L.X, dt), pinned(L.dY, dt)
    Yh = torch.zeros((n, Co), dtype=dt).pin_memory()
    dXh = torch.zeros((n, Ci), dtype=dt).pin_memory()
    dW2 = torch.zeros_like(dW)
    db2 = torch.zeros_like(db)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    hd = ops.make_chunked_host_desc(L.T, L.H, L.W, pinned(L.coords), pinned(L.frame_offsets), Ci, Co, dt,
                                    chunk_frames, X_host=Xh, Wt=Wt, bias=b, Y_host=Yh, dY_host=dYh,
                                    dX_host=dXh, dW=dW2, db=db2, err_flag=flag, kernel=kernel, ksize=ksize)
    hwsb = ops.sv_chunked_host_workspace_bytes(hd, passes)
    assert hwsb >= ops.sv_chunked_workspace_bytes(d, passes)
    hws = torch.empty(max(256, hwsb), dtype=torch.uint8, device="cuda")
    s_h2d, s_d2h = torch.cuda.Stream(), torch.cuda.Stream()
    ops.sv_sparseconv2d_chunked_host(hd, passes, hws, s_h2d, s_d2h)
    torch.cuda.current_stream().synchronize()      # covers the copies as well
    assert int(flag.item()) == 0
    return (Y, dX, dW, db), (Yh, dXh, dW2, db2)


def same(a, b):
    return torch.equal(a.cpu(), b.cpu())


def test_c4_host_streamed():
    """Config 4 (6144 frames as T=3072, chunks of 256) streamed from pinned
    host memory; the workspace stays the same at a tenth of the length."""
    L = wl.make_layer("c4")
    print("c4 host-streamed, n =", L.n, flush=True)
    (Y, dX, dW, db), (Yh, dXh, dW2, db2) = run_both(L, 256, ALL)
    assert same(Y, Yh) and same(dX, dXh)
    assert same(dW, dW2) and same(db, db2)
    _, Nr, _ = O.build_index(L.coords, L.frame_offsets, L.T, L.H, L.W)
    assert_close(host(Yh), O.fwd(L.X, Nr, L.Wt, L.b), "bf16", "c4 host-streamed Y")
    assert_close(host(dXh), O.bwd_dx(L.dY, Nr, L.Wt), "bf16", "c4 host-streamed dX")
    assert_close(host(dW2), O.bwd_dw(L.X, Nr, L.dY), "bf16", "c4 host-streamed dW")
    assert_close(host(db2), O.bwd_db(L.dY), "bf16", "c4 host-streamed db")
    Ls = wl.make_layer("c4", scale_T=256)
    C = L.X.shape[1]
    d_full = ops.make_chunked_host_desc(L.T, L.H, L.W, pinned(L.coords), pinned(L.frame_offsets), C, C,
                                        torch.bfloat16, 256)
    d_short = ops.make_chunked_host_desc(256, Ls.H, Ls.W, pinned(Ls.coords), pinned(Ls.frame_offsets), C, C,
                                         torch.bfloat16, 256)
    assert ops.sv_chunked_host_workspace_bytes(d_full, ALL) <= \
        ops.sv_chunked_host_workspace_bytes(d_short, ALL) * 1.25 + (1 << 20)


@pytest.mark.parametrize("passes", [ALL, ops.SV_PASS_FWD, ops.SV_PASS_DW, ops.SV_PASS_DX | ops.SV_PASS_DW])
def test_ragged_chunks_and_empty_frames(passes):
    """10 frames in chunks of 3 (the last chunk holds one frame), some
    frames empty, one chunk with no tokens at all, bf16 on the MFMA kernels."""
    keep = [40, 0, 96, 12, 0, 0, 0, 150, 1, 64]
    L = wl.make_random_case(31, 10, 12, 13, keep, 128, 128, "bf16")
    print("ragged host-streamed case, passes", passes, "n =", L.n, flush=True)
    (Y, dX, dW, db), (Yh, dXh, dW2, db2) = run_both(L, 3, passes)
    if passes & ops.SV_PASS_FWD:
        assert same(Y, Yh)
    if passes & ops.SV_PASS_DX:
        assert same(dX, dXh)
    if passes & ops.SV_PASS_DW:
        assert same(dW, dW2) and same(db, db2)


@pytest.mark.parametrize("ksize", [1, 5])
def test_kxk_descriptor(ksize):
    """A K x K descriptor through both drivers (ragged chunks, an empty frame)."""
    L = wl.make_random_case(33 + ksize, 5, 14, 14, [60, 0, 120, 7, 196], 128, 128, "bf16", ksize=ksize)
    print("host-streamed K =", ksize, "n =", L.n, flush=True)
    (Y, dX, dW, db), (Yh, dXh, dW2, db2) = run_both(L, 2, ALL, ksize=ksize)
    assert same(Y, Yh) and same(dX, dXh) and same(dW, dW2) and same(db, db2)


def test_fp32_valu_kernels():
    """fp32 (VALU kernels) through the host-streamed driver."""
    L = wl.make_random_case(32, 7, 9, 11, 0.6, 48, 40, "f32")
    print("fp32 host-streamed case, n =", L.n, flush=True)
    (Y, dX, dW, db), (Yh, dXh, dW2, db2) = run_both(L, 2, ALL, dt=torch.float32)
    assert same(Y, Yh) and same(dX, dXh) and same(dW, dW2) and same(db, db2)


def test_back_to_back_calls_share_the_workspace():
    """Two calls on one workspace, enqueued without a synchronisation in
    between and with different inputs: the second call's uploads must wait
    for the first call's chunks, so each result equals its own isolated run."""
    dt = torch.bfloat16
    cases = [wl.make_random_case(41 + i, 12, 10, 11, 0.5, 128, 128, "bf16") for i in range(2)]
    refs = [run_both(L, 2, ALL)[0] for L in cases]
    C = 128
    Wts = [dev(L.Wt, dt) for L in cases]
    bs = [dev(L.b, dt) for L in cases]
    outs, descs = [], []
    for L, Wt, b in zip(cases, Wts, bs):
        n = L.n
        o = dict(Y=torch.zeros((n, C), dtype=dt).pin_memory(), dX=torch.zeros((n, C), dtype=dt).pin_memory(),
                 dW=torch.zeros((9, C, C), dtype=torch.float32, device="cuda"),
                 db=torch.zeros((C,), dtype=torch.float32, device="cuda"))
        descs.append(ops.make_chunked_host_desc(L.T, L.H, L.W, pinned(L.coords), pinned(L.frame_offsets), C, C, dt,
                                                2, X_host=pinned(L.X, dt), Wt=Wt, bias=b, Y_host=o["Y"],
                                                dY_host=pinned(L.dY, dt), dX_host=o["dX"], dW=o["dW"], db=o["db"]))
        outs.append(o)
    wsb = max(ops.sv_chunked_host_workspace_bytes(d, ALL) for d in descs)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    s_h2d, s_d2h = torch.cuda.Stream(), torch.cuda.Stream()
    for d in descs:
        ops.sv_sparseconv2d_chunked_host(d, ALL, ws, s_h2d, s_d2h)
    torch.cuda.current_stream().synchronize()
    for o, (Y, dX, dW, db) in zip(outs, refs):
        assert same(o["Y"], Y) and same(o["dX"], dX) and same(o["dW"], dW) and same(o["db"], db)
