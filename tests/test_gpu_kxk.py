"""K x K neighbourhoods (K = 1, 5, 7; 3 through the K entry points) against
the oracle: the index table bit for bit, forward / input gradient / weight
and bias gradients in fp32 (VALU) and bf16 (VALU and MFMA, window and gather
staging, 32-channel tails, padded dW unit groups), the chunk driver with a
K x K descriptor, a full-size layer on sampled rows, and the 3 x 3 calls
bitwise equal to their K = 3 forms."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_convolution_pruned_amd import ops, workloads as wl
from tests.gpu_util import assert_close, dev, host, sample_rows, tdtype

pytestmark = pytest.mark.gpu


def gpu_passes(L, N, kernel, K):
    dt = tdtype(L.dtype)
    X, Wt, b, dY = dev(L.X, dt), dev(L.Wt, dt), dev(L.b, dt), dev(L.dY, dt)
    Nd = dev(N)
    n, Ci, Co = L.n, L.Wt.shape[1], L.Wt.shape[2]
    Y = torch.empty((n, Co), dtype=dt, device="cuda")
    dX = torch.empty((n, Ci), dtype=dt, device="cuda")
    dW = torch.empty((K * K, Ci, Co), dtype=torch.float32, device="cuda")
    db = torch.empty((Co,), dtype=torch.float32, device="cuda")
    ops.sv_sparseconv2d_fwd_k(X, Nd, Wt, b, Y, kernel)
    ops.sv_sparseconv2d_bwd_dx_k(dY, Nd, Wt, dX, kernel)
    ops.sv_sparseconv2d_bwd_dw_k(X, Nd, dY, dW, db)
    torch.cuda.synchronize()
    return host(Y), host(dX), host(dW), host(db)


def check(L, K, kernel, what):
    st, N, _ = O.build_index(L.coords, L.frame_offsets, L.T, L.H, L.W, K=K)
    assert st == 0 and N.shape == (L.n, K * K)
    Y, dX, dW, db = gpu_passes(L, N, kernel, K)
    assert_close(Y, O.fwd(L.X, N, L.Wt, L.b), L.dtype, f"{what} Y")
    assert_close(dX, O.bwd_dx(L.dY, N, L.Wt), L.dtype, f"{what} dX")
    assert_close(dW, O.bwd_dw(L.X, N, L.dY), L.dtype, f"{what} dW")
    assert_close(db, O.bwd_db(L.dY), L.dtype, f"{what} db")


@pytest.mark.parametrize("K", [1, 3, 5, 7])
@pytest.mark.parametrize("shuffle", [False, True])
def test_index_kxk(K, shuffle):
    L = wl.make_random_case(50 + K, 4, 9, 13, [0, 117, 40, 60], 4, 4, "f32", shuffle=shuffle, ksize=K)
    print(f"index K={K} shuffle={shuffle} n={L.n}", flush=True)
    st, Nr, Mr = O.build_index(L.coords, L.frame_offsets, L.T, L.H, L.W, want_map=True, K=K)
    N, M = ops.build_index(dev(L.coords), dev(L.frame_offsets), L.T, L.H, L.W, with_map=True, K=K)
    assert np.array_equal(host(N), Nr), f"N differs at K={K}"
    assert np.array_equal(host(M).reshape(Mr.shape), Mr), f"M differs at K={K}"


# (seed, T, H, W, keep, Ci, Co, shuffle)
F32_CASES = [
    (31, 2, 9, 11, 0.6, 17, 33, False),
    (32, 3, 12, 12, [0, 144, 40], 8, 65, True),
]


@pytest.mark.parametrize("K", [1, 5, 7])
@pytest.mark.parametrize("case", F32_CASES, ids=lambda c: f"seed{c[0]}")
def test_f32_valu_kxk(case, K):
    seed, T, H, W, keep, Ci, Co, sh = case
    L = wl.make_random_case(seed, T, H, W, keep, Ci, Co, "f32", shuffle=sh, ksize=K)
    print(f"f32 K={K} case {case} n={L.n}", flush=True)
    check(L, K, "valu", f"f32 K={K} {case}")


BF16_CASES = [
    (41, 3, 14, 14, 0.4, 128, 128, False),            # MFMA dW: one padded unit group per tile
    (42, 2, 16, 16, 0.6, 96, 64, True),               # shuffled packing: gather staging
    (43, 4, 14, 14, [0, 1, 196, 60], 256, 128, False),
    (44, 2, 14, 14, 0.5, 160, 64, False),             # 32-channel tail chunk
]


@pytest.mark.parametrize("kernel", ["valu", "mfma"])
@pytest.mark.parametrize("K", [1, 5, 7])
@pytest.mark.parametrize("case", BF16_CASES, ids=lambda c: f"seed{c[0]}")
def test_bf16_kxk(case, K, kernel):
    seed, T, H, W, keep, Ci, Co, sh = case
    L = wl.make_random_case(seed, T, H, W, keep, Ci, Co, "bf16", shuffle=sh, ksize=K)
    print(f"bf16 K={K} {kernel} case {case} n={L.n}", flush=True)
    check(L, K, kernel, f"bf16 K={K} {kernel} {case}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_k3_entry_points_identical(dt):
    """The 3 x 3 calls and their K = 3 forms give the same bits."""
    L = wl.make_random_case(45, 3, 14, 14, 0.5, 128, 128, dt)
    t = tdtype(dt)
    st, N, _ = O.build_index(L.coords, L.frame_offsets, L.T, L.H, L.W)
    X, Wt, b, dY, Nd = dev(L.X, t), dev(L.Wt, t), dev(L.b, t), dev(L.dY, t), dev(N)
    n = L.n
    outs = []
    for k_form in (False, True):
        Nb = torch.empty((n, 9), dtype=torch.int32, device="cuda")
        Y = torch.empty((n, 128), dtype=t, device="cuda")
        dX = torch.empty_like(Y)
        dW = torch.empty((9, 128, 128), dtype=torch.float32, device="cuda")
        db = torch.empty((128,), dtype=torch.float32, device="cuda")
        c, o = dev(L.coords), dev(L.frame_offsets)
        if k_form:
            ops.sv_build_index_k(c, o, L.T, L.H, L.W, 3, Nb)
            ops.sv_sparseconv2d_fwd_k(X, Nd, Wt, b, Y)
            ops.sv_sparseconv2d_bwd_dx_k(dY, Nd, Wt, dX)
            ops.sv_sparseconv2d_bwd_dw_k(X, Nd, dY, dW, db)
        else:
            ops.sv_build_index(c, o, L.T, L.H, L.W, Nb)
            ops.sv_sparseconv2d_fwd(X, Nd, Wt, b, Y)
            ops.sv_sparseconv2d_bwd_dx(dY, Nd, Wt, dX)
            ops.sv_sparseconv2d_bwd_dw(X, Nd, dY, dW, db)
        torch.cuda.synchronize()
        outs.append((Nb, Y, dX, dW, db))
    for a, c in zip(*outs):
        assert torch.equal(a, c)
    assert np.array_equal(host(outs[0][0]), N)


@pytest.mark.parametrize("K", [1, 5])
def test_chunked_kxk(K):
    """The chunk driver with a K x K descriptor: Y and dX equal the
    unchunked calls bit for bit; dW and db match the oracle."""
    L = wl.make_random_case(46 + K, 5, 14, 14, [60, 0, 120, 7, 196], 128, 128, "bf16", ksize=K)
    print(f"chunked K={K} n={L.n}", flush=True)
    t = torch.bfloat16
    coords, offs = dev(L.coords), dev(L.frame_offsets)
    X, Wt, b, dY = dev(L.X, t), dev(L.Wt, t), dev(L.b, t), dev(L.dY, t)
    n = L.n
    Y = torch.empty((n, 128), dtype=t, device="cuda")
    dX = torch.empty_like(Y)
    dW = torch.empty((K * K, 128, 128), dtype=torch.float32, device="cuda")
    db = torch.empty((128,), dtype=torch.float32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    d = ops.make_chunked_desc(L.T, L.H, L.W, coords, offs, torch.from_numpy(L.frame_offsets.copy()), 128, 128, t,
                              2, X=X, Wt=Wt, bias=b, Y=Y, dY=dY, dX=dX, dW=dW, db=db, err_flag=flag, ksize=K)
    passes = ops.SV_PASS_FWD | ops.SV_PASS_DX | ops.SV_PASS_DW
    ws = torch.empty(max(256, ops.sv_chunked_workspace_bytes(d, passes)), dtype=torch.uint8, device="cuda")
    ops.sv_sparseconv2d_chunked(d, passes, ws)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    N = ops.build_index(coords, offs, L.T, L.H, L.W, K=K)
    assert torch.equal(Y, ops.sparseconv2d_fwd(X, N, Wt, b))
    assert torch.equal(dX, ops.sparseconv2d_bwd_dx(dY, N, Wt))
    st, Nr, _ = O.build_index(L.coords, L.frame_offsets, L.T, L.H, L.W, K=K)
    assert np.array_equal(host(N), Nr)
    assert_close(host(dW), O.bwd_dw(L.X, Nr, L.dY), "bf16", f"chunked K={K} dW")
    assert_close(host(db), O.bwd_db(L.dY), "bf16", f"chunked K={K} db")


@pytest.mark.parametrize("K", [1, 5])
def test_full_size_layer_kxk(K):
    """The c3a layer (C = 256, 14 x 14 grid, 59 tokens per frame) with K x K
    weights of the same distribution, on the launch path the benchmark uses,
    against the oracle on sampled rows."""
    L = wl.make_layer("c3a")
    C, taps = L.Wt.shape[1], K * K
    rng = np.random.default_rng(900 + K)
    Wk = wl.round_bf16(rng.standard_normal((taps, C, C)).astype(np.float32) / np.sqrt(taps * C))
    print(f"full-size K={K} n={L.n} C={C}", flush=True)
    t = torch.bfloat16
    coords, offs = dev(L.coords), dev(L.frame_offsets)
    N = ops.build_index(coords, offs, L.T, L.H, L.W, K=K)
    X, Wt, b, dY = dev(L.X, t), dev(Wk, t), dev(L.b, t), dev(L.dY, t)
    Y = ops.sparseconv2d_fwd(X, N, Wt, b)
    dX = ops.sparseconv2d_bwd_dx(dY, N, Wt)
    dW, db = ops.sparseconv2d_bwd_dw(X, N, dY)
    torch.cuda.synchronize()
    st, Nr, _ = O.build_index(L.coords, L.frame_offsets, L.T, L.H, L.W, K=K)
    assert np.array_equal(host(N), Nr)
    rows = sample_rows(L.n, 256, seed=K)
    assert_close(host(Y)[rows], O.fwd_rows(L.X, Nr, Wk, L.b, rows), "bf16", f"K={K} Y")
    assert_close(host(dX)[rows], O.bwd_dx_rows(L.dY, Nr, Wk, rows), "bf16", f"K={K} dX")
    ji = np.unique(np.concatenate([[0, C - 1, taps * C - 1, (taps // 2) * C],
                                   rng.choice(taps * C, size=24, replace=False)])).astype(np.int64)
    assert_close(host(dW).reshape(taps * C, -1)[ji], O.bwd_dw_rows(L.X, Nr, L.dY, ji), "bf16", f"K={K} dW")
    assert_close(host(db), O.bwd_db(L.dY), "bf16", f"K={K} db")


@pytest.mark.parametrize("K", [3, 5])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_split_forms_equal_single_calls(dt, K):
    """Repacked weights then the packed forward equal the forward call; the
    dW partials then their reduction (on a second stream) equal the dW call:
    bit for bit."""
    L = wl.make_random_case(70 + K, 3, 14, 14, 0.5, 128, 128, dt, ksize=K)
    t = tdtype(dt)
    st, N, _ = O.build_index(L.coords, L.frame_offsets, L.T, L.H, L.W, K=K)
    X, Wt, b, dY, Nd = dev(L.X, t), dev(L.Wt, t), dev(L.b, t), dev(L.dY, t), dev(N)
    n, taps = L.n, K * K
    dW1 = torch.empty((taps, 128, 128), dtype=torch.float32, device="cuda")
    db1 = torch.empty((128,), dtype=torch.float32, device="cuda")
    ops.sv_sparseconv2d_bwd_dw_k(X, Nd, dY, dW1, db1)
    dW2, db2 = torch.full_like(dW1, 5.0), torch.full_like(db1, 5.0)
    ws = torch.empty(max(256, ops.sv_workspace_bytes_k(ops.SV_OP_DW, n, K, 128, 128, t)), dtype=torch.uint8,
                     device="cuda")
    ops.sv_sparseconv2d_bwd_dw_partials_k(X, Nd, dY, dW2, db2, ws)
    done = torch.cuda.Event()
    done.record()
    other = torch.cuda.Stream()
    other.wait_event(done)
    ops.sv_sparseconv2d_bwd_dw_reduce_k(dW2, db2, n, t, ws, stream=other)
    torch.cuda.current_stream().wait_stream(other)
    torch.cuda.synchronize()
    assert torch.equal(dW1, dW2) and torch.equal(db1, db2)
    if dt == "bf16":
        Y1 = ops.sparseconv2d_fwd(X, Nd, Wt, b)
        V = torch.empty(max(256, ops.sv_workspace_bytes_k(ops.SV_OP_FWD, n, K, 128, 128, t)), dtype=torch.uint8,
                        device="cuda")
        ops.sv_repack_fwd_k(Wt, V)
        Y2 = torch.empty_like(Y1)
        ops.sv_sparseconv2d_fwd_packed_k(X, Nd, V, b, Y2, K)
        torch.cuda.synchronize()
        assert torch.equal(Y1, Y2)
    else:
        V = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
        with pytest.raises(ops.SvError) as e:
            ops.sv_repack_fwd_k(Wt, V)
        assert e.value.status == ops.SV_ERR_UNSUPPORTED
