"""SparseConv2D kernels (fwd, dX, dW, db) against the oracle on small and
ragged cases: fp32 and bf16, VALU and MFMA kernels, the LDS-window and the
gather staging modes of the MFMA kernel, empty inputs, determinism."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_convolution_pruned_amd import ops, workloads as wl
from tests.gpu_util import assert_close, dev, host, tdtype

pytestmark = pytest.mark.gpu


def run_all(L, N, kernel, with_bias=True):
    dt = tdtype(L.dtype)
    X, Wt, dY = dev(L.X, dt), dev(L.Wt, dt), dev(L.dY, dt)
    b = dev(L.b, dt) if with_bias else None
    Nd = dev(N)
    Y = ops.sparseconv2d_fwd(X, Nd, Wt, b, kernel)
    dX = ops.sparseconv2d_bwd_dx(dY, Nd, Wt, kernel)
    dW, db = ops.sparseconv2d_bwd_dw(X, Nd, dY)
    torch.cuda.synchronize()
    return host(Y), host(dX), host(dW), host(db)


def check_against_oracle(L, N, kernel, with_bias=True, what=""):
    Y, dX, dW, db = run_all(L, N, kernel, with_bias)
    b = L.b if with_bias else None
    assert_close(Y, O.fwd(L.X, N, L.Wt, b), L.dtype, f"{what} Y")
    assert_close(dX, O.bwd_dx(L.dY, N, L.Wt), L.dtype, f"{what} dX")
    assert_close(dW, O.bwd_dw(L.X, N, L.dY), L.dtype, f"{what} dW")
    assert_close(db, O.bwd_db(L.dY), L.dtype, f"{what} db")


# (seed, T, H, W, keep, Ci, Co, shuffle)
F32_CASES = [
    (1, 1, 14, 14, 0.5, 64, 64, False),
    (2, 3, 6, 7, 0.4, 1, 1, True),
    (3, 2, 9, 5, 0.8, 3, 17, False),
    (4, 4, 14, 14, [0, 1, 196, 60], 65, 33, True),
    (5, 2, 16, 16, 0.3, 17, 130, False),
    (6, 1, 1, 1, 1.0, 8, 8, False),
]


@pytest.mark.parametrize("case", F32_CASES, ids=lambda c: f"seed{c[0]}")
def test_f32_valu(case):
    seed, T, H, W, keep, Ci, Co, sh = case
    L = wl.make_random_case(seed, T, H, W, keep, Ci, Co, "f32", shuffle=sh)
    print(f"case {case} n={L.n}", flush=True)
    st, N, _ = O.build_index(L.coords, L.frame_offsets, T, H, W)
    check_against_oracle(L, N, "valu", what=f"f32 {case}")


def dev_at(a, dtype, offset):
    """`a` on the GPU, `offset` elements into its storage (contiguous)."""
    src = dev(a, dtype).reshape(-1)
    buf = torch.zeros(src.numel() + offset, dtype=dtype, device="cuda")
    buf[offset:].copy_(src)
    return buf[offset:].view(a.shape)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("offset", [0, 1])
def test_valu_vector_loads(dt, offset):
    # Channel counts multiples of 4 over 128 x 64 tiles with a ragged token
    # tail and a ragged channel tile (at least 192 tiles per pass, so the
    # wide tile kernel runs): four-channel loads when X, dY and the weights
    # are aligned (offset 0), element-wise staging when they are not (offset
    # 1); both against the oracle.
    L = wl.make_random_case(7, 280, 14, 14, 0.45, 48, 80, dt, shuffle=True)
    assert 192 * 128 < L.n < 193 * 128
    _, N, _ = O.build_index(L.coords, L.frame_offsets, L.T, L.H, L.W)
    t = tdtype(dt)
    X, Wt, dY, b = (dev_at(a, t, offset) for a in (L.X, L.Wt, L.dY, L.b))
    assert (X.data_ptr() % 8 == 0) == (offset == 0)
    Nd = dev(N)
    Y = ops.sparseconv2d_fwd(X, Nd, Wt, b, "valu")
    dX = ops.sparseconv2d_bwd_dx(dY, Nd, Wt, "valu")
    torch.cuda.synchronize()
    assert_close(host(Y), O.fwd(L.X, N, L.Wt, L.b), dt, f"Y offset {offset}")
    assert_close(host(dX), O.bwd_dx(L.dY, N, L.Wt), dt, f"dX offset {offset}")


def pad_rows(a, extra):
    return np.concatenate([a, np.zeros((extra,) + a.shape[1:], a.dtype)])


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("taps", [9, 25])
def test_valu_small_and_wide_tiles_agree(dt, taps):
    # Below 192 tiles of 128 tokens x 64 channels the VALU passes run on
    # 16 x 16 tiles.  Both kernels sum each output's terms in the same order,
    # so a problem on the small tiles and the same rows inside a problem on
    # the wide ones (the extra rows referenced by no one, with no neighbours)
    # give the same bits.  The small problem is also checked against the oracle.
    rng = np.random.default_rng(40 + taps)
    n, big, Ci, Co = 300, 24600, 64, 96
    L = wl.make_random_case(41, 1, 40, 40, [n], Ci, Co, dt, ksize=3 if taps == 9 else 5)
    N = rng.integers(-1, n, size=(n, taps)).astype(np.int32)
    assert -(-n // 128) * -(-Co // 64) < 192 <= -(-big // 128) * -(-Ci // 64)
    t = tdtype(dt)
    Nb = np.concatenate([N, np.full((big - n, taps), -1, np.int32)])
    Wd, bd = dev(L.Wt, t), dev(L.b, t)
    Y = ops.sparseconv2d_fwd(dev(L.X, t), dev(N), Wd, bd, "valu")
    dX = ops.sparseconv2d_bwd_dx(dev(L.dY, t), dev(N), Wd, "valu")
    Yb = ops.sparseconv2d_fwd(dev(pad_rows(L.X, big - n), t), dev(Nb), Wd, bd, "valu")
    dXb = ops.sparseconv2d_bwd_dx(dev(pad_rows(L.dY, big - n), t), dev(Nb), Wd, "valu")
    torch.cuda.synchronize()
    assert torch.equal(Y, Yb[:n]) and torch.equal(dX, dXb[:n])
    assert_close(host(Y), O.fwd(L.X, N, L.Wt, L.b), dt, f"small tiles Y taps {taps}")
    assert_close(host(dX), O.bwd_dx(L.dY, N, L.Wt), dt, f"small tiles dX taps {taps}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_valu_dw_small_and_wide_tiles_agree(dt):
    # The VALU weight gradient runs on 16 x 16 tiles up to 64 x 64 channels,
    # and when its 64 x 64 grid would be under 256 workgroups.
    # dW[:, :64, :64] and db[:64] of a 352-channel problem (wide tiles, 324
    # workgroups; not a multiple of 128, so not the matrix-core kernel in
    # bf16) whose first 64 channels are those of a 64-channel problem
    # (small tiles) are the same sums in the same order: the same bits, also
    # when added to existing values.  Under 512 tokens both take one token
    # slice.  The small problem is also checked against the oracle, and a
    # 2,000-token one with three slices.
    rng = np.random.default_rng(43)
    n, C, Cb = 300, 64, 352
    t = tdtype(dt)
    L = wl.make_random_case(44, 1, 40, 40, [n], Cb, Cb, dt)
    N = dev(rng.integers(-1, n, size=(n, 9)).astype(np.int32))
    Xb, dYb = dev(L.X, t), dev(L.dY, t)
    Xs, dYs = Xb[:, :C].contiguous(), dYb[:, :C].contiguous()
    start = torch.from_numpy(rng.standard_normal((9, Cb, Cb)).astype(np.float32)).cuda()
    dbs0 = torch.from_numpy(rng.standard_normal(Cb).astype(np.float32)).cuda()
    outs = []
    for X, dY, Cc in ((Xs, dYs, C), (Xb, dYb, Cb)):
        dW, db = ops.sparseconv2d_bwd_dw(X, N, dY)
        dWa = start[:, :Cc, :Cc].clone(memory_format=torch.contiguous_format)    # never `start` itself
        dba = dbs0[:Cc].clone()
        ops.sv_sparseconv2d_bwd_dw(X, N, dY, dWa, dba, accumulate=True)
        outs.append((dW, db, dWa, dba))
    torch.cuda.synchronize()
    (dW, db, dWa, dba), (dWb, dbb, dWab, dbab) = outs
    assert torch.equal(dW, dWb[:, :C, :C]) and torch.equal(db, dbb[:C])
    assert torch.equal(dWa, dWab[:, :C, :C]) and torch.equal(dba, dbab[:C])
    Xh, dYh, Nh = host(Xs), host(dYs), host(N)
    assert_close(host(dW), O.bwd_dw(Xh, Nh, dYh), dt, "small-tile dW")
    assert_close(host(db), O.bwd_db(dYh), dt, "small-tile db")
    assert_close(host(dWa), host(start[:, :C, :C]) + O.bwd_dw(Xh, Nh, dYh), dt, "small-tile dW accumulated")
    L2 = wl.make_random_case(45, 1, 50, 50, [2000], C, C, dt)
    _, N2, _ = O.build_index(L2.coords, L2.frame_offsets, 1, 50, 50)
    dW2, db2 = ops.sparseconv2d_bwd_dw(dev(L2.X, t), dev(N2), dev(L2.dY, t))
    torch.cuda.synchronize()
    assert_close(host(dW2), O.bwd_dw(L2.X, N2, L2.dY), dt, "small-tile dW, three slices")
    assert_close(host(db2), O.bwd_db(L2.dY), dt, "small-tile db, three slices")


BF16_CASES = [
    # MFMA-compatible channel counts (C_in % 32, C_out % 16 and the reverse for dX)
    (11, 3, 14, 14, 0.4, 128, 128, False),
    (12, 5, 14, 14, 0.3, 64, 96, False),
    (13, 2, 16, 16, 0.6, 96, 64, True),       # shuffled packing: wide windows -> gather mode
    (14, 9, 14, 14, [0, 1, 2, 196, 0, 77, 5, 196, 33], 256, 128, False),
    (15, 1, 40, 40, 0.9, 32, 32, True),       # 1440 shuffled tokens in one frame
    (16, 2, 14, 14, 0.3, 160, 64, False),     # K tail of 32 channels after full 64-chunks
]


@pytest.mark.parametrize("kernel", ["valu", "mfma"])
@pytest.mark.parametrize("case", BF16_CASES, ids=lambda c: f"seed{c[0]}")
def test_bf16(case, kernel):
    seed, T, H, W, keep, Ci, Co, sh = case
    L = wl.make_random_case(seed, T, H, W, keep, Ci, Co, "bf16", shuffle=sh)
    print(f"case {case} kernel={kernel} n={L.n}", flush=True)
    st, N, _ = O.build_index(L.coords, L.frame_offsets, T, H, W)
    check_against_oracle(L, N, kernel, what=f"bf16 {kernel} {case}")


# Channel counts where the automatic choice splits the passes: the forward
# contracts 32 or 64 channels and produces 16 or 48 (MFMA, a partial output
# tile), the input gradient contracts 16 or 48 (VALU); dW on VALU.
AUTO_SPLIT_CASES = [
    (17, 2, 14, 14, 0.5, 32, 16, False),
    (18, 3, 9, 13, [40, 0, 117], 64, 48, True),
]


@pytest.mark.parametrize("case", AUTO_SPLIT_CASES, ids=lambda c: f"seed{c[0]}")
def test_bf16_auto_partial_tiles(case):
    seed, T, H, W, keep, Ci, Co, sh = case
    L = wl.make_random_case(seed, T, H, W, keep, Ci, Co, "bf16", shuffle=sh)
    print(f"case {case} n={L.n}", flush=True)
    st, N, _ = O.build_index(L.coords, L.frame_offsets, T, H, W)
    check_against_oracle(L, N, "auto", what=f"bf16 auto {case}")
    # forcing the matrix cores where the input gradient's contraction does not fit is refused
    with pytest.raises(ops.SvError) as e:
        run_all(L, N, "mfma")
    assert e.value.status == ops.SV_ERR_UNSUPPORTED


# Token counts for which plain 3 x 3 calls of the MFMA kernel take 192-token
# tiles: with 32 output channels (one channel tile) 128-token tiles need two
# dispatch rounds of the 512 slots (more than 65,536 tokens) where 192-token
# tiles need one (at most 98,304 tokens).  189 of 256 cells kept per frame
# leave a ragged last tile (75,600 tokens); the shuffled packing spreads a
# tile's neighbours too far for the window, so it stages rows tap by tap.
TILE192_CASES = [
    (21, 400, 16, 16, 189, 32, 32, False),
    (22, 300, 16, 16, 230, 32, 32, True),
]


@pytest.mark.parametrize("case", TILE192_CASES, ids=lambda c: f"seed{c[0]}")
def test_bf16_192_token_tiles(case):
    seed, T, H, W, keep, Ci, Co, sh = case
    L = wl.make_random_case(seed, T, H, W, [keep] * T, Ci, Co, "bf16", shuffle=sh)
    assert 65536 < L.n <= 98304
    print(f"case {case} n={L.n}", flush=True)
    st, N, _ = O.build_index(L.coords, L.frame_offsets, T, H, W)
    check_against_oracle(L, N, "mfma", what=f"bf16 192-token tiles {case}")


@pytest.mark.parametrize("kernel", ["valu", "mfma"])
def test_arbitrary_table_gather_mode(kernel):
    """Any N with entries in [-1, n) is a valid table for the kernels; random
    far-apart rows force the MFMA kernel out of its window mode."""
    rng = np.random.default_rng(7)
    n, Ci, Co = 1000, 64, 64
    L = wl.make_random_case(17, 1, 40, 40, [n], Ci, Co, "bf16")
    N = rng.integers(-1, n, size=(n, 9)).astype(np.int32)
    N[rng.random((n, 9)) < 0.2] = -1
    check_against_oracle(L, N, kernel, what=f"random-N {kernel}")


def test_out_of_range_entries_read_as_padding():
    """Entries >= n or < -1 contribute nothing (never read out of bounds)."""
    L = wl.make_random_case(18, 1, 14, 14, 0.5, 64, 64, "bf16")
    _, N, _ = O.build_index(L.coords, L.frame_offsets, 1, 14, 14)
    Nbad = N.copy()
    Nbad[::3, 0] = L.n + 5
    Nbad[1::3, 8] = -7
    Nclean = Nbad.copy()
    Nclean[(Nclean >= L.n) | (Nclean < -1)] = -1
    for kernel in ("valu", "mfma"):
        Y, dX, dW, db = run_all(L, Nbad, kernel)
        assert_close(Y, O.fwd(L.X, Nclean, L.Wt, L.b), "bf16", "Y")
        assert_close(dX, O.bwd_dx(L.dY, Nclean, L.Wt), "bf16", "dX")
        assert_close(dW, O.bwd_dw(L.X, Nclean, L.dY), "bf16", "dW")


def test_mfma_and_valu_agree():
    L = wl.make_random_case(19, 4, 14, 14, 0.4, 128, 128, "bf16")
    _, N, _ = O.build_index(L.coords, L.frame_offsets, L.T, L.H, L.W)
    a = run_all(L, N, "mfma")
    b = run_all(L, N, "valu")
    for x, y, nm in zip(a, b, ("Y", "dX")):
        assert_close(x, y, "bf16", f"mfma vs valu {nm}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_empty_input(dt):
    L = wl.make_random_case(20, 2, 5, 5, 0.0, 64, 64, dt)
    assert L.n == 0
    N = np.zeros((0, 9), np.int32)
    Y, dX, dW, db = run_all(L, N, "auto")
    assert Y.shape == (0, 64) and dX.shape == (0, 64)
    assert np.all(dW == 0) and np.all(db == 0)


def test_dw_accumulate():
    L = wl.make_random_case(21, 3, 14, 14, 0.5, 128, 128, "bf16")
    _, N, _ = O.build_index(L.coords, L.frame_offsets, L.T, L.H, L.W)
    X, dY, Nd = dev(L.X, torch.bfloat16), dev(L.dY, torch.bfloat16), dev(N)
    dW = torch.ones((9, 128, 128), dtype=torch.float32, device="cuda")
    db = torch.ones(128, dtype=torch.float32, device="cuda")
    ops.sv_sparseconv2d_bwd_dw(X, Nd, dY, dW, db, accumulate=True)
    torch.cuda.synchronize()
    assert_close(host(dW), O.bwd_dw(L.X, N, L.dY) + 1.0, "bf16", "dW accumulate")
    assert_close(host(db), O.bwd_db(L.dY) + 1.0, "bf16", "db accumulate")


@pytest.mark.parametrize("kernel", ["valu", "mfma"])
def test_deterministic(kernel):
    L = wl.make_random_case(22, 6, 14, 14, 0.5, 128, 128, "bf16")
    _, N, _ = O.build_index(L.coords, L.frame_offsets, L.T, L.H, L.W)
    a = run_all(L, N, kernel)
    b = run_all(L, N, kernel)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_autograd_function():
    L = wl.make_random_case(23, 2, 14, 14, 0.5, 64, 64, "bf16")
    _, N, _ = O.build_index(L.coords, L.frame_offsets, L.T, L.H, L.W)
    X = dev(L.X, torch.bfloat16).requires_grad_(True)
    Wt = dev(L.Wt, torch.float32).to(torch.bfloat16).requires_grad_(True)
    b = dev(L.b, torch.bfloat16).requires_grad_(True)
    Y = ops.sparseconv2d(X, dev(N), Wt, b)
    Y.backward(dev(L.dY, torch.bfloat16))
    torch.cuda.synchronize()
    assert_close(host(Y), O.fwd(L.X, N, L.Wt, L.b), "bf16", "Y")
    assert_close(host(X.grad), O.bwd_dx(L.dY, N, L.Wt), "bf16", "dX")
    assert_close(host(Wt.grad), O.bwd_dw(L.X, N, L.dY), "bf16", "dW")
    assert_close(host(b.grad), O.bwd_db(L.dY), "bf16", "db")
