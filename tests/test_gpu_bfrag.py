"""The matrix-core kernel that streams the weights in fragment order
(bf16, 3 x 3, 5 x 5, 7 x 7 or 1 x 1, contracted channels a multiple of 64,
produced channels a multiple of 128): forward and input gradient against the oracle in every
staging mode and tile shape, and bit for bit against the kernel that reads
Wt directly (the input gradient without a workspace).  The split forms
(repack, then the packed call) must equal the single calls bit for bit."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_convolution_pruned_amd import ops, workloads as wl
from tests.gpu_util import assert_close, dev, host

pytestmark = pytest.mark.gpu

bf = torch.bfloat16


def dx_both(dY, Nd, Wt):
    """Input gradient with a workspace (fragment-order kernel) and without
    (the kernel that reads Wt directly)."""
    n, Ci = dY.shape[0], Wt.shape[1]
    a = torch.empty((n, Ci), dtype=bf, device="cuda")
    b = torch.empty((n, Ci), dtype=bf, device="cuda")
    ops.sv_sparseconv2d_bwd_dx(dY, Nd, Wt, a, "mfma")
    ops.sv_sparseconv2d_bwd_dx(dY, Nd, Wt, b, "mfma", workspace=0)
    torch.cuda.synchronize()
    return a, b


def check_case(L, N, what):
    X, Wt, b, dY = dev(L.X, bf), dev(L.Wt, bf), dev(L.b, bf), dev(L.dY, bf)
    Nd = dev(N)
    Y = ops.sparseconv2d_fwd(X, Nd, Wt, b, "mfma")
    dXf, dXd = dx_both(dY, Nd, Wt)
    assert torch.equal(dXf.view(torch.int16), dXd.view(torch.int16)), f"{what}: fragment and direct dX differ"
    assert_close(host(Y), O.fwd(L.X, N, L.Wt, L.b), "bf16", f"{what} Y")
    assert_close(host(dXf), O.bwd_dx(L.dY, N, L.Wt), "bf16", f"{what} dX")


# (seed, T, H, W, keep, Ci, Co, shuffle); Co % 128 == 0 puts the forward on
# the fragment kernel, Ci % 128 == 0 the input gradient.
CASES = [
    (31, 3, 16, 16, 0.6, 256, 256, False),              # window mode, ragged last tile, MB = 2
    (32, 4, 16, 16, 0.5, 256, 256, True),               # shuffled packing: gather mode tap by tap
    (33, 2, 40, 40, 0.5, 256, 256, False),              # grid 40 wide: tiles outside the window
    (34, 5, 14, 14, [0, 1, 196, 0, 60], 512, 256, False),  # empty frames; C_in 512 (8 chunks)
    (35, 3, 16, 16, 0.4, 256, 512, False),              # several output-channel tiles
    (37, 90, 16, 16, 0.8, 256, 512, False),             # 18,450 tokens: 192 x 256 tiles forward, 192 x 128 dX
    (38, 6, 14, 14, 0.5, 128, 128, False),              # 128 channels: 128 x 128 tiles
    (39, 40, 14, 14, 0.7, 128, 256, True),              # 128 -> 256, gather mode
    (36, 2, 14, 14, 0.7, 64, 256, False),               # one 64-channel chunk in the forward
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c[0]}")
def test_fragment_kernel(case):
    seed, T, H, W, keep, Ci, Co, sh = case
    L = wl.make_random_case(seed, T, H, W, keep, Ci, Co, "bf16", shuffle=sh)
    print(f"case {case} n={L.n}", flush=True)
    _, N, _ = O.build_index(L.coords, L.frame_offsets, T, H, W)
    check_case(L, N, f"{case}")


# (frames, kept per frame, channels, tokens x channels of the tile the host
# picks: the smallest tile whose grid fits one round of 256 workgroups,
# 256-channel tiles first at equal size; without one, the largest tile)
TILES = [(60, 200, 256, "128x128"), (100, 200, 256, "192x128"), (140, 200, 256, "128x256"),
         (200, 200, 256, "192x256"), (230, 230, 256, "256x256"), (230, 240, 128, "256x128"),
         (300, 240, 128, "256x128 x2 rounds")]
TILE_RANGE = {(256, "128x128"): (0, 128 * 128), (256, "192x128"): (128 * 128, 128 * 192),
              (256, "128x256"): (128 * 192, 256 * 128), (256, "192x256"): (256 * 128, 256 * 192),
              (256, "256x256"): (256 * 192, 10 ** 9), (128, "256x128"): (256 * 192, 256 * 256),
              (128, "256x128 x2 rounds"): (256 * 256, 10 ** 9)}


@pytest.mark.parametrize("n_frames,keep,C,tile", TILES, ids=[t[3] for t in TILES])
def test_tile_shapes(n_frames, keep, C, tile):
    """Token counts that select each tile shape."""
    L = wl.make_random_case(40 + n_frames, n_frames, 16, 16, [keep] * n_frames, C, C, "bf16")
    n = L.n
    lo, hi = TILE_RANGE[(C, tile)]
    assert lo < n <= hi, n
    print(f"n={n} frames={n_frames} C={C} tile={tile}", flush=True)
    _, N, _ = O.build_index(L.coords, L.frame_offsets, L.T, L.H, L.W)
    check_case(L, N, f"tile {tile}")


def test_random_table_and_out_of_range():
    """Any N works: a random table with -1 entries and entries outside
    [0, n) (read as padding) puts every tile in gather mode."""
    L = wl.make_random_case(51, 2, 16, 16, 0.8, 256, 256, "bf16")
    rng = np.random.default_rng(5)
    n = L.n
    N = rng.integers(-1, n, size=(n, 9)).astype(np.int32)
    N[rng.random((n, 9)) < 0.05] = n + 3
    N[rng.random((n, 9)) < 0.05] = -7
    Nclean = np.where((N >= 0) & (N < n), N, -1).astype(np.int32)
    X, Wt, b, dY = dev(L.X, bf), dev(L.Wt, bf), dev(L.b, bf), dev(L.dY, bf)
    Nd = dev(N)
    Y = ops.sparseconv2d_fwd(X, Nd, Wt, b, "mfma")
    dXf, dXd = dx_both(dY, Nd, Wt)
    assert torch.equal(dXf.view(torch.int16), dXd.view(torch.int16))
    assert_close(host(Y), O.fwd(L.X, Nclean, L.Wt, L.b), "bf16", "random N Y")
    assert_close(host(dXf), O.bwd_dx(L.dY, Nclean, L.Wt), "bf16", "random N dX")


def test_split_forms_bitwise():
    """Repack once, then the packed calls: equal to the single calls."""
    L = wl.make_random_case(52, 6, 16, 16, 0.55, 256, 256, "bf16")
    _, N, _ = O.build_index(L.coords, L.frame_offsets, L.T, L.H, L.W)
    X, Wt, b, dY = dev(L.X, bf), dev(L.Wt, bf), dev(L.b, bf), dev(L.dY, bf)
    Nd = dev(N)
    n = L.n
    V = torch.empty(ops.sv_workspace_bytes(ops.SV_OP_FWD, n, 256, 256, bf), dtype=torch.uint8, device="cuda")
    P = torch.empty(ops.sv_workspace_bytes(ops.SV_OP_DX, n, 256, 256, bf), dtype=torch.uint8, device="cuda")
    ops.sv_repack_fwd_k(Wt, V)
    ops.sv_repack_dx_k(Wt, P)
    Y1 = torch.empty((n, 256), dtype=bf, device="cuda")
    dX1 = torch.empty((n, 256), dtype=bf, device="cuda")
    ops.sv_sparseconv2d_fwd_packed_k(X, Nd, V, b, Y1, 3)
    ops.sv_sparseconv2d_bwd_dx_packed_k(dY, Nd, P, dX1, 3)
    Y2 = ops.sparseconv2d_fwd(X, Nd, Wt, b, "mfma")
    dX2 = ops.sparseconv2d_bwd_dx(dY, Nd, Wt, "mfma")
    torch.cuda.synchronize()
    assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))
    assert torch.equal(dX1.view(torch.int16), dX2.view(torch.int16))
    assert_close(host(dX1), O.bwd_dx(L.dY, N, L.Wt), "bf16", "packed dX")


def test_chunk_driver_c256_bitwise():
    """The chunk driver at C = 256 (forward and input gradient on the
    fragment kernel from weights repacked once per call) gives the
    unchunked calls' Y and dX bit for bit."""
    L = wl.make_random_case(53, 12, 16, 16, 0.5, 256, 256, "bf16")
    _, N, _ = O.build_index(L.coords, L.frame_offsets, L.T, L.H, L.W)
    X, Wt, b, dY = dev(L.X, bf), dev(L.Wt, bf), dev(L.b, bf), dev(L.dY, bf)
    n = L.n
    Y = torch.empty((n, 256), dtype=bf, device="cuda")
    dX = torch.empty((n, 256), dtype=bf, device="cuda")
    dW = torch.empty((9, 256, 256), dtype=torch.float32, device="cuda")
    db = torch.empty((256,), dtype=torch.float32, device="cuda")
    desc = ops.make_chunked_desc(L.T, L.H, L.W, dev(L.coords), dev(L.frame_offsets),
                                 torch.from_numpy(L.frame_offsets.copy()), 256, 256, bf, 5, X=X, Wt=Wt, bias=b,
                                 Y=Y, dY=dY, dX=dX, dW=dW, db=db)
    pm = ops.SV_PASS_FWD | ops.SV_PASS_DX | ops.SV_PASS_DW
    ws = torch.empty(max(256, ops.sv_chunked_workspace_bytes(desc, pm)), dtype=torch.uint8, device="cuda")
    ops.sv_sparseconv2d_chunked(desc, pm, ws)
    Nd = dev(N)
    Yr = ops.sparseconv2d_fwd(X, Nd, Wt, b, "mfma")
    dXr = ops.sparseconv2d_bwd_dx(dY, Nd, Wt, "mfma")
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Yr.view(torch.int16))
    assert torch.equal(dX.view(torch.int16), dXr.view(torch.int16))
    assert_close(host(dW), O.bwd_dw(L.X, N, L.dY), "bf16", "chunked dW")


@pytest.mark.parametrize("C", [256, 128, 192])
def test_repack_layers_equals_single_repacks(C):
    """One launch for several layers writes exactly what the per-layer
    repacks write (fragment order at C = 256 and 128; at C = 192 the
    forward's per-tap layout and no input-gradient layout)."""
    g = torch.Generator(device="cuda").manual_seed(3)
    Ws = [torch.randn(9, C, C, device="cuda", generator=g).to(bf) for _ in range(5)]
    nbytes = ops.sv_workspace_bytes(ops.SV_OP_FWD, 1000, C, C, bf)
    new = lambda: torch.full((nbytes,), 0xAB, dtype=torch.uint8, device="cuda")
    V1, V2 = [new() for _ in Ws], [new() for _ in Ws]
    dx = C % 128 == 0
    P1 = [new() for _ in Ws] if dx else None
    P2 = [new() for _ in Ws] if dx else None
    ops.sv_repack_layers_k(Ws, V1, P1)
    for i, W in enumerate(Ws):
        ops.sv_repack_fwd_k(W, V2[i])
        if dx:
            ops.sv_repack_dx_k(W, P2[i])
    torch.cuda.synchronize()
    for i in range(len(Ws)):
        assert torch.equal(V1[i], V2[i]), f"forward layout of layer {i}"
        if dx:
            assert torch.equal(P1[i], P2[i]), f"input-gradient layout of layer {i}"


@pytest.mark.parametrize("Ci,Co", [(512, 256), (1024, 128), (256, 512)])
def test_one_by_one(Ci, Co):
    """1 x 1 layers with at least 512 contracted channels run on the
    fragment kernel (no halo: the window is the tile's own rows); forward
    and input gradient against the oracle."""
    L = wl.make_random_case(61, 5, 14, 14, 0.6, Ci, Co, "bf16", ksize=1)
    _, N, _ = O.build_index(L.coords, L.frame_offsets, L.T, L.H, L.W, K=1)
    print(f"n={L.n} Ci={Ci} Co={Co}", flush=True)
    X, Wt, b, dY = dev(L.X, bf), dev(L.Wt, bf), dev(L.b, bf), dev(L.dY, bf)
    Nd = dev(N)
    Y = ops.sparseconv2d_fwd(X, Nd, Wt, b, "mfma")
    dX = ops.sparseconv2d_bwd_dx(dY, Nd, Wt, "mfma")
    torch.cuda.synchronize()
    assert_close(host(Y), O.fwd(L.X, N, L.Wt, L.b), "bf16", f"1x1 {Ci}->{Co} Y")
    assert_close(host(dX), O.bwd_dx(L.dY, N, L.Wt), "bf16", f"1x1 {Ci}->{Co} dX")


# (seed, T, H, W, keep, Ci, Co, shuffle, K)
KXK_CASES = [
    (71, 4, 14, 14, 0.6, 128, 128, False, 5),    # window mode: reach 2W + 2 = 30 rows
    (72, 4, 16, 16, 0.6, 256, 128, False, 7),    # window mode: reach 3W + 3 = 51 of the 64-row halo
    (73, 3, 16, 16, 0.5, 128, 256, True, 5),     # shuffled packing: gather mode
    (74, 3, 24, 24, 0.5, 128, 128, False, 7),    # 24 wide: reach 75 rows, gather mode
    (75, 9, 14, 14, [0, 1, 196, 0, 60, 3, 150, 0, 77], 256, 256, False, 7),   # empty frames, ragged tail
]


@pytest.mark.parametrize("case", KXK_CASES, ids=lambda c: f"seed{c[0]}-K{c[-1]}")
def test_fragment_kernel_kxk(case):
    """5 x 5 and 7 x 7 layers on the fragment kernel (a 64-row halo):
    forward and input gradient against the oracle, and the input gradient
    bit for bit against the kernel that reads Wt directly."""
    seed, T, H, W, keep, Ci, Co, sh, K = case
    L = wl.make_random_case(seed, T, H, W, keep, Ci, Co, "bf16", shuffle=sh, ksize=K)
    _, N, _ = O.build_index(L.coords, L.frame_offsets, L.T, L.H, L.W, K=K)
    print(f"n={L.n} K={K} Ci={Ci} Co={Co} shuffle={sh}", flush=True)
    X, Wt, b, dY = dev(L.X, bf), dev(L.Wt, bf), dev(L.b, bf), dev(L.dY, bf)
    Nd = dev(N)
    Y = ops.sparseconv2d_fwd(X, Nd, Wt, b, "mfma")
    dXf = torch.empty((L.n, Ci), dtype=bf, device="cuda")
    dXd = torch.empty((L.n, Ci), dtype=bf, device="cuda")
    ops.sv_sparseconv2d_bwd_dx_k(dY, Nd, Wt, dXf, "mfma")
    ops.sv_sparseconv2d_bwd_dx_k(dY, Nd, Wt, dXd, "mfma", workspace=0)
    torch.cuda.synchronize()
    assert torch.equal(dXf.view(torch.int16), dXd.view(torch.int16)), f"K={K}: fragment and direct dX differ"
    assert_close(host(Y), O.fwd(L.X, N, L.Wt, L.b), "bf16", f"K={K} {case} Y")
    assert_close(host(dXf), O.bwd_dx(L.dY, N, L.Wt), "bf16", f"K={K} {case} dX")
