"""Bottleneck adapter (down-projection, K x K SparseConv2D, up-projection,
residual) against the oracle: forward (Y, H1, H2) and backward (dX and the
six parameter gradients), fp32 and bf16, both kernel families, K = 1, 3, 5,
channel counts that send single layers to different kernels, empty input,
bitwise determinism, and the full first-stage token set of the c5 workload
at C = 1024, r = 256, element by element."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_convolution_pruned_amd import ops, workloads as wl
from tests.gpu_util import assert_close, dev, host, tdtype

pytestmark = pytest.mark.gpu

GRADS = ("dX", "dWd", "dbd", "dWc", "dbc", "dWu", "dbu")


def run(A, kernel="auto"):
    t = tdtype(A.dtype)
    X = dev(A.X, t)
    N = ops.build_index(dev(A.coords), dev(A.frame_offsets), A.T, A.H, A.W, K=A.K)
    P = {k: dev(getattr(A, k), t) for k in ("Wd", "bd", "Wc", "bc", "Wu", "bu")}
    Y, H1, H2 = ops.adapter_fwd(X, N, P["Wd"], P["bd"], P["Wc"], P["bc"], P["Wu"], P["bu"], kernel)
    g = ops.adapter_bwd(X, N, P["Wd"], P["Wc"], P["Wu"], H1, H2, dev(A.dY, t), kernel)
    torch.cuda.synchronize()
    return N, Y, H1, H2, g


def check(A, kernel, what):
    print(f"{what}: n={A.n} C={A.X.shape[1]} r={A.Wd.shape[1]} K={A.K} {A.dtype} {kernel}", flush=True)
    N, Y, H1, H2, g = run(A, kernel)
    st, Nr, _ = O.build_index(A.coords, A.frame_offsets, A.T, A.H, A.W, K=A.K)
    assert np.array_equal(host(N), Nr)
    Yr, H1r, H2r = O.adapter_fwd(A.X, Nr, A.Wd, A.bd, A.Wc, A.bc, A.Wu, A.bu)
    assert_close(host(H1), H1r, A.dtype, f"{what} H1")
    assert_close(host(H2), H2r, A.dtype, f"{what} H2")
    assert_close(host(Y), Yr, A.dtype, f"{what} Y")
    # the branch alone, so that the residual cannot hide an error in it
    assert_close(host(Y).astype(np.float64) - A.X, Yr - A.X, A.dtype, f"{what} Y - X")
    gr = O.adapter_bwd(A.X, Nr, A.Wd, A.bd, A.Wc, A.bc, A.Wu, A.dY)
    for k in GRADS:
        assert_close(host(g[k]), gr[k], A.dtype, f"{what} {k}")
    return N, Y, H1, H2, g


# (seed, T, H, W, keep, C, r, shuffle)
CASES = [
    (61, 3, 14, 14, 0.4, 64, 32, False),
    (62, 2, 16, 16, 0.6, 128, 128, True),             # MFMA weight gradients; gather staging
    (63, 4, 9, 11, [0, 99, 5, 60], 48, 16, False),    # down-projection on the VALU kernel
]


@pytest.mark.parametrize("K", [1, 3, 5])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c[0]}")
def test_adapter_f32(case, K):
    seed, T, H, W, keep, C, r, sh = case
    A = wl.make_adapter_case(seed, T, H, W, keep, C, r, K, "f32", sh)
    check(A, "valu", f"f32 {case}")


@pytest.mark.parametrize("kernel", ["auto", "valu"])
@pytest.mark.parametrize("K", [1, 3, 5])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c[0]}")
def test_adapter_bf16(case, K, kernel):
    seed, T, H, W, keep, C, r, sh = case
    A = wl.make_adapter_case(seed, T, H, W, keep, C, r, K, "bf16", sh)
    check(A, kernel, f"bf16 {case}")


def test_adapter_mfma_forced_and_unsupported():
    A = wl.make_adapter_case(64, 2, 14, 14, 0.5, 256, 64, 3, "bf16")
    check(A, "mfma", "bf16 forced mfma")
    B = wl.make_adapter_case(65, 1, 6, 6, 0.5, 48, 16, 3, "bf16")
    with pytest.raises(ops.SvError) as e:
        run(B, "mfma")
    assert e.value.status == ops.SV_ERR_UNSUPPORTED


@pytest.mark.parametrize("C, r, T, keep", [(256, 128, 1, 0.15), (512, 256, 3, 1.0), (256, 64, 5, 0.4)])
def test_adapter_dense_residual_tiles(C, r, T, keep):
    """The residual layers on the dense streaming kernel (output width a
    multiple of 256): fewer tokens than one 64-token tile (38), whole tiles
    only with two 256-wide output blocks (C = 512, 3 full 16 x 16 frames: 768
    tokens), and a ragged last tile (510 tokens, K = 64 contracted channels)."""
    A = wl.make_adapter_case(70 + T, T, 16, 16, keep, C, r, 3, "bf16")
    print(f"n = {A.n}", flush=True)
    check(A, "auto", f"dense residual C={C} r={r} n={A.n}")


def test_adapter_empty_and_deterministic():
    A = wl.make_adapter_case(66, 2, 14, 14, [0, 0], 128, 64, 3, "bf16")
    assert A.n == 0
    N, Y, H1, H2, g = run(A)
    assert Y.shape == (0, 128) and g["dX"].shape == (0, 128)
    for k in ("dWd", "dbd", "dWc", "dbc", "dWu", "dbu"):
        assert torch.count_nonzero(g[k]).item() == 0, f"{k} of an empty input must be zero"
    B = wl.make_adapter_case(67, 6, 16, 16, 0.5, 256, 128, 3, "bf16")
    a, b = run(B), run(B)
    assert all(torch.equal(u, v) for u, v in zip(a[1:4], b[1:4]))
    assert all(torch.equal(a[4][k], b[4][k]) for k in GRADS)


def test_adapter_full_size_stage0():
    """C = 1024 around r = 256 over the 58822 first-stage tokens of the c5
    workload (the benchmark's adapter shape), every output element checked."""
    A = wl.make_adapter_stage0()
    check(A, "auto", "c5 stage 0")


@pytest.mark.parametrize("K", [1, 3])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_adapter_bwd_dw_stream_bitwise(K, dt):
    """The three weight gradients on a second stream give the same bits as
    the one-stream backward: every kernel and its inputs are the same, and
    the caller's stream alone orders the results."""
    A = wl.make_adapter_case(68, 4, 16, 16, 0.6, 256, 128, K, dt)
    t = tdtype(A.dtype)
    X = dev(A.X, t)
    N = ops.build_index(dev(A.coords), dev(A.frame_offsets), A.T, A.H, A.W, K=A.K)
    P = {k: dev(getattr(A, k), t) for k in ("Wd", "bd", "Wc", "bc", "Wu", "bu")}
    Y, H1, H2 = ops.adapter_fwd(X, N, P["Wd"], P["bd"], P["Wc"], P["bc"], P["Wu"], P["bu"])
    dY = dev(A.dY, t)
    a = ops.adapter_bwd(X, N, P["Wd"], P["Wc"], P["Wu"], H1, H2, dY)
    b = ops.adapter_bwd(X, N, P["Wd"], P["Wc"], P["Wu"], H1, H2, dY, dw_stream=torch.cuda.Stream())
    a = {k: v.cpu() for k, v in a.items()}
    b = {k: v.cpu() for k, v in b.items()}      # ordered by the current stream alone
    for k in GRADS:
        assert torch.equal(a[k], b[k]), f"{k} differs with the dW stream"


def test_adapter_bwd_dw_stream_full_size():
    A = wl.make_adapter_stage0()
    t = tdtype(A.dtype)
    X = dev(A.X, t)
    N = ops.build_index(dev(A.coords), dev(A.frame_offsets), A.T, A.H, A.W, K=A.K)
    P = {k: dev(getattr(A, k), t) for k in ("Wd", "bd", "Wc", "bc", "Wu", "bu")}
    Y, H1, H2 = ops.adapter_fwd(X, N, P["Wd"], P["bd"], P["Wc"], P["bc"], P["Wu"], P["bu"])
    dY = dev(A.dY, t)
    a = {k: v.cpu() for k, v in ops.adapter_bwd(X, N, P["Wd"], P["Wc"], P["Wu"], H1, H2, dY).items()}
    b = {k: v.cpu() for k, v in ops.adapter_bwd(X, N, P["Wd"], P["Wc"], P["Wu"], H1, H2, dY,
                                                 dw_stream=torch.cuda.Stream()).items()}
    for k in GRADS:
        assert torch.equal(a[k], b[k]), f"{k} differs with the dW stream"
