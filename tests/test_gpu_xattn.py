"""Asymmetric cross-attention (auxiliary queries over the sparse visual
tokens, keys = values) against the float64 oracle: forward (O, lse) and
backward (dQ, dX), fp32 and bf16, every supported head width, query counts
that cross the kernels' query chunks, no keys, one key, sharp and flat
softmax, the c5 stage-0 and c4 token counts, and bitwise determinism."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_convolution_pruned_amd import ops
from tests.gpu_util import assert_close, dev, host, tdtype

pytestmark = pytest.mark.gpu


def inputs(seed, m, n, d, dt, q_spread=1.0):
    """Queries, tokens and upstream gradient ~ N(0, 1) (the visual tokens
    follow the conv workloads' input distribution), rounded to the storage
    type first so the oracle sees exactly what the GPU reads."""
    rng = np.random.default_rng(seed)
    t = tdtype(dt)
    Q = torch.from_numpy(q_spread * rng.standard_normal((m, d)).astype(np.float32)).to(t)
    X = torch.from_numpy(rng.standard_normal((n, d)).astype(np.float32)).to(t)
    dO = torch.from_numpy(rng.standard_normal((m, d)).astype(np.float32)).to(t)
    return Q, X, dO


def run(Q, X, dO, scale=0.0):
    Qd, Xd, dOd = Q.cuda(), X.cuda(), dO.cuda()
    Od, lse = ops.xattn_fwd(Qd, Xd, scale)
    dQ, dX = ops.xattn_bwd(Qd, Xd, Od, dOd, lse, scale)
    torch.cuda.synchronize()
    return Od, lse, dQ, dX


def check(Q, X, dO, dt, what, scale=0.0):
    print(f"{what}: m={Q.shape[0]} n={X.shape[0]} d={Q.shape[1]} {dt}", flush=True)
    Od, lse, dQ, dX = run(Q, X, dO, scale)
    q, x = host(Q), host(X)
    sc = None if scale == 0.0 else scale
    Or, lr = O.xattn_fwd(q, x, sc)
    assert_close(host(Od), Or, dt, f"{what} O")
    lg = host(lse).astype(np.float64)
    if X.shape[0] == 0:
        assert np.all(np.isneginf(lg)), f"{what} lse"
    else:
        assert np.max(np.abs(lg - lr)) <= 1e-4 * max(1.0, float(np.max(np.abs(lr)))), f"{what} lse"
    dQr, dXr = O.xattn_bwd(q, x, host(dO), sc)
    assert_close(host(dQ), dQr, dt, f"{what} dQ")
    assert_close(host(dX), dXr, dt, f"{what} dX")
    return Od, lse, dQ, dX


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("m,n", [(1, 1000), (3, 17), (5, 2049), (16, 700)])
def test_sizes(dt, d, m, n):
    Q, X, dO = inputs(1000 * m + n + d, m, n, d, dt)
    check(Q, X, dO, dt, "sizes")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_one_key_and_no_keys(dt):
    Q, X, dO = inputs(7, 4, 1, 128, dt)
    Od, lse, dQ, dX = check(Q, X, dO, dt, "one key")
    assert np.array_equal(host(Od), np.repeat(host(X), 4, axis=0)), "one key: O must equal it exactly"
    Q, X, dO = inputs(8, 3, 0, 64, dt)
    Od, lse, dQ, dX = run(Q, X, dO)
    assert np.array_equal(host(Od), np.zeros((3, 64))) and np.all(np.isneginf(host(lse)))
    assert np.array_equal(host(dQ), np.zeros((3, 64))) and dX.shape == (0, 64)


@pytest.mark.parametrize("spread", [0.05, 6.0])
def test_flat_and_sharp_softmax(spread):
    Q, X, dO = inputs(9, 2, 5000, 256, "bf16", q_spread=spread)
    check(Q, X, dO, "bf16", f"spread {spread}")


def test_dq_under_cancellation():
    """Tokens that share one large component (rows = 3u + small noise): the
    two terms of dS = P (dP - D) and the sum over keys of dS X[j] nearly
    cancel.  The kernels shift the keys by O inside those sums (exact in
    exact arithmetic); unshifted fp32 sums are off by 2e-2 here, and D
    taken from the stored bf16 O by a factor of 100."""
    rng = np.random.default_rng(13)
    d, n = 128, 4000
    u = rng.standard_normal(d)
    X = torch.from_numpy((3.0 * u + 0.05 * rng.standard_normal((n, d))).astype(np.float32)).to(torch.bfloat16)
    Q = torch.from_numpy(rng.standard_normal((2, d)).astype(np.float32)).to(torch.bfloat16)
    dO = torch.from_numpy(rng.standard_normal((2, d)).astype(np.float32)).to(torch.bfloat16)
    check(Q, X, dO, "bf16", "cancellation")


def test_explicit_scale():
    Q, X, dO = inputs(10, 2, 3000, 128, "f32")
    check(Q, X, dO, "f32", "scale 0.3", scale=0.3)


@pytest.mark.parametrize("n", [58822, 181248])
def test_full_size_cls(n):
    """One CLS query over the c5 stage-0 tokens and the c4 tokens (d = 256
    and 128), checked in full against the oracle."""
    d = 256 if n == 58822 else 128
    Q, X, dO = inputs(11, 1, n, d, "bf16")
    check(Q, X, dO, "bf16", f"CLS over {n}")


def test_deterministic_and_no_queries():
    Q, X, dO = inputs(12, 5, 20000, 256, "bf16")
    a = run(Q, X, dO)
    b = run(Q, X, dO)
    for u, v in zip(a, b):
        assert torch.equal(u, v), "two runs differ"
    # no queries: dX is zero
    Xd = X.cuda()
    dX = torch.full_like(Xd, 3.0)
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    e = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((0,), dtype=torch.float32, device="cuda")
    dQ = torch.empty((0, 256), dtype=torch.float32, device="cuda")
    ops.sv_xattn_bwd(e, Xd, e, e, lse, dQ, dX, ws)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dX).item() == 0
