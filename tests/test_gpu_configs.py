"""The five workloads at full size, in the launch configuration the
benchmark times, against the oracle: every element of every output (Y, dX,
dW, db, and for c5 every layer's output, upstream gradient, dW and db and
the input gradient).  The oracle takes about a second per tensor on the
host's cores at these sizes."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_convolution_pruned_amd import ops, workloads as wl
from tests.gpu_util import assert_close, dev, host, sample_rows

pytestmark = pytest.mark.gpu


def gpu_layer(L, kernel="auto", passes=("fwd", "dx", "dw")):
    dt = torch.bfloat16 if L.dtype == "bf16" else torch.float32
    coords, offs = dev(L.coords), dev(L.frame_offsets)
    N = ops.build_index(coords, offs, L.T, L.H, L.W)
    X, Wt, b, dY = dev(L.X, dt), dev(L.Wt, dt), dev(L.b, dt), dev(L.dY, dt)
    out = {"N": N}
    if "fwd" in passes:
        out["Y"] = ops.sparseconv2d_fwd(X, N, Wt, b, kernel)
    if "dx" in passes:
        out["dX"] = ops.sparseconv2d_bwd_dx(dY, N, Wt, kernel)
    if "dw" in passes:
        out["dW"], out["db"] = ops.sparseconv2d_bwd_dw(X, N, dY)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in out.items()}


def dw_rows(Ci, seed=0, count=48):
    rng = np.random.default_rng(seed)
    fixed = [0, Ci - 1, 4 * Ci, 4 * Ci + Ci - 1, 9 * Ci - 1, 8 * Ci]
    return np.unique(np.array(fixed + list(rng.choice(9 * Ci, size=count, replace=False)))).astype(np.int64)


def test_c1_full():
    L = wl.make_layer("c1")
    st, Nr, _ = O.build_index(L.coords, L.frame_offsets, L.T, L.H, L.W)
    g = gpu_layer(L)
    assert np.array_equal(g["N"], Nr)
    assert_close(g["Y"], O.fwd(L.X, Nr, L.Wt, L.b), "f32", "c1 Y")
    assert_close(g["dX"], O.bwd_dx(L.dY, Nr, L.Wt), "f32", "c1 dX")
    assert_close(g["dW"], O.bwd_dw(L.X, Nr, L.dY), "f32", "c1 dW")
    assert_close(g["db"], O.bwd_db(L.dY), "f32", "c1 db")


@pytest.mark.parametrize("kernel", ["mfma", "valu"])
def test_c2_full(kernel):
    L = wl.make_layer("c2")
    st, Nr, _ = O.build_index(L.coords, L.frame_offsets, L.T, L.H, L.W)
    g = gpu_layer(L, kernel, passes=("fwd",))
    assert np.array_equal(g["N"], Nr)
    assert_close(g["Y"], O.fwd(L.X, Nr, L.Wt, L.b), "bf16", f"c2 Y ({kernel})")


@pytest.mark.parametrize("key", ["c3a", "c3b"])
def test_c3_full(key):
    L = wl.make_layer(key)
    print(f"config {key} n={L.n}", flush=True)
    st, Nr, _ = O.build_index(L.coords, L.frame_offsets, L.T, L.H, L.W)
    g = gpu_layer(L)
    assert np.array_equal(g["N"], Nr)
    assert_close(g["Y"], O.fwd(L.X, Nr, L.Wt, L.b), "bf16", f"{key} Y")
    assert_close(g["dX"], O.bwd_dx(L.dY, Nr, L.Wt), "bf16", f"{key} dX")
    assert_close(g["dW"], O.bwd_dw(L.X, Nr, L.dY), "bf16", f"{key} dW")
    assert_close(g["db"], O.bwd_db(L.dY), "bf16", f"{key} db")


def test_c4_chunked():
    """Chunks of 256 frames through sv_sparseconv2d_chunked: equal to the
    unchunked kernels (Y, dX bit for bit; dW within tolerance) and to the
    oracle on every element; the workspace does not grow with T."""
    L = wl.make_layer("c4")
    dt = torch.bfloat16
    coords, offs = dev(L.coords), dev(L.frame_offsets)
    X, Wt, b, dY = dev(L.X, dt), dev(L.Wt, dt), dev(L.b, dt), dev(L.dY, dt)
    n, C = L.n, L.X.shape[1]
    Y = torch.empty((n, C), dtype=dt, device="cuda")
    dX = torch.empty((n, C), dtype=dt, device="cuda")
    dW = torch.empty((9, C, C), dtype=torch.float32, device="cuda")
    db = torch.empty((C,), dtype=torch.float32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    offs_h = torch.from_numpy(L.frame_offsets.copy())
    d = ops.make_chunked_desc(L.T, L.H, L.W, coords, offs, offs_h, C, C, dt, 256, X=X, Wt=Wt,
                              bias=b, Y=Y, dY=dY, dX=dX, dW=dW, db=db, err_flag=flag)
    passes = ops.SV_PASS_FWD | ops.SV_PASS_DX | ops.SV_PASS_DW
    wsb = ops.sv_chunked_workspace_bytes(d, passes)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    ops.sv_sparseconv2d_chunked(d, passes, ws)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    # workspace is sized by one chunk: the same for the first 256 frames alone
    Ls = wl.make_layer("c4", scale_T=256)
    d1 = ops.make_chunked_desc(256, L.H, L.W, coords, offs, torch.from_numpy(Ls.frame_offsets.copy()),
                               C, C, dt, 256)
    assert wsb <= ops.sv_chunked_workspace_bytes(d1, passes) * 1.25 + (1 << 20)

    g = gpu_layer(L)   # unchunked
    assert np.array_equal(host(Y), g["Y"])
    assert np.array_equal(host(dX), g["dX"])
    assert_close(host(dW), g["dW"], "bf16", "c4 chunked vs unchunked dW")
    st, Nr, _ = O.build_index(L.coords, L.frame_offsets, L.T, L.H, L.W)
    assert np.array_equal(g["N"], Nr)
    assert_close(host(Y), O.fwd(L.X, Nr, L.Wt, L.b), "bf16", "c4 Y")
    assert_close(host(dX), O.bwd_dx(L.dY, Nr, L.Wt), "bf16", "c4 dX")
    assert_close(host(dW), O.bwd_dw(L.X, Nr, L.dY), "bf16", "c4 dW")
    assert_close(host(db), O.bwd_db(L.dY), "bf16", "c4 db")


def test_c5_staged():
    """Three nested stages, two layers each, forward then backward through
    all six layers, against the oracle run end to end from the same
    inputs (the first stage's tokens, the weights and the last layer's
    upstream gradient; stage transitions as row selections): every layer's
    output and upstream gradient, every dW and db and the gradient of the
    first stage's input, element by element.  Index tables, stage gathers and
    scatters bit-exact."""
    S = wl.make_staged("c5")
    dt = torch.bfloat16
    C = S.X0.shape[1]
    Ns, Nh = [], []
    for stg in S.stages:
        Ns.append(ops.build_index(dev(stg["coords"]), dev(stg["frame_offsets"]), S.T, S.H, S.W))
        st, Nr, _ = O.build_index(stg["coords"], stg["frame_offsets"], S.T, S.H, S.W)
        assert np.array_equal(host(Ns[-1]), Nr)
        Nh.append(Nr)
    Ws = [dev(w, dt) for w in S.weights]
    bs = [dev(b, dt) for b in S.biases]
    sels = [None] + [dev(stg["sel"]) for stg in S.stages[1:]]
    L = len(S.weights)
    stage_of = [l // S.layers_per_stage for l in range(L)]
    first = [l > 0 and stage_of[l - 1] != stage_of[l] for l in range(L)]
    # GPU: forward
    xs, ys = [], []
    x = dev(S.X0, dt)
    for l in range(L):
        s = stage_of[l]
        if first[l]:
            xn = torch.empty((sels[s].shape[0], C), dtype=dt, device="cuda")
            ops.sv_stage_gather(x, sels[s], xn)
            assert np.array_equal(host(xn), host(x)[S.stages[s]["sel"]])
            x = xn
        xs.append(x)
        x = ops.sparseconv2d_fwd(x, Ns[s], Ws[l], bs[l])
        ys.append(x)
    # GPU: backward
    g = dev(S.dY_last, dt)
    gys = [None] * L
    dWs = [None] * L
    dbs = [None] * L
    for l in reversed(range(L)):
        s = stage_of[l]
        gys[l] = g
        dWs[l], dbs[l] = ops.sparseconv2d_bwd_dw(xs[l], Ns[s], g, with_db=True)
        g = ops.sparseconv2d_bwd_dx(g, Ns[s], Ws[l])
        if first[l]:
            prev_n = S.stages[s - 1]["coords"].shape[0]
            gp = torch.empty((prev_n, C), dtype=dt, device="cuda")
            ops.sv_stage_scatter(g, sels[s], gp)
            exp = np.zeros((prev_n, C), np.float32)
            exp[S.stages[s]["sel"]] = host(g)
            assert np.array_equal(host(gp), exp)
            g = gp
    torch.cuda.synchronize()
    gx = host(g)
    assert torch.equal(ys[0], ops.sparseconv2d_fwd(xs[0], Ns[0], Ws[0], bs[0])), "forward not deterministic"
    # oracle: the same chain in float64 from the inputs alone
    print("oracle chain", flush=True)
    xr = []
    x = S.X0
    for l in range(L):
        s = stage_of[l]
        if first[l]:
            x = x[S.stages[s]["sel"]]
        xr.append(x)
        x = O.fwd(x, Nh[s], S.weights[l], S.biases[l])
        assert_close(host(ys[l]), x, "bf16", f"layer {l} Y")
    print("oracle chain forward checked", flush=True)
    g = S.dY_last
    for l in reversed(range(L)):
        s = stage_of[l]
        assert_close(host(gys[l]), g, "bf16", f"layer {l} upstream gradient")
        assert_close(host(dWs[l]), O.bwd_dw(xr[l], Nh[s], g), "bf16", f"layer {l} dW")
        assert_close(host(dbs[l]), O.bwd_db(g), "bf16", f"layer {l} db")
        g = O.bwd_dx(g, Nh[s], S.weights[l])
        if first[l]:
            gp = np.zeros((S.stages[s - 1]["coords"].shape[0], C))
            gp[S.stages[s]["sel"]] = g
            g = gp
        print(f"layer {l} backward checked", flush=True)
    assert_close(gx, g, "bf16", "input gradient")
