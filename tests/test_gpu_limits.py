"""The largest inputs the matrix-core kernels take: their operands are read
through 32-bit buffer offsets, so X, Y, dY and dX may span up to 2 GiB each.
Here they are exactly 2 GiB (16,384 frames of a fully kept 16 x 16 grid:
2^22 tokens x 256 channels bf16).  The neighbour table, the forward and the
input gradient are checked on sampled rows (the first, the last, tile
boundaries and random ones) against the oracle, which computes them one by
one from those rows' neighbours; the weight and bias gradients over all the
tokens with dY nonzero only on the sampled rows.  (One token more is
refused: test_abi.)"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_convolution_pruned_amd import ops
from tests.gpu_util import assert_close, sample_rows

pytestmark = pytest.mark.gpu

T, H, W, C = 16384, 16, 16, 256
CELLS = H * W
n = T * CELLS                                   # 2^22
bf = torch.bfloat16


def rand_dev(g, shape, scale=1.0):
    return (torch.randn(shape, generator=g, device="cuda") * scale).to(bf)


def test_two_gib_operands():
    assert n * C * 2 == 2 ** 31
    g = torch.Generator(device="cuda").manual_seed(2024)
    coords = torch.arange(CELLS, dtype=torch.int32, device="cuda").repeat(T)
    offs = torch.arange(T + 1, dtype=torch.int32, device="cuda") * CELLS
    N = torch.empty((n, 9), dtype=torch.int32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    ops.sv_build_index(coords, offs, T, H, W, N, None, flag)
    Wt = rand_dev(g, (9, C, C), 1.0 / np.sqrt(9 * C))
    b = rand_dev(g, (C,), 0.1)
    X = rand_dev(g, (n, C))
    Y = ops.sparseconv2d_fwd(X, N, Wt, b, "mfma")
    torch.cuda.synchronize()
    print(f"n={n}: forward done", flush=True)
    assert int(flag.item()) == 0

    rows = sample_rows(n, 48, seed=5, tile=256)
    Nh = N[torch.from_numpy(rows).cuda()].cpu().numpy()
    # the neighbour rows against the oracle's table of each sampled row's frame
    _, Nf, _ = O.build_index(np.arange(CELLS, dtype=np.int32), np.array([0, CELLS], np.int32), 1, H, W)
    exp = Nf[rows % CELLS]
    exp = np.where(exp >= 0, exp + (rows // CELLS * CELLS)[:, None], -1)
    assert np.array_equal(Nh, exp), "neighbour table rows differ"

    # compact sub-problems: the sampled rows' neighbours, indices remapped
    need = np.unique(Nh[Nh >= 0])
    remap = np.full(n, -1, np.int64)
    remap[need] = np.arange(need.size)
    Nsub = np.where(Nh >= 0, remap[np.maximum(Nh, 0)], -1).astype(np.int32)
    sub = np.arange(rows.size)
    need_d, rows_d = torch.from_numpy(need).cuda(), torch.from_numpy(rows).cuda()
    Xs = X[need_d].float().cpu().numpy()
    Wh, bh = Wt.float().cpu().numpy(), b.float().cpu().numpy()
    Ys = Y[rows_d].float().cpu().numpy()
    del Y
    assert_close(Ys, O.fwd_rows(Xs, Nsub, Wh, bh, sub), "bf16", "2 GiB forward, sampled rows")

    dY = rand_dev(g, (n, C))
    dX = ops.sparseconv2d_bwd_dx(dY, N, Wt, "mfma")
    torch.cuda.synchronize()
    print(f"n={n}: input gradient done", flush=True)
    dYs = dY[need_d].float().cpu().numpy()
    dXs = dX[rows_d].float().cpu().numpy()
    assert_close(dXs, O.bwd_dx_rows(dYs, Nsub, Wh, sub), "bf16", "2 GiB input gradient, sampled rows")

    # weight and bias gradients over all 2^22 tokens, with dY zero except on
    # the sampled rows: the kernels still address every token (and split
    # them into slices as usual), while the exact sums reduce to those rows,
    # which the oracle computes on a compact problem (the neighbour rows
    # first with no taps and no gradient, then the sampled tokens)
    del dX
    dY.zero_()
    dY[rows_d] = rand_dev(g, (rows.size, C))
    dW, db = ops.sparseconv2d_bwd_dw(X, N, dY)
    torch.cuda.synchronize()
    print(f"n={n}: weight gradient done", flush=True)
    m = need.size
    Xc = np.concatenate([Xs, np.zeros((rows.size, C), np.float32)])
    Nc = np.concatenate([np.full((m, 9), -1, np.int32), Nsub])
    dYc = np.concatenate([np.zeros((m, C), np.float32), dY[rows_d].float().cpu().numpy()])
    assert_close(dW.cpu().numpy(), O.bwd_dw(Xc, Nc, dYc), "bf16", "2 GiB weight gradient")
    assert_close(db.cpu().numpy(), O.bwd_db(dYc), "bf16", "2 GiB bias gradient")
