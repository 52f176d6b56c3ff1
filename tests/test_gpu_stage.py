"""Stage transitions (sv_stage_gather, sv_stage_scatter) against numpy,
byte for byte: 16-, 4- and 2-byte word paths, indices outside the range
skipped, destinations that start with other contents, an empty
selection."""
import numpy as np
import pytest
import torch

from sparse_convolution_pruned_amd import ops

pytestmark = pytest.mark.gpu


def case(seed, n_src, n_sel, C, dt):
    rs = np.random.default_rng(seed)
    src = torch.from_numpy(rs.standard_normal((n_src, C)).astype(np.float32)).to(dt)
    sel = np.sort(rs.choice(n_src, size=n_sel, replace=False)).astype(np.int32)
    return src, sel


def bits(t):
    t = t.cpu()
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("C", [256, 6, 3])      # 16-byte, 4-byte and (bf16, C = 3) 2-byte words
def test_gather_and_scatter(dt, C):
    src, sel = case(5, 1000, 377, C, dt)
    rows = sel.copy()
    rows[[3, 100]] = [-1, 5000]                  # outside [0, n_src): skipped
    g = torch.full((rows.size, C), 7.0, dtype=dt, device="cuda")
    ops.sv_stage_gather(src.cuda(), torch.from_numpy(rows).cuda(), g)
    exp = np.full((rows.size, C), 7.0, np.float32)
    ok = (rows >= 0) & (rows < 1000)
    exp[ok] = src.float().numpy()[rows[ok]]
    assert torch.equal(bits(g), bits(torch.from_numpy(exp).to(dt)))

    # backward of the gather: rows outside [0, n_dst) are skipped, every other row is zero
    small = torch.from_numpy(np.random.default_rng(6).standard_normal((rows.size, C)).astype(np.float32)).to(dt)
    d = torch.full((1000, C), 3.0, dtype=dt, device="cuda")
    ops.sv_stage_scatter(small.cuda(), torch.from_numpy(rows).cuda(), d)
    exp = np.zeros((1000, C), np.float32)
    exp[rows[ok]] = small.float().numpy()[ok]
    assert torch.equal(bits(d), bits(torch.from_numpy(exp).to(dt)))


def test_empty_selection():
    d = torch.full((50, 8), 1.0, dtype=torch.bfloat16, device="cuda")
    rows = torch.zeros(0, dtype=torch.int32, device="cuda")
    ops.sv_stage_scatter(torch.zeros((0, 8), dtype=torch.bfloat16, device="cuda"), rows, d)
    assert torch.count_nonzero(d).item() == 0
