"""GPU index builder (sv_build_index) against the oracle: bit-exact N and M."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_convolution_pruned_amd import ops, workloads as wl
from tests import pins
from tests.gpu_util import dev, host

pytestmark = pytest.mark.gpu


def gpu_index(coords, offs, T, H, W):
    c = dev(np.asarray(coords, np.int32))
    o = dev(np.asarray(offs, np.int32))
    n = c.shape[0]
    N = torch.full((n, 9), -99, dtype=torch.int32, device="cuda")
    M = torch.full((T, H, W), -99, dtype=torch.int32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    ops.sv_build_index(c, o, T, H, W, N, M, flag)
    torch.cuda.synchronize()
    return host(N), host(M), int(flag.item())


CASES = pins.CASES + [
    (40, 5, 14, 14, 0.3, 1, 1, False),
    (41, 3, 16, 16, [256, 0, 1], 1, 1, True),
    (42, 2, 128, 128, 0.05, 1, 1, True),     # largest grid the LDS map holds (16384 cells)
    (43, 1, 1, 16384, 0.5, 1, 1, False),     # one row
    (44, 7, 3, 3, 1.0, 1, 1, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c[0]}")
def test_index_random(case):
    L = pins.case_layer(case)
    print(f"case {case} n={L.n}", flush=True)
    st, Nr, Mr = O.build_index(L.coords, L.frame_offsets, L.T, L.H, L.W, want_map=True)
    assert st == 0
    N, M, flag = gpu_index(L.coords, L.frame_offsets, L.T, L.H, L.W)
    assert flag == 0
    assert np.array_equal(N, Nr)
    assert np.array_equal(M, Mr)


@pytest.mark.parametrize("name", ["index_fwd_bwd_hand_3x4.txt", "index_frames_2x2.txt"])
def test_index_golden(name):
    g = pins.read_golden(name)
    N, _, flag = gpu_index(g["coords"], g["frame_offsets"], g["T"], g["H"], g["W"])
    assert flag == 0 and np.array_equal(N, g["N"])


@pytest.mark.parametrize("key", ["c1", "c2", "c3a", "c4"])
def test_index_configs(key):
    L = wl.make_layer(key)
    print(f"config {key} n={L.n}", flush=True)
    st, Nr, Mr = O.build_index(L.coords, L.frame_offsets, L.T, L.H, L.W, want_map=True)
    assert st == 0
    N, M, flag = gpu_index(L.coords, L.frame_offsets, L.T, L.H, L.W)
    assert flag == 0 and np.array_equal(N, Nr) and np.array_equal(M, Mr)


def test_index_staged_config():
    S = wl.make_staged("c5")
    for s, stg in enumerate(S.stages):
        st, Nr, _ = O.build_index(stg["coords"], stg["frame_offsets"], S.T, S.H, S.W)
        assert st == 0
        N, _, flag = gpu_index(stg["coords"], stg["frame_offsets"], S.T, S.H, S.W)
        assert flag == 0 and np.array_equal(N, Nr), f"stage {s}"


def test_index_empty():
    N, M, flag = gpu_index(np.zeros(0, np.int32), np.zeros(4, np.int32), 3, 4, 5)
    assert N.shape == (0, 9) and flag == 0 and np.all(M == -1)


@pytest.mark.parametrize("coords,bit", [([0, 5, 12], ops.SV_FLAG_COORD_RANGE),
                                        ([0, -1, 2], ops.SV_FLAG_COORD_RANGE),
                                        ([0, 5, 5], ops.SV_FLAG_DUPLICATE)])
def test_index_error_flags(coords, bit):
    _, _, flag = gpu_index(np.array(coords, np.int32), np.array([0, 3], np.int32), 1, 3, 4)
    assert flag & bit
    with pytest.raises(ops.SvError):
        ops.build_index(dev(np.array(coords, np.int32)), dev(np.array([0, 3], np.int32)), 1, 3, 4)


def test_index_bad_offsets_flag():
    # frame 0 claims 3 tokens but the buffer holds 2
    _, _, flag = gpu_index(np.array([0, 1], np.int32), np.array([0, 3], np.int32), 1, 3, 4)
    assert flag & ops.SV_FLAG_BAD_OFFSETS


@pytest.mark.parametrize("offs", [[0, 2], [1, 3], [0, 1, 2]])
def test_index_offsets_must_cover_all_rows(offs):
    # three rows, but the frames cover only rows 0..1, 1..2 or 0..1: some
    # row of N would be left unwritten, which the flag reports
    _, _, flag = gpu_index(np.array([0, 5, 7], np.int32), np.array(offs, np.int32), len(offs) - 1, 3, 4)
    assert flag & ops.SV_FLAG_BAD_OFFSETS


def test_index_grid_too_large_rejected():
    c = dev(np.zeros(1, np.int32))
    o = dev(np.array([0, 1], np.int32))
    N = torch.empty((1, 9), dtype=torch.int32, device="cuda")
    with pytest.raises(ops.SvError) as ei:
        ops.sv_build_index(c, o, 1, 129, 128, N)
    assert ei.value.status == ops.SV_ERR_UNSUPPORTED


def test_sync_check_turns_the_flag_into_a_status(monkeypatch):
    """SV_SYNC_CHECK=1: the index build and the chunk driver wait for their
    stream and return the status the device flag implies."""
    c, o = dev(np.array([0, 5, 5], np.int32)), dev(np.array([0, 3], np.int32))
    N = torch.empty((3, 9), dtype=torch.int32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    ops.sv_build_index(c, o, 1, 3, 4, N, None, flag)          # off: no status
    torch.cuda.synchronize()
    assert int(flag.item()) & ops.SV_FLAG_DUPLICATE
    monkeypatch.setenv("SV_SYNC_CHECK", "1")
    flag.zero_()
    with pytest.raises(ops.SvError) as e:
        ops.sv_build_index(c, o, 1, 3, 4, N, None, flag)
    assert e.value.status == ops.SV_ERR_DUPLICATE_COORD
    flag.zero_()
    c2 = dev(np.array([0, 5, 12], np.int32))
    with pytest.raises(ops.SvError) as e:
        ops.sv_build_index(c2, o, 1, 3, 4, N, None, flag)
    assert e.value.status == ops.SV_ERR_COORD_RANGE
    # a clean call passes, and the chunk driver reports through the same path
    flag.zero_()
    ops.sv_build_index(dev(np.array([0, 5, 11], np.int32)), o, 1, 3, 4, N, None, flag)
    offs_h = torch.tensor([0, 3], dtype=torch.int32)
    X = torch.zeros((3, 8), dtype=torch.float32, device="cuda")
    Wt = torch.zeros((9, 8, 8), dtype=torch.float32, device="cuda")
    Y = torch.empty((3, 8), dtype=torch.float32, device="cuda")
    d = ops.make_chunked_desc(1, 3, 4, c, o, offs_h, 8, 8, torch.float32, 1, X=X, Wt=Wt, Y=Y, err_flag=flag)
    ws = torch.empty(max(256, ops.sv_chunked_workspace_bytes(d, ops.SV_PASS_FWD)), dtype=torch.uint8, device="cuda")
    with pytest.raises(ops.SvError) as e:
        ops.sv_sparseconv2d_chunked(d, ops.SV_PASS_FWD, ws)
    assert e.value.status == ops.SV_ERR_DUPLICATE_COORD
    monkeypatch.delenv("SV_SYNC_CHECK")
    torch.cuda.synchronize()
