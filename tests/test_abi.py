"""The C-ABI library on the CPU: it loads, exports every function
include/svconv.h declares, and its host-only logic (argument validation,
workspace sizing, status strings) behaves as documented.  No call here
reaches the GPU: every call returns before any HIP work is enqueued."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

from sparse_convolution_pruned_amd import ops, workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "svconv.h")
FAKE = ctypes.c_void_p(4096)   # never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sv_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from sparse_convolution_pruned_amd import build
    if not os.path.exists(ops.LIB_PATH):
        build.build()
    return ops.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 11
    for name in names:
        assert hasattr(lib, name), f"{name} declared in svconv.h but not exported"
    assert sorted(ops.SYMBOLS) == names, "binding symbol list differs from the header"


def test_status_strings(lib):
    for code in range(7):
        s = ops.status_string(code)
        assert s.startswith("SV_"), s
    assert "unknown" in ops.status_string(99)
    assert ops.version().startswith("svconv") and "gfx950" in ops.version()


def test_validation_without_device(lib):
    F32, BF16 = ops.SV_F32, ops.SV_BF16
    # negative n, zero channels, bad dtype, bad kernel enum
    assert lib.sv_sparseconv2d_fwd(FAKE, FAKE, FAKE, None, FAKE, -1, 4, 4, F32, 0, None, 0, None) == ops.SV_ERR_INVALID_ARG
    assert lib.sv_sparseconv2d_fwd(FAKE, FAKE, FAKE, None, FAKE, 8, 0, 4, F32, 0, None, 0, None) == ops.SV_ERR_INVALID_ARG
    assert lib.sv_sparseconv2d_fwd(FAKE, FAKE, FAKE, None, FAKE, 8, 4, 4, 7, 0, None, 0, None) == ops.SV_ERR_INVALID_ARG
    assert lib.sv_sparseconv2d_fwd(FAKE, FAKE, FAKE, None, FAKE, 8, 4, 4, F32, 9, None, 0, None) == ops.SV_ERR_INVALID_ARG
    # null required pointers
    assert lib.sv_sparseconv2d_fwd(None, FAKE, FAKE, None, FAKE, 8, 4, 4, F32, 0, None, 0, None) == ops.SV_ERR_INVALID_ARG
    assert lib.sv_sparseconv2d_bwd_dx(FAKE, None, FAKE, FAKE, 8, 4, 4, F32, 0, None, 0, None) == ops.SV_ERR_INVALID_ARG
    # MFMA forced where it does not fit: fp32, or channels not multiples of 32/16
    assert lib.sv_sparseconv2d_fwd(FAKE, FAKE, FAKE, None, FAKE, 8, 64, 64, F32, 2, None, 0, None) == ops.SV_ERR_UNSUPPORTED
    assert lib.sv_sparseconv2d_fwd(FAKE, FAKE, FAKE, None, FAKE, 8, 48, 64, BF16, 2, None, 0, None) == ops.SV_ERR_UNSUPPORTED
    assert lib.sv_sparseconv2d_bwd_dx(FAKE, FAKE, FAKE, FAKE, 8, 64, 40, BF16, 2, None, 0, None) == ops.SV_ERR_UNSUPPORTED
    # the matrix-core kernels read their operands through 32-bit buffer offsets: 2 GiB at most
    # (2^22 tokens of 256 bf16 channels is exactly that; one token more is refused when MFMA is forced)
    lim = 1 << 22
    assert lib.sv_workspace_bytes(ops.SV_OP_FWD, lim, 256, 256, BF16) > 0
    assert lib.sv_sparseconv2d_fwd(FAKE, FAKE, FAKE, None, FAKE, lim + 1, 256, 256, BF16, 2, None, 0,
                                   None) == ops.SV_ERR_UNSUPPORTED
    assert lib.sv_sparseconv2d_bwd_dx(FAKE, FAKE, FAKE, FAKE, lim + 1, 256, 256, BF16, 2, None, 0,
                                      None) == ops.SV_ERR_UNSUPPORTED
    # forward on the matrix cores without its weight workspace
    assert lib.sv_sparseconv2d_fwd(FAKE, FAKE, FAKE, None, FAKE, 8, 64, 64, BF16, 0, None, 0, None) == ops.SV_ERR_WORKSPACE
    assert lib.sv_workspace_bytes(ops.SV_OP_FWD, 8, 64, 64, BF16) >= 9 * 64 * 64 * 2
    assert lib.sv_workspace_bytes(ops.SV_OP_FWD, 8, 64, 64, F32) == 0
    # grid larger than the LDS map
    assert lib.sv_build_index(FAKE, FAKE, 1, 129, 128, 1, FAKE, None, None, None) == ops.SV_ERR_UNSUPPORTED
    assert lib.sv_build_index(FAKE, None, 1, 4, 4, 1, FAKE, None, None, None) == ops.SV_ERR_INVALID_ARG
    assert lib.sv_build_index(FAKE, FAKE, -1, 4, 4, 1, FAKE, None, None, None) == ops.SV_ERR_INVALID_ARG
    # dW workspace missing / too small
    need = lib.sv_workspace_bytes(ops.SV_OP_DW, 22656, 256, 256, BF16)
    assert need > 0
    assert lib.sv_sparseconv2d_bwd_dw(FAKE, FAKE, FAKE, FAKE, None, 22656, 256, 256, BF16, 0,
                                      None, 0, None) == ops.SV_ERR_WORKSPACE
    assert lib.sv_sparseconv2d_bwd_dw(FAKE, FAKE, FAKE, FAKE, None, 22656, 256, 256, BF16, 0,
                                      FAKE, need - 1, None) == ops.SV_ERR_WORKSPACE
    # stage copies
    assert lib.sv_stage_gather(FAKE, 10, FAKE, 5, FAKE, 0, BF16, None) == ops.SV_ERR_INVALID_ARG
    assert lib.sv_stage_scatter(FAKE, FAKE, -1, FAKE, 10, 4, BF16, None) == ops.SV_ERR_INVALID_ARG


def test_workspace_sizes(lib):
    assert lib.sv_workspace_bytes(ops.SV_OP_DX, 1000, 64, 64, ops.SV_BF16) == 0
    assert lib.sv_workspace_bytes(ops.SV_OP_DW, -1, 64, 64, ops.SV_BF16) == 0
    # bounded: never more than 64 slices of partials plus db partials
    for n, C in [(0, 64), (100, 64), (22656, 256), (22656, 512), (181248, 128), (10 ** 7, 256)]:
        b = lib.sv_workspace_bytes(ops.SV_OP_DW, n, C, C, ops.SV_BF16)
        assert b <= 64 * 9 * C * C * 4 + 64 * C * 4 + 512


def _desc(T, offs_h, C=128, chunk=256):
    d = ops.ChunkedDesc()
    d.T, d.H, d.W, d.C_in, d.C_out = T, 14, 14, C, C
    d.dtype, d.kernel, d.chunk_frames = ops.SV_BF16, ops.SV_KERNEL_AUTO, chunk
    d.frame_offsets_host = offs_h.ctypes.data
    return d


def test_chunked_workspace_flat_in_T(lib):
    """The chunk driver's workspace depends on the largest chunk, not on the
    video length: 256 frames and 3072 frames need the same bytes."""
    passes = ops.SV_PASS_FWD | ops.SV_PASS_DX | ops.SV_PASS_DW
    sizes = []
    for T in (256, 768, 3072):
        offs = (np.arange(T + 1, dtype=np.int32) * 59).astype(np.int32)
        d = _desc(T, offs)
        sizes.append(lib.sv_chunked_workspace_bytes(ctypes.byref(d), passes))
    assert sizes[0] > 0 and sizes[0] == sizes[1] == sizes[2]
    # bad descriptors: decreasing offsets, zero chunk size
    offs = np.array([0, 5, 3], dtype=np.int32)
    assert lib.sv_chunked_workspace_bytes(ctypes.byref(_desc(2, offs)), passes) == 0
    offs = np.array([0, 5, 9], dtype=np.int32)
    assert lib.sv_chunked_workspace_bytes(ctypes.byref(_desc(2, offs, chunk=0)), passes) == 0
    assert lib.sv_sparseconv2d_chunked(ctypes.byref(_desc(2, offs, chunk=0)), passes, None, 0, None) \
        == ops.SV_ERR_INVALID_ARG


def test_chunked_workspace_without_host_offsets(lib):
    """Without a host copy of the offsets the workspace is sized for chunks
    of full frames: at least what any actual offsets need."""
    rng = np.random.default_rng(4)
    for C, K, dt, chunk in [(128, 3, ops.SV_BF16, 256), (256, 3, ops.SV_BF16, 8), (64, 5, ops.SV_F32, 3),
                            (512, 3, ops.SV_BF16, 1), (128, 1, ops.SV_BF16, 40)]:
        for passes in (ops.SV_PASS_FWD | ops.SV_PASS_DX | ops.SV_PASS_DW, ops.SV_PASS_DW, ops.SV_PASS_FWD):
            T = 300
            none = _desc(T, np.zeros(1, np.int32), C=C, chunk=chunk)
            none.frame_offsets_host = None
            none.dtype, none.ksize = dt, K
            bound = lib.sv_chunked_workspace_bytes(ctypes.byref(none), passes)
            assert bound > 0
            for keep in (1.0, 0.5, 0.05):
                counts = rng.binomial(196, keep, size=T).astype(np.int32)
                offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
                d = _desc(T, offs, C=C, chunk=chunk)
                d.dtype, d.ksize = dt, K
                exact = lib.sv_chunked_workspace_bytes(ctypes.byref(d), passes)
                assert 0 < exact <= bound, (C, K, chunk, passes, keep, exact, bound)
            # every frame full: the bound's token count is reached
            full_offs = (np.arange(T + 1) * 196).astype(np.int32)     # referenced: the descriptor holds a raw pointer
            full = _desc(T, full_offs, C=C, chunk=chunk)
            full.dtype, full.ksize = dt, K
            if not passes & ops.SV_PASS_DW:
                assert lib.sv_chunked_workspace_bytes(ctypes.byref(full), passes) == bound


def test_chunked_dw_stream_workspace(lib):
    """With a dW stream the workspace holds a second N table (4 * 9 bytes
    per token of the largest chunk, rounded up), and only when the dW pass
    runs beside a forward or input-gradient pass."""
    T = 512
    offs = (np.arange(T + 1, dtype=np.int32) * 59).astype(np.int32)
    d = _desc(T, offs)
    full = ops.SV_PASS_FWD | ops.SV_PASS_DX | ops.SV_PASS_DW
    one = {p: lib.sv_chunked_workspace_bytes(ctypes.byref(d), p) for p in (full, ops.SV_PASS_DW)}
    d.dw_stream = 1     # any non-null handle: only the layout is computed here
    two = {p: lib.sv_chunked_workspace_bytes(ctypes.byref(d), p) for p in (full, ops.SV_PASS_DW)}
    ntab = (256 * 59 * 9 * 4 + 255) // 256 * 256
    assert two[full] == one[full] + ntab
    assert two[ops.SV_PASS_DW] == one[ops.SV_PASS_DW]


def test_workloads_shapes():
    """The synthetic workloads have the sizes the configurations state."""
    assert wl.make_layer("c1").n == 98
    L = wl.make_layer("c2", scale_T=8)
    assert np.all(np.diff(L.frame_offsets) == 78)
    L = wl.make_layer("c3a", scale_T=8)
    assert np.all(np.diff(L.frame_offsets) == 59)
    x = L.X.view(np.uint32)
    assert np.all((x & 0xFFFF) == 0), "bf16 inputs must be bf16-representable"
    S = wl.make_staged("c5", scale_T=16)
    c = [np.diff(s["frame_offsets"]) for s in S.stages]
    assert np.all(c[0] >= 128) and np.all(c[0] <= 180)
    assert np.all(c[1] <= c[0]) and np.all(c[2] <= c[1])
    # nesting: stage s+1 coordinates are a subset of stage s, per frame
    for s in (1, 2):
        prev, cur = S.stages[s - 1], S.stages[s]
        assert np.array_equal(prev["coords"][cur["sel"]], cur["coords"])


def test_chunked_host_validation_and_workspace(lib):
    """Host-streamed driver: workspace flat in T and at least the device
    driver's; distinct streams required; short workspace rejected (all
    before any HIP work)."""
    passes = ops.SV_PASS_FWD | ops.SV_PASS_DX | ops.SV_PASS_DW
    sizes = []
    for T in (256, 768, 3072):
        offs = (np.arange(T + 1, dtype=np.int32) * 59).astype(np.int32)
        d = ops.ChunkedHostDesc()
        d.T, d.H, d.W, d.C_in, d.C_out = T, 14, 14, 128, 128
        d.dtype, d.kernel, d.chunk_frames = ops.SV_BF16, ops.SV_KERNEL_AUTO, 256
        d.frame_offsets_host = offs.ctypes.data
        sizes.append(lib.sv_chunked_host_workspace_bytes(ctypes.byref(d), passes))
        assert sizes[-1] > lib.sv_chunked_workspace_bytes(ctypes.byref(_desc(T, offs)), passes)
    assert sizes[0] > 0 and sizes[0] == sizes[1] == sizes[2]
    # same stream twice; then a missing workspace
    d.coords_host = d.X_host = d.Y_host = d.dY_host = d.dX_host = 4096
    d.Wt = d.dW = 4096
    assert lib.sv_sparseconv2d_chunked_host(ctypes.byref(d), passes, None, 0, FAKE, FAKE, ctypes.c_void_p(8192)) \
        == ops.SV_ERR_INVALID_ARG
    assert lib.sv_sparseconv2d_chunked_host(ctypes.byref(d), passes, None, 0, FAKE, ctypes.c_void_p(8192),
                                            ctypes.c_void_p(12288)) == ops.SV_ERR_WORKSPACE
    assert lib.sv_sparseconv2d_chunked_host(ctypes.byref(d), 8, None, 0, FAKE, ctypes.c_void_p(8192),
                                            ctypes.c_void_p(12288)) == ops.SV_ERR_INVALID_ARG
    d.dX_host = None
    assert lib.sv_sparseconv2d_chunked_host(ctypes.byref(d), passes, None, 0, FAKE, ctypes.c_void_p(8192),
                                            ctypes.c_void_p(12288)) == ops.SV_ERR_INVALID_ARG


def test_xattn_validation_and_workspace(lib):
    F32, BF16 = ops.SV_F32, ops.SV_BF16
    ws = lib.sv_xattn_workspace_bytes
    # unsupported head width, negative sizes, too many queries, bad dtype
    assert lib.sv_xattn_fwd(FAKE, FAKE, 1, 8, 96, 0.0, BF16, FAKE, FAKE, FAKE, 1 << 20, None) == ops.SV_ERR_UNSUPPORTED
    assert lib.sv_xattn_fwd(FAKE, FAKE, -1, 8, 64, 0.0, BF16, FAKE, FAKE, FAKE, 1 << 20, None) == ops.SV_ERR_INVALID_ARG
    assert lib.sv_xattn_fwd(FAKE, FAKE, 70000, 8, 64, 0.0, BF16, FAKE, FAKE, FAKE, 1 << 20, None) == ops.SV_ERR_INVALID_ARG
    assert lib.sv_xattn_fwd(FAKE, FAKE, 1, 8, 64, 0.0, 5, FAKE, FAKE, FAKE, 1 << 20, None) == ops.SV_ERR_INVALID_ARG
    # null pointers, misaligned rows, a non-finite scale
    assert lib.sv_xattn_fwd(None, FAKE, 1, 8, 64, 0.0, F32, FAKE, FAKE, FAKE, 1 << 20, None) == ops.SV_ERR_INVALID_ARG
    assert lib.sv_xattn_fwd(FAKE, ctypes.c_void_p(4100), 1, 8, 64, 0.0, F32, FAKE, FAKE, FAKE, 1 << 20,
                            None) == ops.SV_ERR_INVALID_ARG
    assert lib.sv_xattn_fwd(FAKE, FAKE, 1, 8, 64, float("inf"), F32, FAKE, FAKE, FAKE, 1 << 20,
                            None) == ops.SV_ERR_INVALID_ARG
    # short workspace
    need = ws(0, 3, 50000, 256)
    assert need > 0
    assert lib.sv_xattn_fwd(FAKE, FAKE, 3, 50000, 256, 0.0, BF16, FAKE, FAKE, FAKE, need - 1,
                            None) == ops.SV_ERR_WORKSPACE
    needb = ws(1, 3, 50000, 256)
    assert lib.sv_xattn_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, 3, 50000, 256, 0.0, BF16, FAKE, FAKE, FAKE, needb - 1,
                            None) == ops.SV_ERR_WORKSPACE
    assert lib.sv_xattn_bwd(FAKE, FAKE, FAKE, None, FAKE, 3, 50000, 256, 0.0, BF16, FAKE, FAKE, FAKE, needb,
                            None) == ops.SV_ERR_INVALID_ARG
    # nothing to do: no queries and no keys
    assert lib.sv_xattn_fwd(None, None, 0, 0, 64, 0.0, BF16, None, None, None, 0, None) == ops.SV_OK
    assert lib.sv_xattn_bwd(None, None, None, None, None, 0, 0, 64, 0.0, BF16, None, None, None, 0,
                            None) == ops.SV_OK
    # workspace: block partials only, bounded by ~512 blocks whatever n
    assert ws(0, 1, 10, 100) == 0
    for m, n, d in [(1, 1, 64), (1, 58822, 256), (4, 181248, 128), (16, 10 ** 7, 256)]:
        assert ws(0, m, n, d) <= 520 * m * (d + 2) * 4 + 1024
        assert ws(1, m, n, d) <= 520 * m * (d + 1) * 4 + 512


def test_kxk_validation_and_workspace(lib):
    """K x K entry points: K even or < 1 is an argument error, odd K > 7
    unsupported; workspace sizes scale with K*K and the K = 3 forms size
    exactly as the 3 x 3 calls."""
    F32, BF16 = ops.SV_F32, ops.SV_BF16
    for K, want in [(0, ops.SV_ERR_INVALID_ARG), (4, ops.SV_ERR_INVALID_ARG), (-3, ops.SV_ERR_INVALID_ARG),
                    (9, ops.SV_ERR_UNSUPPORTED)]:
        assert lib.sv_build_index_k(FAKE, FAKE, 1, 4, 4, K, 1, FAKE, None, None, None) == want
        assert lib.sv_sparseconv2d_fwd_k(FAKE, FAKE, FAKE, None, FAKE, 8, K, 4, 4, F32, 0, None, 0, None) == want
        assert lib.sv_sparseconv2d_bwd_dx_k(FAKE, FAKE, FAKE, FAKE, 8, K, 4, 4, F32, 0, None, 0, None) == want
        assert lib.sv_sparseconv2d_bwd_dw_k(FAKE, FAKE, FAKE, FAKE, None, 8, K, 4, 4, F32, 0, None, 0,
                                            None) == want
        assert lib.sv_workspace_bytes_k(ops.SV_OP_FWD, 8, K, 64, 64, BF16) == 0
    # rows beyond 2^31 / (K*K)
    assert lib.sv_sparseconv2d_fwd_k(FAKE, FAKE, FAKE, None, FAKE, (2 ** 31) // 49 + 1, 7, 4, 4, F32, 0, None, 0,
                                     None) == ops.SV_ERR_INVALID_ARG
    # the MFMA forward needs K*K repacked weight taps
    for K in (1, 3, 5, 7):
        b = lib.sv_workspace_bytes_k(ops.SV_OP_FWD, 8, K, 64, 64, BF16)
        assert K * K * 64 * 64 * 2 <= b < K * K * 64 * 64 * 2 + 256
        assert lib.sv_sparseconv2d_fwd_k(FAKE, FAKE, FAKE, None, FAKE, 8, K, 64, 64, BF16, 0, None, 0,
                                         None) == ops.SV_ERR_WORKSPACE
    for op in (ops.SV_OP_FWD, ops.SV_OP_DX, ops.SV_OP_DW):
        for n, C in [(0, 64), (22656, 256), (181248, 128)]:
            assert lib.sv_workspace_bytes_k(op, n, 3, C, C, BF16) == lib.sv_workspace_bytes(op, n, C, C, BF16)
    # dW partials stay bounded by 64 slices of K*K taps
    for K in (1, 5, 7):
        b = lib.sv_workspace_bytes_k(ops.SV_OP_DW, 22656, K, 256, 256, BF16)
        assert 0 < b <= 64 * K * K * 256 * 256 * 4 + 64 * 256 * 4 + 512
    # chunk descriptors: ksize 0 reads as 3, 5 needs more N table, 9 / 2 rejected
    passes = ops.SV_PASS_FWD | ops.SV_PASS_DX | ops.SV_PASS_DW
    offs = (np.arange(257, dtype=np.int32) * 59).astype(np.int32)
    d = _desc(256, offs)
    base = lib.sv_chunked_workspace_bytes(ctypes.byref(d), passes)
    d.ksize = 3
    assert lib.sv_chunked_workspace_bytes(ctypes.byref(d), passes) == base
    d.ksize = 5
    assert lib.sv_chunked_workspace_bytes(ctypes.byref(d), passes) > base
    d.ksize = 2
    assert lib.sv_chunked_workspace_bytes(ctypes.byref(d), passes) == 0
    assert lib.sv_sparseconv2d_chunked(ctypes.byref(d), passes, None, 0, None) == ops.SV_ERR_INVALID_ARG
    d.ksize = 9
    assert lib.sv_sparseconv2d_chunked(ctypes.byref(d), passes, None, 0, None) == ops.SV_ERR_UNSUPPORTED


def test_adapter_validation_and_workspace(lib):
    F32, BF16 = ops.SV_F32, ops.SV_BF16
    ws = lib.sv_adapter_workspace_bytes
    assert ws(0, 100, 3, 64, 0, BF16) == 0 and ws(0, 100, 4, 64, 32, BF16) == 0 and ws(1, -1, 3, 64, 32, BF16) == 0
    # forward: identity table + the largest repacked weight; backward: + dH2, dH1 and dW partials
    f = ws(0, 1000, 3, 1024, 256, BF16)
    assert 1000 * 4 + 1024 * 256 * 2 <= f <= 1000 * 4 + 9 * 256 * 256 * 2 + 1024
    b = ws(1, 58822, 3, 1024, 256, BF16)
    assert b >= 58822 * 4 + 2 * 58822 * 256 * 2
    args = (FAKE, FAKE, 8, 3, 64, 32, FAKE, None, FAKE, None, FAKE, None, FAKE, FAKE, FAKE)
    assert lib.sv_adapter_fwd(*args, BF16, 0, None, 0, None) == ops.SV_ERR_WORKSPACE
    assert lib.sv_adapter_fwd(*args, BF16, 7, FAKE, 1 << 20, None) == ops.SV_ERR_INVALID_ARG
    assert lib.sv_adapter_fwd(*args, F32, 2, FAKE, 1 << 20, None) == ops.SV_ERR_UNSUPPORTED
    bad = (FAKE, FAKE, 8, 2, 64, 32) + args[6:]
    assert lib.sv_adapter_fwd(*bad, BF16, 0, FAKE, 1 << 20, None) == ops.SV_ERR_INVALID_ARG
    assert lib.sv_adapter_fwd(FAKE, FAKE, 8, 3, 64, 32, None, None, FAKE, None, FAKE, None, FAKE, FAKE, FAKE,
                              BF16, 0, FAKE, 1 << 20, None) == ops.SV_ERR_INVALID_ARG
    bargs = (FAKE, FAKE, 8, 3, 64, 32, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE,
             None)
    assert lib.sv_adapter_bwd(*bargs, BF16, 0, None, 0, None, None) == ops.SV_ERR_WORKSPACE
    assert lib.sv_adapter_bwd(*bargs, BF16, 0, ctypes.c_void_p(4097), 1 << 30, None, None) == ops.SV_ERR_INVALID_ARG
    nodw = bargs[:13] + (None,) + bargs[14:]
    assert lib.sv_adapter_bwd(*nodw, BF16, 0, FAKE, 1 << 30, None, None) == ops.SV_ERR_INVALID_ARG


def test_repack_layers_validation(lib):
    F32, BF16 = ops.SV_F32, ops.SV_BF16
    f = lib.sv_repack_layers_k
    arr = lambda k, v=4096: (ctypes.c_void_p * k)(*([v] * k))
    need = lib.sv_workspace_bytes_k(ops.SV_OP_FWD, 8, 3, 256, 256, BF16)
    assert f(0, arr(1), arr(1), need, arr(1), need, 3, 256, 256, BF16, None) == ops.SV_ERR_INVALID_ARG
    assert f(17, arr(17), arr(17), need, arr(17), need, 3, 256, 256, BF16, None) == ops.SV_ERR_INVALID_ARG
    assert f(2, None, arr(2), need, arr(2), need, 3, 256, 256, BF16, None) == ops.SV_ERR_INVALID_ARG
    assert f(2, arr(2), arr(2), need, arr(2), need, 3, 256, 256, F32, None) == ops.SV_ERR_UNSUPPORTED
    assert f(2, arr(2), arr(2), need - 1, arr(2), need, 3, 256, 256, BF16, None) == ops.SV_ERR_WORKSPACE
    assert f(2, arr(2), arr(2), need, arr(2), need - 1, 3, 256, 256, BF16, None) == ops.SV_ERR_WORKSPACE
    assert f(2, arr(2), arr(2, 4100), need, None, 0, 3, 256, 256, BF16, None) == ops.SV_ERR_INVALID_ARG
    # input-gradient layout needs C_in a multiple of 128
    assert f(2, arr(2), None, 0, arr(2), need, 3, 192, 192, BF16, None) == ops.SV_ERR_UNSUPPORTED
    assert f(2, arr(2), arr(2), need, arr(2), need, 4, 256, 256, BF16, None) == ops.SV_ERR_INVALID_ARG


def test_noalloc_validation(lib):
    """The allocation-free weight gradient checks its arguments and the
    size of its partials before it touches a device."""
    F32, BF16 = ops.SV_F32, ops.SV_BF16
    f = lib.sv_sparseconv2d_bwd_dw_noalloc_k
    assert f(FAKE, FAKE, FAKE, FAKE, None, -1, 3, 4, 4, F32, 0, None) == ops.SV_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, None, 8, 4, 4, 4, F32, 0, None) == ops.SV_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, None, 8, 9, 4, 4, F32, 0, None) == ops.SV_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, None, None, 8, 3, 4, 4, F32, 0, None) == ops.SV_ERR_INVALID_ARG
    assert f(FAKE, None, FAKE, FAKE, None, 8, 3, 4, 4, F32, 0, None) == ops.SV_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, None, 8, 3, 4, 4, 7, 0, None) == ops.SV_ERR_INVALID_ARG
    # a 5 x 5 layer with 2M tokens: the planner splits the tokens into
    # several dispatch rounds of slices, whose partials exceed the array
    big = 2_000_000
    assert lib.sv_workspace_bytes_k(ops.SV_OP_DW, big, 5, 512, 512, BF16) > ops.SV_NOALLOC_SCRATCH_BYTES
    assert f(FAKE, FAKE, FAKE, FAKE, None, big, 5, 512, 512, BF16, 0, None) == ops.SV_ERR_WORKSPACE


def test_split_forms_validation(lib):
    F32, BF16 = ops.SV_F32, ops.SV_BF16
    need = lib.sv_workspace_bytes_k(ops.SV_OP_FWD, 8, 3, 64, 64, BF16)
    assert lib.sv_repack_fwd_k(FAKE, 3, 64, 64, F32, FAKE, need, None) == ops.SV_ERR_UNSUPPORTED
    assert lib.sv_repack_fwd_k(FAKE, 3, 64, 64, BF16, FAKE, need - 1, None) == ops.SV_ERR_WORKSPACE
    assert lib.sv_repack_fwd_k(FAKE, 4, 64, 64, BF16, FAKE, need, None) == ops.SV_ERR_INVALID_ARG
    assert lib.sv_repack_fwd_k(None, 3, 64, 64, BF16, FAKE, need, None) == ops.SV_ERR_INVALID_ARG
    # the packed forward runs only on the matrix cores
    assert lib.sv_sparseconv2d_fwd_packed_k(FAKE, FAKE, FAKE, None, FAKE, 8, 3, 48, 64, BF16, None) == \
        ops.SV_ERR_UNSUPPORTED
    assert lib.sv_sparseconv2d_fwd_packed_k(FAKE, FAKE, FAKE, None, FAKE, 8, 3, 64, 64, F32, None) == \
        ops.SV_ERR_UNSUPPORTED
    assert lib.sv_sparseconv2d_fwd_packed_k(FAKE, FAKE, None, None, FAKE, 8, 3, 64, 64, BF16, None) == \
        ops.SV_ERR_INVALID_ARG
    # input gradient in fragment order: bf16 3 x 3, 5 x 5, 7 x 7 with C_out % 64 == 0 and C_in % 128 == 0
    xneed = lib.sv_workspace_bytes_k(ops.SV_OP_DX, 22656, 3, 256, 256, BF16)
    assert xneed == 9 * 256 * 256 * 2
    assert lib.sv_workspace_bytes(ops.SV_OP_DX, 22656, 256, 256, BF16) == xneed
    assert lib.sv_workspace_bytes_k(ops.SV_OP_DX, 22656, 3, 128, 128, BF16) == 9 * 128 * 128 * 2
    assert lib.sv_workspace_bytes_k(ops.SV_OP_DX, 22656, 3, 192, 192, BF16) == 0
    assert lib.sv_workspace_bytes_k(ops.SV_OP_DX, 22656, 3, 256, 256, F32) == 0
    assert lib.sv_workspace_bytes_k(ops.SV_OP_DX, 22656, 5, 256, 256, BF16) == 25 * 256 * 256 * 2
    assert lib.sv_workspace_bytes_k(ops.SV_OP_DX, 22656, 7, 128, 256, BF16) == 49 * 128 * 256 * 2
    assert lib.sv_workspace_bytes_k(ops.SV_OP_DX, 22656, 1, 256, 256, BF16) == 0     # 1 x 1: from 512
    assert lib.sv_workspace_bytes_k(ops.SV_OP_DX, 22656, 1, 256, 512, BF16) == 512 * 256 * 2
    assert lib.sv_sparseconv2d_bwd_dx(FAKE, FAKE, FAKE, FAKE, 22656, 256, 256, BF16, 0, FAKE, xneed - 1,
                                      None) == ops.SV_ERR_WORKSPACE
    assert lib.sv_repack_dx_k(FAKE, 3, 256, 256, BF16, FAKE, xneed - 1, None) == ops.SV_ERR_WORKSPACE
    assert lib.sv_repack_dx_k(FAKE, 3, 192, 192, BF16, FAKE, xneed, None) == ops.SV_ERR_UNSUPPORTED
    assert lib.sv_repack_dx_k(FAKE, 3, 256, 256, F32, FAKE, xneed, None) == ops.SV_ERR_UNSUPPORTED
    assert lib.sv_repack_dx_k(None, 3, 256, 256, BF16, FAKE, xneed, None) == ops.SV_ERR_INVALID_ARG
    assert lib.sv_repack_dx_k(FAKE, 3, 256, 256, BF16, ctypes.c_void_p(4104), xneed, None) == \
        ops.SV_ERR_INVALID_ARG
    assert lib.sv_sparseconv2d_bwd_dx_packed_k(FAKE, FAKE, FAKE, FAKE, 8, 3, 192, 192, BF16, None) == \
        ops.SV_ERR_UNSUPPORTED
    assert lib.sv_sparseconv2d_bwd_dx_packed_k(FAKE, FAKE, None, FAKE, 8, 3, 256, 256, BF16, None) == \
        ops.SV_ERR_INVALID_ARG
    dneed = lib.sv_workspace_bytes_k(ops.SV_OP_DW, 22656, 3, 256, 256, BF16)
    assert lib.sv_sparseconv2d_bwd_dw_partials_k(FAKE, FAKE, FAKE, FAKE, None, 22656, 3, 256, 256, BF16, 0, FAKE,
                                                 dneed - 1, None) == ops.SV_ERR_WORKSPACE
    assert lib.sv_sparseconv2d_bwd_dw_reduce_k(FAKE, None, 22656, 3, 256, 256, BF16, 0, FAKE, dneed - 1,
                                               None) == ops.SV_ERR_WORKSPACE
    assert lib.sv_sparseconv2d_bwd_dw_reduce_k(None, None, 22656, 3, 256, 256, BF16, 0, FAKE, dneed,
                                               None) == ops.SV_ERR_INVALID_ARG
    assert lib.sv_sparseconv2d_bwd_dw_partials_k(FAKE, FAKE, FAKE, FAKE, None, 22656, 6, 256, 256, BF16, 0, FAKE,
                                                 dneed, None) == ops.SV_ERR_INVALID_ARG
