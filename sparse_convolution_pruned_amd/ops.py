"""ctypes binding over libsvconv (include/svconv.h).

Argument marshalling only: every function here takes torch tensors that
already live on the GPU, checks dtype/shape/contiguity, passes raw device
pointers plus the current HIP stream to the C entry point of the same name,
and raises ``SvError`` on a non-OK status.  All arithmetic runs in the HIP
kernels.  If the library is missing or cannot be loaded the first call
raises -- there is no fallback.

Layouts (row-major, contiguous), as in the C header:
  coords int32 [n], frame_offsets int32 [T+1], N int32 [n, 9],
  X [n, C_in], Y [n, C_out], Wt [9, C_in, C_out], bias [C_out],
  dW fp32 [9, C_in, C_out], db fp32 [C_out].
The ``_k`` entry points take a K x K neighbourhood (K odd, 1..7): N has
K*K columns and Wt, dW K*K taps.  The conveniences at the end infer K from
the shapes.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsvconv.so")

SV_OK, SV_ERR_INVALID_ARG, SV_ERR_UNSUPPORTED, SV_ERR_WORKSPACE, SV_ERR_HIP = 0, 1, 2, 3, 4
SV_ERR_COORD_RANGE, SV_ERR_DUPLICATE_COORD = 5, 6
SV_F32, SV_BF16 = 0, 1
SV_KERNEL_AUTO, SV_KERNEL_VALU, SV_KERNEL_MFMA = 0, 1, 2
SV_FLAG_COORD_RANGE, SV_FLAG_DUPLICATE, SV_FLAG_BAD_OFFSETS = 1, 2, 4
SV_PASS_FWD, SV_PASS_DX, SV_PASS_DW = 1, 2, 4
SV_OP_FWD, SV_OP_DX, SV_OP_DW = 0, 1, 2

KERNELS = {"auto": SV_KERNEL_AUTO, "valu": SV_KERNEL_VALU, "mfma": SV_KERNEL_MFMA}

# Exported symbols, in header order.
SYMBOLS = (
    "sv_build_index", "sv_sparseconv2d_fwd", "sv_sparseconv2d_bwd_dx",
    "sv_sparseconv2d_bwd_dw", "sv_workspace_bytes",
    "sv_build_index_k", "sv_sparseconv2d_fwd_k", "sv_sparseconv2d_bwd_dx_k",
    "sv_sparseconv2d_bwd_dw_k", "sv_workspace_bytes_k",
    "sv_repack_fwd_k", "sv_sparseconv2d_fwd_packed_k", "sv_repack_dx_k", "sv_repack_layers_k", "sv_sparseconv2d_bwd_dx_packed_k",
    "sv_sparseconv2d_bwd_dw_partials_k",
    "sv_sparseconv2d_bwd_dw_reduce_k", "sv_sparseconv2d_chunked",
    "sv_chunked_workspace_bytes", "sv_sparseconv2d_chunked_host", "sv_chunked_host_workspace_bytes",
    "sv_adapter_fwd", "sv_adapter_bwd", "sv_adapter_workspace_bytes",
    "sv_stage_gather", "sv_stage_scatter", "sv_status_string", "sv_version",
    "sv_xattn_fwd", "sv_xattn_bwd", "sv_xattn_workspace_bytes",
    "sv_sparseconv2d_bwd_dw_noalloc_k",
)
SV_NOALLOC_SCRATCH_BYTES = 64 << 20


class SvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


class ChunkedDesc(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int32), ("H", ctypes.c_int32), ("W", ctypes.c_int32),
        ("C_in", ctypes.c_int32), ("C_out", ctypes.c_int32),
        ("dtype", ctypes.c_int), ("kernel", ctypes.c_int),
        ("chunk_frames", ctypes.c_int32),
        ("coords", ctypes.c_void_p), ("frame_offsets", ctypes.c_void_p),
        ("frame_offsets_host", ctypes.c_void_p),
        ("X", ctypes.c_void_p), ("Wt", ctypes.c_void_p), ("bias", ctypes.c_void_p),
        ("Y", ctypes.c_void_p), ("dY", ctypes.c_void_p), ("dX", ctypes.c_void_p),
        ("dW", ctypes.c_void_p), ("db", ctypes.c_void_p), ("err_flag", ctypes.c_void_p),
        ("ksize", ctypes.c_int32),
        ("dw_stream", ctypes.c_void_p),
    ]


class ChunkedHostDesc(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int32), ("H", ctypes.c_int32), ("W", ctypes.c_int32),
        ("C_in", ctypes.c_int32), ("C_out", ctypes.c_int32),
        ("dtype", ctypes.c_int), ("kernel", ctypes.c_int),
        ("chunk_frames", ctypes.c_int32),
        ("coords_host", ctypes.c_void_p), ("frame_offsets_host", ctypes.c_void_p),
        ("X_host", ctypes.c_void_p), ("Wt", ctypes.c_void_p), ("bias", ctypes.c_void_p),
        ("Y_host", ctypes.c_void_p), ("dY_host", ctypes.c_void_p), ("dX_host", ctypes.c_void_p),
        ("dW", ctypes.c_void_p), ("db", ctypes.c_void_p), ("err_flag", ctypes.c_void_p),
        ("ksize", ctypes.c_int32),
    ]


_lib = None


def load(path: str = LIB_PATH):
    """Open libsvconv.so and declare its signatures.  torch is imported
    first so that the library binds to the HIP runtime torch already
    loaded (same soname)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libsvconv.so not built ({path}); run "
                           "`python -m sparse_convolution_pruned_amd.build`")
    lib = ctypes.CDLL(path)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    E = ctypes.c_int
    sig = {
        "sv_build_index": ([P, P, i32, i32, i32, i64, P, P, P, P], E),
        "sv_sparseconv2d_fwd": ([P, P, P, P, P, i64, i32, i32, E, E, P, sz, P], E),
        "sv_sparseconv2d_bwd_dx": ([P, P, P, P, i64, i32, i32, E, E, P, sz, P], E),
        "sv_sparseconv2d_bwd_dw": ([P, P, P, P, P, i64, i32, i32, E, i32, P, sz, P], E),
        "sv_workspace_bytes": ([E, i64, i32, i32, E], sz),
        "sv_build_index_k": ([P, P, i32, i32, i32, i32, i64, P, P, P, P], E),
        "sv_sparseconv2d_fwd_k": ([P, P, P, P, P, i64, i32, i32, i32, E, E, P, sz, P], E),
        "sv_sparseconv2d_bwd_dx_k": ([P, P, P, P, i64, i32, i32, i32, E, E, P, sz, P], E),
        "sv_sparseconv2d_bwd_dw_k": ([P, P, P, P, P, i64, i32, i32, i32, E, i32, P, sz, P], E),
        "sv_workspace_bytes_k": ([E, i64, i32, i32, i32, E], sz),
        "sv_repack_fwd_k": ([P, i32, i32, i32, E, P, sz, P], E),
        "sv_sparseconv2d_fwd_packed_k": ([P, P, P, P, P, i64, i32, i32, i32, E, P], E),
        "sv_repack_dx_k": ([P, i32, i32, i32, E, P, sz, P], E),
        "sv_repack_layers_k": ([i32, P, P, sz, P, sz, i32, i32, i32, E, P], E),
        "sv_sparseconv2d_bwd_dx_packed_k": ([P, P, P, P, i64, i32, i32, i32, E, P], E),
        "sv_sparseconv2d_bwd_dw_partials_k": ([P, P, P, P, P, i64, i32, i32, i32, E, i32, P, sz, P], E),
        "sv_sparseconv2d_bwd_dw_reduce_k": ([P, P, i64, i32, i32, i32, E, i32, P, sz, P], E),
        "sv_sparseconv2d_chunked": ([ctypes.POINTER(ChunkedDesc), ctypes.c_uint32, P, sz, P], E),
        "sv_chunked_workspace_bytes": ([ctypes.POINTER(ChunkedDesc), ctypes.c_uint32], sz),
        "sv_sparseconv2d_chunked_host": ([ctypes.POINTER(ChunkedHostDesc), ctypes.c_uint32, P, sz, P, P, P], E),
        "sv_chunked_host_workspace_bytes": ([ctypes.POINTER(ChunkedHostDesc), ctypes.c_uint32], sz),
        "sv_stage_gather": ([P, i64, P, i64, P, i32, E, P], E),
        "sv_stage_scatter": ([P, P, i64, P, i64, i32, E, P], E),
        "sv_xattn_fwd": ([P, P, i64, i64, i32, ctypes.c_float, E, P, P, P, sz, P], E),
        "sv_xattn_bwd": ([P, P, P, P, P, i64, i64, i32, ctypes.c_float, E, P, P, P, sz, P], E),
        "sv_xattn_workspace_bytes": ([i32, i64, i64, i32], sz),
        "sv_adapter_fwd": ([P, P, i64, i32, i32, i32, P, P, P, P, P, P, P, P, P, E, E, P, sz, P], E),
        "sv_adapter_bwd": ([P, P, i64, i32, i32, i32, P, P, P, P, P, P, P, P, P, P, P, P, P, E, E, P, sz, P, P], E),
        "sv_adapter_workspace_bytes": ([i32, i64, i32, i32, i32, E], sz),
        "sv_sparseconv2d_bwd_dw_noalloc_k": ([P, P, P, P, P, i64, i32, i32, i32, E, i32, P], E),
        "sv_status_string": ([E], ctypes.c_char_p),
        "sv_version": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().sv_status_string(int(status)).decode()


def version() -> str:
    return load().sv_version().decode()


# ------------------------------------------------------------------ helpers
def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SV_F32
    if t.dtype == torch.bfloat16:
        return SV_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr() if t.numel() > 0 else None


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(st: int, where: str):
    if st != SV_OK:
        raise SvError(st, where)


def _kernel(kernel) -> int:
    return KERNELS[kernel] if isinstance(kernel, str) else int(kernel)


# ------------------------------------------------------------- entry points
def sv_build_index(coords, frame_offsets, T, H, W, N_out, M_out=None, err_flag=None, stream=None):
    assert coords.dtype == torch.int32 and frame_offsets.dtype == torch.int32
    assert N_out.dtype == torch.int32 and N_out.shape == (coords.shape[0], 9)
    assert frame_offsets.shape == (T + 1,)
    if M_out is not None:
        assert M_out.dtype == torch.int32 and M_out.numel() == T * H * W
    if err_flag is not None:
        assert err_flag.dtype == torch.int32 and err_flag.numel() >= 1
    st = load().sv_build_index(_ptr(coords), _ptr(frame_offsets), int(T), int(H), int(W),
                               int(coords.shape[0]), _ptr(N_out), _ptr(M_out), _ptr(err_flag),
                               _stream(stream))
    _check(st, "sv_build_index")


def sv_sparseconv2d_fwd(X, N, Wt, bias, Y, kernel="auto", workspace=None, stream=None):
    n, Ci = X.shape
    Co = Wt.shape[2]
    assert Wt.shape == (9, Ci, Co) and Y.shape == (n, Co) and N.shape == (n, 9)
    assert X.dtype == Wt.dtype == Y.dtype and N.dtype == torch.int32
    if bias is not None:
        assert bias.dtype == X.dtype and bias.shape == (Co,)
    need = sv_workspace_bytes(SV_OP_FWD, n, Ci, Co, X.dtype)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().sv_sparseconv2d_fwd(_ptr(X), _ptr(N), _ptr(Wt), _ptr(bias), _ptr(Y), n, Ci, Co,
                                    _dt(X), _kernel(kernel), _ptr(workspace), wsb, _stream(stream))
    _check(st, "sv_sparseconv2d_fwd")


def _dx_workspace(workspace, need, device):
    """The input gradient's workspace: allocated when omitted (None), none
    at all for workspace=0 (the kernel that reads Wt directly runs)."""
    if workspace is None:
        return torch.empty(need, dtype=torch.uint8, device=device) if need > 0 else None
    if isinstance(workspace, int) and workspace == 0:
        return None
    return workspace


def sv_sparseconv2d_bwd_dx(dY, N, Wt, dX, kernel="auto", workspace=None, stream=None):
    n, Co = dY.shape
    Ci = Wt.shape[1]
    assert Wt.shape == (9, Ci, Co) and dX.shape == (n, Ci) and N.shape == (n, 9)
    assert dY.dtype == Wt.dtype == dX.dtype and N.dtype == torch.int32
    workspace = _dx_workspace(workspace, sv_workspace_bytes(SV_OP_DX, n, Ci, Co, dY.dtype), dY.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().sv_sparseconv2d_bwd_dx(_ptr(dY), _ptr(N), _ptr(Wt), _ptr(dX), n, Ci, Co,
                                       _dt(dY), _kernel(kernel), _ptr(workspace), wsb, _stream(stream))
    _check(st, "sv_sparseconv2d_bwd_dx")


def sv_workspace_bytes(op, n, C_in, C_out, dtype) -> int:
    dt = SV_BF16 if dtype in (torch.bfloat16, SV_BF16, "bf16") else SV_F32
    return int(load().sv_workspace_bytes(int(op), int(n), int(C_in), int(C_out), dt))


def sv_sparseconv2d_bwd_dw(X, N, dY, dW, db=None, accumulate=False, workspace=None, stream=None):
    n, Ci = X.shape
    Co = dY.shape[1]
    assert dY.shape[0] == n and N.shape == (n, 9) and dW.shape == (9, Ci, Co)
    assert dW.dtype == torch.float32 and X.dtype == dY.dtype
    if db is not None:
        assert db.dtype == torch.float32 and db.shape == (Co,)
    need = sv_workspace_bytes(SV_OP_DW, n, Ci, Co, X.dtype)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().sv_sparseconv2d_bwd_dw(_ptr(X), _ptr(N), _ptr(dY), _ptr(dW), _ptr(db), n, Ci, Co,
                                       _dt(X), 1 if accumulate else 0, _ptr(workspace), wsb,
                                       _stream(stream))
    _check(st, "sv_sparseconv2d_bwd_dw")


def ksize_of_taps(taps: int) -> int:
    """K of a K x K neighbourhood from its tap count (K * K, K odd)."""
    K = int(round(taps ** 0.5))
    if K * K != taps or K % 2 == 0:
        raise ValueError(f"{taps} taps is not an odd K x K neighbourhood")
    return K


def sv_build_index_k(coords, frame_offsets, T, H, W, K, N_out, M_out=None, err_flag=None, stream=None):
    assert coords.dtype == torch.int32 and frame_offsets.dtype == torch.int32
    assert N_out.dtype == torch.int32 and N_out.shape == (coords.shape[0], K * K)
    assert frame_offsets.shape == (T + 1,)
    if M_out is not None:
        assert M_out.dtype == torch.int32 and M_out.numel() == T * H * W
    if err_flag is not None:
        assert err_flag.dtype == torch.int32 and err_flag.numel() >= 1
    st = load().sv_build_index_k(_ptr(coords), _ptr(frame_offsets), int(T), int(H), int(W), int(K),
                                 int(coords.shape[0]), _ptr(N_out), _ptr(M_out), _ptr(err_flag),
                                 _stream(stream))
    _check(st, "sv_build_index_k")


def sv_workspace_bytes_k(op, n, K, C_in, C_out, dtype) -> int:
    dt = SV_BF16 if dtype in (torch.bfloat16, SV_BF16, "bf16") else SV_F32
    return int(load().sv_workspace_bytes_k(int(op), int(n), int(K), int(C_in), int(C_out), dt))


def sv_sparseconv2d_fwd_k(X, N, Wt, bias, Y, kernel="auto", workspace=None, stream=None):
    n, Ci = X.shape
    taps, Co = Wt.shape[0], Wt.shape[2]
    K = ksize_of_taps(taps)
    assert Wt.shape == (taps, Ci, Co) and Y.shape == (n, Co) and N.shape == (n, taps)
    assert X.dtype == Wt.dtype == Y.dtype and N.dtype == torch.int32
    if bias is not None:
        assert bias.dtype == X.dtype and bias.shape == (Co,)
    need = sv_workspace_bytes_k(SV_OP_FWD, n, K, Ci, Co, X.dtype)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().sv_sparseconv2d_fwd_k(_ptr(X), _ptr(N), _ptr(Wt), _ptr(bias), _ptr(Y), n, K, Ci, Co,
                                      _dt(X), _kernel(kernel), _ptr(workspace), wsb, _stream(stream))
    _check(st, "sv_sparseconv2d_fwd_k")


def sv_sparseconv2d_bwd_dx_k(dY, N, Wt, dX, kernel="auto", workspace=None, stream=None):
    n, Co = dY.shape
    taps, Ci = Wt.shape[0], Wt.shape[1]
    K = ksize_of_taps(taps)
    assert Wt.shape == (taps, Ci, Co) and dX.shape == (n, Ci) and N.shape == (n, taps)
    assert dY.dtype == Wt.dtype == dX.dtype and N.dtype == torch.int32
    workspace = _dx_workspace(workspace, sv_workspace_bytes_k(SV_OP_DX, n, K, Ci, Co, dY.dtype), dY.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().sv_sparseconv2d_bwd_dx_k(_ptr(dY), _ptr(N), _ptr(Wt), _ptr(dX), n, K, Ci, Co,
                                         _dt(dY), _kernel(kernel), _ptr(workspace), wsb, _stream(stream))
    _check(st, "sv_sparseconv2d_bwd_dx_k")


def sv_sparseconv2d_bwd_dw_k(X, N, dY, dW, db=None, accumulate=False, workspace=None, stream=None):
    n, Ci = X.shape
    Co = dY.shape[1]
    taps = dW.shape[0]
    K = ksize_of_taps(taps)
    assert dY.shape[0] == n and N.shape == (n, taps) and dW.shape == (taps, Ci, Co)
    assert dW.dtype == torch.float32 and X.dtype == dY.dtype
    if db is not None:
        assert db.dtype == torch.float32 and db.shape == (Co,)
    need = sv_workspace_bytes_k(SV_OP_DW, n, K, Ci, Co, X.dtype)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().sv_sparseconv2d_bwd_dw_k(_ptr(X), _ptr(N), _ptr(dY), _ptr(dW), _ptr(db), n, K, Ci, Co,
                                         _dt(X), 1 if accumulate else 0, _ptr(workspace), wsb,
                                         _stream(stream))
    _check(st, "sv_sparseconv2d_bwd_dw_k")


def sv_repack_fwd_k(Wt, V, stream=None):
    taps, Ci, Co = Wt.shape
    wsb = V.numel() * V.element_size()
    st = load().sv_repack_fwd_k(_ptr(Wt), ksize_of_taps(taps), Ci, Co, _dt(Wt), _ptr(V), wsb, _stream(stream))
    _check(st, "sv_repack_fwd_k")


def sv_sparseconv2d_fwd_packed_k(X, N, V, bias, Y, K, stream=None):
    n, Ci = X.shape
    Co = Y.shape[1]
    assert N.shape == (n, K * K) and Y.shape[0] == n and X.dtype == Y.dtype and N.dtype == torch.int32
    if bias is not None:
        assert bias.dtype == X.dtype and bias.shape == (Co,)
    st = load().sv_sparseconv2d_fwd_packed_k(_ptr(X), _ptr(N), _ptr(V), _ptr(bias), _ptr(Y), n, K, Ci, Co, _dt(X),
                                             _stream(stream))
    _check(st, "sv_sparseconv2d_fwd_packed_k")


def sv_sparseconv2d_bwd_dw_noalloc_k(X, N, dY, dW, db=None, accumulate=False, stream=None):
    """The weight gradient with its partials in the library's device array
    (no workspace argument, nothing allocated)."""
    n, Ci = X.shape
    Co = dY.shape[1]
    taps = dW.shape[0]
    K = ksize_of_taps(taps)
    assert dY.shape[0] == n and N.shape == (n, taps) and dW.shape == (taps, Ci, Co)
    assert dW.dtype == torch.float32 and X.dtype == dY.dtype
    if db is not None:
        assert db.dtype == torch.float32 and db.shape == (Co,)
    st = load().sv_sparseconv2d_bwd_dw_noalloc_k(_ptr(X), _ptr(N), _ptr(dY), _ptr(dW), _ptr(db), n, K, Ci, Co,
                                                 _dt(X), 1 if accumulate else 0, _stream(stream))
    _check(st, "sv_sparseconv2d_bwd_dw_noalloc_k")


def sv_repack_dx_k(Wt, P, stream=None):
    taps, Ci, Co = Wt.shape
    wsb = P.numel() * P.element_size()
    st = load().sv_repack_dx_k(_ptr(Wt), ksize_of_taps(taps), Ci, Co, _dt(Wt), _ptr(P), wsb, _stream(stream))
    _check(st, "sv_repack_dx_k")


def sv_repack_layers_k(Wts, Vs=None, Ps=None, stream=None):
    """One launch repacking every layer's weights (all of one shape) for the
    forward (Vs) and the input gradient (Ps); either list may be None."""
    count = len(Wts)
    taps, Ci, Co = Wts[0].shape
    arr = lambda ts: None if ts is None else (ctypes.c_void_p * count)(*[t.data_ptr() for t in ts])
    vb = 0 if Vs is None else min(v.numel() * v.element_size() for v in Vs)
    pb = 0 if Ps is None else min(p.numel() * p.element_size() for p in Ps)
    st = load().sv_repack_layers_k(count, arr(Wts), arr(Vs), vb, arr(Ps), pb, ksize_of_taps(taps), Ci, Co,
                                   _dt(Wts[0]), _stream(stream))
    _check(st, "sv_repack_layers_k")


def sv_sparseconv2d_bwd_dx_packed_k(dY, N, P, dX, K, stream=None):
    n, Co = dY.shape
    Ci = dX.shape[1]
    assert N.shape == (n, K * K) and dX.shape[0] == n and dY.dtype == dX.dtype and N.dtype == torch.int32
    st = load().sv_sparseconv2d_bwd_dx_packed_k(_ptr(dY), _ptr(N), _ptr(P), _ptr(dX), n, K, Ci, Co, _dt(dY),
                                                _stream(stream))
    _check(st, "sv_sparseconv2d_bwd_dx_packed_k")


def sv_sparseconv2d_bwd_dw_partials_k(X, N, dY, dW, db, workspace, accumulate=False, stream=None):
    n, Ci = X.shape
    taps, Co = dW.shape[0], dY.shape[1]
    assert dY.shape[0] == n and N.shape == (n, taps) and dW.shape == (taps, Ci, Co) and dW.dtype == torch.float32
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().sv_sparseconv2d_bwd_dw_partials_k(_ptr(X), _ptr(N), _ptr(dY), _ptr(dW), _ptr(db), n,
                                                  ksize_of_taps(taps), Ci, Co, _dt(X), 1 if accumulate else 0,
                                                  _ptr(workspace), wsb, _stream(stream))
    _check(st, "sv_sparseconv2d_bwd_dw_partials_k")


def sv_sparseconv2d_bwd_dw_reduce_k(dW, db, n, dtype, workspace, accumulate=False, stream=None):
    taps, Ci, Co = dW.shape
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    dt = SV_BF16 if dtype in (torch.bfloat16, SV_BF16, "bf16") else SV_F32
    st = load().sv_sparseconv2d_bwd_dw_reduce_k(_ptr(dW), _ptr(db), int(n), ksize_of_taps(taps), Ci, Co, dt,
                                                1 if accumulate else 0, _ptr(workspace), wsb, _stream(stream))
    _check(st, "sv_sparseconv2d_bwd_dw_reduce_k")


def make_chunked_desc(T, H, W, coords, frame_offsets, frame_offsets_host, C_in, C_out, dtype,
                      chunk_frames, X=None, Wt=None, bias=None, Y=None, dY=None, dX=None,
                      dW=None, db=None, err_flag=None, kernel="auto", ksize=3, dw_stream=None):
    """Build the descriptor; `frame_offsets_host` is a CPU int32 tensor
    (kept referenced by the returned object) or None: then the workspace is
    sized for chunks of full frames and the call copies the offsets to the
    host, waiting for that copy.  `ksize`: K of the K x K neighbourhood.
    `dw_stream`: a torch stream for the chunks' weight gradients (None:
    everything on the call's stream)."""
    fh = None
    if frame_offsets_host is not None:
        assert frame_offsets_host.device.type == "cpu" and frame_offsets_host.dtype == torch.int32
        fh = frame_offsets_host.contiguous()
    d = ChunkedDesc()
    d.T, d.H, d.W, d.C_in, d.C_out = int(T), int(H), int(W), int(C_in), int(C_out)
    d.dtype = SV_BF16 if dtype == torch.bfloat16 else SV_F32
    d.kernel = _kernel(kernel)
    d.chunk_frames = int(chunk_frames)
    d.coords, d.frame_offsets = _ptr(coords), _ptr(frame_offsets)
    d.frame_offsets_host = None if fh is None else fh.data_ptr()
    d.X, d.Wt, d.bias, d.Y = _ptr(X), _ptr(Wt), _ptr(bias), _ptr(Y)
    d.dY, d.dX, d.dW, d.db, d.err_flag = _ptr(dY), _ptr(dX), _ptr(dW), _ptr(db), _ptr(err_flag)
    d.ksize = int(ksize)
    d.dw_stream = None if dw_stream is None else dw_stream.cuda_stream
    d._keep = (fh, coords, frame_offsets, X, Wt, bias, Y, dY, dX, dW, db, err_flag, dw_stream)
    return d


def sv_chunked_workspace_bytes(desc: ChunkedDesc, passes: int) -> int:
    return int(load().sv_chunked_workspace_bytes(ctypes.byref(desc), ctypes.c_uint32(passes)))


def sv_sparseconv2d_chunked(desc: ChunkedDesc, passes: int, workspace=None, stream=None):
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().sv_sparseconv2d_chunked(ctypes.byref(desc), ctypes.c_uint32(passes),
                                        _ptr(workspace), wsb, _stream(stream))
    _check(st, "sv_sparseconv2d_chunked")


def _host_ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if t.is_cuda or not t.is_pinned():
        raise ValueError("host tensor must be in page-locked (pinned) CPU memory")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr() if t.numel() > 0 else None


def make_chunked_host_desc(T, H, W, coords_host, frame_offsets_host, C_in, C_out, dtype, chunk_frames,
                           X_host=None, Wt=None, bias=None, Y_host=None, dY_host=None, dX_host=None,
                           dW=None, db=None, err_flag=None, kernel="auto", ksize=3):
    """Descriptor of the host-streamed chunk driver: coords, frame offsets
    and the per-token tensors are pinned CPU tensors; Wt, bias, dW, db and
    err_flag live on the GPU (kept referenced by the returned object)."""
    assert frame_offsets_host.dtype == torch.int32 and coords_host.dtype == torch.int32
    d = ChunkedHostDesc()
    d.T, d.H, d.W, d.C_in, d.C_out = int(T), int(H), int(W), int(C_in), int(C_out)
    d.dtype = SV_BF16 if dtype == torch.bfloat16 else SV_F32
    d.kernel = _kernel(kernel)
    d.chunk_frames = int(chunk_frames)
    d.coords_host, d.frame_offsets_host = _host_ptr(coords_host), _host_ptr(frame_offsets_host)
    d.X_host, d.Y_host, d.dY_host, d.dX_host = _host_ptr(X_host), _host_ptr(Y_host), _host_ptr(dY_host), \
        _host_ptr(dX_host)
    d.Wt, d.bias, d.dW, d.db, d.err_flag = _ptr(Wt), _ptr(bias), _ptr(dW), _ptr(db), _ptr(err_flag)
    d.ksize = int(ksize)
    d._keep = (coords_host, frame_offsets_host, X_host, Wt, bias, Y_host, dY_host, dX_host, dW, db, err_flag)
    return d


def sv_chunked_host_workspace_bytes(desc: ChunkedHostDesc, passes: int) -> int:
    return int(load().sv_chunked_host_workspace_bytes(ctypes.byref(desc), ctypes.c_uint32(passes)))


def sv_sparseconv2d_chunked_host(desc: ChunkedHostDesc, passes: int, workspace, h2d_stream, d2h_stream,
                                 stream=None):
    """Enqueue the host-streamed driver: compute on `stream` (default: the
    current stream), copies on the two given streams.  Synchronising the
    compute stream covers the whole call."""
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().sv_sparseconv2d_chunked_host(ctypes.byref(desc), ctypes.c_uint32(passes), _ptr(workspace), wsb,
                                             _stream(stream), _stream(h2d_stream), _stream(d2h_stream))
    _check(st, "sv_sparseconv2d_chunked_host")


def sv_stage_gather(src, rows, dst, stream=None):
    C = src.shape[1]
    assert rows.dtype == torch.int32 and dst.shape == (rows.shape[0], C) and dst.dtype == src.dtype
    st = load().sv_stage_gather(_ptr(src), src.shape[0], _ptr(rows), rows.shape[0], _ptr(dst), C,
                                _dt(src), _stream(stream))
    _check(st, "sv_stage_gather")


def sv_stage_scatter(src, rows, dst, stream=None):
    C = src.shape[1]
    assert rows.dtype == torch.int32 and dst.shape[1] == C and dst.dtype == src.dtype
    st = load().sv_stage_scatter(_ptr(src), _ptr(rows), rows.shape[0], _ptr(dst), dst.shape[0], C,
                                 _dt(src), _stream(stream))
    _check(st, "sv_stage_scatter")


def sv_adapter_workspace_bytes(backward, n, K, C, r, dtype) -> int:
    dt = SV_BF16 if dtype in (torch.bfloat16, SV_BF16, "bf16") else SV_F32
    return int(load().sv_adapter_workspace_bytes(1 if backward else 0, int(n), int(K), int(C), int(r), dt))


def _adapter_shapes(X, N, Wd, Wc, Wu):
    n, C = X.shape
    r = Wd.shape[1]
    taps = Wc.shape[0]
    assert Wd.shape == (C, r) and Wc.shape == (taps, r, r) and Wu.shape == (r, C) and N.shape == (n, taps)
    assert X.dtype == Wd.dtype == Wc.dtype == Wu.dtype and N.dtype == torch.int32
    return n, C, r, ksize_of_taps(taps)


def sv_adapter_fwd(X, N, Wd, bd, Wc, bc, Wu, bu, H1, H2, Y, workspace, kernel="auto", stream=None):
    n, C, r, K = _adapter_shapes(X, N, Wd, Wc, Wu)
    assert H1.shape == H2.shape == (n, r) and Y.shape == (n, C)
    assert H1.dtype == H2.dtype == Y.dtype == X.dtype
    for b, w in ((bd, r), (bc, r), (bu, C)):
        assert b is None or (b.shape == (w,) and b.dtype == X.dtype)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().sv_adapter_fwd(_ptr(X), _ptr(N), n, K, C, r, _ptr(Wd), _ptr(bd), _ptr(Wc), _ptr(bc), _ptr(Wu),
                               _ptr(bu), _ptr(H1), _ptr(H2), _ptr(Y), _dt(X), _kernel(kernel), _ptr(workspace), wsb,
                               _stream(stream))
    _check(st, "sv_adapter_fwd")


def sv_adapter_bwd(X, N, Wd, Wc, Wu, H1, H2, dY, dX, dWd, dbd, dWc, dbc, dWu, dbu, workspace, kernel="auto",
                   stream=None, dw_stream=None):
    n, C, r, K = _adapter_shapes(X, N, Wd, Wc, Wu)
    assert H1.shape == H2.shape == (n, r) and dY.shape == dX.shape == (n, C)
    assert dWd.shape == (C, r) and dWc.shape == Wc.shape and dWu.shape == (r, C)
    for g in (dWd, dbd, dWc, dbc, dWu, dbu):
        assert g is None or g.dtype == torch.float32
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().sv_adapter_bwd(_ptr(X), _ptr(N), n, K, C, r, _ptr(Wd), _ptr(Wc), _ptr(Wu), _ptr(H1), _ptr(H2),
                               _ptr(dY), _ptr(dX), _ptr(dWd), _ptr(dbd), _ptr(dWc), _ptr(dbc), _ptr(dWu),
                               _ptr(dbu), _dt(X), _kernel(kernel), _ptr(workspace), wsb, _stream(stream),
                               None if dw_stream is None else ctypes.c_void_p(dw_stream.cuda_stream))
    _check(st, "sv_adapter_bwd")


# ---------------------------------------------------------- conveniences
def adapter_fwd(X, N, Wd, bd, Wc, bc, Wu, bu, kernel="auto"):
    """Bottleneck adapter Y = X + (conv_K(X Wd + bd) + bc) Wu + bu.
    Returns (Y, H1, H2); H1 and H2 feed adapter_bwd."""
    n, C = X.shape
    r = Wd.shape[1]
    H1 = torch.empty((n, r), dtype=X.dtype, device=X.device)
    H2 = torch.empty_like(H1)
    Y = torch.empty_like(X)
    ws = torch.empty(max(256, sv_adapter_workspace_bytes(False, n, ksize_of_taps(Wc.shape[0]), C, r, X.dtype)),
                     dtype=torch.uint8, device=X.device)
    sv_adapter_fwd(X, N, Wd, bd, Wc, bc, Wu, bu, H1, H2, Y, ws, kernel)
    return Y, H1, H2


def adapter_bwd(X, N, Wd, Wc, Wu, H1, H2, dY, kernel="auto", dw_stream=None):
    """Returns a dict: dX (X's dtype) and fp32 dWd, dbd, dWc, dbc, dWu, dbu.
    `dw_stream`: a torch stream for the three weight gradients (None: all on
    the current stream)."""
    n, C = X.shape
    r = Wd.shape[1]
    f32 = dict(dtype=torch.float32, device=X.device)
    g = {"dX": torch.empty_like(X), "dWd": torch.empty((C, r), **f32), "dbd": torch.empty((r,), **f32),
         "dWc": torch.empty(tuple(Wc.shape), **f32), "dbc": torch.empty((r,), **f32),
         "dWu": torch.empty((r, C), **f32), "dbu": torch.empty((C,), **f32)}
    ws = torch.empty(max(256, sv_adapter_workspace_bytes(True, n, ksize_of_taps(Wc.shape[0]), C, r, X.dtype)),
                     dtype=torch.uint8, device=X.device)
    sv_adapter_bwd(X, N, Wd, Wc, Wu, H1, H2, dY, g["dX"], g["dWd"], g["dbd"], g["dWc"], g["dbc"], g["dWu"],
                   g["dbu"], ws, kernel, dw_stream=dw_stream)
    return g


def sv_xattn_workspace_bytes(backward, m, n, d) -> int:
    return int(load().sv_xattn_workspace_bytes(1 if backward else 0, int(m), int(n), int(d)))


def sv_xattn_fwd(Q, X, O, lse, workspace, scale=0.0, stream=None):
    m, d = Q.shape
    n = X.shape[0]
    assert X.shape[1] == d and O.shape == (m, d) and lse.shape == (m,) and lse.dtype == torch.float32
    assert Q.dtype == X.dtype == O.dtype
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().sv_xattn_fwd(_ptr(Q), _ptr(X), m, n, d, float(scale), _dt(Q), _ptr(O), _ptr(lse),
                             _ptr(workspace), wsb, _stream(stream))
    _check(st, "sv_xattn_fwd")


def sv_xattn_bwd(Q, X, O, dO, lse, dQ, dX, workspace, scale=0.0, stream=None):
    m, d = Q.shape
    n = X.shape[0]
    assert X.shape[1] == d and O.shape == (m, d) and dO.shape == (m, d) and lse.shape == (m,)
    assert dQ.shape == (m, d) and dQ.dtype == torch.float32 and dX.shape == (n, d)
    assert Q.dtype == X.dtype == O.dtype == dO.dtype == dX.dtype
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().sv_xattn_bwd(_ptr(Q), _ptr(X), _ptr(O), _ptr(dO), _ptr(lse), m, n, d, float(scale), _dt(Q),
                             _ptr(dQ), _ptr(dX), _ptr(workspace), wsb, _stream(stream))
    _check(st, "sv_xattn_bwd")


def xattn_fwd(Q, X, scale=0.0):
    """Cross-attention of the auxiliary tokens Q [m,d] over the visual tokens
    X [n,d] (keys = values).  Returns (O [m,d] in Q's dtype, lse [m] fp32)."""
    m, d = Q.shape
    O = torch.empty_like(Q)
    lse = torch.empty((m,), dtype=torch.float32, device=Q.device)
    ws = torch.empty(max(256, sv_xattn_workspace_bytes(False, m, X.shape[0], d)), dtype=torch.uint8,
                     device=Q.device)
    sv_xattn_fwd(Q, X, O, lse, ws, scale)
    return O, lse


def xattn_bwd(Q, X, O, dO, lse, scale=0.0):
    """Returns (dQ [m,d] fp32, dX [n,d] in X's dtype), given the forward's O and lse."""
    m, d = Q.shape
    dQ = torch.empty((m, d), dtype=torch.float32, device=Q.device)
    dX = torch.empty_like(X)
    ws = torch.empty(max(256, sv_xattn_workspace_bytes(True, m, X.shape[0], d)), dtype=torch.uint8,
                     device=Q.device)
    sv_xattn_bwd(Q, X, O, dO, lse, dQ, dX, ws, scale)
    return dQ, dX


def build_index(coords, frame_offsets, T, H, W, with_map=False, check=True, stream=None, K=3):
    """Allocate and fill N [n, K*K] (and M); with `check`, synchronise and
    raise on a coordinate error reported by the device flag."""
    n = coords.shape[0]
    N = torch.empty((n, K * K), dtype=torch.int32, device=coords.device)
    M = torch.empty((T, H, W), dtype=torch.int32, device=coords.device) if with_map else None
    flag = torch.zeros(1, dtype=torch.int32, device=coords.device)
    if K == 3:
        sv_build_index(coords, frame_offsets, T, H, W, N, M, flag, stream)
    else:
        sv_build_index_k(coords, frame_offsets, T, H, W, K, N, M, flag, stream)
    if check:
        f = int(flag.item())
        if f & SV_FLAG_BAD_OFFSETS:
            raise SvError(SV_ERR_INVALID_ARG, "sv_build_index (frame offsets)")
        if f & SV_FLAG_COORD_RANGE:
            raise SvError(SV_ERR_COORD_RANGE, "sv_build_index")
        if f & SV_FLAG_DUPLICATE:
            raise SvError(SV_ERR_DUPLICATE_COORD, "sv_build_index")
    return (N, M) if with_map else N


# The conveniences below take the neighbourhood from the shapes (Wt or N
# with K*K taps); 3 x 3 goes through the original entry points.
def sparseconv2d_fwd(X, N, Wt, bias=None, kernel="auto"):
    Y = torch.empty((X.shape[0], Wt.shape[2]), dtype=X.dtype, device=X.device)
    (sv_sparseconv2d_fwd if Wt.shape[0] == 9 else sv_sparseconv2d_fwd_k)(X, N, Wt, bias, Y, kernel)
    return Y


def sparseconv2d_bwd_dx(dY, N, Wt, kernel="auto"):
    dX = torch.empty((dY.shape[0], Wt.shape[1]), dtype=dY.dtype, device=dY.device)
    (sv_sparseconv2d_bwd_dx if Wt.shape[0] == 9 else sv_sparseconv2d_bwd_dx_k)(dY, N, Wt, dX, kernel)
    return dX


def sparseconv2d_bwd_dw(X, N, dY, with_db=True, workspace=None):
    Ci, Co = X.shape[1], dY.shape[1]
    taps = N.shape[1]
    dW = torch.empty((taps, Ci, Co), dtype=torch.float32, device=X.device)
    db = torch.empty((Co,), dtype=torch.float32, device=X.device) if with_db else None
    (sv_sparseconv2d_bwd_dw if taps == 9 else sv_sparseconv2d_bwd_dw_k)(X, N, dY, dW, db, False, workspace)
    return dW, db


class SparseConv2dFunction(torch.autograd.Function):
    """autograd wrapper: forward via sv_sparseconv2d_fwd, backward via
    sv_sparseconv2d_bwd_dx and sv_sparseconv2d_bwd_dw (gradients of Wt and
    bias returned in the parameters' dtype)."""

    @staticmethod
    def forward(ctx, X, N, Wt, bias=None, kernel="auto"):
        ctx.save_for_backward(X, N, Wt)
        ctx.kernel = kernel
        ctx.has_bias = bias is not None
        return sparseconv2d_fwd(X.contiguous(), N, Wt.contiguous(),
                                None if bias is None else bias.contiguous(), kernel)

    @staticmethod
    def backward(ctx, dY):
        X, N, Wt = ctx.saved_tensors
        dY = dY.contiguous()
        dX = sparseconv2d_bwd_dx(dY, N, Wt, ctx.kernel) if ctx.needs_input_grad[0] else None
        dW = db = None
        if ctx.needs_input_grad[2] or (ctx.has_bias and ctx.needs_input_grad[3]):
            dW, db = sparseconv2d_bwd_dw(X, N, dY, with_db=ctx.has_bias)
            dW = dW.to(Wt.dtype)
            db = None if db is None else db.to(Wt.dtype)
        return dX, None, dW, db, None


def sparseconv2d(X, N, Wt, bias=None, kernel="auto"):
    return SparseConv2dFunction.apply(X, N, Wt, bias, kernel)
