"""Seeded synthetic inputs for SparseConv2D on pruned ViT token sequences.

This module only draws inputs: kept-token masks, packed coordinates, frame
offsets, activations, weights, bias and upstream gradients.  It holds none of
the convolution's arithmetic, so both the HIP path and the CPU oracle can be
fed from it.  Every array is numpy; floating tensors are float32 arrays whose
values are already representable in the workload's dtype (bf16 values are
rounded once, round-to-nearest-even, here on the host).

The shapes follow the pages' setting ("SV-TAD: Native Sparse Convolutions for
Efficient Temporal Action Detection", paper notes page): ViT patch grids of
14x14 or 16x16 per (tubelet-2) frame, attention-guided pruning that keeps a
fraction of the patches per frame (Overall Architecture; Key Findings), tokens
packed frame-major (Key Design 1 builds M per frame from the kept tokens'
grid coordinates).  No trained backbone is available, so a smooth saliency
field (three isotropic Gaussian blobs plus noise) stands in for the attention
scores that drive the selection.

Random streams: ``numpy.random.SeedSequence(seed).spawn(6)`` in the order
[mask, ratios, X, W, b, dY]; each consumer draws from its own child stream.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

STREAMS = ("mask", "ratios", "X", "W", "b", "dY")


def round_bf16(a) -> np.ndarray:
    """float32 -> nearest bf16 value (ties to even), returned as float32."""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(a.shape)


def _streams(seed) -> Dict[str, np.random.Generator]:
    children = np.random.SeedSequence(seed).spawn(len(STREAMS))
    return {name: np.random.Generator(np.random.PCG64(c)) for name, c in zip(STREAMS, children)}


def keep_count(ratio: float, cells: int) -> int:
    """Kept tokens per frame: nearest integer to ratio * cells (halves up)."""
    return int(np.floor(ratio * cells + 0.5))


def saliency_field(rng: np.random.Generator, H: int, W: int, blobs: int = 3,
                   sigma_lo: float = 1.5, sigma_hi: float = 4.0,
                   noise_var: float = 0.1) -> np.ndarray:
    """Sum of `blobs` unit-amplitude isotropic Gaussians evaluated at patch
    centres (y + 0.5, x + 0.5); centres uniform over the grid, sigma uniform in
    [sigma_lo, sigma_hi]; plus i.i.d. normal noise of variance `noise_var`."""
    cy = rng.uniform(0.0, H, size=blobs)
    cx = rng.uniform(0.0, W, size=blobs)
    sg = rng.uniform(sigma_lo, sigma_hi, size=blobs)
    yy, xx = np.meshgrid(np.arange(H) + 0.5, np.arange(W) + 0.5, indexing="ij")
    f = np.zeros((H, W), dtype=np.float64)
    for b in range(blobs):
        d2 = (yy - cy[b]) ** 2 + (xx - cx[b]) ** 2
        f += np.exp(-d2 / (2.0 * sg[b] ** 2))
    f += rng.normal(0.0, np.sqrt(noise_var), size=(H, W))
    return f


def top_cells(field_hw: np.ndarray, count: int) -> np.ndarray:
    """Flat indices of the `count` largest cells (ties toward the lower
    index), returned in ascending flat order (row-major packing)."""
    order = np.argsort(-field_hw.ravel(), kind="stable")
    return np.sort(order[:count]).astype(np.int32)


def pack(frames: List[np.ndarray]):
    """Concatenate per-frame flat coordinates; returns (coords, offsets)."""
    counts = np.array([len(f) for f in frames], dtype=np.int64)
    offs = np.zeros(len(frames) + 1, dtype=np.int64)
    np.cumsum(counts, out=offs[1:])
    coords = np.concatenate(frames).astype(np.int32) if frames else np.zeros(0, np.int32)
    return coords, offs.astype(np.int32)


def _normal(rng, shape, std, dtype):
    a = rng.standard_normal(size=shape).astype(np.float64) * std
    a = a.astype(np.float32)
    return round_bf16(a) if dtype == "bf16" else a


@dataclass
class Layer:
    """One SparseConv2D layer's inputs."""
    T: int
    H: int
    W: int
    coords: np.ndarray          # int32 [n], flat p = y*W + x
    frame_offsets: np.ndarray   # int32 [T+1]
    X: np.ndarray               # float32 [n, Ci] (bf16-exact when dtype == bf16)
    Wt: np.ndarray              # float32 [taps, Ci, Co] (taps = 9 at 3 x 3)
    b: np.ndarray               # float32 [Co]
    dY: np.ndarray              # float32 [n, Co]
    dtype: str
    name: str = ""

    @property
    def n(self) -> int:
        return int(self.coords.shape[0])


@dataclass
class Staged:
    """Layer-varying sparsity: nested stage masks, 2 layers per stage."""
    T: int
    H: int
    W: int
    stages: List[dict]          # each: coords, frame_offsets, sel (rows of the previous stage kept here; None for stage 0)
    weights: List[np.ndarray]   # per layer [9, C, C]
    biases: List[np.ndarray]    # per layer [C]
    X0: np.ndarray              # input of layer 1, [n_0, C]
    dY_last: np.ndarray         # upstream gradient of the last layer, [n_last, C]
    layers_per_stage: int
    dtype: str
    name: str = ""


# The five workloads: sizes, keep ratios and distributions of the setting
# described above, one per tested regime.
CONFIGS = {
    "c1": dict(name="tiny fp32: T=1, 14x14, 98 of 196 kept uniformly, C=64",
               T=1, H=14, W=14, mask="uniform", count=98, C=64, dtype="f32",
               passes=("fwd", "dx", "dw"), seed=1),
    "c2": dict(name="T=384, 14x14, saliency keep 40%, C=128 bf16, forward",
               T=384, H=14, W=14, mask="saliency", keep=0.40, C=128, dtype="bf16",
               passes=("fwd",), seed=2),
    "c3a": dict(name="T=384, 14x14, saliency keep 30%, C=256 bf16, fwd+dX+dW",
                T=384, H=14, W=14, mask="saliency", keep=0.30, C=256, dtype="bf16",
                passes=("fwd", "dx", "dw"), seed=3),
    "c3b": dict(name="T=384, 14x14, saliency keep 30%, C=512 bf16, fwd+dX+dW",
                T=384, H=14, W=14, mask="saliency", keep=0.30, C=512, dtype="bf16",
                passes=("fwd", "dx", "dw"), seed=3),
    "c4": dict(name="T=3072 (6144 frames), 14x14, saliency keep 30%, C=128 bf16, "
                    "chunks of 256 frames, fwd+dX+dW",
               T=3072, H=14, W=14, mask="saliency", keep=0.30, C=128, dtype="bf16",
               passes=("fwd", "dx", "dw"), chunk_frames=256, seed=4),
    "c5": dict(name="T=384, 16x16, 3 nested stages keep U[.5,.7]/U[.3,.5]/U[.15,.3], "
                    "2 layers per stage, C=256 bf16, fwd+bwd through 6 layers",
               T=384, H=16, W=16, stage_ranges=((0.5, 0.7), (0.3, 0.5), (0.15, 0.3)),
               layers_per_stage=2, C=256, dtype="bf16", seed=5),
}


def make_layer(key: str, scale_T: Optional[int] = None) -> Layer:
    """Inputs of configs c1..c4.  `scale_T` (optional) keeps only the first
    scale_T frames, for quick checks of the same recipe."""
    cfg = CONFIGS[key]
    T, H, W, C, dt = cfg["T"], cfg["H"], cfg["W"], cfg["C"], cfg["dtype"]
    if scale_T is not None:
        T = min(T, scale_T)
    rs = _streams(cfg["seed"])
    frames = []
    for _ in range(T):
        if cfg["mask"] == "uniform":
            sel = rs["mask"].choice(H * W, size=cfg["count"], replace=False)
            frames.append(np.sort(sel).astype(np.int32))
        else:
            f = saliency_field(rs["mask"], H, W)
            frames.append(top_cells(f, keep_count(cfg["keep"], H * W)))
    coords, offs = pack(frames)
    n = coords.shape[0]
    X = _normal(rs["X"], (n, C), 1.0, dt)
    Wt = _normal(rs["W"], (9, C, C), 1.0 / np.sqrt(9.0 * C), dt)
    b = np.zeros((C,), dtype=np.float32)
    dY = _normal(rs["dY"], (n, C), 1.0, dt)
    return Layer(T, H, W, coords, offs, X, Wt, b, dY, dt, cfg["name"])


def make_staged(key: str = "c5", scale_T: Optional[int] = None) -> Staged:
    cfg = CONFIGS[key]
    T, H, W, C, dt = cfg["T"], cfg["H"], cfg["W"], cfg["C"], cfg["dtype"]
    if scale_T is not None:
        T = min(T, scale_T)
    rs = _streams(cfg["seed"])
    ranges = cfg["stage_ranges"]
    per_stage_frames: List[List[np.ndarray]] = [[] for _ in ranges]
    for _ in range(T):
        f = saliency_field(rs["mask"], H, W)
        order = np.argsort(-f.ravel(), kind="stable")
        for s, (lo, hi) in enumerate(ranges):
            r = rs["ratios"].uniform(lo, hi)
            cnt = keep_count(r, H * W)
            per_stage_frames[s].append(np.sort(order[:cnt]).astype(np.int32))
    stages = []
    for s in range(len(ranges)):
        coords, offs = pack(per_stage_frames[s])
        sel = None
        if s > 0:
            prev = stages[s - 1]
            rows = []
            for t in range(T):
                pc = per_stage_frames[s - 1][t]
                cc = per_stage_frames[s][t]
                loc = np.searchsorted(pc, cc)
                rows.append(loc.astype(np.int64) + int(prev["frame_offsets"][t]))
            sel = np.concatenate(rows).astype(np.int32) if rows else np.zeros(0, np.int32)
        stages.append(dict(coords=coords, frame_offsets=offs, sel=sel))
    L = len(ranges) * cfg["layers_per_stage"]
    weights = [_normal(rs["W"], (9, C, C), 1.0 / np.sqrt(9.0 * C), dt) for _ in range(L)]
    biases = [np.zeros((C,), dtype=np.float32) for _ in range(L)]
    n0 = stages[0]["coords"].shape[0]
    nl = stages[-1]["coords"].shape[0]
    X0 = _normal(rs["X"], (n0, C), 1.0, dt)
    dY_last = _normal(rs["dY"], (nl, C), 1.0, dt)
    return Staged(T, H, W, stages, weights, biases, X0, dY_last,
                  cfg["layers_per_stage"], dt, cfg["name"])


def make_random_case(seed: int, T: int, H: int, W: int, keep, Ci: int, Co: int,
                     dtype: str = "f32", shuffle: bool = False,
                     bias: bool = True, ksize: int = 3) -> Layer:
    """Small property-test case.  `keep` is a ratio in [0, 1], or a list of
    per-frame counts; frames may be empty.  `shuffle` permutes the tokens
    inside each frame (any order is a valid packing).  `ksize`: K of the
    K x K weights (K*K taps, std 1/sqrt(K*K*C_in))."""
    rs = _streams([7919, seed])
    frames = []
    for t in range(T):
        cnt = keep[t] if isinstance(keep, (list, tuple)) else keep_count(float(keep), H * W)
        cnt = max(0, min(int(cnt), H * W))
        sel = rs["mask"].choice(H * W, size=cnt, replace=False).astype(np.int32)
        sel = rs["mask"].permutation(sel) if shuffle else np.sort(sel)
        frames.append(sel.astype(np.int32))
    coords, offs = pack(frames)
    n = coords.shape[0]
    X = _normal(rs["X"], (n, Ci), 1.0, dtype)
    taps = ksize * ksize
    Wt = _normal(rs["W"], (taps, Ci, Co), 1.0 / np.sqrt(float(taps) * max(Ci, 1)), dtype)
    b = _normal(rs["b"], (Co,), 1.0, dtype) if bias else np.zeros((Co,), np.float32)
    dY = _normal(rs["dY"], (n, Co), 1.0, dtype)
    return Layer(T, H, W, coords, offs, X, Wt, b, dY, dtype, f"random seed={seed}")


@dataclass
class AdapterCase:
    """Inputs of one bottleneck adapter (down-projection C -> r, K x K
    SparseConv2D r -> r, up-projection r -> C, residual) on a token set."""
    T: int
    H: int
    W: int
    coords: np.ndarray          # int32 [n]
    frame_offsets: np.ndarray   # int32 [T+1]
    X: np.ndarray               # [n, C]
    Wd: np.ndarray              # [C, r]
    bd: np.ndarray              # [r]
    Wc: np.ndarray              # [K*K, r, r]
    bc: np.ndarray              # [r]
    Wu: np.ndarray              # [r, C]
    bu: np.ndarray              # [C]
    dY: np.ndarray              # [n, C]
    K: int
    dtype: str
    name: str = ""

    @property
    def n(self) -> int:
        return int(self.coords.shape[0])


def _adapter_params(rs, n, C, r, K, dtype):
    """Weights ~ N(0, 1/fan_in) (so every layer keeps unit scale), biases
    ~ N(0, 0.1^2), X and dY ~ N(0, 1); bf16-representable for bf16."""
    taps = K * K
    return dict(X=_normal(rs["X"], (n, C), 1.0, dtype),
                Wd=_normal(rs["W"], (C, r), 1.0 / np.sqrt(C), dtype),
                bd=_normal(rs["b"], (r,), 0.1, dtype),
                Wc=_normal(rs["W"], (taps, r, r), 1.0 / np.sqrt(taps * r), dtype),
                bc=_normal(rs["b"], (r,), 0.1, dtype),
                Wu=_normal(rs["W"], (r, C), 1.0 / np.sqrt(r), dtype),
                bu=_normal(rs["b"], (C,), 0.1, dtype),
                dY=_normal(rs["dY"], (n, C), 1.0, dtype))


def make_adapter_case(seed: int, T: int, H: int, W: int, keep, C: int, r: int, K: int = 3,
                      dtype: str = "f32", shuffle: bool = False) -> AdapterCase:
    """Small adapter case on a random token set (as make_random_case)."""
    L = make_random_case(seed, T, H, W, keep, 1, 1, dtype, shuffle=shuffle)
    rs = _streams([7927, seed])
    p = _adapter_params(rs, L.n, C, r, K, dtype)
    return AdapterCase(T, H, W, L.coords, L.frame_offsets, K=K, dtype=dtype, name=f"adapter seed={seed}", **p)


def make_adapter_stage0(C: int = 1024, r: int = 256, K: int = 3, scale_T: Optional[int] = None) -> AdapterCase:
    """The adapter on the first-stage token set of the c5 workload (384
    frames of a 16 x 16 grid, keep U[.5, .7]): a ViT width C = 1024 (the
    large video ViT the page evaluates) around a bottleneck of r = 256, the
    channel width of the c5 SparseConv2D layers."""
    S = make_staged("c5", scale_T)
    st = S.stages[0]
    rs = _streams([7933, C, r, K])
    p = _adapter_params(rs, int(st["coords"].shape[0]), C, r, K, "bf16")
    return AdapterCase(S.T, S.H, S.W, st["coords"], st["frame_offsets"], K=K, dtype="bf16",
                       name=f"adapter C={C} r={r} K={K} on c5 stage 0", **p)
