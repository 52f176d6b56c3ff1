#!/usr/bin/env python3
"""SparseConv2D fwd+bwd throughput on one MI355X.

Default workload (one "step" = one pass of the whole hot path over one
batch): T = 384 frames of a 16 x 16 patch grid, three nested pruning stages
(per-frame keep ratios U[.5,.7], U[.3,.5], U[.15,.3]), two adapter layers per
stage, C_in = C_out = 256, bf16 storage with fp32 accumulation:
  per stage: neighbour-table build (sv_build_index), reused by its 2 layers;
  forward through 6 layers with a row gather at each stage change;
  backward through 6 layers: dW + db (split-K), dX, row scatter at stage
  changes.
Inputs are resident in HBM before the timed region starts; the timed region
is K steps between two device synchronisations.

Output: one JSON line (metric, value in effective TFLOP/s over kept tokens,
ms_per_step, a per-kernel breakdown, the roofline of the dominant kernel
measured with HIP events on its launch stream, the CPU oracle timed on
a bounded sample of the same workload, and, as context, the vendor dense
GEMM timed on matrices of the same shapes as each stage's passes).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SparseConv2D fwd+bwd effective TFLOP/s & HBM GB/s vs roofline, 1×MI355X"
PEAK_BF16_TFLOPS = 2516.6    # MI355X dense bf16 MFMA
HBM_TBPS = 8.0               # MI355X HBM3E
# fp32 vector peak of this build: 256 CUs x 4 SIMDs x 16 lanes x 2 FLOP (FMA)
# x 2.4 GHz = 78.6 TFLOP/s.  The 157.3 TFLOP/s of the data sheet counts packed
# fp32 (two FMAs per lane per instruction), which this library's kernels are
# built without.
PEAK_FP32_VALU_TFLOPS = 78.6
PCIE_GBPS_PER_DIRECTION = 64.0   # PCIe 5.0 x16 host link, one direction
PEAK_HBM_GBPS = 8000.0       # MI355X HBM3E


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="c5", choices=["c5", "c1", "c2", "c3a", "c3b", "c4", "c4-host", "xattn",
                                                                "adapter"])
    p.add_argument("--kernel", default="auto", choices=["auto", "mfma", "valu"])
    p.add_argument("--ksize", type=int, default=3, choices=[1, 3, 5, 7],
                   help="single-layer workloads: K of a K x K neighbourhood (weights of the same "
                        "distribution, std 1/sqrt(K*K*C))")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-configs", action="store_true",
                   help="c5: skip measuring the other configurations (c1, c2, c3a, c3b, c4) for the record")
    p.add_argument("--no-dense-gemm", action="store_true",
                   help="c5: skip timing the vendor dense GEMMs of the same shapes (context only)")
    p.add_argument("--cold", action="store_true",
                   help="c5 and single-layer workloads: write a 1 GiB scratch buffer between steps (outside "
                        "the timed events) so that no input stays in the caches; warm (default) is primary")
    p.add_argument("--dw-stream", choices=["side", "same"], default="side",
                   help="run each layer's weight gradient on a second stream, concurrent with its "
                        "input gradient (side), or in order on one stream (same); for c4 the chunk "
                        "driver's dW stream")
    p.add_argument("--cpu-frames", type=int, default=384,
                   help="frames of the workload the CPU oracle is timed on")
    p.add_argument("--calibrate-copy-mib", type=int, default=0,
                   help="also run one plain device copy of this size (HBM counter calibration)")
    a = p.parse_args()
    if a.ksize != 3 and a.workload not in ("c1", "c2", "c3a", "c3b", "c4", "adapter"):
        p.error("--ksize applies to the single-layer workloads c1, c2, c3a, c3b, c4 and to the adapter")
    return a


# ---------------------------------------------------------------- workloads
class StagedRun:
    """Config c5: nested stages, 2 layers per stage, fwd + bwd through all."""

    def __init__(self, kernel="auto", dw_stream="side"):
        import torch
        from sparse_convolution_pruned_amd import ops, workloads as wl

        self.ops, self.torch, self.kernel = ops, torch, kernel
        S = wl.make_staged("c5")
        self.S = S
        bf = torch.bfloat16
        dev = lambda a, d=None: (torch.from_numpy(a).to(d) if d is not None else torch.from_numpy(a)).cuda()
        C = S.X0.shape[1]
        self.C = C
        self.L = len(S.weights)
        self.lps = S.layers_per_stage
        self.stage_of = [l // self.lps for l in range(self.L)]
        self.coords = [dev(s["coords"]) for s in S.stages]
        self.offs = [dev(s["frame_offsets"]) for s in S.stages]
        self.sels = [None] + [dev(s["sel"]) for s in S.stages[1:]]
        self.ns = [int(s["coords"].shape[0]) for s in S.stages]
        self.N = [torch.empty((n, 9), dtype=torch.int32, device="cuda") for n in self.ns]
        self.flag = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.W = [dev(w, bf) for w in S.weights]
        self.b = [dev(b, bf) for b in S.biases]
        self.x0 = dev(S.X0, bf)
        self.dy_last = dev(S.dY_last, bf)
        # activations: xs[l] = input of layer l; ys[l] = output
        self.xs, self.ys = [], []
        for l in range(self.L):
            s = self.stage_of[l]
            if l == 0:
                self.xs.append(self.x0)
            elif self.stage_of[l - 1] != s:
                self.xs.append(torch.empty((self.ns[s], C), dtype=bf, device="cuda"))
            else:
                self.xs.append(self.ys[l - 1])
            self.ys.append(torch.empty((self.ns[s], C), dtype=bf, device="cuda"))
        # gradients: gy[l] = dL/dY_l ; gx[l] = dL/dX_l
        self.gx = [torch.empty((self.ns[self.stage_of[l]], C), dtype=bf, device="cuda") for l in range(self.L)]
        self.gscat = {l: torch.empty((self.ns[self.stage_of[l] - 1], C), dtype=bf, device="cuda")
                      for l in range(1, self.L) if self.stage_of[l - 1] != self.stage_of[l]}
        self.dW = [torch.empty((9, C, C), dtype=torch.float32, device="cuda") for _ in range(self.L)]
        self.db = [torch.empty((C,), dtype=torch.float32, device="cuda") for _ in range(self.L)]
        wsb = max(ops.sv_workspace_bytes(ops.SV_OP_DW, n, C, C, bf) for n in self.ns)
        self.ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device="cuda")
        self.fws = torch.empty(max(256, ops.sv_workspace_bytes(ops.SV_OP_FWD, 0, C, C, bf)),
                               dtype=torch.uint8, device="cuda")
        # dW and dX of a layer both read dY and nothing else either writes, so
        # dW can run on a second stream (default priority) while dX runs on
        # the caller's; the streams join at the end of the step.  The side
        # stream also builds the later stages' index tables and repacks the
        # later layers' forward weights at the start of the step, off the
        # forward chain.
        self.side = torch.cuda.Stream() if dw_stream == "side" else None
        self.ready = [torch.cuda.Event() for _ in range(self.L)]
        self.ev_start, self.ev_prep, self.ev_join = torch.cuda.Event(), torch.cuda.Event(), torch.cuda.Event()
        self.plan = None
        vb = max(256, ops.sv_workspace_bytes(ops.SV_OP_FWD, max(self.ns), C, C, bf))
        self.V = [torch.empty(vb, dtype=torch.uint8, device="cuda") for _ in range(self.L)]
        # the input gradient's weights in fragment order, per layer
        pb = max(256, ops.sv_workspace_bytes(ops.SV_OP_DX, max(self.ns), C, C, bf))
        self.P = [torch.empty(pb, dtype=torch.uint8, device="cuda") for _ in range(self.L)]

    def flops(self):
        """Effective FLOPs per step: 2 * n * 9 * C_in * C_out per pass, all
        9 taps counted, over kept tokens; 3 passes per layer."""
        C = self.C
        return sum(3 * 2 * self.ns[self.stage_of[l]] * 9 * C * C for l in range(self.L))

    def step(self, ev=None, overlap=True):
        """One pass of the whole hot path.  With `overlap` and the side stream
        the step is scheduled over two streams (see __init__; the MFMA
        kernels only: with --kernel valu the step runs in order); without it
        (the instrumented repeat) every call runs alone, in order, on the
        current stream, so that its HIP events bracket that call's kernels
        only."""
        if overlap and self.side is not None and self.kernel != "valu":
            return self._step_streams()
        ops, kern = self.ops, self.kernel
        rec = ev.record if ev is not None else (lambda *a, **k: None)
        S = self.S
        packed = kern != "valu"
        for s in range(len(self.ns)):
            t = rec("index", None)
            ops.sv_build_index(self.coords[s], self.offs[s], S.T, S.H, S.W, self.N[s], None, self.flag)
            rec("index", t, units=self.ns[s])
        if packed:
            # every layer's weights, repacked for the forward and the input gradient in one launch
            t = rec("repack", None)
            ops.sv_repack_layers_k(self.W, self.V, self.P)
            rec("repack", t, units=self.L)
        for l in range(self.L):
            s = self.stage_of[l]
            if l > 0 and self.stage_of[l - 1] != s:
                t = rec("gather", None)
                ops.sv_stage_gather(self.ys[l - 1], self.sels[s], self.xs[l])
                rec("gather", t, units=self.ns[s])
            t = rec("fwd", None)
            if packed:
                ops.sv_sparseconv2d_fwd_packed_k(self.xs[l], self.N[s], self.V[l], self.b[l], self.ys[l], 3)
            else:
                ops.sv_sparseconv2d_fwd(self.xs[l], self.N[s], self.W[l], self.b[l], self.ys[l], kern,
                                        workspace=self.fws)
            rec("fwd", t, units=self.ns[s])
        g = self.dy_last
        for l in reversed(range(self.L)):
            s = self.stage_of[l]
            t = rec("dw", None)
            ops.sv_sparseconv2d_bwd_dw(self.xs[l], self.N[s], g, self.dW[l], self.db[l], False, self.ws)
            rec("dw", t, units=self.ns[s])
            t = rec("dx", None)
            if packed:
                ops.sv_sparseconv2d_bwd_dx_packed_k(g, self.N[s], self.P[l], self.gx[l], 3)
            else:
                ops.sv_sparseconv2d_bwd_dx(g, self.N[s], self.W[l], self.gx[l], kern)
            rec("dx", t, units=self.ns[s])
            g = self.gx[l]
            if l > 0 and self.stage_of[l - 1] != s:
                t = rec("scatter", None)
                ops.sv_stage_scatter(g, self.sels[s], self.gscat[l])
                rec("scatter", t, units=self.ns[s])
                g = self.gscat[l]

    def _step_streams(self):
        """The timed step over two streams; every kernel of the in-order
        step runs, with the same inputs and outputs.  Its library calls are
        prepared once (arguments converted, entry points looked up), so that
        issuing a step costs the host a few microseconds per call: through
        the checking wrappers the ~60 calls of a step took longer on the host
        than the step takes on the GPU."""
        if self.plan is None:
            self.plan = self._prepare_streams()
        for f in self.plan:
            f()

    def _prepare_streams(self):
        import ctypes

        ops, torch, S = self.ops, self.torch, self.S
        lib = ops.load()
        main, side = torch.cuda.current_stream(), self.side
        hs = {id(x): ctypes.c_void_p(x.cuda_stream) for x in (main, side)}
        P = lambda t: None if t is None else t.data_ptr()
        bf, C, K = ops.SV_BF16, self.C, 3
        plan = []

        def call(name, *args):
            fn = getattr(lib, name)

            def f():
                st = fn(*args)
                if st != ops.SV_OK:
                    raise ops.SvError(st, name)
            plan.append(f)

        # Cross-stream ordering uses HIP events created without the system
        # scope fence (and without timing): every producer and consumer here
        # is a kernel on this device, so a device-scope release suffices.
        # With torch's events each record cost the queue ~6 us (a
        # system-scope cache write-back) before the next kernel could start.
        hip = ctypes.CDLL("libamdhip64.so")
        hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        hip.hipStreamWaitEvent.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint]
        hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        flags = 0x2 | 0x20000000          # hipEventDisableTiming | hipEventDisableSystemFence
        events = {}

        def hev(ev):
            if id(ev) not in events:
                h = ctypes.c_void_p()
                if hip.hipEventCreateWithFlags(ctypes.byref(h), flags) != 0:
                    raise RuntimeError("hipEventCreateWithFlags failed")
                events[id(ev)] = h
            return events[id(ev)]
        self._hip_events = events

        def record(ev, stream):
            e, s_ = hev(ev), hs[id(stream)]

            def f():
                if hip.hipEventRecord(e, s_) != 0:
                    raise RuntimeError("hipEventRecord failed")
            plan.append(f)

        def wait(stream, ev):
            e, s_ = hev(ev), hs[id(stream)]

            def f():
                if hip.hipStreamWaitEvent(s_, e, 0) != 0:
                    raise RuntimeError("hipStreamWaitEvent failed")
            plan.append(f)

        def index(s, stream):
            call("sv_build_index", P(self.coords[s]), P(self.offs[s]), S.T, S.H, S.W, self.ns[s], P(self.N[s]),
                 None, P(self.flag), hs[id(stream)])

        # every layer's weights, repacked for the forward and the input
        # gradient in one launch (host arrays of device pointers, kept alive)
        self._rp = [(ctypes.c_void_p * self.L)(*[t.data_ptr() for t in ts]) for ts in (self.W, self.V, self.P)]

        vb = self.ws.numel()
        # side stream: the later stages' index tables
        record(self.ev_start, main)
        wait(side, self.ev_start)
        for s in range(1, len(self.ns)):
            index(s, side)
        record(self.ev_prep, side)
        # main stream: index, all weights, forward
        index(0, main)
        call("sv_repack_layers_k", self.L, self._rp[0], self._rp[1], self.V[0].numel(), self._rp[2], self.P[0].numel(),
             K, C, C, bf, hs[id(main)])
        for l in range(self.L):
            s = self.stage_of[l]
            if l == self.lps:
                wait(main, self.ev_prep)        # the stage-1 and stage-2 tables
            if l > 0 and self.stage_of[l - 1] != s:
                call("sv_stage_gather", P(self.ys[l - 1]), self.ns[s - 1], P(self.sels[s]), self.ns[s], P(self.xs[l]),
                     C, bf, hs[id(main)])
            call("sv_sparseconv2d_fwd_packed_k", P(self.xs[l]), P(self.N[s]), P(self.V[l]), P(self.b[l]),
                 P(self.ys[l]), self.ns[s], K, C, C, bf, hs[id(main)])
        # backward: each layer's dW (partials and their reduction) on the
        # side stream, dX and the stage scatters on main
        g = self.dy_last
        for l in reversed(range(self.L)):
            s = self.stage_of[l]
            record(self.ready[l], main)         # dY of this layer is ready on the main stream
            wait(side, self.ready[l])
            call("sv_sparseconv2d_bwd_dw", P(self.xs[l]), P(self.N[s]), P(g), P(self.dW[l]), P(self.db[l]),
                 self.ns[s], C, C, bf, 0, P(self.ws), vb, hs[id(side)])
            call("sv_sparseconv2d_bwd_dx_packed_k", P(g), P(self.N[s]), P(self.P[l]), P(self.gx[l]), self.ns[s], K,
                 C, C, bf, hs[id(main)])
            g = self.gx[l]
            if l > 0 and self.stage_of[l - 1] != s:
                call("sv_stage_scatter", P(g), P(self.sels[s]), self.ns[s], P(self.gscat[l]), self.ns[s - 1], C, bf,
                     hs[id(main)])
                g = self.gscat[l]
        # the next step overwrites the activations and the workspace the
        # side stream reads
        record(self.ev_join, side)
        wait(main, self.ev_join)
        return plan

    def cpu_sample(self, frames, min_seconds=10.0):
        """The oracle on the first `frames` frames of the same workload:
        index build per stage, fwd through 6 layers, then dW, db, dX back
        through them (float64 loops), the same chain as a GPU step; repeated
        until at least `min_seconds` have elapsed (at most 4 passes)."""
        import numpy as np
        from oracle import oracle as O
        from sparse_convolution_pruned_amd import workloads as wl

        Ssub = wl.make_staged("c5", scale_T=frames)
        ns = [int(st["coords"].shape[0]) for st in Ssub.stages]
        stage_of = self.stage_of
        fl = sum(3 * 2 * ns[stage_of[l]] * 9 * self.C * self.C for l in range(self.L))
        passes, total = 0, 0.0
        while passes == 0 or (total < min_seconds and passes < 4):
            total += self._cpu_pass(Ssub, ns)
            passes += 1
        return fl * passes, total, O.threads(), passes

    def _cpu_pass(self, Ssub, ns):
        import numpy as np
        from oracle import oracle as O

        stage_of = self.stage_of
        t0 = time.perf_counter()
        Ns = []
        for st in Ssub.stages:
            _, N, _ = O.build_index(st["coords"], st["frame_offsets"], Ssub.T, Ssub.H, Ssub.W)
            Ns.append(N)
        xs = []
        x = Ssub.X0.astype(np.float64)
        for l in range(self.L):
            s = stage_of[l]
            if l > 0 and stage_of[l - 1] != s:
                x = x[Ssub.stages[s]["sel"]]
            xs.append(x)
            x = O.fwd(x, Ns[s], Ssub.weights[l], Ssub.biases[l])
        g = Ssub.dY_last.astype(np.float64)
        for l in reversed(range(self.L)):
            s = stage_of[l]
            O.bwd_dw(xs[l], Ns[s], g)
            O.bwd_db(g)
            g = O.bwd_dx(g, Ns[s], Ssub.weights[l])
            if l > 0 and stage_of[l - 1] != s:
                gp = np.zeros((ns[s - 1], g.shape[1]))
                gp[Ssub.stages[s]["sel"]] = g
                g = gp
        return time.perf_counter() - t0


class Events:
    """HIP events around each entry-point call, on the stream the kernels
    are launched on (torch's current stream)."""

    def __init__(self, torch):
        self.torch = torch
        self.items = []

    def record(self, kind, start, units=0):
        t = self.torch
        e = t.cuda.Event(enable_timing=True)
        e.record(t.cuda.current_stream())
        if start is None:
            return e
        self.items.append((kind, start, e, units))
        return None

    def per_units(self, kind):
        """Average duration in microseconds of one kind's calls, grouped by
        the number of tokens they processed."""
        g = {}
        for k, s, e, units in self.items:
            if k == kind:
                g.setdefault(units, []).append(s.elapsed_time(e) * 1e3)
        return {u: sum(v) / len(v) for u, v in g.items()}

    def summary(self):
        out = {}
        for kind, s, e, units in self.items:
            d = out.setdefault(kind, {"ms": 0.0, "launches": 0, "units": 0})
            d["ms"] += s.elapsed_time(e)
            d["launches"] += 1
            d["units"] += units
        return out


def dense_gemm_context(torch, ns, C, ev, reps=20):
    """The vendor library on dense bf16 GEMMs of the same shapes as the c5
    passes, with no gather: [n, 9C] x [9C, C] for a forward or input
    gradient and [9C, n] x [n, C] for a weight gradient, timed with HIP
    events beside this library's own per-stage input-gradient and
    weight-gradient calls (from the instrumented region).  Context for the
    roofline fraction: what a tuned dense GEMM reaches at these sizes."""
    g = torch.Generator(device="cuda").manual_seed(7)
    K = 9 * C

    def timeit(f):
        for _ in range(3):
            f()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            f()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) * 1e3 / reps

    conv_us, dw_us = [], []
    for n in ns:
        A = torch.randn(n, K, device="cuda", dtype=torch.bfloat16, generator=g)
        B = torch.randn(K, C, device="cuda", dtype=torch.bfloat16, generator=g)
        D = torch.randn(n, C, device="cuda", dtype=torch.bfloat16, generator=g)
        conv_us.append(timeit(lambda: A @ B))
        At = A.t()
        dw_us.append(timeit(lambda: At @ D))
        del A, B, D, At
    dx, dw = ev.per_units("dx"), ev.per_units("dw")
    fl = [2.0 * n * K * C for n in ns]
    r = lambda v: [round(x, 1) for x in v]
    return {
        "library": f"torch.matmul (hipBLASLt) bf16, dense operands, torch {torch.__version__}",
        "tokens_per_stage": ns,
        "dense_conv_shape_us": r(conv_us),
        "dense_conv_shape_tflops": r([f / t / 1e6 for f, t in zip(fl, conv_us)]),
        "ours_dx_us": r([dx[n] for n in ns]),
        "ours_dx_tflops": r([f / dx[n] / 1e6 for f, n in zip(fl, ns)]),
        "dense_dw_shape_us": r(dw_us),
        "dense_dw_shape_tflops": r([f / t / 1e6 for f, t in zip(fl, dw_us)]),
        "ours_dw_us": r([dw[n] for n in ns]),
        "ours_dw_tflops": r([f / dw[n] / 1e6 for f, n in zip(fl, ns)]),
    }


def timed_cold(torch, step, steps):
    """Seconds of `steps` steps, each timed by HIP events on the current
    stream, with 1 GiB of scratch written between steps (outside the
    events): the 256 MB MALL and the L2s then hold none of the inputs."""
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    total = 0.0
    for i in range(steps):
        scratch.fill_(i & 0xff)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step()
        e1.record()
        e1.synchronize()
        total += e0.elapsed_time(e1) * 1e-3
    del scratch
    return total


def host_cpu():
    """The host CPU's model name, for the CPU baseline."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def source_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_record(kernel_name, kernel_files):
    """HBM bytes per launch of `kernel_name` from the committed rocprofv3
    --pmc summary, only when it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kernel_name}_c5_hbm_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    files = kernel_files + ["sparse_convolution_pruned_amd/csrc/internal.h",
                            "sparse_convolution_pruned_amd/csrc/mfma.h"]
    if rec.get("source_sha") != source_sha(files):
        return None
    return rec


def measure_layer(key, kernel="auto", ksize=3, steps=20, warmup=3, dw_stream="side", cold=False, scale_T=None):
    """One single-layer configuration (c1, c2, c3a, c3b, c4) timed on the
    GPU: the whole configuration per step (index build and its passes; c4
    through the chunk driver), then each pass alone over `steps`
    back-to-back calls between HIP events on the calling stream.  Returns a
    dict: ms per step and per pass, effective TFLOP/s, the fraction of the
    bf16 MFMA peak (fp32 vector peak for fp32), the gather-model HBM rate and
    its fraction, peak device memory and the workspace."""
    import numpy as np
    import torch
    from sparse_convolution_pruned_amd import ops, workloads as wl

    L = wl.make_layer(key, scale_T=scale_T) if scale_T else wl.make_layer(key)
    cfg = wl.CONFIGS[key]
    dt = torch.bfloat16 if L.dtype == "bf16" else torch.float32
    es = 2 if L.dtype == "bf16" else 4
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats()
    mem0 = torch.cuda.memory_allocated()
    dev = lambda a, d=None: (torch.from_numpy(a).to(d) if d is not None else torch.from_numpy(a)).cuda()
    coords, offs = dev(L.coords), dev(L.frame_offsets)
    K = ksize
    taps = K * K
    n, Ci, Co = L.n, L.X.shape[1], L.Wt.shape[2]
    Wk = L.Wt
    if K != 3:
        rng = np.random.default_rng(900 + K)
        Wk = wl.round_bf16(rng.standard_normal((taps, Ci, Co)).astype(np.float32) / np.sqrt(taps * Ci))
    X, Wt, b, dY = dev(L.X, dt), dev(Wk, dt), dev(L.b, dt), dev(L.dY, dt)
    N = torch.empty((n, taps), dtype=torch.int32, device="cuda")
    Y = torch.empty((n, Co), dtype=dt, device="cuda")
    dX = torch.empty((n, Ci), dtype=dt, device="cuda")
    dW = torch.empty((taps, Ci, Co), dtype=torch.float32, device="cuda")
    db = torch.empty((Co,), dtype=torch.float32, device="cuda")
    passes = cfg["passes"]
    chunked = "chunk_frames" in cfg
    if chunked:
        # the chunks' weight gradients on a second stream (default priority),
        # beside the next chunks' index builds and convolutions
        dws = torch.cuda.Stream() if dw_stream == "side" else None
        desc = ops.make_chunked_desc(L.T, L.H, L.W, coords, offs, torch.from_numpy(L.frame_offsets.copy()),
                                     Ci, Co, dt, cfg["chunk_frames"], X=X, Wt=Wt, bias=b, Y=Y, dY=dY,
                                     dX=dX, dW=dW, db=db, kernel=kernel, ksize=K, dw_stream=dws)
        pm = ops.SV_PASS_FWD | ops.SV_PASS_DX | ops.SV_PASS_DW
        ws = torch.empty(max(256, ops.sv_chunked_workspace_bytes(desc, pm)), dtype=torch.uint8, device="cuda")

        def step():
            ops.sv_sparseconv2d_chunked(desc, pm, ws)
    else:
        ws = torch.empty(max(256, ops.sv_workspace_bytes_k(ops.SV_OP_DW, n, K, Ci, Co, dt)), dtype=torch.uint8,
                         device="cuda")
        fws = torch.empty(max(256, ops.sv_workspace_bytes_k(ops.SV_OP_FWD, n, K, Ci, Co, dt)), dtype=torch.uint8,
                          device="cuda")
        xws = torch.empty(max(256, ops.sv_workspace_bytes_k(ops.SV_OP_DX, n, K, Ci, Co, dt)), dtype=torch.uint8,
                          device="cuda")
        if K == 3:
            run = {"index": lambda: ops.sv_build_index(coords, offs, L.T, L.H, L.W, N),
                   "fwd": lambda: ops.sv_sparseconv2d_fwd(X, N, Wt, b, Y, kernel, workspace=fws),
                   "dx": lambda: ops.sv_sparseconv2d_bwd_dx(dY, N, Wt, dX, kernel, workspace=xws),
                   "dw": lambda: ops.sv_sparseconv2d_bwd_dw(X, N, dY, dW, db, False, ws)}
        else:
            run = {"index": lambda: ops.sv_build_index_k(coords, offs, L.T, L.H, L.W, K, N),
                   "fwd": lambda: ops.sv_sparseconv2d_fwd_k(X, N, Wt, b, Y, kernel, workspace=fws),
                   "dx": lambda: ops.sv_sparseconv2d_bwd_dx_k(dY, N, Wt, dX, kernel, workspace=xws),
                   "dw": lambda: ops.sv_sparseconv2d_bwd_dw_k(X, N, dY, dW, db, False, ws)}

        def step():
            run["index"]()
            run["fwd"]()
            if "dx" in passes:
                run["dx"]()
            if "dw" in passes:
                run["dw"]()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    if cold:
        sec = timed_cold(torch, step, steps) / steps
    else:
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        sec = (time.perf_counter() - t0) / steps
    # each pass alone (device time of `steps` back-to-back calls)
    pass_ms = {}
    if not chunked:
        for name in ["index", "fwd"] + [p for p in ("dx", "dw") if p in passes]:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                run[name]()
            e1.record()
            torch.cuda.synchronize()
            pass_ms[name] = round(e0.elapsed_time(e1) / steps, 4)
    fl_pass = 2 * n * taps * Ci * Co
    fl = len(passes) * fl_pass
    # gather model per conv pass: every neighbour row read from memory, no reuse
    gather_bytes = n * (taps * es * Ci + es * Co + 4 * taps)
    # fp32 data, or the VALU kernel on bf16 data: fp32 FMAs on the vector ALUs
    on_valu = kernel == "valu" or L.dtype != "bf16"
    peak = PEAK_FP32_VALU_TFLOPS if on_valu else PEAK_BF16_TFLOPS
    out = {"name": cfg["name"], "kernel": kernel, "ksize": K, "n": n, "dtype": L.dtype,
           "valid_tap_fraction": None if chunked else round(float((N >= 0).sum().item()) / max(N.numel(), 1), 4),
           "ms_per_step": round(sec * 1e3, 4), "passes": list(passes),
           "tflops": round(fl / sec / 1e12, 3),
           "roofline_fp32_vector" if on_valu else "roofline_mfma":
               {"peak_tflops": peak, "frac": round(fl / sec / 1e12 / peak, 4)},
           "roofline_hbm_gather_model": {"gbps": round(len(passes) * gather_bytes / sec / 1e9, 1),
                                         "frac": round(len(passes) * gather_bytes / sec / 1e9 / PEAK_HBM_GBPS, 4)},
           "peak_mem_mb": round((torch.cuda.max_memory_allocated() - mem0) / 2 ** 20, 1),
           "workspace_mb": round(ws.numel() / 2 ** 20, 2)}
    if pass_ms:
        out["pass_ms"] = pass_ms
        out["pass_tflops"] = {k: round(fl_pass / (v * 1e-3) / 1e12, 2) for k, v in pass_ms.items() if k != "index"}
        # each conv pass alone against the gather-model HBM roofline (the
        # index build and the weight repack excluded: a table and repacked
        # weights serve every pass and layer that share them)
        out["pass_frac_hbm_gather_model"] = {k: round(gather_bytes / (v * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)
                                             for k, v in pass_ms.items() if k in ("fwd", "dx")}
    if chunked:
        out["dw_stream"] = dw_stream
    return out


def configs_record(steps=20, warmup=3):
    """The other configurations, for the driver-run record beside the c5
    headline: c1 (fp32), c2 on both kernels, c3a, c3b, c4 (chunked) and c4's
    device memory at 384 frames (the workspace does not grow with T); each
    with ms per step and per pass, TFLOP/s and its roofline fractions."""
    rec = {}
    rec["c1"] = measure_layer("c1", steps=steps, warmup=warmup)
    rec["c2_mfma"] = measure_layer("c2", "mfma", steps=steps, warmup=warmup)
    rec["c2_valu"] = measure_layer("c2", "valu", steps=max(3, steps // 4), warmup=1)
    rec["c3a"] = measure_layer("c3a", steps=steps, warmup=warmup)
    rec["c3b"] = measure_layer("c3b", steps=steps, warmup=warmup)
    rec["c4"] = measure_layer("c4", steps=steps, warmup=warmup)
    short = measure_layer("c4", steps=3, warmup=1, scale_T=384)
    rec["c4"]["memory_by_T"] = {"384": {"peak_mem_mb": short["peak_mem_mb"], "workspace_mb": short["workspace_mb"]},
                                "3072": {"peak_mem_mb": rec["c4"]["peak_mem_mb"],
                                         "workspace_mb": rec["c4"]["workspace_mb"]}}
    return rec


def index_build_cpu_ms(reps=5):
    """The oracle's index build alone on the host for the c5 first stage
    (58,822 tokens over 384 frames of a 16 x 16 grid): context for the
    page's index build on the CPU."""
    from oracle import oracle as O
    from sparse_convolution_pruned_amd import workloads as wl

    S = wl.make_staged("c5")
    st = S.stages[0]
    O.build_index(st["coords"], st["frame_offsets"], S.T, S.H, S.W)
    best = 1e30
    for _ in range(reps):
        t0 = time.perf_counter()
        O.build_index(st["coords"], st["frame_offsets"], S.T, S.H, S.W)
        best = min(best, time.perf_counter() - t0)
    return {"ms": round(best * 1e3, 3), "tokens": int(st["coords"].shape[0]), "frames": S.T,
            "note": "best of %d, single call of the float64/int32 oracle on the host (index arithmetic only)" % reps}


def layer_workload(args):
    """Single-layer workloads (c1, c2, c3a, c3b, c4), for the design notes'
    per-configuration table; prints one JSON line of its own."""
    r = measure_layer(args.workload, args.kernel, args.ksize, args.steps, args.warmup, args.dw_stream, args.cold)
    r["workload"] = args.workload
    r["cache"] = "cold" if args.cold else "warm"
    print(json.dumps(r), flush=True)


def host_stream_workload(args):
    """Config 4 through the host-streamed chunk driver: X, dY, Y, dX and the
    coordinates stay in pinned host memory and stream through two device
    staging sets; the device holds the weights, dW/db and the workspace.
    Reports the PCIe-inclusive rate and the device memory at the full length
    and at 256 frames (flat in T)."""
    import torch
    from sparse_convolution_pruned_amd import ops, workloads as wl

    cfg = wl.CONFIGS["c4"]
    bf = torch.bfloat16
    pm = ops.SV_PASS_FWD | ops.SV_PASS_DX | ops.SV_PASS_DW

    def setup(L):
        n, C = L.n, L.X.shape[1]
        pin = lambda a, d=None: (torch.from_numpy(a).to(d) if d is not None else torch.from_numpy(a)).pin_memory()
        h = dict(coords=pin(L.coords), offs=pin(L.frame_offsets), X=pin(L.X, bf), dY=pin(L.dY, bf),
                 Y=torch.empty((n, C), dtype=bf).pin_memory(), dX=torch.empty((n, C), dtype=bf).pin_memory())
        Wt = torch.from_numpy(L.Wt).to(bf).cuda()
        b = torch.from_numpy(L.b).to(bf).cuda()
        dW = torch.empty((9, C, C), dtype=torch.float32, device="cuda")
        db = torch.empty((C,), dtype=torch.float32, device="cuda")
        d = ops.make_chunked_host_desc(L.T, L.H, L.W, h["coords"], h["offs"], C, C, bf, cfg["chunk_frames"],
                                       X_host=h["X"], Wt=Wt, bias=b, Y_host=h["Y"], dY_host=h["dY"],
                                       dX_host=h["dX"], dW=dW, db=db, kernel=args.kernel)
        ws = torch.empty(max(256, ops.sv_chunked_host_workspace_bytes(d, pm)), dtype=torch.uint8, device="cuda")
        return d, ws, (h, Wt, b, dW, db)

    s_h2d, s_d2h = torch.cuda.Stream(), torch.cuda.Stream()
    peaks = {}
    for frames in (256, None):
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        L = wl.make_layer("c4", scale_T=frames)
        d, ws, keep = setup(L)
        reps = args.warmup if frames is not None else 0
        for _ in range(max(reps, 1)):
            ops.sv_sparseconv2d_chunked_host(d, pm, ws, s_h2d, s_d2h)
        torch.cuda.synchronize()
        peaks[L.T] = (torch.cuda.max_memory_allocated() - base) / 2 ** 20
        if frames is None:
            for _ in range(args.warmup):
                ops.sv_sparseconv2d_chunked_host(d, pm, ws, s_h2d, s_d2h)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                ops.sv_sparseconv2d_chunked_host(d, pm, ws, s_h2d, s_d2h)
            torch.cuda.synchronize()
            sec = (time.perf_counter() - t0) / args.steps
            n, C = L.n, L.X.shape[1]
            h2d = 4 * n + 4 * (L.T + 1) + 2 * (2 * n * C)     # coords, offsets, X, dY
            d2h = 2 * (2 * n * C)                             # Y, dX
            fl = 3 * 2 * n * 9 * C * C
            out = {"workload": "c4-host", "name": cfg["name"] + ", activations in pinned host memory",
                   "kernel": args.kernel, "n": n, "ms_per_step": round(sec * 1e3, 4),
                   "tflops_pcie_inclusive": round(fl / sec / 1e12, 3),
                   "h2d_gbps": round(h2d / sec / 1e9, 2), "d2h_gbps": round(d2h / sec / 1e9, 2),
                   "roofline": {"bound": "pcie", "achieved": round(max(h2d, d2h) / sec / 1e9, 2),
                                "peak": PCIE_GBPS_PER_DIRECTION, "unit": "GB/s per direction",
                                "frac": round(max(h2d, d2h) / sec / 1e9 / PCIE_GBPS_PER_DIRECTION, 4)},
                   "workspace_mb": round(ws.numel() / 2 ** 20, 2)}
    out["device_mem_mb_by_T"] = {str(k): round(v, 1) for k, v in sorted(peaks.items())}
    print(json.dumps(out), flush=True)


def xattn_workload(args):
    """Asymmetric cross-attention of auxiliary queries (CLS: m = 1; and
    m = 4) over the c5 stage-0 visual tokens (n = 58,822, d = 256, bf16),
    forward and backward.  Memory-bound: the algorithmic bytes are the
    token rows read (forward) and read plus written as dX (backward)."""
    import numpy as np
    import torch
    from sparse_convolution_pruned_amd import ops, workloads as wl

    S = wl.make_staged("c5")
    X = torch.from_numpy(S.X0).to(torch.bfloat16).cuda()
    n, d = X.shape
    rng = np.random.default_rng(5)
    res = []
    for m in (1, 4):
        Q = torch.from_numpy(rng.standard_normal((m, d)).astype(np.float32)).to(torch.bfloat16).cuda()
        dO = torch.from_numpy(rng.standard_normal((m, d)).astype(np.float32)).to(torch.bfloat16).cuda()
        O = torch.empty_like(Q)
        lse = torch.empty((m,), dtype=torch.float32, device="cuda")
        dQ = torch.empty((m, d), dtype=torch.float32, device="cuda")
        dX = torch.empty_like(X)
        wf = torch.empty(max(256, ops.sv_xattn_workspace_bytes(False, m, n, d)), dtype=torch.uint8, device="cuda")
        wb = torch.empty(max(256, ops.sv_xattn_workspace_bytes(True, m, n, d)), dtype=torch.uint8, device="cuda")
        for _ in range(args.warmup):
            ops.sv_xattn_fwd(Q, X, O, lse, wf)
            ops.sv_xattn_bwd(Q, X, O, dO, lse, dQ, dX, wb)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        torch.cuda.synchronize()
        tf = tb = 0.0
        for _ in range(args.steps):
            ev[0].record()
            ops.sv_xattn_fwd(Q, X, O, lse, wf)
            ev[1].record()
            ops.sv_xattn_bwd(Q, X, O, dO, lse, dQ, dX, wb)
            ev[2].record()
            torch.cuda.synchronize()
            tf += ev[0].elapsed_time(ev[1]) * 1e-3
            tb += ev[1].elapsed_time(ev[2]) * 1e-3
        tf /= args.steps
        tb /= args.steps
        bf_ = 2 * n * d
        bb_ = 2 * 2 * n * d
        res.append({"m": m, "fwd_us": round(tf * 1e6, 2), "bwd_us": round(tb * 1e6, 2),
                    "fwd_gbps": round(bf_ / tf / 1e9, 1), "bwd_gbps": round(bb_ / tb / 1e9, 1),
                    "fwd_frac_hbm": round(bf_ / tf / 1e9 / 8000.0, 4),
                    "bwd_frac_hbm": round(bb_ / tb / 1e9 / 8000.0, 4)})
    print(json.dumps({"workload": "xattn", "name": "auxiliary queries over the c5 stage-0 tokens, keys = values",
                      "n": n, "d": d, "dtype": "bf16", "results": res,
                      "note": "times are whole calls (partial + merge launches) between HIP events on the "
                              "calling stream; bytes are the token rows read (fwd) and read + written (bwd)"}),
          flush=True)


def adapter_workload(args):
    """The bottleneck adapter (down-projection C -> r, K x K SparseConv2D
    r -> r, up-projection r -> C, residual) over the c5 first-stage tokens
    (n = 58,822 of a 16 x 16 grid, 384 frames) at C = 1024, r = 256, bf16:
    forward and backward timed separately with HIP events on the stream
    they run on."""
    import torch
    from sparse_convolution_pruned_amd import ops, workloads as wl

    K = args.ksize
    A = wl.make_adapter_stage0(K=K)
    bf = torch.bfloat16
    dev = lambda a, d=None: (torch.from_numpy(a).to(d) if d is not None else torch.from_numpy(a)).cuda()
    X = dev(A.X, bf)
    N = ops.build_index(dev(A.coords), dev(A.frame_offsets), A.T, A.H, A.W, K=K)
    P = {k: dev(getattr(A, k), bf) for k in ("Wd", "bd", "Wc", "bc", "Wu", "bu")}
    dY = dev(A.dY, bf)
    n, C = A.X.shape
    r, taps = A.Wd.shape[1], K * K
    H1 = torch.empty((n, r), dtype=bf, device="cuda")
    H2 = torch.empty_like(H1)
    Y = torch.empty_like(X)
    dX = torch.empty_like(X)
    f32 = dict(dtype=torch.float32, device="cuda")
    dWd, dbd = torch.empty((C, r), **f32), torch.empty((r,), **f32)
    dWc, dbc = torch.empty((taps, r, r), **f32), torch.empty((r,), **f32)
    dWu, dbu = torch.empty((r, C), **f32), torch.empty((C,), **f32)
    wf = torch.empty(max(256, ops.sv_adapter_workspace_bytes(False, n, K, C, r, bf)), dtype=torch.uint8, device="cuda")
    wb = torch.empty(max(256, ops.sv_adapter_workspace_bytes(True, n, K, C, r, bf)), dtype=torch.uint8, device="cuda")

    def fwd():
        ops.sv_adapter_fwd(X, N, P["Wd"], P["bd"], P["Wc"], P["bc"], P["Wu"], P["bu"], H1, H2, Y, wf, args.kernel)

    # the three weight gradients on a second stream (default priority),
    # beside the input gradients
    dws = torch.cuda.Stream() if args.dw_stream == "side" else None

    def bwd():
        ops.sv_adapter_bwd(X, N, P["Wd"], P["Wc"], P["Wu"], H1, H2, dY, dX, dWd, dbd, dWc, dbc, dWu, dbu, wb,
                           args.kernel, dw_stream=dws)

    for _ in range(args.warmup):
        fwd()
        bwd()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(args.steps):
        fwd()
    ev[1].record()
    for _ in range(args.steps):
        bwd()
    ev[2].record()
    torch.cuda.synchronize()
    tf = ev[0].elapsed_time(ev[1]) * 1e-3 / args.steps
    tb = ev[1].elapsed_time(ev[2]) * 1e-3 / args.steps
    fl_f = 2.0 * n * (C * r + taps * r * r + r * C)
    fl_b = 2 * fl_f
    print(json.dumps({"workload": "adapter", "name": A.name, "n": n, "C": C, "r": r, "ksize": K,
                      "kernel": args.kernel, "fwd_ms": round(tf * 1e3, 4), "bwd_ms": round(tb * 1e3, 4),
                      "fwd_tflops": round(fl_f / tf / 1e12, 2), "bwd_tflops": round(fl_b / tb / 1e12, 2),
                      "step_tflops": round((fl_f + fl_b) / (tf + tb) / 1e12, 2),
                      "frac_bf16_peak": round((fl_f + fl_b) / (tf + tb) / 1e12 / PEAK_BF16_TFLOPS, 4),
                      "workspace_mb": {"fwd": round(wf.numel() / 2 ** 20, 2), "bwd": round(wb.numel() / 2 ** 20, 2)},
                      "dw_stream": args.dw_stream}),
          flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                                   "(multi-GPU sharding by frames is described in the design notes, not built)"}))
        sys.exit(2)
    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.workload == "c4-host":
        return host_stream_workload(args)
    if args.workload == "xattn":
        return xattn_workload(args)
    if args.workload == "adapter":
        return adapter_workload(args)
    if args.workload != "c5":
        return layer_workload(args)

    run = StagedRun(args.kernel, args.dw_stream)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        run.step()
    torch.cuda.synchronize()
    assert int(run.flag.item()) == 0, "index build reported a coordinate error"
    torch.cuda.reset_peak_memory_stats()

    # timed region: K steps, no instrumentation
    torch.cuda.synchronize()
    if args.cold:
        wall = timed_cold(torch, run.step, args.steps)
    else:
        t0 = time.perf_counter()
        for _ in range(args.steps):
            run.step()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    ms = wall * 1e3 / args.steps
    fl = run.flops()
    tflops = fl / (wall / args.steps) / 1e12

    # instrumented timed region: the same K steps with HIP events per call,
    # every call alone on the current stream (no dW/dX overlap), so that
    # the per-kernel durations are the kernels' own.  The host issues these
    # calls slower than the GPU runs them, and an event pair around a call
    # would then also time the host's gap before the kernel; so the region
    # starts behind a spin kernel long enough for the host to queue all of
    # it, and the GPU runs the calls back to back.
    ev = Events(torch)
    torch.cuda.synchronize()
    torch.cuda._sleep(int(6.0e6 * args.steps))          # ~3 ms per step at ~2 GHz: the host's pace here
    for _ in range(args.steps):
        run.step(ev, overlap=False)
    torch.cuda.synchronize()
    kinds = ev.summary()
    C = run.C
    per_unit = {  # algorithmic FLOPs and compulsory HBM bytes per token (bf16)
        "fwd": (2 * 9 * C * C, 2 * (C + C) + 36),
        "dx": (2 * 9 * C * C, 2 * (C + C) + 36),
        "dw": (2 * 9 * C * C, 2 * (C + C) + 36),
        "index": (0, 40),
        "gather": (0, 4 * C + 4),
        "scatter": (0, 4 * C + 4),
        # per layer: Wt read and written twice (forward and input-gradient layouts)
        "repack": (0, 4 * 9 * C * C * 2),
    }
    # gather model: each of the 9 neighbour rows read from memory, no reuse
    gather_unit = 9 * 2 * C + 2 * C + 36
    breakdown = {}
    for k, d in kinds.items():
        f_unit, b_unit = per_unit[k]
        sec = d["ms"] / 1e3
        breakdown[k] = {
            "ms_per_step": round(d["ms"] / args.steps, 4),
            "launches_per_step": d["launches"] // args.steps,
            "avg_launch_us": round(d["ms"] * 1e3 / d["launches"], 2),
            "tflops": round(f_unit * d["units"] / sec / 1e12, 2) if f_unit else None,
            "gbps_compulsory": round(b_unit * d["units"] / sec / 1e9, 1),
        }
        if k in ("fwd", "dx", "dw"):
            g = gather_unit * d["units"] / sec / 1e9
            breakdown[k]["gbps_gather_model"] = round(g, 1)
            breakdown[k]["frac_hbm_gather_model"] = round(g / (HBM_TBPS * 1e3), 4)
    # Dominant kernel: the conv kernel runs in every forward and every input
    # gradient (k_conv_bfrag at C = 256: the packed entry points launch it
    # alone, so their HIP events time exactly that kernel).
    conv_ms = kinds["fwd"]["ms"] + kinds["dx"]["ms"]
    valu = args.kernel == "valu"
    if conv_ms >= kinds["dw"]["ms"]:
        dom = ("fwd", "dx")
        kname = "k_conv_valu" if valu else "k_conv_bfrag"
        kfiles = ["sparse_convolution_pruned_amd/csrc/" + ("conv_valu.hip" if valu else "conv_bfrag.hip")]
    else:
        dom, kname, kfiles = ("dw",), "k_dw_mfma", ["sparse_convolution_pruned_amd/csrc/dw.hip"]
    # the VALU conv kernels are bound by fp32 vector arithmetic
    bound, peak = ("alu", PEAK_FP32_VALU_TFLOPS) if (valu and dom != ("dw",)) else ("mfma", PEAK_BF16_TFLOPS)
    d = {"ms": sum(kinds[k]["ms"] for k in dom), "units": sum(kinds[k]["units"] for k in dom),
         "launches": sum(kinds[k]["launches"] for k in dom)}
    # per launch: FLOPs of the tokens it processed / its duration, averaged
    # over launches weighted by duration (sum of FLOPs / sum of durations)
    achieved = per_unit[dom[0]][0] * d["units"] / (d["ms"] / 1e3) / 1e12
    tr = traffic_record(kname, kfiles)
    roofline = {
        "bound": bound,
        "kernel": kname,
        "achieved": round(achieved, 2),
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": round(achieved / peak, 4),
        "traffic": None if tr is None else tr["bytes_per_launch"],
        "avg_launch_us": round(d["ms"] * 1e3 / d["launches"], 2),
        "flops_per_launch": round(per_unit[dom[0]][0] * d["units"] / d["launches"]),
        "launches_timed": d["launches"],
    }
    step_bytes = sum(per_unit[k][1] * kinds[k]["units"] for k in kinds) / args.steps
    out = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "T=384 frames, 16x16 grid, 3 nested pruning stages (keep U[.5,.7]/U[.3,.5]/"
                        "U[.15,.3]), 2 layers per stage, C_in=C_out=256, fwd+bwd through 6 layers",
            "tokens_per_stage": run.ns,
            "valid_tap_fraction": [round(float((Nt >= 0).sum().item()) / Nt.numel(), 4) for Nt in run.N],
            "cache": "cold" if args.cold else "warm",
            "kernel": args.kernel,
            "dw_stream": args.dw_stream,
            "flops_per_step": fl,
        },
        "hbm_gbps_compulsory": round(step_bytes / (wall / args.steps) / 1e9, 1),
        "peak_mem_mb": round(torch.cuda.max_memory_allocated() / 2 ** 20, 1),
        "kernels": breakdown,
        "roofline": roofline,
    }
    if not args.no_dense_gemm and args.kernel != "valu":
        out["dense_gemm_same_shape"] = dense_gemm_context(torch, run.ns, C, ev)
    if not args.no_configs and args.kernel == "auto":
        out["configs"] = configs_record()
    if args.calibrate_copy_mib:
        nb = args.calibrate_copy_mib * 2 ** 20
        a = torch.empty(nb, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        out["calibration_copy_bytes"] = nb
    if not args.no_cpu_baseline:
        cfl, cdt, threads, passes = run.cpu_sample(args.cpu_frames)
        out["cpu_baseline"] = {
            "value": round(cfl / cdt / 1e12, 6),
            "unit": "TFLOP/s",
            "cores": threads,
            "kind": "oracle",
            "cpu": host_cpu(),
            "sample": f"{passes} pass(es) over the first {args.cpu_frames} of 384 frames of the same "
                      f"workload: index build per stage, fwd through 6 layers, dW+db+dX back "
                      f"through them, float64 loops ({cdt:.1f} s)",
            "index_build": index_build_cpu_ms(),
        }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
