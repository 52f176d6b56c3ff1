"""The benchmark's step over two streams (later index tables and forward
weights prepared on a second stream at the start, each layer's weight
gradient there concurrently with its input gradient) computes exactly what
the in-order step computes: the streams only reorder independent work and
every kernel is deterministic, so all outputs must match bit for bit, on
every repeat."""
import os
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
def test_overlapped_step_matches_ordered_step():
    sys.path.insert(0, ROOT)
    import bench

    run = bench.StagedRun("auto", "side")
    print("c5 staged run, tokens per stage", run.ns, flush=True)
    run.step(overlap=False)
    torch.cuda.synchronize()
    ref = [t.clone() for t in run.ys + run.dW + run.db + run.gx + run.N + list(run.gscat.values())]
    for rep in range(3):
        run.step(overlap=True)
        torch.cuda.synchronize()
        got = run.ys + run.dW + run.db + run.gx + run.N + list(run.gscat.values())
        for i, (a, b) in enumerate(zip(ref, got)):
            assert torch.equal(a, b), f"repeat {rep}: output tensor {i} differs between schedules"

