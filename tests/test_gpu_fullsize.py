"""GPU parity at the five workloads' full sizes, in the launch configuration
the benchmark times (its input factory and plan options, the device's CU
count): every output where the oracle is cheap (sparse, long-context D256,
ragged), and a fixed sample of (row, head) outputs of every sequence for the
dense MTP4 batches (and the same FP8 batch with QL 2), compared element by
element with the oracle within atol = rtol = 0.005 (aiter PR #6617,
Validation)."""

from __future__ import annotations

import numpy as np
import pytest

from bench import make_inputs
from gpu_helpers import announce, compare, run
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _sample(p, heads):
    """All query rows of every sequence, at the given heads."""
    return np.array([(r, h) for r in range(p.rows) for h in heads], dtype=np.int64)


@pytest.mark.parametrize("workload", ["sparse", "long_d256", "ragged", "tiny"])
def test_full_size_every_output(workload):
    inp, plan_kw = make_inputs(workload)
    announce(f"full size {workload}: every output")
    got, plan = run(inp, **plan_kw)
    compare(got, O.attend(inp), f"{workload} full size")


@pytest.mark.parametrize("workload", ["dense_mtp4_fp8", "dense_mtp4_bf16", "dense_mtp2_fp8"])
def test_full_size_sampled(workload):
    inp, plan_kw = make_inputs(workload)
    p = inp.problem
    sel = _sample(p, [0, 5, 10, 15])
    announce(f"full size {workload}: {len(sel)} sampled outputs")
    got, plan = run(inp, **plan_kw)
    assert plan.info().num_items >= plan.info().cu_count  # the benchmark's partitioning
    g = np.stack([got[r, h] for r, h in sel])
    compare(g, O.attend(inp, sel=sel), f"{workload} full size, sampled")
