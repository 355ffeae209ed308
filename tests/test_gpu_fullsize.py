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


def test_long_mtp4_c200k_sampled():
    """The pages' MI355X shape (B200, MTP4, every context 200 000 tokens,
    FP8 per-token, 10.56 GB of KV drawn on the device), in the benchmark's
    launch configuration (five partitions per sequence): all 4 rows of two
    sequences at heads 0, 7 and 15 against the oracle on a host copy of those
    sequences."""
    import torch

    from paged_attention_decode_plan_amd import workloads as W

    inp, plan_kw = make_inputs("long_mtp4_c200k")
    p = inp.problem
    announce(f"long MTP4 C200k: {p.num_seqs} sequences, {p.num_pages} pages")
    got, plan = run(inp, **plan_kw)
    assert plan.info().num_items == 5 * p.num_seqs
    seqs = [0, 137]
    sub = W.host_subset(inp, seqs)
    del inp
    torch.cuda.empty_cache()
    sel = np.array([(r, h) for r in range(sub.problem.rows) for h in (0, 7, 15)], dtype=np.int64)
    rows = [s * p.query_len + i for s in seqs for i in range(p.query_len)]
    g = np.stack([got[rows[r], h] for r, h in sel])
    compare(g, O.attend(sub, sel=sel), "long MTP4 C200k, sampled")
