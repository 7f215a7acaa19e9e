"""GPU parity of lrkv_decode at the workloads' full sizes, in the launch configuration the
benchmark uses (automatic split, max_seq_len = longest request); every output is compared.

- B=8, T=4096, H=16, d_h=128, r=56: cache rows are the oracle's Algorithm-1 append of
  X ~ N(0,1) through N(0, 1/fan_in) weights.
- B=32, T_b ~ U{512..32768}, permuted pages, NaN-filled tail slots (the balanced split).
- B=4, T=131072, H=32, d_h=128, r=32, permuted pages (long chunks, 64 per request).

The two large caches are projections of X ~ N(0,1) through N(0, 1/fan_in) weights too,
computed on the device by torch in float32 and rounded to bf16 (tests/lrkv_case.py,
projected_case_device); the oracle reads the host copy of the packed pool.
Bar: max |gpu - ref| <= 1e-2 max|ref| over all outputs.  lrkv_decode_pq (the private
queries formed once per row by lrkv_private_queries, as the decode step does) must then give
the very bits lrkv_decode gave, at each of these sizes.
"""

import numpy as np
import pytest
import torch

import synth
from lrkv_case import (from_dev, log, max_rel_err, projected_case, projected_case_device,
                       reference_by_request, tolerance)
from test_pq_gpu import run_pq

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def compare_all(case, got, ref, what):
    assert np.all(np.isfinite(got)), what
    assert np.all(np.isfinite(ref)), what
    err = max_rel_err(got, ref)
    log(f"{what}: all {ref.shape[0] * ref.shape[2]} (request, head) outputs, "
        f"max rel err {err:.3e} (bar {tolerance(case.L.dtype):.0e})")
    assert err <= tolerance(case.L.dtype), what


def run_both(case):
    """lrkv_decode's outputs as float64, after checking that lrkv_decode_pq gives the same
    bits."""
    out = case.run()
    pq = run_pq(case)
    assert torch.equal(pq, out), "lrkv_decode_pq differs from lrkv_decode"
    log("lrkv_decode_pq bit-identical to lrkv_decode")
    return from_dev(out, case.L.dtype)


def test_c1_full_all_outputs():
    log("B=8 T=4096 bf16: oracle append of 32768 rows (float64 projection)")
    case = projected_case(11, synth.C1)
    log("decode on the GPU (automatic split)")
    got = run_both(case)
    log("oracle decode of all 128 (request, head) outputs")
    compare_all(case, got, case.reference(), "B=8 T=4096")


def test_c1_full_peaked_queries():
    """Queries scaled by 8 (sharply peaked softmax over 4096 keys)."""
    log("B=8 T=4096, q x 8")
    case = projected_case(12, synth.C1, q_scale=8.0)
    got = run_both(case)
    compare_all(case, got, case.reference(), "B=8 T=4096 peaked")


def test_c2_full_ragged_all_outputs():
    work = synth.C2
    lens = list(work.lens)
    log(f"B=32 ragged lengths {min(lens)}..{max(lens)}, {sum(lens)} tokens: projecting rows")
    case = projected_case_device(21, work, permute=True, fill=0x7FC0)
    log("decode on the GPU (automatic split: balanced page ranges)")
    got = run_both(case)
    ref = reference_by_request(case, "B=32 ragged")
    compare_all(case, got, ref, "B=32 ragged")


def test_c3_full_long_context_all_outputs():
    work = synth.C3
    log("B=4 T=131072 H=32 r=32: projecting 524288 rows")
    case = projected_case_device(31, work, permute=True, fill=0x7FC0)
    log("decode on the GPU (automatic split)")
    got = run_both(case)
    ref = reference_by_request(case, "B=4 T=131072")
    compare_all(case, got, ref, "B=4 T=131072")
