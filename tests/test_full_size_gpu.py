"""GPU parity of lrkv_decode at the workloads' full sizes, in the launch configuration the
benchmark uses (automatic chunking, max_seq_len = longest request).

- B=8, T=4096, H=16, d_h=128, r=56: cache rows are the oracle's Algorithm-1 append of
  X ~ N(0,1) through N(0, 1/fan_in) weights; every output is compared.
- B=32, T_b ~ U{512..32768}, permuted pages, NaN-filled tail slots: sampled requests
  (shortest, longest and others) and heads are compared, and every output must be finite.
- B=4, T=131072, H=32, r=32, permuted pages: sampled (request, head) outputs.

The two large caches hold i.i.d. N(0,1) rows (the large-d law of the projections; projecting
half a million rows in float64 would take teraflops).  Bar: max |gpu - ref| <= 1e-2 max|ref|.
"""

import numpy as np
import pytest

import oracle as O
import synth
from lrkv_case import iid_case, log, max_rel_err, projected_case, tolerance

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def check_sampled(case, got, sample, what):
    ref = case.reference(sample=sample)
    mask = ~np.isnan(ref)
    assert mask.any()
    err = max_rel_err(got, ref, mask)
    log(f"{what}: {len(sample)} sampled outputs, max rel err {err:.3e}")
    assert err <= tolerance(case.L.dtype), what


def test_c1_full_all_outputs():
    log("B=8 T=4096 bf16: oracle append of 32768 rows (float64 projection)")
    case = projected_case(11, synth.C1)
    log("decode on the GPU (automatic chunks)")
    got = case.run_f64()
    log("oracle decode of all 128 (request, head) outputs")
    ref = case.reference()
    err = max_rel_err(got, ref)
    log(f"B=8 T=4096: max rel err {err:.3e}")
    assert err <= tolerance(case.L.dtype)


def test_c1_full_peaked_queries():
    """Queries scaled by 8 (sharply peaked softmax over 4096 keys)."""
    log("B=8 T=4096, q x 8")
    case = projected_case(12, synth.C1, q_scale=8.0)
    got = case.run_f64()
    sample = [(b, 0, h) for b in (0, 5) for h in range(16)]
    check_sampled(case, got, sample, "B=8 T=4096 peaked")


def test_c2_full_ragged_sampled():
    work = synth.C2
    lens = list(work.lens)
    log(f"B=32 ragged lengths {min(lens)}..{max(lens)}, {sum(lens)} tokens: drawing rows")
    case = iid_case(21, work.H, work.d_h, work.r, O.BF16, lens, permute=True, fill=0x7FC0)
    log("decode on the GPU (automatic chunks)")
    got = case.run_f64()
    assert np.all(np.isfinite(got))
    order = np.argsort(lens)
    reqs = sorted({int(order[0]), int(order[-1]), int(order[len(lens) // 2]), 3, 17})
    sample = [(b, 0, h) for b in reqs for h in (0, 9, 15)]
    check_sampled(case, got, sample, "B=32 ragged")


def test_c3_full_long_context_sampled():
    work = synth.C3
    log("B=4 T=131072 H=32 r=32: drawing 524288 rows")
    case = iid_case(31, work.H, work.d_h, work.r, O.BF16, list(work.lens), permute=True)
    log("decode on the GPU (automatic chunks)")
    got = case.run_f64()
    assert np.all(np.isfinite(got))
    sample = [(0, 0, 0), (1, 0, 31), (2, 0, 16), (3, 0, 7)]
    check_sampled(case, got, sample, "B=4 T=131072")
