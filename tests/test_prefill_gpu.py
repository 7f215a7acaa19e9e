"""GPU parity of multi-query (prefill) lrkv_decode calls against the float64 oracle.

A bf16 call with q_len >= 64 query rows per request takes the MFMA multi-query kernel.  Row
i of request b sits at position seq_len[b] - q_len + i and sees positions 0..that one; rows
with no visible position return zeros.  Bar: max |gpu - ref| <= 1e-2 max|ref| (bf16 cache,
float32 accumulation).
"""

import math

import numpy as np
import pytest

import oracle as O
import synth
from lrkv_case import Case, as_codes, codes_f64, iid_case, log, max_rel_err, tolerance

pytestmark = pytest.mark.gpu


def check(case, got, ref, what, mask=None):
    err = max_rel_err(got, ref, mask)
    log(f"{what}: max rel err {err:.3e}")
    assert err <= tolerance(case.L.dtype), what
    assert np.all(np.isfinite(got if mask is None else got[mask]))


@pytest.mark.parametrize("lens,q_len", [([300, 200], 96), ([256], 256), ([129, 64, 190], 64)])
def test_c1_shape_multi_query(lens, q_len):
    """Ragged requests, permuted pages, NaN-filled tail slots; every output compared."""
    log(f"prefill H=16 r=56, lens {lens}, q_len {q_len}")
    case = iid_case(601, 16, 128, 56, O.BF16, lens, q_len=q_len, permute=True, fill=0x7FC0)
    check(case, case.run_f64(), case.reference(), f"prefill lens {lens} q_len {q_len}")


def test_c3_shape_multi_query():
    log("prefill H=32 r=32")
    case = iid_case(602, 32, 128, 32, O.BF16, [200, 77], q_len=130, permute=True, fill=0x7FC0)
    got = case.run_f64()
    ref = case.reference()
    # request 1 (77 tokens) has 53 leading rows with no visible position: zeros
    assert np.all(got[1, :53] == 0.0)
    check(case, got, ref, "prefill H=32")


def test_long_request_crosses_page_id_blocks():
    """4500 positions = 71 key tiles of 64: the page ids the kernel keeps in LDS (64 tiles at
    a time) are refilled mid-request."""
    case = iid_case(606, 32, 128, 32, O.BF16, [4500, 300], q_len=64, permute=True, fill=0x7FC0)
    check(case, case.run_f64(), case.reference(), "prefill 4500 positions")


def test_rows_before_the_first_position_are_zero():
    case = iid_case(603, 16, 128, 56, O.BF16, [100], q_len=128, permute=True, fill=0x7FC0)
    got = case.run_f64()
    assert np.all(got[0, :28] == 0.0)
    check(case, got, case.reference(), "q_len > seq_len")


def test_peaked_queries():
    """Queries scaled by 8: sharply peaked rows exercise the rescale of the running max."""
    case = iid_case(604, 16, 128, 56, O.BF16, [320], q_len=192, permute=True, q_scale=8.0)
    check(case, case.run_f64(), case.reference(), "prefill peaked")


@pytest.mark.parametrize("shape", [(16, 128, 56), (32, 128, 32)])
def test_multi_query_is_deterministic_and_page_order_free(shape):
    """Same bits on every run and for any page order (each workgroup's arithmetic order is
    fixed; page placement only changes addresses)."""
    H, dh, r = shape
    lens = [300, 140, 70]
    a = iid_case(605, H, dh, r, O.BF16, lens, q_len=96, permute=False)
    b = iid_case(605, H, dh, r, O.BF16, lens, q_len=96, permute=True)
    oa = a.run().cpu().numpy()
    for _ in range(3):
        assert np.array_equal(oa, a.run().cpu().numpy())
    assert np.array_equal(oa, b.run().cpu().numpy())


@pytest.mark.slow
def test_c4_full_prefill_sampled():
    """B=4 prompts of 8192 tokens, d=2048: the cache is the oracle's Algorithm-1 append of
    X ~ N(0,1), Q = X W_q (float64, rounded to bf16), permuted pages; the GPU computes all
    32768 x 16 outputs, sampled (row, head) outputs are compared with the oracle."""
    work = synth.C4
    L = O.Layout(work.H, work.d_h, work.r, work.page_size, O.BF16)
    n = work.tokens
    log("C4: weights, activations")
    w = synth.projection_weights(41, work.d, work.H, work.d_h, work.r, with_wq=True)
    wc = {k: as_codes(v, O.BF16) for k, v in w.items()}
    w64 = {k: codes_f64(v, O.BF16) for k, v in wc.items()}
    X64 = codes_f64(as_codes(synth.activations(42, n, work.d), O.BF16), O.BF16)
    table, npg = synth.page_assignment(43, list(work.lens), work.page_size, True)
    req = np.repeat(np.arange(work.B), work.lens[0])
    pos = np.tile(np.arange(work.lens[0]), work.B)
    log("C4: oracle append of 32768 rows")
    pool = O.append_reference(np.zeros(npg * O.page_bytes(L), np.uint8), L, X64, w64["W_SK"],
                              w64["W_SV"], w64["U_K"], w64["U_V"], req, pos, table)
    log("C4: Q = X W_q")
    Q = (X64 @ w64["W_q"]).reshape(work.B, work.lens[0], work.H, work.d_h)
    qc = O.f64_to_bf16_bits(Q)
    del X64, Q
    case = Case(L, pool, table, list(work.lens), qc, wc["B_K"], wc["B_V"], npg)
    log("C4: GPU prefill")
    got = case.run_f64()
    assert np.all(np.isfinite(got))
    g = np.random.default_rng(44)
    rows = sorted({0, 1, 15, 16, 63, 64, 127, 128, 1000, 4095, 4096, 8191,
                   *g.integers(0, work.lens[0], 6).tolist()})
    sample = [(b, i, h) for b in range(work.B) for i in rows for h in (0, 9, 15)]
    log(f"C4: oracle on {len(sample)} sampled outputs")
    ref = case.reference(sample=sample)
    check(case, got, ref, "C4 prefill sampled", mask=~np.isnan(ref))
