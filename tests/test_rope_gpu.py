"""GPU parity of lrkv_decode_rope (rotary keys over the unrotated factored cache, LRKV notes
§8) against the float64 oracle's decode_reference_rope, through the C ABI.  Bar: max |gpu -
ref| <= 1e-2 max|ref| (bf16 cache, float32 accumulation)."""

import numpy as np
import pytest

import oracle as O
import synth
from lrkv_case import iid_case, log, max_rel_err, projected_case, tolerance

pytestmark = pytest.mark.gpu


def check(got, ref, what, mask=None):
    err = max_rel_err(got, ref, mask)
    log(f"{what}: max rel err {err:.3e} (bar 1e-02)")
    assert np.all(np.isfinite(got if mask is None else got[mask])), what
    assert err <= tolerance(O.BF16), what


@pytest.mark.parametrize("shape", [(16, 128, 56), (32, 128, 32)])
@pytest.mark.parametrize("chunk", [0, 16, 48])
def test_rope_ragged_permuted_nan_tails(shape, chunk):
    H, dh, r = shape
    lens = [1, 17, 100, 16, 33, 250, 0]
    case = iid_case(401 + H, H, dh, r, O.BF16, lens, permute=True, fill=0x7FC0)
    cs = synth.rope_table(256, dh)
    got = case.run_rope(cs, chunk_tokens=chunk)
    ref = case.reference_rope(cs)
    assert np.all(got[6] == 0.0)  # a request with no token gives zeros
    check(got[:6], ref[:6], f"rope {shape} chunk {chunk}")


def test_rope_differs_from_unrotated_decode():
    """The turn matters: with a real table the outputs are far from the unrotated ones, and
    the rotary oracle is what the kernel matches."""
    case = iid_case(403, 16, 128, 56, O.BF16, [300, 77], permute=True)
    cs = synth.rope_table(300, 128)
    got = case.run_rope(cs)
    plain = case.reference()
    assert max_rel_err(got, plain) > 0.05
    check(got, case.reference_rope(cs), "rope vs its oracle")


def test_rope_zero_angle_matches_plain_decode_oracle():
    case = iid_case(404, 32, 128, 32, O.BF16, [129, 64], permute=True, fill=0x7FC0)
    cs = np.zeros((129, 64, 2), np.float32)
    cs[..., 0] = 1.0
    check(case.run_rope(cs), case.reference(), "rope, zero angles, vs plain oracle")


def test_rope_multi_row_queries_causal():
    case = iid_case(405, 16, 128, 56, O.BF16, [40, 7, 16], q_len=5, permute=True, fill=0x7FC0)
    cs = synth.rope_table(40, 128)
    check(case.run_rope(cs, chunk_tokens=16), case.reference_rope(cs), "rope multi-row")


def test_rope_peaked_queries_and_long_table():
    """q x 8 (peaked softmax), a table longer than the history (rows past it unused)."""
    case = iid_case(406, 16, 128, 56, O.BF16, [513, 1000, 31], permute=True, q_scale=8.0)
    cs = synth.rope_table(4096, 128)
    check(case.run_rope(cs), case.reference_rope(cs), "rope peaked")


def test_rope_keys_near_half_precision_range():
    """Private key parts z B_K^T up to 4.7e4, close to the largest finite f16 (65504) in
    which the call holds them for the pair products (cached key rows x 9e3, which bf16
    holds; the query x 4.4e-4 so that the scores stay moderate, its smallest entries below
    the f16 normal range)."""
    case = iid_case(407, 16, 128, 56, O.BF16, [300, 45], permute=True, q_scale=4.4e-4,
                    key_scale=9e3, fill=0x7FC0)
    cs = synth.rope_table(300, 128)
    check(case.run_rope(cs), case.reference_rope(cs), "rope, private key parts up to 4.7e4")


@pytest.mark.slow
def test_rope_full_b8_t4096_all_outputs():
    """B=8, T=4096, H=16, d_h=128, r=56, rows from the oracle's append of X through
    1/sqrt(fan_in) weights, every output."""
    case = projected_case(13, synth.C1)
    cs = synth.rope_table(4096, 128)
    log("rope decode B=8 x 4096 on the GPU")
    got = case.run_rope(cs)
    log("oracle")
    check(got, case.reference_rope(cs), "rope B=8 T=4096 (all 128 outputs)")
