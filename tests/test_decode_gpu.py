"""GPU parity of lrkv_decode against the float64 oracle, through the C-ABI library.

Bars (max over compared outputs of |gpu - ref| / max|ref|): 1e-2 for a bf16 cache, 1e-5 for
float32.  Page-table indexing is checked bit-exactly: a permuted pool must give the same
output bits as the identity pool.
"""

import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from lrkv_case import (Case, as_codes, codes_f64, from_dev, iid_case, log, max_rel_err,
                       projected_case, tolerance, to_dev)

pytestmark = pytest.mark.gpu


def check(case: Case, got, ref, mask=None, what=""):
    err = max_rel_err(got, ref, mask)
    log(f"{what}: max rel err {err:.3e} (bar {tolerance(case.L.dtype):.0e})")
    assert err <= tolerance(case.L.dtype), what
    assert np.all(np.isfinite(got if mask is None else got[mask]))


# --------------------------------------------------------------------------------------
# small shapes: every output compared
# --------------------------------------------------------------------------------------


def test_c0_fp32_decode():
    log("c0 fp32 decode, 64 cached + 1 new token, contiguous")
    case = projected_case(0, synth.C0)
    check(case, case.run_f64(), case.reference(), what="c0")


def test_c0_fp32_end_to_end_from_x():
    """C0 from the raw inputs: GPU append of X, then GPU decode of q = x_new W_q, against the
    oracle's per-head projection W_h = W_S + U_h B_h^T applied to X directly (eq 2)."""
    import factored_rank_kv_amd as F
    from lrkv_case import layout_c, output_major

    work = synth.C0
    w = synth.projection_weights(0, work.d, work.H, work.d_h, work.r, with_wq=True)
    X = synth.activations(1, 65, work.d)
    L = O.Layout(work.H, work.d_h, work.r, 16, O.F32)
    table, npg = synth.page_assignment(2, [65], 16, False)
    pool = torch.zeros(npg * O.page_bytes(L), dtype=torch.uint8, device="cuda:0")
    dev = {k: torch.from_numpy(output_major(w[k])).to("cuda:0")
           for k in ("W_SK", "W_SV", "U_K", "U_V")}
    Xd = torch.from_numpy(X).to("cuda:0")
    req = torch.zeros(65, dtype=torch.int32, device="cuda:0")
    pos = torch.arange(65, dtype=torch.int32, device="cuda:0")
    tab = torch.from_numpy(table).to("cuda:0")
    log("c0 append 65 rows")
    F.lrkv_append(layout_c(L), Xd, 65, work.d, dev["W_SK"], dev["W_SV"], dev["U_K"], dev["U_V"],
                  req, pos, tab, table.shape[1], pool, npg)
    q = (X[64].astype(np.float64) @ w["W_q"].astype(np.float64)).astype(np.float32)
    q = q.reshape(1, 1, work.H, work.d_h)
    case = Case(L, None, table, [65], q.view(np.uint32), w["B_K"].view(np.uint32),
                w["B_V"].view(np.uint32), npg)
    log("c0 decode")
    got = from_dev(case.run(pool=pool), O.F32)
    X64 = X.astype(np.float64)
    K = O.full_projection_kv(X64, w["W_SK"], w["U_K"], w["B_K"])
    V = O.full_projection_kv(X64, w["W_SV"], w["U_V"], w["B_V"])
    ref = np.stack([O.softmax_attention(q[0, 0, h].astype(np.float64), K[h], V[h],
                                        1 / math.sqrt(work.d_h)) for h in range(work.H)])
    err = max_rel_err(got[0, 0], ref)
    log(f"c0 end to end: max rel err {err:.3e}")
    assert err <= 1e-5


@pytest.mark.parametrize("chunk", [0, 16, 48])
def test_c1_shape_ragged_paged_nan_tails(chunk):
    log(f"c1 shape, ragged lengths, permuted pool, NaN tails, chunk={chunk}")
    case = iid_case(101, 16, 128, 56, O.BF16, [1, 17, 100, 16, 33, 250], permute=True,
                    fill=0x7FC0)
    check(case, case.run_f64(chunk_tokens=chunk), case.reference(), what=f"c1 ragged chunk {chunk}")


BALANCED_SHAPES = [(16, 128, 56, O.BF16), (32, 128, 32, O.BF16), (4, 16, 4, O.F32)]


def balanced_lens(kind):
    g = np.random.default_rng(120)
    if kind == "mixed":  # zero, one, page edges, long and short requests
        return [0, 1, 15, 16, 17, 300, 1000, 33] + g.integers(0, 700, 16).tolist()
    if kind == "short_many":  # 100 requests of 3 pages: ranges of 1-2 pages
        return [48] * 100
    if kind == "equal":  # 20 x 700 tokens: about 55 pages a range
        return [700] * 20
    if kind == "few_pages_100":  # 16 x 7 pages = 112 pages, fewer than the 256 ranges
        return [100] * 16
    if kind == "few_pages_48":  # 16 x 3 pages = 48 pages
        return [48] * 16
    if kind == "few_pages_ragged":  # 20 requests, 0..3 pages each, some empty
        return [0, 1, 17, 48, 0, 33, 16, 2, 47, 0, 5, 31, 32, 18, 0, 9, 40, 1, 16, 3]
    raise ValueError(kind)


@pytest.mark.parametrize("shape", BALANCED_SHAPES, ids=["h16r56", "h32r32", "h4r4f32"])
@pytest.mark.parametrize("lens_kind", ["mixed", "short_many", "equal", "few_pages_100",
                                       "few_pages_48", "few_pages_ragged"])
def test_balanced_split(shape, lens_kind):
    """Automatic splits of 16 or more single-row requests cut the batch's pages into equal
    ranges per workgroup; ranges cross request boundaries (one segment and record per
    request met), requests of 0 tokens own no pages, and a batch of fewer pages than
    workgroups gets one range per page.  The workspace starts as NaN bytes, so a merged
    record the split did not write shows.  Every output against the oracle, and against
    the chunked split (explicit chunk_tokens) within the same bar."""
    H, dh, r, dt = shape
    lens = balanced_lens(lens_kind)
    nan_fill = 0x7FC0 if dt == O.BF16 else 0x7FC00000
    log(f"balanced split {shape}, {len(lens)} requests, {sum(lens)} tokens ({lens_kind})")
    case = iid_case(121 + len(lens) + H, H, dh, r, dt, lens, permute=True, fill=nan_fill)
    got = case.run_f64()
    ref = case.reference()
    for b, t in enumerate(lens):
        if t == 0:
            assert np.all(got[b] == 0.0)
    live = np.array(lens) > 0
    check(case, got[live], ref[live], what=f"balanced {shape} {lens_kind}")
    chunked = case.run_f64(chunk_tokens=64)
    check(case, chunked[live], ref[live], what=f"chunked {shape} {lens_kind}")


def test_c3_shape_small():
    log("c3 shape (32 heads, r=32), ragged, permuted, NaN tails")
    case = iid_case(102, 32, 128, 32, O.BF16, [5, 64, 129], permute=True, fill=0x7FC0)
    check(case, case.run_f64(chunk_tokens=32), case.reference(), what="c3 small")


def test_c0_shape_ragged():
    log("c0 shape, ragged, permuted, NaN tails")
    case = iid_case(103, 4, 16, 4, O.F32, [1, 15, 16, 17, 90], permute=True, fill=0x7FC00000)
    check(case, case.run_f64(chunk_tokens=16), case.reference(), what="c0 ragged")


def test_empty_and_single_token_requests():
    log("seq_len 0, 1 and 17")
    case = iid_case(104, 16, 128, 56, O.BF16, [0, 1, 17], permute=True, fill=0x7FC0)
    got = case.run_f64()
    ref = case.reference()
    assert np.all(got[0] == 0.0)
    check(case, got[1:], ref[1:], what="lens 1, 17")


def test_permuted_pool_is_bit_identical_to_identity():
    """Page-table indexing is exact: the same rows in a permuted pool decode to the same bits."""
    lens = [70, 33, 129]
    a = iid_case(105, 16, 128, 56, O.BF16, lens, permute=False)
    b = iid_case(105, 16, 128, 56, O.BF16, lens, permute=True)
    assert not np.array_equal(a.table, b.table)
    for chunk in (16, 64, 0):
        log(f"identity vs permuted, chunk={chunk}")
        oa = a.run(chunk_tokens=chunk).cpu()
        ob = b.run(chunk_tokens=chunk).cpu()
        assert torch.equal(oa, ob)


@pytest.mark.parametrize("shape", [(16, 128, 56), (32, 128, 32)])
def test_merge_in_several_passes(shape):
    """More chunk records per query row than the merge holds in LDS at once (65 at H=16,
    74 at H=32): 2100 tokens in 16-token chunks are 132 records, merged in passes of that
    many; the weights of every pass are taken against the row's global max."""
    H, dh, r = shape
    log(f"merge in passes, shape {shape}")
    case = iid_case(130 + H, H, dh, r, O.BF16, [2100, 1100, 5], permute=True, fill=0x7FC0)
    check(case, case.run_f64(chunk_tokens=16), case.reference(), what=f"merge passes {shape}")


def test_chunk_sizes_agree():
    case = iid_case(106, 16, 128, 56, O.BF16, [300, 77], permute=True)
    ref = case.reference()
    for chunk in (16, 32, 304):
        log(f"chunk={chunk}")
        check(case, case.run_f64(chunk_tokens=chunk), ref, what=f"chunk {chunk}")


def test_peaked_softmax_max_in_last_chunk():
    """q scaled by 8 and the last token's shared key aligned with every head's query: the
    running max jumps in the last chunk and every earlier chunk must be rescaled to ~0."""
    lens = [200, 64]
    case = iid_case(107, 16, 128, 56, O.BF16, lens, permute=True, q_scale=8.0)
    L = case.L
    # rebuild S_K of each request's last token as half the sum of that request's queries
    pool = case.pool.copy()
    for b, T in enumerate(lens):
        key = 0.5 * case.q64[b, 0].sum(axis=0)
        SK_rows = O.gather_request(pool, L, case.table[b], T)
        new_sk = O.round_to_dtype(key, L.dtype)
        SK, SV = SK_rows["SK"], SK_rows["SV"]
        pool = O.write_rows(pool, L, case.table, [b], [T - 1], new_sk[None], SV[T - 1:T],
                            np.transpose(SK_rows["RK"][:, T - 1:T], (1, 0, 2)),
                            np.transpose(SK_rows["RV"][:, T - 1:T], (1, 0, 2)))
    case = Case(L, pool, case.table, lens, case.q_codes, case.BK_codes, case.BV_codes,
                case.num_pages)
    ref = case.reference()
    for chunk in (16, 0):
        log(f"peaked, chunk={chunk}")
        check(case, case.run_f64(chunk_tokens=chunk), ref, what=f"peaked chunk {chunk}")


def test_one_workspace_across_calls():
    """One workspace, NaN-filled once and sized for the largest call, serves calls of
    different batches, lengths, layouts and splits in a row, as each left it: in the
    one-launch form the merge of a row waits until every chunk of the row has marked its
    record done for this very call, so neither an earlier call's records and marks (other
    layouts put them at other offsets) nor the NaN fill can pass for this call's.  Every
    output against the oracle."""
    from lrkv_case import fresh_workspace, layout_c
    import factored_rank_kv_amd as F

    big = iid_case(150, 16, 128, 56, O.BF16, [2100, 1100, 5, 700], permute=True, fill=0x7FC0)
    small = iid_case(151, 16, 128, 56, O.BF16, [90, 17], permute=True, fill=0x7FC0)
    many = iid_case(152, 16, 128, 56, O.BF16, [48] * 20 + [300], permute=True, fill=0x7FC0)
    wide = iid_case(153, 32, 128, 32, O.BF16, [64, 129, 700], permute=True, fill=0x7FC0)
    tiny = iid_case(154, 4, 16, 4, O.F32, [1, 15, 90], permute=True, fill=0x7FC00000)
    cases = (big, small, many, wide, tiny)
    nbytes = max(F.lrkv_decode_workspace_bytes(layout_c(c.L), c.B, c.q_len, int(c.lens.max()), ch)
                 for c in cases for ch in (0, 16))
    ws = fresh_workspace(nbytes)
    for c, chunk, what in ((big, 16, "big chunk 16"), (small, 32, "small chunk 32"),
                           (wide, 16, "32 heads chunk 16"), (small, 16, "small chunk 16"),
                           (many, 0, "many automatic"), (many, 16, "many chunk 16"),
                           (tiny, 16, "fp32 chunk 16"), (big, 48, "big chunk 48"),
                           (wide, 0, "32 heads automatic"), (small, 0, "small automatic"),
                           (big, 16, "big chunk 16 again")):
        log(f"shared workspace: {what}")
        got = c.run_f64(chunk_tokens=chunk, ws=ws)
        live = np.array(c.lens) > 0
        check(c, got[live], c.reference()[live], what=what)


def test_repeat_runs_are_bitwise_equal():
    case = iid_case(108, 16, 128, 56, O.BF16, [513, 1000, 31], permute=True)
    log("determinism")
    a = case.run().cpu()
    b = case.run().cpu()
    assert torch.equal(a, b)


@pytest.mark.parametrize("shape", [(4, 16, 4, O.F32), (16, 128, 56, O.BF16)])
def test_multi_row_queries_causal(shape):
    """q_len > 1: row i sees positions j <= T - q_len + i."""
    H, dh, r, dt = shape
    log(f"multi-row queries, shape {shape}")
    case = iid_case(109, H, dh, r, dt, [40, 7, 16], q_len=5, permute=True,
                    fill=0x7FC0 if dt == O.BF16 else 0x7FC00000)
    check(case, case.run_f64(chunk_tokens=16), case.reference(), what=f"multi-row {shape}")


@pytest.mark.parametrize("shape", [(16, 128, 56, O.BF16), (32, 128, 32, O.BF16)])
def test_near_cancelling_shared_and_private(shape):
    """LRKV notes §9 asks for small inputs where the shared key and the private correction
    nearly cancel.  Head 0's shared rows are set to -R[0] B[0]^T plus a small term (keys and
    values alike), so its full keys and values are ~1/100 of either branch; the factored
    sums cancel in float32.  Bar: 1e-2 of max|ref| over all outputs, and also over head 0's
    own outputs alone (a hundred times smaller)."""
    H, dh, r, dt = shape
    lens = [300, 1000, 17]
    g = np.random.default_rng(140 + H)
    L = O.Layout(H, dh, r, 16, dt)
    n = sum(lens)
    bf = lambda x: O.round_to_dtype(np.asarray(x, np.float64), dt)
    RK = bf(g.standard_normal((n, H, r)))
    RV = bf(g.standard_normal((n, H, r)))
    BK = bf(g.standard_normal((H, dh, r)) / np.sqrt(r))
    BV = bf(g.standard_normal((H, dh, r)) / np.sqrt(r))
    SK = bf(-RK[:, 0] @ BK[0].T + 0.01 * g.standard_normal((n, dh)))
    SV = bf(-RV[:, 0] @ BV[0].T + 0.01 * g.standard_normal((n, dh)))
    table, npg = synth.page_assignment(141, lens, 16, True)
    enc = lambda a: O.f64_to_bf16_bits(a)
    pool = O.pack_pool(L, table, lens, enc(SK), enc(SV), enc(RK), enc(RV), npg, fill=0x7FC0)
    q = synth.queries(142, len(lens), 1, H, dh)
    case = Case(L, pool, table, lens, as_codes(q, dt), enc(BK), enc(BV), npg)
    ref = case.reference()
    k0 = O.reconstruct(SK, np.transpose(RK, (1, 0, 2))[:1], BK[:1])[0]
    assert np.abs(k0).max() < 0.1 * np.abs(SK).max()  # the cancellation is real
    for chunk in (0, 16):
        got = case.run_f64(chunk_tokens=chunk)
        check(case, got, ref, what=f"near-cancel {shape} chunk {chunk}, all heads")
        err0 = max_rel_err(got[:, :, 0], ref[:, :, 0])
        log(f"near-cancel {shape} chunk {chunk}: head 0 alone max rel err {err0:.3e}, "
            f"max|ref| {np.abs(ref[:, :, 0]).max():.2e} vs {np.abs(ref).max():.2e} overall")
        assert err0 <= tolerance(dt)
