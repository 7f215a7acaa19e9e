"""GPU parity of lrkv_append (Algorithm 1) against the oracle, through the C-ABI library.

Placement is bit-exact for every input: each byte of the pool is either the projected value
at its (page, slot, section) or the sentinel it held before.  Values are bit-exact when the
arithmetic is exact (entries of X and the weights in {-1, 0, 1}, or one-hot rows); for
Gaussian inputs float32 accumulation then rounding may differ from float64-then-rounding by
one unit in the last place of the cache dtype, and only there.
"""

import numpy as np
import pytest
import torch

import factored_rank_kv_amd as F
import oracle as O
import synth
from lrkv_case import as_codes, codes_f64, layout_c, log, output_major, to_dev

pytestmark = pytest.mark.gpu

SENTINEL_BF16 = 0x7FBF  # a NaN code: no finite projection can produce it


def run_append(L, Xc, wc, req, pos, table, npg, start_pool):
    d = Xc.shape[1]
    pool = to_dev(start_pool)
    dev = {k: to_dev(output_major(v)) for k, v in wc.items()}
    F.lrkv_append(layout_c(L), to_dev(Xc), Xc.shape[0], d, dev["W_SK"], dev["W_SV"], dev["U_K"],
                  dev["U_V"], to_dev(np.asarray(req, np.int32)), to_dev(np.asarray(pos, np.int32)),
                  to_dev(np.ascontiguousarray(table, np.int32)), table.shape[1], pool, npg)
    torch.cuda.synchronize()
    return pool.cpu().numpy()


def expected(L, Xc, wc, req, pos, table, start_pool):
    w64 = {k: codes_f64(v, L.dtype) for k, v in wc.items()}
    return O.append_reference(start_pool, L, codes_f64(Xc, L.dtype), w64["W_SK"], w64["W_SV"],
                              w64["U_K"], w64["U_V"], req, pos, table)


def ternary(g, shape):
    return g.integers(-1, 2, shape).astype(np.float32)


@pytest.mark.parametrize("shape", [(16, 128, 56), (32, 128, 32)])
@pytest.mark.parametrize("n_rows", [1, 5, 8, 9, 13])
def test_exact_inputs_bit_exact_with_sentinels(shape, n_rows):
    """Up to 8 rows go through the two-k-blocks-per-product kernel, 9 to 63 through the
    16-row one: both bit-exact on inputs whose products and sums are exact in float32."""
    H, dh, r = shape
    L = O.Layout(H, dh, r, 16, O.BF16)
    d = 256
    g = np.random.default_rng(200 + n_rows)
    X = ternary(g, (n_rows, d))
    w = {"W_SK": ternary(g, (d, dh)), "W_SV": ternary(g, (d, dh)),
         "U_K": ternary(g, (d, H, r)), "U_V": ternary(g, (d, H, r))}
    wc = {k: as_codes(v, O.BF16) for k, v in w.items()}
    lens = [70, 33, 129]
    table, npg = synth.page_assignment(201, lens, 16, True)
    # distinct (request, position) pairs
    pairs = g.permutation([(b, p) for b, t in enumerate(lens) for p in range(t)])[:n_rows]
    req, pos = pairs[:, 0], pairs[:, 1]
    start = np.full(npg * O.page_elems(L), SENTINEL_BF16, np.uint16).view(np.uint8)
    log(f"append exact, shape {shape}, {n_rows} rows")
    got = run_append(L, as_codes(X, O.BF16), wc, req, pos, table, npg, start)
    exp = expected(L, as_codes(X, O.BF16), wc, req, pos, table, start)
    assert np.array_equal(got, exp)
    assert (got.view(np.uint16) == SENTINEL_BF16).sum() == npg * O.page_elems(L) - \
        n_rows * (2 * dh + 2 * H * r)


@pytest.mark.parametrize("n_rows,d", [(3, 8), (7, 72), (21, 40), (50, 96)])
def test_exact_inputs_small_widths(n_rows, d):
    """Few-row appends with d below one 32-wide block per wavefront (d = 8: only the first
    wavefront has k; d = 40, 72: a partial block, 72 through the 8-row kernel, whose second
    block of each pair lies past d) and with several 16-row blocks."""
    H, dh, r = 16, 128, 56
    L = O.Layout(H, dh, r, 16, O.BF16)
    g = np.random.default_rng(270 + d)
    X = ternary(g, (n_rows, d))
    w = {"W_SK": ternary(g, (d, dh)), "W_SV": ternary(g, (d, dh)),
         "U_K": ternary(g, (d, H, r)), "U_V": ternary(g, (d, H, r))}
    wc = {k: as_codes(v, O.BF16) for k, v in w.items()}
    lens = [40, 33]
    table, npg = synth.page_assignment(271, lens, 16, True)
    pairs = g.permutation([(b, p) for b, t in enumerate(lens) for p in range(t)])[:n_rows]
    req, pos = pairs[:, 0], pairs[:, 1]
    start = np.full(npg * O.page_elems(L), SENTINEL_BF16, np.uint16).view(np.uint8)
    log(f"append exact, {n_rows} rows, d={d}")
    got = run_append(L, as_codes(X, O.BF16), wc, req, pos, table, npg, start)
    exp = expected(L, as_codes(X, O.BF16), wc, req, pos, table, start)
    assert np.array_equal(got, exp)


@pytest.mark.parametrize("shape", [(16, 128, 56), (32, 128, 32)])
@pytest.mark.parametrize("n_rows,d", [(64, 256), (300, 256), (300, 264), (470, 256), (96, 32),
                                      (200, 64), (130, 128), (257, 192), (257, 96)])
def test_exact_inputs_bit_exact_many_rows(shape, n_rows, d):
    """Prefill-sized appends (the MFMA product; d = 32, 96 and 264 are not multiples of its
    64-wide K stage and take the row kernel; d = 64, 128, 192 give one, two and three K
    stages, i.e. the last stage with no next one, one refill, two): exact arithmetic,
    bit-exact pool with sentinels, a ragged last block of rows, permuted pages and scattered
    positions."""
    H, dh, r = shape
    L = O.Layout(H, dh, r, 16, O.BF16)
    g = np.random.default_rng(250 + n_rows + d)
    X = ternary(g, (n_rows, d))
    w = {"W_SK": ternary(g, (d, dh)), "W_SV": ternary(g, (d, dh)),
         "U_K": ternary(g, (d, H, r)), "U_V": ternary(g, (d, H, r))}
    wc = {k: as_codes(v, O.BF16) for k, v in w.items()}
    lens = [200, 150, 129]
    table, npg = synth.page_assignment(251, lens, 16, True)
    pairs = g.permutation([(b, p) for b, t in enumerate(lens) for p in range(t)])[:n_rows]
    req, pos = pairs[:, 0], pairs[:, 1]
    start = np.full(npg * O.page_elems(L), SENTINEL_BF16, np.uint16).view(np.uint8)
    log(f"append exact, shape {shape}, {n_rows} rows, d={d}")
    got = run_append(L, as_codes(X, O.BF16), wc, req, pos, table, npg, start)
    exp = expected(L, as_codes(X, O.BF16), wc, req, pos, table, start)
    assert np.array_equal(got, exp)
    assert (got.view(np.uint16) == SENTINEL_BF16).sum() == npg * O.page_elems(L) - \
        n_rows * (2 * dh + 2 * H * r)


def test_round_to_nearest_even_ties_many_rows():
    """The tie rows of the test below, 48 of each, through the MFMA product (d = 320, five
    K stages)."""
    L = O.Layout(16, 128, 56, 16, O.BF16)
    d, n = 320, 96
    X = np.zeros((n, d), np.float32)
    X[0::2, :257] = 1
    X[1::2, :259] = 1
    ones = lambda s: np.ones(s, np.float32)
    wc = {k: as_codes(v, O.BF16) for k, v in
          {"W_SK": ones((d, 128)), "W_SV": ones((d, 128)), "U_K": ones((d, 16, 56)),
           "U_V": ones((d, 16, 56))}.items()}
    table = np.arange(6, dtype=np.int32)[None, :]
    start = np.zeros(6 * O.page_elems(L), np.uint16).view(np.uint8)
    log("append ties, 96 rows")
    got = run_append(L, as_codes(X, O.BF16), wc, [0] * n, list(range(n)), table, 6, start)
    rows = O.gather_request(got, L, table[0], n)
    assert np.all(rows["SK"][0::2] == 256) and np.all(rows["SK"][1::2] == 260)
    assert np.all(rows["RK"][:, 0::2] == 256) and np.all(rows["RV"][:, 1::2] == 260)


def test_round_to_nearest_even_ties():
    """Products 257 and 259 are ties at bfloat16 spacing 2: they must land on 256 and 260."""
    L = O.Layout(16, 128, 56, 16, O.BF16)
    d = 264
    X = np.zeros((2, d), np.float32)
    X[0, :257] = 1
    X[1, :259] = 1
    ones = lambda s: np.ones(s, np.float32)
    wc = {k: as_codes(v, O.BF16) for k, v in
          {"W_SK": ones((d, 128)), "W_SV": ones((d, 128)), "U_K": ones((d, 16, 56)),
           "U_V": ones((d, 16, 56))}.items()}
    table = np.array([[0]], np.int32)
    start = np.zeros(O.page_elems(L), np.uint16).view(np.uint8)
    log("append ties")
    got = run_append(L, as_codes(X, O.BF16), wc, [0, 0], [0, 1], table, 1, start)
    rows = O.gather_request(got, L, table[0], 2)
    assert np.all(rows["SK"][0] == 256) and np.all(rows["SK"][1] == 260)
    assert np.all(rows["RV"][:, 0] == 256) and np.all(rows["RV"][:, 1] == 260)
    exp = expected(L, as_codes(X, O.BF16), wc, [0, 0], [0, 1], table, start)
    assert np.array_equal(got, exp)


def bf16_ulp(x):
    """Spacing of bfloat16 numbers at |x| (normal range)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0**-126)))
    return 2.0 ** (e - 7)


@pytest.mark.parametrize("work,n_rows", [(synth.C1, 8), (synth.C1, 37), (synth.C3, 4),
                                         (synth.C1, 300), (synth.C3, 200)])
def test_gaussian_rows_within_accumulation_bound(work, n_rows):
    """Gaussian rows: placement bit-exact; each value g (float32 sums, then nearest even)
    against the float64 projection s and its rounding e:
        |g - e| <= ulp(e)/2 + ulp(g)/2 + 2 (d + 2) 2^-24 sum_k |x_k w_k|,
    the rounding of both sides plus the float32 summation error bound (doubled, for any
    summation order).  Away from cancellation this is one ulp; near-cancelling sums (tiny s
    made of large terms) may differ by more, and that is what the bound allows."""
    L = O.Layout(work.H, work.d_h, work.r, 16, O.BF16)
    w = synth.projection_weights(300, work.d, work.H, work.d_h, work.r)
    wc = {k: as_codes(v, O.BF16) for k, v in w.items() if k in ("W_SK", "W_SV", "U_K", "U_V")}
    X = as_codes(synth.activations(301, n_rows, work.d), O.BF16)
    lens = [n_rows + 20, 40]
    table, npg = synth.page_assignment(302 + n_rows, lens, 16, True)
    req = np.zeros(n_rows, np.int64)
    pos = np.arange(n_rows) + 3
    start = np.full(npg * O.page_elems(L), SENTINEL_BF16, np.uint16).view(np.uint8)
    log(f"append gaussian {work.name}, {n_rows} rows")
    got = run_append(L, X, wc, req, pos, table, npg, start)
    exp = expected(L, X, wc, req, pos, table, start)
    g16, e16 = got.view(np.uint16), exp.view(np.uint16)
    placed = e16 != SENTINEL_BF16
    assert np.array_equal(g16[~placed], e16[~placed])  # every other byte untouched
    frac = float(np.mean(g16[placed] != e16[placed]))
    log(f"codes differing from the float64 rounding: {frac:.2e}")
    assert frac < 0.01

    X64 = codes_f64(X, O.BF16)
    w64 = {k: codes_f64(v, O.BF16) for k, v in wc.items()}
    exact = O.project_rows(X64, w64["W_SK"], w64["W_SV"], w64["U_K"], w64["U_V"])
    rows = O.gather_request(got, L, table[0], n_rows + 3)
    gpu = (rows["SK"][3:], rows["SV"][3:], np.transpose(rows["RK"][:, 3:], (1, 0, 2)),
           np.transpose(rows["RV"][:, 3:], (1, 0, 2)))
    gamma = 2 * (work.d + 2) * 2.0 ** -24
    for name, s_val, g_val, W64 in zip(("S_K", "S_V", "R_K", "R_V"), exact, gpu,
                                       (w64["W_SK"], w64["W_SV"], w64["U_K"], w64["U_V"])):
        s_val = s_val.reshape(n_rows, -1)
        g_val = g_val.reshape(n_rows, -1)
        e_val = O.round_to_dtype(s_val, O.BF16)
        mag = np.abs(X64) @ np.abs(W64.reshape(work.d, -1))
        bound = 0.5 * bf16_ulp(e_val) + 0.5 * bf16_ulp(g_val) + gamma * mag
        excess = np.abs(g_val - e_val) / bound
        log(f"{name}: max |g - e| / bound = {excess.max():.3f}")
        assert np.all(excess <= 1.0), name


def test_fp32_rows_within_rounding_bound():
    work = synth.C0
    L = O.Layout(work.H, work.d_h, work.r, 16, O.F32)
    w = synth.projection_weights(0, work.d, work.H, work.d_h, work.r)
    wc = {k: v.view(np.uint32) for k, v in w.items() if k in ("W_SK", "W_SV", "U_K", "U_V")}
    X = synth.activations(1, 65, work.d)
    table, npg = synth.page_assignment(2, [65], 16, True)
    start = np.zeros(npg * O.page_bytes(L), np.uint8)
    log("append fp32 c0")
    got = run_append(L, X.view(np.uint32), wc, np.zeros(65, int), np.arange(65), table, npg, start)
    rows_got = O.gather_request(got, L, table[0], 65)
    SK, SV, RK, RV = O.project_rows(X, w["W_SK"], w["W_SV"], w["U_K"], w["U_V"])
    absd = lambda A, B: np.abs(X.astype(np.float64)) @ np.abs(np.asarray(B, np.float64).reshape(work.d, -1))
    bound_s = absd(X, w["W_SK"]) * (work.d + 1) * 2.0**-24
    assert np.all(np.abs(rows_got["SK"] - SK) <= bound_s)
    bound_r = (absd(X, w["U_V"]) * (work.d + 1) * 2.0**-24).reshape(65, work.H, work.r)
    assert np.all(np.abs(np.transpose(rows_got["RV"], (1, 0, 2)) - RV) <= bound_r)


def test_full_prefill_size_one_hot_rows_bit_exact():
    """C4-sized append: 4 prompts x 8192 rows, d = 2048, into a permuted 2048-page pool.  Each
    row of X is a signed one-hot vector, so every projected value is an exact copy of one
    weight entry and the whole pool must match bit for bit."""
    work = synth.C4
    L = O.Layout(work.H, work.d_h, work.r, 16, O.BF16)
    n = work.tokens
    g = np.random.default_rng(400)
    idx = g.integers(0, work.d, n)
    sign = np.where(g.random(n) < 0.5, -1.0, 1.0).astype(np.float32)
    X = np.zeros((n, work.d), np.float32)
    X[np.arange(n), idx] = sign
    w = synth.projection_weights(401, work.d, work.H, work.d_h, work.r)
    wc = {k: as_codes(v, O.BF16) for k, v in w.items() if k in ("W_SK", "W_SV", "U_K", "U_V")}
    table, npg = synth.page_assignment(402, list(work.lens), 16, True)
    req = np.repeat(np.arange(work.B), work.lens[0])
    pos = np.tile(np.arange(work.lens[0]), work.B)
    start = np.full(npg * O.page_elems(L), SENTINEL_BF16, np.uint16).view(np.uint8)
    Xc = as_codes(X, O.BF16)
    log(f"append one-hot, {n} rows, {npg} pages")
    got = run_append(L, Xc, wc, req, pos, table, npg, start)
    log("oracle expected pool")
    # the projection of a signed one-hot row is a signed copy of one weight row: the oracle
    # computes it as a float64 product like any other row
    exp = expected(L, Xc, wc, req, pos, table, start)
    assert np.array_equal(got, exp)


def test_reappend_after_wipe_is_bit_identical():
    """Recovery by re-append: wipe the pool, append the same rows again, same bytes."""
    work = synth.C1
    L = O.Layout(work.H, work.d_h, work.r, 16, O.BF16)
    w = synth.projection_weights(500, work.d, work.H, work.d_h, work.r)
    wc = {k: as_codes(v, O.BF16) for k, v in w.items() if k in ("W_SK", "W_SV", "U_K", "U_V")}
    X = as_codes(synth.activations(501, 48, work.d), O.BF16)
    table, npg = synth.page_assignment(502, [48], 16, True)
    start = np.zeros(npg * O.page_bytes(L), np.uint8)
    a = run_append(L, X, wc, np.zeros(48, int), np.arange(48), table, npg, start)
    b = run_append(L, X, wc, np.zeros(48, int), np.arange(48), table, npg, start)
    assert np.array_equal(a, b)


def test_rows_spanning_more_than_4_gib_of_x():
    """X rows spanning more than 4 GiB (d = 8192: 262,656 rows of 16 KiB, 4.3 GB) go out in
    several launches, the product addressing X rows by 32-bit offsets.  One-hot rows (each
    projected value is one weight entry, so the result is exact); every 5th row of the last
    1,600 (the region holding the launch boundary) and a spread of earlier rows are compared
    with the oracle: its projection of those rows, written over a copy of the library's
    pages that hold them, must leave those pages unchanged byte for byte."""
    L = O.Layout(16, 128, 56, 16, O.BF16)
    d, n = 8192, 262_656
    assert n * d * 2 > 2**32
    g = np.random.default_rng(410)
    idx = g.integers(0, d, n)
    neg = g.random(n) < 0.5
    dev = torch.device("cuda")
    log(f"append of {n} one-hot rows, d = {d} ({n * d * 2 / 1e9:.2f} GB of X)")
    X = torch.zeros((n, d), dtype=torch.int16, device=dev)
    one = torch.from_numpy(np.where(neg, np.int16(-16512), np.int16(0x3F80))).to(dev)  # -1.0, 1.0
    X[torch.arange(n, device=dev), torch.from_numpy(idx).to(dev)] = one
    w = synth.projection_weights(411, d, L.num_heads, L.head_dim, L.rank)
    wc = {k: as_codes(v, O.BF16) for k, v in w.items() if k in ("W_SK", "W_SV", "U_K", "U_V")}
    table, npg = synth.page_assignment(412, [n], 16, True)
    pb = O.page_bytes(L)
    pool = torch.full((npg * pb // 2,), SENTINEL_BF16, dtype=torch.int16, device=dev)
    pool = pool.view(torch.uint8)
    wdev = {k: to_dev(output_major(v)) for k, v in wc.items()}
    req = torch.zeros(n, dtype=torch.int32, device=dev)
    pos = torch.arange(n, dtype=torch.int32, device=dev)
    F.lrkv_append(layout_c(L), X, n, d, wdev["W_SK"], wdev["W_SV"], wdev["U_K"], wdev["U_V"], req,
                  pos, to_dev(np.ascontiguousarray(table, np.int32)), table.shape[1], pool, npg)
    torch.cuda.synchronize()
    del X
    rows = np.unique(np.concatenate([np.arange(n - 1600, n, 5), g.integers(0, n - 1600, 64),
                                     [0, n - 1]]))
    pages = table[0, rows // 16]
    uniq, inv = np.unique(pages, return_inverse=True)
    got = pool.view(npg, pb)[torch.from_numpy(uniq.astype(np.int64)).to(dev)].cpu().numpy()
    got = got.reshape(-1)
    table_c = np.zeros_like(table)
    table_c[0, rows // 16] = inv
    Xs = np.zeros((len(rows), d), np.float64)
    Xs[np.arange(len(rows)), idx[rows]] = np.where(neg[rows], -1.0, 1.0)
    w64 = {k: codes_f64(v, O.BF16) for k, v in wc.items()}
    log(f"oracle projection of {len(rows)} sampled rows over {len(uniq)} pages")
    exp = O.append_reference(got.copy(), L, Xs, w64["W_SK"], w64["W_SV"], w64["U_K"], w64["U_V"],
                             np.zeros(len(rows), np.int64), rows, table_c)
    assert np.array_equal(got, exp)
