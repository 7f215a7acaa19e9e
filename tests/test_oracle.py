"""Pins of the float64 oracle against what the page and the mathematics fix.

Each test checks the oracle against something other than itself: values printed on the
LRKV notes page (golden fixtures, cited inside them), closed forms, library routines that
reduce to textbook attention (torch scaled-dot-product attention in float64), brute force
in pure Python on tiny inputs, and mutants planted here on the CPU that must fail.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# --------------------------------------------------------------------------------------
# helpers that build small paged caches from random codes (oracle placement + synth draws)
# --------------------------------------------------------------------------------------


def random_case(seed, H, d_h, r, dtype, lens, q_len=1, permute=True, fill=0):
    L = O.Layout(H, d_h, r, 16, dtype)
    g = np.random.default_rng(seed)
    n = int(sum(lens))

    def codes(shape):
        x = g.standard_normal(shape).astype(np.float32)
        if dtype == O.BF16:
            return synth.to_bf16_bits(x)
        return x.view(np.uint32)

    SK, SV = codes((n, d_h)), codes((n, d_h))
    RK, RV = codes((n, H, r)), codes((n, H, r))
    table, num_pages = synth.page_assignment(seed + 1, lens, 16, permute)
    pool = O.pack_pool(L, table, lens, SK, SV, RK, RV, num_pages, fill=fill)
    q = g.standard_normal((len(lens), q_len, H, d_h))
    BK = g.standard_normal((H, d_h, r)) / math.sqrt(max(r, 1))
    BV = g.standard_normal((H, d_h, r)) / math.sqrt(max(r, 1))
    return L, pool, table, np.asarray(lens), q, BK, BV


def sdpa(q, K, V):
    """torch's scaled-dot-product attention, float64, CPU, one query row."""
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(np.asarray(q, np.float64))[None, None, None, :],
        torch.from_numpy(np.asarray(K, np.float64))[None, None],
        torch.from_numpy(np.asarray(V, np.float64))[None, None])
    return out[0, 0, 0].numpy()


# --------------------------------------------------------------------------------------
# worked example (LRKV notes §3)
# --------------------------------------------------------------------------------------


def test_worked_example_scores():
    g = gold("worked_example.json")
    q = np.array(g["q"], float)
    S = np.array([g["shared_key"]], float)  # [T=1, d_h=2]
    R = np.array([[[g["private_coordinate"]]]], float)  # [H=1, T=1, r=1]
    Bm = np.array([[[g["basis_column"][0]], [g["basis_column"][1]]]], float)  # [1, 2, 1]
    K = O.reconstruct(S, R, Bm)[0, 0]
    assert K.tolist() == g["full_key"]
    assert q @ K == g["score_unscaled"]
    assert q @ S[0] == g["shared_score_unscaled"]
    p = q @ Bm[0]
    assert p.tolist() == [g["private_query"]]
    assert float(p @ R[0, 0]) == g["private_score_unscaled"]


def test_worked_example_values_through_softmax():
    """Two keys whose scaled scores differ by ln 3 get weights 1/4 and 3/4; with private
    value coordinates 2 and 6 and basis column (1, -1), the output is (5, -5)."""
    g = gold("worked_example.json")
    q = np.array(g["q"], float)
    d_h = 2
    rho1 = g["private_coordinate"]
    rho0 = rho1 - math.sqrt(d_h) * math.log(3.0)
    S_K = np.array([g["shared_key"], g["shared_key"]], float)
    R_K = np.array([[[rho0], [rho1]]])
    col = np.array(g["basis_column"], float).reshape(1, 2, 1)
    S_V = np.zeros((2, 2))  # the example has no shared value term
    R_V = np.array([[[c] for c in g["private_value_coordinates"]]], float)
    K = O.reconstruct(S_K, R_K, col)[0]
    V = O.reconstruct(S_V, R_V, col)[0]
    o = O.softmax_attention(q, K, V, 1.0 / math.sqrt(d_h))
    assert np.allclose(o, g["output"], rtol=0, atol=1e-12)
    # the same through block state + one expansion (the softmax, value and output steps of Algorithm 2)
    s = (S_K @ q + (R_K[0] @ (q @ col[0]))) / math.sqrt(d_h)
    st = O.block_state(s, S_V, R_V[0])
    w = np.exp(s - st[0]) / st[1]
    assert np.allclose(w, g["weights"], atol=1e-15)
    assert abs(st[3][0] / st[1] - g["reduced_private"]) < 1e-12
    assert np.allclose(O.finish_state(st, col[0]), g["output"], atol=1e-12)


# --------------------------------------------------------------------------------------
# single softmax over summed branches; scale 1/sqrt(d_h)  (LRKV notes §2)
# --------------------------------------------------------------------------------------


def _two_branch_case():
    """Shared scaled scores (2, 0), private scaled scores (0, 2); values chosen so the two
    value branches read different coordinates."""
    d_h = 2
    q = np.array([2 * math.sqrt(2), 0.0])
    S_K = np.array([[1.0, 0.0], [0.0, 0.0]])
    R_K = np.array([[[0.0], [1.0]]])
    B_K = np.array([[[1.0], [0.0]]])
    S_V = np.array([[1.0, 0.0], [0.0, 0.0]])
    R_V = np.array([[[0.0], [1.0]]])
    B_V = np.array([[[0.0], [1.0]]])
    return d_h, q, S_K, R_K, B_K, S_V, R_V, B_V


def test_single_softmax_over_summed_branches():
    d_h, q, S_K, R_K, B_K, S_V, R_V, B_V = _two_branch_case()
    scale = 1 / math.sqrt(d_h)
    assert np.allclose(S_K @ q * scale, [2, 0])
    assert np.allclose(R_K[0] @ (q @ B_K[0]) * scale, [0, 2])
    K = O.reconstruct(S_K, R_K, B_K)[0]
    V = O.reconstruct(S_V, R_V, B_V)[0]
    o = O.softmax_attention(q, K, V, scale)
    assert np.allclose(o, [0.5, 0.5], atol=1e-15)  # summed scores (2, 2): weights 1/2, 1/2


def test_mutant_separate_softmax_fails():
    """Planted mistake: one softmax per branch.  It must miss the oracle by far more than any
    tolerance used for the GPU path."""
    d_h, q, S_K, R_K, B_K, S_V, R_V, B_V = _two_branch_case()
    scale = 1 / math.sqrt(d_h)
    sh = S_K @ q * scale
    pr = R_K[0] @ (q @ B_K[0]) * scale
    a_sh = np.exp(sh - sh.max()) / np.exp(sh - sh.max()).sum()
    a_pr = np.exp(pr - pr.max()) / np.exp(pr - pr.max()).sum()
    mutant = a_sh @ S_V + (a_pr @ R_V[0]) @ B_V[0].T
    good = O.softmax_attention(q, O.reconstruct(S_K, R_K, B_K)[0],
                               O.reconstruct(S_V, R_V, B_V)[0], scale)
    assert rel_err(mutant, good) > 0.5


def test_scale_closed_form():
    """Two keys with unscaled scores x and 0: weight of the first is 1 / (1 + e^(-x/sqrt(d_h)))."""
    d_h, x = 16, 8.0
    q = np.zeros(d_h)
    q[0] = x
    K = np.zeros((2, d_h))
    K[0, 0] = 1.0
    V = np.eye(2, d_h)
    o = O.softmax_attention(q, K, V, 1 / math.sqrt(d_h))
    a0 = 1 / (1 + math.exp(-x / math.sqrt(d_h)))
    assert abs(o[0] - a0) < 1e-15 and abs(o[1] - (1 - a0)) < 1e-15


def test_mutant_sqrt_r_scale_fails():
    """Planted mistake: dividing by sqrt(r) instead of sqrt(d_h) misses the oracle on a C0-sized
    case by much more than the 1e-5 float32 tolerance."""
    L, pool, table, lens, q, BK, BV = random_case(3, 4, 16, 4, O.F32, [65], permute=False)
    good = O.decode_reference(L, q, BK, BV, pool, table, lens)
    rows = O.gather_request(pool, L, table[0], 65)
    mut = np.zeros_like(good)
    for h in range(4):
        K = O.reconstruct(rows["SK"], rows["RK"][h:h + 1], BK[h:h + 1])[0]
        V = O.reconstruct(rows["SV"], rows["RV"][h:h + 1], BV[h:h + 1])[0]
        mut[0, 0, h] = O.softmax_attention(q[0, 0, h], K, V, 1 / math.sqrt(4))
    assert rel_err(mut, good) > 1e-2


# --------------------------------------------------------------------------------------
# special cases that reduce to textbook attention (torch SDPA, float64)
# --------------------------------------------------------------------------------------


def test_rank0_is_mqa():
    L, pool, table, lens, q, BK, BV = random_case(5, 3, 16, 0, O.F32, [37])
    out = O.decode_reference(L, q, BK, BV, pool, table, lens)
    SK, SV = O.gather_shared(pool, L, table[0], 37)
    for h in range(3):
        assert rel_err(out[0, 0, h], sdpa(q[0, 0, h], SK, SV)) < 1e-13
    out2 = O.decode_algorithm2(L, q, BK, BV, pool, table, lens)
    assert rel_err(out2, out) < 1e-13


def test_zero_basis_is_mqa():
    L, pool, table, lens, q, BK, BV = random_case(6, 4, 16, 4, O.F32, [29])
    z = np.zeros_like(BK)
    out = O.decode_reference(L, q, z, z, pool, table, lens)
    SK, SV = O.gather_shared(pool, L, table[0], 29)
    for h in range(4):
        assert rel_err(out[0, 0, h], sdpa(q[0, 0, h], SK, SV)) < 1e-13


def test_full_rank_identity_basis_is_mha():
    """r = d_h with S = 0 and B = I: every head attends over its own private rows (MHA)."""
    H, d_h, n = 2, 8, 21
    L = O.Layout(H, d_h, d_h, 16, O.F32)
    g = np.random.default_rng(7)
    RK = g.standard_normal((n, H, d_h)).astype(np.float32)
    RV = g.standard_normal((n, H, d_h)).astype(np.float32)
    z = np.zeros((n, d_h), np.float32)
    table, npg = synth.page_assignment(8, [n], 16, True)
    pool = O.pack_pool(L, table, [n], z.view(np.uint32), z.view(np.uint32),
                       RK.view(np.uint32), RV.view(np.uint32), npg)
    q = g.standard_normal((1, 1, H, d_h))
    eye = np.stack([np.eye(d_h)] * H)
    out = O.decode_reference(L, q, eye, eye, pool, table, [n])
    for h in range(H):
        ref = sdpa(q[0, 0, h], RK[:, h].astype(np.float64), RV[:, h].astype(np.float64))
        assert rel_err(out[0, 0, h], ref) < 1e-13


def test_one_visible_token_returns_its_value():
    L, pool, table, lens, q, BK, BV = random_case(9, 4, 16, 4, O.F32, [1])
    out = O.decode_reference(L, q, BK, BV, pool, table, lens)
    rows = O.gather_request(pool, L, table[0], 1)
    V = O.reconstruct(rows["SV"], rows["RV"], BV)
    assert np.array_equal(out[0, 0], V[:, 0, :])


def test_zero_query_gives_mean_value():
    L, pool, table, lens, q, BK, BV = random_case(10, 4, 16, 4, O.F32, [23])
    q = np.zeros_like(q)
    out = O.decode_reference(L, q, BK, BV, pool, table, lens)
    rows = O.gather_request(pool, L, table[0], 23)
    V = O.reconstruct(rows["SV"], rows["RV"], BV)
    assert rel_err(out[0, 0], V.mean(axis=1)) < 1e-14


def test_dominant_key_selects_its_value():
    d_h = 16
    g = np.random.default_rng(11)
    K = g.standard_normal((9, d_h))
    V = g.standard_normal((9, d_h))
    q = 400.0 * K[4] / np.linalg.norm(K[4]) ** 2  # q.K[4] = 400, the others are far below
    K[np.arange(9) != 4] *= 0.01
    o = O.softmax_attention(q, K, V, 1 / math.sqrt(d_h))
    assert np.allclose(o, V[4], atol=1e-12)


def test_empty_request_is_zero():
    L, pool, table, lens, q, BK, BV = random_case(12, 4, 16, 4, O.F32, [0, 5])
    out = O.decode_reference(L, q, BK, BV, pool, table, lens)
    assert np.all(out[0] == 0)
    assert np.all(np.isfinite(out[1]))


# --------------------------------------------------------------------------------------
# the two codings of the path agree; brute force on tiny inputs
# --------------------------------------------------------------------------------------


@pytest.mark.parametrize("dtype", [O.F32, O.BF16])
@pytest.mark.parametrize("q_len", [1, 3])
def test_algorithm2_matches_plain_definition(dtype, q_len):
    d_h, r = (16, 8) if dtype == O.BF16 else (16, 4)
    L, pool, table, lens, q, BK, BV = random_case(13 + q_len, 4, d_h, r, dtype,
                                                  [40, 1, 17, 0, 33], q_len=q_len)
    a = O.decode_reference(L, q, BK, BV, pool, table, lens)
    b = O.decode_algorithm2(L, q, BK, BV, pool, table, lens)
    assert rel_err(b, a) < 1e-12


def test_brute_force_tiny():
    """Pure-Python loops (no numpy arithmetic) for one tiny request, all heads, q_len = 2."""
    H, d_h, r, n = 2, 4, 4, 5
    L, pool, table, lens, q, BK, BV = random_case(21, H, d_h, r, O.F32, [n], q_len=2)
    rows = O.gather_request(pool, L, table[0], n)  # page walk pinned separately below
    SK, SV, RK, RV = (rows[k].tolist() for k in ("SK", "SV", "RK", "RV"))
    out = O.decode_reference(L, q, BK, BV, pool, table, lens)
    for i in range(2):
        vis = n - 2 + i + 1
        for h in range(H):
            keys, vals = [], []
            for j in range(vis):
                keys.append([SK[j][k] + sum(RK[h][j][m] * BK[h][k][m] for m in range(r))
                             for k in range(d_h)])
                vals.append([SV[j][k] + sum(RV[h][j][m] * BV[h][k][m] for m in range(r))
                             for k in range(d_h)])
            s = [sum(q[0, i, h, k] * keys[j][k] for k in range(d_h)) / math.sqrt(d_h)
                 for j in range(vis)]
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            tot = sum(e)
            o = [sum(e[j] / tot * vals[j][k] for j in range(vis)) for k in range(d_h)]
            assert rel_err(out[0, i, h], o) < 1e-13


def test_factored_rows_equal_full_projection():
    """eq 2-5: S + R_h B_h^T built from the cached factors equals X (W_S + U_h B_h^T)."""
    w = synth.projection_weights(0, 64, 4, 16, 4)
    X = synth.activations(100, 65, 64)
    SK, SV, RK, RV = O.project_rows(X, w["W_SK"], w["W_SV"], w["U_K"], w["U_V"])
    K_fac = O.reconstruct(SK, np.transpose(RK, (1, 0, 2)), w["B_K"])
    V_fac = O.reconstruct(SV, np.transpose(RV, (1, 0, 2)), w["B_V"])
    assert rel_err(K_fac, O.full_projection_kv(X, w["W_SK"], w["U_K"], w["B_K"])) < 1e-13
    assert rel_err(V_fac, O.full_projection_kv(X, w["W_SV"], w["U_V"], w["B_V"])) < 1e-13


def test_visible_count():
    assert O.visible_count(10, 1, 0) == 10  # decode sees every cached token
    assert [O.visible_count(4, 4, i) for i in range(4)] == [1, 2, 3, 4]  # causal prefill
    assert [O.visible_count(6, 2, i) for i in range(2)] == [5, 6]
    assert O.visible_count(0, 1, 0) == 0


# --------------------------------------------------------------------------------------
# split / merge of block states (fused blockwise paragraph of §3)
# --------------------------------------------------------------------------------------


def test_merge_of_blocks_equals_whole_and_definition():
    L, pool, table, lens, q, BK, BV = random_case(31, 4, 16, 4, O.F32, [77])
    ref = O.decode_reference(L, q, BK, BV, pool, table, lens)
    rows = O.gather_request(pool, L, table[0], 77)
    for h in range(4):
        p = q[0, 0, h] @ BK[h]
        s = (rows["SK"] @ q[0, 0, h] + rows["RK"][h] @ p) / math.sqrt(16)
        whole = O.block_state(s, rows["SV"], rows["RV"][h])
        cuts = [0, 5, 16, 17, 48, 77]
        parts = [O.block_state(s[a:b], rows["SV"][a:b], rows["RV"][h][a:b])
                 for a, b in zip(cuts, cuts[1:])]
        merged = O.merge_states(parts)
        merged_rev = O.merge_states(parts[::-1])
        for x, y in zip(merged, whole):
            assert rel_err(x, y) < 1e-13
        for x, y in zip(merged_rev, merged):
            assert rel_err(x, y) < 1e-13
        assert rel_err(O.finish_state(merged, BV[h]), ref[0, 0, h]) < 1e-13
    # peaked scores with the max in the last block still merge exactly
    s = np.array([0.0, -3.0, 1.0, 60.0])
    sv = np.eye(4)
    st = O.merge_states([O.block_state(s[:2], sv[:2], sv[:2]), O.block_state(s[2:], sv[2:], sv[2:])])
    assert rel_err(st[2] / st[1], np.exp(s - 60) / np.exp(s - 60).sum()) < 1e-15


# --------------------------------------------------------------------------------------
# cache size and cost models (LRKV notes §4, eq 9) against the page's printed numbers
# --------------------------------------------------------------------------------------


def _pct(fr, nd):
    return f"{float(fr) * 100:.{nd}f}"


def test_printed_cache_percentages():
    g = gold("cache_figures.json")
    for row in g["ratios"]:
        nd = len(row["percent"].split(".")[1])
        assert _pct(O.cache_ratio(row["H"], row["r"], row["d_h"]), nd) == row["percent"], row
    t12 = g["payload_ratio_table12"]
    assert f"{t12['lrkv'] / t12['mha'] * 100:.2f}" == t12["percent"]
    assert _pct(O.cache_ratio(18, 64, 128), 2) == t12["percent"]


def test_printed_mib_budgets():
    for row in gold("cache_figures.json")["budgets_mib"]:
        mha = O.mha_cache_bytes(row["bytes_per_elem"], row["layers"], row["tokens"], row["d_h"],
                                row["H"])
        lrkv = O.lrkv_cache_bytes(row["bytes_per_elem"], row["layers"], row["tokens"],
                                  row["d_h"], row["H"], row["r"])
        assert Fraction(mha, 2**20) == Fraction(row["mha_mib"]).limit_denominator(10**6)
        assert Fraction(lrkv, 2**20) == Fraction(str(row["lrkv_mib"]))


def test_rank_budgets_and_workload_ratios():
    g = gold("cache_figures.json")
    for row in g["rank_budgets"]:
        assert O.rank_budget(row["d_h"], Fraction(*row["c"]), row["H"]) == row["r_max"]
    # the workloads' own shapes
    assert O.rank_budget(128, Fraction(1, 2), 16) == 56
    assert O.cache_ratio(16, 56, 128) == Fraction(1, 2)
    assert O.cache_ratio(32, 32, 128) == Fraction(9, 32)  # 0.28125
    assert O.cache_ratio(4, 4, 16) == Fraction(1, 2)


def test_cost_models():
    g = gold("cache_figures.json")
    pr = g["param_ratio"]
    assert _pct(O.param_ratio(pr["H"], pr["r"], pr["d_h"], pr["d"]), 1) == pr["percent"]
    dm = g["decode_multiplier"]
    assert f"{float(O.decode_arith_ratio(10**9, dm['r'], dm['d_h'])):.2f}" == dm["value"]
    assert O.decode_arith_ratio(4096, 55, 128) == 1 + Fraction(55, 128) + Fraction(55, 4096)
    for row in g["tp_replication"]:
        assert _pct(O.tp_replicated_ratio(row["P"], row["H"], row["r"], row["d_h"]), 1) == \
            row["percent"]


def test_roofline_time_takes_the_larger_term():
    """t >= max(bytes / bandwidth, flops / rate) (LRKV notes §4): with unequal terms the
    bound is the larger one, whichever it is (a min, a sum or a swapped pair fails)."""
    # bandwidth-bound: 1.6e9 B at 8e12 B/s = 0.2 ms against 1e11 FLOP at 2.5e15/s = 0.04 ms
    assert O.roofline_time(1.6e9, 1e11, 8e12, 2.5e15) == pytest.approx(2e-4, rel=1e-15)
    # compute-bound: 8e8 B = 0.1 ms against 1e12 FLOP = 0.4 ms
    assert O.roofline_time(8e8, 1e12, 8e12, 2.5e15) == pytest.approx(4e-4, rel=1e-15)
    # the workload's own numbers: 134,217,728 B at 8 TB/s is 16.78 us; 389,545,984 FLOP at
    # 157.3 TFLOP/s is 2.48 us, so the bytes decide
    assert O.roofline_time(134217728, 389545984, 8e12, 157.3e12) == pytest.approx(
        134217728 / 8e12, rel=1e-15)


@pytest.mark.parametrize("shape", [(4, 16, 4, O.F32), (16, 128, 56, O.BF16),
                                   (32, 128, 32, O.BF16), (18, 128, 56, O.BF16)])
def test_page_bytes_ratio_equals_eq9(shape):
    H, d_h, r, dt = shape
    L = O.Layout(H, d_h, r, 16, dt)
    dense_page = 16 * 2 * H * d_h * L.elem_bytes
    assert Fraction(O.page_bytes(L), dense_page) == O.cache_ratio(H, r, d_h)


# --------------------------------------------------------------------------------------
# element encodings
# --------------------------------------------------------------------------------------


def test_bf16_round_to_nearest_even_ties():
    x = np.array([257.0, 259.0, 258.0, -257.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8])
    got = O.bf16_bits_to_f64(O.f64_to_bf16_bits(x))
    assert got.tolist() == [256.0, 260.0, 258.0, -256.0, 1.0, 1.0 + 2**-6]


def test_bf16_matches_torch_on_float32_inputs():
    g = np.random.default_rng(41)
    x = np.concatenate([
        g.standard_normal(20000).astype(np.float32),
        (g.standard_normal(2000) * 1e-39).astype(np.float32),  # subnormal range
        (g.standard_normal(2000) * 1e37).astype(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, 3.4e38, 1e-45], np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.f64_to_bf16_bits(x.astype(np.float64))
    assert np.array_equal(got, ref)
    assert O.f64_to_bf16_bits(np.array([np.nan]))[0] == 0x7FC0


def test_bf16_rounds_float64_once():
    # 1 + 2^-8 + 2^-40 lies just above a tie: one rounding goes up; rounding to float32 first
    # would land exactly on the tie and go down to 1.0
    x = np.array([1.0 + 2**-8 + 2**-40])
    assert O.bf16_bits_to_f64(O.f64_to_bf16_bits(x))[0] == 1.0 + 2**-7


# --------------------------------------------------------------------------------------
# page layout: hand-worked byte map, bulk packing vs per-row placement vs page walk
# --------------------------------------------------------------------------------------


def test_page_layout_byte_map():
    g = gold("page_layout.json")
    L = O.Layout(**g["layout"])
    assert O.page_bytes(L) == g["page_bytes"]
    width = {"SK": L.head_dim, "SV": L.head_dim, "RK": L.rank, "RV": L.rank}
    for e in g["elements"]:
        idx = O.section_base(L, e["section"], e["head"]) + O.in_block_index(
            L, width[e["section"]], np.array(e["t"]), np.array(e["k"]))
        assert int(idx) * L.elem_bytes == e["byte"], e


@pytest.mark.parametrize("dtype", [O.F32, O.BF16])
def test_pack_walk_roundtrip_and_permutation_invariance(dtype):
    H, d_h, r = (3, 16, 8)
    lens = [33, 16, 1, 0, 50]
    L = O.Layout(H, d_h, r, 16, dtype)
    g = np.random.default_rng(51)
    n = sum(lens)
    st = O.storage_dtype(L)
    if dtype == O.BF16:
        mk = lambda s: synth.to_bf16_bits(g.standard_normal(s).astype(np.float32))
    else:
        mk = lambda s: g.standard_normal(s).astype(np.float32).view(st)
    SK, SV, RK, RV = mk((n, d_h)), mk((n, d_h)), mk((n, H, r)), mk((n, H, r))
    results = []
    for permute in (False, True):
        table, npg = synth.page_assignment(52, lens, 16, permute)
        pool = O.pack_pool(L, table, lens, SK, SV, RK, RV, npg, fill=0x7FC0 if dtype else 0)
        off = 0
        rows_all = []
        for b, T in enumerate(lens):
            rows = O.gather_request(pool, L, table[b], T)
            dec = lambda c: O.decode_elems(np.ascontiguousarray(c).view(np.uint8), dtype).reshape(c.shape)
            assert np.array_equal(rows["SK"], dec(SK[off:off + T]))
            assert np.array_equal(rows["SV"], dec(SV[off:off + T]))
            assert np.array_equal(rows["RK"], np.transpose(dec(RK[off:off + T]), (1, 0, 2)))
            assert np.array_equal(rows["RV"], np.transpose(dec(RV[off:off + T]), (1, 0, 2)))
            rows_all.append(rows)
            off += T
        results.append(rows_all)
    for a, b in zip(*results):
        for k in a:
            assert np.array_equal(a[k], b[k])


def test_write_rows_agrees_with_bulk_packing():
    H, d_h, r, lens = 2, 16, 8, [20, 35]
    L = O.Layout(H, d_h, r, 16, O.BF16)
    g = np.random.default_rng(61)
    n = sum(lens)
    vals = lambda s: O.round_to_dtype(g.standard_normal(s), O.BF16)
    SK, SV, RK, RV = vals((n, d_h)), vals((n, d_h)), vals((n, H, r)), vals((n, H, r))
    table, npg = synth.page_assignment(62, lens, 16, True)
    codes = lambda a: O.f64_to_bf16_bits(a)
    bulk = O.pack_pool(L, table, lens, codes(SK), codes(SV), codes(RK), codes(RV), npg, fill=0x1234)
    req = np.repeat(np.arange(2), lens)
    pos = np.concatenate([np.arange(t) for t in lens])
    start = np.full(npg * O.page_elems(L), 0x1234, np.uint16).view(np.uint8)
    order = g.permutation(n)  # placement order must not matter
    rowwise = O.write_rows(start, L, table, req[order], pos[order], SK[order], SV[order],
                           RK[order], RV[order])
    assert np.array_equal(bulk, rowwise)


# --------------------------------------------------------------------------------------
# Algorithm 1 append oracle
# --------------------------------------------------------------------------------------


def test_append_exact_integer_inputs_and_sentinels():
    """X and weights in {-1, 0, 1} with d <= 256: every projection is an integer of magnitude
    <= 256, exact in bfloat16; the expected pool must hold exactly the integer products at the
    rows' slots, and the sentinel everywhere else."""
    H, d_h, r, d = 2, 16, 8, 256
    L = O.Layout(H, d_h, r, 16, O.BF16)
    g = np.random.default_rng(71)
    X = g.integers(-1, 2, (5, d))
    W_SK, W_SV = g.integers(-1, 2, (d, d_h)), g.integers(-1, 2, (d, d_h))
    U_K, U_V = g.integers(-1, 2, (d, H, r)), g.integers(-1, 2, (d, H, r))
    table, npg = synth.page_assignment(72, [40, 9], 16, True)
    req = np.array([0, 1, 0, 1, 0])
    pos = np.array([39, 0, 16, 8, 3])
    start = np.full(npg * O.page_elems(L), 0xBEEF, np.uint16).view(np.uint8)
    got = O.append_reference(start, L, X, W_SK, W_SV, U_K, U_V, req, pos, table)
    exp = start.copy().view(np.uint16)
    pe = O.page_elems(L)
    ints = {"SK": X @ W_SK, "SV": X @ W_SV,
            "RK": (X @ U_K.reshape(d, -1)).reshape(-1, H, r),
            "RV": (X @ U_V.reshape(d, -1)).reshape(-1, H, r)}
    for n in range(5):
        page = table[req[n], pos[n] // 16]
        t = pos[n] % 16
        for sec in ("SK", "SV"):
            for k in range(d_h):
                i = page * pe + O.section_base(L, sec) + O.in_block_index(L, d_h, t, k)
                exp[i] = O.f64_to_bf16_bits(np.array([float(ints[sec][n, k])]))[0]
        for sec in ("RK", "RV"):
            for h in range(H):
                for k in range(r):
                    i = page * pe + O.section_base(L, sec, h) + O.in_block_index(L, r, t, k)
                    exp[i] = O.f64_to_bf16_bits(np.array([float(ints[sec][n, h, k])]))[0]
    assert np.array_equal(got.view(np.uint16), exp)
    assert np.abs(ints["SK"]).max() <= 256


def test_append_rne_ties():
    """Dot products equal to 257 and 259 are ties at bfloat16 spacing 2 and must round to
    256 and 260 (nearest even)."""
    L = O.Layout(1, 16, 8, 16, O.BF16)
    d = 259
    X = np.ones((2, d))
    X[0, 257:] = 0  # row 0 sums 257 ones, row 1 sums 259
    W = np.ones((d, 16))
    U = np.ones((d, 1, 8))
    table = np.array([[0]], np.int32)
    start = np.zeros(O.page_elems(L), np.uint16).view(np.uint8)
    got = O.append_reference(start, L, X, W, W, U, U, [0, 0], [0, 1], table)
    rows = O.gather_request(got, L, table[0], 2)
    assert rows["SK"][:, 0].tolist() == [256.0, 260.0]
    assert rows["RV"][0, :, 7].tolist() == [256.0, 260.0]


# --------------------------------------------------------------------------------------
# planted mistakes in the oracle itself (on the CPU): each must make a pin above fail
# --------------------------------------------------------------------------------------


def _drop_private(S, R, Bm):
    S = np.asarray(S, np.float64)
    return np.broadcast_to(S[None], (np.shape(R)[0],) + S.shape).copy()


def _untransposed_basis(S, R, Bm):
    return np.asarray(S, np.float64)[None] + np.matmul(np.asarray(R, np.float64),
                                                       np.asarray(Bm, np.float64))


def test_full_rank_random_basis_matches_full_projection():
    """r = d_h with a random (non-symmetric) basis: the oracle over the factored cache equals
    textbook attention over keys and values projected straight through W_h = W_S + U_h B_h^T
    (eq 2), so an oracle that applied B_h instead of B_h^T would miss."""
    H, d_h, d, n = 2, 8, 24, 19
    w = synth.projection_weights(90, d, H, d_h, d_h, with_wq=True)
    X = synth.activations(91, n, d).astype(np.float64)
    L = O.Layout(H, d_h, d_h, 16, O.F32)
    SK, SV, RK, RV = O.project_rows(X, w["W_SK"], w["W_SV"], w["U_K"], w["U_V"])
    f32 = lambda a: np.ascontiguousarray(a, np.float32).view(np.uint32)
    table, npg = synth.page_assignment(92, [n], 16, True)
    pool = O.pack_pool(L, table, [n], f32(SK), f32(SV), f32(RK), f32(RV), npg)
    rnd = lambda a: np.asarray(a, np.float32).astype(np.float64)
    q = X[-1] @ w["W_q"].astype(np.float64)
    q = q.reshape(1, 1, H, d_h)
    out = O.decode_reference(L, q, w["B_K"], w["B_V"], pool, table, [n])
    # keys and values straight from the stored (float32) factors and the full per-head weight
    for h in range(H):
        K = rnd(SK) + rnd(RK[:, h]) @ w["B_K"][h].astype(np.float64).T
        V = rnd(SV) + rnd(RV[:, h]) @ w["B_V"][h].astype(np.float64).T
        assert rel_err(out[0, 0, h], sdpa(q[0, 0, h], K, V)) < 1e-12
    # and the factors themselves equal the projection through W_h (eq 2-5)
    Kfull = O.full_projection_kv(X, w["W_SK"], w["U_K"], w["B_K"])
    Kfac = O.reconstruct(SK, np.transpose(RK, (1, 0, 2)), w["B_K"])
    assert rel_err(Kfac, Kfull) < 1e-12


def test_mutant_dropped_private_term_fails(monkeypatch):
    """Planted mistake: reconstruct returns the shared rows only.  The worked example's full
    key (5, -1) and the full-rank pin must both fail."""
    monkeypatch.setattr(O, "reconstruct", _drop_private)
    with pytest.raises(AssertionError):
        test_worked_example_scores()
    with pytest.raises(AssertionError):
        test_full_rank_random_basis_matches_full_projection()


def test_mutant_untransposed_basis_fails(monkeypatch):
    """Planted mistake: R_h B_h instead of R_h B_h^T.  With r < d_h the shapes do not even
    agree; with r = d_h (a square, non-symmetric basis) the full-rank pin must fail."""
    monkeypatch.setattr(O, "reconstruct", _untransposed_basis)
    with pytest.raises((AssertionError, ValueError)):
        test_factored_rows_equal_full_projection()
    with pytest.raises(AssertionError):
        test_full_rank_random_basis_matches_full_projection()


def test_mutant_wrong_slot_index_fails(monkeypatch):
    """Planted mistake: token slot t placed at slot t + 1 (mod P) inside each chunk column.
    The hand-worked byte map must fail (the page walk and the packer share the rule, so
    their round trip alone could not see it)."""
    good = O.in_block_index

    def shifted(L, width, t, k):
        return good(L, width, (np.asarray(t) + 1) % L.page_size, k)

    monkeypatch.setattr(O, "in_block_index", shifted)
    with pytest.raises(AssertionError):
        test_page_layout_byte_map()


# --------------------------------------------------------------------------------------
# rotary position encoding over the factored cache (LRKV notes §8)
# --------------------------------------------------------------------------------------


def test_rope_two_dimensional_counterexample():
    """The page's counterexample: the exact path turns the reconstructed key to the vertical
    axis (score 1 with a vertical query); any low-dimensional turn of the single private
    coordinate keeps the key horizontal (score 0), whatever the turn."""
    g = gold("rope_counterexample.json")
    S = np.array([g["shared_key"]])
    R = np.array([[[g["private_coordinate"]]]])
    Bm = np.array(g["basis_column"], float).reshape(1, 2, 1)
    c, s = g["rotation_cos_sin"]
    K = O.rope_keys(S, R, Bm, np.array([[c]]), np.array([[s]]))[0, 0]
    assert O.reconstruct(S, R, Bm)[0, 0].tolist() == g["reconstructed_key"]
    assert K.tolist() == g["turned_key"]
    q = np.array(g["query_turned"])
    assert q @ K == g["exact_score_unscaled"]
    sc = O.rope_scores_per_position(q, S, R[0], Bm[0], np.array([[c]]), np.array([[s]]))
    assert sc.tolist() == [g["exact_score_unscaled"]]
    for e in (-3.0, -1.0, 0.0, 0.5, 1.0, 7.0):  # E_j z B^T for any scalar turn E_j = e
        low = O.reconstruct(S, R * e, Bm)[0, 0]
        assert q @ low == g["low_dimensional_path_score_unscaled"]


def test_rope_zero_angle_is_plain_decode():
    L, pool, table, lens, q, BK, BV = random_case(81, 4, 16, 4, O.F32, [40, 0, 17])
    cs = np.zeros((64, 8, 2), np.float32)
    cs[..., 0] = 1.0
    a = O.decode_reference_rope(L, q, BK, BV, pool, table, lens, cs)
    b = O.decode_reference(L, q, BK, BV, pool, table, lens)
    assert np.array_equal(a, b)


def _complex_turn(x, cs):
    """x [T, d] turned by complex multiplication: pair (x_2m, x_2m+1) as x_2m + i x_2m+1,
    times cos + i sin (an independent coding of the row-vector turn)."""
    z = torch.view_as_complex(torch.from_numpy(np.ascontiguousarray(x, np.float64)).reshape(
        x.shape[0], -1, 2))
    w = torch.view_as_complex(torch.from_numpy(np.asarray(cs, np.float64)))
    return torch.view_as_real(z * w).reshape(x.shape[0], -1).numpy()


def test_rope_full_rank_identity_basis_is_rotary_mha():
    """r = d_h, S = 0, B = I: every head's keys are its private rows, and the rotary decode
    equals torch's float64 attention over those rows turned by complex multiplication."""
    H, d_h, n = 2, 8, 37
    L = O.Layout(H, d_h, d_h, 16, O.F32)
    g = np.random.default_rng(82)
    RK = g.standard_normal((n, H, d_h)).astype(np.float32)
    RV = g.standard_normal((n, H, d_h)).astype(np.float32)
    z = np.zeros((n, d_h), np.float32)
    table, npg = synth.page_assignment(83, [n], 16, True)
    pool = O.pack_pool(L, table, [n], z.view(np.uint32), z.view(np.uint32),
                       RK.view(np.uint32), RV.view(np.uint32), npg)
    cs = synth.rope_table(48, d_h)
    q = g.standard_normal((1, 1, H, d_h))
    eye = np.stack([np.eye(d_h)] * H)
    out = O.decode_reference_rope(L, q, eye, eye, pool, table, [n], cs)
    for h in range(H):
        K = _complex_turn(RK[:, h].astype(np.float64), cs[:n])
        ref = sdpa(q[0, 0, h], K, RV[:, h].astype(np.float64))
        assert rel_err(out[0, 0, h], ref) < 1e-13


def test_rope_per_position_private_query_agrees():
    """The page's exact path, a private query (q~ D_j^T B_h) per key position, equals the
    turned reconstructed keys (second coding against the first), on random factors."""
    g = np.random.default_rng(84)
    T, d_h, r = 50, 16, 4
    S = g.standard_normal((T, d_h))
    R = g.standard_normal((1, T, r))
    Bm = g.standard_normal((1, d_h, r))
    cs = synth.rope_table(T, d_h)
    q = g.standard_normal(d_h)
    K = O.rope_keys(S, R, Bm, cs[:, :, 0], cs[:, :, 1])[0]
    sc = O.rope_scores_per_position(q, S, R[0], Bm[0], cs[:, :, 0], cs[:, :, 1])
    assert rel_err(sc, K @ q) < 1e-13


def test_rope_mutant_low_dimensional_turn_fails(monkeypatch):
    """Planted mistake: turning only the shared rows and leaving the private term in the
    basis's span (the low-dimensional path the page shows to be wrong) must fail the
    counterexample."""
    def shared_only(S, R, Bm, cos, sin):
        Sr = O.rotate_rows(S, cos, sin)
        return Sr[None] + np.matmul(np.asarray(R, np.float64),
                                    np.transpose(np.asarray(Bm, np.float64), (0, 2, 1)))

    monkeypatch.setattr(O, "rope_keys", shared_only)
    with pytest.raises(AssertionError):
        test_rope_two_dimensional_counterexample()


# --------------------------------------------------------------------------------------
# RMSNorm joint denominator (LRKV notes §8)
# --------------------------------------------------------------------------------------


def test_key_norm_expansion_of_the_page():
    """The page expands the squared norm of k = s + z B^T into its shared, cross and private
    terms: d_h n^2 = |s|^2 + 2 s B z^T + z B^T B z^T + d_h eps.  The oracle's reciprocal
    (which reconstructs k) must equal 1 / n from that expansion, coded here term by term."""
    g = np.random.default_rng(85)
    H, d_h, r, eps = 3, 16, 4, 1e-6
    s_row = g.standard_normal(d_h)
    z = g.standard_normal((H, r))
    Bm = g.standard_normal((H, d_h, r))
    got = O.key_rms_reciprocal(s_row, z, Bm, eps)
    for h in range(H):
        Bh = Bm[h]
        dn2 = (s_row @ s_row + 2 * s_row @ Bh @ z[h] + z[h] @ (Bh.T @ Bh) @ z[h] + d_h * eps)
        assert abs(got[h] - 1 / math.sqrt(dn2 / d_h)) < 1e-14 * got[h]


def test_key_norm_exact_values():
    """Keys of all entries +-2 have n = 2 exactly (eps = 0): reciprocal 0.5 in any dtype; a
    key scaled by 4 has a reciprocal 4 times smaller (the norm is homogeneous)."""
    d_h = 16
    s_row = 2.0 * np.where(np.arange(d_h) % 3 == 0, -1.0, 1.0)
    assert O.key_rms_reciprocal(s_row, np.zeros((1, 4)), np.ones((1, d_h, 4)), 0.0).tolist() == [0.5]
    g = np.random.default_rng(86)
    s2, z2, B2 = g.standard_normal(d_h), g.standard_normal((2, 4)), g.standard_normal((2, d_h, 4))
    a = O.key_rms_reciprocal(s2, z2, B2, 0.0)
    b = O.key_rms_reciprocal(4 * s2, 4 * z2, B2, 0.0)
    assert np.allclose(b, a / 4, rtol=1e-15, atol=0)


def test_key_norm_page_bytes_add_one_over_two_dh():
    """One stored reciprocal per head and position costs 1/(2 d_h) of the dense K/V cache on
    top of eq 9's 1/H + r/d_h (LRKV notes §8); the page is then padded to a whole KiB, by
    less than 1 KiB (65,536 + 512 -> 66,560 bytes at H=16, d_h=128, r=56, bf16)."""
    for H, d_h, r, dt in ((16, 128, 56, O.BF16), (32, 128, 32, O.BF16), (4, 16, 4, O.F32)):
        L = O.Layout(H, d_h, r, 16, dt, key_norm=True)
        dense = 16 * 2 * H * d_h * L.elem_bytes
        assert Fraction(O.page_data_bytes(L), dense) == O.cache_ratio(H, r, d_h) + Fraction(1, 2 * d_h)
        assert O.page_bytes(L) % 1024 == 0
        assert 0 <= O.page_bytes(L) - O.page_data_bytes(L) < 1024
    assert O.page_bytes(O.Layout(16, 128, 56, 16, O.BF16, key_norm=True)) == 66560
    # layouts without the section are not padded
    assert O.page_bytes(O.Layout(16, 128, 56, 16, O.BF16)) == O.page_data_bytes(
        O.Layout(16, 128, 56, 16, O.BF16)) == 65536


def _norm_case(seed, H, d_h, r, dtype, lens, eps, permute=True):
    """Random cached rows; the reciprocals written by the oracle's own key-norm step."""
    L = O.Layout(H, d_h, r, 16, dtype, key_norm=True)
    _, pool, table, lens, q, BK, BV = random_case(seed, H, d_h, r, dtype, lens, permute=permute)
    # repack into the key-norm layout (same rows), then fill N by the key-norm step
    L0 = O.Layout(H, d_h, r, 16, dtype)
    n = int(sum(lens))
    SK, SV, RK, RV = [], [], [], []
    for b, T in enumerate(lens):
        rows = O.gather_request(pool, L0, table[b], T)
        SK.append(rows["SK"]); SV.append(rows["SV"])
        RK.append(np.transpose(rows["RK"], (1, 0, 2))); RV.append(np.transpose(rows["RV"], (1, 0, 2)))
    enc = lambda a: O.encode_elems(np.concatenate(a), dtype).view(O.storage_dtype(L))
    npg = int(table.max()) + 1
    pool_n = O.pack_pool(L, table, lens, enc(SK).reshape(n, d_h), enc(SV).reshape(n, d_h),
                         enc(RK).reshape(n, H, r), enc(RV).reshape(n, H, r), npg)
    req = np.repeat(np.arange(len(lens)), lens)
    pos = np.concatenate([np.arange(t) for t in lens])
    pool_n = O.key_norms_reference(pool_n, L, BK, eps, req, pos, table)
    return L, pool_n, table, lens, q, BK, BV


def test_key_norm_decode_is_attention_over_normalised_keys():
    """r = d_h, S = 0, B = I: the normalised keys are the private rows divided by their RMS;
    the decode equals torch's float64 attention over those, and Algorithm 2 with the stored
    reciprocal multiplied into the summed score agrees."""
    H, d_h, n, eps = 2, 8, 21, 1e-5
    L = O.Layout(H, d_h, d_h, 16, O.F32, key_norm=True)
    g = np.random.default_rng(87)
    RK = g.standard_normal((n, H, d_h)).astype(np.float32)
    RV = g.standard_normal((n, H, d_h)).astype(np.float32)
    z = np.zeros((n, d_h), np.float32)
    table, npg = synth.page_assignment(88, [n], 16, True)
    pool = O.pack_pool(L, table, [n], z.view(np.uint32), z.view(np.uint32),
                       RK.view(np.uint32), RV.view(np.uint32), npg)
    eye = np.stack([np.eye(d_h)] * H)
    pool = O.key_norms_reference(pool, L, eye, eps, np.zeros(n, int), np.arange(n), table)
    q = g.standard_normal((1, 1, H, d_h))
    out = O.decode_reference(L, q, eye, eye, pool, table, [n])
    for h in range(H):
        k = RK[:, h].astype(np.float64)
        inv = np.float32(1.0) / np.sqrt(np.mean(k * k, axis=1) + eps)  # in the cache dtype
        inv = inv.astype(np.float32).astype(np.float64)
        ref = sdpa(q[0, 0, h], k * inv[:, None], RV[:, h].astype(np.float64))
        assert rel_err(out[0, 0, h], ref) < 1e-6  # the stored reciprocal is float32-rounded
    out2 = O.decode_algorithm2(L, q, eye, eye, pool, table, [n])
    assert rel_err(out2, out) < 1e-13


def test_key_norm_makes_scores_scale_free():
    """With eps = 0 the normalised key does not depend on the key's length: scaling every
    cached row of one token by 4 (exact in bf16) leaves the decode output unchanged."""
    L, pool, table, lens, q, BK, BV = _norm_case(89, 3, 16, 8, O.BF16, [37], 0.0, permute=False)
    base = O.decode_reference(L, q, BK, BV, pool, table, lens)
    rows = O.gather_request(pool, L, table[0], 37)
    j = 11
    scaled = O.write_rows(pool, L, table, [0], [j], 4 * rows["SK"][j:j + 1], rows["SV"][j:j + 1],
                          4 * np.transpose(rows["RK"][:, j:j + 1], (1, 0, 2)),
                          np.transpose(rows["RV"][:, j:j + 1], (1, 0, 2)))
    scaled = O.key_norms_reference(scaled, L, BK, 0.0, [0], [j], table)
    assert not np.array_equal(scaled, pool)
    after = O.decode_reference(L, q, BK, BV, scaled, table, lens)
    assert rel_err(after, base) < 1e-14


def test_key_norm_step_writes_only_the_norm_section():
    L, pool, table, lens, q, BK, BV = _norm_case(90, 2, 16, 8, O.BF16, [20, 35], 1e-6)
    sentinel = pool.copy()
    pe = O.page_elems(L)
    el = sentinel.view(np.uint16).reshape(-1, pe)
    base = O.section_base(L, "N", 0)
    el[:, base:base + L.num_heads * 16] = 0xBEEF  # wipe the norm section
    redo = O.key_norms_reference(sentinel, L, BK, 1e-6, np.repeat([0, 1], lens),
                                 np.concatenate([np.arange(t) for t in lens]), table)
    # every appended (page, slot) restored; slots past a request's end keep the sentinel
    expect = pool.copy()
    ex = expect.view(np.uint16).reshape(-1, pe)
    for b, T in enumerate(lens):
        for j in range(T, -(-T // 16) * 16):
            for h in range(L.num_heads):
                ex[table[b, j // 16], O.section_base(L, "N", h) + j % 16] = 0xBEEF
    assert np.array_equal(redo, expect)


def test_key_norm_mutant_without_cross_term_fails(monkeypatch):
    """Planted mistake: the squared norm taken as |s|^2 + |z B^T|^2 (branches normalised as if
    orthogonal, the cross term 2 s B z^T dropped) must fail the page's expansion."""
    def no_cross(s_row, z_rows, Bm, eps):
        s_row = np.asarray(s_row, np.float64)
        P_ = np.einsum("hr,hdr->hd", np.asarray(z_rows, np.float64), np.asarray(Bm, np.float64))
        d_h = s_row.shape[0]
        return 1.0 / np.sqrt((s_row @ s_row + np.sum(P_ * P_, axis=1)) / d_h + eps)

    monkeypatch.setattr(O, "key_rms_reciprocal", no_cross)
    with pytest.raises(AssertionError):
        test_key_norm_expansion_of_the_page()


def test_rope_with_key_norm():
    """Rotary keys over a key-norm layout: with zero angles the rotary decode equals the plain
    key-norm decode; with a real table, the reciprocal stored from the unturned key is the
    turned key's too (a turn keeps the length), checked against attention over the turned
    keys divided by their own RMS."""
    L, pool, table, lens, q, BK, BV = _norm_case(91, 2, 16, 8, O.F32, [37, 5], 0.0)
    cs0 = np.zeros((40, 8, 2), np.float32)
    cs0[..., 0] = 1.0
    a = O.decode_reference_rope(L, q, BK, BV, pool, table, lens, cs0)
    assert rel_err(a, O.decode_reference(L, q, BK, BV, pool, table, lens)) < 1e-14
    cs = synth.rope_table(40, 16)
    got = O.decode_reference_rope(L, q, BK, BV, pool, table, lens, cs)
    rows = O.gather_request(pool, L, table[0], 37)
    for h in range(2):
        K = O.rope_keys(rows["SK"], rows["RK"][h:h + 1], BK[h:h + 1], cs[:37, :, 0],
                        cs[:37, :, 1])[0]
        K = K / np.sqrt(np.mean(K * K, axis=1))[:, None]
        V = O.reconstruct(rows["SV"], rows["RV"][h:h + 1], BV[h:h + 1])[0]
        ref = sdpa(q[0, 0, h], K, V)
        assert rel_err(got[0, 0, h], ref) < 1e-6  # table rows are float32-rounded turns


# --------------------------------------------------------------------------------------
# one shared block per group of heads (LRKV notes §3, after the gradient formulas)
# --------------------------------------------------------------------------------------


def _grouped_case(seed, H, d_h, r, G, dtype, lens, permute=True):
    g = np.random.default_rng(seed)
    L = O.Layout(H, d_h, r, 16, dtype, groups=G)
    n = int(sum(lens))
    code = (lambda x: synth.to_bf16_bits(x.astype(np.float32))) if dtype == O.BF16 else \
        (lambda x: x.astype(np.float32).view(np.uint32))
    SK, SV = code(g.standard_normal((n, G, d_h))), code(g.standard_normal((n, G, d_h)))
    RK, RV = code(g.standard_normal((n, H, r))), code(g.standard_normal((n, H, r)))
    table, npg = synth.page_assignment(seed + 1, lens, 16, permute)
    pool = O.pack_pool(L, table, lens, SK, SV, RK, RV, npg)
    q = g.standard_normal((len(lens), 1, H, d_h))
    BK = g.standard_normal((H, d_h, r)) / math.sqrt(r)
    BV = g.standard_normal((H, d_h, r)) / math.sqrt(r)
    return L, pool, table, lens, q, BK, BV, (SK, SV, RK, RV)


def test_grouped_cache_size_is_the_replicated_shared_formula():
    """G shared blocks store the shared features G times: page bytes over the dense page is
    G/H + r/d_h, the page's own formula for shared rows held in P copies (LRKV notes §4,
    tensor-parallel replication, with P = G), and eq 9's bytes with G d_h in place of d_h."""
    for H, d_h, r, G in ((32, 128, 32, 2), (16, 128, 56, 4), (32, 128, 32, 32), (4, 16, 4, 2)):
        L = O.Layout(H, d_h, r, 16, O.BF16, groups=G)
        dense = 16 * 2 * H * d_h * 2
        assert Fraction(O.page_bytes(L), dense) == O.tp_replicated_ratio(G, H, r, d_h)
        assert O.grouped_cache_bytes(2, 1, 16, d_h, H, r, G) == O.page_bytes(L)
    assert O.grouped_cache_bytes(2, 1, 16, 128, 16, 56, 1) == O.lrkv_cache_bytes(2, 1, 16, 128,
                                                                                  16, 56)


def test_one_group_is_the_plain_layout():
    L, pool, table, lens, q, BK, BV, rows = _grouped_case(92, 4, 16, 4, 1, O.F32, [37, 5])
    L1 = O.Layout(4, 16, 4, 16, O.F32)
    SK, SV, RK, RV = rows
    plain = O.pack_pool(L1, table, lens, SK[:, 0], SV[:, 0], RK, RV, int(table.max()) + 1)
    assert np.array_equal(pool, plain)


def test_grouped_decode_is_each_groups_own_lrkv():
    """A grouped cache decodes, head by head, exactly as G independent one-group caches, one
    per group holding that group's shared rows and its heads' private rows (packed and
    decoded on their own)."""
    H, d_h, r, G = 4, 16, 4, 2
    L, pool, table, lens, q, BK, BV, rows = _grouped_case(93, H, d_h, r, G, O.F32, [37, 5, 16])
    got = O.decode_reference(L, q, BK, BV, pool, table, lens)
    got2 = O.decode_algorithm2(L, q, BK, BV, pool, table, lens)
    assert rel_err(got2, got) < 1e-13
    SK, SV, RK, RV = rows
    Hg = H // G
    Lg = O.Layout(Hg, d_h, r, 16, O.F32)
    for g in range(G):
        hs = slice(g * Hg, (g + 1) * Hg)
        sub = O.pack_pool(Lg, table, lens, SK[:, g], SV[:, g], RK[:, hs], RV[:, hs],
                          int(table.max()) + 1)
        ref = O.decode_reference(Lg, q[:, :, hs], BK[hs], BV[hs], sub, table, lens)
        assert np.array_equal(got[:, :, hs], ref)


def test_one_group_per_head_rank_zero_is_mha():
    """G = H and r = 0: every head has its own shared block, i.e. plain multi-head attention
    over it (torch float64 attention)."""
    H, d_h, n = 3, 8, 19
    g = np.random.default_rng(94)
    L = O.Layout(H, d_h, 0, 16, O.F32, groups=H)
    SK = g.standard_normal((n, H, d_h)).astype(np.float32)
    SV = g.standard_normal((n, H, d_h)).astype(np.float32)
    z = np.zeros((n, H, 0), np.float32)
    table, npg = synth.page_assignment(95, [n], 16, True)
    pool = O.pack_pool(L, table, [n], SK.view(np.uint32), SV.view(np.uint32), z.view(np.uint32),
                       z.view(np.uint32), npg)
    q = g.standard_normal((1, 1, H, d_h))
    none = np.zeros((H, d_h, 0))
    out = O.decode_reference(L, q, none, none, pool, table, [n])
    for h in range(H):
        assert rel_err(out[0, 0, h], sdpa(q[0, 0, h], SK[:, h].astype(np.float64),
                                          SV[:, h].astype(np.float64))) < 1e-13


def test_grouped_mutant_wrong_group_fails(monkeypatch):
    """Planted mistake: heads assigned to groups round robin (h mod G) instead of in
    contiguous runs must fail the per-group decomposition."""
    monkeypatch.setattr(O.Layout, "group_of", lambda self, h: h % self.groups)
    with pytest.raises(AssertionError):
        test_grouped_decode_is_each_groups_own_lrkv()


def test_grouped_append_places_each_groups_projection():
    """Algorithm 1 with one shared projection per group: S_K[g] = X W_SK[g], placed in group
    g's block; exact-integer inputs, compared with the per-group one-group append."""
    H, d_h, r, G, d = 4, 16, 8, 2, 64
    g = np.random.default_rng(96)
    L = O.Layout(H, d_h, r, 16, O.BF16, groups=G)
    X = g.integers(-1, 2, (5, d)).astype(np.float64)
    WK, WV = g.integers(-1, 2, (G, d, d_h)), g.integers(-1, 2, (G, d, d_h))
    UK, UV = g.integers(-1, 2, (d, H, r)), g.integers(-1, 2, (d, H, r))
    table, npg = synth.page_assignment(97, [20, 9], 16, True)
    req, pos = np.array([0, 1, 0, 1, 0]), np.array([19, 0, 16, 8, 3])
    start = np.zeros(npg * O.page_elems(L), np.uint16).view(np.uint8)
    got = O.append_reference(start, L, X, WK, WV, UK, UV, req, pos, table)
    Lg = O.Layout(H // G, d_h, r, 16, O.BF16)
    blk = O.page_elems(Lg)
    el = got.view(np.uint16).reshape(npg, -1)
    for gg in range(G):
        hs = slice(gg * 2, gg * 2 + 2)
        sub = O.append_reference(np.zeros(npg * blk, np.uint16).view(np.uint8), Lg, X, WK[gg],
                                 WV[gg], UK[:, hs], UV[:, hs], req, pos, table)
        assert np.array_equal(el[:, gg * blk:(gg + 1) * blk], sub.view(np.uint16).reshape(npg, blk))
