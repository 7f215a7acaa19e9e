"""GPU parity of the key-norm path (LRKV notes §8, RMSNorm paragraph), through the C ABI:
lrkv_key_norms against the oracle's key-norm step (bit-exact on exact-arithmetic keys,
within one bf16 ulp on Gaussian rows, no other byte touched), and lrkv_decode /
lrkv_decode_rope over key-norm layouts against the oracle (1e-2 of max|ref|)."""

import math

import numpy as np
import pytest
import torch

import factored_rank_kv_amd as F
import oracle as O
import synth
from lrkv_case import (as_codes, codes_f64, iid_case, layout_c, log, max_rel_err, output_major,
                       tolerance, to_dev)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def gpu_norms(L, pool, table, BK_codes, eps, req, pos):
    """lrkv_key_norms on a device copy of `pool`; returns the resulting pool bytes."""
    d_pool = torch.from_numpy(pool.copy()).to(DEV)
    F.lrkv_key_norms(layout_c(L), to_dev(BK_codes), eps, to_dev(np.asarray(req, np.int32)),
                     to_dev(np.asarray(pos, np.int32)), len(req), to_dev(table), table.shape[1],
                     d_pool, len(pool) // O.page_bytes(L))
    torch.cuda.synchronize()
    return d_pool.cpu().numpy()


def norm_codes(L, pool, table, lens):
    """The N-section codes of every cached (request, position, head), [sum(lens), H]."""
    pe = O.page_elems(L)
    el = pool.view(np.uint16).reshape(-1, pe)
    out = []
    for b, T in enumerate(lens):
        for j in range(T):
            pg = table[b, j // 16]
            out.append([el[pg, O.section_base(L, "N", h) + j % 16] for h in range(L.num_heads)])
    return np.array(out, np.uint16)


@pytest.mark.parametrize("shape", [(16, 128, 56), (32, 128, 32)])
def test_key_norms_bit_exact_on_exact_keys(shape):
    """Keys whose entries all have one power-of-two magnitude have an exact RMS: rows with
    S_K entries +-a and R_K = 0, and rows with S_K = 0 and z B^T = +-c (B_K entries +-1/4
    times a one-hot z of 4 c).  eps = 0.  Every byte must equal the oracle's pool."""
    H, dh, r = shape
    L = O.Layout(H, dh, r, 16, O.BF16, key_norm=True)
    g = np.random.default_rng(501 + H)
    lens = [37, 20]
    n = sum(lens)
    signs = lambda s: np.where(g.random(s) < 0.5, -1.0, 1.0)
    SK = np.zeros((n, dh))
    RK = np.zeros((n, H, r))
    for i in range(n):
        if i % 2 == 0:
            SK[i] = signs(dh) * 2.0 ** int(g.integers(-3, 4))
        else:
            RK[i, :, int(g.integers(0, r))] = 4.0 * 2.0 ** int(g.integers(-2, 3))
    BK = signs((H, dh, r)) / 4
    SV = g.standard_normal((n, dh))
    RV = g.standard_normal((n, H, r))
    enc = lambda a: O.f64_to_bf16_bits(a)
    table, npg = synth.page_assignment(502, lens, 16, True)
    pool = O.pack_pool(L, table, lens, enc(SK), enc(SV), enc(RK), enc(RV), npg, fill=0xBEEF,
                       NR=np.full((n, H), 0xBEEF, np.uint16))
    req = np.repeat(np.arange(2), lens)
    pos = np.concatenate([np.arange(t) for t in lens])
    order = g.permutation(n)
    want = O.key_norms_reference(pool, L, BK, 0.0, req, pos, table)  # BK exact in bf16
    got = gpu_norms(L, pool, table, enc(BK), 0.0, req[order], pos[order])
    log(f"key norms {shape}: {np.count_nonzero(got != want)} differing bytes")
    assert np.array_equal(got, want)
    vals = O.bf16_bits_to_f64(norm_codes(L, got, table, lens))
    assert set(np.unique(vals)) <= {2.0 ** k for k in range(-6, 6)}


@pytest.mark.parametrize("shape", [(16, 128, 56), (32, 128, 32)])
@pytest.mark.parametrize("n_rows", [8, 100])
def test_key_norms_gaussian_within_one_ulp(shape, n_rows):
    """Gaussian rows (eps 1e-6): each stored reciprocal within one bf16 ulp of the oracle's
    (float32 accumulation of the squares against float64); other bytes untouched."""
    H, dh, r = shape
    lens = [n_rows, 3]
    case = iid_case(503 + n_rows, H, dh, r, O.BF16, lens, permute=True, fill=0x7FC0,
                    key_norm_eps=1e-6)
    L = case.L
    want = case.pool
    # wipe the N section of the appended rows, then recompute it on the GPU
    wiped = want.copy()
    el = wiped.view(np.uint16).reshape(-1, O.page_elems(L))
    base = O.section_base(L, "N", 0)
    el[:, base:base + H * 16] = 0x1234
    req = np.repeat(np.arange(2), lens)
    pos = np.concatenate([np.arange(t) for t in lens])
    got = gpu_norms(L, wiped, case.table, case.BK_codes, 1e-6, req, pos)
    a = norm_codes(L, got, case.table, lens).astype(np.int32)
    b = norm_codes(L, want, case.table, lens).astype(np.int32)
    diff = np.abs(a - b)  # same-sign bf16 codes: code distance = ulps
    log(f"key norms {shape} n={n_rows}: {np.count_nonzero(diff)} of {diff.size} off by "
        f"{diff.max()} ulp")
    assert diff.max() <= 1
    # every byte outside the N section equals the input pool's
    keep = np.ones(O.page_elems(L), bool)
    keep[base:base + H * 16] = False
    assert np.array_equal(got.view(np.uint16).reshape(-1, O.page_elems(L))[:, keep],
                          want.view(np.uint16).reshape(-1, O.page_elems(L))[:, keep])


@pytest.mark.parametrize("shape", [(16, 128, 56), (32, 128, 32)])
def test_decode_over_key_norm_layout(shape):
    """Chunked, 16-token chunks and (20+ requests) balanced splits, and the rotary decode."""
    H, dh, r = shape
    lens = [1, 17, 100, 16, 33, 250, 0]
    case = iid_case(510 + H, H, dh, r, O.BF16, lens, permute=True, fill=0x7FC0,
                    key_norm_eps=1e-6)
    ref = case.reference()
    live = np.array(lens) > 0
    for chunk in (0, 16):
        got = case.run_f64(chunk_tokens=chunk)
        assert np.all(got[~live] == 0)
        err = max_rel_err(got[live], ref[live])
        log(f"key-norm decode {shape} chunk {chunk}: max rel err {err:.3e}")
        assert err <= tolerance(O.BF16)
    cs = synth.rope_table(256, dh)
    got = case.run_rope(cs)
    err = max_rel_err(got[live], case.reference_rope(cs)[live])
    log(f"key-norm rotary decode {shape}: max rel err {err:.3e}")
    assert err <= tolerance(O.BF16)
    big = [48] * 10 + [300, 0, 5, 17, 1000, 64, 33, 2, 129, 700]
    bal = iid_case(520 + H, H, dh, r, O.BF16, big, permute=True, fill=0x7FC0, key_norm_eps=1e-6)
    got = bal.run_f64()
    lv = np.array(big) > 0
    err = max_rel_err(got[lv], bal.reference()[lv])
    log(f"key-norm balanced decode {shape}: max rel err {err:.3e}")
    assert err <= tolerance(O.BF16)


def test_key_norm_multi_query_rows():
    """q_len = 70 (prefill-sized) over a key-norm layout runs the split kernels."""
    case = iid_case(530, 16, 128, 56, O.BF16, [150, 70], q_len=70, permute=True, fill=0x7FC0,
                    key_norm_eps=1e-5)
    err = max_rel_err(case.run_f64(), case.reference())
    log(f"key-norm multi-query (q_len 70): max rel err {err:.3e}")
    assert err <= tolerance(O.BF16)


def test_end_to_end_append_norms_decode():
    """X -> lrkv_append -> lrkv_key_norms -> lrkv_decode on the GPU, against the oracle's
    append, key-norm step and decode from the same inputs (B=3, H=16, d=2048)."""
    H, dh, r, d = 16, 128, 56, 2048
    L = O.Layout(H, dh, r, 16, O.BF16, key_norm=True)
    lens = [70, 16, 33]
    n = sum(lens)
    w = synth.projection_weights(540, d, H, dh, r)
    wc = {k: as_codes(v, O.BF16) for k, v in w.items()}
    w64 = {k: codes_f64(v, O.BF16) for k, v in wc.items()}
    X = as_codes(synth.activations(541, n, d), O.BF16)
    table, npg = synth.page_assignment(542, lens, 16, True)
    req = np.repeat(np.arange(3), lens).astype(np.int32)
    pos = np.concatenate([np.arange(t) for t in lens]).astype(np.int32)
    start = np.zeros(npg * O.page_bytes(L), np.uint8)
    ref_pool = O.append_reference(start, L, codes_f64(X, O.BF16), w64["W_SK"], w64["W_SV"],
                                  w64["U_K"], w64["U_V"], req, pos, table)
    ref_pool = O.key_norms_reference(ref_pool, L, w64["B_K"], 1e-6, req, pos, table)
    d_pool = torch.zeros(len(start), dtype=torch.uint8, device=DEV)
    lay = layout_c(L)
    om = {k: to_dev(output_major(wc[k])) for k in ("W_SK", "W_SV", "U_K", "U_V")}
    F.lrkv_append(lay, to_dev(X), n, d, om["W_SK"], om["W_SV"], om["U_K"], om["U_V"],
                  to_dev(req), to_dev(pos), to_dev(table), table.shape[1], d_pool, npg)
    F.lrkv_key_norms(lay, to_dev(wc["B_K"]), 1e-6, to_dev(req), to_dev(pos), n, to_dev(table),
                     table.shape[1], d_pool, npg)
    q = as_codes(synth.queries(543, 3, 1, H, dh), O.BF16)
    lens_d = to_dev(np.array(lens, np.int32))
    ws_n = F.lrkv_decode_workspace_bytes(lay, 3, 1, max(lens), 0)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=DEV)
    out = torch.empty((3, 1, H, dh), dtype=torch.int16, device=DEV)
    F.lrkv_decode(lay, to_dev(q), 3, 1, to_dev(wc["B_K"]), to_dev(wc["B_V"]), d_pool,
                  to_dev(table), table.shape[1], lens_d, max(lens), 0, out, ws, ws_n)
    torch.cuda.synchronize()
    got_pool = d_pool.cpu().numpy()
    # placement of every byte as the oracle's; values within the accumulation bound (the
    # Gaussian append is checked elsewhere), so compare decode outputs over the GPU pool too
    ref = O.decode_reference(L, codes_f64(q, O.BF16), w64["B_K"], w64["B_V"], ref_pool, table,
                             lens)
    got = O.bf16_bits_to_f64(out.cpu().numpy().view(np.uint16))
    err = max_rel_err(got, ref)
    log(f"end to end with key norms: max rel err {err:.3e}; pool bytes differing from the "
        f"oracle's: {np.count_nonzero(got_pool != ref_pool)} of {len(ref_pool)}")
    assert err <= tolerance(O.BF16)
