"""GPU parity of grouped layouts (one shared block per group of heads, LRKV notes §3): 32
heads of rank 32 in 2 groups of 16.  lrkv_append against the oracle's grouped Algorithm-1
append (bit-exact on exact-arithmetic inputs, every other byte untouched), lrkv_decode
against the oracle's grouped decode (1e-2 of max|ref|)."""

import math

import numpy as np
import pytest
import torch

import factored_rank_kv_amd as F
import oracle as O
import synth
from lrkv_case import Case, as_codes, layout_c, log, max_rel_err, output_major, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
H, DH, R, G = 32, 128, 32, 2


def grouped_case(seed, lens, q_len=1, permute=True, fill=0x7FC0):
    L = O.Layout(H, DH, R, 16, O.BF16, groups=G)
    g = np.random.default_rng(seed)
    n = int(sum(lens))
    code = lambda s: synth.to_bf16_bits(g.standard_normal(s, dtype=np.float32))
    SK, SV, RK, RV = code((n, G, DH)), code((n, G, DH)), code((n, H, R)), code((n, H, R))
    table, npg = synth.page_assignment(seed + 1, lens, 16, permute)
    pool = O.pack_pool(L, table, lens, SK, SV, RK, RV, npg, fill=fill)
    q = as_codes(synth.queries(seed + 2, len(lens), q_len, H, DH), O.BF16)
    bk = as_codes((g.standard_normal((H, DH, R)) / math.sqrt(R)).astype(np.float32), O.BF16)
    bv = as_codes((g.standard_normal((H, DH, R)) / math.sqrt(R)).astype(np.float32), O.BF16)
    return Case(L, pool, table, lens, q, bk, bv, npg)


@pytest.mark.parametrize("chunk", [0, 16, 64])
def test_grouped_decode_ragged(chunk):
    lens = [1, 17, 100, 16, 33, 250, 0]
    case = grouped_case(801, lens)
    got = case.run_f64(chunk_tokens=chunk)
    ref = case.reference()
    live = np.array(lens) > 0
    assert np.all(got[~live] == 0)
    err = max_rel_err(got[live], ref[live])
    log(f"grouped decode chunk {chunk}: max rel err {err:.3e}")
    assert err <= 1e-2


def test_grouped_decode_balanced_and_multi_query():
    lens = [48] * 10 + [300, 0, 5, 17, 1000, 64, 33, 2, 129, 700]
    case = grouped_case(802, lens)
    got = case.run_f64()
    live = np.array(lens) > 0
    err = max_rel_err(got[live], case.reference()[live])
    log(f"grouped balanced decode (20 requests): max rel err {err:.3e}")
    assert err <= 1e-2
    mq = grouped_case(803, [150, 70], q_len=70)
    err = max_rel_err(mq.run_f64(), mq.reference())
    log(f"grouped multi-query (q_len 70): max rel err {err:.3e}")
    assert err <= 1e-2


def test_grouped_decode_larger_all_outputs():
    lens = [8192, 3000, 12000, 1]
    case = grouped_case(804, lens)
    err = max_rel_err(case.run_f64(), case.reference())
    log(f"grouped decode, lengths {lens}: all outputs, max rel err {err:.3e}")
    assert err <= 1e-2


@pytest.mark.parametrize("n_rows", [5, 100])
def test_grouped_append_bit_exact(n_rows):
    """X and weights in {-1, 0, 1}, d = 256: exact integers.  The few-rows (5) and product
    (100 rows) paths, each group's shared projection into its block; sentinel elsewhere."""
    L = O.Layout(H, DH, R, 16, O.BF16, groups=G)
    d = 256
    g = np.random.default_rng(805 + n_rows)
    X = g.integers(-1, 2, (n_rows, d)).astype(np.float64)
    WK, WV = g.integers(-1, 2, (G, d, DH)), g.integers(-1, 2, (G, d, DH))
    UK, UV = g.integers(-1, 2, (d, H, R)), g.integers(-1, 2, (d, H, R))
    lens = [n_rows // 2 + 1, n_rows - n_rows // 2 - 1 + 3]
    table, npg = synth.page_assignment(806, lens, 16, True)
    req = np.concatenate([np.zeros(lens[0], int), np.ones(n_rows - lens[0], int)])
    pos = np.concatenate([np.arange(lens[0]), np.arange(n_rows - lens[0]) + 3])
    order = g.permutation(n_rows)
    req, pos = req[order], pos[order]
    start = np.full(npg * O.page_elems(L), 0xBEEF, np.uint16).view(np.uint8)
    want = O.append_reference(start, L, X, WK, WV, UK, UV, req, pos, table)
    f32 = lambda a: as_codes(np.asarray(a, np.float32), O.BF16)
    # shared weights per group, output-major [G][d_h][d]; private [H][r][d]
    wsk = to_dev(np.ascontiguousarray(np.transpose(f32(WK), (0, 2, 1))))
    wsv = to_dev(np.ascontiguousarray(np.transpose(f32(WV), (0, 2, 1))))
    pool = torch.from_numpy(start.copy()).to(DEV)
    F.lrkv_append(layout_c(L), to_dev(f32(X)), n_rows, d, wsk, wsv, to_dev(output_major(f32(UK))),
                  to_dev(output_major(f32(UV))), to_dev(req.astype(np.int32)),
                  to_dev(pos.astype(np.int32)), to_dev(table), table.shape[1], pool, npg)
    torch.cuda.synchronize()
    got = pool.cpu().numpy()
    log(f"grouped append {n_rows} rows: {np.count_nonzero(got != want)} differing bytes")
    assert np.array_equal(got, want)
