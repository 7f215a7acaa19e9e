"""GPU parity of the decode with the private queries formed once per query row:
lrkv_private_queries (or lrkv_append_pq, the step's new rows and p in one launch) forms
p = q B_K (LRKV notes §2: the query carried into each head's rank-r space), and
lrkv_decode_pq runs the split decode on them in place of forming them in every split
workgroup.  The split and merge kernels are those of lrkv_decode, fed the same p, so the
outputs must equal lrkv_decode's bit for bit; each case is also held to the oracle's decode
at the cache type's tolerance."""

import numpy as np
import pytest
import torch

import factored_rank_kv_amd as F
import oracle as O
import synth
from lrkv_case import (as_codes, fresh_workspace, from_dev, iid_case, layout_c, log,
                       max_rel_err, output_major, to_dev, tolerance)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def grouped_case(seed, lens, q_len=1):
    from test_grouped_gpu import grouped_case as make
    return make(seed, lens, q_len=q_len)


def run_pq(case, chunk_tokens=0, p_fill=0xFF):
    d = case.dev
    lay = layout_c(case.L)
    msl = int(case.lens.max())
    pb = F.lrkv_private_queries_bytes(lay, case.B, case.q_len)
    assert pb > 0
    p = fresh_workspace(pb, p_fill)
    F.lrkv_private_queries(lay, d["q"], case.B, case.q_len, d["BK"], p, pb)
    nb = F.lrkv_decode_workspace_bytes(lay, case.B, case.q_len, msl, chunk_tokens)
    ws = fresh_workspace(nb, 0xFF)
    out = torch.empty(case.q_codes.shape, dtype=d["q"].dtype, device=DEV)
    F.lrkv_decode_pq(lay, d["q"], p, pb, case.B, case.q_len, d["BV"], d["pool"], d["table"],
                     case.table.shape[1], d["lens"], msl, chunk_tokens, out, ws, nb)
    torch.cuda.synchronize()
    return out


CASES = {
    "C1 ragged": (dict(H=16, dh=128, r=56, dtype=O.BF16, lens=[300, 17, 1, 129, 0]), (0, 64)),
    "C1 balanced, 20 requests": (dict(H=16, dh=128, r=56, dtype=O.BF16, lens=[200, 33] * 10),
                                 (0,)),
    "C1 five query rows": (dict(H=16, dh=128, r=56, dtype=O.BF16, lens=[90, 12], q_len=5),
                           (0, 32)),
    "C3 ragged": (dict(H=32, dh=128, r=32, dtype=O.BF16, lens=[500, 3, 64, 0, 16]), (0, 128)),
    "C3 balanced, 24 requests": (dict(H=32, dh=128, r=32, dtype=O.BF16,
                                      lens=[48, 1, 130] * 8), (0,)),
    "C0 float32, three query rows": (dict(H=4, dh=16, r=4, dtype=O.F32, lens=[40, 7, 0],
                                          q_len=3), (0, 16)),
    "C1 key norm": (dict(H=16, dh=128, r=56, dtype=O.BF16, lens=[300, 17, 1, 0],
                         key_norm_eps=1e-6), (0, 64)),
    "C1 key norm, balanced": (dict(H=16, dh=128, r=56, dtype=O.BF16, lens=[70, 5] * 9,
                                   key_norm_eps=1e-6), (0,)),
    "C3 key norm, 70 query rows": (dict(H=32, dh=128, r=32, dtype=O.BF16, lens=[150, 90],
                                        q_len=70, key_norm_eps=1e-6), (0,)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_decode_pq_matches_decode(name):
    kw, chunks = dict(CASES[name][0]), CASES[name][1]
    lens = kw.pop("lens")
    case = iid_case(900 + list(CASES).index(name), kw.pop("H"), kw.pop("dh"), kw.pop("r"),
                    kw.pop("dtype"), lens, permute=True, fill=0x7FC0, **kw)
    ref = case.reference()
    live = np.repeat(np.array(lens) > 0, case.q_len * case.L.num_heads * case.L.head_dim)
    live = live.reshape(ref.shape)
    for chunk in chunks:
        want = case.run(chunk_tokens=chunk)
        got = run_pq(case, chunk)
        assert torch.equal(got, want), f"{name}, chunk {chunk}: differs from lrkv_decode"
        g64 = from_dev(got, case.L.dtype)
        assert np.all(g64[~live] == 0)
        err = max_rel_err(g64[live], ref[live])
        log(f"{name}, chunk {chunk}: bit-identical to lrkv_decode, max rel err {err:.3e}")
        assert err <= tolerance(case.L.dtype)


@pytest.mark.parametrize("lens,q_len,chunks", [
    ([1, 17, 100, 16, 33, 250, 0], 1, (0, 64)),        # chunked
    ([48] * 10 + [300, 0, 5, 17, 1000, 64], 1, (0,)),  # balanced
    ([150, 70], 70, (0,)),                             # 70 query rows through the split
])
def test_decode_pq_grouped(lens, q_len, chunks):
    """Grouped layout (32 heads, r=32, 2 blocks of 16): p formed per group, the output equal
    to lrkv_decode's bit for bit."""
    case = grouped_case(990 + len(lens), lens, q_len)
    for chunk in chunks:
        want = case.run(chunk_tokens=chunk)
        got = run_pq(case, chunk)
        assert torch.equal(got, want), f"grouped, chunk {chunk}: differs from lrkv_decode"
    log(f"grouped decode_pq ({len(lens)} requests, q_len {q_len}): bit-identical to lrkv_decode")


def test_private_queries_written_whole():
    """Every byte of the private-query buffer that lrkv_private_queries_bytes sizes is
    written (two fills give the same buffer), and nothing past it."""
    case = iid_case(950, 16, 128, 56, O.BF16, [20, 5, 9])
    d = case.dev
    lay = layout_c(case.L)
    pb = F.lrkv_private_queries_bytes(lay, case.B, 1)
    bufs = []
    for fill in (0x00, 0xFF):
        p = fresh_workspace(pb + 4096, fill)
        F.lrkv_private_queries(lay, d["q"], case.B, 1, d["BK"], p, pb)
        torch.cuda.synchronize()
        assert torch.all(p[pb:] == fill), "written past the sized buffer"
        bufs.append(p[:pb].clone())
    assert torch.equal(bufs[0], bufs[1])


def test_decode_pq_reuses_private_queries():
    """p formed once serves any number of decode calls over the same query rows: two calls
    on one buffer (the second over a table whose lengths drop the last pages) each match
    lrkv_decode on the same arguments."""
    lens = [250, 64, 3]
    case = iid_case(951, 16, 128, 56, O.BF16, lens, fill=0x7FC0)
    d = case.dev
    lay = layout_c(case.L)
    pb = F.lrkv_private_queries_bytes(lay, case.B, 1)
    p = fresh_workspace(pb, 0xFF)
    F.lrkv_private_queries(lay, d["q"], case.B, 1, d["BK"], p, pb)
    for shorter in (0, 40):
        lens_now = np.maximum(np.array(lens) - shorter, 0).astype(np.int32)
        lens_dev = torch.from_numpy(lens_now).to(DEV)
        msl = int(case.table.shape[1] * case.L.page_size)
        nb = F.lrkv_decode_workspace_bytes(lay, case.B, 1, msl, 0)
        outs = []
        for use_p in (False, True):
            ws = fresh_workspace(nb, 0xFF)
            out = torch.empty(case.q_codes.shape, dtype=d["q"].dtype, device=DEV)
            if use_p:
                F.lrkv_decode_pq(lay, d["q"], p, pb, case.B, 1, d["BV"], d["pool"], d["table"],
                                 case.table.shape[1], lens_dev, msl, 0, out, ws, nb)
            else:
                F.lrkv_decode(lay, d["q"], case.B, 1, d["BK"], d["BV"], d["pool"], d["table"],
                              case.table.shape[1], lens_dev, msl, 0, out, ws, nb)
            torch.cuda.synchronize()
            outs.append(out)
        assert torch.equal(outs[0], outs[1]), f"lengths shortened by {shorter}"
    log("one private-query buffer, two decode calls: both bit-identical to lrkv_decode")


def append_inputs(seed, L, n_rows, d, lens):
    g = np.random.default_rng(seed)
    H, dh, r = L.num_heads, L.head_dim, L.rank
    X = as_codes(g.standard_normal((n_rows, d)).astype(np.float32), L.dtype)
    w = {"W_SK": (d, dh), "W_SV": (d, dh), "U_K": (d, H, r), "U_V": (d, H, r)}
    wdev = {k: to_dev(output_major(as_codes((g.standard_normal(s) / np.sqrt(d)).astype(np.float32),
                                            L.dtype)))
            for k, s in w.items()}
    table, npg = synth.page_assignment(seed + 1, lens, L.page_size, True)
    slots = [(b, t) for b in range(len(lens)) for t in range(lens[b])]
    pick = g.choice(len(slots), n_rows, replace=False)  # distinct (request, position) slots
    req = np.array([slots[i][0] for i in pick], np.int32)
    pos = np.array([slots[i][1] for i in pick], np.int32)
    return to_dev(X), wdev, table, npg, to_dev(req), to_dev(pos)


@pytest.mark.parametrize("H,dh,r,dtype,n_rows,q_len", [
    (16, 128, 56, O.BF16, 8, 1),   # the decode step: one launch
    (16, 128, 56, O.BF16, 3, 2),   # one launch, fewer rows
    (32, 128, 32, O.BF16, 8, 1),   # one launch
    (16, 128, 56, O.BF16, 13, 1),  # more than 8 rows: the two calls in turn
    (4, 16, 4, O.F32, 6, 3),       # float32: the two calls in turn
    (16, 128, 56, -1, 8, 1),       # key-norm pages (dtype -1: bf16 with the N section)
])
def test_append_pq_matches_the_two_calls(H, dh, r, dtype, n_rows, q_len):
    """lrkv_append_pq leaves the pool lrkv_append leaves, byte for byte, and the private
    queries lrkv_private_queries forms, bit for bit."""
    key_norm = dtype == -1
    dtype = O.BF16 if key_norm else dtype
    L = O.Layout(H, dh, r, 16, dtype, key_norm=key_norm)
    lay = layout_c(L)
    d = 256
    seed = 960 + n_rows + H + key_norm
    lens = [70, 33, 150]
    Xd, wdev, table, npg, reqd, posd = append_inputs(seed, L, n_rows, d, lens)
    tabd = to_dev(np.ascontiguousarray(table, np.int32))
    B = len(lens)
    q = to_dev(as_codes(synth.queries(seed + 5, B, q_len, H, dh), dtype))
    BK = to_dev(as_codes((np.random.default_rng(seed + 6).standard_normal((H, dh, r)) /
                          np.sqrt(r)).astype(np.float32), dtype))
    pb = F.lrkv_private_queries_bytes(lay, B, q_len)
    pools, ps = [], []
    for fused in (False, True):
        pool = torch.full((npg * O.page_bytes(L),), 0x5A, dtype=torch.uint8, device=DEV)
        p = fresh_workspace(pb, 0xFF if fused else 0x00)
        args = (Xd, n_rows, d, wdev["W_SK"], wdev["W_SV"], wdev["U_K"], wdev["U_V"], reqd, posd,
                tabd, table.shape[1], pool, npg)
        if fused:
            F.lrkv_append_pq(lay, *args, q, B, q_len, BK, p, pb)
        else:
            F.lrkv_append(lay, *args)
            F.lrkv_private_queries(lay, q, B, q_len, BK, p, pb)
        torch.cuda.synchronize()
        pools.append(pool)
        ps.append(p)
    assert int((pools[0] != 0x5A).sum()) > 0
    assert torch.equal(pools[0], pools[1]), "pool differs from lrkv_append's"
    assert torch.equal(ps[0], ps[1]), "private queries differ from lrkv_private_queries'"
    log(f"lrkv_append_pq H={H} r={r} {n_rows} rows, {B}x{q_len} query rows: pool and p "
        "identical to the two calls")


def test_append_pq_step_then_decode_pq():
    """A decode step as a serving loop runs it: lrkv_append_pq writes the step's new row of
    each request and forms p, then lrkv_decode_pq attends over the grown cache; the output
    equals lrkv_append followed by lrkv_decode, bit for bit."""
    H, dh, r, d = 16, 128, 56, 512
    L = O.Layout(H, dh, r, 16, O.BF16)
    lay = layout_c(L)
    lens_before = [100, 16, 47, 1, 200, 63, 30, 9]
    B = len(lens_before)
    case = iid_case(970, H, dh, r, O.BF16, [t + 1 for t in lens_before], fill=0x7FC0)
    dv = case.dev
    g = np.random.default_rng(971)
    Xd = to_dev(as_codes(g.standard_normal((B, d)).astype(np.float32), O.BF16))
    wdev = {k: to_dev(output_major(as_codes((g.standard_normal(s) / np.sqrt(d)).astype(np.float32),
                                            O.BF16)))
            for k, s in {"W_SK": (d, dh), "W_SV": (d, dh), "U_K": (d, H, r),
                         "U_V": (d, H, r)}.items()}
    reqd = to_dev(np.arange(B, dtype=np.int32))
    posd = to_dev(np.array(lens_before, np.int32))
    msl = int(case.lens.max())
    nb = F.lrkv_decode_workspace_bytes(lay, B, 1, msl, 0)
    pb = F.lrkv_private_queries_bytes(lay, B, 1)
    outs = []
    for fused in (False, True):
        pool = dv["pool"].clone()
        ws = fresh_workspace(nb, 0xFF)
        out = torch.empty(case.q_codes.shape, dtype=dv["q"].dtype, device=DEV)
        args = (Xd, B, d, wdev["W_SK"], wdev["W_SV"], wdev["U_K"], wdev["U_V"], reqd, posd,
                dv["table"], case.table.shape[1], pool, case.num_pages)
        if fused:
            p = fresh_workspace(pb, 0xFF)
            F.lrkv_append_pq(lay, *args, dv["q"], B, 1, dv["BK"], p, pb)
            F.lrkv_decode_pq(lay, dv["q"], p, pb, B, 1, dv["BV"], pool, dv["table"],
                             case.table.shape[1], dv["lens"], msl, 0, out, ws, nb)
        else:
            F.lrkv_append(lay, *args)
            F.lrkv_decode(lay, dv["q"], B, 1, dv["BK"], dv["BV"], pool, dv["table"],
                          case.table.shape[1], dv["lens"], msl, 0, out, ws, nb)
        torch.cuda.synchronize()
        outs.append(out)
    assert torch.equal(outs[0], outs[1])
    log("append_pq + decode_pq step: bit-identical to append + decode")
