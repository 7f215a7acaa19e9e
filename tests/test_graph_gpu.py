"""HIP graph capture of the library's calls, as a serving loop replays one graph per decode
step: lrkv_append (decode-step and prompt-sized), lrkv_decode (chunked and balanced split),
lrkv_decode_noalloc, lrkv_decode_rope and the step lrkv_append_pq + lrkv_decode_pq, each
captured by torch's graph capture on the
launch stream and replayed several times, with eager work on the same stream between the
replays (the output and the workspace poisoned, an unrelated reduction).  Every replay must
give the eager call's result bit for bit: the kernels are deterministic, and the library
records no memory-set nodes (it clears nothing with hipMemsetAsync)."""

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
REPLAYS = 4


def capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    return g


def replay_and_check(g, got, want, clobber, what):
    for i in range(REPLAYS):
        clobber(i)
        torch.randn(1 << 20, device=DEV).sum().item()  # unrelated eager work in between
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"{what}: replay {i} differs from the eager call"
    log(f"{what}: {REPLAYS} replays bit-identical to the eager call")


def decode_setup(case, rope_cs=None):
    d = case.dev
    lay = layout_c(case.L)
    msl = int(case.lens.max())
    if rope_cs is None:
        nb = F.lrkv_decode_workspace_bytes(lay, case.B, case.q_len, msl, 0)
    else:
        nb = F.lrkv_decode_rope_workspace_bytes(lay, case.B, case.q_len, msl, 0)
    ws = fresh_workspace(nb, 0xFF)
    out = torch.empty(case.q_codes.shape, dtype=d["q"].dtype, device=DEV)
    return d, lay, msl, nb, ws, out


@pytest.mark.parametrize("lens,what", [([300, 17, 1, 129, 0], "chunked split"),
                                       ([200, 33] * 10, "balanced split, 20 requests")])
def test_decode_replays(lens, what):
    case = iid_case(501, 16, 128, 56, O.BF16, lens, permute=True, fill=0x7FC0)
    d, lay, msl, nb, ws, out = decode_setup(case)

    def call():
        F.lrkv_decode(lay, d["q"], case.B, 1, d["BK"], d["BV"], d["pool"], d["table"],
                      case.table.shape[1], d["lens"], msl, 0, out, ws, nb)

    call()
    torch.cuda.synchronize()
    want = out.clone()
    assert max_rel_err(from_dev(want, O.BF16), case.reference()) <= tolerance(O.BF16)
    g = capture(call)

    def clobber(i):
        out.fill_(-1)
        ws.fill_(0xFF if i % 2 else 0x00)  # the workspace need not be initialised

    replay_and_check(g, out, want, clobber, f"lrkv_decode, {what}")


def test_noalloc_decode_replays():
    case = iid_case(502, 32, 128, 32, O.BF16, [1000, 5, 64], permute=True, fill=0x7FC0)
    d = case.dev
    lay = layout_c(case.L)
    msl = int(case.lens.max())
    out = torch.empty(case.q_codes.shape, dtype=d["q"].dtype, device=DEV)

    def call():
        F.lrkv_decode_noalloc(lay, d["q"], case.B, 1, d["BK"], d["BV"], d["pool"], d["table"],
                              case.table.shape[1], d["lens"], msl, 0, out)

    call()
    torch.cuda.synchronize()
    want = out.clone()
    assert torch.equal(want.cpu(), case.run().cpu())  # the same kernels as lrkv_decode
    g = capture(call)
    replay_and_check(g, out, want, lambda i: out.fill_(-1), "lrkv_decode_noalloc")


def test_rope_decode_replays():
    case = iid_case(503, 16, 128, 56, O.BF16, [250, 16, 3], permute=True, fill=0x7FC0)
    cs = synth.rope_table(250, 128)
    d, lay, msl, nb, ws, out = decode_setup(case, cs)
    cs_dev = torch.from_numpy(np.ascontiguousarray(cs, np.float32)).to(DEV)

    def call():
        F.lrkv_decode_rope(lay, d["q"], case.B, 1, d["BK"], d["BV"], d["pool"], d["table"],
                           case.table.shape[1], d["lens"], msl, 0, cs_dev, cs.shape[0], out, ws,
                           nb)

    call()
    torch.cuda.synchronize()
    want = out.clone()
    assert max_rel_err(from_dev(want, O.BF16), case.reference_rope(cs)) <= tolerance(O.BF16)
    g = capture(call)

    def clobber(i):
        out.fill_(-1)
        ws.fill_(0xFF if i % 2 else 0x00)

    replay_and_check(g, out, want, clobber, "lrkv_decode_rope")


@pytest.mark.parametrize("n_rows", [8, 70])
def test_append_replays(n_rows):
    """8 rows (the decode step's kernel) and 70 rows (the prompt-sized product)."""
    H, dh, r, d = 16, 128, 56, 256
    L = O.Layout(H, dh, r, 16, O.BF16)
    g = np.random.default_rng(504 + n_rows)
    X = as_codes(g.standard_normal((n_rows, d)).astype(np.float32), O.BF16)
    w = {"W_SK": (d, dh), "W_SV": (d, dh), "U_K": (d, H, r), "U_V": (d, H, r)}
    wdev = {k: to_dev(output_major(as_codes((g.standard_normal(s) / np.sqrt(d)).astype(np.float32),
                                            O.BF16)))
            for k, s in w.items()}
    lens = [n_rows + 10, 40]
    table, npg = synth.page_assignment(505, lens, 16, True)
    req = np.zeros(n_rows, np.int32)
    pos = np.arange(n_rows, dtype=np.int32) + 5
    pool0 = torch.zeros(npg * O.page_bytes(L), dtype=torch.uint8, device=DEV)
    pool = pool0.clone()
    Xd, reqd, posd, tabd = (to_dev(X), to_dev(req), to_dev(pos),
                            to_dev(np.ascontiguousarray(table, np.int32)))
    lay = layout_c(L)

    def call():
        F.lrkv_append(lay, Xd, n_rows, d, wdev["W_SK"], wdev["W_SV"], wdev["U_K"], wdev["U_V"],
                      reqd, posd, tabd, table.shape[1], pool, npg)

    call()
    torch.cuda.synchronize()
    want = pool.clone()
    assert int((want != 0).sum()) > 0
    gr = capture(call)
    replay_and_check(gr, pool, want, lambda i: pool.copy_(pool0), f"lrkv_append, {n_rows} rows")


def test_append_pq_decode_pq_step_replays():
    """The decode step with the private queries formed beside the append: lrkv_append_pq
    then lrkv_decode_pq, captured as one graph; p, the output and the workspace are poisoned
    between the replays."""
    H, dh, r, d = 16, 128, 56, 256
    lens_before = [120, 7, 64, 31]
    B = len(lens_before)
    case = iid_case(506, H, dh, r, O.BF16, [t + 1 for t in lens_before], fill=0x7FC0)
    dv = case.dev
    L = case.L
    lay = layout_c(L)
    g = np.random.default_rng(507)
    Xd = to_dev(as_codes(g.standard_normal((B, d)).astype(np.float32), O.BF16))
    wdev = {k: to_dev(output_major(as_codes((g.standard_normal(s) / np.sqrt(d)).astype(np.float32),
                                            O.BF16)))
            for k, s in {"W_SK": (d, dh), "W_SV": (d, dh), "U_K": (d, H, r),
                         "U_V": (d, H, r)}.items()}
    reqd = to_dev(np.arange(B, dtype=np.int32))
    posd = to_dev(np.array(lens_before, np.int32))
    msl = int(case.lens.max())
    nb = F.lrkv_decode_workspace_bytes(lay, B, 1, msl, 0)
    ws = fresh_workspace(nb, 0xFF)
    pb = F.lrkv_private_queries_bytes(lay, B, 1)
    p = fresh_workspace(pb, 0xFF)
    pool = dv["pool"].clone()
    out = torch.empty(case.q_codes.shape, dtype=dv["q"].dtype, device=DEV)

    def call():
        F.lrkv_append_pq(lay, Xd, B, d, wdev["W_SK"], wdev["W_SV"], wdev["U_K"], wdev["U_V"], reqd,
                         posd, dv["table"], case.table.shape[1], pool, case.num_pages, dv["q"], B, 1,
                         dv["BK"], p, pb)
        F.lrkv_decode_pq(lay, dv["q"], p, pb, B, 1, dv["BV"], pool, dv["table"], case.table.shape[1],
                         dv["lens"], msl, 0, out, ws, nb)

    call()
    torch.cuda.synchronize()
    want = out.clone()
    pool_want = pool.clone()
    # the eager step against lrkv_append + lrkv_decode on a fresh copy of the cache
    pool2 = dv["pool"].clone()
    out2 = torch.empty_like(out)
    F.lrkv_append(lay, Xd, B, d, wdev["W_SK"], wdev["W_SV"], wdev["U_K"], wdev["U_V"], reqd, posd,
                  dv["table"], case.table.shape[1], pool2, case.num_pages)
    F.lrkv_decode(lay, dv["q"], B, 1, dv["BK"], dv["BV"], pool2, dv["table"], case.table.shape[1],
                  dv["lens"], msl, 0, out2, fresh_workspace(nb, 0xFF), nb)
    torch.cuda.synchronize()
    assert torch.equal(want, out2) and torch.equal(pool_want, pool2)
    gr = capture(call)

    def clobber(i):
        out.fill_(-1)
        p.fill_(0xFF if i % 2 else 0x00)
        ws.fill_(0x00 if i % 2 else 0xFF)

    replay_and_check(gr, out, want, clobber, "lrkv_append_pq + lrkv_decode_pq")
    assert torch.equal(pool, pool_want)
