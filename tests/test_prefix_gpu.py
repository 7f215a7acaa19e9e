"""Shared-prefix page reuse and reclamation on the GPU (LRKV notes §3, the note after
Algorithm 1: shared and private rows of a position keep one page, one numbering and one
lifetime).  A request forks from another's 40-token prefix (two full pages shared, the
partial third page copied on write), both append different tokens past it, the parent is
released and its reclaimed pages reused by a new request, then the child is released and
the old prefix pages reused in turn.

Rows are exact-arithmetic (X and weights in {-1, 0, 1}, d = 256), so after every step the
GPU pool must equal, byte for byte, the pool the oracle builds by its own Algorithm-1
append through the same page tables; decode outputs are compared against the oracle's
decode of its own pool (1e-2 of max|ref|), and a request whose pages were not touched must
decode to the same bits as before."""

import numpy as np
import pytest
import torch

import factored_rank_kv_amd as F
import oracle as O
from oracle.page_pool import PagePoolModel
from lrkv_case import as_codes, layout_c, log, max_rel_err, output_major, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
H, DH, R, D, P = 16, 128, 56, 256, 16


class World:
    """Device pool + oracle pool, kept in step through the same page tables."""

    def __init__(self, num_pages, seed):
        self.L = O.Layout(H, DH, R, P, O.BF16)
        self.lay = layout_c(self.L)
        self.pb = O.page_bytes(self.L)
        self.num_pages = num_pages
        self.dev = torch.full((num_pages * self.pb,), 0x5A, dtype=torch.uint8, device=DEV)
        self.ref = np.full(num_pages * self.pb, 0x5A, np.uint8)
        g = np.random.default_rng(seed)
        self.g = g
        self.w = {k: g.integers(-1, 2, s).astype(np.float64) for k, s in
                  (("W_SK", (D, DH)), ("W_SV", (D, DH)), ("U_K", (D, H, R)), ("U_V", (D, H, R)))}
        self.BK = O.round_to_dtype(g.standard_normal((H, DH, R)) / np.sqrt(R), O.BF16)
        self.BV = O.round_to_dtype(g.standard_normal((H, DH, R)) / np.sqrt(R), O.BF16)
        self.wd = {k: to_dev(output_major(as_codes(v.astype(np.float32), O.BF16)))
                   for k, v in self.w.items()}
        self.pages = F.PagePool(num_pages)
        self.model = PagePoolModel(num_pages)

    def alloc(self, n):
        ids = np.zeros(n, np.int32)
        F.lrkv_pages_alloc(self.pages, n, ids)
        st, mids = self.model.alloc(n)
        assert st == 0 and ids.tolist() == mids
        return ids.tolist()

    def release(self, ids):
        F.lrkv_pages_release(self.pages, np.array(ids, np.int32), len(ids))
        assert self.model.release(list(ids)) == 0
        assert self.pages.refcount.tolist() == self.model.ref

    def append(self, row_table, start, n):
        """n new exact rows at positions start.. of the request whose pages are row_table."""
        X = self.g.integers(-1, 2, (n, D)).astype(np.float64)
        table = np.array([row_table], np.int32)
        req = np.zeros(n, np.int32)
        pos = np.arange(start, start + n, dtype=np.int32)
        F.lrkv_append(self.lay, to_dev(as_codes(X.astype(np.float32), O.BF16)), n, D,
                      self.wd["W_SK"], self.wd["W_SV"], self.wd["U_K"], self.wd["U_V"],
                      to_dev(req), to_dev(pos), to_dev(table), table.shape[1], self.dev,
                      self.num_pages)
        self.ref = O.append_reference(self.ref, self.L, X, self.w["W_SK"], self.w["W_SV"],
                                      self.w["U_K"], self.w["U_V"], req, pos, table)

    def fork(self, parent_row, prefix_len, width):
        child = np.full(width, -1, np.int32)
        row = np.array(parent_row + [0] * (width - len(parent_row)), np.int32)
        F.lrkv_fork_prefix(self.lay, self.pages, row, prefix_len, child, width, self.dev)
        st, mchild, copy = self.model.fork(parent_row, prefix_len, P)
        assert st == 0 and child[:len(mchild)].tolist() == mchild
        if copy is not None:  # the oracle's own copy of every section of the page
            s, d = copy
            self.ref[d * self.pb:(d + 1) * self.pb] = self.ref[s * self.pb:(s + 1) * self.pb]
        return mchild

    def check_pool(self, what):
        torch.cuda.synchronize()
        got = self.dev.cpu().numpy()
        diff = np.count_nonzero(got != self.ref)
        log(f"{what}: pool bytes differing from the oracle's: {diff}")
        assert diff == 0

    def decode(self, rows, lens, q):
        width = max(len(r) for r in rows)
        table = np.array([r + [0] * (width - len(r)) for r in rows], np.int32)
        lay = self.lay
        msl = max(lens)
        n = F.lrkv_decode_workspace_bytes(lay, len(rows), 1, msl, 16)
        ws = torch.empty(n, dtype=torch.uint8, device=DEV)
        out = torch.empty((len(rows), 1, H, DH), dtype=torch.int16, device=DEV)
        F.lrkv_decode(lay, to_dev(as_codes(q, O.BF16)), len(rows), 1, to_dev(as_codes(
            self.BK.astype(np.float32), O.BF16)), to_dev(as_codes(self.BV.astype(np.float32),
                                                                O.BF16)),
            self.dev, to_dev(table), width, to_dev(np.array(lens, np.int32)), msl, 16, out, ws, n)
        torch.cuda.synchronize()
        got = O.bf16_bits_to_f64(out.cpu().numpy().view(np.uint16))
        q64 = O.bf16_bits_to_f64(as_codes(q, O.BF16))
        ref = O.decode_reference(self.L, q64, self.BK, self.BV, self.ref, table, lens)
        return got, ref, out.cpu()


def test_shared_prefix_fork_release_reuse():
    w = World(16, 700)
    qg = np.random.default_rng(701)
    q = lambda n: qg.standard_normal((n, 1, H, DH)).astype(np.float32)
    A = w.alloc(3)  # 40 tokens: two full pages and 8 slots of the third
    w.append(A, 0, 40)
    w.check_pool("request A, 40 tokens")
    B = w.fork(A, 40, 8)  # shares A's two full pages, copies the partial third
    assert B[:2] == A[:2] and B[2] not in A
    assert w.pages.refcount[A[0]] == 2 and w.pages.refcount[A[2]] == 1
    w.check_pool("fork at 40 tokens (tail page copied)")
    w.append(A, 40, 8)  # fills A's third page
    A += w.alloc(1)
    w.append(A, 48, 2)
    w.append(B, 40, 8)  # B's own copy of the third page
    B += w.alloc(1)
    w.append(B, 48, 4)
    w.check_pool("A +10 tokens, B +12 different tokens")
    qa = q(2)
    got, ref, out_ab = w.decode([A, B], [50, 52], qa)
    err = max_rel_err(got, ref)
    log(f"decode A (50) and B (52) over shared prefix pages: max rel err {err:.3e}")
    assert err <= 1e-2
    assert max_rel_err(got[0], got[1]) > 1e-3  # different histories past the prefix

    w.release(A)  # the prefix pages stay (B holds them); A's own pages are reclaimed
    assert w.pages.refcount[A[0]] == 1 and w.pages.refcount[A[2]] == 0
    C = w.alloc(2)
    assert set(C) <= set(A)  # reclaimed pages reused
    w.append(C, 0, 20)
    w.check_pool("A released, C (20 tokens) in A's reclaimed pages")
    got2, ref2, out_bc = w.decode([B, C], [52, 20], np.stack([qa[1], q(1)[0]]))
    assert torch.equal(out_bc[0], out_ab[1])  # B's pages untouched: the same bits
    err = max_rel_err(got2, ref2)
    log(f"decode B again and C: max rel err {err:.3e}; B bit-identical to before")
    assert err <= 1e-2

    w.release(B)  # now the old prefix pages are free too
    assert w.pages.refcount[B[0]] == 0
    Dr = w.alloc(4)
    assert set(B[:2]) <= set(Dr)  # the reclaimed prefix pages are reused
    w.append(Dr, 0, 61)
    w.check_pool("B released, D (61 tokens) reusing the old prefix pages")
    got3, ref3, out_cd = w.decode([C, Dr], [20, 61], np.stack([q(1)[0], q(1)[0]]))
    err = max_rel_err(got3, ref3)
    log(f"decode C and D: max rel err {err:.3e}")
    assert err <= 1e-2
    assert w.pages.num_free == 16 - 2 - 4


def test_copy_pages_moves_every_section_of_a_key_norm_page():
    """lrkv_copy_pages on a key-norm layout: destination pages equal their sources byte for
    byte (S_K, S_V, R_K, R_V and the norm reciprocals), every other page unchanged."""
    lay = F.lrkv_layout(16, 128, 56, 16, F.LRKV_BF16, 1)
    pb = F.lrkv_page_bytes(lay)
    g = np.random.default_rng(702)
    host = g.integers(0, 256, 8 * pb, dtype=np.uint8)
    dev = torch.from_numpy(host.copy()).to(DEV)
    src, dst = np.array([5, 0, 7], np.int32), np.array([1, 6, 2], np.int32)
    F.lrkv_copy_pages(lay, dev, to_dev(src), to_dev(dst), 3)
    torch.cuda.synchronize()
    want = host.copy()
    for s, d in zip(src, dst):
        want[d * pb:(d + 1) * pb] = host[s * pb:(s + 1) * pb]
    assert np.array_equal(dev.cpu().numpy(), want)
