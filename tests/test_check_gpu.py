"""GPU checks of lrkv_check_indices: it counts exactly the index values that break the
page layout's rules (lengths, the page ids a length covers, appended rows' request,
position and page), and nothing else.  Only the checking kernels run: no call here
reads the pool, so the bad values planted below are never dereferenced."""

import numpy as np
import pytest
import torch

import factored_rank_kv_amd as F
from lrkv_case import log

pytestmark = pytest.mark.gpu

LAY = F.lrkv_layout(16, 128, 56, 16, F.LRKV_BF16)
DEV = "cuda:0"


def count(table, lens, max_seq_len, num_pages, rows=None):
    t = torch.from_numpy(np.ascontiguousarray(table, dtype=np.int32)).to(DEV)
    s = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    rq = rp = None
    n = 0
    if rows is not None:
        rq = torch.tensor([r for r, _ in rows], dtype=torch.int32, device=DEV)
        rp = torch.tensor([p for _, p in rows], dtype=torch.int32, device=DEV)
        n = len(rows)
    err = torch.full((1,), -7, dtype=torch.int32, device=DEV)  # must be overwritten
    F.lrkv_check_indices(LAY, t, table.shape[0], table.shape[1], s, max_seq_len, rq, rp, n,
                         num_pages, err)
    torch.cuda.synchronize()
    return int(err.item())


def valid_case(seed=0, B=5, max_pages=20):
    g = np.random.default_rng(seed)
    lens = g.integers(0, max_pages * 16 + 1, B).tolist()
    num_pages = B * max_pages
    table = g.permutation(num_pages).astype(np.int32).reshape(B, max_pages)
    return table, lens, num_pages


def test_valid_tables_count_zero():
    table, lens, npg = valid_case()
    log(f"valid tables, lengths {lens}")
    rows = [(b, p) for b in range(len(lens)) for p in (0, 17, 319)]
    assert count(table, lens, 320, npg, rows) == 0
    assert count(table, None, 320, npg, rows) == 0
    assert count(table, lens, 320, npg) == 0


def test_unused_table_entries_are_not_checked():
    """Entries past a request's last page may hold anything (here -1): they are never read."""
    table, lens, npg = valid_case(1)
    lens = [33, 0, 16, 320, 1]
    table = table.copy()
    for b, T in enumerate(lens):
        table[b, (T + 15) // 16:] = -1
    assert count(table, lens, 320, npg) == 0


def test_each_planted_violation_is_counted():
    table, lens, npg = valid_case(2)
    lens = [320, 300, 17, 64, 5]
    t = table.copy()
    t[0, 3] = npg          # page id one past the pool
    t[1, 18] = -5          # negative page id, covered by length 300 (19 pages)
    t[2, 1] = 10 ** 9      # covered by length 17 (2 pages)
    t[2, 2] = -1           # not covered: not counted
    bad_lens = list(lens)
    bad_lens[3] = 321      # above max_seq_len: counted once, its pages skipped
    bad_lens[4] = -2       # negative length
    log("planted: 3 page ids, 2 lengths")
    assert count(t, bad_lens, 320, npg) == 5
    rows = [(0, 0), (5, 0), (-1, 3), (1, 320), (1, -1), (0, 48), (1, 300)]
    # (5, 0) request past the batch; (-1, 3) negative request; (1, 320) position past the
    # table row; (1, -1) negative position; (0, 48) lands on the bad page t[0, 3]; (1, 300)
    # lands on t[1, 18]
    log("planted: 6 bad rows among 7")
    assert count(t, None, 320, npg, rows) == 6
    assert count(t, bad_lens, 320, npg, rows) == 11


def test_large_table_many_blocks():
    """A table larger than one dispatch wave of the index-check kernel (grid-stride loop), with the
    violations spread over it."""
    B, max_pages = 64, 4096
    npg = B * max_pages
    table = np.arange(npg, dtype=np.int32).reshape(B, max_pages)
    lens = [max_pages * 16] * B
    g = np.random.default_rng(3)
    idx = g.choice(npg, 37, replace=False)
    table.reshape(-1)[idx] = npg + 1
    log("262144 entries, 37 bad")
    assert count(table, lens, max_pages * 16, npg) == 37
