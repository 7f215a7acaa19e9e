"""Reference model of the page bookkeeping for shared-prefix reuse and reclamation.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``): plain Python lists, what the C
library's page allocator must agree with, operation by operation.

LRKV notes §3, the note after Algorithm 1: under paged allocation, shared pages and
per-head private pages must keep the same token numbering and reclamation lifetime, or a
reused prefix or a released request can leave the two paths of one position pointing at
different histories.  The layout puts every section of a token in one page, so the model
only has to count, per page, the requests that hold it:

* alloc(n): n free pages, taken from the top of a stack of free ids, each held once;
* retain(ids): one more holder per listed page (a request that shares it), only for pages
  in use;
* release(ids): one holder less per listing; a page left with none goes back on the stack
  (in list order, once);
* fork(parent_row, prefix_len, P): a request continuing the first prefix_len tokens of
  another shares its full pages and gets a copy of the page holding the prefix's last
  tokens when that page is only partly covered (so the two can append independently).

Status codes: OK 0, INVALID_ARG -1, NO_PAGES -5 (the C header's values).
"""

from collections import Counter

OK, INVALID_ARG, NO_PAGES = 0, -1, -5


class PagePoolModel:
    def __init__(self, num_pages: int):
        self.n = num_pages
        self.ref = [0] * num_pages
        self.free = list(range(num_pages - 1, -1, -1))  # the top (end) is page 0

    def alloc(self, k: int):
        if k > len(self.free):
            return NO_PAGES, []
        ids = [self.free.pop() for _ in range(k)]
        for i in ids:
            self.ref[i] = 1
        return OK, ids

    def retain(self, ids):
        if any(not 0 <= i < self.n or self.ref[i] <= 0 for i in ids):
            return INVALID_ARG
        for i in ids:
            self.ref[i] += 1
        return OK

    def release(self, ids):
        if any(not 0 <= i < self.n for i in ids):
            return INVALID_ARG
        if any(self.ref[i] < c for i, c in Counter(ids).items()):
            return INVALID_ARG
        for i in ids:
            self.ref[i] -= 1
        pushed = set()
        for i in ids:
            if self.ref[i] == 0 and i not in pushed:
                self.free.append(i)
                pushed.add(i)
        return OK

    def fork(self, parent_row, prefix_len: int, page_size: int):
        """Returns (status, child pages of the prefix, (source, destination) of the copy or
        None)."""
        full, part = divmod(prefix_len, page_size)
        part = 1 if part else 0
        need = list(parent_row[:full + part])
        if any(not 0 <= i < self.n or self.ref[i] <= 0 for i in need):
            return INVALID_ARG, [], None
        copy = None
        child = list(parent_row[:full])
        if part:
            st, ids = self.alloc(1)
            if st != OK:
                return st, [], None
            copy = (parent_row[full], ids[0])
            child.append(ids[0])
        self.retain(parent_row[:full])
        return OK, child, copy
