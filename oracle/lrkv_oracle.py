"""Plain float64 CPU oracle for Low-Rank Key Value attention (LRKV).

TEST INFRASTRUCTURE ONLY.  This module is what the tests compare the library against,
not the product.  It may be imported only by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``.  The library in ``factored_rank_kv_amd/`` never imports, links or runs
it, and it shares no code with that library.

What it follows
---------------
"LRKV notes" below means the web page *Low-Rank Key Value Attention｜共享缓存与逐头残差*
(Zhongzhu Zhou's reading notes on O'Neill, Clancy, Matskevichus and Reid, arXiv 2601.11471).
The method reaches exactly, up to rounding order, the result of plain softmax attention
over the reconstructed per-head keys and values (LRKV notes §3, the associativity argument
around eq 6-7 and the worked 2-D example).  So the oracle *is* that plain definition:

1. page walk: read the cached rows of one request out of the paged pool;
2. reconstruct K_h = S_K + R_K[h] B_K[h]^T and V_h = S_V + R_V[h] B_V[h]^T (eq 2-5);
3. score each visible key with q_h k_j^T / sqrt(d_h) (§2, the attention definition and the
   remark that the divisor is the full head width);
4. one softmax over the visible positions (§2);
5. o_h = sum_j a_j v_j (§2).

A second, independent coding follows Algorithm 2 of §3 step by step (private query formed
once, summed branch scores, one softmax, both value branches reduced with the same weights,
one expansion through B_V[h]^T).  It is used only to check the first one.

The append oracle follows Algorithm 1 of §3: the shared projections X W_S_K and X W_S_V and
the per-head projections X U_K[h], X U_V[h], computed in float64 and rounded to nearest
even into the cache dtype, then placed at the rows' token positions.

The cache-size and cost formulas of §4 (eq 9, rank budget, parameter ratio, decode
arithmetic ratio, tensor-parallel replication) are written with exact rationals.

Readings where the page is silent (each is also listed in the design notes):
* the visible set of query row i of request b is positions j <= T_b - q_len + i, so a
  single-row decode sees all T_b cached tokens including the token just appended;
* masked positions are removed by selection, never multiplied by zero, so whatever bytes sit
  in unused page slots cannot leak into a result;
* a request with no visible token returns zeros;
* Algorithm 2's scaling step names the square root of the head width without saying
  whether to multiply or divide; the oracle divides by sqrt(d_h), as the attention formula
  of §2 does, and never uses sqrt(r).

Parity pins: every function here is pinned by tests/test_oracle.py against values the page
prints (worked example, cache percentages and MiB figures), closed forms, textbook library
routines (torch scaled-dot-product attention in float64 for the r = 0 and r = d_h cases)
and brute force on tiny inputs.  Nothing here is "parity unpinned".
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from fractions import Fraction

import numpy as np

F32 = 0
BF16 = 1
_ELEM_BYTES = {F32: 4, BF16: 2}

# ---------------------------------------------------------------------------------------
# Element encodings
# ---------------------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact bfloat16 -> float64: the 16 stored bits are the high half of a binary32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16, ties to even; return the 16-bit codes.

    Written from the format's definition (8 significant bits, binary32 exponent range),
    rounding the float64 value once (no detour through binary32, which could round twice).
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_x = x.reshape(-1)
    flat_o = out.reshape(-1)
    nan = np.isnan(flat_x)
    flat_o[nan] = 0x7FC0
    fin = ~nan
    v = flat_x[fin]
    sign = np.signbit(v)
    a = np.abs(v)
    # exponent e with 2^(e-1) <= a < 2^e (frexp mantissa in [0.5, 1)); zeros give e = 0
    _, e = np.frexp(a)
    # spacing of bf16 numbers in [2^(e-1), 2^e) is 2^(e-1-7); subnormals share 2^-133
    e_eff = np.maximum(e, -125)
    spacing = np.ldexp(1.0, (e_eff - 8).astype(np.int64))
    q = np.rint(a / spacing)  # numpy rint rounds half to even
    r = q * spacing  # exact: q has at most 9 significant bits
    r = np.where(r >= 2.0**128, np.inf, r)  # past the largest finite bf16 magnitude
    r = np.where(np.isinf(a), np.inf, r)
    bits = (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(sign, bits | np.uint16(0x8000), bits)
    flat_o[fin] = bits
    return out


def decode_elems(raw: np.ndarray, dtype: int) -> np.ndarray:
    """Bytes of a cache region -> float64 values (exact widening)."""
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    if dtype == BF16:
        return bf16_bits_to_f64(raw.view(np.uint16))
    if dtype == F32:
        return raw.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype}")


def encode_elems(x: np.ndarray, dtype: int) -> np.ndarray:
    """float64 values -> bytes in the cache dtype, rounding to nearest even."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == BF16:
        return f64_to_bf16_bits(x).view(np.uint8).reshape(-1)
    if dtype == F32:
        return x.astype(np.float32).view(np.uint8).reshape(-1)
    raise ValueError(f"unknown dtype {dtype}")


def round_to_dtype(x: np.ndarray, dtype: int) -> np.ndarray:
    """float64 -> nearest value of the cache dtype, returned as float64."""
    return decode_elems(encode_elems(x, dtype), dtype).reshape(np.shape(x))


# ---------------------------------------------------------------------------------------
# Factored paged cache layout (LRKV notes §3: shared and private rows of one token share
# one page id, so token numbering and page lifetime are identical for both paths)
# ---------------------------------------------------------------------------------------


@dataclass(frozen=True)
class Layout:
    num_heads: int  # H
    head_dim: int  # d_h, width of a shared row S_K[j], S_V[j]
    rank: int  # r, width of a private row R_K[h, j], R_V[h, j]
    page_size: int  # P tokens per page
    dtype: int  # F32 or BF16
    # LRKV notes §8 (RMSNorm paragraph): one stored reciprocal of the joint key denominator
    # per head and position, in the cache dtype, as a fifth section N[h][t] of each page
    key_norm: bool = False
    # LRKV notes §3 (after the gradient formulas): one shared block per group of heads.
    # Heads h of group g = h // (H / groups) use S_K[g], S_V[g]; 1 = one block for all heads
    groups: int = 1

    def group_of(self, h: int) -> int:
        return h // (self.num_heads // self.groups)

    @property
    def elem_bytes(self) -> int:
        return _ELEM_BYTES[self.dtype]

    @property
    def chunk(self) -> int:
        """Elements per 16-byte chunk."""
        return 16 // self.elem_bytes


# A page of a key-norm layout is padded to a multiple of this many bytes (zero to 1 KiB - 16
# bytes of padding at its end, never read or written): the pages fix which rows a page
# holds, not its byte length, and reads of pages that start off a 1 KiB boundary were
# measured markedly slower on the target device.  Other layouts are multiples already.
KEY_NORM_PAGE_ALIGN = 1024


def page_data_bytes(L: Layout) -> int:
    """Bytes of the rows of one page: P tokens x (2 shared rows of d_h per group + 2H
    private rows of r), plus P x H key-norm reciprocals when the layout keeps them."""
    extra = L.page_size * L.num_heads if L.key_norm else 0
    return (L.page_size * 2 * (L.groups * L.head_dim + L.num_heads * L.rank) + extra) * L.elem_bytes


def page_bytes(L: Layout) -> int:
    """Bytes from one page to the next: the rows, and for a key-norm layout the padding up
    to a multiple of KEY_NORM_PAGE_ALIGN."""
    raw = page_data_bytes(L)
    if L.key_norm:
        raw = -(-raw // KEY_NORM_PAGE_ALIGN) * KEY_NORM_PAGE_ALIGN
    return raw


def page_elems(L: Layout) -> int:
    """Elements from one page to the next (rows and padding)."""
    return page_bytes(L) // L.elem_bytes


def section_base(L: Layout, section: str, head: int = 0) -> int:
    """Element offset, inside a page, of a section: `head` is the group for the shared
    sections "SK", "SV" and the head for the private ones.

    A page is one block per group of heads, in group order; block g holds S_K[g], S_V[g]
    (P x d_h each), then R_K of the group's heads, then R_V of the group's heads (P x r
    each), so with one group: S_K, S_V, R_K[0..H-1], R_V[0..H-1].  The key-norm section
    (one group only) follows: N[h], P elements per head.
    """
    P, dh, r, H, G = L.page_size, L.head_dim, L.rank, L.num_heads, L.groups
    Hg = H // G
    block = P * 2 * (dh + Hg * r)
    if section == "SK":
        return head * block
    if section == "SV":
        return head * block + P * dh
    g, j = divmod(head, Hg)  # private sections: group and place of the head in it
    if section == "RK":
        return g * block + 2 * P * dh + j * P * r
    if section == "RV":
        return g * block + 2 * P * dh + Hg * P * r + j * P * r
    if section == "N" and L.key_norm and G == 1:  # head h's P reciprocals, token after token
        return 2 * P * dh + 2 * H * P * r + head * P
    raise ValueError(section)


def in_block_index(L: Layout, width: int, t: np.ndarray, k: np.ndarray) -> np.ndarray:
    """Element index of (token slot t, feature k) inside a block of P rows of `width`.

    Chunk-major: the block is a sequence of 16-byte chunk columns; chunk column c holds the
    P tokens' features [c*C, (c+1)*C) back to back, C = 16 / element bytes.
    """
    C = L.chunk
    if width % C:
        raise ValueError(f"width {width} is not a multiple of the {C}-element chunk")
    return ((k // C) * L.page_size + t) * C + (k % C)


def _positions_to_pages(L: Layout, table_row: np.ndarray, n: int):
    j = np.arange(n)
    return np.asarray(table_row, dtype=np.int64)[j // L.page_size], j % L.page_size


def _read_block(pool, L: Layout, pages, t, section, head, width):
    pe = page_elems(L)
    b = L.elem_bytes
    k = np.arange(width)
    idx = (pages[:, None] * pe + section_base(L, section, head)
           + in_block_index(L, width, t[:, None], k[None, :]))
    byte_idx = (idx[..., None] * b + np.arange(b)).reshape(-1)
    return decode_elems(pool[byte_idx], L.dtype).reshape(len(pages), width)


def gather_shared(pool, L: Layout, table_row, n_tokens: int, group: int = 0):
    """Page walk for the shared rows of tokens 0..n_tokens-1 (of one group of heads): S_K,
    S_V as [n, d_h] float64.

    Token j lives in page table_row[j // P], slot j % P.
    """
    pool = np.asarray(pool, dtype=np.uint8).reshape(-1)
    pages, t = _positions_to_pages(L, table_row, n_tokens)
    return (_read_block(pool, L, pages, t, "SK", group, L.head_dim),
            _read_block(pool, L, pages, t, "SV", group, L.head_dim))


def gather_private(pool, L: Layout, table_row, n_tokens: int, h: int):
    """Page walk for head h's private rows: R_K[h], R_V[h] as [n, r] float64."""
    pool = np.asarray(pool, dtype=np.uint8).reshape(-1)
    if L.rank == 0:
        return np.zeros((n_tokens, 0)), np.zeros((n_tokens, 0))
    pages, t = _positions_to_pages(L, table_row, n_tokens)
    return (_read_block(pool, L, pages, t, "RK", h, L.rank),
            _read_block(pool, L, pages, t, "RV", h, L.rank))


def gather_norms(pool, L: Layout, table_row, n_tokens: int, h: int):
    """Page walk for head h's stored key-norm reciprocals of tokens 0..n_tokens-1 [n]."""
    pool = np.asarray(pool, dtype=np.uint8).reshape(-1)
    pages, t = _positions_to_pages(L, table_row, n_tokens)
    idx = pages * page_elems(L) + section_base(L, "N", h) + t
    byte_idx = (idx[:, None] * L.elem_bytes + np.arange(L.elem_bytes)).reshape(-1)
    return decode_elems(pool[byte_idx], L.dtype).reshape(n_tokens)


def gather_request(pool: np.ndarray, L: Layout, table_row: np.ndarray, n_tokens: int) -> dict:
    """Page walk over every section: S_K, S_V [n, d_h] (grouped layouts: [G, n, d_h]) and
    R_K, R_V [H, n, r], float64."""
    if L.groups == 1:
        SK, SV = gather_shared(pool, L, table_row, n_tokens)
    else:
        sh = [gather_shared(pool, L, table_row, n_tokens, g) for g in range(L.groups)]
        SK, SV = np.stack([a for a, _ in sh]), np.stack([b for _, b in sh])
    priv = [gather_private(pool, L, table_row, n_tokens, h) for h in range(L.num_heads)]
    return {"SK": SK, "SV": SV,
            "RK": np.stack([p[0] for p in priv]) if priv else np.zeros((0, n_tokens, L.rank)),
            "RV": np.stack([p[1] for p in priv]) if priv else np.zeros((0, n_tokens, L.rank))}


def storage_dtype(L: Layout):
    """numpy type holding one cache element's bits."""
    return np.uint16 if L.dtype == BF16 else np.uint32


def pack_pool(L: Layout, page_table, lens, SK, SV, RK, RV, num_pages: int, fill: int = 0,
              NR=None):
    """Bulk placement of whole requests into a fresh pool (the placement rule of
    `write_rows`, coded separately as a reshape per page so the two check each other).

    SK, SV [sum(lens), d_h] and RK, RV [sum(lens), H, r] hold element *codes* (uint16
    bfloat16 codes, or uint32 float32 bit patterns), requests back to back in order.
    Every slot not written (pages no request owns, slots past a request's last token) holds
    the code `fill`.  Returns the pool as uint8 [num_pages * page_bytes].  Grouped layouts
    take SK, SV as [sum(lens), G, d_h].
    """
    st = storage_dtype(L)
    P, dh, r, H, C = L.page_size, L.head_dim, L.rank, L.num_heads, L.chunk
    pe = page_elems(L)
    if L.groups > 1:
        return _pack_pool_grouped(L, page_table, lens, SK, SV, RK, RV, num_pages, fill)
    pool = np.full((num_pages, pe), fill, dtype=st)
    off = 0
    for b, T in enumerate(lens):
        T = int(T)
        n_pages = -(-T // P)
        if n_pages == 0:
            continue
        ids = np.asarray(page_table[b][:n_pages], dtype=np.int64)

        def blocks(rows, width, heads):
            # rows [T, heads, width] -> [n_pages, heads * width * P] in chunk-major order
            padded = np.full((n_pages * P, heads, width), fill, dtype=st)
            padded[:T] = rows.reshape(T, heads, width)
            x = padded.reshape(n_pages, P, heads, width // C, C)
            return x.transpose(0, 2, 3, 1, 4).reshape(n_pages, heads * width * P)

        sk = np.asarray(SK[off:off + T]).view(st) if np.asarray(SK).dtype != st else SK[off:off + T]
        sv = np.asarray(SV[off:off + T]).view(st) if np.asarray(SV).dtype != st else SV[off:off + T]
        pool[ids, 0:P * dh] = blocks(sk, dh, 1)
        pool[ids, P * dh:2 * P * dh] = blocks(sv, dh, 1)
        if r:
            rk = np.asarray(RK[off:off + T])
            rv = np.asarray(RV[off:off + T])
            rk = rk.view(st) if rk.dtype != st else rk
            rv = rv.view(st) if rv.dtype != st else rv
            base = 2 * P * dh
            pool[ids, base:base + H * P * r] = blocks(rk, r, H)
            pool[ids, base + H * P * r:base + 2 * H * P * r] = blocks(rv, r, H)
        if L.key_norm and NR is not None:  # [T, H] codes -> N[h][t] of each page
            nr = np.asarray(NR[off:off + T])
            nr = nr.view(st) if nr.dtype != st else nr
            padded = np.full((n_pages * P, H), fill, dtype=st)
            padded[:T] = nr
            base = 2 * P * dh + 2 * H * P * r
            pool[ids, base:base + H * P] = padded.reshape(n_pages, P, H).transpose(0, 2, 1).reshape(
                n_pages, H * P)
        off += T
    return pool.view(np.uint8).reshape(-1)


def _pack_pool_grouped(L: Layout, page_table, lens, SK, SV, RK, RV, num_pages, fill):
    """Grouped layouts: each group's block is placed like a one-group page of its heads."""
    G, H = L.groups, L.num_heads
    Hg = H // G
    Lg = Layout(Hg, L.head_dim, L.rank, L.page_size, L.dtype)
    st = storage_dtype(L)
    blk = page_elems(Lg)
    pool = np.full((num_pages, page_elems(L)), fill, dtype=st)
    for g in range(G):
        part = pack_pool(Lg, page_table, lens, np.asarray(SK)[:, g], np.asarray(SV)[:, g],
                         np.asarray(RK)[:, g * Hg:(g + 1) * Hg],
                         np.asarray(RV)[:, g * Hg:(g + 1) * Hg], num_pages, fill)
        pool[:, g * blk:(g + 1) * blk] = part.view(st).reshape(num_pages, blk)
    return pool.view(np.uint8).reshape(-1)


def write_rows(pool: np.ndarray, L: Layout, page_table: np.ndarray, row_req, row_pos,
               SK, SV, RK, RV) -> np.ndarray:
    """Place already-rounded rows at their (request, position) in a copy of the pool.

    SK, SV: [n, d_h]; RK, RV: [n, H, r] (float64 values exactly representable in the dtype).
    Row n goes to page page_table[row_req[n]][row_pos[n] // P], slot row_pos[n] % P, in each
    section; only those elements change.  Rows must address distinct positions.
    """
    out = np.array(pool, dtype=np.uint8, copy=True).reshape(-1)
    elems = out.view(storage_dtype(L))
    pe = page_elems(L)
    H, dh, r = L.num_heads, L.head_dim, L.rank
    row_req = np.asarray(row_req, np.int64)
    row_pos = np.asarray(row_pos, np.int64)
    pages = np.asarray(page_table, np.int64)[row_req, row_pos // L.page_size]
    t = row_pos % L.page_size

    def put(section, head, width, vals):
        idx = (pages[:, None] * pe + section_base(L, section, head)
               + in_block_index(L, width, t[:, None], np.arange(width)[None, :]))
        elems[idx.reshape(-1)] = encode_elems(vals, L.dtype).view(storage_dtype(L))

    if L.groups == 1:
        put("SK", 0, dh, np.asarray(SK))
        put("SV", 0, dh, np.asarray(SV))
    else:  # SK, SV [n, G, d_h]
        for g in range(L.groups):
            put("SK", g, dh, np.asarray(SK)[:, g])
            put("SV", g, dh, np.asarray(SV)[:, g])
    for h in range(H if r else 0):
        put("RK", h, r, np.asarray(RK)[:, h])
        put("RV", h, r, np.asarray(RV)[:, h])
    return out


# ---------------------------------------------------------------------------------------
# Algorithm 1: build / append the factored cache (LRKV notes §3)
# ---------------------------------------------------------------------------------------


def project_rows(X, W_SK, W_SV, U_K, U_V):
    """Factored projections of new rows, float64 (eq 2-5; the projection and cache-write steps of Algorithm 1).

    X [n, d]; W_SK, W_SV [d, d_h] (one shared block per group of heads: [G, d, d_h]);
    U_K, U_V [d, H, r].
    Returns S_K, S_V [n, d_h] (grouped: [n, G, d_h]) and R_K, R_V [n, H, r].
    """
    X = np.asarray(X, np.float64)
    if np.ndim(W_SK) == 3:
        SK = np.stack([X @ np.asarray(w, np.float64) for w in W_SK], axis=1)
        SV = np.stack([X @ np.asarray(w, np.float64) for w in W_SV], axis=1)
    else:
        SK = X @ np.asarray(W_SK, np.float64)
        SV = X @ np.asarray(W_SV, np.float64)
    d, H, r = np.shape(U_K)
    RK = (X @ np.asarray(U_K, np.float64).reshape(d, H * r)).reshape(-1, H, r)
    RV = (X @ np.asarray(U_V, np.float64).reshape(d, H * r)).reshape(-1, H, r)
    return SK, SV, RK, RV


def append_reference(pool, L: Layout, X, W_SK, W_SV, U_K, U_V, row_req, row_pos, page_table):
    """Expected pool after appending rows X (Algorithm 1): project in float64, round each
    value to nearest even in the cache dtype, write it at the row's (page, slot) in all
    four sections; every other byte keeps its old value."""
    SK, SV, RK, RV = project_rows(X, W_SK, W_SV, U_K, U_V)
    rnd = lambda a: round_to_dtype(a, L.dtype)
    return write_rows(pool, L, np.asarray(page_table), np.asarray(row_req), np.asarray(row_pos),
                      rnd(SK), rnd(SV), rnd(RK), rnd(RV))


# ---------------------------------------------------------------------------------------
# RMSNorm of the full key (LRKV notes §8, "RMSNorm has one more per-head joint quantity"):
# the key k = s + z B_h^T is normalised by n = sqrt(|k|^2 / d_h + eps), a quantity of the
# full key that neither branch knows alone; its reciprocal is computed when the token is
# appended and stored per head and position, and scoring multiplies it onto the summed
# score.  A fixed per-channel gain moves to the query side and is not the cache's concern.
# ---------------------------------------------------------------------------------------


def key_rms_reciprocal(s_row, z_rows, Bm, eps: float) -> np.ndarray:
    """1 / n_h for one token: s_row [d_h], z_rows [H, r], Bm [H, d_h, r] -> [H], float64,
    with n_h = sqrt(|s + z_h B_h^T|^2 / d_h + eps) (the full key, reconstructed)."""
    s_row = np.asarray(s_row, np.float64)
    K = s_row[None, :] + np.einsum("hr,hdr->hd", np.asarray(z_rows, np.float64),
                                   np.asarray(Bm, np.float64))
    d_h = s_row.shape[0]
    return 1.0 / np.sqrt(np.sum(K * K, axis=1) / d_h + eps)


def key_norms_reference(pool, L: Layout, B_K, eps: float, row_req, row_pos, page_table):
    """Expected pool after the key-norm step of an append: for every appended row and head,
    the reciprocal of the joint denominator of the key as stored (the row's S_K and R_K[h]
    read back from the pool), rounded to nearest even in the cache dtype and written at
    N[h][slot] of the row's page; every other byte keeps its value."""
    assert L.key_norm
    out = np.array(pool, dtype=np.uint8, copy=True).reshape(-1)
    elems = out.view(storage_dtype(L))
    pe = page_elems(L)
    table = np.asarray(page_table, np.int64)
    for req, pos in zip(np.asarray(row_req, np.int64), np.asarray(row_pos, np.int64)):
        page = table[req, pos // L.page_size]
        t = pos % L.page_size
        pg, sl = np.array([page]), np.array([t])
        src = np.asarray(pool, dtype=np.uint8).reshape(-1)
        # the stored rows of this position, read back through the page layout
        s_row = _read_block(src, L, pg, sl, "SK", 0, L.head_dim)[0]
        z = np.stack([_read_block(src, L, pg, sl, "RK", h, L.rank)[0]
                      for h in range(L.num_heads)])
        inv = key_rms_reciprocal(s_row, z, B_K, eps)
        for h in range(L.num_heads):
            elems[page * pe + section_base(L, "N", h) + t] = encode_elems(
                inv[h:h + 1], L.dtype).view(storage_dtype(L))[0]
    return out


# ---------------------------------------------------------------------------------------
# Plain attention over reconstructed keys / values (LRKV notes §2 and eq 2-5)
# ---------------------------------------------------------------------------------------


def reconstruct(S: np.ndarray, R: np.ndarray, Bm: np.ndarray) -> np.ndarray:
    """Full per-head rows from the factored cache: S + R_h B_h^T (eq 2-5).

    S [T, d_h]; R [H, T, r]; Bm [H, d_h, r]  ->  [H, T, d_h].
    """
    S = np.asarray(S, np.float64)
    R = np.asarray(R, np.float64)
    Bm = np.asarray(Bm, np.float64)
    return S[None, :, :] + np.matmul(R, np.transpose(Bm, (0, 2, 1)))


def softmax_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Textbook single-query attention: a = softmax(K q * scale), o = a V (§2).

    K, V hold only the visible rows.  With no visible row the result is zero.
    """
    if K.shape[0] == 0:
        return np.zeros(V.shape[1])
    s = (K @ q) * scale
    e = np.exp(s - s.max())  # subtracting the max changes nothing in exact arithmetic
    a = e / e.sum()
    return a @ V


def visible_count(seq_len: int, q_len: int, i: int) -> int:
    """Query row i of a request holding seq_len tokens sits at position seq_len - q_len + i
    and sees positions 0..that position (causal mask of §2)."""
    return max(0, min(seq_len, seq_len - q_len + i + 1))


def decode_reference(L: Layout, q, B_K, B_V, pool, page_table, seq_lens, sample=None):
    """Expected output of the LRKV decode call, by the plain definition.

    q [B, q_len, H, d_h]; B_K, B_V [H, d_h, r]; page_table [B, max_pages]; seq_lens [B].
    Returns float64 out [B, q_len, H, d_h].  With `sample` (an iterable of (b, i, h)), only
    those entries are computed; the rest of the returned array is NaN.
    """
    q = np.asarray(q, np.float64)
    Bn, q_len, H, dh = q.shape
    out = np.full((Bn, q_len, H, dh), np.nan)
    want = {}
    if sample is None:
        for b in range(Bn):
            want[b] = {(i, h) for i in range(q_len) for h in range(H)}
    else:
        for b, i, h in sample:
            want.setdefault(int(b), set()).add((int(i), int(h)))
    scale = 1.0 / math.sqrt(dh)
    BK = np.asarray(B_K, np.float64)
    BV = np.asarray(B_V, np.float64)
    for b, items in sorted(want.items()):
        T = int(seq_lens[b])
        shared = [gather_shared(pool, L, page_table[b], T, g) for g in range(L.groups)]
        for h in sorted({h for _, h in items}):
            SK, SV = shared[L.group_of(h)]  # the shared block of the head's group
            RK, RV = gather_private(pool, L, page_table[b], T, h)
            K = reconstruct(SK, RK[None], BK[h:h + 1])[0]
            if L.key_norm:  # normalised key: the full key times its stored reciprocal
                K = K * gather_norms(pool, L, page_table[b], T, h)[:, None]
            V = reconstruct(SV, RV[None], BV[h:h + 1])[0]
            for i, hh in sorted(items):
                if hh != h:
                    continue
                n = visible_count(T, q_len, i)
                out[b, i, h] = softmax_attention(q[b, i, h], K[:n], V[:n], scale)
    return out


def decode_algorithm2(L: Layout, q, B_K, B_V, pool, page_table, seq_lens):
    """Second coding, used only to check `decode_reference`: Algorithm 2 of §3, per head.

    p = q B_K[h] once; score_j = (q.S_K[j] + p.R_K[h, j]) / sqrt(d_h); one softmax over the
    visible rows; a.S_V + (a.R_V[h]) B_V[h]^T.
    """
    q = np.asarray(q, np.float64)
    Bn, q_len, H, dh = q.shape
    BK = np.asarray(B_K, np.float64)
    BV = np.asarray(B_V, np.float64)
    out = np.zeros((Bn, q_len, H, dh))
    for b in range(Bn):
        T = int(seq_lens[b])
        rows = gather_request(pool, L, page_table[b], T)
        for i in range(q_len):
            n = visible_count(T, q_len, i)
            if n == 0:
                continue
            for h in range(H):
                qh = q[b, i, h]
                SKh = rows["SK"] if L.groups == 1 else rows["SK"][L.group_of(h)]
                SVh = rows["SV"] if L.groups == 1 else rows["SV"][L.group_of(h)]
                p = qh @ BK[h]  # private query, formed once for the whole history
                shared = SKh[:n] @ qh
                private = rows["RK"][h, :n] @ p
                s = (shared + private) / math.sqrt(dh)  # one score per position, then softmax
                if L.key_norm:  # the stored reciprocal multiplies the summed score
                    s = s * gather_norms(pool, L, page_table[b], T, h)[:n]
                w = np.exp(s - s.max())
                a = w / w.sum()
                red_shared = a @ SVh[:n]
                red_private = a @ rows["RV"][h, :n]  # same weights as the shared branch
                out[b, i, h] = red_shared + red_private @ BV[h].T  # expand once
    return out


def full_projection_kv(X, W_S, U, Bm):
    """Per-head rows straight from eq 2: X (W_S + U_h B_h^T), never forming S or R.

    X [n, d]; W_S [d, d_h]; U [d, H, r]; Bm [H, d_h, r]  ->  [H, n, d_h].
    """
    X = np.asarray(X, np.float64)
    W_S = np.asarray(W_S, np.float64)
    U = np.asarray(U, np.float64)
    Bm = np.asarray(Bm, np.float64)
    H = U.shape[1]
    return np.stack([X @ (W_S + U[:, h, :] @ Bm[h].T) for h in range(H)])


# ---------------------------------------------------------------------------------------
# Rotary position encoding over the factored cache (LRKV notes §8, "can RoPE's rotation pass
# through the low-rank basis").  The rotation D_j of position j acts on the row vector of a
# key: feature pairs (2m, 2m+1) turn by the angle whose cosine and sine are the table's
# entry (j, m):  (x_2m, x_2m+1) D = (x_2m c - x_2m+1 s,  x_2m s + x_2m+1 c).  The key at
# position j is the reconstructed key turned by D_j, k_j = (s_j + z_j B_h^T) D_j; the query
# comes already turned at its own position (q~).  The cache holds the unrotated rows.
# ---------------------------------------------------------------------------------------


def rotate_rows(X: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Row vectors X [n, d] turned pair by pair: row i, pair m by (cos[i, m], sin[i, m])."""
    X = np.asarray(X, np.float64)
    c = np.asarray(cos, np.float64)
    s = np.asarray(sin, np.float64)
    out = np.empty_like(X)
    out[:, 0::2] = X[:, 0::2] * c - X[:, 1::2] * s
    out[:, 1::2] = X[:, 0::2] * s + X[:, 1::2] * c
    return out


def rope_keys(S, R, Bm, cos, sin) -> np.ndarray:
    """Full rotated keys of a history, by the plain definition: reconstruct every head's
    keys S + R_h B_h^T (eq 2-5), then turn row j by D_j.

    S [T, d_h]; R [H, T, r]; Bm [H, d_h, r]; cos, sin [T, d_h/2] (row j: position j)."""
    K = reconstruct(S, R, Bm)
    return np.stack([rotate_rows(K[h], cos, sin) for h in range(K.shape[0])])


def decode_reference_rope(L: Layout, q, B_K, B_V, pool, page_table, seq_lens, rope_cs,
                          sample=None):
    """Expected output of the rotary decode: textbook attention of the turned query q~ over
    the turned keys (S_K[j] + R_K[h, j] B_K[h]^T) D_j, values unrotated.

    rope_cs [rows, d_h/2, 2] holds (cos, sin) of position j at row j.  Other arguments as
    in `decode_reference`."""
    q = np.asarray(q, np.float64)
    Bn, q_len, H, dh = q.shape
    cs = np.asarray(rope_cs, np.float64)
    out = np.full((Bn, q_len, H, dh), np.nan)
    want = {}
    if sample is None:
        for b in range(Bn):
            want[b] = {(i, h) for i in range(q_len) for h in range(H)}
    else:
        for b, i, h in sample:
            want.setdefault(int(b), set()).add((int(i), int(h)))
    scale = 1.0 / math.sqrt(dh)
    BK = np.asarray(B_K, np.float64)
    BV = np.asarray(B_V, np.float64)
    for b, items in sorted(want.items()):
        T = int(seq_lens[b])
        shared = [gather_shared(pool, L, page_table[b], T, g) for g in range(L.groups)]
        for h in sorted({h for _, h in items}):
            SK, SV = shared[L.group_of(h)]
            RK, RV = gather_private(pool, L, page_table[b], T, h)
            K = rope_keys(SK, RK[None], BK[h:h + 1], cs[:T, :, 0], cs[:T, :, 1])[0]
            if L.key_norm:  # a turn keeps the key's length: the same stored reciprocal
                K = K * gather_norms(pool, L, page_table[b], T, h)[:, None]
            V = reconstruct(SV, RV[None], BV[h:h + 1])[0]
            for i, hh in sorted(items):
                if hh != h:
                    continue
                n = visible_count(T, q_len, i)
                out[b, i, h] = softmax_attention(q[b, i, h], K[:n], V[:n], scale)
    return out


def rope_scores_per_position(q_rot, S, R_h, B_h, cos, sin) -> np.ndarray:
    """Second coding of the rotary scores, used only to check `rope_keys`: the page's exact
    path with a private query formed anew for every key position,
        score_j = (q~ D_j^T) . s_j + ((q~ D_j^T) B_h) . z_j,
    D_j^T being the turn by the opposite angle.  Unscaled; S [T, d_h], R_h [T, r]."""
    q_rot = np.asarray(q_rot, np.float64)
    T = np.shape(S)[0]
    qj = rotate_rows(np.broadcast_to(q_rot, (T, q_rot.shape[0])), cos, -np.asarray(sin))
    p = qj @ np.asarray(B_h, np.float64)  # one private query per position
    return np.sum(qj * np.asarray(S, np.float64), axis=1) + np.sum(p * np.asarray(R_h, np.float64), axis=1)


# ---------------------------------------------------------------------------------------
# Blockwise online softmax and the merge of partial results (LRKV notes §3, the fused
# blockwise paragraph after Algorithm 2: running max, exp-sum and two value accumulators,
# all rescaled by one factor when the max moves; division by the exp-sum at the end)
# ---------------------------------------------------------------------------------------


def block_state(scores, SV, RV):
    """State of one block of positions: (m, l, acc_S, acc_R) with m the block max,
    l = sum exp(s - m), acc_S = sum exp(s - m) S_V[j], acc_R = sum exp(s - m) R_V[j]."""
    s = np.asarray(scores, np.float64)
    m = s.max()
    e = np.exp(s - m)
    return m, e.sum(), e @ np.asarray(SV, np.float64), e @ np.asarray(RV, np.float64)


def merge_states(states):
    """Combine block states: m* = max m_s, w_s = exp(m_s - m*), l = sum w_s l_s, and the
    same weights on both accumulators."""
    m_star = max(st[0] for st in states)
    w = [math.exp(st[0] - m_star) for st in states]
    l = sum(wi * st[1] for wi, st in zip(w, states))
    acc_s = sum(wi * st[2] for wi, st in zip(w, states))
    acc_r = sum(wi * st[3] for wi, st in zip(w, states))
    return m_star, l, acc_s, acc_r


def finish_state(state, BV_h):
    """o = (acc_S + acc_R B_V[h]^T) / l (the output steps of Algorithm 2, without W_O)."""
    _, l, acc_s, acc_r = state
    return (acc_s + acc_r @ np.asarray(BV_h, np.float64).T) / l


# ---------------------------------------------------------------------------------------
# Cache size and cost models (LRKV notes §4), exact rationals
# ---------------------------------------------------------------------------------------


def lrkv_cache_bytes(b: int, N: int, tokens: int, d_h: int, H: int, r: int) -> int:
    """eq 9: 2 b N (B T) (d_h + H r); `tokens` is B*T, or the sum of actual lengths."""
    return 2 * b * N * tokens * (d_h + H * r)


def mha_cache_bytes(b: int, N: int, tokens: int, d_h: int, H: int) -> int:
    """Dense multi-head baseline of §4: 2 b N (B T) H d_h."""
    return 2 * b * N * tokens * H * d_h


def cache_ratio(H: int, r: int, d_h: int) -> Fraction:
    """eq 9 ratio: 1/H + r/d_h."""
    return Fraction(1, H) + Fraction(r, d_h)


def rank_budget(d_h: int, c: Fraction, H: int) -> int:
    """Largest rank whose cache stays within fraction c of the dense one: floor(d_h (c - 1/H))."""
    return math.floor(Fraction(d_h) * (Fraction(c) - Fraction(1, H)))


def param_ratio(H: int, r: int, d_h: int, d: int) -> Fraction:
    """K/V projection parameters relative to dense: 1/H + (r/d_h)(1 + d_h/d)."""
    return Fraction(1, H) + Fraction(r, d_h) * (1 + Fraction(d_h, d))


def decode_arith_ratio(T: int, r: int, d_h: int) -> Fraction:
    """Decode multiply-adds relative to dense: (2 T d_h + 2 T r + 2 r d_h) / (2 T d_h)."""
    return Fraction(2 * T * d_h + 2 * T * r + 2 * r * d_h, 2 * T * d_h)


def grouped_cache_bytes(b: int, N: int, tokens: int, d_h: int, H: int, r: int, G: int) -> int:
    """One shared block per group of heads (LRKV notes §3): the shared features are stored
    G times, 2 b N (B T) (G d_h + H r)."""
    return 2 * b * N * tokens * (G * d_h + H * r)


def tp_replicated_ratio(P: int, H: int, r: int, d_h: int) -> Fraction:
    """Total payload relative to dense when the shared rows are copied to P devices: P/H + r/d_h."""
    return Fraction(P, H) + Fraction(r, d_h)


def roofline_time(bytes_moved: float, flops: float, beta: float, phi: float) -> float:
    """Lower bound of §4: time >= max(bytes / bandwidth, flops / compute rate)."""
    return max(bytes_moved / beta, flops / phi)
