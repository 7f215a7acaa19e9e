"""Python binding of liblrkv.so, the LRKV C-ABI library (include/lrkv.h).

The functions below carry the C entry points' names and argument order and do argument
marshalling only: a pointer argument may be a torch tensor (its data_ptr() is passed), an
int address or None; `stream` defaults to torch's current HIP stream.  Every step of the
computation runs in the library's HIP kernels.  A non-OK status raises LRKVError.

The library is built in-tree by ``python -m factored_rank_kv_amd.build``.  It is loaded on
the first call; without it every call raises ImportError.  There is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblrkv.so")

LRKV_F32 = 0
LRKV_BF16 = 1

LRKV_OK = 0
LRKV_ERR_INVALID_ARG = -1
LRKV_ERR_UNSUPPORTED = -2
LRKV_ERR_HIP = -3
LRKV_ERR_SCRATCH = -4
LRKV_ERR_NO_PAGES = -5


class lrkv_layout(ctypes.Structure):
    _fields_ = [
        ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("rank", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("key_norm", ctypes.c_int32),
        ("groups", ctypes.c_int32),
    ]

    def __repr__(self):
        return (f"lrkv_layout(H={self.num_heads}, d_h={self.head_dim}, r={self.rank}, "
                f"P={self.page_size}, dtype={'bf16' if self.dtype == LRKV_BF16 else 'f32'}, "
                f"key_norm={self.key_norm}, groups={self.groups})")


class lrkv_page_pool(ctypes.Structure):
    _fields_ = [
        ("num_pages", ctypes.c_int64),
        ("num_free", ctypes.c_int64),
        ("refcount", ctypes.POINTER(ctypes.c_int32)),
        ("free_stack", ctypes.POINTER(ctypes.c_int32)),
    ]


class LRKVError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {lrkv_status_string(status)} ({status})")


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing; build it with "
                          "`python -m factored_rank_kv_amd.build` (needs hipcc)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    LP = ctypes.POINTER(lrkv_layout)
    lib.lrkv_page_bytes.argtypes = [LP]
    lib.lrkv_page_bytes.restype = SZ
    lib.lrkv_append.argtypes = [LP, P, I32, I32, P, P, P, P, P, P, P, I32, P, I64, P]
    lib.lrkv_append.restype = ctypes.c_int
    lib.lrkv_decode_workspace_bytes.argtypes = [LP, I32, I32, I32, I32]
    lib.lrkv_decode_workspace_bytes.restype = SZ
    lib.lrkv_decode.argtypes = [LP, P, I32, I32, P, P, P, P, I32, P, I32, I32, P, P, SZ, P]
    lib.lrkv_decode.restype = ctypes.c_int
    lib.lrkv_decode_rope.argtypes = [LP, P, I32, I32, P, P, P, P, I32, P, I32, I32, P, I32, P,
                                     P, SZ, P]
    lib.lrkv_decode_rope.restype = ctypes.c_int
    lib.lrkv_decode_rope_workspace_bytes.argtypes = [LP, I32, I32, I32, I32]
    lib.lrkv_decode_rope_workspace_bytes.restype = SZ
    PP = ctypes.POINTER(lrkv_page_pool)
    lib.lrkv_pages_init.argtypes = [PP, P, P, I64]
    lib.lrkv_pages_alloc.argtypes = [PP, I32, P]
    lib.lrkv_pages_retain.argtypes = [PP, P, I32]
    lib.lrkv_pages_release.argtypes = [PP, P, I32]
    lib.lrkv_fork_prefix.argtypes = [LP, PP, P, I32, P, I32, P, P]
    lib.lrkv_copy_pages.argtypes = [LP, P, P, P, I32, P]
    for fn in ("lrkv_pages_init", "lrkv_pages_alloc", "lrkv_pages_retain", "lrkv_pages_release",
               "lrkv_fork_prefix", "lrkv_copy_pages"):
        getattr(lib, fn).restype = ctypes.c_int
    lib.lrkv_key_norms.argtypes = [LP, P, ctypes.c_float, P, P, I32, P, I32, P, I64, P]
    lib.lrkv_key_norms.restype = ctypes.c_int
    lib.lrkv_decode_noalloc.argtypes = [LP, P, I32, I32, P, P, P, P, I32, P, I32, I32, P, P]
    lib.lrkv_decode_noalloc.restype = ctypes.c_int
    lib.lrkv_check_indices.argtypes = [LP, P, I32, I32, P, I32, P, P, I32, I64, P, P]
    lib.lrkv_check_indices.restype = ctypes.c_int
    lib.lrkv_read_probe.argtypes = [P, ctypes.c_uint64, I32, P, P]
    lib.lrkv_read_probe.restype = ctypes.c_int
    lib.lrkv_status_string.argtypes = [ctypes.c_int]
    lib.lrkv_status_string.restype = ctypes.c_char_p
    lib.lrkv_private_queries_bytes.argtypes = [LP, I32, I32]
    lib.lrkv_private_queries_bytes.restype = SZ
    lib.lrkv_private_queries.argtypes = [LP, P, I32, I32, P, P, SZ, P]
    lib.lrkv_private_queries.restype = ctypes.c_int
    lib.lrkv_decode_pq.argtypes = [LP, P, P, SZ, I32, I32, P, P, P, I32, P, I32, I32, P, P, SZ, P]
    lib.lrkv_decode_pq.restype = ctypes.c_int
    lib.lrkv_append_pq.argtypes = [LP, P, I32, I32, P, P, P, P, P, P, P, I32, P, I64, P, I32, I32,
                                   P, P, SZ, P]
    lib.lrkv_append_pq.restype = ctypes.c_int
    _lib = lib
    return lib


EXPORTS = ("lrkv_page_bytes", "lrkv_append", "lrkv_decode_workspace_bytes", "lrkv_decode",
           "lrkv_decode_noalloc", "lrkv_decode_rope", "lrkv_decode_rope_workspace_bytes",
           "lrkv_key_norms", "lrkv_pages_init", "lrkv_pages_alloc", "lrkv_pages_retain",
           "lrkv_pages_release", "lrkv_fork_prefix", "lrkv_copy_pages",
           "lrkv_check_indices", "lrkv_read_probe", "lrkv_status_string",
           "lrkv_private_queries_bytes", "lrkv_private_queries", "lrkv_decode_pq",
           "lrkv_append_pq")


def library():
    """The loaded ctypes library (loads it on first use)."""
    return _load()


def _ptr(x):
    """Address of a buffer argument: a device tensor's data_ptr(), an int address, or None.
    Host tensors and strided views are refused here: the kernels would read a host address
    as device memory, or a view's storage as if it were dense."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_cuda:
        raise ValueError("LRKV buffers live in device memory; got a host tensor")
    if not x.is_contiguous():
        raise ValueError("LRKV buffers are dense; got a non-contiguous tensor view")
    return x.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch

    if torch.cuda.is_available() and torch.cuda.is_initialized():
        return torch.cuda.current_stream().cuda_stream
    return None


def _layout(L):
    if isinstance(L, lrkv_layout):
        return ctypes.byref(L)
    return ctypes.byref(lrkv_layout(*L))


def lrkv_status_string(status: int) -> str:
    return _load().lrkv_status_string(int(status)).decode()


def lrkv_page_bytes(layout) -> int:
    return int(_load().lrkv_page_bytes(_layout(layout)))


def lrkv_decode_workspace_bytes(layout, batch, q_len, max_seq_len, chunk_tokens) -> int:
    return int(_load().lrkv_decode_workspace_bytes(_layout(layout), batch, q_len, max_seq_len,
                                                    chunk_tokens))


def lrkv_append(layout, X, n_rows, d, W_SK, W_SV, U_K, U_V, row_req, row_pos, page_table,
                max_pages_per_req, pool, num_pages, stream=None, check=True) -> int:
    st = _load().lrkv_append(_layout(layout), _ptr(X), n_rows, d, _ptr(W_SK), _ptr(W_SV),
                             _ptr(U_K), _ptr(U_V), _ptr(row_req), _ptr(row_pos),
                             _ptr(page_table), max_pages_per_req, _ptr(pool), num_pages,
                             _stream(stream))
    if check and st != LRKV_OK:
        raise LRKVError(st, "lrkv_append")
    return st


def lrkv_decode(layout, q, batch, q_len, B_K, B_V, pool, page_table, max_pages_per_req,
                seq_lens, max_seq_len, chunk_tokens, out, workspace, workspace_bytes,
                stream=None, check=True) -> int:
    st = _load().lrkv_decode(_layout(layout), _ptr(q), batch, q_len, _ptr(B_K), _ptr(B_V),
                             _ptr(pool), _ptr(page_table), max_pages_per_req, _ptr(seq_lens),
                             max_seq_len, chunk_tokens, _ptr(out), _ptr(workspace),
                             workspace_bytes, _stream(stream))
    if check and st != LRKV_OK:
        raise LRKVError(st, "lrkv_decode")
    return st


def _host_i32(a):
    """Address of a host numpy int32 array (the page allocator works on host memory)."""
    import numpy as np

    if a is None:
        return None
    if not (isinstance(a, np.ndarray) and a.dtype == np.int32 and a.flags.c_contiguous):
        raise ValueError("page bookkeeping arrays are contiguous host numpy int32 arrays")
    return a.ctypes.data


def lrkv_pages_init(pp: "lrkv_page_pool", refcount, free_stack, num_pages: int,
                    check=True) -> int:
    st = _load().lrkv_pages_init(ctypes.byref(pp), _host_i32(refcount), _host_i32(free_stack),
                                 num_pages)
    if check and st != LRKV_OK:
        raise LRKVError(st, "lrkv_pages_init")
    return st


class PagePool:
    """Caller-owned page bookkeeping (lrkv_page_pool over two host int32 arrays)."""

    def __init__(self, num_pages: int):
        import numpy as np

        self.refcount = np.zeros(num_pages, np.int32)
        self.free_stack = np.zeros(num_pages, np.int32)
        self.c = lrkv_page_pool()
        lrkv_pages_init(self.c, self.refcount, self.free_stack, num_pages)

    @property
    def num_free(self) -> int:
        return int(self.c.num_free)


def lrkv_pages_alloc(pool: PagePool, n: int, ids, check=True) -> int:
    st = _load().lrkv_pages_alloc(ctypes.byref(pool.c), n, _host_i32(ids))
    if check and st != LRKV_OK:
        raise LRKVError(st, "lrkv_pages_alloc")
    return st


def lrkv_pages_retain(pool: PagePool, ids, n: int, check=True) -> int:
    st = _load().lrkv_pages_retain(ctypes.byref(pool.c), _host_i32(ids), n)
    if check and st != LRKV_OK:
        raise LRKVError(st, "lrkv_pages_retain")
    return st


def lrkv_pages_release(pool: PagePool, ids, n: int, check=True) -> int:
    st = _load().lrkv_pages_release(ctypes.byref(pool.c), _host_i32(ids), n)
    if check and st != LRKV_OK:
        raise LRKVError(st, "lrkv_pages_release")
    return st


def lrkv_fork_prefix(layout, pool: PagePool, parent_row, prefix_len, child_row,
                     max_pages_per_req, dev_pool, stream=None, check=True) -> int:
    st = _load().lrkv_fork_prefix(_layout(layout), ctypes.byref(pool.c), _host_i32(parent_row),
                                  prefix_len, _host_i32(child_row), max_pages_per_req,
                                  _ptr(dev_pool), _stream(stream))
    if check and st != LRKV_OK:
        raise LRKVError(st, "lrkv_fork_prefix")
    return st


def lrkv_copy_pages(layout, dev_pool, src_ids, dst_ids, n, stream=None, check=True) -> int:
    st = _load().lrkv_copy_pages(_layout(layout), _ptr(dev_pool), _ptr(src_ids), _ptr(dst_ids),
                                 n, _stream(stream))
    if check and st != LRKV_OK:
        raise LRKVError(st, "lrkv_copy_pages")
    return st


def lrkv_key_norms(layout, B_K, eps, row_req, row_pos, n_rows, page_table, max_pages_per_req,
                   pool, num_pages, stream=None, check=True) -> int:
    st = _load().lrkv_key_norms(_layout(layout), _ptr(B_K), float(eps), _ptr(row_req),
                                _ptr(row_pos), n_rows, _ptr(page_table), max_pages_per_req,
                                _ptr(pool), num_pages, _stream(stream))
    if check and st != LRKV_OK:
        raise LRKVError(st, "lrkv_key_norms")
    return st


def lrkv_decode_rope_workspace_bytes(layout, batch, q_len, max_seq_len, chunk_tokens) -> int:
    return int(_load().lrkv_decode_rope_workspace_bytes(_layout(layout), batch, q_len,
                                                         max_seq_len, chunk_tokens))


def lrkv_decode_rope(layout, q, batch, q_len, B_K, B_V, pool, page_table, max_pages_per_req,
                     seq_lens, max_seq_len, chunk_tokens, rope_cs, rope_rows, out, workspace,
                     workspace_bytes, stream=None, check=True) -> int:
    st = _load().lrkv_decode_rope(_layout(layout), _ptr(q), batch, q_len, _ptr(B_K), _ptr(B_V),
                                  _ptr(pool), _ptr(page_table), max_pages_per_req,
                                  _ptr(seq_lens), max_seq_len, chunk_tokens, _ptr(rope_cs),
                                  rope_rows, _ptr(out), _ptr(workspace), workspace_bytes,
                                  _stream(stream))
    if check and st != LRKV_OK:
        raise LRKVError(st, "lrkv_decode_rope")
    return st


def lrkv_private_queries_bytes(layout, batch, q_len) -> int:
    return _load().lrkv_private_queries_bytes(_layout(layout), batch, q_len)


def lrkv_private_queries(layout, q, batch, q_len, B_K, p, p_bytes, stream=None,
                         check=True) -> int:
    st = _load().lrkv_private_queries(_layout(layout), _ptr(q), batch, q_len, _ptr(B_K), _ptr(p),
                                      p_bytes, _stream(stream))
    if check and st != LRKV_OK:
        raise LRKVError(st, "lrkv_private_queries")
    return st


def lrkv_append_pq(layout, X, n_rows, d, W_SK, W_SV, U_K, U_V, row_req, row_pos, page_table,
                   max_pages_per_req, pool, num_pages, q, batch, q_len, B_K, p, p_bytes,
                   stream=None, check=True) -> int:
    st = _load().lrkv_append_pq(_layout(layout), _ptr(X), n_rows, d, _ptr(W_SK), _ptr(W_SV),
                                _ptr(U_K), _ptr(U_V), _ptr(row_req), _ptr(row_pos),
                                _ptr(page_table), max_pages_per_req, _ptr(pool), num_pages,
                                _ptr(q), batch, q_len, _ptr(B_K), _ptr(p), p_bytes,
                                _stream(stream))
    if check and st != LRKV_OK:
        raise LRKVError(st, "lrkv_append_pq")
    return st


def lrkv_decode_pq(layout, q, p, p_bytes, batch, q_len, B_V, pool, page_table,
                   max_pages_per_req, seq_lens, max_seq_len, chunk_tokens, out, workspace,
                   workspace_bytes, stream=None, check=True) -> int:
    st = _load().lrkv_decode_pq(_layout(layout), _ptr(q), _ptr(p), p_bytes, batch, q_len,
                                _ptr(B_V),
                                _ptr(pool), _ptr(page_table), max_pages_per_req, _ptr(seq_lens),
                                max_seq_len, chunk_tokens, _ptr(out), _ptr(workspace),
                                workspace_bytes, _stream(stream))
    if check and st != LRKV_OK:
        raise LRKVError(st, "lrkv_decode_pq")
    return st


def lrkv_decode_noalloc(layout, q, batch, q_len, B_K, B_V, pool, page_table, max_pages_per_req,
                        seq_lens, max_seq_len, chunk_tokens, out, stream=None,
                        check=True) -> int:
    st = _load().lrkv_decode_noalloc(_layout(layout), _ptr(q), batch, q_len, _ptr(B_K),
                                     _ptr(B_V), _ptr(pool), _ptr(page_table), max_pages_per_req,
                                     _ptr(seq_lens), max_seq_len, chunk_tokens, _ptr(out),
                                     _stream(stream))
    if check and st != LRKV_OK:
        raise LRKVError(st, "lrkv_decode_noalloc")
    return st


def lrkv_read_probe(buf, nbytes, workgroups, sink, stream=None, check=True) -> int:
    """Streaming read of nbytes of `buf` (measurement only; see include/lrkv.h)."""
    st = _load().lrkv_read_probe(_ptr(buf), nbytes, workgroups, _ptr(sink), _stream(stream))
    if check and st != LRKV_OK:
        raise LRKVError(st, "lrkv_read_probe")
    return st


def lrkv_check_indices(layout, page_table, batch, max_pages_per_req, seq_lens, max_seq_len,
                       row_req, row_pos, n_rows, num_pages, errors, stream=None,
                       check=True) -> int:
    st = _load().lrkv_check_indices(_layout(layout), _ptr(page_table), batch, max_pages_per_req,
                                    _ptr(seq_lens), max_seq_len, _ptr(row_req), _ptr(row_pos),
                                    n_rows, num_pages, _ptr(errors), _stream(stream))
    if check and st != LRKV_OK:
        raise LRKVError(st, "lrkv_check_indices")
    return st
