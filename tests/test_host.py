"""CPU-side checks of the C-ABI library: it loads, exports every entry point the header
declares, sizes pages and workspaces by the layout rules, and rejects bad arguments on the
host before any launch (no call here reaches a kernel)."""

import ctypes
import os
import re

import pytest

import factored_rank_kv_amd as F
import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lrkv.h")


@pytest.fixture(scope="session", autouse=True)
def built_library():
    if not os.path.exists(F.LIB_PATH):
        from factored_rank_kv_amd import build

        build.build()
    return F.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lrkv_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function(built_library):
    names = declared_functions()
    assert set(names) == set(F.EXPORTS)
    for name in names:
        assert hasattr(built_library, name), name
        assert callable(getattr(F, name)), name


C1 = F.lrkv_layout(16, 128, 56, 16, F.LRKV_BF16)
C0 = F.lrkv_layout(4, 16, 4, 16, F.LRKV_F32)
C3 = F.lrkv_layout(32, 128, 32, 16, F.LRKV_BF16)


@pytest.mark.parametrize("lay", [C0, C1, C3, F.lrkv_layout(18, 128, 56, 32, F.LRKV_BF16)])
def test_page_bytes_matches_layout_rule(lay):
    L = O.Layout(lay.num_heads, lay.head_dim, lay.rank, lay.page_size, lay.dtype)
    assert F.lrkv_page_bytes(lay) == O.page_bytes(L)


def test_page_bytes_rejects_invalid_layouts():
    assert F.lrkv_page_bytes(F.lrkv_layout(16, 128, 56, 12, F.LRKV_BF16)) == 0  # P not 2^k
    assert F.lrkv_page_bytes(F.lrkv_layout(16, 128, 50, 16, F.LRKV_BF16)) == 0  # r % 8
    assert F.lrkv_page_bytes(F.lrkv_layout(16, 130, 56, 16, F.LRKV_BF16)) == 0
    assert F.lrkv_page_bytes(F.lrkv_layout(16, 128, 56, 16, 7)) == 0
    assert F.lrkv_page_bytes(F.lrkv_layout(0, 128, 56, 16, F.LRKV_BF16)) == 0


def test_workspace_sizes():
    w = F.lrkv_decode_workspace_bytes(C1, 8, 1, 4096, 0)
    assert w > 0 and w % 256 == 0
    # explicit chunks: one partial tuple per (row, chunk, head)
    w16 = F.lrkv_decode_workspace_bytes(C1, 8, 1, 4096, 16)
    rows, H, r, dh = 8, 16, 56, 128
    rec = -(-(2 + dh + r) // 4) * 4  # partial records padded to 16 bytes
    part = -(-rows * 256 * H * rec * 4 // 256) * 256
    assert w16 == part
    # automatic chunks: B=8, T=4096 spreads over one wave of 256 groups (128-token chunks)
    assert F.lrkv_decode_workspace_bytes(C1, 8, 1, 4096, 0) == \
        F.lrkv_decode_workspace_bytes(C1, 8, 1, 4096, 128)
    # B=4, T=131072 also fills one wave: 2048-token chunks (the automatic maximum)
    assert F.lrkv_decode_workspace_bytes(C3, 4, 1, 131072, 0) == \
        F.lrkv_decode_workspace_bytes(C3, 4, 1, 131072, 2048)
    # B=32 padded to 32768 tokens would want 4096: capped at 2048 when asked for explicitly
    assert F.lrkv_decode_workspace_bytes(C1, 32, 1, 32768, 2048) == \
        -(-32 * 16 * H * rec * 4 // 256) * 256
    # automatic splits of 16 or more single-row requests are balanced: one record per
    # (workgroup, request it meets), at most groups + batch of them; groups = 256, or more
    # when the page ranges would outgrow 255 pages (B=32 x 2048 pages: 258)
    assert F.lrkv_decode_workspace_bytes(C1, 32, 1, 32768, 0) == \
        -(-(258 + 32) * H * rec * 4 // 256) * 256
    assert F.lrkv_decode_workspace_bytes(C1, 16, 1, 4096, 0) == \
        -(-(256 + 16) * H * rec * 4 // 256) * 256
    # several query rows keep the chunked split
    assert F.lrkv_decode_workspace_bytes(C1, 32, 2, 4096, 0) == \
        F.lrkv_decode_workspace_bytes(C1, 32, 2, 4096, 1024)
    assert F.lrkv_decode_workspace_bytes(C1, 8, 1, 4096, 4096 + 16) == 0  # chunk too long
    assert F.lrkv_decode_workspace_bytes(C1, 8, 1, 4096, 24) == 0  # not a multiple of P
    assert F.lrkv_decode_workspace_bytes(C1, 0, 1, 4096, 0) == 0


FAKE = 0x10000  # an aligned address that is never dereferenced: every call below is
                # rejected on the host before any launch


def decode_status(lay=C1, **over):
    args = dict(q=FAKE, batch=2, q_len=1, B_K=FAKE, B_V=FAKE, pool=FAKE, page_table=FAKE,
                max_pages_per_req=4, seq_lens=FAKE, max_seq_len=64, chunk_tokens=0, out=FAKE,
                workspace=FAKE, workspace_bytes=1 << 30)
    args.update(over)
    return F.lrkv_decode(lay, check=False, stream=0, **args)


def test_decode_rejects_bad_arguments_before_launch():
    bad = F.LRKV_ERR_INVALID_ARG
    assert decode_status(q=None) == bad
    assert decode_status(out=None) == bad
    assert decode_status(workspace=None) == bad
    assert decode_status(q=FAKE + 8) == bad  # misaligned
    assert decode_status(workspace=FAKE + 16) == bad  # workspace needs 256-byte alignment
    assert decode_status(batch=0) == bad
    assert decode_status(q_len=0) == bad
    assert decode_status(chunk_tokens=24) == bad
    assert decode_status(max_seq_len=65) == bad  # more than max_pages * P
    assert decode_status(workspace_bytes=16) == bad
    assert decode_status(F.lrkv_layout(16, 128, 56, 12, F.LRKV_BF16)) == bad
    unsupported = F.LRKV_ERR_UNSUPPORTED
    assert decode_status(F.lrkv_layout(8, 128, 56, 16, F.LRKV_BF16)) == unsupported
    assert decode_status(F.lrkv_layout(16, 128, 56, 32, F.LRKV_BF16)) == unsupported
    assert decode_status(F.lrkv_layout(16, 128, 56, 16, F.LRKV_F32)) == unsupported


def test_decode_noalloc_rejects_before_any_device_call():
    """Argument errors and calls whose partials exceed the fixed 16 MiB scratch are refused
    on the host (no GPU here: a device call would fail with LRKV_ERR_HIP instead)."""
    def st(**over):
        args = dict(q=FAKE, batch=8, q_len=1, B_K=FAKE, B_V=FAKE, pool=FAKE, page_table=FAKE,
                    max_pages_per_req=256, seq_lens=FAKE, max_seq_len=4096, chunk_tokens=16,
                    out=FAKE)
        args.update(over)
        return F.lrkv_decode_noalloc(C1, check=False, stream=0, **args)

    # 8 requests x 256 chunks x 16 heads x 752 B = 24 MiB of partials
    assert F.lrkv_decode_workspace_bytes(C1, 8, 1, 4096, 16) > 16 << 20
    assert st() == F.LRKV_ERR_SCRATCH
    assert st(q=None) == F.LRKV_ERR_INVALID_ARG
    assert st(chunk_tokens=24) == F.LRKV_ERR_INVALID_ARG
    assert F.lrkv_status_string(F.LRKV_ERR_SCRATCH).startswith("LRKV_ERR_SCRATCH")


def test_decode_rope_rejects_bad_arguments_before_launch():
    def st(lay=C1, **over):
        args = dict(q=FAKE, batch=2, q_len=1, B_K=FAKE, B_V=FAKE, pool=FAKE, page_table=FAKE,
                    max_pages_per_req=4, seq_lens=FAKE, max_seq_len=64, chunk_tokens=0,
                    rope_cs=FAKE, rope_rows=64, out=FAKE, workspace=FAKE,
                    workspace_bytes=1 << 30)
        args.update(over)
        return F.lrkv_decode_rope(lay, check=False, stream=0, **args)

    bad = F.LRKV_ERR_INVALID_ARG
    assert st(rope_cs=None) == bad
    assert st(rope_cs=FAKE + 4) == bad
    assert st(rope_rows=63) == bad  # fewer table rows than positions
    assert st(workspace_bytes=256) == bad
    assert st(chunk_tokens=8) == bad
    assert st(C0) == F.LRKV_ERR_UNSUPPORTED  # bf16 variants only
    n = F.lrkv_decode_rope_workspace_bytes(C1, 8, 1, 4096, 0)
    # 16 chunks of 256 tokens x 8 requests x 16 heads x 188 floats
    assert n == 16 * 8 * 16 * 188 * 4
    assert F.lrkv_decode_rope_workspace_bytes(C1, 8, 1, 4096, 24) == 0


def test_key_norm_layouts_and_argument_checks():
    C1N = F.lrkv_layout(16, 128, 56, 16, F.LRKV_BF16, 1)
    L = O.Layout(16, 128, 56, 16, O.BF16, key_norm=True)
    # the rows and reciprocals (65,536 + 512 bytes), padded to a whole KiB
    assert F.lrkv_page_bytes(C1N) == O.page_bytes(L) == 66560
    assert F.lrkv_page_bytes(F.lrkv_layout(16, 128, 56, 16, F.LRKV_BF16, 2)) == 0

    def st(lay=C1N, **over):
        args = dict(B_K=FAKE, eps=1e-6, row_req=FAKE, row_pos=FAKE, n_rows=4, page_table=FAKE,
                    max_pages_per_req=4, pool=FAKE, num_pages=8)
        args.update(over)
        return F.lrkv_key_norms(lay, check=False, stream=0, **args)

    bad = F.LRKV_ERR_INVALID_ARG
    assert st(C1) == bad  # a layout without the norm section
    assert st(B_K=None) == bad
    assert st(eps=-1.0) == bad
    assert st(eps=float("nan")) == bad
    assert st(pool=FAKE + 8) == bad
    assert st(F.lrkv_layout(4, 16, 4, 16, F.LRKV_F32, 1)) == F.LRKV_ERR_UNSUPPORTED
    assert st(n_rows=0) == F.LRKV_OK


def append_status(lay=C1, **over):
    args = dict(X=FAKE, n_rows=4, d=2048, W_SK=FAKE, W_SV=FAKE, U_K=FAKE, U_V=FAKE,
                row_req=FAKE, row_pos=FAKE, page_table=FAKE, max_pages_per_req=4, pool=FAKE,
                num_pages=8)
    args.update(over)
    return F.lrkv_append(lay, check=False, stream=0, **args)


def test_append_rejects_bad_arguments_before_launch():
    bad = F.LRKV_ERR_INVALID_ARG
    assert append_status(X=None) == bad
    assert append_status(d=100) == bad
    assert append_status(n_rows=-1) == bad
    assert append_status(pool=FAKE + 4) == bad
    assert append_status(num_pages=0) == bad
    assert append_status(F.lrkv_layout(16, 64, 56, 16, F.LRKV_BF16)) == F.LRKV_ERR_UNSUPPORTED
    assert append_status(n_rows=0) == F.LRKV_OK  # nothing to do, nothing launched


def test_private_query_calls_reject_bad_arguments_before_launch():
    """lrkv_private_queries / lrkv_append_pq / lrkv_decode_pq: sizes follow the layout (a
    key-norm layout's are its plain twin's, a grouped layout's one block per group); decode
    calls of 64 or more query rows per request over a one-group bf16 layout without key norms
    (those take the multi-query kernel) are refused."""
    n1 = F.lrkv_private_queries_bytes(C1, 1, 1)
    assert n1 > 0 and n1 % 16 == 0
    assert F.lrkv_private_queries_bytes(C1, 8, 3) == 24 * n1
    assert F.lrkv_private_queries_bytes(C3, 2, 1) > 0
    assert F.lrkv_private_queries_bytes(C0, 2, 5) > 0
    C1N = F.lrkv_layout(16, 128, 56, 16, F.LRKV_BF16, 1)
    C3G = F.lrkv_layout(32, 128, 32, 16, F.LRKV_BF16, 0, 2)
    assert F.lrkv_private_queries_bytes(C1N, 1, 1) == n1
    n3 = F.lrkv_private_queries_bytes(C3, 1, 1)
    assert F.lrkv_private_queries_bytes(C3G, 1, 1) == n3  # 2 blocks of 16 heads
    assert F.lrkv_private_queries_bytes(C1, 0, 1) == 0

    def pq(lay=C1, **over):
        args = dict(q=FAKE, batch=2, q_len=1, B_K=FAKE, p=FAKE, p_bytes=1 << 30)
        args.update(over)
        return F.lrkv_private_queries(lay, check=False, stream=0, **args)

    bad = F.LRKV_ERR_INVALID_ARG
    assert pq(q=None) == bad
    assert pq(p=FAKE + 8) == bad
    assert pq(batch=0) == bad
    assert pq(p_bytes=2 * n1 - 16) == bad
    assert pq(C3G, p_bytes=2 * n3 - 16) == bad

    def dec(lay=C1, **over):
        args = dict(q=FAKE, p=FAKE, p_bytes=1 << 30, batch=2, q_len=1, B_V=FAKE, pool=FAKE,
                    page_table=FAKE, max_pages_per_req=4, seq_lens=FAKE, max_seq_len=64,
                    chunk_tokens=0, out=FAKE, workspace=FAKE, workspace_bytes=1 << 30)
        args.update(over)
        return F.lrkv_decode_pq(lay, check=False, stream=0, **args)

    assert dec(p=None) == bad
    assert dec(p=FAKE + 4) == bad
    assert dec(workspace=FAKE + 16) == bad
    assert dec(workspace_bytes=16) == bad
    assert dec(p_bytes=2 * n1 - 16) == bad  # smaller than lrkv_private_queries_bytes
    assert dec(C3G, p_bytes=2 * n3 - 16) == bad
    assert dec(chunk_tokens=24) == bad
    assert dec(C3G, q_len=64, max_seq_len=64, workspace_bytes=1) == bad  # accepted up to the size check
    assert dec(q_len=64, max_seq_len=64) == F.LRKV_ERR_UNSUPPORTED
    assert dec(C1N, q_len=64, max_seq_len=64, workspace_bytes=1) == bad  # accepted up to the size check

    def apq(lay=C1, **over):
        args = dict(X=FAKE, n_rows=8, d=2048, W_SK=FAKE, W_SV=FAKE, U_K=FAKE, U_V=FAKE,
                    row_req=FAKE, row_pos=FAKE, page_table=FAKE, max_pages_per_req=4, pool=FAKE,
                    num_pages=8, q=FAKE, batch=8, q_len=1, B_K=FAKE, p=FAKE, p_bytes=8 * n1)
        args.update(over)
        return F.lrkv_append_pq(lay, check=False, stream=0, **args)

    # a bad argument of either step stops the call before anything is launched
    assert apq(X=None) == bad
    assert apq(d=100) == bad
    assert apq(q=None) == bad
    assert apq(p_bytes=8 * n1 - 16) == bad
    assert apq(batch=0) == bad
    assert apq(C3G, p_bytes=8 * n3 - 16) == bad


def check_status(lay=C1, **over):
    args = dict(page_table=FAKE, batch=2, max_pages_per_req=4, seq_lens=FAKE, max_seq_len=64,
                row_req=FAKE, row_pos=FAKE, n_rows=3, num_pages=8, errors=FAKE)
    args.update(over)
    return F.lrkv_check_indices(lay, check=False, stream=0, **args)


def test_check_indices_rejects_bad_arguments_before_launch():
    bad = F.LRKV_ERR_INVALID_ARG
    assert check_status(page_table=None) == bad
    assert check_status(errors=None) == bad
    assert check_status(row_pos=None) == bad  # one of the row arrays without the other
    assert check_status(errors=FAKE + 2) == bad  # misaligned int32
    assert check_status(batch=0) == bad
    assert check_status(max_pages_per_req=0) == bad
    assert check_status(num_pages=0) == bad
    assert check_status(n_rows=-1) == bad
    assert check_status(max_seq_len=65) == bad  # more than max_pages * P
    assert check_status(max_seq_len=-1) == bad
    assert check_status(F.lrkv_layout(16, 128, 56, 12, F.LRKV_BF16)) == bad


def test_status_strings():
    for st in (F.LRKV_OK, F.LRKV_ERR_INVALID_ARG, F.LRKV_ERR_UNSUPPORTED, F.LRKV_ERR_HIP,
               F.LRKV_ERR_SCRATCH):
        assert F.lrkv_status_string(st).startswith("LRKV")
    with pytest.raises(F.LRKVError) as e:
        F.lrkv_decode(C1, None, 1, 1, FAKE, FAKE, FAKE, FAKE, 1, FAKE, 16, 0, FAKE, FAKE, 1 << 20,
                      stream=0)
    assert e.value.status == F.LRKV_ERR_INVALID_ARG


def test_header_is_plain_c():
    """The header compiles as C with no HIP or torch headers."""
    import shutil
    import subprocess
    import tempfile

    cc = shutil.which("gcc")
    if not cc:
        pytest.skip("no gcc")
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "t.c")
        with open(src, "w") as f:
            f.write('#include "lrkv.h"\nint main(void){lrkv_layout L={16,128,56,16,LRKV_BF16,0,1};'
                    'return (int)sizeof(L) - 28;}\n')
        r = subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER),
                            "-c", src, "-o", os.path.join(d, "t.o")], capture_output=True,
                           text=True)
        assert r.returncode == 0, r.stderr
    assert ctypes.sizeof(F.lrkv_layout) == 28


def test_binding_refuses_host_tensors():
    """A host tensor never reaches the library (its address would be read as device memory)."""
    import torch

    host = torch.zeros(64, dtype=torch.int32)
    with pytest.raises(ValueError):
        F.lrkv_check_indices(C1, host, 2, 4, None, 64, None, None, 0, 8, host, stream=0)
    with pytest.raises(ValueError):
        F.lrkv_decode(C1, host, 1, 1, FAKE, FAKE, FAKE, FAKE, 1, FAKE, 16, 0, FAKE, FAKE, 1 << 20,
                      stream=0)


def test_page_allocator_matches_reference_model():
    """Seeded random sequences of alloc / retain / release / fork (whole-page prefixes, no
    device copy) on the C allocator and on the oracle's reference model: the same status,
    ids, reference counts and free stack after every operation."""
    import numpy as np

    from oracle.page_pool import PagePoolModel

    g = np.random.default_rng(600)
    lay = F.lrkv_layout(16, 128, 56, 16, F.LRKV_BF16)
    for trial in range(20):
        n = int(g.integers(1, 40))
        pool, model = F.PagePool(n), PagePoolModel(n)
        held = []  # page lists of live "requests"
        for step in range(200):
            op = g.integers(0, 4)
            if op == 0:
                k = int(g.integers(0, 6))
                ids = np.zeros(max(k, 1), np.int32)
                st = F.lrkv_pages_alloc(pool, k, ids, check=False)
                mst, mids = model.alloc(k)
                assert st == mst and list(ids[:k] if st == 0 else []) == (mids if st == 0 else [])
                if st == 0 and k:
                    held.append(list(mids))
            elif op == 1 and held:
                ids = held[int(g.integers(0, len(held)))]
                if g.random() < 0.2:
                    ids = ids + [int(g.integers(-2, n + 2))]  # sometimes an invalid id
                a = np.array(ids, np.int32)
                st = F.lrkv_pages_retain(pool, a, len(ids), check=False)
                assert st == model.retain(ids)
                if st == 0:
                    held.append(list(ids))
            elif op == 2 and held:
                ids = held.pop(int(g.integers(0, len(held))))
                if g.random() < 0.2:
                    ids = ids + ids[:1]  # sometimes one listing too many
                a = np.array(ids, np.int32)
                st = F.lrkv_pages_release(pool, a, len(ids), check=False)
                assert st == model.release(ids)
                if st != 0:
                    held.append(ids[:-1])
            elif op == 3 and held:
                parent = held[int(g.integers(0, len(held)))]
                plen = 16 * int(g.integers(0, len(parent) + 1))  # whole pages: no copy
                row = np.array(parent + [0], np.int32)
                child = np.full(len(parent) + 1, -7, np.int32)
                st = F.lrkv_fork_prefix(lay, pool, row, plen, child, len(row), 16, check=False)
                mst, mchild, mcopy = model.fork(parent, plen, 16)
                assert st == mst and mcopy is None
                if st == 0:
                    assert list(child[:len(mchild)]) == mchild
                    if mchild:
                        held.append(mchild)
            assert pool.refcount.tolist() == model.ref
            assert pool.num_free == len(model.free)
            assert pool.free_stack[:pool.num_free].tolist() == model.free


def test_page_allocator_host_errors():
    import numpy as np

    pool = F.PagePool(3)
    ids = np.zeros(4, np.int32)
    assert F.lrkv_pages_alloc(pool, 4, ids, check=False) == F.LRKV_ERR_NO_PAGES
    assert pool.num_free == 3  # nothing taken
    assert F.lrkv_pages_alloc(pool, 2, ids) == 0 and ids[:2].tolist() == [0, 1]
    assert F.lrkv_pages_retain(pool, np.array([2], np.int32), 1, check=False) == \
        F.LRKV_ERR_INVALID_ARG  # a free page cannot gain a holder
    assert F.lrkv_pages_release(pool, np.array([0, 0], np.int32), 2, check=False) == \
        F.LRKV_ERR_INVALID_ARG
    assert pool.refcount.tolist() == [1, 1, 0]  # the failed release changed nothing
    with pytest.raises(ValueError):
        F.lrkv_pages_retain(pool, [0], 1)  # host numpy int32 arrays only
