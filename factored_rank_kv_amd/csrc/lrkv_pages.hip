// Page bookkeeping for shared-prefix reuse and reclamation (LRKV notes §3, the note after
// Algorithm 1: with paged allocation, the shared pages and the per-head private pages must
// keep the same token numbering and the same reclamation lifetime, or reusing a prefix or
// releasing a request can leave the two paths of one position pointing at different
// histories).  In this layout one page id holds every section of its tokens (S_K, S_V,
// R_K[h], R_V[h] and, if kept, the key-norm reciprocals), so sharing, copying and freeing a
// page moves all of them together by construction.
//
// The allocator is host code over caller-owned arrays (a reference count per page and a
// stack of free page ids); it keeps no state of its own.  The one device operation is the
// copy of whole pages, used when a forked request must write into a partially filled page
// it would otherwise share (copy on write).
#include "../../include/lrkv.h"
#include "lrkv_launch.h"

namespace lrkv {

namespace {

// One workgroup per page: 16-byte chunks of the source page to the destination page.
__global__ void __launch_bounds__(256)
copy_pages_kernel(uint8_t* __restrict__ pool, const int32_t* __restrict__ src,
                  const int32_t* __restrict__ dst, int n, long long page_bytes, int single_src,
                  int single_dst) {
  const int i = (int)blockIdx.x;
  if (i >= n) return;
  const long long s = src ? src[i] : single_src;
  const long long d = dst ? dst[i] : single_dst;
  const uint4* from = reinterpret_cast<const uint4*>(pool + s * page_bytes);
  uint4* to = reinterpret_cast<uint4*>(pool + d * page_bytes);
  for (long long c = threadIdx.x; c < page_bytes / 16; c += blockDim.x) to[c] = from[c];
}

}  // namespace

hipError_t launch_copy_pages(uint8_t* pool, const int32_t* src, const int32_t* dst, int n,
                             long long page_bytes, int single_src, int single_dst,
                             hipStream_t stream) {
  hipLaunchKernelGGL(copy_pages_kernel, dim3(n), dim3(256), 0, stream, pool, src, dst, n,
                     page_bytes, single_src, single_dst);
  return hipGetLastError();
}

}  // namespace lrkv

namespace {

bool pool_valid(const lrkv_page_pool* pp) {
  return pp && pp->refcount && pp->free_stack && pp->num_pages > 0 && pp->num_free >= 0 &&
         pp->num_free <= pp->num_pages;
}

bool id_ok(const lrkv_page_pool* pp, int32_t id) { return id >= 0 && id < pp->num_pages; }

}  // namespace

extern "C" {

int lrkv_pages_init(lrkv_page_pool* pp, int32_t* refcount, int32_t* free_stack,
                    int64_t num_pages) {
  if (!pp || !refcount || !free_stack || num_pages <= 0 || num_pages > 0x7fffffffLL)
    return LRKV_ERR_INVALID_ARG;
  pp->num_pages = num_pages;
  pp->refcount = refcount;
  pp->free_stack = free_stack;
  for (int64_t i = 0; i < num_pages; ++i) {
    refcount[i] = 0;
    free_stack[i] = (int32_t)(num_pages - 1 - i);  // top of the stack: page 0
  }
  pp->num_free = num_pages;
  return LRKV_OK;
}

int lrkv_pages_alloc(lrkv_page_pool* pp, int32_t n, int32_t* ids) {
  if (!pool_valid(pp) || n < 0 || (n > 0 && !ids)) return LRKV_ERR_INVALID_ARG;
  if (n > pp->num_free) return LRKV_ERR_NO_PAGES;  // nothing taken
  for (int32_t k = 0; k < n; ++k) {
    const int32_t id = pp->free_stack[--pp->num_free];
    pp->refcount[id] = 1;
    ids[k] = id;
  }
  return LRKV_OK;
}

int lrkv_pages_retain(lrkv_page_pool* pp, const int32_t* ids, int32_t n) {
  if (!pool_valid(pp) || n < 0 || (n > 0 && !ids)) return LRKV_ERR_INVALID_ARG;
  for (int32_t k = 0; k < n; ++k)  // every id must be in use; otherwise nothing changes
    if (!id_ok(pp, ids[k]) || pp->refcount[ids[k]] <= 0 || pp->refcount[ids[k]] == 0x7fffffff)
      return LRKV_ERR_INVALID_ARG;
  for (int32_t k = 0; k < n; ++k) ++pp->refcount[ids[k]];
  return LRKV_OK;
}

int lrkv_pages_release(lrkv_page_pool* pp, const int32_t* ids, int32_t n) {
  if (!pool_valid(pp) || n < 0 || (n > 0 && !ids)) return LRKV_ERR_INVALID_ARG;
  for (int32_t k = 0; k < n; ++k)
    if (!id_ok(pp, ids[k])) return LRKV_ERR_INVALID_ARG;
  // every id must hold at least as many references as it appears in the list: drop them
  // one by one and undo all of it at the first page that would go below zero
  for (int32_t k = 0; k < n; ++k) {
    if (pp->refcount[ids[k]] <= 0) {
      for (int32_t j = 0; j < k; ++j) ++pp->refcount[ids[j]];
      return LRKV_ERR_INVALID_ARG;
    }
    --pp->refcount[ids[k]];
  }
  // pages left without a reference go back on the free stack, in list order
  for (int32_t k = 0; k < n; ++k)
    if (pp->refcount[ids[k]] == 0) {
      pp->free_stack[pp->num_free++] = ids[k];
      pp->refcount[ids[k]] = -1;  // mark: pushed once even if listed twice
    }
  for (int32_t k = 0; k < n; ++k)
    if (pp->refcount[ids[k]] == -1) pp->refcount[ids[k]] = 0;
  return LRKV_OK;
}

int lrkv_fork_prefix(const lrkv_layout* L, lrkv_page_pool* pp, const int32_t* parent_row,
                     int32_t prefix_len, int32_t* child_row, int32_t max_pages_per_req,
                     void* pool, void* stream) {
  const size_t page_bytes = lrkv_page_bytes(L);
  if (!page_bytes || !pool_valid(pp) || !parent_row || !child_row || prefix_len < 0 ||
      max_pages_per_req <= 0 || !pool || (reinterpret_cast<uintptr_t>(pool) & 15u))
    return LRKV_ERR_INVALID_ARG;
  const int32_t P = L->page_size;
  const int32_t full = prefix_len / P;
  const int32_t part = prefix_len % P ? 1 : 0;
  if (full + part > max_pages_per_req) return LRKV_ERR_INVALID_ARG;
  for (int32_t k = 0; k < full + part; ++k)
    if (!id_ok(pp, parent_row[k]) || pp->refcount[parent_row[k]] <= 0) return LRKV_ERR_INVALID_ARG;
  int32_t fresh = -1;
  if (part) {
    const int st = lrkv_pages_alloc(pp, 1, &fresh);
    if (st != LRKV_OK) return st;  // no page free: nothing changed
  }
  const int st = lrkv_pages_retain(pp, parent_row, full);  // checked above: cannot fail
  if (st != LRKV_OK) return st;
  for (int32_t k = 0; k < full; ++k) child_row[k] = parent_row[k];
  if (part) {
    child_row[full] = fresh;
    const hipError_t e = lrkv::launch_copy_pages(static_cast<uint8_t*>(pool), nullptr, nullptr, 1,
                                                 (long long)page_bytes, parent_row[full], fresh,
                                                 static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return LRKV_ERR_HIP;
  }
  return LRKV_OK;
}

int lrkv_copy_pages(const lrkv_layout* L, void* pool, const int32_t* src_ids,
                    const int32_t* dst_ids, int32_t n, void* stream) {
  const size_t page_bytes = lrkv_page_bytes(L);
  if (!page_bytes || !pool || !src_ids || !dst_ids || n < 0 || n > 0x7fffffff ||
      (reinterpret_cast<uintptr_t>(pool) & 15u) || (reinterpret_cast<uintptr_t>(src_ids) & 3u) ||
      (reinterpret_cast<uintptr_t>(dst_ids) & 3u))
    return LRKV_ERR_INVALID_ARG;
  if (n == 0) return LRKV_OK;
  const hipError_t e = lrkv::launch_copy_pages(static_cast<uint8_t*>(pool), src_ids, dst_ids, n,
                                               (long long)page_bytes, 0, 0,
                                               static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LRKV_OK : LRKV_ERR_HIP;
}

}  // extern "C"
