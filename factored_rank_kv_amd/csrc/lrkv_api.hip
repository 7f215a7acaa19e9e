// C-ABI entry points of the LRKV library (declared and documented in include/lrkv.h):
// host-side argument checks, shape dispatch, workspace sizing, launches on the caller's
// stream.  Nothing here allocates, frees or synchronizes.
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "../../include/lrkv.h"
#include "lrkv_launch.h"

// Fixed scratch of lrkv_decode_noalloc: one array per GPU, in the library's device code, held
// until the process ends.  On the host, `scratch` names a host-side stand-in, not device
// memory: its device address on a GPU is found once per device by hipGetSymbolAddress (with
// that device current) and only that address is ever passed to a kernel or copy.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

using namespace lrkv;

enum Variant { V_NONE = -1, V_C0 = 0, V_C1 = 1, V_C3 = 2, V_C1N = 3, V_C3N = 4, V_C3G2 = 5 };

// shared blocks of a layout (0 and 1 both mean one block for all heads)
int groups_of(const lrkv_layout* L) { return L->groups > 1 ? L->groups : 1; }

// The split kernel holds one chunk's page ids in LDS (256 pages of 16 tokens).
constexpr int kMaxChunkTokens = 256 * 16;

bool layout_valid(const lrkv_layout* L) {
  if (!L) return false;
  if (L->dtype != LRKV_F32 && L->dtype != LRKV_BF16) return false;
  if (L->num_heads <= 0 || L->head_dim <= 0 || L->rank <= 0) return false;
  if (L->page_size < 16 || (L->page_size & (L->page_size - 1))) return false;
  const int chunk = L->dtype == LRKV_BF16 ? 8 : 4;
  if (L->head_dim % chunk || L->rank % chunk) return false;
  if (L->key_norm != 0 && L->key_norm != 1) return false;
  if (L->groups < 0 || L->num_heads % groups_of(L)) return false;
  // the norm section (H x P elements) keeps pages whole 16-byte units
  if (L->key_norm && ((long long)L->num_heads * L->page_size * (L->dtype == LRKV_BF16 ? 2 : 4)) % 16)
    return false;
  return true;
}

Variant find_variant(const lrkv_layout* L) {
  if (L->page_size != kPage) return V_NONE;
  const int H = L->num_heads, dh = L->head_dim, r = L->rank;
  const bool nk = L->key_norm != 0;
  const int G = groups_of(L);
  if (G == 2 && !nk && L->dtype == LRKV_BF16 && H == 32 && dh == 128 && r == 32) return V_C3G2;
  if (G != 1) return V_NONE;
  if (L->dtype == LRKV_F32 && H == 4 && dh == 16 && r == 4 && !nk) return V_C0;
  if (L->dtype == LRKV_BF16 && H == 16 && dh == 128 && r == 56) return nk ? V_C1N : V_C1;
  if (L->dtype == LRKV_BF16 && H == 32 && dh == 128 && r == 32) return nk ? V_C3N : V_C3;
  return V_NONE;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Tokens per chunk of the split: the caller's value, or, for 0, a size from the batch's
// padded work (batch x q_len x max_seq_len tokens).  A split workgroup fills one compute unit
// (512 threads at up to 256 VGPRs), so one dispatch wave is 256 groups: the work is spread
// over that many chunks (measured best for equal lengths: B=8 x 4096 in 128-token chunks,
// B=4 x 131072 in 2048-token chunks, 84 % of 8 TB/s), at least 4 pages and at most
// kAutoChunkTokens long.  A grouped layout's split runs its G groups side by side, so its
// wave holds 256 / G chunks per group.  The host does not see the lengths (they stay on the device), so a
// ragged batch is sized by its longest request; such a batch does better with several
// waves of shorter chunks (B=32, lengths 512..32768: 768-token chunks, 405-420 µs), which
// a caller who knows the lengths can ask for.
constexpr long long kAutoChunkTokens = 2048;

int pick_chunk(const lrkv_layout* L, int batch, int q_len, int max_seq_len, int chunk_tokens) {
  if (chunk_tokens > 0) return chunk_tokens;
  const int P = L->page_size;
  const long long work = (long long)batch * q_len * (long long)max_seq_len;
  const long long one_wave = 256 / groups_of(L);
  long long c = (work + one_wave - 1) / one_wave;
  c = (c + P - 1) / P * P;
  if (c < 4LL * P) c = 4LL * P;
  if (c > kAutoChunkTokens) c = kAutoChunkTokens;
  const long long cap = ((long long)max_seq_len + P - 1) / P * P;
  if (c > cap && cap > 0) c = cap;
  if (c < P) c = P;
  return (int)c;
}

// Automatic splits of a batch of at least this many single-row requests (and at most
// kBalancedMaxBatch) take the balanced split: equal page ranges per workgroup whatever the
// lengths (B=32, lengths 512..32768: 310-340 µs against 405-420 µs for the best chunk
// size).  Smaller batches keep the chunked split, whose shorter start (no length scan)
// suits them.
constexpr int kBalancedMinBatch = 16;
constexpr int kBalancedGroups = 256;     // one wave of split workgroups

struct DecodeSizes {
  int chunk;
  int n_split;
  int groups;
  size_t p_bytes;
  size_t part_bytes;
  size_t total;
};

DecodeSizes decode_sizes(const lrkv_layout* L, int batch, int q_len, int max_seq_len,
                         int chunk_tokens) {
  DecodeSizes z{};
  if (L->dtype == LRKV_BF16 && !L->key_norm && groups_of(L) == 1 && q_len >= kPrefillMinRows) {
    // multi-query kernel: no split, no workspace (one 256-byte block keeps the pointer
    // contract uniform)
    z.chunk = chunk_tokens > 0 ? chunk_tokens : L->page_size;
    z.n_split = 1;
    z.total = 256;
    return z;
  }
  const size_t H = L->num_heads, r = L->rank, dh = L->head_dim;
  const size_t rec = (2 + dh + r + 3) / 4 * 4;  // padded partial record, floats
  if (q_len == 1 && chunk_tokens == 0 && batch >= kBalancedMinBatch &&
      batch <= kBalancedMaxBatch) {
    // every range fits the page ids a workgroup holds (kMaxChunkPages - 1 pages and a part)
    const long long pages = (long long)batch * ((max_seq_len + L->page_size - 1) / L->page_size);
    long long g = (pages + (kMaxChunkTokens / L->page_size) - 2) / ((kMaxChunkTokens / L->page_size) - 1);
    if (g < kBalancedGroups / groups_of(L)) g = kBalancedGroups / groups_of(L);  // one wave
    z.groups = (int)g;
    z.chunk = 0;
    z.n_split = 0;
    z.p_bytes = 0;
    z.part_bytes = align_up(((size_t)z.groups + batch) * H * rec * sizeof(float), 256);
    z.total = z.part_bytes;
    return z;
  }
  z.chunk = pick_chunk(L, batch, q_len, max_seq_len, chunk_tokens);
  z.n_split = max_seq_len > 0 ? (max_seq_len + z.chunk - 1) / z.chunk : 1;
  const size_t rows = (size_t)batch * q_len;
  z.p_bytes = 0;  // private queries live in the split kernel's LDS
  z.part_bytes = align_up(rows * (size_t)z.n_split * H * rec * sizeof(float), 256);
  z.total = z.p_bytes + z.part_bytes;
  return z;
}

int hip_status(hipError_t e) { return e == hipSuccess ? LRKV_OK : LRKV_ERR_HIP; }

// Rotary decode: always the chunked split.  Its workgroups take kRopeHeadsPerWorkgroup heads
// each and two fit a compute unit, so for 0 the batch's padded work over
// kRopeWaveWorkgroups / (H / kRopeHeadsPerWorkgroup) chunks, 64 to 2048 tokens, else the
// caller's multiple of P.
DecodeSizes rope_sizes(const lrkv_layout* L, int batch, int q_len, int max_seq_len,
                       int chunk_tokens) {
  DecodeSizes z{};
  const int P = L->page_size;
  long long c = chunk_tokens;
  if (c == 0) {
    const long long groups = L->num_heads / kRopeHeadsPerWorkgroup > 0
                                 ? L->num_heads / kRopeHeadsPerWorkgroup : 1;
    const long long per_wave = kRopeWaveWorkgroups / groups > 0 ? kRopeWaveWorkgroups / groups : 1;
    const long long work = (long long)batch * q_len * (long long)max_seq_len;
    c = (work + per_wave - 1) / per_wave;
    c = (c + P - 1) / P * P;
    if (c < 4LL * P) c = 4LL * P;
    if (c > kAutoChunkTokens) c = kAutoChunkTokens;
    const long long cap = ((long long)max_seq_len + P - 1) / P * P;
    if (c > cap && cap > 0) c = cap;
    if (c < P) c = P;
  }
  z.chunk = (int)c;
  z.n_split = max_seq_len > 0 ? (max_seq_len + z.chunk - 1) / z.chunk : 1;
  const size_t rec = ((size_t)2 + L->head_dim + L->rank + 3) / 4 * 4;
  z.part_bytes = align_up((size_t)batch * q_len * (size_t)z.n_split * L->num_heads * rec *
                              sizeof(float), 256);
  z.total = z.part_bytes;
  return z;
}

// Host-side checks of a decode call (everything but the workspace); fills the split sizes.
int decode_check(const lrkv_layout* L, const void* q, int32_t batch, int32_t q_len,
                 const void* B_K, const void* B_V, const void* pool, const int32_t* page_table,
                 int32_t max_pages_per_req, const int32_t* seq_lens, int32_t max_seq_len,
                 int32_t chunk_tokens, void* out, DecodeSizes* z) {
  if (!layout_valid(L)) return LRKV_ERR_INVALID_ARG;
  if (batch <= 0 || q_len <= 0 || max_pages_per_req <= 0 || max_seq_len < 0)
    return LRKV_ERR_INVALID_ARG;
  if (batch > 65535 || q_len > 65535) return LRKV_ERR_INVALID_ARG;
  if ((long long)max_seq_len > (long long)max_pages_per_req * L->page_size)
    return LRKV_ERR_INVALID_ARG;
  if (chunk_tokens < 0 || chunk_tokens % L->page_size || chunk_tokens > kMaxChunkTokens)
    return LRKV_ERR_INVALID_ARG;
  if (!q || !B_K || !B_V || !pool || !page_table || !seq_lens || !out)
    return LRKV_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(B_K) || !aligned16(B_V) || !aligned16(pool) ||
      !aligned16(page_table) || !aligned16(seq_lens) || !aligned16(out))
    return LRKV_ERR_INVALID_ARG;
  if (find_variant(L) == V_NONE) return LRKV_ERR_UNSUPPORTED;
  *z = decode_sizes(L, batch, q_len, max_seq_len, chunk_tokens);
  if (z->n_split > 65535) return LRKV_ERR_INVALID_ARG;
  // one-dimensional grids of the split and merge kernels (rounded up to 8 blocks)
  if ((long long)batch * q_len * (z->n_split > L->num_heads ? z->n_split : L->num_heads) >
      0x7fffffffLL - 8)
    return LRKV_ERR_INVALID_ARG;
  return LRKV_OK;
}

// Launches of a checked decode call on `workspace` (at least z.total bytes, 256-aligned).
int decode_launch(const lrkv_layout* L, const void* q, int32_t batch, int32_t q_len,
                  const void* B_K, const void* B_V, const void* pool, const int32_t* page_table,
                  int32_t max_pages_per_req, const int32_t* seq_lens, void* out,
                  void* workspace, const DecodeSizes& z, void* stream,
                  const void* p_ext = nullptr) {
  DecodeArgs a{};
  a.p_ext = p_ext;
  a.q = q;
  a.batch = batch;
  a.q_len = q_len;
  a.B_K = B_K;
  a.B_V = B_V;
  a.pool = pool;
  a.page_table = page_table;
  a.max_pages = max_pages_per_req;
  a.seq_lens = seq_lens;
  a.n_split = z.n_split;
  a.chunk = z.chunk;
  a.groups = z.groups;
  a.out = out;
  a.part_ws = reinterpret_cast<float*>(static_cast<char*>(workspace) + z.p_bytes);
  a.stream = static_cast<hipStream_t>(stream);
  switch (find_variant(L)) {
    case V_C0: return hip_status(launch_decode<ShapeC0>(a));
    case V_C1: return hip_status(launch_decode<ShapeC1>(a));
    case V_C3: return hip_status(launch_decode<ShapeC3>(a));
    case V_C1N: return hip_status(launch_decode<ShapeC1N>(a));
    case V_C3N: return hip_status(launch_decode<ShapeC3N>(a));
    case V_C3G2: return hip_status(launch_decode_grouped<ShapeC3G, ShapeC3>(a, 2));
    default: return LRKV_ERR_UNSUPPORTED;
  }
}

// ---- fixed scratch of the no-allocation decode (the array is declared above the namespace)
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];  // device address of `scratch`, per device, once found

int scratch_address(hipStream_t stream, void** ws) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return LRKV_ERR_HIP;
  int dev = cur;
  if (stream) {
    hipDevice_t sd = 0;
    if (hipStreamGetDevice(stream, &sd) != hipSuccess) return LRKV_ERR_HIP;
    dev = (int)sd;
  }
  if (dev < 0 || dev >= kMaxDevices) return LRKV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return LRKV_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p) return LRKV_ERR_HIP;
    g_scratch_dev[dev] = p;
  }
  *ws = g_scratch_dev[dev];
  return LRKV_OK;
}

// private queries formed once per query row: every compiled layout (the key-norm section
// does not enter p, so a key-norm layout's block is its plain twin's; a grouped layout's row
// holds one block per group)
bool pq_variant(Variant v) {
  return v == V_C0 || v == V_C1 || v == V_C3 || v == V_C1N || v == V_C3N || v == V_C3G2;
}

size_t pq_row_bytes(Variant v) {
  switch (v) {
    case V_C0: return private_query_row_bytes<ShapeC0>();
    case V_C1: case V_C1N: return private_query_row_bytes<ShapeC1>();
    case V_C3: case V_C3N: return private_query_row_bytes<ShapeC3>();
    case V_C3G2: return 2 * private_query_row_bytes<ShapeC3G>();  // each group's block
    default: return 0;
  }
}

// lrkv_private_queries' argument checks (no launch)
int private_queries_check(const lrkv_layout* L, const void* q, int32_t batch, int32_t q_len,
                          const void* B_K, const void* p, size_t p_bytes) {
  if (!layout_valid(L)) return LRKV_ERR_INVALID_ARG;
  if (batch <= 0 || q_len <= 0 || batch > 65535 || q_len > 65535) return LRKV_ERR_INVALID_ARG;
  if (!q || !B_K || !p || !aligned16(q) || !aligned16(B_K) || !aligned16(p))
    return LRKV_ERR_INVALID_ARG;
  if (!pq_variant(find_variant(L))) return LRKV_ERR_UNSUPPORTED;
  if ((long long)batch * q_len > kMaxPrivateQueryRows) return LRKV_ERR_INVALID_ARG;
  if (p_bytes < (size_t)batch * (size_t)q_len * pq_row_bytes(find_variant(L)))
    return LRKV_ERR_INVALID_ARG;
  return LRKV_OK;
}

// lrkv_append's argument checks; fills *a on success (no launch)
int append_check(const lrkv_layout* L, const void* X, int32_t n_rows, int32_t d,
                 const void* W_SK, const void* W_SV, const void* U_K, const void* U_V,
                 const int32_t* row_req, const int32_t* row_pos, const int32_t* page_table,
                 int32_t max_pages_per_req, void* pool, int64_t num_pages, void* stream,
                 AppendArgs* a) {
  if (!layout_valid(L)) return LRKV_ERR_INVALID_ARG;
  if (n_rows < 0 || d <= 0 || d % 8 || max_pages_per_req <= 0 || num_pages <= 0)
    return LRKV_ERR_INVALID_ARG;
  if (n_rows > 65535 * 8) return LRKV_ERR_INVALID_ARG;
  if (!X || !W_SK || !W_SV || !U_K || !U_V || !row_req || !row_pos || !page_table || !pool)
    return LRKV_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(W_SK) || !aligned16(W_SV) || !aligned16(U_K) ||
      !aligned16(U_V) || !aligned16(row_req) || !aligned16(row_pos) || !aligned16(page_table) ||
      !aligned16(pool))
    return LRKV_ERR_INVALID_ARG;
  if (find_variant(L) == V_NONE) return LRKV_ERR_UNSUPPORTED;
  *a = AppendArgs{};
  a->X = X;
  a->n_rows = n_rows;
  a->d = d;
  a->W_SK = W_SK;
  a->W_SV = W_SV;
  a->U_K = U_K;
  a->U_V = U_V;
  a->row_req = row_req;
  a->row_pos = row_pos;
  a->page_table = page_table;
  a->max_pages = max_pages_per_req;
  a->pool = pool;
  a->stream = static_cast<hipStream_t>(stream);
  return LRKV_OK;
}

}  // namespace

extern "C" {

size_t lrkv_page_bytes(const lrkv_layout* L) {
  if (!layout_valid(L)) return 0;
  const size_t b = L->dtype == LRKV_BF16 ? 2 : 4;
  const size_t norm = L->key_norm ? (size_t)L->page_size * L->num_heads * b : 0;
  const size_t data = (size_t)L->page_size * 2 *
                          ((size_t)groups_of(L) * L->head_dim + (size_t)L->num_heads * L->rank) * b +
                      norm;
  return L->key_norm ? (data + 1023) / 1024 * 1024 : data;  // key-norm pages: whole KiB
}

const char* lrkv_status_string(int status) {
  switch (status) {
    case LRKV_OK: return "LRKV_OK";
    case LRKV_ERR_INVALID_ARG: return "LRKV_ERR_INVALID_ARG: invalid argument";
    case LRKV_ERR_UNSUPPORTED: return "LRKV_ERR_UNSUPPORTED: no kernel variant for this shape";
    case LRKV_ERR_HIP: return "LRKV_ERR_HIP: HIP runtime error at launch";
    case LRKV_ERR_NO_PAGES: return "LRKV_ERR_NO_PAGES: not enough free pages in the page pool";
    case LRKV_ERR_SCRATCH:
      return "LRKV_ERR_SCRATCH: the call needs more workspace than the 16 MiB fixed scratch of "
             "lrkv_decode_noalloc holds (use lrkv_decode with a caller workspace)";
    default: return "LRKV: unknown status";
  }
}

size_t lrkv_decode_workspace_bytes(const lrkv_layout* L, int32_t batch, int32_t q_len,
                                   int32_t max_seq_len, int32_t chunk_tokens) {
  if (!layout_valid(L) || batch <= 0 || q_len <= 0 || max_seq_len < 0 || chunk_tokens < 0)
    return 0;
  if (chunk_tokens % L->page_size || chunk_tokens > kMaxChunkTokens) return 0;
  return decode_sizes(L, batch, q_len, max_seq_len, chunk_tokens).total;
}

int lrkv_decode(const lrkv_layout* L, const void* q, int32_t batch, int32_t q_len,
                const void* B_K, const void* B_V, const void* pool, const int32_t* page_table,
                int32_t max_pages_per_req, const int32_t* seq_lens, int32_t max_seq_len,
                int32_t chunk_tokens, void* out, void* workspace, size_t workspace_bytes,
                void* stream) {
  DecodeSizes z{};
  const int st = decode_check(L, q, batch, q_len, B_K, B_V, pool, page_table, max_pages_per_req,
                              seq_lens, max_seq_len, chunk_tokens, out, &z);
  if (st != LRKV_OK) return st;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return LRKV_ERR_INVALID_ARG;
  if (workspace_bytes < z.total) return LRKV_ERR_INVALID_ARG;
  return decode_launch(L, q, batch, q_len, B_K, B_V, pool, page_table, max_pages_per_req,
                       seq_lens, out, workspace, z, stream);
}

// ---- private queries formed once per query row, and the decode that takes them ----------
size_t lrkv_private_queries_bytes(const lrkv_layout* L, int32_t batch, int32_t q_len) {
  if (!layout_valid(L) || batch <= 0 || q_len <= 0) return 0;
  const Variant v = find_variant(L);
  if (!pq_variant(v)) return 0;
  return (size_t)batch * (size_t)q_len * pq_row_bytes(v);
}

int lrkv_private_queries(const lrkv_layout* L, const void* q, int32_t batch, int32_t q_len,
                         const void* B_K, void* p, size_t p_bytes, void* stream) {
  const int st = private_queries_check(L, q, batch, q_len, B_K, p, p_bytes);
  if (st != LRKV_OK) return st;
  const int rows = batch * q_len;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (find_variant(L)) {
    case V_C0: return hip_status(launch_private_queries<ShapeC0>(q, B_K, rows, p, s));
    case V_C1: return hip_status(launch_private_queries<ShapeC1>(q, B_K, rows, p, s));
    case V_C3: return hip_status(launch_private_queries<ShapeC3>(q, B_K, rows, p, s));
    case V_C1N: return hip_status(launch_private_queries<ShapeC1>(q, B_K, rows, p, s));
    case V_C3N: return hip_status(launch_private_queries<ShapeC3>(q, B_K, rows, p, s));
    case V_C3G2: return hip_status(launch_private_queries<ShapeC3G>(q, B_K, rows, p, s, 2));
    default: return LRKV_ERR_UNSUPPORTED;
  }
}

int lrkv_append_pq(const lrkv_layout* L, const void* X, int32_t n_rows, int32_t d,
                   const void* W_SK, const void* W_SV, const void* U_K, const void* U_V,
                   const int32_t* row_req, const int32_t* row_pos, const int32_t* page_table,
                   int32_t max_pages_per_req, void* pool, int64_t num_pages, const void* q,
                   int32_t batch, int32_t q_len, const void* B_K, void* p, size_t p_bytes,
                   void* stream) {
  // every argument of both steps is checked before anything is launched
  int st = private_queries_check(L, q, batch, q_len, B_K, p, p_bytes);
  if (st != LRKV_OK) return st;
  AppendArgs a{};
  st = append_check(L, X, n_rows, d, W_SK, W_SV, U_K, U_V, row_req, row_pos, page_table,
                    max_pages_per_req, pool, num_pages, stream, &a);
  if (st != LRKV_OK) return st;
  const int rows = batch * q_len;
  const Variant v = find_variant(L);
  if (n_rows >= 1 && n_rows <= 8 && L->dtype == LRKV_BF16 && d >= 8) {  // one launch
    if (v == V_C1) return hip_status(launch_append_pq<ShapeC1>(a, q, B_K, rows, p));
    if (v == V_C3) return hip_status(launch_append_pq<ShapeC3>(a, q, B_K, rows, p));
    if (v == V_C1N) return hip_status(launch_append_pq<ShapeC1N>(a, q, B_K, rows, p));
    if (v == V_C3N) return hip_status(launch_append_pq<ShapeC3N>(a, q, B_K, rows, p));
  }
  st = lrkv_append(L, X, n_rows, d, W_SK, W_SV, U_K, U_V, row_req, row_pos, page_table,
                   max_pages_per_req, pool, num_pages, stream);
  if (st != LRKV_OK) return st;
  return lrkv_private_queries(L, q, batch, q_len, B_K, p, p_bytes, stream);
}

int lrkv_decode_pq(const lrkv_layout* L, const void* q, const void* p, size_t p_bytes,
                   int32_t batch, int32_t q_len, const void* B_V, const void* pool, const int32_t* page_table,
                   int32_t max_pages_per_req, const int32_t* seq_lens, int32_t max_seq_len,
                   int32_t chunk_tokens, void* out, void* workspace, size_t workspace_bytes,
                   void* stream) {
  DecodeSizes z{};
  // p takes the place of B_K in the common checks (non-null, 16-byte aligned)
  const int st = decode_check(L, q, batch, q_len, p, B_V, pool, page_table, max_pages_per_req,
                              seq_lens, max_seq_len, chunk_tokens, out, &z);
  if (st != LRKV_OK) return st;
  const Variant v = find_variant(L);
  if (!pq_variant(v)) return LRKV_ERR_UNSUPPORTED;
  if ((long long)batch * q_len > kMaxPrivateQueryRows) return LRKV_ERR_INVALID_ARG;
  if (p_bytes < (size_t)batch * (size_t)q_len * pq_row_bytes(v)) return LRKV_ERR_INVALID_ARG;
  // the multi-query kernel forms its own private queries: such calls go to lrkv_decode
  // (key-norm and grouped layouts take every query row through the split kernel, either way)
  if (L->dtype == LRKV_BF16 && !L->key_norm && groups_of(L) == 1 && q_len >= kPrefillMinRows)
    return LRKV_ERR_UNSUPPORTED;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return LRKV_ERR_INVALID_ARG;
  if (workspace_bytes < z.total) return LRKV_ERR_INVALID_ARG;
  return decode_launch(L, q, batch, q_len, nullptr, B_V, pool, page_table, max_pages_per_req,
                       seq_lens, out, workspace, z, stream, p);
}

size_t lrkv_decode_rope_workspace_bytes(const lrkv_layout* L, int32_t batch, int32_t q_len,
                                        int32_t max_seq_len, int32_t chunk_tokens) {
  if (!layout_valid(L) || batch <= 0 || q_len <= 0 || max_seq_len < 0 || chunk_tokens < 0)
    return 0;
  if (chunk_tokens % L->page_size || chunk_tokens > kMaxChunkTokens) return 0;
  return rope_sizes(L, batch, q_len, max_seq_len, chunk_tokens).total;
}

int lrkv_decode_rope(const lrkv_layout* L, const void* q, int32_t batch, int32_t q_len,
                     const void* B_K, const void* B_V, const void* pool,
                     const int32_t* page_table, int32_t max_pages_per_req,
                     const int32_t* seq_lens, int32_t max_seq_len, int32_t chunk_tokens,
                     const float* rope_cs, int32_t rope_rows, void* out, void* workspace,
                     size_t workspace_bytes, void* stream) {
  DecodeSizes z{};
  int st = decode_check(L, q, batch, q_len, B_K, B_V, pool, page_table, max_pages_per_req,
                        seq_lens, max_seq_len, chunk_tokens, out, &z);
  if (st != LRKV_OK) return st;
  if (!rope_cs || !aligned16(rope_cs) || rope_rows < max_seq_len || rope_rows <= 0)
    return LRKV_ERR_INVALID_ARG;
  const Variant v = find_variant(L);
  if (v == V_C0 || v == V_NONE || v == V_C3G2) return LRKV_ERR_UNSUPPORTED;  // bf16, one group
  z = rope_sizes(L, batch, q_len, max_seq_len, chunk_tokens);
  if (z.n_split > 65535) return LRKV_ERR_INVALID_ARG;
  if ((long long)batch * q_len * z.n_split * (L->num_heads / kRopeHeadsPerWorkgroup) >
      0x7fffffffLL - 8)
    return LRKV_ERR_INVALID_ARG;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return LRKV_ERR_INVALID_ARG;
  if (workspace_bytes < z.total) return LRKV_ERR_INVALID_ARG;
  DecodeArgs a{};
  a.q = q;
  a.batch = batch;
  a.q_len = q_len;
  a.B_K = B_K;
  a.B_V = B_V;
  a.pool = pool;
  a.page_table = page_table;
  a.max_pages = max_pages_per_req;
  a.seq_lens = seq_lens;
  a.n_split = z.n_split;
  a.chunk = z.chunk;
  a.groups = 0;
  a.out = out;
  a.part_ws = static_cast<float*>(workspace);
  a.stream = static_cast<hipStream_t>(stream);
  switch (v) {
    case V_C1: return hip_status(launch_decode_rope<ShapeC1>(a, rope_cs, rope_rows));
    case V_C3: return hip_status(launch_decode_rope<ShapeC3>(a, rope_cs, rope_rows));
    case V_C1N: return hip_status(launch_decode_rope<ShapeC1N>(a, rope_cs, rope_rows));
    case V_C3N: return hip_status(launch_decode_rope<ShapeC3N>(a, rope_cs, rope_rows));
    default: return LRKV_ERR_UNSUPPORTED;
  }
}

int lrkv_decode_noalloc(const lrkv_layout* L, const void* q, int32_t batch, int32_t q_len,
                        const void* B_K, const void* B_V, const void* pool,
                        const int32_t* page_table, int32_t max_pages_per_req,
                        const int32_t* seq_lens, int32_t max_seq_len, int32_t chunk_tokens,
                        void* out, void* stream) {
  DecodeSizes z{};
  const int st = decode_check(L, q, batch, q_len, B_K, B_V, pool, page_table, max_pages_per_req,
                              seq_lens, max_seq_len, chunk_tokens, out, &z);
  if (st != LRKV_OK) return st;
  if (z.total > kScratchBytes) return LRKV_ERR_SCRATCH;  // before any device call
  void* ws = nullptr;
  const int sst = scratch_address(static_cast<hipStream_t>(stream), &ws);
  if (sst != LRKV_OK) return sst;
  return decode_launch(L, q, batch, q_len, B_K, B_V, pool, page_table, max_pages_per_req,
                       seq_lens, out, ws, z, stream);
}

int lrkv_append(const lrkv_layout* L, const void* X, int32_t n_rows, int32_t d,
                const void* W_SK, const void* W_SV, const void* U_K, const void* U_V,
                const int32_t* row_req, const int32_t* row_pos, const int32_t* page_table,
                int32_t max_pages_per_req, void* pool, int64_t num_pages, void* stream) {
  AppendArgs a{};
  const int st = append_check(L, X, n_rows, d, W_SK, W_SV, U_K, U_V, row_req, row_pos,
                              page_table, max_pages_per_req, pool, num_pages, stream, &a);
  if (st != LRKV_OK) return st;
  if (n_rows == 0) return LRKV_OK;
  switch (find_variant(L)) {
    case V_C0: return hip_status(launch_append<ShapeC0>(a));
    case V_C1: return hip_status(launch_append<ShapeC1>(a));
    case V_C3: return hip_status(launch_append<ShapeC3>(a));
    case V_C1N: return hip_status(launch_append<ShapeC1N>(a));
    case V_C3N: return hip_status(launch_append<ShapeC3N>(a));
    case V_C3G2: {  // each group's block as a one-group page of its 16 heads
      for (int g = 0; g < 2; ++g) {
        AppendArgs b = a;
        const size_t wsh = (size_t)L->head_dim * d * 2, wpr = (size_t)16 * L->rank * d * 2;
        b.W_SK = static_cast<const uint8_t*>(W_SK) + g * wsh;
        b.W_SV = static_cast<const uint8_t*>(W_SV) + g * wsh;
        b.U_K = static_cast<const uint8_t*>(U_K) + g * wpr;
        b.U_V = static_cast<const uint8_t*>(U_V) + g * wpr;
        b.page_elems = 2 * (ShapeC3G::PAGE / 2);
        b.elem_off = (long long)g * (ShapeC3G::PAGE / 2);
        const int st = hip_status(launch_append<ShapeC3G>(b));
        if (st != LRKV_OK) return st;
      }
      return LRKV_OK;
    }
    default: return LRKV_ERR_UNSUPPORTED;
  }
}

int lrkv_key_norms(const lrkv_layout* L, const void* B_K, float eps, const int32_t* row_req,
                   const int32_t* row_pos, int32_t n_rows, const int32_t* page_table,
                   int32_t max_pages_per_req, void* pool, int64_t num_pages, void* stream) {
  if (!layout_valid(L) || !L->key_norm) return LRKV_ERR_INVALID_ARG;
  if (n_rows < 0 || max_pages_per_req <= 0 || num_pages <= 0) return LRKV_ERR_INVALID_ARG;
  if (!(eps >= 0.0f) || eps > 1e30f) return LRKV_ERR_INVALID_ARG;  // also refuses NaN
  if (!B_K || !row_req || !row_pos || !page_table || !pool) return LRKV_ERR_INVALID_ARG;
  if (!aligned16(B_K) || !aligned16(pool) || (reinterpret_cast<uintptr_t>(row_req) & 3u) ||
      (reinterpret_cast<uintptr_t>(row_pos) & 3u) || (reinterpret_cast<uintptr_t>(page_table) & 3u))
    return LRKV_ERR_INVALID_ARG;
  const Variant v = find_variant(L);
  if (v != V_C1N && v != V_C3N) return LRKV_ERR_UNSUPPORTED;
  if (n_rows == 0) return LRKV_OK;
  NormArgs a{};
  a.B_K = B_K;
  a.eps = eps;
  a.row_req = row_req;
  a.row_pos = row_pos;
  a.n_rows = n_rows;
  a.page_table = page_table;
  a.max_pages = max_pages_per_req;
  a.pool = pool;
  a.stream = static_cast<hipStream_t>(stream);
  if (v == V_C1N) return hip_status(launch_key_norms<ShapeC1N>(a));
  return hip_status(launch_key_norms<ShapeC3N>(a));
}

int lrkv_check_indices(const lrkv_layout* L, const int32_t* page_table, int32_t batch,
                       int32_t max_pages_per_req, const int32_t* seq_lens, int32_t max_seq_len,
                       const int32_t* row_req, const int32_t* row_pos, int32_t n_rows,
                       int64_t num_pages, int32_t* errors, void* stream) {
  if (!layout_valid(L)) return LRKV_ERR_INVALID_ARG;
  if (batch <= 0 || max_pages_per_req <= 0 || max_seq_len < 0 || n_rows < 0 || num_pages <= 0)
    return LRKV_ERR_INVALID_ARG;
  if ((long long)max_seq_len > (long long)max_pages_per_req * L->page_size)
    return LRKV_ERR_INVALID_ARG;
  if ((long long)max_pages_per_req * L->page_size > 0x7fffffffLL) return LRKV_ERR_INVALID_ARG;
  if (!page_table || !errors || (!row_req) != (!row_pos)) return LRKV_ERR_INVALID_ARG;
  auto aligned4 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; };
  if (!aligned4(page_table) || !aligned4(errors) || (seq_lens && !aligned4(seq_lens)) ||
      (row_req && (!aligned4(row_req) || !aligned4(row_pos))))
    return LRKV_ERR_INVALID_ARG;
  CheckArgs a{};
  a.page_table = page_table;
  a.batch = batch;
  a.max_pages = max_pages_per_req;
  a.seq_lens = seq_lens;
  a.max_seq_len = max_seq_len;
  a.row_req = row_req;
  a.row_pos = row_pos;
  a.n_rows = row_req ? n_rows : 0;
  a.num_pages = num_pages;
  a.page_size = L->page_size;
  a.errors = errors;
  a.stream = static_cast<hipStream_t>(stream);
  return hip_status(launch_check(a));
}

}  // extern "C"
