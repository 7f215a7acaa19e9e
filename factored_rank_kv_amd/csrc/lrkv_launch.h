// Host-side launch interface between the C-ABI entry points and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lrkv_device.h"

namespace lrkv {

// The compiled kernel variants: (H, d_h, r, dtype).
using ShapeC0 = Shape<4, 16, 4, false>;    // float32 single-layer check
using ShapeC1 = Shape<16, 128, 56, true>;  // bf16, 16 heads, rank 56 (half the dense cache)
using ShapeC3 = Shape<32, 128, 32, true>;  // bf16, 32 heads, rank 32
// the same bf16 shapes with the key-norm section in every page
using ShapeC1N = Shape<16, 128, 56, true, true>;
using ShapeC3N = Shape<32, 128, 32, true, true>;
// one block of a grouped page: 16 heads of rank 32 (the 32-head layout in 2 groups)
using ShapeC3G = Shape<16, 128, 32, true>;

struct DecodeArgs {
  const void* q;
  int batch;
  int q_len;
  const void* B_K;
  const void* B_V;
  const void* pool;
  const int32_t* page_table;
  int max_pages;
  const int32_t* seq_lens;
  int n_split;   // chunks per (request, query row)
  int chunk;     // tokens per chunk, a multiple of the page size
  int groups;    // > 0: balanced split over this many workgroups (q_len = 1)
  void* out;
  // partial records of 2 + d_h + r floats (padded to 4) per head: [batch][q_len][n_split][H],
  // or, balanced, [groups + batch][H]
  float* part_ws;
  hipStream_t stream;
  // lrkv_decode_pq: the rows' private queries as private_queries_kernel writes them (null:
  // the split workgroups form them from B_K)
  const void* p_ext;
};

struct AppendArgs {
  const void* X;
  int n_rows;
  int d;
  const void* W_SK;
  const void* W_SV;
  const void* U_K;
  const void* U_V;
  const int32_t* row_req;
  const int32_t* row_pos;
  const int32_t* page_table;
  int max_pages;
  void* pool;
  hipStream_t stream;
  // grouped pages: elements from page to page, and the group block's first element (0 and
  // 0: a one-group page of shape S)
  long long page_elems;
  long long elem_off;
};

template <class S>
hipError_t launch_decode(const DecodeArgs& a);

// Private queries formed once per query row, for lrkv_decode_pq (plain layouts): bytes per
// row of the block, and the launch over `rows` rows of q.
template <class S>
size_t private_query_row_bytes();
template <class S>
hipError_t launch_private_queries(const void* q, const void* BK, int rows, void* p, hipStream_t stream,
                                  int groups = 1);
// The append of a.n_rows (1..8) bf16 rows and the private queries of `rows` query rows in
// one launch on a.stream: workgroups of the formation, then the 8-row append's.
template <class S>
hipError_t launch_append_pq(const AppendArgs& a, const void* q, const void* BK, int rows, void* p);

// Grouped layout of G blocks of shape Sg (G * Sg::H = S::H heads): the split kernels run
// per group on its block, one merge of shape S covers every head.
template <class Sg, class S>
hipError_t launch_decode_grouped(const DecodeArgs& a, int G);

// The merge + expansion of a chunked split's partial records (records [batch][q_len]
// [n_split][H], chunk tokens a.chunk), on a.stream.
template <class S>
hipError_t launch_merge(const DecodeArgs& a);

// Rotary decode (chunked split, then launch_merge); rope_cs is [rope_rows][d_h/2][2] float32.
template <class S>
hipError_t launch_decode_rope(const DecodeArgs& a, const float* rope_cs, int rope_rows);

// Head groups (workgroups per chunk) of the rotary decode.
template <class S>
int rope_groups();

template <class S>
hipError_t launch_append(const AppendArgs& a);

// Largest batch the balanced split handles (its kernels hold the batch's page counts in LDS).
constexpr int kBalancedMaxBatch = 1024;

// Query rows per request at or above which a bf16 lrkv_decode call takes the multi-query
// (prefill) kernel; it needs no workspace.
constexpr int kPrefillMinRows = 64;

// Most query rows (batch x q_len) of one private-query formation (its grid, H workgroups
// per block of 9 or more rows, stays well under 2^31 workgroups).
constexpr long long kMaxPrivateQueryRows = 1LL << 22;

// Rotary decode: heads per workgroup (one wavefront each) and the workgroups one wave of the
// grid holds (one per compute unit: eight wavefronts, two per SIMD, fill its registers).
constexpr int kRopeHeadsPerWorkgroup = 8;
constexpr int kRopeWaveWorkgroups = 256;

template <class S>
hipError_t launch_prefill(const DecodeArgs& a);

struct CheckArgs {
  const int32_t* page_table;
  int batch;
  int max_pages;
  const int32_t* seq_lens;  // may be null: lengths and their pages not checked
  int max_seq_len;
  const int32_t* row_req;   // may be null (then row_pos too): rows not checked
  const int32_t* row_pos;
  int n_rows;
  long long num_pages;
  int page_size;
  int32_t* errors;
  hipStream_t stream;
};

// Key-norm step of an append: reciprocal joint RMS denominators of the appended rows' keys.
struct NormArgs {
  const void* B_K;
  float eps;
  const int32_t* row_req;
  const int32_t* row_pos;
  int n_rows;
  const int32_t* page_table;
  int max_pages;
  void* pool;
  hipStream_t stream;
};

template <class S>
hipError_t launch_key_norms(const NormArgs& a);

// Copies whole pages of `page_bytes` bytes: page src[i] to dst[i] for i < n, or, with
// null id arrays, the one page single_src to single_dst.
hipError_t launch_copy_pages(uint8_t* pool, const int32_t* src, const int32_t* dst, int n,
                             long long page_bytes, int single_src, int single_dst,
                             hipStream_t stream);

// Zeroes *errors, then adds the number of index values that break the layout's rules.
hipError_t launch_check(const CheckArgs& a);

}  // namespace lrkv
