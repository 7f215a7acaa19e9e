// Key-norm step of an append for gfx950: the RMSNorm paragraph of the LRKV notes §8.  The
// normalising denominator of a key depends on the full key k = s + z B_h^T, which neither
// branch holds alone (its square expands into a shared term, a cross term 2 s B_h z^T and a
// private term); so, when a token is appended, the reciprocal 1/n_h with
//   n_h = sqrt(|s + z B_h^T|^2 / d_h + eps)
// is computed once per head from the token's stored rows and kept in the page's N section;
// decode multiplies it onto the summed score.
//
// Workgroup = (16 appended rows, 4 heads), 4 wavefronts, one head each, so that the heads
// of a decode step's few rows run side by side on H/4 compute units rather than one after
// another on one.  For its head a wavefront forms the 16 x d_h block of full keys on MFMA
// (v_mfma_f32_16x16x32_bf16: A = the rows' R_K[h] chunks read from their pages, B =
// B_K[h]^T, the accumulator starting from the rows' S_K), squares it and sums over the
// features of each row.
#include "lrkv_device.h"
#include "lrkv_launch.h"

namespace lrkv {

namespace {

typedef __bf16 bf16x8_n __attribute__((ext_vector_type(8)));
typedef float f32x4_n __attribute__((ext_vector_type(4)));

template <class S>
struct NormCfg {
  static constexpr int ROWS = 16;
  static constexpr int NT = 256;
  static constexpr int NTILE = S::DH / 16;
  static constexpr int KB = (S::R + 31) / 32;
  static_assert(S::BF && S::NORM && S::P == 16, "bf16 key-norm layouts");
  static_assert(S::DHC * ROWS == NT, "one S_K chunk of one row per thread");
  static_assert(S::H % 4 == 0, "heads in groups of four");
};

template <class S>
__global__ void __launch_bounds__(256, 2) key_norm_kernel(const NormArgs a) {
  using C = NormCfg<S>;
  __shared__ __align__(16) uint16_t skt[S::DH * C::ROWS];  // S_K of the rows, [feature][row]
  __shared__ long long row_page[C::ROWS];                  // byte offset of the row's page, -1: none
  __shared__ int row_slot[C::ROWS];
  const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = (int)blockIdx.x * C::ROWS;
  const int n = lane & 15, g = lane >> 4;
  const int h = 4 * (int)blockIdx.y + wave;
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
  // B_K[h] operands depend on nothing: requested first, beside the rows' destinations.
  // B: B_K[h][16nt + lane%16][k0 .. k0 + 8), k0 = 32 kb + 8 (lane/16); k0 past r reads a
  // valid chunk and is zeroed
  const uint8_t* bkh = static_cast<const uint8_t*>(a.B_K) + (size_t)h * S::DH * S::R * 2;
  uint4 bvv[C::KB][C::NTILE];
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb) {
    const int k0 = 32 * kb + 8 * g;
    const int kc = min(k0, S::R - 8);
#pragma unroll
    for (int nt = 0; nt < C::NTILE; ++nt) {
      const uint4 v = *reinterpret_cast<const uint4*>(bkh + ((size_t)(16 * nt + n) * S::R + kc) * 2);
      bvv[kb][nt] = k0 < S::R ? v : zero;
    }
  }
  if (tid < C::ROWS) {
    const int nr = n0 + tid;
    long long off = -1;
    int slot = 0;
    if (nr < a.n_rows) {
      const int req = a.row_req[nr], pos = a.row_pos[nr];
      off = (long long)a.page_table[(size_t)req * a.max_pages + pos / S::P] * S::PAGE;
      slot = pos % S::P;
    }
    row_page[tid] = off;
    row_slot[tid] = slot;
  }
  __syncthreads();
  const uint8_t* pool = static_cast<const uint8_t*>(a.pool);
  // the rows' S_K chunks (thread (row i, chunk c)) and this lane's R_K[h] chunks, requested
  // together (rows past the last read page 0 and are zeroed)
  const int i_s = tid / S::DHC, c_s = tid % S::DHC;
  const long long p_s = row_page[i_s];
  const uint4 sk0 = *reinterpret_cast<const uint4*>(pool + (p_s >= 0 ? p_s : 0) +
                                                    (c_s * S::P + row_slot[i_s]) * 16);
  const long long my_page = row_page[lane & 15];  // the A operand's row: lane % 16
  const int my_slot = row_slot[lane & 15];
  uint4 av[C::KB];
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb) {
    const int c = 4 * kb + g;  // A: R_K[h] chunk c of row lane % 16
    const int cl = min(c, S::RC - 1);
    const uint4 x = *reinterpret_cast<const uint4*>(pool + (my_page >= 0 ? my_page : 0) + S::OFF_RK +
                                                    h * S::SEC_R + (cl * S::P + my_slot) * 16);
    av[kb] = (c < S::RC && my_page >= 0) ? x : zero;
  }
  {  // S_K of the rows, transposed into skt
    const uint4 v = p_s >= 0 ? sk0 : zero;
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      skt[(8 * c_s + 2 * e) * C::ROWS + i_s] = (uint16_t)(w4[e] & 0xffffu);
      skt[(8 * c_s + 2 * e + 1) * C::ROWS + i_s] = (uint16_t)(w4[e] >> 16);
    }
  }
  __syncthreads();

  {
    f32x4_n acc[C::NTILE];
#pragma unroll
    for (int nt = 0; nt < C::NTILE; ++nt) {
      const uint2 v = *reinterpret_cast<const uint2*>(skt + (16 * nt + n) * C::ROWS + 4 * g);
      acc[nt] = f32x4_n{bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y)};
    }
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int nt = 0; nt < C::NTILE; ++nt)
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_n, av[kb]),
                                                          __builtin_bit_cast(bf16x8_n, bvv[kb][nt]),
                                                          acc[nt], 0, 0, 0);
    // lane holds rows 4g..4g+3 of feature 16nt + lane%16: sum of squares over the features
    float ss[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < C::NTILE; ++nt)
#pragma unroll
      for (int e = 0; e < 4; ++e) ss[e] = fmaf(acc[nt][e], acc[nt][e], ss[e]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float tot = r16_sum(ss[e]);
      const int i = 4 * g + e;
      if (n == 0 && row_page[i] >= 0) {
        const float inv = 1.0f / sqrtf(tot / (float)S::DH + a.eps);
        *reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(a.pool) + row_page[i] + S::OFF_N +
                                     (h * S::P + row_slot[i]) * 2) = (uint16_t)f32_to_bf16_rne(inv);
      }
    }
  }
}

}  // namespace

template <class S>
hipError_t launch_key_norms(const NormArgs& a) {
  const int blocks = (a.n_rows + NormCfg<S>::ROWS - 1) / NormCfg<S>::ROWS;
  hipLaunchKernelGGL((key_norm_kernel<S>), dim3(blocks, S::H / 4), dim3(NormCfg<S>::NT), 0,
                     a.stream, a);
  return hipGetLastError();
}

template hipError_t launch_key_norms<ShapeC1N>(const NormArgs&);
template hipError_t launch_key_norms<ShapeC3N>(const NormArgs&);

}  // namespace lrkv
