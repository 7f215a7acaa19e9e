// Device-side helpers and compile-time shapes shared by the LRKV kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lrkv {

constexpr int kPage = 16;  // tokens per page of every compiled variant

// Compile-time description of one kernel variant.  Page layout as in include/lrkv.h:
// sections S_K, S_V, R_K[0..H-1], R_V[0..H-1], each chunk-major ([chunk][token][16 B]).
// NORM_: the page also keeps, after R_V, one key-norm reciprocal per head and token slot,
// section N[h][t] (the joint RMSNorm denominator of the full key, LRKV notes §8).
template <int H_, int DH_, int R_, bool BF16_, bool NORM_ = false>
struct Shape {
  static constexpr int H = H_;
  static constexpr int DH = DH_;
  static constexpr int R = R_;
  static constexpr bool BF = BF16_;
  static constexpr bool NORM = NORM_;
  static constexpr int EB = BF ? 2 : 4;         // element bytes
  static constexpr int CE = 16 / EB;            // elements per 16-byte chunk
  static constexpr int DHC = DH / CE;           // chunks in a shared row
  static constexpr int RC = R / CE;             // chunks in a private row
  static constexpr int P = kPage;
  static constexpr int SEC_S = P * DH * EB;     // bytes of a shared section
  static constexpr int SEC_R = P * R * EB;      // bytes of one head's private block
  static constexpr int SEC_N = NORM ? H * P * EB : 0;  // bytes of the key-norm section
  // bytes from one page to the next: a key-norm page is padded to a whole KiB (pages
  // starting off a 1 KiB boundary read markedly slower); the others are whole KiB already
  static constexpr int PAGE_DATA = 2 * SEC_S + 2 * H * SEC_R + SEC_N;
  static constexpr int PAGE = NORM ? (PAGE_DATA + 1023) / 1024 * 1024 : PAGE_DATA;
  static constexpr int OFF_SV = SEC_S;
  static constexpr int OFF_RK = 2 * SEC_S;
  static constexpr int OFF_RV = 2 * SEC_S + H * SEC_R;
  static constexpr int OFF_N = 2 * SEC_S + 2 * H * SEC_R;  // N[h][t] at OFF_N + (h P + t) EB
  static constexpr int PART = 2 + DH + R;       // floats of a chunk's partial tuple per head
  static constexpr int PART_PAD = (PART + 3) / 4 * 4;  // record stride (16-byte rows)
  static_assert(DH % CE == 0 && R % CE == 0, "widths must be whole 16-byte chunks");
};

// ---- bfloat16 <-> float32 --------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float f32x2_v __attribute__((ext_vector_type(2)));

// float32 -> bfloat16, round to nearest even (v_cvt_pk_bf16_f32); NaN stays a NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// two values in one conversion: lo in bits 0..15, hi in bits 16..31
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_v{lo, hi}, bf16x2_v));
}

// 2^x by v_exp_f32 (results below the float32 normal range may flush to zero: they only
// ever weigh softmax terms next to a weight of at least 1)
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// a.x*b.x + a.y*b.y + c on bfloat16 pairs with float32 accumulation (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, a),
                                         __builtin_bit_cast(bf16x2_v, b), c, false);
}

// ---- lane reductions inside rows of 16 lanes (one head per row) -------------------------

__device__ __forceinline__ float row16_max(float x) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) x = fmaxf(x, __shfl_xor(x, o, 16));
  return x;
}
__device__ __forceinline__ float row16_sum(float x) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) x += __shfl_xor(x, o, 16);
  return x;
}

// ---- DPP reductions inside a row of 16 lanes ----------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141; // lane i <-> 7-i inside each half row
constexpr int kMirror = 0x140;     // lane i <-> 15-i inside the row

__device__ __forceinline__ float r16_max(float x) {
  x = __builtin_fmaxf(x, dpp_f<kQuadSwap1>(x));
  x = __builtin_fmaxf(x, dpp_f<kQuadSwap2>(x));
  x = __builtin_fmaxf(x, dpp_f<kHalfMirror>(x));
  x = __builtin_fmaxf(x, dpp_f<kMirror>(x));
  return x;
}
__device__ __forceinline__ float r16_sum(float x) {
  x += dpp_f<kQuadSwap1>(x);
  x += dpp_f<kQuadSwap2>(x);
  x += dpp_f<kHalfMirror>(x);
  x += dpp_f<kMirror>(x);
  return x;
}

// max over the four 16-lane rows of a wavefront (v_permlane16_swap pairs rows 0-1 and 2-3,
// v_permlane32_swap the two halves); every lane gets the result
__device__ __forceinline__ float rows4_max(float m) {
  const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  m = __builtin_fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
  const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return __builtin_fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
}
__device__ __forceinline__ float rows4_sum(float m) {
  const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  m = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
  const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
}

__device__ __forceinline__ float readlane_f(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// Query row i of a request holding T tokens sits at position T - q_len + i and sees
// positions 0..that position.
__device__ __forceinline__ int visible_tokens(int T, int q_len, int i) {
  int v = T - q_len + i + 1;
  v = v < T ? v : T;
  return v > 0 ? v : 0;
}

}  // namespace lrkv
