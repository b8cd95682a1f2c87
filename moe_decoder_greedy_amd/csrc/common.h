// Internal helpers shared by the HIP sources of libmoev: device types, MFMA
// fragments, wavefront reductions and host-side argument validation.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <string>

#include "moev.h"

namespace moev {

typedef uint16_t u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- host side

void set_error(const char* fmt, ...);
void clear_error();

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validation helpers: each returns false after recording the reason.  Buffers
// read or written with 16-byte vector accesses need align = 16; int32/fp32
// arrays touched one element at a time need align = 4.
bool need_ptr(const void* p, const char* name, unsigned align = 16);
bool opt_ptr(const void* p, const char* name, unsigned align = 16);  // NULL allowed
bool check_dtype(int dt);

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

moev_status launch_status(const char* what);  // hipGetLastError -> status

inline size_t align_up(size_t n, size_t a) { return (n + a - 1) / a * a; }

// ---------------------------------------------------------------- device side

__device__ __forceinline__ float bf16_to_f32(u16 b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ u16 f32_to_bf16(float f) {
  return __builtin_bit_cast(u16, static_cast<__bf16>(f));
}

template <typename WT> __device__ __forceinline__ float to_f32(WT v);
template <> __device__ __forceinline__ float to_f32<u16>(u16 v) { return bf16_to_f32(v); }
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }

template <typename WT> __device__ __forceinline__ WT from_f32(float v);
template <> __device__ __forceinline__ u16 from_f32<u16>(float v) { return f32_to_bf16(v); }
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }

// Sum across the 64 lanes of a wavefront, butterfly order (the same for every
// call site, so results are reproducible).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// DPP lane move of a float (gfx9 data-parallel primitives): CTRL selects the
// pattern; rows outside ROW_MASK receive 0.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf, false));
}

// Sum across the 64 lanes with DPP steps (VALU latency, no LDS round trips):
// pairs, quads, half rows, rows, then rows 0+1 and 0+1+2+3 via row broadcasts.
// The complete sum is in lane 63; the order of additions is fixed.
__device__ __forceinline__ float wave_sum_lane63(float v) {
  v += dpp_mov<0xb1>(v);        // quad_perm [1,0,3,2]
  v += dpp_mov<0x4e>(v);        // quad_perm [2,3,0,1]
  v += dpp_mov<0x141>(v);       // row_half_mirror
  v += dpp_mov<0x140>(v);       // row_mirror
  v += dpp_mov<0x142, 0xa>(v);  // row_bcast:15 -> rows 1, 3
  v += dpp_mov<0x143, 0xc>(v);  // row_bcast:31 -> rows 2, 3
  return v;
}

__device__ __forceinline__ float lane63(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

// (value, index) maximum with the lower index winning exact ties.  Every lane
// ends with the same pair.
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    float ov = __shfl_xor(v, m, kWave);
    int oi = __shfl_xor(i, m, kWave);
    if (better(ov, oi, v, i)) { v = ov; i = oi; }
  }
}

// Greedy prefix acceptance of one sequence ("The speed comes from three
// layers working together", Jina-OCR-v1 explainer on kg.zhiyong.dev):
// tk = (last committed token, d_1 .. d_K), gr = the main model's greedy token
// at each of those K+1 positions.  n = the number of leading drafts with
// d_j == gr[j-1]; cm (K+1 entries) receives d_1 .. d_n, then gr[n] (the
// correction, or the extra token when n == K), then -1 padding.  Returns n.
__device__ __forceinline__ int accept_prefix(const int32_t* tk, const int32_t* gr, int K, int32_t* cm) {
  int n = 0;
  while (n < K && tk[n + 1] == gr[n]) ++n;
  for (int j = 0; j <= K; ++j) cm[j] = j < n ? tk[j + 1] : (j == n ? gr[n] : -1);
  return n;
}

// ------------------------------------------------------------ MFMA fragments
//
// One 16x16 output tile accumulates over K in blocks of 32.  Lane l supplies
// row (l % 16) of A and column (l % 16) of B, with the 8 consecutive k values
// 8*(l / 16) .. 8*(l / 16)+7 of the block; the 16x16 fp32 result sits in lane
// l as rows 4*(l / 16) + v (v = 0..3) of column l % 16.
//
// bf16: one v_mfma_f32_16x16x32_bf16 per block.  fp32: eight
// v_mfma_f32_16x16x4_f32, the i-th taking k = 8*(l/16) + i from every lane, so
// both types accumulate a block's 32 products into the same output layout.

template <typename WT> struct Frag;

template <> struct Frag<u16> {
  bf16x8 v;
  __device__ __forceinline__ void load(const u16* p) { v = *reinterpret_cast<const bf16x8*>(p); }
};

template <> struct Frag<float> {
  f32x4 lo, hi;
  __device__ __forceinline__ void load(const float* p) {
    lo = *reinterpret_cast<const f32x4*>(p);
    hi = *reinterpret_cast<const f32x4*>(p + 4);
  }
};

__device__ __forceinline__ f32x4 mma(const Frag<u16>& a, const Frag<u16>& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mma(const Frag<float>& a, const Frag<float>& b, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[0], b.lo[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[1], b.lo[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[2], b.lo[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[3], b.lo[3], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[0], b.hi[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[1], b.hi[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[2], b.hi[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[3], b.hi[3], c, 0, 0, 0);
  return c;
}

}  // namespace moev

// Argument-check macros for the C entry points (return before any HIP call).
#define MOEV_REQUIRE(cond, code, ...)  \
  do {                                 \
    if (!(cond)) {                     \
      ::moev::set_error(__VA_ARGS__);  \
      return code;                     \
    }                                  \
  } while (0)

#define MOEV_CHECK(expr, code) \
  do {                         \
    if (!(expr)) return code;  \
  } while (0)
