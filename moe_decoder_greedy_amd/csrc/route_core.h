// Per-token arithmetic of the router ("The speed comes from three layers
// working together", Jina-OCR-v1 explainer on kg.zhiyong.dev: top-6 of 64
// routed experts).  Every block shape of the router kernel calls these, so a
// token gets the same bits whichever instantiation routes it; every
// multiply-add is written out, because a contraction left to the compiler
// could be formed differently in different instantiations.
#pragma once

#include "common.h"

namespace moev {

template <typename WT> struct Vec4;
template <> struct Vec4<u16> {
  using Raw = uint2;  // four bf16 as loaded
  __device__ static Raw load_raw(const u16* p) { return *reinterpret_cast<const uint2*>(p); }
  __device__ static float4 from_raw(uint2 u) {
    return make_float4(bf16_to_f32(u.x & 0xFFFF), bf16_to_f32(u.x >> 16), bf16_to_f32(u.y & 0xFFFF),
                       bf16_to_f32(u.y >> 16));
  }
  __device__ static float4 load(const u16* p) { return from_raw(load_raw(p)); }
  __device__ static uint2 pack(float4 v) {
    uint2 u;
    u.x = static_cast<uint32_t>(f32_to_bf16(v.x)) | (static_cast<uint32_t>(f32_to_bf16(v.y)) << 16);
    u.y = static_cast<uint32_t>(f32_to_bf16(v.z)) | (static_cast<uint32_t>(f32_to_bf16(v.w)) << 16);
    return u;
  }
  __device__ static void store(u16* p, float4 v) { *reinterpret_cast<uint2*>(p) = pack(v); }
};
template <> struct Vec4<float> {
  using Raw = float4;
  __device__ static Raw load_raw(const float* p) { return *reinterpret_cast<const float4*>(p); }
  __device__ static float4 from_raw(float4 v) { return v; }
  __device__ static float4 load(const float* p) { return *reinterpret_cast<const float4*>(p); }
  __device__ static void store(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
};

// ss + v.x^2 + v.y^2 + v.z^2 + v.w^2, one fused multiply-add at a time
__device__ __forceinline__ float sumsq_step(float ss, float4 v) {
  ss = fmaf(v.x, v.x, ss);
  ss = fmaf(v.y, v.y, ss);
  ss = fmaf(v.z, v.z, ss);
  return fmaf(v.w, v.w, ss);
}

// acc + x . w over four elements, one fused multiply-add at a time
__device__ __forceinline__ float dot_step(float acc, float4 x, float4 w) {
  acc = fmaf(x.x, w.x, acc);
  acc = fmaf(x.y, w.y, acc);
  acc = fmaf(x.z, w.z, acc);
  return fmaf(x.w, w.w, acc);
}

// The S expert slots ys[0], ys[h4], ... of one 4-element column (S <=
// kMaxSlots), every load issued before any is used and none under a branch
// (entries past S repeat slot S - 1 and are not summed).
template <int kMaxSlots>
__device__ __forceinline__ void load_slots(float4 (&sv)[kMaxSlots], const float4* ys, int S, size_t h4) {
#pragma unroll
  for (int sl = 0; sl < kMaxSlots; ++sl) sv[sl] = ys[static_cast<size_t>(min(sl, S - 1)) * h4];
}

// h + the S loaded slots added left to right (the order the combine kernel
// uses)
template <int kMaxSlots>
__device__ __forceinline__ float4 sum_slots(float4 h, const float4 (&sv)[kMaxSlots], int S) {
  float4 acc = sv[0];
#pragma unroll
  for (int sl = 1; sl < kMaxSlots; ++sl)
    if (sl < S) {
      acc.x += sv[sl].x;
      acc.y += sv[sl].y;
      acc.z += sv[sl].z;
      acc.w += sv[sl].w;
    }
  return make_float4(h.x + acc.x, h.y + acc.y, h.z + acc.z, h.w + acc.w);
}

// RMSNorm scale from the wave's sum of squares (lane 63 holds the total)
__device__ __forceinline__ float rms_scale(float ss_lanes, int H, float eps) {
  const float ss = lane63(wave_sum_lane63(ss_lanes));
  return 1.0f / sqrtf(ss / static_cast<float>(H) + eps);
}

// Part of the rank of this lane's logit v among the 64 entries of an LDS row
// (entries past the expert count hold -inf): the number of entries j in
// [j0, j0 + N) that beat it (larger, or equal with a lower index).  The rank
// is the sum of the parts over a partition of the 64 entries.
template <int N>
__device__ __forceinline__ int logit_rank_part(const float* row, int j0, float v, int lane) {
  static_assert(N % 4 == 0, "whole float4 reads");
  int rank = 0;
#pragma unroll
  for (int j4 = 0; j4 < N / 4; ++j4) {
    const int j = j0 + 4 * j4;
    const float4 r = *reinterpret_cast<const float4*>(row + j);
    rank += better(r.x, j + 0, v, lane) ? 1 : 0;
    rank += better(r.y, j + 1, v, lane) ? 1 : 0;
    rank += better(r.z, j + 2, v, lane) ? 1 : 0;
    rank += better(r.w, j + 3, v, lane) ? 1 : 0;
  }
  return rank;
}

// Renormalised softmax weight of the chosen logit sel[lane] over the k chosen
// ones, rank order: exp(l_r - l_0) / sum_j exp(l_j - l_0)
__device__ __forceinline__ float topk_weight(const float* sel, int k, int lane) {
  const float top0 = sel[0];
  float sum = 0.f;
  for (int j = 0; j < k; ++j) sum += expf(sel[j] - top0);
  return expf(sel[lane] - top0) / sum;
}

}  // namespace moev
