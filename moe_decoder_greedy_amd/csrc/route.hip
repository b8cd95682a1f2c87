// Embedding gather and the fused RMSNorm + top-k router.
//
// Router ("The speed comes from three layers working together", Jina-OCR-v1
// explainer on kg.zhiyong.dev: top-6 of 64 routed experts): RMSNorm in fp32,
// router logits from the unrounded normalised state, selection of the k
// largest logits (lower expert index first on ties), and weights equal to the
// softmax renormalised over the selected experts, i.e. exp(l_r - l_max) over
// the sum of the k chosen exp(l_j - l_max).
//
// Layout of one block (256 threads = 4 wavefronts, TPB tokens):
//   phase 1  one wave per token: sum of squares (per-lane strided partials,
//            then a butterfly), x = h * rsqrt-scale * gamma into LDS (fp32)
//            and to x_out (rounded to the operand type);
//   phase 2  wave w computes the logits of experts w, w+4, ... for all TPB
//            tokens, streaming each router row once per block (coalesced
//            8-byte bf16 loads) against the LDS copy of x;
//   phase 3  one wave per token, one lane per expert: k rounds of a wavefront
//            (value, index) arg max, then the renormalised softmax weights.
// Every reduction has a fixed order, so a token's outputs do not depend on
// which block or batch it lands in.
#include "launch.h"

namespace moev {
namespace {

constexpr int kRouteTPB = 4;

template <typename WT> struct Vec4;
template <> struct Vec4<u16> {
  __device__ static float4 load(const u16* p) {
    uint2 u = *reinterpret_cast<const uint2*>(p);
    return make_float4(bf16_to_f32(u.x & 0xFFFF), bf16_to_f32(u.x >> 16), bf16_to_f32(u.y & 0xFFFF),
                       bf16_to_f32(u.y >> 16));
  }
  __device__ static void store(u16* p, float4 v) {
    uint2 u;
    u.x = static_cast<uint32_t>(f32_to_bf16(v.x)) | (static_cast<uint32_t>(f32_to_bf16(v.y)) << 16);
    u.y = static_cast<uint32_t>(f32_to_bf16(v.z)) | (static_cast<uint32_t>(f32_to_bf16(v.w)) << 16);
    *reinterpret_cast<uint2*>(p) = u;
  }
};
template <> struct Vec4<float> {
  __device__ static float4 load(const float* p) { return *reinterpret_cast<const float4*>(p); }
  __device__ static void store(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
};

template <typename WT>
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ tokens,
                                                    const WT* __restrict__ emb, int T, int H, int V,
                                                    float* __restrict__ h) {
  const int t = blockIdx.x;
  int tok = tokens[t];
  tok = tok < 0 ? 0 : (tok >= V ? V - 1 : tok);
  const WT* src = emb + static_cast<size_t>(tok) * H;
  float* dst = h + static_cast<size_t>(t) * H;
  for (int i = threadIdx.x * 4; i < H; i += 1024)
    *reinterpret_cast<float4*>(dst + i) = Vec4<WT>::load(src + i);
}

template <typename WT>
__global__ __launch_bounds__(256) void route_kernel(
    const float* __restrict__ h, const WT* __restrict__ norm_w, float eps,
    const WT* __restrict__ wr, const float* __restrict__ bias, int T, int H, int E, int k,
    WT* __restrict__ x_out, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    float* __restrict__ logits_out) {
  extern __shared__ float smem[];
  float* xs = smem;                   // [TPB][H]
  float* lg = smem + kRouteTPB * H;   // [TPB][64]
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * kRouteTPB;

  // phase 1: RMSNorm, wave `wave` takes token t0 + wave
  {
    const int t = t0 + wave;
    if (t < T) {
      const float* hr = h + static_cast<size_t>(t) * H;
      float ss = 0.f;
      for (int i = lane * 4; i < H; i += 256) {
        float4 v = *reinterpret_cast<const float4*>(hr + i);
        ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
      }
      ss = wave_sum(ss);
      const float r = 1.0f / sqrtf(ss / static_cast<float>(H) + eps);
      for (int i = lane * 4; i < H; i += 256) {
        float4 v = *reinterpret_cast<const float4*>(hr + i);
        float4 g = norm_w ? Vec4<WT>::load(norm_w + i) : make_float4(1.f, 1.f, 1.f, 1.f);
        float4 x = make_float4(v.x * r * g.x, v.y * r * g.y, v.z * r * g.z, v.w * r * g.w);
        *reinterpret_cast<float4*>(xs + wave * H + i) = x;
        Vec4<WT>::store(x_out + static_cast<size_t>(t) * H + i, x);
      }
    }
  }
  __syncthreads();

  // phase 2: router logits
  const int nt = min(kRouteTPB, T - t0);
  for (int e = wave; e < E; e += 4) {
    const WT* w = wr + static_cast<size_t>(e) * H;
    float acc[kRouteTPB];
#pragma unroll
    for (int tt = 0; tt < kRouteTPB; ++tt) acc[tt] = 0.f;
    for (int i = lane * 4; i < H; i += 256) {
      float4 wv = Vec4<WT>::load(w + i);
#pragma unroll
      for (int tt = 0; tt < kRouteTPB; ++tt) {
        float4 x = *reinterpret_cast<const float4*>(xs + tt * H + i);
        acc[tt] += x.x * wv.x + x.y * wv.y + x.z * wv.z + x.w * wv.w;
      }
    }
    const float b = bias ? bias[e] : 0.f;
#pragma unroll
    for (int tt = 0; tt < kRouteTPB; ++tt) {
      float s = wave_sum(acc[tt]);
      if (lane == 0 && tt < nt) lg[tt * 64 + e] = s + b;
    }
  }
  __syncthreads();

  // phase 3: top-k + renormalised softmax, one wave per token
  {
    const int t = t0 + wave;
    if (t < T) {
      float v = lane < E ? lg[wave * 64 + lane] : -INFINITY;
      if (logits_out != nullptr && lane < E) logits_out[static_cast<size_t>(t) * E + lane] = v;
      float top0 = 0.f, mine = 0.f;
      int mine_idx = 0;
      for (int r = 0; r < k; ++r) {
        float bv = v;
        int bi = lane;
        wave_argmax(bv, bi);
        if (r == 0) top0 = bv;
        if (lane == r) { mine = bv; mine_idx = bi; }
        if (lane == bi) v = -INFINITY;
      }
      const float ex = lane < k ? expf(mine - top0) : 0.f;
      const float sum = wave_sum(ex);
      if (lane < k) {
        topk_idx[static_cast<size_t>(t) * k + lane] = mine_idx;
        topk_w[static_cast<size_t>(t) * k + lane] = ex / sum;
      }
    }
  }
}

moev_status check_hidden(int H) {
  if (H < 64 || H > 4032 || H % 64 != 0) {
    set_error("hidden size %d must be a multiple of 64 in [64, 4032]", H);
    return MOEV_ERR_UNSUPPORTED;
  }
  return MOEV_OK;
}

}  // namespace

// Launchers shared with the whole-step driver (no validation).
void launch_embed(const int32_t* tokens, const void* emb, int T, int H, int V, int dt, float* h,
                  hipStream_t s) {
  if (dt == MOEV_BF16)
    embed_kernel<u16><<<T, 256, 0, s>>>(tokens, static_cast<const u16*>(emb), T, H, V, h);
  else
    embed_kernel<float><<<T, 256, 0, s>>>(tokens, static_cast<const float*>(emb), T, H, V, h);
}

void launch_route(const float* h, const void* norm_w, float eps, const void* w_router,
                  const float* bias, int T, int H, int E, int k, int dt, void* x_out,
                  int32_t* topk_idx, float* topk_w, float* logits_out, hipStream_t s) {
  const int blocks = (T + kRouteTPB - 1) / kRouteTPB;
  const size_t lds = (static_cast<size_t>(kRouteTPB) * H + kRouteTPB * 64) * sizeof(float);
  if (dt == MOEV_BF16)
    route_kernel<u16><<<blocks, 256, lds, s>>>(h, static_cast<const u16*>(norm_w), eps,
                                                static_cast<const u16*>(w_router), bias, T, H, E, k,
                                                static_cast<u16*>(x_out), topk_idx, topk_w,
                                                logits_out);
  else
    route_kernel<float><<<blocks, 256, lds, s>>>(h, static_cast<const float*>(norm_w), eps,
                                                  static_cast<const float*>(w_router), bias, T, H, E,
                                                  k, static_cast<float*>(x_out), topk_idx, topk_w,
                                                  logits_out);
}

moev_status validate_route(const float* h, const void* norm_w, const void* w_router,
                           const float* bias, int T, int H, int E, int k, int dt,
                           const void* x_out, const int32_t* topk_idx, const float* topk_w,
                           const float* logits_out) {
  MOEV_CHECK(check_dtype(dt), MOEV_ERR_UNSUPPORTED);
  if (moev_status st = check_hidden(H)) return st;
  MOEV_REQUIRE(T >= 0, MOEV_ERR_INVALID_ARG, "T must be >= 0 (got %d)", T);
  MOEV_REQUIRE(E >= 1 && E <= 64, MOEV_ERR_UNSUPPORTED, "routed experts E=%d must be in [1, 64]", E);
  MOEV_REQUIRE(k >= 1 && k <= E, MOEV_ERR_UNSUPPORTED, "top-k k=%d must be in [1, E=%d]", k, E);
  if (T == 0) return MOEV_OK;
  MOEV_CHECK(need_ptr(h, "h") && opt_ptr(norm_w, "norm_w") && need_ptr(w_router, "w_router") &&
                 opt_ptr(bias, "bias") && need_ptr(x_out, "x_out") &&
                 need_ptr(topk_idx, "topk_idx") && need_ptr(topk_w, "topk_w") &&
                 opt_ptr(logits_out, "logits_out"),
             MOEV_ERR_INVALID_ARG);
  return MOEV_OK;
}

moev_status validate_embed(const int32_t* tokens, const void* emb, int T, int H, int V, int dt,
                           const float* h_out) {
  MOEV_CHECK(check_dtype(dt), MOEV_ERR_UNSUPPORTED);
  if (moev_status st = check_hidden(H)) return st;
  MOEV_REQUIRE(T >= 0 && V >= 1, MOEV_ERR_INVALID_ARG, "need T >= 0 and V >= 1 (T=%d V=%d)", T, V);
  if (T == 0) return MOEV_OK;
  MOEV_CHECK(need_ptr(tokens, "tokens") && need_ptr(emb, "emb") && need_ptr(h_out, "h_out"),
             MOEV_ERR_INVALID_ARG);
  return MOEV_OK;
}

}  // namespace moev

extern "C" moev_status moe_embed(const int32_t* tokens, const void* emb, int T, int H, int V,
                                 int dt, float* h_out, void* stream) {
  if (moev_status st = moev::validate_embed(tokens, emb, T, H, V, dt, h_out)) return st;
  if (T == 0) return MOEV_OK;
  moev::launch_embed(tokens, emb, T, H, V, dt, h_out, moev::as_stream(stream));
  return moev::launch_status("moe_embed");
}

extern "C" moev_status moe_route(const float* h, const void* norm_w, float eps,
                                 const void* w_router, const float* bias, int T, int H, int E,
                                 int k, int dt, void* x_out, int32_t* topk_idx, float* topk_w,
                                 float* logits_out, void* stream) {
  if (moev_status st = moev::validate_route(h, norm_w, w_router, bias, T, H, E, k, dt, x_out,
                                            topk_idx, topk_w, logits_out))
    return st;
  if (T == 0) return MOEV_OK;
  moev::launch_route(h, norm_w, eps, w_router, bias, T, H, E, k, dt, x_out, topk_idx, topk_w,
                     logits_out, moev::as_stream(stream));
  return moev::launch_status("moe_route");
}
