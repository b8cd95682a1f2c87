// Embedding gather and the fused RMSNorm + top-k router.
//
// Router ("The speed comes from three layers working together", Jina-OCR-v1
// explainer on kg.zhiyong.dev: top-6 of 64 routed experts): RMSNorm in fp32,
// router logits from the unrounded normalised state, selection of the k
// largest logits (lower expert index first on ties), and weights equal to the
// softmax renormalised over the selected experts, i.e. exp(l_r - l_max) over
// the sum of the k chosen exp(l_j - l_max).
//
// Layout of one block (1024 threads = 16 wavefronts, TPB = 1, 2 or 8
// tokens: more blocks in flight for small batches, more tokens per fetch of
// the router matrix for large ones):
//   phase 0  the block's residual rows (with the previous layer's expert
//            slots added, when fused) into LDS; at decode sizes wave w also
//            requests the router rows of experts 4w..4w+3 into registers
//            right behind them (coalesced 8-byte bf16 loads, all in flight),
//            so the weight fetch overlaps phases 0 and 1;
//   phase 1  waves 0..TPB-1, one per token: sum of squares (per-lane strided
//            partials, then a DPP reduction), x = h * rsqrt-scale * gamma into
//            LDS (fp32) and to x_out (rounded to the operand type);
//   phase 2  every wave multiplies its 4 router rows against the LDS copy of
//            the block's tokens, 4 tokens at a time;
//   phase 3  one wave per token, one lane per expert: each lane's rank is
//            the number of experts that beat it (read back from LDS), the
//            k best file themselves by rank, then the renormalised softmax
//            weights are formed in rank order.
// Lane sums use DPP row/broadcast steps rather than LDS shuffles.
// Every reduction has a fixed order, so a token's outputs do not depend on
// which block or batch it lands in.
#include "launch.h"
#include "route_core.h"

namespace moev {
namespace {

constexpr int kRouteGroupMax = 4;    // tokens per logit pass
constexpr int kRouteThreads = 1024;   // 16 wavefronts
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kExpertsPerWave = 4;    // 16 waves x 4 = 64 experts
constexpr int kMaxSlots = 16;         // k + ns limit of the fused combine

template <typename WT>
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ tokens,
                                                    const WT* __restrict__ emb, int T, int H, int V,
                                                    float* __restrict__ h, TokenSets sets, int* zero,
                                                    int n_zero) {
  const int t = blockIdx.x;
  if (sets.masks != nullptr) {
    // the blocks clear the mask sets of every layer between them
    const size_t n = sets.n_sets * set_layer_words(sets.E, sets.W * 64);
    for (size_t i = t * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) sets.masks[i] = 0ull;
  }
  for (int i = t * blockDim.x + threadIdx.x; i < n_zero; i += gridDim.x * blockDim.x) zero[i] = 0;
  int tok = tokens[t];
  tok = tok < 0 ? 0 : (tok >= V ? V - 1 : tok);
  const WT* src = emb + static_cast<size_t>(tok) * H;
  float* dst = h + static_cast<size_t>(t) * H;
  for (int i = threadIdx.x * 4; i < H; i += 1024)
    *reinterpret_cast<float4*>(dst + i) = Vec4<WT>::load(src + i);
}

struct RouteArgs {
  const float* h;        // residual stream in [T, H]
  const float* y;        // previous layer's expert slots [T, S, H] or NULL
  int S;                 // slots per token of y
  float* h_out;          // h + sum_s y[:, s] (written when y != NULL; may equal h)
  const void* norm_w;
  float eps;
  const void* wr;
  const float* bias;
  int T, H, E, k;
  void* x_out;
  int32_t* topk_idx;
  float* topk_w;
  float* logits_out;
  uint64_t* masks;       // token sets (optional): this layer's [W][E] mask words
  int2* pinfo;           //   and [T][E] pair entries {weight bits, slot}
  int W;
};

// NCH = ceil(H / 256): 4-element chunks per lane per row, a compile-time count
// so that every router-row load of a wave is in flight at once.
// COMBINE: phase 0 first adds the previous layer's expert slots to the
// residual (the same left-to-right slot order as the combine kernel, so the
// bits are identical) and writes the new residual; SL >= S bounds the
// unrolled slot loads.
// PRELOAD (decode sizes, one block per CU): every load of the block is
// issued up front -- the small operands (bias, RMSNorm gain), the residual
// rows and slots, then the router rows -- and the block's global stores
// (new residual, normalised operand) wait until the logits are done, so no
// wait for a load is also a wait for a store (the vector memory counter
// counts both, in order).  Without PRELOAD each chunk of the router rows is
// fetched inside the logit loop and the stores go out as soon as their
// values exist, which keeps the block small enough for two per CU (8 waves
// per SIMD: the second launch bound): while one block computes logits, the
// other streams its residual rows and expert slots.  The arithmetic of every
// logit is the same either way.
template <typename WT, int NCH, bool COMBINE, int kRouteTPB, bool PRELOAD, int SL = kMaxSlots>
__global__ __launch_bounds__(kRouteThreads, PRELOAD ? 1 : 8) void route_kernel(RouteArgs a) {
  extern __shared__ float smem[];
  const int H = a.H, E = a.E, k = a.k, T = a.T;
  const WT* __restrict__ wr = static_cast<const WT*>(a.wr);
  const WT* __restrict__ norm_w = static_cast<const WT*>(a.norm_w);
  WT* __restrict__ x_out = static_cast<WT*>(a.x_out);
  float* xs = smem;                                             // [TPB][H]
  float* lg = smem + kRouteTPB * H;                             // [TPB][64]
  float* sel_v = lg + kRouteTPB * 64;                           // [TPB][64]
  int* sel_i = reinterpret_cast<int*>(sel_v + kRouteTPB * 64);  // [TPB][64]
  int* rpart = sel_i + kRouteTPB * 64;                          // [TPB][kWpt][64]
  // the wave index is uniform: expert indices and bias reads stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * kRouteTPB;
  const int e0 = wave * kExpertsPerWave;
  const int nt = min(kRouteTPB, T - t0);
  constexpr int kStageIt = (kRouteTPB * NCH * 64 + kRouteThreads - 1) / kRouteThreads;
  constexpr bool kDefer = PRELOAD;  // stores after the logits
  static_assert(64 % kRouteTPB == 0, "a block's tokens share one 64-bit mask word");
  // with several tokens per block: their token-set bits per expert, gathered
  // here and sent with one global OR per expert (fewer atomics on a hot
  // expert's mask words when the routing is skewed)
  __shared__ unsigned long long blk_bits[kRouteTPB > 1 ? 64 : 1];
  if (kRouteTPB > 1 && threadIdx.x < 64) blk_bits[threadIdx.x] = 0ull;
  constexpr int kWpt = kRouteWaves / kRouteTPB;  // waves counting one token's ranks
  constexpr int kEpw = 64 / kWpt;                // entries each of them compares
  static_assert(kEpw % 4 == 0, "rank parts over whole float4 reads");

  // bias entries of this wave's experts: read unconditionally (from the
  // residual rows, T * H >= 64 floats, when there is no bias) and selected,
  // so no branch waits for them here
  const float* bsrc = a.bias != nullptr ? a.bias : a.h;
  float bv[kExpertsPerWave];
#pragma unroll
  for (int u = 0; u < kExpertsPerWave; ++u) bv[u] = bsrc[min(e0 + u, E - 1)];
  // RMSNorm gain for the waves that normalise a token, kept raw until used
  typename Vec4<WT>::Raw graw[NCH];
  const bool has_gain = norm_w != nullptr;
  if (wave < kRouteTPB && has_gain) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) graw[c] = Vec4<WT>::load_raw(norm_w + min(lane * 4 + c * 256, H - 4));
  }
  float4 wv[kExpertsPerWave][PRELOAD ? NCH : 1];
  auto preload_router = [&]() {
    if constexpr (PRELOAD) {
#pragma unroll
      for (int u = 0; u < kExpertsPerWave; ++u) {
        const int e = min(e0 + u, E - 1);
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          const int i = min(lane * 4 + c * 256, H - 4);
          wv[u][c] = Vec4<WT>::load(wr + static_cast<size_t>(e) * H + i);
        }
      }
    }
  };

  // phase 0: all threads stage the block's residual rows into LDS (xs),
  // adding the previous layer's expert slots first when COMBINE; every slot
  // load of a thread is issued before the sum, which runs left to right in
  // slot order exactly as the combine kernel does
  float4 hkeep[kDefer ? kStageIt : 1];  // new residual, stored after the logits
  {
    const int h4 = H / 4;
#pragma unroll
    for (int it = 0; it < kStageIt; ++it) {
      const int f = threadIdx.x + it * kRouteThreads;
      const bool live = f < nt * h4;
      const int tt = f / h4;
      const int i = (f - tt * h4) * 4;
      const size_t t = static_cast<size_t>(t0 + tt);
      float4 v, sv[SL];
      const float4* ys = reinterpret_cast<const float4*>(a.y + t * a.S * H + i);
      if (live) {
        v = *reinterpret_cast<const float4*>(a.h + t * H + i);
        if (COMBINE) load_slots<SL>(sv, ys, a.S, h4);
      }
      if (it == 0) preload_router();
      if (!live) continue;
      if (COMBINE) {
        v = sum_slots<SL>(v, sv, a.S);
        if constexpr (kDefer) hkeep[it] = v;
        else *reinterpret_cast<float4*>(a.h_out + t * H + i) = v;
      }
      *reinterpret_cast<float4*>(xs + tt * H + i) = v;
    }
  }
  __syncthreads();

  // phase 1: RMSNorm in place in LDS, wave w < TPB takes token t0 + w; the
  // logit row's entries past E are set to -inf (never ranked above a real one)
  float4 xkeep[kDefer ? NCH : 1];  // normalised operand, stored after the logits
  if (wave < kRouteTPB) {
    const int t = t0 + wave;
    if (lane >= E) lg[wave * 64 + lane] = -INFINITY;
    if (t < T) {
      float4 hv[NCH];
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int i = lane * 4 + c * 256;
        hv[c] = i < H ? *reinterpret_cast<const float4*>(xs + wave * H + i) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < NCH; ++c) ss = sumsq_step(ss, hv[c]);
      const float r = rms_scale(ss, H, a.eps);
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int i = lane * 4 + c * 256;
        if (i < H) {
          const float4 v = hv[c];
          const float4 g = has_gain ? Vec4<WT>::from_raw(graw[c]) : make_float4(1.f, 1.f, 1.f, 1.f);
          const float4 x = make_float4(v.x * r * g.x, v.y * r * g.y, v.z * r * g.z, v.w * r * g.w);
          *reinterpret_cast<float4*>(xs + wave * H + i) = x;
          if constexpr (kDefer) xkeep[c] = x;
          else Vec4<WT>::store(x_out + static_cast<size_t>(t) * H + i, x);
        }
      }
    }
  }
  __syncthreads();

  // phase 2: router logits of this wave's experts for the block's tokens,
  // kRouteGroup tokens per pass (the same per-token arithmetic whatever TPB)
  constexpr int kRouteGroup = kRouteTPB < kRouteGroupMax ? kRouteTPB : kRouteGroupMax;
  if (e0 < E) {
#pragma unroll
    for (int t1 = 0; t1 < kRouteTPB; t1 += kRouteGroup) {
      float acc[kExpertsPerWave][kRouteGroup];
#pragma unroll
      for (int u = 0; u < kExpertsPerWave; ++u)
#pragma unroll
        for (int tt = 0; tt < kRouteGroup; ++tt) acc[u][tt] = 0.f;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int i = lane * 4 + c * 256;
        if (i < H) {
          const int cw = PRELOAD ? c : 0;
          if constexpr (!PRELOAD) {
#pragma unroll
            for (int u = 0; u < kExpertsPerWave; ++u)
              wv[u][0] = Vec4<WT>::load(wr + static_cast<size_t>(min(e0 + u, E - 1)) * H + i);
          }
#pragma unroll
          for (int tt = 0; tt < kRouteGroup; ++tt) {
            const float4 x = *reinterpret_cast<const float4*>(xs + (t1 + tt) * H + i);
#pragma unroll
            for (int u = 0; u < kExpertsPerWave; ++u)
              acc[u][tt] = dot_step(acc[u][tt], x, wv[u][cw]);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kExpertsPerWave; ++u) {
        const int e = e0 + u;
        if (e < E) {
          const float b = a.bias != nullptr ? bv[u] : 0.f;
#pragma unroll
          for (int tt = 0; tt < kRouteGroup; ++tt) {
            const float s = wave_sum_lane63(acc[u][tt]);
            if (lane == 63 && t1 + tt < nt) lg[(t1 + tt) * 64 + e] = s + b;
          }
        }
      }
    }
  }
  __syncthreads();

  // phase 3: top-k + renormalised softmax, one lane per expert.  Each lane's
  // rank is the number of experts that beat it (larger logit, or equal logit
  // and lower index); the kWpt waves of a token count it over kEpw entries
  // each, then one wave per token adds the parts, and the k lanes of rank < k
  // file themselves into sel_* by rank.
  {
    const int tt = wave / kWpt, pw = wave - tt * kWpt;
    if (t0 + tt < T) {
      const float* row = lg + tt * 64;
      rpart[(tt * kWpt + pw) * 64 + lane] = logit_rank_part<kEpw>(row, pw * kEpw, row[lane], lane);
    }
  }
  __syncthreads();
  if (wave < kRouteTPB) {
    const int t = t0 + wave;
    if (t < T) {
      const float* row = lg + wave * 64;
      const float v = row[lane];
      int rank = 0;
#pragma unroll
      for (int pw = 0; pw < kWpt; ++pw) rank += rpart[(wave * kWpt + pw) * 64 + lane];
      if (lane < E && rank < k) {
        sel_v[wave * 64 + rank] = v;
        sel_i[wave * 64 + rank] = lane;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      // the ranks are a permutation for finite logits; the clamp keeps the
      // token-set writes in bounds whatever the inputs
      const int e = min(max(sel_i[wave * 64 + min(lane, k - 1)], 0), E - 1);
      if (a.logits_out != nullptr && lane < E) a.logits_out[static_cast<size_t>(t) * E + lane] = v;
      if constexpr (kDefer) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          const int i = lane * 4 + c * 256;
          if (i < H) Vec4<WT>::store(x_out + static_cast<size_t>(t) * H + i, xkeep[c]);
        }
      }
      if (lane < k) {
        const float wgt = topk_weight(sel_v + wave * 64, k, lane);
        a.topk_idx[static_cast<size_t>(t) * k + lane] = e;
        a.topk_w[static_cast<size_t>(t) * k + lane] = wgt;
        if (a.masks != nullptr) {
          // token t joins expert e's set (no value returned, nothing waits)
          if constexpr (kRouteTPB > 1)
            __hip_atomic_fetch_or(&blk_bits[e], 1ull << (t & 63), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          else
            __hip_atomic_fetch_or(a.masks + set_word(a.E, e, t >> 6), 1ull << (t & 63),
                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          a.pinfo[static_cast<size_t>(t) * E + e] = make_int2(__float_as_int(wgt), lane);
        }
      }
    }
  }
  if constexpr (kRouteTPB > 1) {
    if (a.masks != nullptr) {
      __syncthreads();
      if (threadIdx.x < E) {
        const unsigned long long bits = blk_bits[threadIdx.x];
        if (bits != 0ull)
          __hip_atomic_fetch_or(a.masks + set_word(a.E, threadIdx.x, t0 >> 6), bits,
                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  // the new residual (all staging threads), after the logits
  if constexpr (kDefer && COMBINE) {
    const int h4 = H / 4;
#pragma unroll
    for (int it = 0; it < kStageIt; ++it) {
      const int f = threadIdx.x + it * kRouteThreads;
      if (f < nt * h4) {
        const int tt = f / h4;
        const int i = (f - tt * h4) * 4;
        *reinterpret_cast<float4*>(a.h_out + static_cast<size_t>(t0 + tt) * H + i) = hkeep[it];
      }
    }
  }
}

template <typename WT, bool COMBINE, int TPB, bool PRELOAD, int SL>
void launch_route_t(int nch, dim3 grid, size_t lds, hipStream_t s, const RouteArgs& a) {
#define MOEV_ROUTE_CASE(N)                                                               \
  case N:                                                                                \
    route_kernel<WT, N, COMBINE, TPB, PRELOAD, SL><<<grid, kRouteThreads, lds, s>>>(a);   \
    break;
  switch (nch) {
    MOEV_ROUTE_CASE(1) MOEV_ROUTE_CASE(2) MOEV_ROUTE_CASE(3) MOEV_ROUTE_CASE(4)
    MOEV_ROUTE_CASE(5) MOEV_ROUTE_CASE(6) MOEV_ROUTE_CASE(7) MOEV_ROUTE_CASE(8)
    MOEV_ROUTE_CASE(9) MOEV_ROUTE_CASE(10) MOEV_ROUTE_CASE(11) MOEV_ROUTE_CASE(12)
    MOEV_ROUTE_CASE(13) MOEV_ROUTE_CASE(14) MOEV_ROUTE_CASE(15)
    default: break;  // H <= 3072 is validated, so nch <= 15
  }
#undef MOEV_ROUTE_CASE
}

template <typename WT, int TPB, bool PRELOAD>
void launch_route_tpb(const RouteArgs& a, hipStream_t s) {
  const dim3 grid((a.T + TPB - 1) / TPB);
  // xs, lg, sel_v, sel_i, then the rank parts [TPB][16 / TPB][64]
  const size_t lds = (static_cast<size_t>(TPB) * a.H + 3 * TPB * 64 + 64 * kRouteWaves) * sizeof(float);
  const int nch = (a.H + 255) / 256;
  // the slot loads of the fused combine are unrolled to a compile-time bound
  if (a.y == nullptr) launch_route_t<WT, false, TPB, PRELOAD, 8>(nch, grid, lds, s, a);
  else if (a.S <= 8) launch_route_t<WT, true, TPB, PRELOAD, 8>(nch, grid, lds, s, a);
  else launch_route_t<WT, true, TPB, PRELOAD, kMaxSlots>(nch, grid, lds, s, a);
}

// Tokens per block: 1 for decode-sized batches (more blocks in flight, router
// rows preloaded), 2 for mid-sized ones (256 blocks at 512 tokens), and 8
// once there are enough tokens to fill the GPU with two blocks per CU (router
// rows fetched per chunk; the LDS copy of 8 rows fits twice).
template <typename WT>
void launch_route_dispatch(const RouteArgs& a, hipStream_t s) {
  if (a.T >= 2048 && a.H <= 2048) launch_route_tpb<WT, 8, false>(a, s);
  else if (a.T > 256) launch_route_tpb<WT, 2, true>(a, s);
  else launch_route_tpb<WT, 1, true>(a, s);
}

moev_status check_hidden(int H) {
  if (H < 64 || H > 3072 || H % 64 != 0) {
    set_error("hidden size %d must be a multiple of 64 in [64, 3072]", H);
    return MOEV_ERR_UNSUPPORTED;
  }
  return MOEV_OK;
}

}  // namespace

// Launchers shared with the whole-step driver (no validation).
void launch_embed(const int32_t* tokens, const void* emb, int T, int H, int V, int dt, float* h,
                  hipStream_t s, const TokenSets* sets, int* zero, int n_zero) {
  TokenSets ts{};
  if (sets != nullptr) ts = *sets;
  if (zero == nullptr) n_zero = 0;
  if (dt == MOEV_BF16)
    embed_kernel<u16><<<T, 256, 0, s>>>(tokens, static_cast<const u16*>(emb), T, H, V, h, ts, zero, n_zero);
  else
    embed_kernel<float><<<T, 256, 0, s>>>(tokens, static_cast<const float*>(emb), T, H, V, h, ts, zero, n_zero);
}

void launch_route(const float* h, const void* norm_w, float eps, const void* w_router,
                  const float* bias, int T, int H, int E, int k, int dt, void* x_out,
                  int32_t* topk_idx, float* topk_w, float* logits_out, hipStream_t s) {
  RouteArgs a{};
  a.h = h;
  a.norm_w = norm_w;
  a.eps = eps;
  a.wr = w_router;
  a.bias = bias;
  a.T = T;
  a.H = H;
  a.E = E;
  a.k = k;
  a.x_out = x_out;
  a.topk_idx = topk_idx;
  a.topk_w = topk_w;
  a.logits_out = logits_out;
  if (dt == MOEV_BF16) launch_route_dispatch<u16>(a, s);
  else launch_route_dispatch<float>(a, s);
}

void launch_route_fused(const float* h, const float* y_prev, int S_prev, float* h_out,
                        const void* norm_w, float eps, const void* w_router, const float* bias,
                        int T, int H, int E, int k, int dt, void* x_out, int32_t* topk_idx,
                        float* topk_w, hipStream_t s, uint64_t* masks, int2* pinfo) {
  RouteArgs a{};
  a.masks = masks;
  a.pinfo = pinfo;
  a.W = set_words(T);
  a.h = h;
  a.y = y_prev;
  a.S = S_prev;
  a.h_out = h_out;
  a.norm_w = norm_w;
  a.eps = eps;
  a.wr = w_router;
  a.bias = bias;
  a.T = T;
  a.H = H;
  a.E = E;
  a.k = k;
  a.x_out = x_out;
  a.topk_idx = topk_idx;
  a.topk_w = topk_w;
  if (dt == MOEV_BF16) launch_route_dispatch<u16>(a, s);
  else launch_route_dispatch<float>(a, s);
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
                 opt_ptr(bias, "bias", 4) && need_ptr(x_out, "x_out") &&
                 need_ptr(topk_idx, "topk_idx", 4) && need_ptr(topk_w, "topk_w", 4) &&
                 opt_ptr(logits_out, "logits_out", 4),
             MOEV_ERR_INVALID_ARG);
  return MOEV_OK;
}

moev_status validate_embed(const int32_t* tokens, const void* emb, int T, int H, int V, int dt,
                           const float* h_out) {
  MOEV_CHECK(check_dtype(dt), MOEV_ERR_UNSUPPORTED);
  if (moev_status st = check_hidden(H)) return st;
  MOEV_REQUIRE(T >= 0 && V >= 1, MOEV_ERR_INVALID_ARG, "need T >= 0 and V >= 1 (T=%d V=%d)", T, V);
  if (T == 0) return MOEV_OK;
  MOEV_CHECK(need_ptr(tokens, "tokens", 4) && need_ptr(emb, "emb") && need_ptr(h_out, "h_out"),
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
