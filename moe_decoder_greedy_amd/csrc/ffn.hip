// Weight-streaming grouped GEMMs on bf16 (or fp32) MFMA: the SwiGLU expert
// FFN (gate/up with a fused SiLU-multiply, down with the router-weight scale
// and the scatter to the token's slot) and the LM head with a blocked arg max.
//
// Experts: "The speed comes from three layers working together" (Jina-OCR-v1
// explainer, kg.zhiyong.dev) -- 64 routed and two always-on shared experts,
// top-6 routing.  Greedy head: "Why FastMTP fits OCR particularly well" (same
// page) -- verification reproduces greedy decoding, so the head's output is an
// arg max with a fixed tie rule (lowest vocabulary index).
//
// Design (decode shapes are weight-bandwidth bound: every expert's weights
// are read from HBM exactly once per call):
//   * one workgroup = 4 wavefronts owns a slab of weight rows of one group
//     and ALL of that group's tokens (in passes of up to 128), so no weight
//     byte is fetched twice;
//   * each wavefront owns RT tiles of 16 weight rows; its A fragments come
//     straight from global memory (16 contiguous bytes per lane per 32-wide K
//     block) through a register ring kNB chunks deep, so HBM requests for
//     later K chunks are in flight while the current one is multiplied;
//   * the token operand (gathered rows of x, or the group's activation rows)
//     is staged through LDS in 64-wide K chunks, shared by the 4 wavefronts,
//     double-buffered through registers (the next chunk is fetched while the
//     current one is consumed); LDS rows are padded by 16 bytes so the
//     16-byte B-fragment reads of 16 rows hit distinct banks;
//   * every output element is a single fp32 accumulation over K in the same
//     block order whatever the token count, so a token's result does not
//     depend on its batch companions.
#include "launch.h"

namespace moev {
namespace {

enum Mode { kGateUp = 0, kDown = 1, kHead = 2 };

constexpr int kThreads = 256;
constexpr int kMaxTok = 128;  // tokens per pass: 8 MFMA column tiles
constexpr int kKC = 64;       // K elements per LDS chunk: 2 MFMA K blocks
constexpr int kNB = 4;        // weight ring depth in chunks
constexpr int kRtDown = 1;    // 16-row tiles per wave, down projection
constexpr int kRtHead = 2;    // 16-row tiles per wave, LM head

template <typename WT> struct Cfg {
  static constexpr int kEpv = 16 / sizeof(WT);                     // elements per 16 B
  static constexpr int kRowBytes = kKC * sizeof(WT) + 16;          // padded LDS row
  static constexpr int kVecPerRow = kKC * sizeof(WT) / 16;         // 16-B vectors per row
  static constexpr int kStage = kMaxTok * kVecPerRow / kThreads;   // vectors per thread
};

struct GemmArgs {
  const void* w0;           // [G, N, K] (gate/up: gate; down: w_down; head: w_lm)
  const void* w1;           // gate/up: up, else unused
  long long w_group;        // elements between consecutive groups
  int N, K;                 // weight rows per group, contraction length
  const void* x;            // operand rows
  const int32_t* offsets;   // [G+1] (gate/up, down)
  const int32_t* sorted_src;
  int S, k, P, T;           // slots, routed slots, pairs, tokens
  const float* topk_w;      // [T, k] (down)
  void* out;                // gate/up: act [P, N] WT; down: y [P, N] fp32; head: pmax
  int32_t* out_idx;         // head: partial arg max [blocks, T]
  float* logits;            // head: optional logits [T, N]
};

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

template <typename WT> __device__ __forceinline__ void store4(WT* p, f32x4 v);
template <> __device__ __forceinline__ void store4<u16>(u16* p, f32x4 v) {
  uint2 u;
  u.x = static_cast<uint32_t>(f32_to_bf16(v[0])) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
  u.y = static_cast<uint32_t>(f32_to_bf16(v[2])) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
  *reinterpret_cast<uint2*>(p) = u;
}
template <> __device__ __forceinline__ void store4<float>(float* p, f32x4 v) {
  *reinterpret_cast<f32x4*>(p) = v;
}

template <typename WT, int MODE, int RT>
__global__ __launch_bounds__(kThreads) void stream_gemm(GemmArgs a) {
  using C = Cfg<WT>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[kMaxTok * C::kRowBytes];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r16 = lane & 15;
  const int q = lane >> 4;

  int g = 0, off = 0, M;
  if (MODE == kHead) {
    M = a.T;
  } else {
    g = blockIdx.y;
    off = clampi(a.offsets[g], 0, a.P);
    M = clampi(a.offsets[g + 1], off, a.P) - off;
  }
  if (M <= 0) return;

  const WT* __restrict__ w0 = static_cast<const WT*>(a.w0);
  const WT* __restrict__ w1 = static_cast<const WT*>(a.w1);
  const WT* __restrict__ xsrc = static_cast<const WT*>(a.x);
  const int K = a.K;
  const int nchunks = K / kKC;

  // weight rows of this wave's tiles; lane pointer = row (rowbase + r16), k = 8q
  const WT* wp[RT];
  int rowbase[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int rb = (MODE == kGateUp) ? blockIdx.x * 64 + wave * 16
                                     : blockIdx.x * (64 * RT) + wave * (16 * RT) + rt * 16;
    rowbase[rt] = rb;
    const int row = min(rb + r16, a.N - 1);
    const WT* base = (MODE == kGateUp && rt == 1) ? w1 : w0;
    wp[rt] = base + static_cast<long long>(g) * a.w_group + static_cast<long long>(row) * K + q * 8;
  }

  for (int m0 = 0; m0 < M; m0 += kMaxTok) {
    const int mp = min(kMaxTok, M - m0);
    const int mt = (mp + 15) >> 4;

    // source rows for this thread's staging vectors
    const WT* src[C::kStage];
#pragma unroll
    for (int s = 0; s < C::kStage; ++s) {
      const int v = tid + s * kThreads;
      const int row = v / C::kVecPerRow;
      const int cv = v - row * C::kVecPerRow;
      src[s] = nullptr;
      if (row < mp) {
        long long xr;
        if (MODE == kGateUp) {
          const int p = clampi(a.sorted_src[off + m0 + row], 0, a.P - 1);
          xr = p / a.S;
        } else if (MODE == kDown) {
          xr = off + m0 + row;
        } else {
          xr = m0 + row;
        }
        src[s] = xsrc + xr * K + cv * C::kEpv;
      }
    }
    uint4 stage[C::kStage];
#pragma unroll
    for (int s = 0; s < C::kStage; ++s)
      stage[s] = src[s] ? *reinterpret_cast<const uint4*>(src[s]) : make_uint4(0, 0, 0, 0);

    f32x4 acc[RT][8];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[rt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    Frag<WT> ring[kNB][RT][2];
#pragma unroll
    for (int u = 0; u < kNB; ++u)
      if (u < nchunks)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) ring[u][rt][kk].load(wp[rt] + u * kKC + kk * 32);

    for (int c0 = 0; c0 < nchunks; c0 += kNB) {
#pragma unroll
      for (int u = 0; u < kNB; ++u) {
        const int c = c0 + u;
        if (c < nchunks) {
          __syncthreads();
#pragma unroll
          for (int s = 0; s < C::kStage; ++s) {
            const int v = tid + s * kThreads;
            const int row = v / C::kVecPerRow;
            const int cv = v - row * C::kVecPerRow;
            *reinterpret_cast<uint4*>(lds + row * C::kRowBytes + cv * 16) = stage[s];
          }
          __syncthreads();
          if (c + 1 < nchunks) {
#pragma unroll
            for (int s = 0; s < C::kStage; ++s)
              if (src[s]) stage[s] = *reinterpret_cast<const uint4*>(src[s] + (c + 1) * kKC);
          }
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              if (j < mt) {
                Frag<WT> b;
                b.load(reinterpret_cast<const WT*>(lds + (j * 16 + r16) * C::kRowBytes) + kk * 32 + q * 8);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) acc[rt][j] = mma(ring[u][rt][kk], b, acc[rt][j]);
              }
            }
          }
          if (c + kNB < nchunks) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
              for (int kk = 0; kk < 2; ++kk)
                ring[u][rt][kk].load(wp[rt] + (c + kNB) * kKC + kk * 32);
          }
        }
      }
    }

    // ------------------------------------------------------------ epilogues
    if (MODE == kGateUp) {
      WT* act = static_cast<WT*>(a.out);
      const int n = rowbase[0] + 4 * q;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int m = j * 16 + r16;
        if (j < mt && m < mp) {
          f32x4 gv = acc[0][j], uv = acc[1][j], o;
#pragma unroll
          for (int v = 0; v < 4; ++v) o[v] = gv[v] / (1.0f + expf(-gv[v])) * uv[v];
          store4<WT>(act + static_cast<long long>(off + m0 + m) * a.N + n, o);
        }
      }
    } else if (MODE == kDown) {
      float* y = static_cast<float*>(a.out);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int m = j * 16 + r16;
        if (j < mt && m < mp) {
          const int p = clampi(a.sorted_src[off + m0 + m], 0, a.P - 1);
          const int t = p / a.S;
          const int slot = p - t * a.S;
          const float wgt = slot < a.k ? a.topk_w[static_cast<long long>(t) * a.k + slot] : 1.0f;
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            f32x4 o = acc[rt][j];
#pragma unroll
            for (int v = 0; v < 4; ++v) o[v] *= wgt;
            store4<float>(y + static_cast<long long>(p) * a.N + rowbase[rt] + 4 * q, o);
          }
        }
      }
    } else {
      // per token column: best (value, vocab index) over this wave's rows
      __syncthreads();  // every wave is done reading the staged chunk
      float* red_v = reinterpret_cast<float*>(lds);                 // [4][128]
      int* red_i = reinterpret_cast<int*>(lds) + 4 * kMaxTok;       // [4][128]
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < mt) {
          const int m = j * 16 + r16;
          float best = -INFINITY;
          int bi = 0x7fffffff;
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int n = rowbase[rt] + 4 * q + v;
              if (n < a.N) {
                const float val = acc[rt][j][v];
                if (a.logits != nullptr && m < mp)
                  a.logits[static_cast<long long>(m0 + m) * a.N + n] = val;
                if (better(val, n, best, bi)) { best = val; bi = n; }
              }
            }
#pragma unroll
          for (int msk = 16; msk <= 32; msk <<= 1) {
            const float ov = __shfl_xor(best, msk, kWave);
            const int oi = __shfl_xor(bi, msk, kWave);
            if (better(ov, oi, best, bi)) { best = ov; bi = oi; }
          }
          if (q == 0) {
            red_v[wave * kMaxTok + m] = best;
            red_i[wave * kMaxTok + m] = bi;
          }
        }
      }
      __syncthreads();
      if (tid < mp) {
        float best = red_v[tid];
        int bi = red_i[tid];
#pragma unroll
        for (int w = 1; w < 4; ++w) {
          const float ov = red_v[w * kMaxTok + tid];
          const int oi = red_i[w * kMaxTok + tid];
          if (better(ov, oi, best, bi)) { best = ov; bi = oi; }
        }
        const long long o = static_cast<long long>(blockIdx.x) * a.T + m0 + tid;
        static_cast<float*>(a.out)[o] = best;
        a.out_idx[o] = bi;
      }
    }
  }
}

// Final RMSNorm of the head input, rounded to the operand type.
template <typename WT>
__global__ __launch_bounds__(256) void norm_cast_kernel(const float* __restrict__ h,
                                                        const WT* __restrict__ gamma, float eps,
                                                        int T, int H, WT* __restrict__ xo) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  const float* hr = h + static_cast<long long>(t) * H;
  float ss = 0.f;
  for (int i = lane * 4; i < H; i += 256) {
    float4 v = *reinterpret_cast<const float4*>(hr + i);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / static_cast<float>(H) + eps);
  for (int i = lane * 4; i < H; i += 256) {
    float4 v = *reinterpret_cast<const float4*>(hr + i);
    f32x4 o;
    o[0] = v.x * r * (gamma ? to_f32<WT>(gamma[i + 0]) : 1.f);
    o[1] = v.y * r * (gamma ? to_f32<WT>(gamma[i + 1]) : 1.f);
    o[2] = v.z * r * (gamma ? to_f32<WT>(gamma[i + 2]) : 1.f);
    o[3] = v.w * r * (gamma ? to_f32<WT>(gamma[i + 3]) : 1.f);
    store4<WT>(xo + static_cast<long long>(t) * H + i, o);
  }
}

// Second pass of the blocked arg max: one wavefront per token.
__global__ __launch_bounds__(64) void argmax_reduce_kernel(const float* __restrict__ pmax,
                                                           const int32_t* __restrict__ pidx,
                                                           int nblk, int T,
                                                           int32_t* __restrict__ argmax_out,
                                                           float* __restrict__ max_out) {
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  for (int b = lane; b < nblk; b += 64) {
    const float v = pmax[static_cast<long long>(b) * T + t];
    const int i = pidx[static_cast<long long>(b) * T + t];
    if (better(v, i, best, bi)) { best = v; bi = i; }
  }
  wave_argmax(best, bi);
  if (lane == 0) {
    argmax_out[t] = bi;
    if (max_out) max_out[t] = best;
  }
}

template <typename WT, int MODE, int RT>
void launch_gemm(const GemmArgs& args, dim3 grid, hipStream_t s) {
  stream_gemm<WT, MODE, RT><<<grid, kThreads, 0, s>>>(args);
}

int head_blocks(int V) { return (V + 64 * kRtHead - 1) / (64 * kRtHead); }

size_t esize(int dt) { return dt == MOEV_BF16 ? 2 : 4; }

moev_status check_inter(int I) {
  MOEV_REQUIRE(I >= 64 && I <= 8192 && I % 64 == 0, MOEV_ERR_UNSUPPORTED,
               "intermediate size %d must be a multiple of 64 in [64, 8192]", I);
  return MOEV_OK;
}

moev_status check_hid(int H) {
  MOEV_REQUIRE(H >= 64 && H <= 4032 && H % 64 == 0, MOEV_ERR_UNSUPPORTED,
               "hidden size %d must be a multiple of 64 in [64, 4032]", H);
  return MOEV_OK;
}

}  // namespace

size_t grouped_ffn_ws_bytes(int T, int I, int k, int ns, int dt) {
  return align_up(static_cast<size_t>(T) * (k + ns) * I * esize(dt), 256);
}

size_t lmhead_ws_bytes(int T, int H, int V, int dt) {
  const size_t xf = align_up(static_cast<size_t>(T) * H * esize(dt), 256);
  const size_t part = align_up(static_cast<size_t>(head_blocks(V)) * T * 4, 256);
  return xf + 2 * part;
}

void launch_grouped_ffn(const void* x, const int32_t* sorted_src, const int32_t* offsets,
                        const float* topk_w, const void* w_gate, const void* w_up,
                        const void* w_down, int T, int H, int I, int E, int k, int ns, int dt,
                        float* y_slots, void* ws, hipStream_t s) {
  const int G = E + ns;
  GemmArgs up{};
  up.w0 = w_gate;
  up.w1 = w_up;
  up.w_group = static_cast<long long>(I) * H;
  up.N = I;
  up.K = H;
  up.x = x;
  up.offsets = offsets;
  up.sorted_src = sorted_src;
  up.S = k + ns;
  up.k = k;
  up.P = T * (k + ns);
  up.T = T;
  up.out = ws;
  GemmArgs dn = up;
  dn.w0 = w_down;
  dn.w1 = nullptr;
  dn.N = H;
  dn.K = I;
  dn.x = ws;
  dn.topk_w = topk_w;
  dn.out = y_slots;
  const dim3 gu(I / 64, G), gd(H / (64 * kRtDown), G);
  if (dt == MOEV_BF16) {
    launch_gemm<u16, kGateUp, 2>(up, gu, s);
    launch_gemm<u16, kDown, kRtDown>(dn, gd, s);
  } else {
    launch_gemm<float, kGateUp, 2>(up, gu, s);
    launch_gemm<float, kDown, kRtDown>(dn, gd, s);
  }
}

void launch_lmhead(const float* h, const void* norm_f, float eps, const void* w_lm, int T, int H,
                   int V, int dt, int32_t* argmax_out, float* max_out, float* logits_out,
                   void* ws, hipStream_t s) {
  const size_t xf_bytes = align_up(static_cast<size_t>(T) * H * esize(dt), 256);
  const int nblk = head_blocks(V);
  const size_t part = align_up(static_cast<size_t>(nblk) * T * 4, 256);
  unsigned char* base = static_cast<unsigned char*>(ws);
  void* xf = base;
  float* pmax = reinterpret_cast<float*>(base + xf_bytes);
  int32_t* pidx = reinterpret_cast<int32_t*>(base + xf_bytes + part);
  GemmArgs hd{};
  hd.w0 = w_lm;
  hd.w_group = 0;
  hd.N = V;
  hd.K = H;
  hd.x = xf;
  hd.T = T;
  hd.out = pmax;
  hd.out_idx = pidx;
  hd.logits = logits_out;
  const int nb = (T + 3) / 4;
  if (dt == MOEV_BF16) {
    norm_cast_kernel<u16><<<nb, 256, 0, s>>>(h, static_cast<const u16*>(norm_f), eps, T, H,
                                              static_cast<u16*>(xf));
    launch_gemm<u16, kHead, kRtHead>(hd, dim3(nblk), s);
  } else {
    norm_cast_kernel<float><<<nb, 256, 0, s>>>(h, static_cast<const float*>(norm_f), eps, T, H,
                                                static_cast<float*>(xf));
    launch_gemm<float, kHead, kRtHead>(hd, dim3(nblk), s);
  }
  argmax_reduce_kernel<<<T, 64, 0, s>>>(pmax, pidx, nblk, T, argmax_out, max_out);
}

moev_status validate_grouped_ffn(const void* x, const int32_t* sorted_src, const int32_t* offsets,
                                 const float* topk_w, const void* w_gate, const void* w_up,
                                 const void* w_down, int T, int H, int I, int E, int k, int ns,
                                 int dt, const float* y_slots, const void* ws, size_t ws_bytes) {
  MOEV_CHECK(check_dtype(dt), MOEV_ERR_UNSUPPORTED);
  if (moev_status st = check_hid(H)) return st;
  if (moev_status st = check_inter(I)) return st;
  MOEV_REQUIRE(T >= 0, MOEV_ERR_INVALID_ARG, "T must be >= 0 (got %d)", T);
  MOEV_REQUIRE(E >= 1 && E <= 64, MOEV_ERR_UNSUPPORTED, "routed experts E=%d must be in [1, 64]", E);
  MOEV_REQUIRE(k >= 1 && k <= E, MOEV_ERR_UNSUPPORTED, "top-k k=%d must be in [1, E=%d]", k, E);
  MOEV_REQUIRE(ns >= 0 && ns <= 8, MOEV_ERR_UNSUPPORTED, "shared experts ns=%d must be in [0, 8]", ns);
  MOEV_REQUIRE(static_cast<long long>(T) * (k + ns) < (1ll << 31), MOEV_ERR_UNSUPPORTED,
               "T*(k+ns) must be < 2^31");
  if (T == 0) return MOEV_OK;
  MOEV_CHECK(need_ptr(x, "x") && need_ptr(sorted_src, "sorted_src") &&
                 need_ptr(offsets, "group_offsets") && need_ptr(topk_w, "topk_w") &&
                 need_ptr(w_gate, "w_gate") && need_ptr(w_up, "w_up") &&
                 need_ptr(w_down, "w_down") && need_ptr(y_slots, "y_slots"),
             MOEV_ERR_INVALID_ARG);
  MOEV_REQUIRE(ws != nullptr && aligned16(ws), MOEV_ERR_WORKSPACE,
               "workspace must be non-NULL and 16-byte aligned");
  const size_t need = grouped_ffn_ws_bytes(T, I, k, ns, dt);
  MOEV_REQUIRE(ws_bytes >= need, MOEV_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu",
               ws_bytes, need);
  return MOEV_OK;
}

moev_status validate_lmhead(const float* h, const void* norm_f, const void* w_lm, int T, int H,
                            int V, int dt, const int32_t* argmax_out, const float* max_out,
                            const float* logits_out, const void* ws, size_t ws_bytes) {
  MOEV_CHECK(check_dtype(dt), MOEV_ERR_UNSUPPORTED);
  if (moev_status st = check_hid(H)) return st;
  MOEV_REQUIRE(T >= 0, MOEV_ERR_INVALID_ARG, "T must be >= 0 (got %d)", T);
  MOEV_REQUIRE(V >= 1, MOEV_ERR_INVALID_ARG, "vocabulary V must be >= 1 (got %d)", V);
  if (T == 0) return MOEV_OK;
  MOEV_CHECK(need_ptr(h, "h") && opt_ptr(norm_f, "norm_f") && need_ptr(w_lm, "w_lm") &&
                 need_ptr(argmax_out, "argmax_out") && opt_ptr(max_out, "max_out") &&
                 opt_ptr(logits_out, "logits_out"),
             MOEV_ERR_INVALID_ARG);
  MOEV_REQUIRE(ws != nullptr && aligned16(ws), MOEV_ERR_WORKSPACE,
               "workspace must be non-NULL and 16-byte aligned");
  const size_t need = lmhead_ws_bytes(T, H, V, dt);
  MOEV_REQUIRE(ws_bytes >= need, MOEV_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu",
               ws_bytes, need);
  return MOEV_OK;
}

}  // namespace moev

extern "C" size_t moe_grouped_ffn_workspace_size(int T, int I, int k, int ns, int dt) {
  if (T < 0 || I < 0 || k < 0 || ns < 0) return 0;
  return moev::grouped_ffn_ws_bytes(T, I, k, ns, dt);
}

extern "C" moev_status moe_grouped_ffn(const void* x, const int32_t* sorted_src,
                                       const int32_t* group_offsets, const float* topk_w,
                                       const void* w_gate, const void* w_up, const void* w_down,
                                       int T, int H, int I, int E, int k, int ns, int dt,
                                       float* y_slots, void* ws, size_t ws_bytes, void* stream) {
  if (moev_status st = moev::validate_grouped_ffn(x, sorted_src, group_offsets, topk_w, w_gate,
                                                  w_up, w_down, T, H, I, E, k, ns, dt, y_slots,
                                                  ws, ws_bytes))
    return st;
  if (T == 0) return MOEV_OK;
  moev::launch_grouped_ffn(x, sorted_src, group_offsets, topk_w, w_gate, w_up, w_down, T, H, I, E,
                           k, ns, dt, y_slots, ws, moev::as_stream(stream));
  return moev::launch_status("moe_grouped_ffn");
}

extern "C" size_t lmhead_argmax_workspace_size(int T, int H, int V, int dt) {
  if (T < 0 || H < 0 || V < 1) return 0;
  return moev::lmhead_ws_bytes(T, H, V, dt);
}

extern "C" moev_status lmhead_argmax(const float* h, const void* norm_f, float eps,
                                     const void* w_lm, int T, int H, int V, int dt,
                                     int32_t* argmax_out, float* max_out, float* logits_out,
                                     void* ws, size_t ws_bytes, void* stream) {
  if (moev_status st = moev::validate_lmhead(h, norm_f, w_lm, T, H, V, dt, argmax_out, max_out,
                                             logits_out, ws, ws_bytes))
    return st;
  if (T == 0) return MOEV_OK;
  moev::launch_lmhead(h, norm_f, eps, w_lm, T, H, V, dt, argmax_out, max_out, logits_out, ws,
                      moev::as_stream(stream));
  return moev::launch_status("lmhead_argmax");
}
