// Expert sort of the (token, slot) pairs: a stable counting sort by expert
// group, integer work only, so the result is exact and identical on every run.
//
// Workgroup c owns routed pairs [c*C, (c+1)*C) (C = kPermChunk).  Every
// workgroup histograms all routed pairs (for the group offsets) and the pairs
// before its chunk (for where its own pairs of each group start), counting
// with ballots over the expert-id bits rather than atomics.  Then
// it scatters its chunk in pair order: rank within the wavefront from the
// ballots, per-wave counts into an LDS table [waves][64 experts], one thread
// per expert turning its column into running bases in wave order.  Each
// shared expert holds every token in order, so its segment is written
// directly, spread over the workgroups.  The histograms are recomputed by
// every workgroup rather than exchanged: no workspace and no waiting between
// workgroups.
#include "launch.h"

namespace moev {
namespace {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / kWave;
constexpr int kPermChunk = 2048;  // routed pairs per workgroup (multiple of kPermThreads)
constexpr int kHistUnroll = 16;   // ids in flight per thread while counting

__device__ __forceinline__ int clamp_expert(int g, int E) { return g < 0 ? 0 : (g >= E ? E - 1 : g); }

// Lanes of this wavefront holding the same 7-bit key as this lane.
__device__ __forceinline__ unsigned long long same_key(int g) {
  unsigned long long match = ~0ull;
#pragma unroll
  for (int b = 0; b < 7; ++b) {
    const bool bit = (g >> b) & 1;
    const unsigned long long bal = __ballot(bit);
    match &= bit ? bal : ~bal;
  }
  return match;
}

__global__ __launch_bounds__(kPermThreads) void permute_kernel(const int32_t* __restrict__ idx, int T,
                                                               int k, int E, int ns,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ sorted_src) {
  __shared__ int cnt_all[64];
  __shared__ int cnt_before[64];
  __shared__ int base[64];
  __shared__ int wcnt[kPermWaves][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int S = k + ns;
  const int n = T * k;
  const int q0 = blockIdx.x * kPermChunk;
  const int q1 = min(n, q0 + kPermChunk);
  const unsigned long long lower = (1ull << lane) - 1ull;

  // Histograms without atomics: after the ballots over the id bits of 64
  // pairs, lane e forms the mask of lanes holding expert e and adds its
  // population count to a register; per-wave counts are summed through LDS.
  // kHistUnroll ids per thread are requested before any is counted.  A
  // wavefront's 64 pairs all lie before q0 or none does (q0 and the first
  // pair of a wavefront are multiples of 64).
  {
    int my_all = 0, my_before = 0;
    for (int c0 = 0; c0 < n; c0 += kHistUnroll * kPermThreads) {
      int g[kHistUnroll];
#pragma unroll
      for (int j = 0; j < kHistUnroll; ++j) {
        const int q = c0 + j * kPermThreads + tid;
        g[j] = q < n ? clamp_expert(idx[q], E) : 127;  // 127: no pair, never a lane's expert
      }
#pragma unroll
      for (int j = 0; j < kHistUnroll; ++j) {
        if (c0 + j * kPermThreads >= n) break;  // uniform: no pairs left
        unsigned long long m = ~0ull;
#pragma unroll
        for (int b = 0; b < 7; ++b) {
          const unsigned long long bal = __ballot((g[j] >> b) & 1);
          m &= ((lane >> b) & 1) ? bal : ~bal;
        }
        const int c = __popcll(m);
        my_all += c;
        if (c0 + j * kPermThreads + wave * kWave < q0) my_before += c;
      }
    }
    wcnt[wave][lane] = my_all;
    __syncthreads();
    if (tid < 64) {
      int s = 0;
#pragma unroll
      for (int w = 0; w < kPermWaves; ++w) s += wcnt[w][tid];
      cnt_all[tid] = s;
    }
    __syncthreads();
    if (gridDim.x > 1) {  // one workgroup: nothing lies before its chunk
      wcnt[wave][lane] = my_before;
      __syncthreads();
      if (tid < 64) {
        int s = 0;
#pragma unroll
        for (int w = 0; w < kPermWaves; ++w) s += wcnt[w][tid];
        cnt_before[tid] = s;
      }
      __syncthreads();
    } else if (tid < 64) {
      cnt_before[tid] = 0;
    }
  }
  // group offsets: exclusive prefix sum over the experts, one lane each
  if (wave == 0) {
    const int c = lane < E ? cnt_all[lane] : 0;
    int incl = c;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d);
      if (lane >= d) incl += v;
    }
    const int excl = incl - c;
    const int total = __shfl(incl, 63);
    if (lane < E) {
      base[lane] = excl + cnt_before[lane];
      if (blockIdx.x == 0) offsets[lane] = excl;
    }
    if (blockIdx.x == 0 && lane <= ns) offsets[E + lane] = total + lane * T;
  }
  __syncthreads();

  for (int c0 = q0; c0 < q1; c0 += kPermThreads) {
    const int q = c0 + tid;
    const bool valid = q < q1;
    const int g = valid ? clamp_expert(idx[q], E) : 127;
    const unsigned long long match = same_key(g);
    const int rank = __popcll(match & lower);
    const int wave_count = __popcll(match);

    wcnt[wave][lane] = 0;
    __syncthreads();
    if (valid && rank == 0) wcnt[wave][g] = wave_count;
    __syncthreads();
    if (tid < E) {
      int c[kPermWaves];
#pragma unroll
      for (int w = 0; w < kPermWaves; ++w) c[w] = wcnt[w][tid];
      int run = base[tid];
#pragma unroll
      for (int w = 0; w < kPermWaves; ++w) {
        wcnt[w][tid] = run;
        run += c[w];
      }
      base[tid] = run;
    }
    __syncthreads();
    if (valid) {
      const int t = q / k;
      const int r = q - t * k;
      sorted_src[wcnt[wave][g] + rank] = t * S + r;
    }
    __syncthreads();
  }

  const int stride = gridDim.x * kPermThreads;
  for (int i = blockIdx.x * kPermThreads + tid; i < T * ns; i += stride) {
    const int s = i / T;
    const int t = i - s * T;
    sorted_src[n + i] = t * S + k + s;
  }
}

}  // namespace

void launch_permute(const int32_t* topk_idx, int T, int k, int E, int ns, int32_t* offsets,
                    int32_t* sorted_src, hipStream_t s) {
  const int n = T * k;
  const int grid = n > 0 ? (n + kPermChunk - 1) / kPermChunk : 1;
  permute_kernel<<<grid, kPermThreads, 0, s>>>(topk_idx, T, k, E, ns, offsets, sorted_src);
}

moev_status validate_permute(const int32_t* topk_idx, int T, int k, int E, int ns,
                             const int32_t* offsets, const int32_t* sorted_src) {
  MOEV_REQUIRE(T >= 0, MOEV_ERR_INVALID_ARG, "T must be >= 0 (got %d)", T);
  MOEV_REQUIRE(E >= 1 && E <= 64, MOEV_ERR_UNSUPPORTED, "routed experts E=%d must be in [1, 64]", E);
  MOEV_REQUIRE(k >= 1 && k <= E, MOEV_ERR_UNSUPPORTED, "top-k k=%d must be in [1, E=%d]", k, E);
  MOEV_REQUIRE(ns >= 0 && ns <= 8, MOEV_ERR_UNSUPPORTED, "shared experts ns=%d must be in [0, 8]", ns);
  MOEV_REQUIRE(static_cast<long long>(T) * (k + ns) < (1ll << 31), MOEV_ERR_UNSUPPORTED,
               "T*(k+ns) must be < 2^31");
  MOEV_CHECK(need_ptr(offsets, "group_offsets", 4), MOEV_ERR_INVALID_ARG);
  if (T == 0) return MOEV_OK;
  MOEV_CHECK(need_ptr(topk_idx, "topk_idx", 4) && need_ptr(sorted_src, "sorted_src", 4),
             MOEV_ERR_INVALID_ARG);
  return MOEV_OK;
}

}  // namespace moev

extern "C" moev_status moe_permute(const int32_t* topk_idx, int T, int k, int E, int ns,
                                   int32_t* group_offsets, int32_t* sorted_src, void* stream) {
  if (moev_status st = moev::validate_permute(topk_idx, T, k, E, ns, group_offsets, sorted_src))
    return st;
  // T == 0 still writes the (all-zero) offsets so callers can rely on them.
  moev::launch_permute(topk_idx, T, k, E, ns, group_offsets, sorted_src, moev::as_stream(stream));
  return moev::launch_status("moe_permute");
}
