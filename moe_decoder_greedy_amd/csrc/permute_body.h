// Stable counting sort of the (token, slot) pairs by expert group, executed
// by one workgroup of kPermThreads threads.  Shared by the stand-alone
// permute kernel and the router's last workgroup.
//
//   histogram of the T*k routed pairs in LDS -> exclusive prefix sum ->
//   scatter in pair order: within a wavefront, lanes with the same expert find
//   each other with ballots over the expert-id bits (rank = matching lower
//   lanes); per-wave counts go to an LDS table [waves][64 experts]; one thread
//   per expert turns its column into running bases in wave order.
// Each shared expert holds every token in order, so its segment is written
// directly.  Integer work only: the result is exact and identical on every run.
#pragma once

#include "common.h"

namespace moev {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / kWave;

// LOAD reads topk_idx[q] (plain, or coherent across workgroups).
template <typename LOAD>
__device__ __forceinline__ void permute_block(LOAD load_idx, int T, int k, int E, int ns,
                                              int32_t* __restrict__ offsets,
                                              int32_t* __restrict__ sorted_src) {
  __shared__ int cnt[64];
  __shared__ int base[64];
  __shared__ int wcnt[kPermWaves][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int S = k + ns;
  const int n_routed_pairs = T * k;

  if (tid < 64) cnt[tid] = 0;
  __syncthreads();
  for (int q = tid; q < n_routed_pairs; q += kPermThreads) {
    int g = load_idx(q);
    g = g < 0 ? 0 : (g >= E ? E - 1 : g);
    atomicAdd(&cnt[g], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int g = 0; g < E; ++g) {
      base[g] = run;
      offsets[g] = run;
      run += cnt[g];
    }
    for (int s = 0; s <= ns; ++s) offsets[E + s] = run + s * T;
  }
  __syncthreads();

  const unsigned long long lower = (1ull << lane) - 1ull;
  for (int c0 = 0; c0 < n_routed_pairs; c0 += kPermThreads) {
    const int q = c0 + tid;
    const bool valid = q < n_routed_pairs;
    int g = 127;  // sentinel: never equal to a real expert id
    if (valid) {
      g = load_idx(q);
      g = g < 0 ? 0 : (g >= E ? E - 1 : g);
    }
    unsigned long long match = ~0ull;
#pragma unroll
    for (int b = 0; b < 7; ++b) {
      const bool bit = (g >> b) & 1;
      const unsigned long long bal = __ballot(bit);
      match &= bit ? bal : ~bal;
    }
    const int rank = __popcll(match & lower);
    const int wave_count = __popcll(match);

    wcnt[wave][lane] = 0;
    __syncthreads();
    if (valid && rank == 0) wcnt[wave][g] = wave_count;
    __syncthreads();
    if (tid < E) {
      int run = base[tid];
      for (int w = 0; w < kPermWaves; ++w) {
        const int c = wcnt[w][tid];
        wcnt[w][tid] = run;
        run += c;
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

  for (int i = tid; i < T * ns; i += kPermThreads) {
    const int s = i / T;
    const int t = i - s * T;
    sorted_src[n_routed_pairs + i] = t * S + k + s;
  }
}

}  // namespace moev
