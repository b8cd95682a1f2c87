// Expert sort of the (token, slot) pairs: histogram -> exclusive prefix sum
// -> stable scatter, in one workgroup of 1024 threads with the bookkeeping in
// LDS.  Only the T*k routed pairs need sorting; each shared expert holds every
// token in order, so its segment is written directly.
//
// Stable scatter of one 1024-pair chunk (pairs in increasing id order):
//   * within a wavefront, lanes with the same expert find each other with
//     ballots over the expert-id bits; a lane's rank is the number of
//     matching lower lanes;
//   * the per-wave counts go to an LDS table [16 waves][64 experts]; one
//     thread per expert turns its column into running bases (in wave order)
//     and advances the expert's cursor;
//   * position = cursor base for (wave, expert) + rank.
// Integer work only, so the result is exact and identical on every run.
#include "launch.h"

namespace moev {
namespace {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / kWave;

__global__ __launch_bounds__(kPermThreads) void permute_kernel(const int32_t* __restrict__ idx,
                                                               int T, int k, int E, int ns,
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
    int g = idx[q];
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
      g = idx[q];
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

  const int shared_base = n_routed_pairs;
  for (int i = tid; i < T * ns; i += kPermThreads) {
    const int s = i / T;
    const int t = i - s * T;
    sorted_src[shared_base + i] = t * S + k + s;
  }
}

}  // namespace

void launch_permute(const int32_t* topk_idx, int T, int k, int E, int ns, int32_t* offsets,
                    int32_t* sorted_src, hipStream_t s) {
  permute_kernel<<<1, kPermThreads, 0, s>>>(topk_idx, T, k, E, ns, offsets, sorted_src);
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
