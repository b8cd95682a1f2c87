// Expert sort of the (token, slot) pairs as its own kernel (one workgroup);
// the algorithm is in permute_body.h.
#include "launch.h"
#include "permute_body.h"

namespace moev {
namespace {

__global__ __launch_bounds__(kPermThreads) void permute_kernel(const int32_t* __restrict__ idx,
                                                               int T, int k, int E, int ns,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ sorted_src) {
  permute_block([idx](int q) { return idx[q]; }, T, k, E, ns, offsets, sorted_src);
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
