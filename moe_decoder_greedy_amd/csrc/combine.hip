// Residual combine of the expert slots and the FastMTP prefix-accept step.
//
// Combine: each token's slot outputs (routed by rank, then shared, each
// already scaled by its router weight) are added left to right in fp32 and
// then added to the residual stream -- a fixed order, no atomics, so the sum
// is reproducible bit for bit.
//
// Verify ("The speed comes from three layers working together" and "Why
// FastMTP fits OCR particularly well", Jina-OCR-v1 explainer on
// kg.zhiyong.dev; "Scope & Claims", Section 3.1 / Eq. 2, evolve.pub review):
// drafts are accepted while each equals the main model's greedy token at the
// previous position; the main model's token at the first disagreement (or
// after the last draft) is committed as well.
#include "launch.h"

namespace moev {
namespace {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const float* h_in, int T, int H4, int S,
                                                      float* h_out) {
  const long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<long long>(T) * H4) return;
  const long long t = i / H4;
  const long long c = i - t * H4;
  const float4* ys = reinterpret_cast<const float4*>(y) + t * S * H4 + c;
  float4 acc = ys[0];
  for (int s = 1; s < S; ++s) {
    const float4 v = ys[static_cast<long long>(s) * H4];
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  if (h_in != nullptr) {
    const float4 hv = reinterpret_cast<const float4*>(h_in)[i];
    acc.x = hv.x + acc.x;
    acc.y = hv.y + acc.y;
    acc.z = hv.z + acc.z;
    acc.w = hv.w + acc.w;
  }
  reinterpret_cast<float4*>(h_out)[i] = acc;
}

__global__ __launch_bounds__(256) void verify_kernel(const int32_t* __restrict__ tokens,
                                                     const int32_t* __restrict__ greedy, int B,
                                                     int K, int32_t* __restrict__ n_accept,
                                                     int32_t* __restrict__ commit,
                                                     int32_t* __restrict__ commit_len,
                                                     int32_t* __restrict__ next_last) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int32_t* tk = tokens + static_cast<long long>(b) * (K + 1);
  const int32_t* gr = greedy + static_cast<long long>(b) * (K + 1);
  const int n = accept_prefix(tk, gr, K, commit + static_cast<long long>(b) * (K + 1));
  n_accept[b] = n;
  if (commit_len) commit_len[b] = n + 1;
  if (next_last) next_last[b] = gr[n];
}

}  // namespace

__global__ __launch_bounds__(256) void gather_last_kernel(const float* __restrict__ h,
                                                          const float* __restrict__ y, int S, int H4,
                                                          int seq_len, float* __restrict__ out) {
  const long long t = static_cast<long long>(blockIdx.x) * seq_len + seq_len - 1;
  for (int c = threadIdx.x; c < H4; c += blockDim.x) {
    float4 v = reinterpret_cast<const float4*>(h)[t * H4 + c];
    if (y != nullptr) {
      const float4* ys = reinterpret_cast<const float4*>(y) + t * S * H4 + c;
      float4 acc = ys[0];
      for (int sl = 1; sl < S; ++sl) {
        const float4 w = ys[static_cast<long long>(sl) * H4];
        acc.x += w.x;
        acc.y += w.y;
        acc.z += w.z;
        acc.w += w.w;
      }
      v = make_float4(v.x + acc.x, v.y + acc.y, v.z + acc.z, v.w + acc.w);
    }
    reinterpret_cast<float4*>(out)[static_cast<long long>(blockIdx.x) * H4 + c] = v;
  }
}

void launch_gather_last(const float* h, const float* y, int S, int H, int n_seq, int seq_len,
                        float* out, hipStream_t s) {
  if (n_seq > 0) gather_last_kernel<<<n_seq, 256, 0, s>>>(h, y, S, H / 4, seq_len, out);
}

void launch_combine(const float* y, const float* h_in, int T, int H, int S, float* h_out,
                    hipStream_t s) {
  const long long n = static_cast<long long>(T) * (H / 4);
  const int blocks = static_cast<int>((n + 255) / 256);
  combine_kernel<<<blocks, 256, 0, s>>>(y, h_in, T, H / 4, S, h_out);
}

void launch_verify(const int32_t* tokens, const int32_t* greedy, int B, int K, int32_t* n_accept,
                   int32_t* commit, int32_t* commit_len, int32_t* next_last, hipStream_t s) {
  verify_kernel<<<(B + 255) / 256, 256, 0, s>>>(tokens, greedy, B, K, n_accept, commit,
                                                 commit_len, next_last);
}

moev_status validate_combine(const float* y, const float* h_in, int T, int H, int S,
                             const float* h_out) {
  MOEV_REQUIRE(T >= 0, MOEV_ERR_INVALID_ARG, "T must be >= 0 (got %d)", T);
  MOEV_REQUIRE(H >= 4 && H % 4 == 0, MOEV_ERR_UNSUPPORTED, "H=%d must be a positive multiple of 4", H);
  MOEV_REQUIRE(S >= 1 && S <= 72, MOEV_ERR_UNSUPPORTED, "slots S=%d must be in [1, 72]", S);
  if (T == 0) return MOEV_OK;
  MOEV_CHECK(need_ptr(y, "y_slots") && opt_ptr(h_in, "h_in") && need_ptr(h_out, "h_out"),
             MOEV_ERR_INVALID_ARG);
  return MOEV_OK;
}

moev_status validate_verify(const int32_t* tokens, const int32_t* greedy, int B, int K,
                            const int32_t* n_accept, const int32_t* commit) {
  MOEV_REQUIRE(B >= 0 && K >= 0, MOEV_ERR_INVALID_ARG, "need B >= 0 and K >= 0 (B=%d K=%d)", B, K);
  MOEV_REQUIRE(K <= 64, MOEV_ERR_UNSUPPORTED, "K=%d drafts exceeds 64", K);
  if (B == 0) return MOEV_OK;
  MOEV_CHECK(need_ptr(tokens, "tokens", 4) && need_ptr(greedy, "greedy", 4) &&
                 need_ptr(n_accept, "n_accept", 4) && need_ptr(commit, "commit", 4),
             MOEV_ERR_INVALID_ARG);
  return MOEV_OK;
}

}  // namespace moev

extern "C" moev_status moe_combine(const float* y_slots, const float* h_in, int T, int H, int S,
                                   float* h_out, void* stream) {
  if (moev_status st = moev::validate_combine(y_slots, h_in, T, H, S, h_out)) return st;
  if (T == 0) return MOEV_OK;
  moev::launch_combine(y_slots, h_in, T, H, S, h_out, moev::as_stream(stream));
  return moev::launch_status("moe_combine");
}

extern "C" moev_status mtp_verify(const int32_t* tokens, const int32_t* greedy, int B, int K,
                                  int32_t* n_accept, int32_t* commit, int32_t* commit_len,
                                  int32_t* next_last, void* stream) {
  if (moev_status st = moev::validate_verify(tokens, greedy, B, K, n_accept, commit)) return st;
  if (B == 0) return MOEV_OK;
  moev::launch_verify(tokens, greedy, B, K, n_accept, commit, commit_len, next_last,
                      moev::as_stream(stream));
  return moev::launch_status("mtp_verify");
}
