// FastMTP draft block: K recursive applications of one dense block on the
// device ("The speed comes from three layers working together" on
// kg.zhiyong.dev: one dense draft block proposes up to three tokens by being
// applied recursively; the aipolix.com page, "A document parser, not just a
// text recognizer": a shared block drafts three positions).
//
// Step j, from the hidden state z and token t of step j-1:
//   u   = [RMSNorm(z) * norm_z ; RMSNorm(Emb[t]) * norm_e]
//   z'  = W_p u
//   z_j = z' + W_down (SiLU(W_gate x) * (W_up x)),  x = RMSNorm(z') * norm_ffn
//   t_j = arg max W_lm (RMSNorm(z_j) * norm_out)
//
// Every contraction runs on the grouped expert GEMMs in token-set mode: the
// projection is the down GEMM over 2 groups (the z half and the embedding half
// of W_p, each holding every row, weight 1), summed in group order; the dense
// SwiGLU of width n*I is the grouped FFN over its n intermediate slices, each
// holding every row, again summed in slice order.  These GEMMs span only 2 or
// n groups, so each runs split K (a workgroup's four waves take a quarter of
// the contraction each and add in wave order).  Every sum order is fixed, so
// a row's draft does not depend on the batch.  Per step: one input kernel,
// the projection GEMM, one norm kernel (z' and x), gate/up, down, and the LM
// head, whose norm kernel also forms z_j = z' + the slice sum.
#include "launch.h"

namespace moev {
namespace {

constexpr int kDraftThreads = 128;  // wave 0: the hidden-state half, wave 1: the embedding half

template <typename WT> __device__ __forceinline__ float4 load4(const WT* p);
template <> __device__ __forceinline__ float4 load4<u16>(const u16* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(bf16_to_f32(u.x & 0xFFFF), bf16_to_f32(u.x >> 16), bf16_to_f32(u.y & 0xFFFF),
                     bf16_to_f32(u.y >> 16));
}
template <> __device__ __forceinline__ float4 load4<float>(const float* p) {
  return *reinterpret_cast<const float4*>(p);
}

struct DraftInArgs {
  const float* z;           // hidden states, fp32 rows of H
  const int32_t* n_accept;  // row map: row b*K1 + n_accept[b] of z (NULL: row b)
  int K1;
  const int32_t* tok;       // token of row b at tok[b * tok_stride]
  int tok_stride;
  int32_t* tok_copy;        // optional: tok_copy[b * copy_stride] = that token
  int copy_stride;
  const void* emb;
  int V, B, H;
  const void* norm_z;
  const void* norm_e;
  float eps;
  void* x2;                 // [2][B][H] operand rows of the projection
};

// Block b: wave 0 normalises z's row, wave 1 the embedding row of the token.
template <typename WT>
__global__ __launch_bounds__(kDraftThreads) void draft_in_kernel(DraftInArgs a) {
  const int b = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int H = a.H;
  const int raw = a.tok[static_cast<long long>(b) * a.tok_stride];
  if (a.tok_copy != nullptr && threadIdx.x == 0) a.tok_copy[static_cast<long long>(b) * a.copy_stride] = raw;
  const int t = raw < 0 ? 0 : (raw >= a.V ? a.V - 1 : raw);

  const WT* gamma = static_cast<const WT*>(wave == 0 ? a.norm_z : a.norm_e);
  const float* zr = nullptr;
  const WT* er = nullptr;
  if (wave == 0) {
    long long row = b;
    if (a.n_accept != nullptr) {
      int n = a.n_accept[b];
      n = n < 0 ? 0 : (n >= a.K1 ? a.K1 - 1 : n);
      row = static_cast<long long>(b) * a.K1 + n;
    }
    zr = a.z + row * H;
  } else {
    er = static_cast<const WT*>(a.emb) + static_cast<long long>(t) * H;
  }
  auto value = [&](int i) { return wave == 0 ? *reinterpret_cast<const float4*>(zr + i) : load4<WT>(er + i); };
  float ss = 0.f;
  for (int i = lane * 4; i < H; i += 256) {
    const float4 v = value(i);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = lane63(wave_sum_lane63(ss));
  const float r = 1.0f / sqrtf(ss / static_cast<float>(H) + a.eps);
  WT* out = static_cast<WT*>(a.x2) + (static_cast<long long>(wave) * a.B + b) * H;
  for (int i = lane * 4; i < H; i += 256) {
    const float4 v = value(i);
    const float4 g = gamma != nullptr ? load4<WT>(gamma + i) : make_float4(1.f, 1.f, 1.f, 1.f);
    WT* o = out + i;
    o[0] = from_f32<WT>(v.x * r * g.x);
    o[1] = from_f32<WT>(v.y * r * g.y);
    o[2] = from_f32<WT>(v.z * r * g.z);
    o[3] = from_f32<WT>(v.w * r * g.w);
  }
}

size_t esz(int dt) { return dt == MOEV_BF16 ? 2 : 4; }

struct DraftLayout {
  size_t x2, yp, zp, xf, act, yf, z[2], head, total;
};

DraftLayout draft_layout(const moev_model& m, int n, int B) {
  const size_t H = m.hidden, I = m.inter, e = esz(m.dtype), Bz = B;
  DraftLayout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes, 256);
    return at;
  };
  L.x2 = take(2 * Bz * H * e);
  L.yp = take(Bz * 2 * H * 4);
  L.zp = take(Bz * H * 4);
  L.xf = take(Bz * H * e);
  L.act = take(static_cast<size_t>(n) * Bz * I * e);
  L.yf = take(Bz * n * H * 4);
  L.z[0] = take(Bz * H * 4);
  L.z[1] = take(Bz * H * 4);
  L.head = take(lmhead_ws_bytes(B, m.hidden, m.vocab, m.dtype));
  L.total = o;
  return L;
}

}  // namespace

size_t draft_ws_bytes(const moev_model& m, const moev_draft_weights& d, int B) {
  return draft_layout(m, d.n_slices, B).total;
}

moev_status validate_draft(const moev_model* m, const moev_draft_weights* d, int B) {
  if (moev_status st = validate_model_rows(m, B)) return st;
  MOEV_REQUIRE(d != nullptr, MOEV_ERR_INVALID_ARG, "draft weights must not be NULL");
  MOEV_REQUIRE(d->n_slices >= 1 && d->n_slices <= 16, MOEV_ERR_UNSUPPORTED,
               "draft n_slices=%d must be in [1, 16]", d->n_slices);
  MOEV_CHECK(need_ptr(d->w_proj, "draft w_proj") && need_ptr(d->w_gate, "draft w_gate") &&
                 need_ptr(d->w_up, "draft w_up") && need_ptr(d->w_down, "draft w_down") &&
                 opt_ptr(d->norm_z, "draft norm_z") && opt_ptr(d->norm_e, "draft norm_e") &&
                 opt_ptr(d->norm_ffn, "draft norm_ffn") &&
                 opt_ptr(d->norm_out, "draft norm_out"),
             MOEV_ERR_INVALID_ARG);
  return MOEV_OK;
}

void run_draft(const moev_model& m, const moev_draft_weights& d, const float* z_src,
               const int32_t* n_accept, int K1, const int32_t* t0, int B, int K, int32_t* out,
               int out_stride, int out_col0, int32_t* t0_copy, float* z_out, unsigned char* ws,
               hipStream_t s) {
  const int n = d.n_slices;
  const DraftLayout L = draft_layout(m, n, B);
  const int H = m.hidden, I = m.inter, dt = m.dtype;
  void* x2 = ws + L.x2;
  float* yp = reinterpret_cast<float*>(ws + L.yp);
  float* zp = reinterpret_cast<float*>(ws + L.zp);
  void* xf = ws + L.xf;
  void* act = ws + L.act;
  float* yf = reinterpret_cast<float*>(ws + L.yf);
  float* zb[2] = {reinterpret_cast<float*>(ws + L.z[0]), reinterpret_cast<float*>(ws + L.z[1])};
  for (int j = 0; j < K; ++j) {
    DraftInArgs a{};
    a.z = j == 0 ? z_src : zb[(j - 1) & 1];
    a.n_accept = j == 0 ? n_accept : nullptr;
    a.K1 = K1;
    a.tok = j == 0 ? t0 : out + out_col0 + (j - 1);
    a.tok_stride = j == 0 ? 1 : out_stride;
    a.tok_copy = j == 0 ? t0_copy : nullptr;
    a.copy_stride = out_stride;
    a.emb = m.emb;
    a.V = m.vocab;
    a.B = B;
    a.H = H;
    a.norm_z = d.norm_z;
    a.norm_e = d.norm_e;
    a.eps = m.eps;
    a.x2 = x2;
    if (dt == MOEV_BF16) draft_in_kernel<u16><<<B, kDraftThreads, 0, s>>>(a);
    else draft_in_kernel<float><<<B, kDraftThreads, 0, s>>>(a);
    // z' = W_p[:, :H] u_z + W_p[:, H:] u_e: two groups of K = H, weight 1,
    // each holding every row (pair b * 2 + group); the FFN's n slices
    // likewise (pair b * n + slice).  These GEMMs cover 2 or n groups only:
    // split K fills the GPU.
    launch_ffn_down_sets(x2, nullptr, nullptr, d.w_proj, B, H, H, 0, 0, 2, dt, yp, s, true);
    launch_norm_cast(nullptr, yp, 2, d.norm_ffn, m.eps, B, H, dt, xf, zp, s);
    launch_ffn_gate_up_sets(xf, nullptr, d.w_gate, d.w_up, B, H, I, 0, 0, n, dt, act, s, true);
    launch_ffn_down_sets(act, nullptr, nullptr, d.w_down, B, H, I, 0, 0, n, dt, yf, s, true);
    float* zj = (j == K - 1 && z_out != nullptr) ? z_out : zb[j & 1];
    launch_lmhead(zp, d.norm_out, m.eps, m.w_lm, B, H, m.vocab, dt, out + out_col0 + j, nullptr,
                  nullptr, ws + L.head, s, yf, n, zj, out_stride);
  }
}

}  // namespace moev

extern "C" size_t moev_draft_workspace_size(const moev_model* m, const moev_draft_weights* d, int B) {
  using namespace moev;
  if (m == nullptr || d == nullptr || B < 0 || d->n_slices < 1) return 0;
  return draft_ws_bytes(*m, *d, B);
}

extern "C" moev_status moev_draft(const moev_model* m, const moev_draft_weights* d, const float* z0,
                                  const int32_t* t0, int B, int K, int32_t* drafts, float* z_out,
                                  void* ws, size_t ws_bytes, void* stream) {
  using namespace moev;
  clear_error();
  MOEV_REQUIRE(B >= 0 && K >= 0, MOEV_ERR_INVALID_ARG, "need B >= 0 and K >= 0 (B=%d K=%d)", B, K);
  if (moev_status st = validate_draft(m, d, B)) return st;
  if (B == 0 || K == 0) return MOEV_OK;
  MOEV_CHECK(need_ptr(z0, "z0") && need_ptr(t0, "t0", 4) && need_ptr(drafts, "drafts", 4) &&
                 opt_ptr(z_out, "z_out"),
             MOEV_ERR_INVALID_ARG);
  const size_t need = draft_ws_bytes(*m, *d, B);
  MOEV_REQUIRE(ws != nullptr && aligned16(ws), MOEV_ERR_WORKSPACE,
               "workspace must be non-NULL and 16-byte aligned");
  MOEV_REQUIRE(ws_bytes >= need, MOEV_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes,
               need);
  run_draft(*m, *d, z0, nullptr, 1, t0, B, K, drafts, K, 0, nullptr, z_out,
            static_cast<unsigned char*>(ws), as_stream(stream));
  return launch_status("moev_draft");
}
