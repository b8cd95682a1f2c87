// Whole FastMTP verify step on one stream: embedding gather, the decoder's
// MoE layers (route -> expert grouping -> grouped FFN -> combine), the greedy
// head and the prefix-accept kernel.  All scratch lives in one caller-provided
// workspace; nothing here allocates or synchronises, so a step can be
// captured into a HIP graph and replayed.
//
// The verification itself follows "The speed comes from three layers working
// together" (Jina-OCR-v1 explainer, kg.zhiyong.dev): the K drafted tokens are
// checked by the main decoder in one pass, here as T = B*(K+1) rows of one
// batch.  moev_verify_step_attn runs the same step with an attention sublayer
// before every MoE sublayer (per-sequence key/value caches, positions
// advanced by the accepted length on the device).
#include "launch.h"

namespace moev {
namespace {

struct StepLayout {
  size_t h, x, idx, w, offsets, sorted, masks, pinfo, y, ffn, head, total;
};

// Decode-sized steps route through token sets filled by the router (no
// permute launch); larger ones through the sorted pair order.
bool use_sets(const moev_model& m, int T) { return sets_fit(T, m.hidden, m.inter); }

size_t esz(int dt) { return dt == MOEV_BF16 ? 2 : 4; }

StepLayout layout(const moev_model& m, int T) {
  const int S = m.top_k + m.n_shared;
  const int G = m.n_routed + m.n_shared;
  const size_t P = static_cast<size_t>(T) * S;
  StepLayout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes, 256);
    return at;
  };
  L.h = take(static_cast<size_t>(T) * m.hidden * 4);
  L.x = take(static_cast<size_t>(T) * m.hidden * esz(m.dtype));
  L.idx = take(static_cast<size_t>(T) * m.top_k * 4);
  L.w = take(static_cast<size_t>(T) * m.top_k * 4);
  const bool sets = use_sets(m, T);
  L.offsets = take(static_cast<size_t>(G + 1) * 4);
  // sorted pair order [P] (without token sets)
  L.sorted = take(sets ? 0 : P * 4);
  // token sets: one mask set [E][W] per layer, pair entries [T][E]
  L.masks = take(sets ? static_cast<size_t>(m.n_layers > 0 ? m.n_layers : 1) * set_layer_words(m.n_routed, T) * 8 : 0);
  L.pinfo = take(sets ? static_cast<size_t>(T) * m.n_routed * 8 : 0);
  L.y = take(P * m.hidden * 4);
  // gate/up activations: [P, I] in sorted order, or [G*T, I] by token set
  L.ffn = take(sets ? static_cast<size_t>(G) * T * m.inter * esz(m.dtype)
                    : grouped_ffn_ws_bytes(T, m.inter, m.top_k, m.n_shared, m.dtype));
  L.head = take(lmhead_ws_bytes(T, m.hidden, m.vocab, m.dtype));
  L.total = o;
  return L;
}

}  // namespace

// Checks of the model and of T = B * (K + 1) (or the prefill's token count).
moev_status validate_model_rows(const moev_model* m, long long T) {
  MOEV_REQUIRE(m != nullptr, MOEV_ERR_INVALID_ARG, "model must not be NULL");
  MOEV_CHECK(check_dtype(m->dtype), MOEV_ERR_UNSUPPORTED);
  MOEV_REQUIRE(m->hidden >= 64 && m->hidden <= 3072 && m->hidden % 64 == 0, MOEV_ERR_UNSUPPORTED,
               "hidden size %d must be a multiple of 64 in [64, 3072]", m->hidden);
  MOEV_REQUIRE(m->inter >= 64 && m->inter <= 8192 && m->inter % 64 == 0, MOEV_ERR_UNSUPPORTED,
               "intermediate size %d must be a multiple of 64 in [64, 8192]", m->inter);
  MOEV_REQUIRE(m->n_routed >= 1 && m->n_routed <= 64, MOEV_ERR_UNSUPPORTED,
               "routed experts E=%d must be in [1, 64]", m->n_routed);
  MOEV_REQUIRE(m->top_k >= 1 && m->top_k <= m->n_routed, MOEV_ERR_UNSUPPORTED,
               "top-k k=%d must be in [1, E=%d]", m->top_k, m->n_routed);
  MOEV_REQUIRE(m->n_shared >= 0 && m->n_shared <= 8, MOEV_ERR_UNSUPPORTED,
               "shared experts ns=%d must be in [0, 8]", m->n_shared);
  MOEV_REQUIRE(m->top_k + m->n_shared <= 16, MOEV_ERR_UNSUPPORTED,
               "the whole-step driver needs k + ns <= 16 (got %d)", m->top_k + m->n_shared);
  MOEV_REQUIRE(m->vocab >= 1, MOEV_ERR_INVALID_ARG, "vocabulary must be >= 1");
  MOEV_REQUIRE(m->n_layers >= 0, MOEV_ERR_INVALID_ARG, "n_layers must be >= 0");
  MOEV_REQUIRE(T * (m->top_k + m->n_shared) < (1ll << 31), MOEV_ERR_UNSUPPORTED,
               "tokens*(k+ns) must be < 2^31 (tokens=%lld)", T);
  MOEV_CHECK(need_ptr(m->emb, "model.emb") && opt_ptr(m->norm_f, "model.norm_f") &&
                 need_ptr(m->w_lm, "model.w_lm"),
             MOEV_ERR_INVALID_ARG);
  MOEV_REQUIRE(m->n_layers == 0 || m->layers != nullptr, MOEV_ERR_INVALID_ARG,
               "model.layers must not be NULL");
  for (int l = 0; l < m->n_layers; ++l) {
    const moev_layer_weights& lw = m->layers[l];
    if (!(opt_ptr(lw.norm, "layer.norm") && need_ptr(lw.w_router, "layer.w_router") &&
          opt_ptr(lw.bias, "layer.bias", 4) && need_ptr(lw.w_gate, "layer.w_gate") &&
          need_ptr(lw.w_up, "layer.w_up") && need_ptr(lw.w_down, "layer.w_down"))) {
      set_error("layer %d: %s", l, moev_last_error());
      return MOEV_ERR_INVALID_ARG;
    }
  }
  return MOEV_OK;
}

namespace {

moev_status validate_model(const moev_model* m, int B, int K) {
  MOEV_REQUIRE(B >= 0 && K >= 0, MOEV_ERR_INVALID_ARG, "need B >= 0 and K >= 0 (B=%d K=%d)", B, K);
  MOEV_REQUIRE(K <= 64, MOEV_ERR_UNSUPPORTED, "K=%d drafts exceeds 64", K);
  return validate_model_rows(m, static_cast<long long>(B) * (K + 1));
}

// Prefill workspace: the layer loop's buffers for T rows, then the last rows'
// combined residual [n_seq, H] and their head workspace.
struct PrefillLayout {
  StepLayout L;
  size_t h_last, head_last, total;
};

PrefillLayout prefill_layout(const moev_model& m, int n_seq, int seq_len) {
  PrefillLayout P{};
  P.L = layout(m, n_seq * seq_len);
  size_t o = P.L.total;
  P.h_last = o;
  o += align_up(static_cast<size_t>(n_seq) * m.hidden * 4, 256);
  P.head_last = o;
  o += align_up(lmhead_ws_bytes(n_seq, m.hidden, m.vocab, m.dtype), 256);
  P.total = o;
  return P;
}

}  // namespace
}  // namespace moev

extern "C" size_t moev_verify_step_workspace_size(const moev_model* m, int B, int K) {
  if (m == nullptr || B < 0 || K < 0) return 0;
  return moev::layout(*m, B * (K + 1)).total;
}

namespace moev {
namespace {

// The attention sublayer's device buffers and weights for one pass (see
// moev_verify_step_attn); rows = K + 1 verify rows per sequence.
struct AttnHook {
  const moev_attn* a;
  int B, rows;
  const int32_t* pos;
  float* q;        // [T, H]
  float* ao;       // [T, H] the attention output's W_o projection, added to h by the router
  float* part;     // attention's per-split softmax states
  int* cnt;        // [B, n_heads] split counts of the fused merge (cleared by the embedding)
};

__global__ void pos_advance_kernel(int32_t* pos, const int32_t* commit_len, int B) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) pos[b] += commit_len[b];
}

// The attention sublayer of layer l on the residual stream h (to which the
// previous layer's expert slots y_prev are added first).  Leaves its output
// projection in hook.ao for the router to add.
void run_attn_sublayer(const moev_model* m, const AttnHook& at, int l, float* h, const float* y_prev,
                       int S, void* x, hipStream_t s) {
  const moev_attn_layer& al = at.a->layers[l];
  const int H = m->hidden, dt = m->dtype, T = at.B * at.rows;
  launch_norm_cast(h, y_prev, S, nullptr, m->eps, T, H, dt, x, h, s);
  // dense projections (one group holding every row): every 32-token pass of
  // a row tile in its own workgroup
  const int passes = (T + 31) / 32;
  // the Q/K/V projection's epilogue writes q, and the pass's keys and values
  // into the caches at pos[b] + i
  const QkvScatter qkv{at.pos, at.rows, at.a->max_len, H / at.a->n_heads, at.q, al.k_cache, al.v_cache};
  launch_ffn_down_sets(x, nullptr, nullptr, al.w_qkv, T, 3 * H, H, 0, 0, 1, dt, nullptr, s, true, passes, &qkv);
  // the attention output goes straight into x in the operand type
  launch_attn_decode(at.q, al.k_cache, al.v_cache, at.pos, at.B, at.rows, at.a->max_len, H,
                     at.a->n_heads, dt, x, true, at.part, s, at.cnt);
  launch_ffn_down_sets(x, nullptr, nullptr, al.w_o, T, H, H, 0, 0, 1, dt, at.ao, s, true, passes);
}

// Embedding and the decoder layers for T rows.  On return h holds the residual
// stream before the last layer's expert outputs, y those outputs: the caller
// folds the last combine into whatever reads h next.
void run_layers(const moev_model* m, const int32_t* tokens, int T, const StepLayout& L,
                unsigned char* base, const moev_step_probe* probe, hipStream_t s,
                const AttnHook* at = nullptr) {
  float* h = reinterpret_cast<float*>(base + L.h);
  void* x = base + L.x;
  int32_t* idx = reinterpret_cast<int32_t*>(base + L.idx);
  float* w = reinterpret_cast<float*>(base + L.w);
  int32_t* offsets = reinterpret_cast<int32_t*>(base + L.offsets);
  int32_t* sorted = reinterpret_cast<int32_t*>(base + L.sorted);
  uint64_t* masks = reinterpret_cast<uint64_t*>(base + L.masks);
  int2* pinfo = reinterpret_cast<int2*>(base + L.pinfo);
  float* y = reinterpret_cast<float*>(base + L.y);
  void* ffn_ws = base + L.ffn;
  const int H = m->hidden, E = m->n_routed, k = m->top_k, ns = m->n_shared, I = m->inter;
  const int dt = m->dtype;

  // probe events around one stage (index = layer, or 0 for the head)
  auto mark = [&](int stage, int index, bool after) {
    if (probe == nullptr || probe->stage != stage || index >= probe->n) return;
    // a failed record stays in the runtime's last error, which launch_status reports
    (void)hipEventRecord(static_cast<hipEvent_t>(after ? probe->after[index] : probe->before[index]), s);
  };

  // Launches per layer: router (with the previous layer's combine folded in),
  // permute (only without token sets), gate/up, down.  The last layer's
  // combine happens inside the head's norm kernel.  With token sets the
  // embedding kernel clears one mask set per layer and the router adds each
  // pair to its expert's set.
  const int S = k + ns;
  const bool sets = use_sets(*m, T);
  const int W = set_words(T);
  TokenSets ts{masks, pinfo, m->n_layers, E, W};
  launch_embed(tokens, m->emb, T, H, m->vocab, dt, h, s, sets && m->n_layers > 0 ? &ts : nullptr,
               at != nullptr ? at->cnt : nullptr, at != nullptr ? at->B * at->a->n_heads : 0);
  for (int l = 0; l < m->n_layers; ++l) {
    const moev_layer_weights& lw = m->layers[l];
    const float* y_prev = l > 0 ? y : nullptr;
    int s_prev = S;
    if (at != nullptr) {
      // attention first: the previous layer's slots go into h there, and the
      // router adds the attention's output projection as a single slot
      run_attn_sublayer(m, *at, l, h, y_prev, S, x, s);
      y_prev = at->ao;
      s_prev = 1;
    }
    uint64_t* mk = masks + static_cast<size_t>(l) * set_layer_words(E, T);
    mark(MOEV_STAGE_ROUTE, l, false);
    launch_route_fused(h, y_prev, s_prev, h, lw.norm, m->eps, lw.w_router, lw.bias, T, H, E, k, dt, x,
                       idx, w, s, sets ? mk : nullptr, sets ? pinfo : nullptr);
    mark(MOEV_STAGE_ROUTE, l, true);
    mark(MOEV_STAGE_PERMUTE, l, false);
    if (!sets) launch_permute(idx, T, k, E, ns, offsets, sorted, s);
    mark(MOEV_STAGE_PERMUTE, l, true);
    mark(MOEV_STAGE_GATE_UP, l, false);
    if (sets)
      launch_ffn_gate_up_sets(x, mk, lw.w_gate, lw.w_up, T, H, I, E, k, ns, dt, ffn_ws, s);
    else
      launch_ffn_gate_up(x, sorted, offsets, lw.w_gate, lw.w_up, T, H, I, E, k, ns, dt, ffn_ws, s);
    mark(MOEV_STAGE_GATE_UP, l, true);
    mark(MOEV_STAGE_DOWN, l, false);
    if (sets)
      launch_ffn_down_sets(ffn_ws, mk, pinfo, lw.w_down, T, H, I, E, k, ns, dt, y, s);
    else
      launch_ffn_down(ffn_ws, sorted, offsets, w, lw.w_down, T, H, I, E, k, ns, dt, y, s);
    mark(MOEV_STAGE_DOWN, l, true);
  }
}

moev_status run_step(const moev_model* m, const int32_t* tokens, int B, int K, int32_t* greedy,
                     int32_t* n_accept, int32_t* commit, int32_t* commit_len, int32_t* next_last,
                     void* ws, size_t ws_bytes, const moev_step_probe* probe, void* stream,
                     float* h_final = nullptr, const AttnHook* at = nullptr) {
  if (moev_status st = validate_model(m, B, K)) return st;
  if (B == 0) return MOEV_OK;
  MOEV_CHECK(need_ptr(tokens, "tokens", 4) && need_ptr(greedy, "greedy", 4) &&
                 need_ptr(n_accept, "n_accept", 4) && need_ptr(commit, "commit", 4),
             MOEV_ERR_INVALID_ARG);
  if (probe != nullptr) {
    MOEV_REQUIRE(probe->stage >= MOEV_STAGE_ROUTE && probe->stage <= MOEV_STAGE_HEAD &&
                     probe->n >= 0 && (probe->n == 0 || (probe->before && probe->after)),
                 MOEV_ERR_INVALID_ARG, "bad probe");
  }
  const int T = B * (K + 1);
  const StepLayout L = layout(*m, T);
  MOEV_REQUIRE(ws != nullptr && aligned16(ws), MOEV_ERR_WORKSPACE,
               "workspace must be non-NULL and 16-byte aligned");
  MOEV_REQUIRE(ws_bytes >= L.total, MOEV_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu",
               ws_bytes, L.total);

  unsigned char* base = static_cast<unsigned char*>(ws);
  const hipStream_t s = as_stream(stream);
  run_layers(m, tokens, T, L, base, probe, s, at);
  const int S = m->top_k + m->n_shared;
  float* h = reinterpret_cast<float*>(base + L.h);
  float* y = reinterpret_cast<float*>(base + L.y);
  void* head_ws = base + L.head;
  auto mark = [&](int stage, int index, bool after) {
    if (probe == nullptr || probe->stage != stage || index >= probe->n) return;
    // a failed record stays in the runtime's last error, which launch_status reports
    (void)hipEventRecord(static_cast<hipEvent_t>(after ? probe->after[index] : probe->before[index]), s);
  };
  const int H = m->hidden, dt = m->dtype;
  // the head's last kernel also applies the prefix acceptance
  VerifyFuse vf{tokens, B, K, n_accept, commit, commit_len, next_last};
  if (at != nullptr) {
    vf.pos = at->pos;
    vf.max_len = at->a->max_len;
  }
  mark(MOEV_STAGE_HEAD, 0, false);
  launch_lmhead(h, m->norm_f, m->eps, m->w_lm, T, H, m->vocab, dt, greedy, nullptr, nullptr,
                head_ws, s, m->n_layers > 0 ? y : nullptr, S, h_final, 1, &vf);
  mark(MOEV_STAGE_HEAD, 0, true);
  return launch_status("moev_verify_step");
}

// Prefill: every prompt row through the layers; the head only for each
// sequence's last row.
moev_status run_prefill(const moev_model* m, const int32_t* tokens, int n_seq, int seq_len,
                        int32_t* next_token, float* h_out, void* ws, size_t ws_bytes,
                        const moev_step_probe* probe, void* stream) {
  MOEV_REQUIRE(n_seq >= 0 && seq_len >= 1, MOEV_ERR_INVALID_ARG,
               "need n_seq >= 0 and seq_len >= 1 (n_seq=%d seq_len=%d)", n_seq, seq_len);
  const long long T64 = static_cast<long long>(n_seq) * seq_len;
  MOEV_REQUIRE(T64 < (1ll << 31), MOEV_ERR_UNSUPPORTED, "n_seq*seq_len must be < 2^31");
  if (moev_status st = validate_model_rows(m, T64)) return st;
  if (n_seq == 0) return MOEV_OK;
  MOEV_CHECK(need_ptr(tokens, "tokens", 4) && need_ptr(next_token, "next_token", 4) &&
                 opt_ptr(h_out, "h_out"),
             MOEV_ERR_INVALID_ARG);
  if (probe != nullptr) {
    MOEV_REQUIRE(probe->stage >= MOEV_STAGE_ROUTE && probe->stage <= MOEV_STAGE_HEAD &&
                     probe->n >= 0 && (probe->n == 0 || (probe->before && probe->after)),
                 MOEV_ERR_INVALID_ARG, "bad probe");
  }
  const int T = static_cast<int>(T64);
  const PrefillLayout P = prefill_layout(*m, n_seq, seq_len);
  MOEV_REQUIRE(ws != nullptr && aligned16(ws), MOEV_ERR_WORKSPACE,
               "workspace must be non-NULL and 16-byte aligned");
  MOEV_REQUIRE(ws_bytes >= P.total, MOEV_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu",
               ws_bytes, P.total);

  unsigned char* base = static_cast<unsigned char*>(ws);
  const hipStream_t s = as_stream(stream);
  run_layers(m, tokens, T, P.L, base, probe, s);
  const int S = m->top_k + m->n_shared;
  float* h = reinterpret_cast<float*>(base + P.L.h);
  const float* y = m->n_layers > 0 ? reinterpret_cast<const float*>(base + P.L.y) : nullptr;
  float* h_last = reinterpret_cast<float*>(base + P.h_last);
  // the last layer's combine: for every row when the caller wants the
  // residual stream, else only for the rows the head reads
  if (h_out != nullptr) {
    if (y != nullptr) launch_combine(y, h, T, m->hidden, S, h_out, s);
    else if (hipMemcpyAsync(h_out, h, static_cast<size_t>(T) * m->hidden * 4, hipMemcpyDeviceToDevice, s) !=
             hipSuccess)
      return launch_status("moev_prefill");
  }
  launch_gather_last(h, y, S, m->hidden, n_seq, seq_len, h_last, s);
  auto mark = [&](int stage, int index, bool after) {
    if (probe == nullptr || probe->stage != stage || index >= probe->n) return;
    // a failed record stays in the runtime's last error, which launch_status reports
    (void)hipEventRecord(static_cast<hipEvent_t>(after ? probe->after[index] : probe->before[index]), s);
  };
  mark(MOEV_STAGE_HEAD, 0, false);
  launch_lmhead(h_last, m->norm_f, m->eps, m->w_lm, n_seq, m->hidden, m->vocab, m->dtype, next_token,
                nullptr, nullptr, base + P.head_last, s);
  mark(MOEV_STAGE_HEAD, 0, true);
  return launch_status("moev_prefill");
}

}  // namespace
}  // namespace moev

extern "C" size_t moev_prefill_workspace_size(const moev_model* m, int n_seq, int seq_len) {
  if (m == nullptr || n_seq < 0 || seq_len < 1) return 0;
  return moev::prefill_layout(*m, n_seq, seq_len).total;
}

extern "C" moev_status moev_prefill(const moev_model* m, const int32_t* tokens, int n_seq, int seq_len,
                                    int32_t* next_token, float* h_out, void* ws, size_t ws_bytes,
                                    void* stream) {
  return moev::run_prefill(m, tokens, n_seq, seq_len, next_token, h_out, ws, ws_bytes, nullptr, stream);
}

extern "C" moev_status moev_prefill_probed(const moev_model* m, const int32_t* tokens, int n_seq,
                                           int seq_len, int32_t* next_token, float* h_out, void* ws,
                                           size_t ws_bytes, const moev_step_probe* probe, void* stream) {
  return moev::run_prefill(m, tokens, n_seq, seq_len, next_token, h_out, ws, ws_bytes, probe, stream);
}

extern "C" moev_status moev_verify_step(const moev_model* m, const int32_t* tokens, int B, int K,
                                        int32_t* greedy, int32_t* n_accept, int32_t* commit,
                                        int32_t* commit_len, int32_t* next_last, void* ws,
                                        size_t ws_bytes, void* stream) {
  return moev::run_step(m, tokens, B, K, greedy, n_accept, commit, commit_len, next_last, ws,
                        ws_bytes, nullptr, stream);
}

extern "C" moev_status moev_verify_step_probed(const moev_model* m, const int32_t* tokens, int B,
                                               int K, int32_t* greedy, int32_t* n_accept,
                                               int32_t* commit, int32_t* commit_len,
                                               int32_t* next_last, void* ws, size_t ws_bytes,
                                               const moev_step_probe* probe, void* stream) {
  return moev::run_step(m, tokens, B, K, greedy, n_accept, commit, commit_len, next_last, ws,
                        ws_bytes, probe, stream);
}

namespace moev {
namespace {

// Speculative step workspace: the verify step's, then the final residual
// [T, H] (when the caller passes none), next_last [B] and the draft block's.
struct SpecLayout {
  size_t h_final, next_last, draft, total;
};

SpecLayout spec_layout(const moev_model& m, const moev_draft_weights& d, int B, int K) {
  SpecLayout S{};
  const int T = B * (K + 1);
  size_t o = layout(m, T).total;
  S.h_final = o;
  o += align_up(static_cast<size_t>(T) * m.hidden * 4, 256);
  S.next_last = o;
  o += align_up(static_cast<size_t>(B) * 4, 256);
  S.draft = o;
  o += draft_ws_bytes(m, d, B);
  S.total = o;
  return S;
}

}  // namespace
}  // namespace moev

extern "C" size_t moev_spec_step_workspace_size(const moev_model* m, const moev_draft_weights* d,
                                                int B, int K) {
  if (m == nullptr || d == nullptr || B < 0 || K < 0 || d->n_slices < 1) return 0;
  return moev::spec_layout(*m, *d, B, K).total;
}

extern "C" moev_status moev_spec_step(const moev_model* m, const moev_draft_weights* d,
                                      const int32_t* tokens, int B, int K, int32_t* greedy,
                                      int32_t* n_accept, int32_t* commit, int32_t* commit_len,
                                      int32_t* next_tokens, float* h_final, void* ws,
                                      size_t ws_bytes, void* stream) {
  using namespace moev;
  clear_error();
  MOEV_REQUIRE(B >= 0 && K >= 1, MOEV_ERR_INVALID_ARG, "need B >= 0 and K >= 1 (B=%d K=%d)", B, K);
  if (moev_status st = validate_model(m, B, K)) return st;
  if (moev_status st = validate_draft(m, d, B)) return st;
  if (B == 0) return MOEV_OK;
  MOEV_CHECK(need_ptr(next_tokens, "next_tokens", 4) && opt_ptr(h_final, "h_final"),
             MOEV_ERR_INVALID_ARG);
  const SpecLayout S = spec_layout(*m, *d, B, K);
  MOEV_REQUIRE(ws != nullptr && aligned16(ws), MOEV_ERR_WORKSPACE,
               "workspace must be non-NULL and 16-byte aligned");
  MOEV_REQUIRE(ws_bytes >= S.total, MOEV_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu",
               ws_bytes, S.total);
  unsigned char* base = static_cast<unsigned char*>(ws);
  float* hf = h_final != nullptr ? h_final : reinterpret_cast<float*>(base + S.h_final);
  int32_t* next_last = reinterpret_cast<int32_t*>(base + S.next_last);
  if (moev_status st = run_step(m, tokens, B, K, greedy, n_accept, commit, commit_len, next_last,
                                ws, ws_bytes, nullptr, stream, hf))
    return st;
  // drafts for the next pass: from row b*(K+1) + n_accept[b] of the final
  // residual and from next_last[b], which also becomes column 0
  run_draft(*m, *d, hf, n_accept, K + 1, next_last, B, K, next_tokens, K + 1, 1, next_tokens,
            nullptr, base + S.draft, as_stream(stream));
  return launch_status("moev_spec_step");
}

namespace moev {
namespace {

// Attention step workspace: the verify step's, then the dense-GEMM row list
// and the attention sublayer's buffers.
struct AttnLayout {
  size_t q, ao, part, cnt, total;
};

AttnLayout attn_layout(const moev_model& m, const moev_attn& a, int B, int K) {
  const int T = B * (K + 1);
  const size_t rowf = static_cast<size_t>(T) * m.hidden * 4;
  AttnLayout A{};
  size_t o = layout(m, T).total;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes, 256);
    return at;
  };
  A.q = take(rowf);
  A.ao = take(rowf);
  A.part = take(a.n_heads >= 1 ? attn_ws_bytes(B, K + 1, m.hidden, a.n_heads) : 0);
  A.cnt = take(static_cast<size_t>(B) * (a.n_heads >= 1 ? a.n_heads : 0) * sizeof(int));
  A.total = o;
  return A;
}

// rows of one pass with attention
constexpr int kAttnMaxRows = 512;

moev_status validate_attn(const moev_model* m, const moev_attn* a, int B, int K) {
  MOEV_REQUIRE(a != nullptr, MOEV_ERR_INVALID_ARG, "attention weights must not be NULL");
  MOEV_REQUIRE(K + 1 <= 16, MOEV_ERR_UNSUPPORTED, "K=%d: attention takes at most 16 rows per sequence", K);
  MOEV_REQUIRE(static_cast<long long>(B) * (K + 1) <= kAttnMaxRows, MOEV_ERR_UNSUPPORTED,
               "B*(K+1)=%lld rows exceeds %d", static_cast<long long>(B) * (K + 1), kAttnMaxRows);
  MOEV_REQUIRE(a->n_heads >= 1 && m->hidden % a->n_heads == 0, MOEV_ERR_UNSUPPORTED,
               "hidden size %d must be a multiple of n_heads=%d", m->hidden, a->n_heads);
  const int D = m->hidden / a->n_heads;
  MOEV_REQUIRE(D == 64 || D == 128 || D == 256, MOEV_ERR_UNSUPPORTED, "head width %d must be 64, 128 or 256",
               D);
  MOEV_REQUIRE(a->max_len >= K + 1, MOEV_ERR_INVALID_ARG, "max_len=%d must be >= K+1=%d", a->max_len, K + 1);
  MOEV_REQUIRE(m->n_layers == 0 || a->layers != nullptr, MOEV_ERR_INVALID_ARG,
               "attention layers must not be NULL");
  for (int l = 0; l < m->n_layers; ++l) {
    const moev_attn_layer& al = a->layers[l];
    if (!(need_ptr(al.w_qkv, "attn.w_qkv") && need_ptr(al.w_o, "attn.w_o") &&
          need_ptr(al.k_cache, "attn.k_cache") && need_ptr(al.v_cache, "attn.v_cache"))) {
      set_error("attention layer %d: %s", l, moev_last_error());
      return MOEV_ERR_INVALID_ARG;
    }
  }
  return MOEV_OK;
}

}  // namespace
}  // namespace moev

extern "C" size_t moev_verify_step_attn_workspace_size(const moev_model* m, const moev_attn* a, int B,
                                                       int K) {
  if (m == nullptr || a == nullptr || B < 0 || K < 0) return 0;
  return moev::attn_layout(*m, *a, B, K).total;
}

extern "C" moev_status moev_verify_step_attn(const moev_model* m, const moev_attn* a, const int32_t* tokens,
                                             int B, int K, int32_t* pos, int32_t* greedy, int32_t* n_accept,
                                             int32_t* commit, int32_t* commit_len, int32_t* next_last,
                                             void* ws, size_t ws_bytes, void* stream) {
  using namespace moev;
  clear_error();
  if (moev_status st = validate_model(m, B, K)) return st;
  if (moev_status st = validate_attn(m, a, B, K)) return st;
  if (B == 0) return MOEV_OK;
  MOEV_CHECK(need_ptr(pos, "pos", 4) && need_ptr(commit_len, "commit_len", 4) &&
                 need_ptr(next_last, "next_last", 4),
             MOEV_ERR_INVALID_ARG);
  const AttnLayout A = attn_layout(*m, *a, B, K);
  MOEV_REQUIRE(ws != nullptr && aligned16(ws), MOEV_ERR_WORKSPACE,
               "workspace must be non-NULL and 16-byte aligned");
  MOEV_REQUIRE(ws_bytes >= A.total, MOEV_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes,
               A.total);
  unsigned char* base = static_cast<unsigned char*>(ws);
  const hipStream_t s = as_stream(stream);
  const AttnHook at{a, B, K + 1, pos, reinterpret_cast<float*>(base + A.q),
                    reinterpret_cast<float*>(base + A.ao), reinterpret_cast<float*>(base + A.part),
                    reinterpret_cast<int*>(base + A.cnt)};
  if (moev_status st = run_step(m, tokens, B, K, greedy, n_accept, commit, commit_len, next_last, ws,
                                ws_bytes, nullptr, stream, nullptr, &at))
    return st;
  pos_advance_kernel<<<(B + 255) / 256, 256, 0, s>>>(pos, commit_len, B);
  return launch_status("moev_verify_step_attn");
}
