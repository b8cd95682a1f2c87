// Internal launchers and validators shared between the per-call entry points
// and the whole-step driver.  Launchers do no validation.
#pragma once

#include "common.h"

namespace moev {

// Token sets (the whole-step driver's replacement for the sorted pair order
// up to kSetMaxTokens rows, see sets_fit): routed group g < E holds the tokens
// whose bit is set in its mask words (bit t % 64 of word t / 64, W =
// ceil(T / 64); word w of group g at masks[set_word(E, g, w)]), in increasing
// token order, and pair (t, g) has pinfo[t*E + g] = {bits of its renormalised
// router weight, its slot}.  The router sets both with no returned value to
// wait for (an atomic OR and a store).
// Groups g >= E (the shared experts, and every group of a dense projection,
// E = 0) hold every token in order, slot k + g - E, weight 1.  Group g's m-th
// token has act row g*T + m.
struct TokenSets {
  uint64_t* masks;  // [n_sets][W][E]: one set per layer
  int2* pinfo;      // [T][E]
  int n_sets, E, W;
};
// Token sets serve the streaming GEMM schedule (up to 128 rows, a set in two
// 64-bit words) and the tiled one above it, up to this many rows (8 words)
constexpr int kSetMaxTokens = 512;
constexpr int set_words(int T) { return (T + 63) / 64; }
// Mask words are stored word-major ([W][E]): the words of one heavily routed
// expert sit in different cache lines, so under skewed routing its atomic ORs
// do not all queue on one line.
__host__ __device__ constexpr size_t set_word(int E, int g, int w) { return static_cast<size_t>(w) * E + g; }
// 64-bit words of one layer's token sets
__host__ __device__ constexpr size_t set_layer_words(int E, int T) { return static_cast<size_t>(set_words(T)) * E; }
// Whether a step of T rows runs on token sets: up to 128 rows always, above
// that when both expert GEMMs take the tiled schedule at this shape.
bool sets_fit(int T, int H, int I);

// sets != NULL: also clears every mask set; zero[0 .. n_zero) is cleared too
// (the attention step's merge counts).
void launch_embed(const int32_t* tokens, const void* emb, int T, int H, int V, int dt, float* h,
                  hipStream_t s, const TokenSets* sets = nullptr, int* zero = nullptr, int n_zero = 0);
void launch_route(const float* h, const void* norm_w, float eps, const void* w_router,
                  const float* bias, int T, int H, int E, int k, int dt, void* x_out,
                  int32_t* topk_idx, float* topk_w, float* logits_out, hipStream_t s);
// Router with the previous layer's combine folded in (y_prev != NULL: h_out =
// h + the sum of y_prev's S_prev slots, in slot order); h_out may equal h.
// masks != NULL: each token's k pairs also go into the token sets (masks of
// this layer's set, pinfo; T <= kSetMaxTokens).
void launch_route_fused(const float* h, const float* y_prev, int S_prev, float* h_out,
                        const void* norm_w, float eps, const void* w_router, const float* bias,
                        int T, int H, int E, int k, int dt, void* x_out, int32_t* topk_idx,
                        float* topk_w, hipStream_t s, uint64_t* masks = nullptr,
                        int2* pinfo = nullptr);
void launch_permute(const int32_t* topk_idx, int T, int k, int E, int ns, int32_t* offsets,
                    int32_t* sorted_src, hipStream_t s);
void launch_grouped_ffn(const void* x, const int32_t* sorted_src, const int32_t* offsets,
                        const float* topk_w, const void* w_gate, const void* w_up,
                        const void* w_down, int T, int H, int I, int E, int k, int ns, int dt,
                        float* y_slots, void* ws, hipStream_t s);
void launch_ffn_gate_up(const void* x, const int32_t* sorted_src, const int32_t* offsets,
                        const void* w_gate, const void* w_up, int T, int H, int I, int E, int k,
                        int ns, int dt, void* act, hipStream_t s);
void launch_ffn_down(const void* act, const int32_t* sorted_src, const int32_t* offsets,
                     const float* topk_w, const void* w_down, int T, int H, int I, int E, int k,
                     int ns, int dt, float* y_slots, hipStream_t s);
// Model checks shared by the whole-step entry points (T rows).
moev_status validate_model_rows(const moev_model* m, long long T);

// FastMTP draft block (draft.hip).  run_draft enqueues K draft steps for B
// rows: step 1 reads z_src row b*K1 + n_accept[b] (row b when n_accept is
// NULL) and token t0[b]; draft j lands in out[b*out_stride + out_col0 + j-1]
// and is step j+1's token; t0_copy (optional) receives t0 at
// t0_copy[b*out_stride]; z_out (optional) receives z_K.
size_t draft_ws_bytes(const moev_model& m, const moev_draft_weights& d, int B);
moev_status validate_draft(const moev_model* m, const moev_draft_weights* d, int B);
void run_draft(const moev_model& m, const moev_draft_weights& d, const float* z_src,
               const int32_t* n_accept, int K1, const int32_t* t0, int B, int K, int32_t* out,
               int out_stride, int out_col0, int32_t* t0_copy, float* z_out, unsigned char* ws,
               hipStream_t s);

// Expert GEMMs over token sets (sets_fit(T, H, I); masks and pinfo may be
// NULL when E = 0): act holds G*T rows.  split_k: each workgroup's waves split
// one row tile's K range (passes of at most 32 tokens, every size): several
// times the workgroups for GEMMs over a few groups, with rounding that
// differs from split_k = false, so a caller keeps one setting.
void launch_ffn_gate_up_sets(const void* x, const uint64_t* masks, const void* w_gate,
                             const void* w_up, int T, int H, int I, int E, int k, int ns, int dt,
                             void* act, hipStream_t s, bool split_k = false);
// Destination of a fused Q/K/V projection (one dense group, output width 3H):
// row t = b*rows + i, columns [0, H) go to q [T, H] (fp32), [H, 2H) and
// [2H, 3H) to the head-major key and value caches [B, H/D, max_len, D] (D a
// power of two) at
// position pos[b] + i, rounded to the cache type.  A sequence whose cache has
// no room for the pass (pos[b] < 0 or pos[b] + rows > max_len) gets none of
// its rows written.
struct QkvScatter {
  const int32_t* pos;
  int rows, max_len, D;
  float* q;
  void* k_cache;
  void* v_cache;
};
// pass_split (split_k only): the 32-token passes are spread over this many
// workgroups per row tile (grid z), for dense projections of a whole batch;
// with pass_split > 1 a workgroup takes two 16-row tiles (H % 32 == 0).
// scatter (optional, E = 0 with one group): the epilogue writes the rows
// there instead of y_slots (NULL then).
void launch_ffn_down_sets(const void* act, const uint64_t* masks, const int2* pinfo,
                          const void* w_down, int T, int H, int I, int E, int k, int ns, int dt,
                          float* y_slots, hipStream_t s, bool split_k = false, int pass_split = 1,
                          const QkvScatter* scatter = nullptr);
void launch_combine(const float* y, const float* h_in, int T, int H, int S, float* h_out,
                    hipStream_t s);
// out[i] = h[t] + the sum of y's S slots of row t (y may be NULL), t = the
// last row of sequence i (rows i*seq_len .. (i+1)*seq_len - 1); the same
// slot order as launch_combine.
void launch_gather_last(const float* h, const float* y, int S, int H, int n_seq, int seq_len,
                        float* out, hipStream_t s);
// Prefix acceptance fused into the head's last kernel: rows b*(K+1) .. of the
// head are sequence b's (last, d_1 .. d_K), tokens as mtp_verify takes them.
struct VerifyFuse {
  const int32_t* tokens;
  int B, K;
  int32_t* n_accept;
  int32_t* commit;
  int32_t* commit_len;
  int32_t* next_last;
  // with attention: a sequence whose cache has no room for the pass
  // (pos[b] < 0 or pos[b] + K + 1 > max_len) commits nothing (see
  // moev_verify_step_attn); pos NULL without attention
  const int32_t* pos = nullptr;
  int max_len = 0;
};
// y_prev (optional): the last layer's expert slots, added to h before the norm.
// h_out (optional): the combined residual h + sum of y_prev's slots, fp32;
// argmax_out[t * out_stride] receives token t's arg max.  vf (optional): run
// the prefix acceptance too (argmax_out then holds T = B*(K+1) contiguous rows).
void launch_lmhead(const float* h, const void* norm_f, float eps, const void* w_lm, int T, int H,
                   int V, int dt, int32_t* argmax_out, float* max_out, float* logits_out,
                   void* ws, hipStream_t s, const float* y_prev = nullptr, int S_prev = 0,
                   float* h_out = nullptr, int out_stride = 1, const VerifyFuse* vf = nullptr);
// xo = RMSNorm(v) * gamma cast to dt, v = h (NULL: zeros) + the S slots of y
// (NULL: none) in slot order; h_out (optional) receives v in fp32.
void launch_norm_cast(const float* h, const float* y, int S, const void* gamma, float eps, int T,
                      int H, int dt, void* xo, float* h_out, hipStream_t s);
void launch_verify(const int32_t* tokens, const int32_t* greedy, int B, int K, int32_t* n_accept,
                   int32_t* commit, int32_t* commit_len, int32_t* next_last, hipStream_t s);

// Decode attention (moev_attn_decode's kernels, arguments already checked).
// out: fp32, or dt when out_dt (the operand of the output projection); part:
// attn_ws_bytes() of fp32 workspace for the splits' states.  fuse_cnt (with
// out_dt): B * n_heads counts, zero before the call and zero again after it;
// the last split of each (sequence, head) merges, so there is one launch.
size_t attn_ws_bytes(int B, int rows, int H, int n_heads);
void launch_attn_decode(const float* q, const void* k_cache, const void* v_cache, const int32_t* pos,
                        int B, int rows, int max_len, int H, int n_heads, int dt, void* out, bool out_dt,
                        float* part, hipStream_t s, int* fuse_cnt = nullptr);

size_t grouped_ffn_ws_bytes(int T, int I, int k, int ns, int dt);
// moe_grouped_ffn's argument checks (ws_bytes: the workspace's size)
moev_status validate_grouped_ffn(const void* x, const int32_t* sorted_src, const int32_t* offsets,
                                 const float* topk_w, const void* w_gate, const void* w_up,
                                 const void* w_down, int T, int H, int I, int E, int k, int ns,
                                 int dt, const float* y_slots, const void* ws, size_t ws_bytes);
size_t lmhead_ws_bytes(int T, int H, int V, int dt);

}  // namespace moev
