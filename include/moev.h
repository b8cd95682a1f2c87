/*
 * moev.h -- C ABI of the MI355X (gfx950) library for the FastMTP verify step
 * through a Jina-OCR-v1 style mixture-of-experts decoder.
 *
 * Sources (web pages on Jina-OCR-v1):
 *   [P1] "Jina AI's jina-ocr-v1 Is Selling Throughput, Not the OCR Crown"
 *        (kg.zhiyong.dev explainer);
 *   [P2] aipolix.com news analysis of Jina-OCR-v1 (document parsing, FastMTP,
 *        non-commercial weights);
 *   [P3] "Jina-OCR-v1: Efficient Document Parsing with Speculative Decoding and
 *        Dense Verifiable Rewards" (evolve.pub review of the arXiv paper).
 *
 * Conventions for every entry point
 *   - Device pointers are caller-owned device memory (for example torch
 *     tensors), row-major and contiguous.  int32 arrays, router weights,
 *     biases, arg max / max / logits outputs need 4-byte alignment; every
 *     other buffer (hidden states, operands, weights, expert slots,
 *     workspaces) 16-byte alignment.  The library
 *     allocates nothing and keeps no state between calls; scratch space comes
 *     from a caller-provided workspace sized by the matching *_workspace_size.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = default stream) and
 *     the call returns without synchronising.  No entry point synchronises the
 *     host, so a step can be captured in a HIP graph.
 *   - Arguments are validated before any HIP call.  A failed check returns a
 *     status code and enqueues nothing; moev_last_error() then describes it.
 *     T == 0 (or B == 0) is a valid no-op.  Indices a kernel reads from device
 *     memory (token ids, expert ids, pair ids) are a caller contract: a value
 *     out of range is clamped so that every memory access stays in bounds, and
 *     the result is then unspecified.
 *   - After the launches, a failure reported by hipGetLastError() is returned
 *     as MOEV_ERR_HIP.
 *   - Calls on one stream run in order; concurrent calls on different streams
 *     must not share output or workspace buffers.
 *
 * Shapes: T tokens, H hidden, E routed experts, k routed experts per token,
 * ns shared experts, G = E + ns expert groups (routed 0..E-1, shared E..G-1),
 * S = k + ns slots per token, I expert intermediate width, V vocabulary.
 * Limits: 1 <= E <= 64, 1 <= k <= E, 0 <= ns <= 8, H and I multiples of 64,
 * 64 <= H <= 3072, 64 <= I <= 8192, T * S < 2^31.
 * Weight/operand type `dt`: MOEV_BF16 (bf16 bit patterns, GEMMs on bf16 MFMA
 * with fp32 accumulation) or MOEV_F32 (fp32 MFMA).  Residual stream, router
 * weights out, expert outputs and logits are always fp32.
 */
#ifndef MOEV_H
#define MOEV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOEV_OK = 0,
  MOEV_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size or shape */
  MOEV_ERR_UNSUPPORTED = 2, /* shape outside the limits above, unknown dtype */
  MOEV_ERR_WORKSPACE = 3,   /* workspace pointer null or too small */
  MOEV_ERR_HIP = 4          /* the HIP runtime reported an error */
} moev_status;

typedef enum { MOEV_F32 = 0, MOEV_BF16 = 1 } moev_dtype;

/* Text for a status code (static storage). */
const char* moev_status_string(int status);
/* Detail of the last failed call on this host thread ("" if none). */
const char* moev_last_error(void);
/* Library version, major * 10000 + minor * 100 + patch. */
int moev_version(void);

/*
 * Fragment-packed weights.  Every expert and LM-head weight argument below
 * (w_gate, w_up, w_down, w_lm, and the same fields of moev_model) is taken in
 * this layout, made from row-major [G, N, K] by moev_pack_weights: for group
 * g, row tile t (rows 16t..16t+15, rows past N zero) and K block b (columns
 * 32b..32b+31), the 512 elements
 *   packed[((g*ceil(N/16) + t)*(K/32) + b)*512 + lane*8 + e]
 *     = W[g][16t + lane % 16][32b + 8*(lane / 16) + e],   lane < 64, e < 8
 * are the 64 lanes' MFMA A fragments of that 16x32 block, stored
 * contiguously, with the blocks of a tile adjacent along K.  A wavefront then
 * streams one contiguous region of HBM per 16-row tile.
 * moev_packed_size: bytes of the packed form (0 for invalid arguments).
 * moev_pack_weights: src dt [G, N, K] row-major -> dst packed; K % 32 == 0.
 */
size_t moev_packed_size(int G, int N, int K, int dt);
moev_status moev_pack_weights(const void* src, void* dst, int G, int N, int K, int dt,
                              void* stream);

/*
 * moe_embed -- residual stream input: h_out[t, :] = emb[tokens[t], :] as fp32.
 *   tokens  int32 [T] device, each in [0, V)
 *   emb     dt [V, H] device
 *   h_out   fp32 [T, H] device (written)
 * Glue in front of the decoder layers; the pages do not describe the
 * embedding, and the synthetic decoder uses an untied table.
 */
moev_status moe_embed(const int32_t* tokens, const void* emb, int T, int H, int V, int dt,
                      float* h_out, void* stream);

/*
 * moe_route -- pre-norm RMSNorm and the top-k router of one MoE layer.
 * [P1] "The speed comes from three layers working together": each token is
 * routed to the top 6 of 64 routed experts.
 *   x = h / sqrt(mean(h^2) + eps) * norm_w          (fp32)
 *   logits = x . w_router^T (+ bias)                (fp32, x unrounded)
 *   topk_idx[t, r] = expert with the r-th largest logit (ties: lower index),
 *   topk_w[t, r]   = softmax(logits)[that expert] renormalised over the k
 *                    chosen experts (the k weights sum to 1).
 *   h        fp32 [T, H]
 *   norm_w   dt [H] or NULL (gain 1)
 *   w_router dt [E, H]
 *   bias     fp32 [E] or NULL (added to the logits before softmax)
 *   x_out    dt [T, H] (written): x rounded to dt, the expert GEMM operand
 *   topk_idx int32 [T, k], topk_w fp32 [T, k] (written, rank order)
 *   logits_out fp32 [T, E] or NULL (written when non-NULL; for checking)
 */
moev_status moe_route(const float* h, const void* norm_w, float eps, const void* w_router,
                      const float* bias, int T, int H, int E, int k, int dt, void* x_out,
                      int32_t* topk_idx, float* topk_w, float* logits_out, void* stream);

/*
 * moe_permute -- group the (token, slot) pairs by expert.
 * [P1] "The speed comes from three layers working together": each token
 * goes to its top 6 of the 64 routed experts and to the two shared experts,
 * so each expert's FFN runs over the subset of tokens that chose it.  The
 * pages do not describe the dispatch; this call is the plain stable counting
 * sort that lets each expert's GEMM read its tokens as one contiguous
 * segment.  It returns no tile list: the grouped GEMMs derive their tile
 * schedule on the device from group_offsets.
 * Pair p = t*S + slot.  Slot r < k belongs to routed expert topk_idx[t, r];
 * slot k+s to shared expert s (group E+s), which therefore holds every token.
 *   group_offsets int32 [G+1] (written): exclusive prefix sum of group sizes
 *   sorted_src    int32 [T*S] (written): pair ids, group by group, increasing
 *                 pair id within a group (a stable counting sort)
 */
moev_status moe_permute(const int32_t* topk_idx, int T, int k, int E, int ns,
                        int32_t* group_offsets, int32_t* sorted_src, void* stream);

/*
 * moe_grouped_ffn -- SwiGLU experts over the permuted pairs, weighted.
 * [P1] same section: 64 routed and two shared experts; shared experts are
 * always on.  For every pair (t, slot) in group g:
 *   a = SiLU(w_gate[g] . x[t]) * (w_up[g] . x[t])   (a rounded to dt)
 *   y_slots[t, slot, :] = wgt * (w_down[g] . a)
 * with wgt = topk_w[t, slot] for a routed slot and 1 for a shared slot.
 *   x        dt [T, H] (moe_route's x_out)
 *   sorted_src, group_offsets from moe_permute
 *   topk_w   fp32 [T, k]
 *   w_gate, w_up  dt [G, I, H];  w_down dt [G, H, I]  (shared experts last),
 *            all fragment-packed
 *   y_slots  fp32 [T, S, H] (written, every slot)
 *   ws       workspace of moe_grouped_ffn_workspace_size() bytes
 * Each output element is a fixed-order fp32 sum, so a token's result does not
 * depend on the other tokens in the batch.
 */
size_t moe_grouped_ffn_workspace_size(int T, int I, int k, int ns, int dt);
moev_status moe_grouped_ffn(const void* x, const int32_t* sorted_src, const int32_t* group_offsets,
                            const float* topk_w, const void* w_gate, const void* w_up,
                            const void* w_down, int T, int H, int I, int E, int k, int ns, int dt,
                            float* y_slots, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_grouped_ffn_noalloc -- moe_grouped_ffn with no workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  The SwiGLU
 * activations go to a scratch array of MOEV_NOALLOC_SCRATCH_BYTES (16 MiB)
 * that the library keeps in the memory of each GPU it runs on until the
 * process ends; its device address is looked up (hipGetSymbolAddress) on the
 * first call on each device, so make that first call outside graph capture.
 * Nothing is allocated or freed by the call.  Arguments, results and every
 * other check are those of moe_grouped_ffn.  A call whose activations,
 * moe_grouped_ffn_workspace_size(T, I, k, ns, dt) bytes, exceed the scratch
 * (for the decoder's I = 896, k + ns = 8, bf16: T > 1170) returns
 * MOEV_ERR_WORKSPACE before any HIP call.  All calls on one GPU share the
 * array: calls on one stream run in order and are safe, calls that overlap
 * in time on one GPU (several streams, several host threads) race and give
 * undefined results.  Nothing in the scratch needs to start at zero; it keeps
 * the last call's activations.
 */
#define MOEV_NOALLOC_SCRATCH_BYTES (16u << 20)
moev_status moe_grouped_ffn_noalloc(const void* x, const int32_t* sorted_src, const int32_t* group_offsets,
                                    const float* topk_w, const void* w_gate, const void* w_up,
                                    const void* w_down, int T, int H, int I, int E, int k, int ns, int dt,
                                    float* y_slots, void* stream);

/*
 * The two stages of moe_grouped_ffn as separate calls (same kernels).
 * moe_ffn_gate_up: act[j, :] = SiLU(w_gate[g] . x[t]) * (w_up[g] . x[t]),
 *   rounded to dt, for every row j of the sorted pair order (pair
 *   sorted_src[j] = t*S + slot, j in group g's segment).  act: dt [T*S, I].
 * moe_ffn_down: y_slots[t, slot, :] = wgt * (w_down[g] . act[j, :]) for the
 *   same rows, wgt as in moe_grouped_ffn.
 */
moev_status moe_ffn_gate_up(const void* x, const int32_t* sorted_src, const int32_t* group_offsets,
                            const void* w_gate, const void* w_up, int T, int H, int I, int E,
                            int k, int ns, int dt, void* act, void* stream);
moev_status moe_ffn_down(const void* act, const int32_t* sorted_src, const int32_t* group_offsets,
                         const float* topk_w, const void* w_down, int T, int H, int I, int E,
                         int k, int ns, int dt, float* y_slots, void* stream);

/*
 * moe_combine -- residual add of every slot's expert output.
 * [P1] "The speed comes from three layers working together": a token's MoE
 * output is the mix of its chosen experts' outputs (weighted by the
 * router's renormalised gates, already applied by moe_grouped_ffn) plus the
 * always-on shared experts; in the pre-norm decoder it is added to the
 * residual stream.  Summation order is fixed:
 *   h_out[t, :] = h_in[t, :] + sum_{slot = 0..S-1} y_slots[t, slot, :]
 * summed in slot order (routed by rank, then shared).  h_in NULL: no residual.
 * h_out may alias h_in.
 */
moev_status moe_combine(const float* y_slots, const float* h_in, int T, int H, int S,
                        float* h_out, void* stream);

/*
 * lmhead_argmax -- final RMSNorm, LM head and greedy token.
 * Greedy decoding is the rule the verification must reproduce ([P1] "Why
 * FastMTP fits OCR particularly well"; [P2] "What the speed claims actually
 * measure").
 *   x = RMSNorm(h) * norm_f rounded to dt;  logits = w_lm . x  (fp32 acc)
 *   argmax_out[t] = lowest index of the largest logit
 *   h        fp32 [T, H];  norm_f dt [H] or NULL;  w_lm dt [V, H] fragment-packed
 *   argmax_out int32 [T] (written);  max_out fp32 [T] or NULL
 *   logits_out fp32 [T, V] or NULL (written when non-NULL; for checking)
 *   ws       workspace of lmhead_argmax_workspace_size() bytes
 */
size_t lmhead_argmax_workspace_size(int T, int H, int V, int dt);
moev_status lmhead_argmax(const float* h, const void* norm_f, float eps, const void* w_lm,
                          int T, int H, int V, int dt, int32_t* argmax_out, float* max_out,
                          float* logits_out, void* ws, size_t ws_bytes, void* stream);

/*
 * mtp_verify -- FastMTP greedy prefix acceptance ([P1] "The speed comes from
 * three layers working together" and "Why FastMTP fits OCR particularly
 * well"; [P3] "Scope & Claims", Section 3.1 / Eq. 2).
 *   tokens[b, :] = (last committed token, d_1 .. d_K)   int32 [B, K+1]
 *   greedy[b, j] = greedy token after tokens[b, j]        int32 [B, K+1]
 *   n_accept[b]  = largest n <= K with d_i == greedy[b, i-1] for all i <= n
 *   commit[b, :] = d_1 .. d_n, greedy[b, n], then -1 padding   int32 [B, K+1]
 *   commit_len[b] = n + 1;  next_last[b] = greedy[b, n]
 * commit_len / next_last may be NULL.
 */
moev_status mtp_verify(const int32_t* tokens, const int32_t* greedy, int B, int K,
                       int32_t* n_accept, int32_t* commit, int32_t* commit_len,
                       int32_t* next_last, void* stream);

/* ------------------------------------------------------------------------ */
/* Whole verify step: embed -> n_layers x (route, permute, grouped FFN,
 * combine) -> lmhead_argmax -> mtp_verify, enqueued on one stream.          */

typedef struct moev_layer_weights {
  const void* norm;     /* dt [H] or NULL */
  const void* w_router; /* dt [E, H] */
  const float* bias;    /* fp32 [E] or NULL */
  const void* w_gate;   /* dt [G, I, H], fragment-packed */
  const void* w_up;     /* dt [G, I, H], fragment-packed */
  const void* w_down;   /* dt [G, H, I], fragment-packed */
} moev_layer_weights;

typedef struct moev_model {
  int hidden, n_routed, inter, top_k, n_shared, vocab, n_layers;
  int dtype;    /* moev_dtype */
  float eps;    /* RMSNorm epsilon */
  const void* emb;    /* dt [V, H] */
  const void* norm_f; /* dt [H] or NULL */
  const void* w_lm;   /* dt [V, H], fragment-packed */
  const moev_layer_weights* layers; /* host array of n_layers entries */
} moev_model;

/*
 * moev_verify_step -- one FastMTP verification pass of B sequences, each
 * bringing its last committed token and K drafts (T = B*(K+1) tokens).
 *   tokens   int32 [B, K+1] device
 *   greedy   int32 [B, K+1] (written): greedy token after every input token
 *   n_accept, commit, commit_len, next_last: as mtp_verify
 *   ws       workspace of moev_verify_step_workspace_size() bytes
 * K = 0 is plain greedy decoding of one token per sequence.  Needs k + ns <= 16
 * (each layer's residual add is folded into the next router launch).
 */
size_t moev_verify_step_workspace_size(const moev_model* m, int B, int K);
moev_status moev_verify_step(const moev_model* m, const int32_t* tokens, int B, int K,
                             int32_t* greedy, int32_t* n_accept, int32_t* commit,
                             int32_t* commit_len, int32_t* next_last, void* ws, size_t ws_bytes,
                             void* stream);

/*
 * moev_verify_step_probed -- moev_verify_step with timing events: for every
 * layer l < probe->n (and for the head when stage == MOEV_STAGE_HEAD, using
 * index 0), records probe->before[l] / probe->after[l] on `stream` right
 * before / after the launches of stage `probe->stage`.  Events are
 * hipEvent_t handles created by the caller; probe == NULL is
 * moev_verify_step.  For measurement only.
 */
enum {
  MOEV_STAGE_ROUTE = 0, MOEV_STAGE_PERMUTE = 1, MOEV_STAGE_GATE_UP = 2, MOEV_STAGE_DOWN = 3,
  MOEV_STAGE_COMBINE = 4, MOEV_STAGE_HEAD = 5
};
typedef struct moev_step_probe {
  int stage;
  int n;
  void* const* before;
  void* const* after;
} moev_step_probe;
moev_status moev_verify_step_probed(const moev_model* m, const int32_t* tokens, int B, int K,
                                    int32_t* greedy, int32_t* n_accept, int32_t* commit,
                                    int32_t* commit_len, int32_t* next_last, void* ws,
                                    size_t ws_bytes, const moev_step_probe* probe, void* stream);

/*
 * moev_prefill -- a page-shaped prompt through the whole decoder ("What the
 * speed claims actually measure" on the aipolix.com page and "Start with the
 * result" on kg.zhiyong.dev: a page brings about a thousand visual tokens plus
 * the prompt before the first decode step).  Every one of the n_seq * seq_len
 * prompt rows runs through all n_layers layers (route, grouped FFN, combine);
 * the final norm, LM head and arg max run only for each sequence's last row.
 *   tokens      int32 [n_seq, seq_len] device (row r = i * seq_len + j)
 *   next_token  int32 [n_seq] (written): greedy token after token[i, seq_len-1]
 *   h_out       fp32 [n_seq * seq_len, H] or NULL (written): the residual
 *               stream after the last layer, before the final norm
 *   ws          workspace of moev_prefill_workspace_size() bytes, 16-byte aligned
 * The decoder has no attention (each row's result depends on its own token
 * only), so next_token[i] equals the verify step's greedy token for the same
 * token, bit for bit.  n_seq = 0 is a no-op; seq_len >= 1.  Same model limits
 * as moev_verify_step.  Nothing allocates or synchronises.
 */
size_t moev_prefill_workspace_size(const moev_model* m, int n_seq, int seq_len);
moev_status moev_prefill(const moev_model* m, const int32_t* tokens, int n_seq, int seq_len,
                         int32_t* next_token, float* h_out, void* ws, size_t ws_bytes, void* stream);
/* moev_prefill with the timing events of moev_verify_step_probed (measurement only). */
moev_status moev_prefill_probed(const moev_model* m, const int32_t* tokens, int n_seq, int seq_len,
                                int32_t* next_token, float* h_out, void* ws, size_t ws_bytes,
                                const moev_step_probe* probe, void* stream);

/*
 * FastMTP draft block ("The speed comes from three layers working together" on
 * kg.zhiyong.dev: one dense draft block proposes up to three tokens, applied
 * recursively; the aipolix.com page's "A document parser, not just a text
 * recognizer": a shared block drafts three positions).  The pages give no
 * more of its structure; this library computes, for draft step j = 1..K from
 * the hidden state z (fp32 [H]) and token t of step j-1:
 *   u   = [RMSNorm(z) * norm_z ; RMSNorm(Emb[t]) * norm_e]        (2H)
 *   z'  = W_p u                                                   (H)
 *   z_j = z' + W_down (SiLU(W_gate x) * (W_up x)),  x = RMSNorm(z') * norm_ffn
 *   t_j = arg max W_lm (RMSNorm(z_j) * norm_out)  (the model's LM head and
 *         embedding; lowest index on exact ties)
 * Weights are stored as the slices the grouped GEMMs take, each
 * fragment-packed by moev_pack_weights:
 *   w_proj [2][H][H]  slice g = columns g*H .. (g+1)*H-1 of W_p (g = 0: the
 *                     hidden-state half, g = 1: the embedding half)
 *   w_gate, w_up [n][I][H] and w_down [n][H][I]: the dense SwiGLU of width n*I
 *                     split along its intermediate axis (I = the model's inter)
 * norm_* are dt [H] or NULL (ones).  n_slices in [1, 16].
 */
typedef struct moev_draft_weights {
  const void* norm_z;
  const void* norm_e;
  const void* w_proj;
  const void* norm_ffn;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const void* norm_out;
  int n_slices;
} moev_draft_weights;

/*
 * moev_draft -- K recursive draft steps for B sequences.
 *   z0      fp32 [B, H] device: hidden state entering step 1
 *   t0      int32 [B] device: token entering step 1
 *   drafts  int32 [B, K] (written): t_1 .. t_K
 *   z_out   fp32 [B, H] or NULL (written): z_K
 *   ws      workspace of moev_draft_workspace_size() bytes, 16-byte aligned
 * B = 0 or K = 0 is a no-op.  Token ids outside [0, V) are clamped.  Nothing
 * allocates or synchronises.
 */
size_t moev_draft_workspace_size(const moev_model* m, const moev_draft_weights* d, int B);
moev_status moev_draft(const moev_model* m, const moev_draft_weights* d, const float* z0,
                       const int32_t* t0, int B, int K, int32_t* drafts, float* z_out, void* ws,
                       size_t ws_bytes, void* stream);

/*
 * moev_spec_step -- one whole speculative step on the device: the verify pass
 * of moev_verify_step on tokens [B, K+1], then K draft steps for the next
 * pass, started from the verifier's final residual state at each sequence's
 * last accepted position (row b*(K+1) + n_accept[b], whose greedy token is
 * next_last[b]) and from next_last[b] itself.
 *   greedy, n_accept, commit, commit_len: as moev_verify_step
 *   next_tokens int32 [B, K+1] (written): next_last, then the K drafts -- the
 *               tokens argument of the next call
 *   h_final     fp32 [B*(K+1), H] or NULL (written): the residual stream after
 *               the last layer, before the final norm
 *   ws          workspace of moev_spec_step_workspace_size() bytes
 * K >= 1.  A chain of calls, each fed the previous next_tokens, runs the
 * speculative loop without the host.
 */
size_t moev_spec_step_workspace_size(const moev_model* m, const moev_draft_weights* d, int B,
                                     int K);
moev_status moev_spec_step(const moev_model* m, const moev_draft_weights* d,
                           const int32_t* tokens, int B, int K, int32_t* greedy,
                           int32_t* n_accept, int32_t* commit, int32_t* commit_len,
                           int32_t* next_tokens, float* h_final, void* ws, size_t ws_bytes,
                           void* stream);

/*
 * moev_attn_decode -- causal multi-head attention of each sequence's verify
 * rows over its cached prefix (the decoder's attention sublayer in a verify
 * pass: "The speed comes from three layers working together" on
 * kg.zhiyong.dev has the main decoder check all K drafts in one pass; the
 * pages do not describe its attention, so this is plain multi-head attention,
 * scale 1/sqrt(head width), no positional rotation).  Row i of sequence b is
 * at position pos[b] + i and sees positions 0 .. pos[b] + i; per head
 * (columns h*D .. (h+1)*D - 1, D = H / n_heads):
 *   out = sum_j softmax_j(q . k_j / sqrt(D)) v_j
 *   q        fp32 [B*rows, H] device (row b*rows + i)
 *   k_cache, v_cache  dt [B, n_heads, max_len, D] device, head-major: the
 *            prefix at positions 0 .. pos[b]-1 and the verify rows' own keys
 *            and values at pos[b] .. pos[b]+rows-1 (caller-owned; not
 *            modified)
 *   pos      int32 [B] device; clamped on the device so that at most max_len
 *            positions are read
 *   out      fp32 [B*rows, H] device (written)
 *   ws       workspace of moev_attn_decode_workspace_size() bytes, 16-byte
 *            aligned (each (sequence, head) runs as several workgroups over
 *            fixed position chunks whose softmax states are merged in order)
 * 1 <= rows <= 16; D in {64, 128, 256}.  B = 0 is a no-op.  Nothing
 * allocates or synchronises.
 */
size_t moev_attn_decode_workspace_size(int B, int rows, int H, int n_heads);
moev_status moev_attn_decode(const float* q, const void* k_cache, const void* v_cache, const int32_t* pos,
                             int B, int rows, int max_len, int H, int n_heads, int dt, float* out,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * moev_verify_step_attn -- the verify pass of moev_verify_step through a
 * decoder whose layers each run a causal attention sublayer before the MoE
 * sublayer (the main model checks all K drafts in one pass, "The speed comes
 * from three layers working together" on kg.zhiyong.dev; the pages do not
 * describe the attention, so it is plain pre-norm multi-head attention, unit
 * norm gain, no positional rotation).  Per layer, for the rows of sequence b
 * at positions pos[b] .. pos[b]+K:
 *   x = RMSNorm(h);  [q | k | v] = x [W_q; W_k; W_v]^T
 *   k, v rounded to dt into the caches at those positions
 *   h += W_o attn(q, caches)   (moev_attn_decode), then the MoE sublayer.
 * After the head and the prefix acceptance, pos[b] += commit_len[b]: the
 * sequence's last token and its accepted drafts stay in the cache, and the
 * rows written for rejected drafts are overwritten by the next pass.
 *   attn->layers[l].w_qkv  dt [3H, H] fragment-packed (W_q, W_k, W_v stacked)
 *   attn->layers[l].w_o    dt [H, H] fragment-packed
 *   attn->layers[l].k_cache, v_cache  dt [B, n_heads, max_len, H/n_heads]
 *            device (head-major, as moev_attn_decode reads them), updated
 *   pos      int32 [B] device, read then advanced.  A sequence whose cache
 *            has no room for the pass (pos[b] < 0 or pos[b] + K + 1 >
 *            max_len) is left as it is: no cache row is written, pos[b]
 *            stays, commit_len[b] = 0, n_accept[b] = -1, its commit row is
 *            all -1 and next_last[b] = its input last token (its greedy
 *            row is unspecified); the caller retires or resets it
 *   greedy, n_accept, commit, commit_len, next_last: as moev_verify_step
 *   ws       workspace of moev_verify_step_attn_workspace_size() bytes
 * Needs B*(K+1) <= 512, K + 1 <= 16, H / n_heads in {64, 128, 256} and
 * max_len >= K + 1.  K = 0 is plain greedy decoding of one token per
 * sequence.  Nothing allocates or synchronises.
 */
typedef struct moev_attn_layer {
  const void* w_qkv;
  const void* w_o;
  void* k_cache;
  void* v_cache;
} moev_attn_layer;

typedef struct moev_attn {
  int n_heads, max_len;
  const moev_attn_layer* layers; /* host array of n_layers entries */
} moev_attn;

size_t moev_verify_step_attn_workspace_size(const moev_model* m, const moev_attn* a, int B, int K);
moev_status moev_verify_step_attn(const moev_model* m, const moev_attn* a, const int32_t* tokens,
                                  int B, int K, int32_t* pos, int32_t* greedy, int32_t* n_accept,
                                  int32_t* commit, int32_t* commit_len, int32_t* next_last,
                                  void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOEV_H */
