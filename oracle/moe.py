"""Plain float64 reference of the FastMTP verify step through the MoE decoder.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP library or its binding; inputs come from the seeded generators in
``synth`` and from the caller.

What is computed, and where it is defined
-----------------------------------------
Sources are three web pages on Jina-OCR-v1:

* [P1] "Jina AI's jina-ocr-v1 Is Selling Throughput, Not the OCR Crown"
  (kg.zhiyong.dev explainer);
* [P2] aipolix.com news analysis of Jina-OCR-v1 (document parsing, FastMTP,
  non-commercial weights);
* [P3] "Jina-OCR-v1: Efficient Document Parsing with Speculative Decoding and
  Dense Verifiable Rewards" (evolve.pub review of the arXiv paper).

1. MoE decoder layer ([P1] "The speed comes from three layers working
   together"; [P2] "A document parser, not just a text recognizer"): every
   token goes to its top-6 of 64 routed experts plus two shared experts.
   Pre-norm RMSNorm, SwiGLU experts, a softmax router renormalised over the
   chosen experts and a residual add fill in what the pages leave open
   (readings listed in the design notes).
2. Greedy head: logits = W_lm . RMSNorm(h); the greedy token is the arg max,
   lowest index on exact ties.
3. FastMTP verification ([P1] same section and "Why FastMTP fits OCR
   particularly well"; [P2] "What the speed claims actually measure"; [P3]
   "Scope & Claims", Section 3.1 / Eq. 2): each sequence brings its last
   committed token and K drafts; one pass of the main decoder yields the greedy
   token at all K+1 positions; the longest prefix of drafts that agrees with
   those greedy tokens is accepted, and the main model's own token at the first
   disagreement (or after the last draft, the bonus token) is committed too, so
   every step commits n+1 tokens.  The committed stream equals plain greedy
   decoding ("lossless").
4. FastMTP draft block ([P1] "The speed comes from three layers working
   together": one dense draft block proposes up to three tokens by being
   applied recursively; [P2] "A document parser, not just a text recognizer":
   a shared block drafts three positions; [P3] Summary / Scope & Claims,
   Section 3.1).  The pages give no more of its structure; ``draft_block``
   takes the multi-token-prediction module reading listed in the design
   notes (hidden state and next-token embedding, each RMS-normalised,
   projected to H; one pre-norm dense SwiGLU with residual; the verifier's
   LM head behind the block's own final norm).
5. Decode attention (the causal self-attention sublayer of a decoder layer,
   which the verify pass runs for its K+1 rows against each sequence's
   cached prefix; the pages name the decoder but not its attention, so
   ``attn_decode`` takes the plain multi-head reading listed in the design
   notes: no positional rotation, scale 1/sqrt(head width)).
6. tau = mean committed tokens per step; for independent per-position draft
   acceptances a_1..a_K its expectation is 1 + sum_m prod_{j<=m} a_j, which
   with Table 8's 0.830/0.663/0.636 gives the printed 2.73 ([P3] Strengths,
   speculative-decoding analysis).

Precision
---------
All arithmetic is float64.  bf16 weights enter as exact upcasts of their bit
patterns.  ``operands="bf16"`` additionally rounds (nearest, ties to even) the
activations that a bf16 contraction consumes -- the normalised hidden state
entering the expert and head GEMMs and the SwiGLU activation entering the down
projection -- which is the precision the bf16 path defines for its GEMM
operands.  ``operands="exact"`` skips those roundings.  The router always sees
the unrounded normalised state.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

__all__ = [
    "to_f64", "round_bf16", "rmsnorm", "silu", "softmax", "route", "route_gap",
    "pair_groups", "permute", "grouped_ffn", "combine", "moe_layer",
    "embed", "lm_head", "first_argmax", "mtp_verify", "model_greedy",
    "verify_step", "greedy_rollout", "expected_tau", "acceptance_rate",
    "draft_dense", "draft_block", "attn_decode", "attn_sublayer", "cached_greedy",
    "cached_verify_step", "cached_rollout",
]


# ---------------------------------------------------------------------------
# number formats

def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored tensor -> float64.  "bf16": uint16 bit patterns (the bf16 value is
    the float32 whose upper half is those bits); "f32": float32 values; "f64":
    float64 values (the oracle's own caches)."""
    a = np.asarray(a)
    if dtype == "bf16":
        assert a.dtype == np.uint16
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return a.astype(np.float64)
    if dtype == "f64":
        return a.astype(np.float64)
    raise ValueError(dtype)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (8 significant bits, ties to
    even), returned as float64.  Finite, in-range inputs; subnormals use the
    fixed bf16 subnormal spacing 2^-133."""
    x = np.asarray(x, dtype=np.float64)
    m, p = np.frexp(x)                # x = m * 2^p, 0.5 <= |m| < 1
    p = np.maximum(p, -125)           # below the normal range the spacing is fixed
    q = np.ldexp(x, 8 - p)            # |q| < 256: bf16 keeps the integer part
    return np.ldexp(np.rint(q), p - 8)  # rint rounds half to even


# ---------------------------------------------------------------------------
# layer pieces

def rmsnorm(h: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """x = h / sqrt(mean(h^2) + eps) * gamma, over the last axis."""
    h = np.asarray(h, dtype=np.float64)
    ms = np.mean(h * h, axis=-1, keepdims=True)
    return h / np.sqrt(ms + eps) * gamma


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + e^-z)."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def softmax(l: np.ndarray) -> np.ndarray:
    e = np.exp(l - l.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def route(x: np.ndarray, w_router: np.ndarray, k: int, bias: Optional[np.ndarray] = None):
    """Router: logits = x W_r^T (+ bias); p = softmax over the routed experts;
    the k experts with the largest p (lower expert index first on equal p), in
    rank order; their weights p / sum of the chosen p (so they sum to 1).

    Returns (idx int32 [T,k], w float64 [T,k], logits float64 [T,E]).
    """
    logits = np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T
    if bias is not None:
        logits = logits + np.asarray(bias, np.float64)[None, :]
    p = softmax(logits)
    T, E = p.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-p[t, e], e))
        sel = order[:k]
        idx[t] = sel
        w[t] = p[t, sel] / p[t, sel].sum()
    return idx, w, logits


def route_gap(logits: np.ndarray, k: int) -> np.ndarray:
    """Per token, the gap between the k-th and (k+1)-th largest router logit
    (inf when every expert is chosen).  Small gaps mark tokens whose chosen set
    can flip under rounding."""
    s = -np.sort(-np.asarray(logits, np.float64), axis=-1)
    if k >= s.shape[-1]:
        return np.full(s.shape[0], np.inf)
    return s[:, k - 1] - s[:, k]


def pair_groups(idx: np.ndarray, n_routed: int, n_shared: int) -> np.ndarray:
    """Group of every (token, slot) pair, flattened as pair p = t*(k+ns) + slot.
    Slots 0..k-1 go to the routed experts the router chose (rank order); slot
    k+s goes to shared expert s, which is group n_routed + s."""
    T, k = idx.shape
    g = np.empty((T, k + n_shared), np.int64)
    g[:, :k] = idx
    for s in range(n_shared):
        g[:, k + s] = n_routed + s
    return g.reshape(-1)


def permute(idx: np.ndarray, n_routed: int, n_shared: int):
    """Counting sort of the pairs by group, stable in the pair id.

    Returns (offsets int32 [G+1]: exclusive prefix sum of the group sizes;
    sorted_src int32 [P]: pair ids, group by group, increasing within a group).
    """
    groups = pair_groups(idx, n_routed, n_shared)
    G = n_routed + n_shared
    counts = [0] * G
    for g in groups:
        counts[g] += 1
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    cursor = list(offsets[:-1])
    sorted_src = np.empty(len(groups), np.int32)
    for p, g in enumerate(groups):
        sorted_src[cursor[g]] = p
        cursor[g] += 1
    return np.asarray(offsets, np.int32), sorted_src


def grouped_ffn(x_op: np.ndarray, sorted_src: np.ndarray, offsets: np.ndarray,
                topk_w: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray,
                w_down: np.ndarray, dtype: str, k: int, n_shared: int,
                round_act: bool = False) -> np.ndarray:
    """Expert outputs per (token, slot).

    For group g and each of its pairs (t, slot):
      a = SiLU(W_gate[g] x_t) * (W_up[g] x_t)      (rounded to bf16 if round_act)
      y_slots[t, slot] = w * (W_down[g] a)
    with w the router weight of that slot, or 1 for a shared-expert slot.
    ``x_op`` holds the operand values the expert contractions consume.
    Returns float64 [T, k+ns, H].
    """
    x_op = np.asarray(x_op, np.float64)
    T, H = x_op.shape
    S = k + n_shared
    y = np.zeros((T, S, H), np.float64)
    for g in range(len(offsets) - 1):
        a, b = int(offsets[g]), int(offsets[g + 1])
        if a == b:
            continue
        pairs = np.asarray(sorted_src[a:b], np.int64)
        t, s = pairs // S, pairs % S
        X = x_op[t]
        wg, wu, wd = to_f64(w_gate[g], dtype), to_f64(w_up[g], dtype), to_f64(w_down[g], dtype)
        act = silu(X @ wg.T) * (X @ wu.T)
        if round_act:
            act = round_bf16(act)
        out = act @ wd.T
        scale = np.ones(len(pairs))
        routed = s < k
        scale[routed] = np.asarray(topk_w, np.float64)[t[routed], s[routed]]
        y[t, s] = scale[:, None] * out
    return y


def combine(y_slots: np.ndarray, h_in: Optional[np.ndarray]) -> np.ndarray:
    """h_out = h_in + sum over every slot's expert output."""
    y = np.asarray(y_slots, np.float64).sum(axis=1)
    return y if h_in is None else np.asarray(h_in, np.float64) + y


def moe_layer(h: np.ndarray, layer: dict, dtype: str, k: int, n_routed: int, n_shared: int,
              eps: float, operands: str = "bf16") -> dict:
    """One pre-norm MoE layer with residual, keeping every stage's value.

    x = RMSNorm(h); route(x); permute; grouped SwiGLU experts; h_out = h + sum.
    """
    rnd = operands == "bf16" and dtype == "bf16"
    gamma = to_f64(layer["norm"], dtype)
    x = rmsnorm(h, gamma, eps)
    x_op = round_bf16(x) if rnd else x
    idx, w, logits = route(x, to_f64(layer["w_router"], dtype), k, layer.get("bias"))
    offsets, sorted_src = permute(idx, n_routed, n_shared)
    y = grouped_ffn(x_op, sorted_src, offsets, w, layer["w_gate"], layer["w_up"],
                    layer["w_down"], dtype, k, n_shared, round_act=rnd)
    return {"x": x, "x_op": x_op, "idx": idx, "w": w, "logits": logits,
            "gap": route_gap(logits, k), "offsets": offsets, "sorted_src": sorted_src,
            "y_slots": y, "h_out": combine(y, h)}


# ---------------------------------------------------------------------------
# head and verification

def embed(tokens: np.ndarray, emb: np.ndarray, dtype: str) -> np.ndarray:
    """Residual stream input: the embedding row of each token."""
    return to_f64(np.asarray(emb)[np.asarray(tokens, np.int64)], dtype)


def first_argmax(rows: np.ndarray) -> np.ndarray:
    """Smallest index attaining each row's maximum."""
    rows = np.asarray(rows)
    return (rows == rows.max(axis=-1, keepdims=True)).argmax(axis=-1)


def lm_head(h: np.ndarray, norm_f: np.ndarray, w_lm: np.ndarray, dtype: str, eps: float,
            operands: str = "bf16", keep_logits: bool = False, chunk: int = 16384) -> dict:
    """Greedy head: logits = W_lm . RMSNorm(h); greedy token = arg max (lowest
    index on ties).  Also returns the max logit and the gap between the two
    largest logits (0 when the maximum is shared).  Works through the
    vocabulary in row chunks to bound memory."""
    x = rmsnorm(h, to_f64(norm_f, dtype), eps)
    if operands == "bf16" and dtype == "bf16":
        x = round_bf16(x)
    T = x.shape[0]
    V = np.asarray(w_lm).shape[0]
    best = np.full(T, -np.inf)
    second = np.full(T, -np.inf)
    arg = np.zeros(T, np.int64)
    logits_all = np.empty((T, V)) if keep_logits else None
    for c0 in range(0, V, chunk):
        lg = x @ to_f64(np.asarray(w_lm)[c0:c0 + chunk], dtype).T
        if keep_logits:
            logits_all[:, c0:c0 + lg.shape[1]] = lg
        cmax = lg.max(axis=1)
        carg = first_argmax(lg) + c0
        # second largest inside the chunk: max after removing one copy of the max
        tmp = lg.copy()
        tmp[np.arange(T), carg - c0] = -np.inf
        csec = tmp.max(axis=1) if lg.shape[1] > 1 else np.full(T, -np.inf)
        newer = cmax > best          # strict: an earlier chunk keeps equal maxima
        second = np.where(newer, np.maximum(best, csec), np.maximum(second, cmax))
        best = np.where(newer, cmax, best)
        arg = np.where(newer, carg, arg)
    out = {"x": x, "argmax": arg.astype(np.int32), "max": best, "gap": best - second}
    if keep_logits:
        out["logits"] = logits_all
    return out


def mtp_verify(tokens: np.ndarray, greedy: np.ndarray):
    """Greedy prefix acceptance for one verify pass.

    tokens[b] = (last committed token, d_1 .. d_K); greedy[b, j] = the main
    model's greedy token at position j.  n_b is the largest m <= K with
    d_i == greedy[b, i-1] for every i <= m.  Commit d_1..d_n then greedy[b, n]
    (the correction at the first disagreement, or the bonus token when n == K).
    Returns (n_accept [B], commit [B, K+1] padded with -1, commit_len [B] = n+1,
    next_last [B] = greedy[b, n]).
    """
    tokens = np.asarray(tokens)
    greedy = np.asarray(greedy)
    B, K1 = tokens.shape
    K = K1 - 1
    n_acc = np.zeros(B, np.int32)
    commit = np.full((B, K1), -1, np.int32)
    for b in range(B):
        n = 0
        while n < K and tokens[b, n + 1] == greedy[b, n]:
            n += 1
        n_acc[b] = n
        commit[b, :n] = tokens[b, 1:n + 1]
        commit[b, n] = greedy[b, n]
    last = greedy[np.arange(B), n_acc].astype(np.int32)
    return n_acc, commit, n_acc + 1, last


def model_greedy(tokens: np.ndarray, model: dict, operands: str = "bf16",
                 keep: bool = False) -> dict:
    """Greedy token for each input token of the synthetic decoder (no
    attention: every position is computed independently).  Returns argmax,
    head gap, and the smallest router gap seen by each token over the layers;
    with ``keep`` also every layer's stage values."""
    shape = model["shape"]
    dt = model["dtype"]
    tokens = np.asarray(tokens, np.int64).reshape(-1)
    h = embed(tokens, model["emb"], dt)
    min_rgap = np.full(len(tokens), np.inf)
    stages = []
    for layer in model["layers"]:
        st = moe_layer(h, layer, dt, shape.top_k, shape.n_routed, shape.n_shared,
                       shape.eps, operands)
        min_rgap = np.minimum(min_rgap, st["gap"])
        h = st["h_out"]
        if keep:
            stages.append(st)
    head = lm_head(h, model["norm_f"], model["w_lm"], dt, shape.eps, operands)
    out = {"argmax": head["argmax"], "gap": head["gap"], "max": head["max"],
           "router_gap": min_rgap, "h": h}
    if keep:
        out["stages"] = stages
    return out


def verify_step(last: np.ndarray, drafts: np.ndarray, model: dict, operands: str = "bf16") -> dict:
    """One FastMTP verify pass: run (last, d_1..d_K) of every sequence through
    the decoder as one batch, then accept (see ``mtp_verify``)."""
    last = np.asarray(last, np.int32).reshape(-1, 1)
    drafts = np.asarray(drafts, np.int32).reshape(last.shape[0], -1)
    tokens = np.concatenate([last, drafts], axis=1)
    B, K1 = tokens.shape
    fwd = model_greedy(tokens, model, operands)
    greedy = fwd["argmax"].reshape(B, K1)
    n_acc, commit, clen, nxt = mtp_verify(tokens, greedy)
    return {"tokens": tokens, "greedy": greedy, "n_accept": n_acc, "commit": commit,
            "commit_len": clen, "next_last": nxt, "gap": fwd["gap"].reshape(B, K1),
            "router_gap": fwd["router_gap"].reshape(B, K1)}


def greedy_rollout(last: np.ndarray, model: dict, n_tokens: int, operands: str = "bf16") -> np.ndarray:
    """Plain greedy decoding: n_tokens successive greedy tokens after each
    sequence's last token.  Returns int32 [B, n_tokens]."""
    cur = np.asarray(last, np.int32).reshape(-1)
    out = np.empty((cur.shape[0], n_tokens), np.int32)
    for i in range(n_tokens):
        cur = model_greedy(cur, model, operands)["argmax"].astype(np.int32)
        out[:, i] = cur
    return out


# ---------------------------------------------------------------------------
# FastMTP draft block

def draft_dense(draft: dict) -> dict:
    """The dense matrices of a draft block stored as slices: W_p [H, 2H] =
    [w_proj[0] | w_proj[1]], W_gate / W_up [n*I, H] = the slices stacked along
    the intermediate axis, W_down [H, n*I] = the down slices side by side."""
    dt = draft["dtype"]
    wp = to_f64(draft["w_proj"], dt)
    return {
        "w_p": np.concatenate([wp[0], wp[1]], axis=1),
        "w_gate": np.concatenate(list(to_f64(draft["w_gate"], dt)), axis=0),
        "w_up": np.concatenate(list(to_f64(draft["w_up"], dt)), axis=0),
        "w_down": np.concatenate(list(to_f64(draft["w_down"], dt)), axis=1),
    }


def draft_block(z0: np.ndarray, t0: np.ndarray, draft: dict, model: dict, K: int,
                operands: str = "bf16") -> dict:
    """K recursive steps of the FastMTP draft block (see the module notes).

    Step j (j = 1..K), from the hidden state z_{j-1} (z_0 = the verifier's
    final residual state at the position that produced the last committed
    token) and the token t_{j-1} (t_0 = that token):
        u   = [RMSNorm(z_{j-1}) * norm_z ; RMSNorm(Emb[t_{j-1}]) * norm_e]
        z'  = W_p u
        x   = RMSNorm(z') * norm_ffn
        z_j = z' + W_down (SiLU(W_gate x) * (W_up x))
        t_j = arg max W_lm (RMSNorm(z_j) * norm_out)   (lowest index on ties)
    With ``operands="bf16"`` and bf16 weights, u, x, the SwiGLU activation and
    the head's input are rounded to bf16 as the GEMMs that consume them take
    them.  Returns drafts [B, K] int32, z [B, H] (= z_K), and per step the head
    gap (``gap`` [B, K]) and z_j (``zs`` [K, B, H]).
    """
    shape = model["shape"]
    dt = model["dtype"]
    eps = shape.eps
    dd = draft_dense(draft)
    rb = (lambda a: round_bf16(a)) if (operands == "bf16" and dt == "bf16") else (lambda a: a)
    z = np.asarray(z0, np.float64)
    t = np.asarray(t0, np.int64).reshape(-1)
    B = z.shape[0]
    drafts = np.zeros((B, K), np.int32)
    gaps = np.zeros((B, K))
    zs = np.zeros((K, B, z.shape[1]))
    for j in range(K):
        u = np.concatenate([rmsnorm(z, to_f64(draft["norm_z"], dt), eps),
                            rmsnorm(embed(t, model["emb"], dt), to_f64(draft["norm_e"], dt), eps)],
                           axis=1)
        zp = rb(u) @ dd["w_p"].T
        x = rb(rmsnorm(zp, to_f64(draft["norm_ffn"], dt), eps))
        a = silu(x @ dd["w_gate"].T) * (x @ dd["w_up"].T)
        z = zp + rb(a) @ dd["w_down"].T
        head = lm_head(z, draft["norm_out"], model["w_lm"], dt, eps, operands)
        t = head["argmax"].astype(np.int64)
        drafts[:, j] = t
        gaps[:, j] = head["gap"]
        zs[j] = z
    return {"drafts": drafts, "z": z, "gap": gaps, "zs": zs}


# ---------------------------------------------------------------------------
# decode attention

def attn_decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, pos: np.ndarray,
                rows: int, n_heads: int, dtype: str) -> np.ndarray:
    """Causal multi-head attention of each sequence's verify rows over its
    cache (see the module notes).

    q [B*rows, H] (row b*rows + i is row i of sequence b, at position
    pos[b] + i); k_cache, v_cache [B, L, H] in the stored dtype, holding the
    sequence's prefix at positions 0..pos[b]-1 and the verify rows' own keys
    and values at pos[b]..pos[b]+rows-1.  Row i attends to positions
    0..pos[b]+i; per head (columns h*d .. (h+1)*d - 1, d = H / n_heads):
        o = sum_j softmax_j(q . k_j / sqrt(d)) v_j.
    Returns float64 [B*rows, H].
    """
    q = np.asarray(q, np.float64)
    B, L, H = k_cache.shape
    d = H // n_heads
    out = np.zeros((B * rows, H))
    for b in range(B):
        K = to_f64(k_cache[b], dtype)
        V = to_f64(v_cache[b], dtype)
        for i in range(rows):
            n = int(pos[b]) + i + 1
            for h in range(n_heads):
                c = slice(h * d, (h + 1) * d)
                s = K[:n, c] @ q[b * rows + i, c] / np.sqrt(d)
                p = np.exp(s - s.max())
                out[b * rows + i, c] = (p @ V[:n, c]) / p.sum()
    return out


def attn_sublayer(h: np.ndarray, attn: dict, cache: dict, pos: np.ndarray, rows: int, n_heads: int,
                  dtype: str, eps: float, operands: str = "bf16") -> np.ndarray:
    """Pre-norm causal attention sublayer with residual, for B sequences of
    ``rows`` rows (h [B*rows, H]; row i of sequence b at position pos[b] + i).

    x = RMSNorm(h) (gain 1); q, k, v = x W_q^T, x W_k^T, x W_v^T; the rows' k
    and v are written into the sequence's cache at positions pos[b] + i
    (rounded to bf16 for a bf16 model, as the cache stores them); o =
    attn_decode(q, cache); h_out = h + o W_o^T.  With ``operands="bf16"`` and
    a bf16 model, x and o are rounded to bf16 as the projections take them.
    ``cache`` = {"k", "v"}: float64 [B, L, H], updated in place.
    """
    rnd = operands == "bf16" and dtype == "bf16"
    x = rmsnorm(h, 1.0, eps)
    x_op = round_bf16(x) if rnd else x
    q = x_op @ to_f64(attn["w_q"], dtype).T
    k = x_op @ to_f64(attn["w_k"], dtype).T
    v = x_op @ to_f64(attn["w_v"], dtype).T
    if dtype == "bf16":
        k, v = round_bf16(k), round_bf16(v)
    B = len(pos)
    for b in range(B):
        for i in range(rows):
            cache["k"][b, int(pos[b]) + i] = k[b * rows + i]
            cache["v"][b, int(pos[b]) + i] = v[b * rows + i]
    o = attn_decode(q, cache["k"], cache["v"], pos, rows, n_heads, "f64")
    o_op = round_bf16(o) if rnd else o
    return h + o_op @ to_f64(attn["w_o"], dtype).T


def cached_greedy(tokens: np.ndarray, model: dict, attn: list, caches: list, pos: np.ndarray,
                  n_heads: int, operands: str = "bf16") -> dict:
    """Greedy tokens of the decoder with an attention sublayer before every
    MoE sublayer (tokens int [B, rows], row i of sequence b at position
    pos[b] + i; ``caches`` one {"k", "v"} per layer, updated in place).
    Also returns each row's head gap and its smallest router gap over the
    layers (the near-tie margins of the greedy token)."""
    shape = model["shape"]
    dt = model["dtype"]
    tokens = np.asarray(tokens, np.int64)
    B, rows = tokens.shape
    h = embed(tokens.reshape(-1), model["emb"], dt)
    min_rgap = np.full(B * rows, np.inf)
    for layer, at, cache in zip(model["layers"], attn, caches):
        h = attn_sublayer(h, at, cache, pos, rows, n_heads, dt, shape.eps, operands)
        st = moe_layer(h, layer, dt, shape.top_k, shape.n_routed, shape.n_shared, shape.eps, operands)
        min_rgap = np.minimum(min_rgap, st["gap"])
        h = st["h_out"]
    head = lm_head(h, model["norm_f"], model["w_lm"], dt, shape.eps, operands)
    return {"argmax": head["argmax"].reshape(B, rows), "gap": head["gap"].reshape(B, rows), "h": h,
            "router_gap": min_rgap.reshape(B, rows)}


def cached_verify_step(last: np.ndarray, drafts: np.ndarray, model: dict, attn: list, caches: list,
                       pos: np.ndarray, n_heads: int, operands: str = "bf16") -> dict:
    """One verify pass with attention: (last, d_1..d_K) of sequence b at
    positions pos[b] .. pos[b]+K, accept as ``mtp_verify``; the sequence's
    position then advances by n_b + 1 (its last token and the n accepted
    drafts stay in the cache; the rows past them are overwritten later)."""
    last = np.asarray(last, np.int64).reshape(-1, 1)
    tokens = np.concatenate([last, np.asarray(drafts, np.int64).reshape(last.shape[0], -1)], axis=1)
    fwd = cached_greedy(tokens, model, attn, caches, pos, n_heads, operands)
    n_acc, commit, clen, nxt = mtp_verify(tokens, fwd["argmax"])
    return {"greedy": fwd["argmax"], "gap": fwd["gap"], "router_gap": fwd["router_gap"],
            "n_accept": n_acc, "commit": commit, "commit_len": clen, "next_last": nxt,
            "pos": np.asarray(pos) + n_acc + 1}


def cached_rollout(last: np.ndarray, model: dict, attn: list, caches: list, pos: np.ndarray,
                   n_heads: int, n_tokens: int, operands: str = "bf16") -> np.ndarray:
    """Plain greedy decoding with attention: one row per sequence per step."""
    cur = np.asarray(last, np.int64).reshape(-1)
    pos = np.asarray(pos).copy()
    out = np.empty((len(cur), n_tokens), np.int64)
    for s in range(n_tokens):
        cur = cached_greedy(cur[:, None], model, attn, caches, pos, n_heads, operands)["argmax"][:, 0]
        out[:, s] = cur
        pos = pos + 1
    return out


def expected_tau(accept: Sequence[float]) -> float:
    """E[committed tokens per step] = 1 + sum_{m=1..K} prod_{j<=m} a_j when the
    j-th draft is right with probability a_j given the earlier ones were."""
    tau, run = 1.0, 1.0
    for a in accept:
        run *= a
        tau += run
    return tau


def acceptance_rate(tau: float, K: int) -> float:
    """Mean fraction of drafts accepted: (tau - 1) / K."""
    return (tau - 1.0) / K
