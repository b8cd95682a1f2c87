"""Seeded synthetic inputs for the FastMTP verify step through the MoE decoder.

This module is the one piece shared by the CPU oracle and the HIP path: it
draws the synthetic weights, hidden states, token batches and draft tokens
that both sides consume.  It holds none of the method's arithmetic (no norm,
routing, expert, head or accept step); it only fixes *what the inputs are*.

Shapes follow the Jina-OCR-v1 decoder as the pages describe it: 64 routed
experts, two shared experts and top-6 routing ("The speed comes from three
layers working together", kg.zhiyong.dev explainer); the remaining dimensions
(hidden 1280, expert intermediate 896, vocabulary 129280, 12 layers) and the
N(0, 0.02) weight law are a synthetic stand-in for the trained weights, which
are not used.

Random streams
--------------
* Weight tensors: ``numpy.random.Generator(PCG64(SeedSequence(seed,
  spawn_key=(model_id, layer, tensor_code, index))))`` drawing float32
  standard normals, scaled by float32 std, rounded to bf16 (round to nearest,
  ties to even) for bf16 models.  One stream per (layer, tensor, expert) or per
  row chunk, so any sub-model (one layer, one expert) regenerates identically.
* Draft tokens and the first committed tokens: a counter-based generator,
  SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014), keyed by (seed, sequence, trajectory position,
  draft position, stream), so a draft depends only on where its sequence
  stands, never on batch composition or call order.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "ModelShape", "Workload", "TINY", "DECODER", "WORKLOADS",
    "model_weights", "hidden_states", "initial_tokens", "prompt_tokens", "draft_tokens",
    "zipf_bias", "f32_to_bf16_bits", "splitmix64", "counter_uniform",
    "counter_randint", "weight_bytes", "draft_weights", "draft_states", "attention_inputs",
    "attention_weights",
]

# tensor codes in the spawn key
_ROUTER, _GATE, _UP, _DOWN, _LM, _EMB, _HIDDEN, _ZIPF = 0, 1, 2, 3, 4, 5, 6, 7
_DPROJ, _DGATE, _DUP, _DDOWN, _DSTATE = 8, 9, 10, 11, 12
_AQ, _AK, _AV = 13, 14, 15
_WQ, _WK, _WV, _WO = 16, 17, 18, 19
_DRAFT_LAYER = 1000  # layer field of the draft block's streams
_ATTN_LAYER = 2000   # layer field of the attention inputs' streams
_ROW_CHUNK = 4096  # rows per stream for the vocabulary-sized tensors


@dataclass(frozen=True)
class ModelShape:
    """Dimensions of a synthetic MoE decoder.

    Groups 0..n_routed-1 are routed experts; groups n_routed..n_routed+n_shared-1
    are the always-on shared experts (same SwiGLU form and width).
    """
    name: str
    hidden: int          # H
    n_routed: int        # E
    inter: int           # I (every expert, routed and shared)
    top_k: int           # k
    n_shared: int        # ns
    vocab: int           # V
    n_layers: int        # L
    dtype: str           # "bf16" or "f32": weights and GEMM operand type
    model_id: int        # RNG stream id
    weight_std: float = 0.02
    emb_std: float = 1.0
    eps: float = 1e-6
    zipf: bool = False   # per-layer Zipf(1.1) router bias

    @property
    def n_groups(self) -> int:
        return self.n_routed + self.n_shared

    @property
    def slots(self) -> int:
        return self.top_k + self.n_shared


TINY = ModelShape("tiny", hidden=128, n_routed=8, inter=64, top_k=2, n_shared=1,
                  vocab=512, n_layers=1, dtype="f32", model_id=0)
DECODER = ModelShape("decoder", hidden=1280, n_routed=64, inter=896, top_k=6,
                     n_shared=2, vocab=129280, n_layers=12, dtype="bf16", model_id=1)


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: a model shape plus the batch it runs on."""
    name: str
    shape: ModelShape
    batch: int = 0                  # B sequences (verify workloads)
    drafts: int = 0                 # K drafts per sequence
    tokens: int = 0                 # T for single-layer and prefill workloads
    accept: Tuple[float, ...] = ()  # per-position draft-correct probability
    draft_mode: str = "exclude"     # "exclude": a wrong draft avoids the truth
    steps: int = 0                  # verify steps in a trajectory run
    layer_only: bool = False        # one MoE layer on h ~ N(0,1), no head

    @property
    def n_tokens(self) -> int:
        return self.tokens if (self.layer_only or self.tokens) else self.batch * (1 + self.drafts)


# Conditional draft acceptance by position, K=3: 0.830 / 0.663 / 0.636
# (evolve.pub review of Jina-OCR-v1, Strengths: speculative-decoding analysis,
# Table 8).
PAGE_ACCEPT = (0.830, 0.663, 0.636)

WORKLOADS: Dict[str, Workload] = {
    # 4 sequences x (1 committed + 3 drafts) through a one-layer fp32 model.
    "tiny_verify_b4k3": Workload("tiny_verify_b4k3", TINY, batch=4, drafts=3,
                                 accept=(0.7, 0.7, 0.7), draft_mode="uniform",
                                 steps=16),
    # One decoder layer at decode shape: 32 sequences x 4 tokens.
    "decode_layer_t128": Workload("decode_layer_t128", replace(DECODER, n_layers=1),
                                  tokens=128, layer_only=True),
    # One decoder layer at prefill shape: 8 pages x (1156 visual + 64 prompt).
    "prefill_layer_t9760": Workload("prefill_layer_t9760", replace(DECODER, n_layers=1),
                                    tokens=9760, layer_only=True),
    # Page-shaped prefill through all 12 layers + the head on each page's
    # last token: 8 pages x (1156 visual + 64 prompt) tokens.
    "prefill_model_t9760": Workload("prefill_model_t9760", DECODER, batch=8, tokens=9760),
    # The full verify step: 12 layers + head, 32 sequences x (1+3).
    "verify_step_b32k3": Workload("verify_step_b32k3", DECODER, batch=32, drafts=3,
                                  accept=PAGE_ACCEPT, steps=64),
}
# The same step with K = 0 (plain greedy decoding), 1 and 2 drafts, for the
# choice of K: drafts at the first K of the page's acceptances.
for _k in (0, 1, 2):
    _n = f"verify_step_b32k{_k}"
    WORKLOADS[_n] = Workload(_n, DECODER, batch=32, drafts=_k, accept=PAGE_ACCEPT[:_k], steps=64)
# Larger batches of the same step (uniform routing): 64 and 128 sequences x (1+3).
for _b in (64, 128):
    _n = f"verify_step_b{_b}k3"
    WORKLOADS[_n] = Workload(_n, DECODER, batch=_b, drafts=3, accept=PAGE_ACCEPT, steps=16)
for _b in (1, 8, 32, 128):
    for _k, _acc in ((3, PAGE_ACCEPT), (1, PAGE_ACCEPT[:1])):
        _n = f"zipf_verify_b{_b}k{_k}"
        WORKLOADS[_n] = Workload(_n, replace(DECODER, zipf=True), batch=_b, drafts=_k,
                                 accept=_acc, steps=16)


# ---------------------------------------------------------------------------
# bf16 encoding of generated values (input definition, not method arithmetic)

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Finite inputs only (the generators never produce inf/NaN).
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    u = u + (((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF))
    return (u >> np.uint32(16)).astype(np.uint16)


def _pool_workers() -> int:
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, n))


def _normal_block(seed: int, key: Tuple[int, ...], n: int, std: float, bf16: bool) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))
    a = rng.standard_normal(n, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return f32_to_bf16_bits(a) if bf16 else a


def _fill(jobs, workers: Optional[int] = None):
    """Run (out_view, seed, key, std, bf16) jobs on a thread pool (numpy's
    generators release the GIL while filling)."""
    def run(job):
        out, seed, key, std, bf16 = job
        out[...] = _normal_block(seed, key, out.size, std, bf16).reshape(out.shape)
    with ThreadPoolExecutor(workers or _pool_workers()) as ex:
        for _ in ex.map(run, jobs):
            pass


def _empty(shape, bf16: bool) -> np.ndarray:
    return np.empty(shape, dtype=np.uint16 if bf16 else np.float32)


def _ones(n: int, bf16: bool) -> np.ndarray:
    # gamma = 1 exactly; bf16(1.0) = 0x3F80
    return np.full(n, 0x3F80, np.uint16) if bf16 else np.ones(n, np.float32)


def zipf_bias(shape: ModelShape, layer: int, seed: int = 3) -> np.ndarray:
    """Per-expert router bias from a Zipf(1.1) ranking, as float32 [E].

    A seeded permutation assigns each expert a rank r in 1..E; the bias is
    -1.1 * ln(r), then centred to zero mean.  Added to the router logits it
    multiplies the pre-normalisation weight of the rank-r expert by r^-1.1.
    """
    rng = np.random.Generator(np.random.PCG64(
        np.random.SeedSequence(seed, spawn_key=(shape.model_id, _ZIPF, layer))))
    r = rng.permutation(shape.n_routed).astype(np.float64) + 1.0
    b = -1.1 * np.log(r)
    return (b - b.mean()).astype(np.float32)


def model_weights(shape: ModelShape, seed: int = 0, layers: Optional[Sequence[int]] = None,
                  head: bool = True, workers: Optional[int] = None) -> dict:
    """Synthetic weights of ``shape``.

    Returns a dict with ``dtype`` ("bf16": uint16 bit patterns, "f32": float32),
    ``layers`` (list of per-layer dicts: norm [H], w_router [E,H], w_gate [G,I,H],
    w_up [G,I,H], w_down [G,H,I], bias [E] float32 or None) and, when ``head``,
    ``emb`` [V,H], ``norm_f`` [H], ``w_lm`` [V,H].  ``layers`` picks a subset of
    layer indices (default all); each layer's values depend only on its index.
    """
    bf16 = shape.dtype == "bf16"
    H, E, I, G = shape.hidden, shape.n_routed, shape.inter, shape.n_groups
    mid, std = shape.model_id, shape.weight_std
    layer_ids = list(range(shape.n_layers)) if layers is None else list(layers)
    jobs = []
    out_layers: List[dict] = []
    for l in layer_ids:
        d = {
            "norm": _ones(H, bf16),
            "w_router": _empty((E, H), bf16),
            "w_gate": _empty((G, I, H), bf16),
            "w_up": _empty((G, I, H), bf16),
            "w_down": _empty((G, H, I), bf16),
            "bias": zipf_bias(shape, l) if shape.zipf else None,
        }
        jobs.append((d["w_router"], seed, (mid, l, _ROUTER, 0), std, bf16))
        for g in range(G):
            jobs.append((d["w_gate"][g], seed, (mid, l, _GATE, g), std, bf16))
            jobs.append((d["w_up"][g], seed, (mid, l, _UP, g), std, bf16))
            jobs.append((d["w_down"][g], seed, (mid, l, _DOWN, g), std, bf16))
        out_layers.append(d)
    out = {"dtype": shape.dtype, "shape": shape, "layers": out_layers, "layer_ids": layer_ids}
    if head:
        V = shape.vocab
        out["emb"] = _empty((V, H), bf16)
        out["w_lm"] = _empty((V, H), bf16)
        out["norm_f"] = _ones(H, bf16)
        for c in range(0, V, _ROW_CHUNK):
            ci = c // _ROW_CHUNK
            jobs.append((out["emb"][c:c + _ROW_CHUNK], seed, (mid, 0, _EMB, ci), shape.emb_std, bf16))
            jobs.append((out["w_lm"][c:c + _ROW_CHUNK], seed, (mid, 0, _LM, ci), std, bf16))
    _fill(jobs, workers)
    return out


def draft_weights(shape: ModelShape, seed: int = 0, workers: Optional[int] = None) -> dict:
    """Synthetic weights of the FastMTP draft block for a decoder of ``shape``.

    Stored as the slices the kernels consume (see the oracle for the dense
    block they make up): ``w_proj`` [2, H, H] (slice g = columns g*H..(g+1)*H-1
    of the [H, 2H] input projection: g = 0 acts on the normalised hidden state,
    g = 1 on the normalised token embedding), ``w_gate`` / ``w_up`` [n, I, H]
    and ``w_down`` [n, H, I] (the dense SwiGLU of width n*I split along its
    intermediate axis, n = top_k + n_shared), and RMSNorm weights ``norm_z``,
    ``norm_e`` (the two inputs), ``norm_ffn`` (before the FFN) and ``norm_out``
    (before the shared LM head), all ones.
    """
    bf16 = shape.dtype == "bf16"
    H, I = shape.hidden, shape.inter
    n = shape.top_k + shape.n_shared
    mid, std = shape.model_id, shape.weight_std
    d = {
        "dtype": shape.dtype, "n_slices": n,
        "norm_z": _ones(H, bf16), "norm_e": _ones(H, bf16),
        "norm_ffn": _ones(H, bf16), "norm_out": _ones(H, bf16),
        "w_proj": _empty((2, H, H), bf16),
        "w_gate": _empty((n, I, H), bf16),
        "w_up": _empty((n, I, H), bf16),
        "w_down": _empty((n, H, I), bf16),
    }
    jobs = []
    for g in range(2):
        jobs.append((d["w_proj"][g], seed, (mid, _DRAFT_LAYER, _DPROJ, g), std, bf16))
    for s in range(n):
        jobs.append((d["w_gate"][s], seed, (mid, _DRAFT_LAYER, _DGATE, s), std, bf16))
        jobs.append((d["w_up"][s], seed, (mid, _DRAFT_LAYER, _DUP, s), std, bf16))
        jobs.append((d["w_down"][s], seed, (mid, _DRAFT_LAYER, _DDOWN, s), std, bf16))
    _fill(jobs, workers)
    return d


def draft_states(shape: ModelShape, batch: int, seed: int = 4) -> np.ndarray:
    """Hidden states entering a draft block, float32 [batch, H] ~ N(0, 1)."""
    out = np.empty((batch, shape.hidden), np.float32)
    out[:] = _normal_block(seed, (shape.model_id, _DRAFT_LAYER, _DSTATE, 0), batch * shape.hidden,
                           1.0, False).reshape(batch, shape.hidden)
    return out


def weight_bytes(w: dict) -> int:
    n = 0
    for d in w["layers"]:
        n += sum(d[k].nbytes for k in ("norm", "w_router", "w_gate", "w_up", "w_down"))
    for k in ("emb", "w_lm", "norm_f"):
        if k in w:
            n += w[k].nbytes
    return n


def attention_weights(shape: ModelShape, seed: int = 0) -> list:
    """Per decoder layer, the attention sublayer's projections W_q, W_k, W_v,
    W_o, each [H, H] ~ N(0, weight_std^2) (bf16 bit patterns for a bf16
    model), on streams of their own."""
    bf16 = shape.dtype == "bf16"
    H = shape.hidden
    out = []
    for layer in range(shape.n_layers):
        d = {key: _empty((H, H), bf16) for key in ("w_q", "w_k", "w_v", "w_o")}
        jobs = [(d[key], seed, (shape.model_id, layer, code, 0), shape.weight_std, bf16)
                for key, code in (("w_q", _WQ), ("w_k", _WK), ("w_v", _WV), ("w_o", _WO))]
        _fill(jobs)
        out.append(d)
    return out


def attention_inputs(batch: int, rows: int, hidden: int, max_len: int, prefix: Tuple[int, int],
                     seed: int = 7, kv_std: float = 0.72, bf16: bool = True) -> dict:
    """Inputs of decode attention for ``batch`` sequences of ``rows`` verify
    rows each: queries float32 [batch*rows, hidden] ~ N(0, 1); a key and a
    value cache [batch, max_len, hidden] ~ N(0, kv_std^2) (bf16 bit patterns
    when ``bf16``), standing in for a page prefix and the verify rows' own keys;
    and per sequence the number of cached positions before its first verify
    row, uniform in [prefix[0], prefix[1]] and at most max_len - rows.  The
    default kv_std is the spread of a 1280-wide N(0, 0.02) projection of a
    unit-RMS state."""
    lo, hi = prefix
    hi = min(hi, max_len - rows)
    assert 0 <= lo <= hi, "prefix range does not fit max_len"
    key = lambda code, i: (0, _ATTN_LAYER, code, i)
    q = _normal_block(seed, key(_AQ, 0), batch * rows * hidden, 1.0, False).reshape(batch * rows, hidden)
    kc = _empty((batch, max_len, hidden), bf16)
    vc = _empty((batch, max_len, hidden), bf16)
    jobs = []
    for b in range(batch):
        jobs.append((kc[b], seed, key(_AK, b), kv_std, bf16))
        jobs.append((vc[b], seed, key(_AV, b), kv_std, bf16))
    _fill(jobs)
    pos = (lo + counter_randint(hi - lo + 1, seed, np.arange(batch), -2)).astype(np.int32)
    return {"q": q, "k_cache": kc, "v_cache": vc, "pos": pos, "rows": rows,
            "dtype": "bf16" if bf16 else "f32"}


def hidden_states(shape: ModelShape, n_tokens: int, seed: int = 1) -> np.ndarray:
    """Residual-stream input h ~ N(0, 1), float32 [T, H], drawn in 128-row
    chunks so a shorter batch is a prefix of a longer one."""
    H = shape.hidden
    h = np.empty((n_tokens, H), np.float32)
    jobs = [(h[c:c + 128], seed, (shape.model_id, 0, _HIDDEN, c // 128), 1.0, False)
            for c in range(0, n_tokens, 128)]
    _fill(jobs)
    return h


# ---------------------------------------------------------------------------
# Counter-based draws for tokens and drafts (SplitMix64 finaliser)

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64(x) -> np.ndarray:
    """One SplitMix64 output for state ``x`` (uint64, vectorised, wraps mod 2^64)."""
    with np.errstate(over="ignore"):
        z = np.asarray(x, dtype=np.uint64) + _GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def _key(seed: int, *fields) -> np.ndarray:
    h = splitmix64(np.uint64(seed))
    for f in fields:
        h = splitmix64(h ^ np.asarray(f, dtype=np.int64).astype(np.uint64))
    return h


def counter_uniform(seed: int, *fields) -> np.ndarray:
    """Uniform [0, 1) doubles from the top 53 bits of the keyed hash."""
    return (_key(seed, *fields) >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


def counter_randint(n: int, seed: int, *fields) -> np.ndarray:
    """Integers in [0, n) (modulo reduction of a 64-bit hash; bias < n / 2^64)."""
    return (_key(seed, *fields) % np.uint64(n)).astype(np.int64)


def initial_tokens(batch: int, vocab: int, seed: int = 2) -> np.ndarray:
    """First committed token of each sequence, uniform over the vocabulary."""
    b = np.arange(batch)
    return counter_randint(vocab, seed, b, -1, -1, 0).astype(np.int32)


def prompt_tokens(n_seq: int, seq_len: int, vocab: int, seed: int = 5) -> np.ndarray:
    """Page-shaped prompts [n_seq, seq_len], token ids uniform over the
    vocabulary (standing in for the visual and prompt tokens of a page)."""
    i = np.arange(n_seq)[:, None]
    j = np.arange(seq_len)[None, :]
    return counter_randint(vocab, seed, np.broadcast_to(i, (n_seq, seq_len)),
                           np.broadcast_to(j, (n_seq, seq_len)), -1, 1).astype(np.int32)


def draft_tokens(cont: np.ndarray, pos: np.ndarray, accept: Sequence[float], vocab: int,
                 mode: str = "exclude", seed: int = 2) -> np.ndarray:
    """Synthetic drafts standing in for the FastMTP draft block.

    ``cont[b, j]`` is the true greedy continuation (token j+1 after the last
    committed token of sequence b, which sits at trajectory position
    ``pos[b]``).  Draft j equals it with probability ``accept[j]``, drawn
    independently per position; otherwise it is a uniform token, over the
    vocabulary minus the true token (``mode="exclude"``) or over the whole
    vocabulary (``mode="uniform"``).  Draws are keyed by
    (seed, sequence, position, draft index), so they never depend on batch
    composition.  Returns int32 [B, K].
    """
    cont = np.asarray(cont, dtype=np.int64)
    B, K = cont.shape
    assert len(accept) >= K
    b = np.arange(B)[:, None]
    j = np.arange(K)[None, :]
    p = np.asarray(pos, dtype=np.int64)[:, None]
    u = counter_uniform(seed, b, p, j, 1)
    hit = u < np.asarray(accept[:K], dtype=np.float64)[None, :]
    if mode == "exclude":
        alt = counter_randint(vocab - 1, seed, b, p, j, 2)
        alt = alt + (alt >= cont)
    elif mode == "uniform":
        alt = counter_randint(vocab, seed, b, p, j, 2)
    else:
        raise ValueError(mode)
    return np.where(hit, cont, alt).astype(np.int32)
