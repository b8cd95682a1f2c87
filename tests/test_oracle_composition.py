"""Pins of the oracle's multi-layer decoder, its attention sublayer and its
embedding against independent float64 compositions written with torch on the
CPU (no oracle helper is reused: RMSNorm is written out here, projections are
``F.linear``, attention is ``F.scaled_dot_product_attention`` with an explicit
causal-offset mask, the router is ``softmax`` + ``topk``, and the experts run
densely -- every expert on every token, gate 0 where unchosen).

What these catch that the oracle's other pins do not: a key/value cache row
written at the wrong position, keys and values taken from the un-normalised
state, a dropped residual in either sublayer, a layer applied twice or out of
order in the layer loop, and an embedding row taken from the wrong token.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth

HEADS = 2          # 64-wide heads at H = 128
TOL = 1e-10        # float64: only summation order differs


def _t(a, dtype):
    """Stored tensor -> float64 torch tensor, decoded by torch itself."""
    a = np.asarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64)
    return torch.from_numpy(a.astype(np.float64))


def _rb(x, on):
    """Round float64 to bf16 (nearest, ties to even) when ``on``.

    torch converts float64 to bf16 through float32, which rounds twice (a
    value just above a bf16 midpoint can land on it in float32 and then go
    down).  So the float32 step here rounds to odd -- truncate, then set the
    last bit if anything was cut (Boldo and Melquiond's rule, exact for a
    later rounding to fewer bits) -- and torch's float32 -> bf16 conversion
    does the one real rounding."""
    if not on:
        return x
    a = x.numpy()
    f = a.astype(np.float32)
    over = np.abs(f.astype(np.float64)) > np.abs(a)
    f = np.where(over, np.nextafter(f, np.float32(0)), f).astype(np.float32)
    bits = f.view(np.uint32).copy()
    bits[f.astype(np.float64) != a] |= np.uint32(1)
    return torch.from_numpy(bits.view(np.float32)).to(torch.bfloat16).to(torch.float64)


def _norm(h, gain, eps):
    return h * torch.rsqrt((h * h).mean(dim=-1, keepdim=True) + eps) * gain


def _moe(h, layer, shape, dt, rnd):
    """Dense pre-norm MoE sublayer with residual; returns (h_out, router gap)."""
    x = _norm(h, _t(layer["norm"], dt), shape.eps)
    xo = _rb(x, rnd)
    logits = F.linear(x, _t(layer["w_router"], dt))
    if layer.get("bias") is not None:
        logits = logits + torch.from_numpy(np.asarray(layer["bias"], np.float64))
    p = torch.softmax(logits, dim=-1)
    top_p, top_i = torch.topk(p, shape.top_k, dim=-1)
    gate = torch.zeros_like(p).scatter(1, top_i, top_p / top_p.sum(dim=-1, keepdim=True))
    wg, wu, wd = (_t(layer[n], dt) for n in ("w_gate", "w_up", "w_down"))
    out = torch.zeros_like(h)
    for g in range(shape.n_groups):
        a = _rb(F.silu(F.linear(xo, wg[g])) * F.linear(xo, wu[g]), rnd)
        f = F.linear(a, wd[g])
        out = out + (gate[:, g:g + 1] * f if g < shape.n_routed else f)
    srt = torch.sort(logits, dim=-1, descending=True).values
    gap = (srt[:, shape.top_k - 1] - srt[:, shape.top_k]) if shape.top_k < shape.n_routed \
        else torch.full((h.shape[0],), float("inf"), dtype=torch.float64)
    return h + out, gap


def _head(h, model, shape, dt, rnd):
    x = _rb(_norm(h, _t(model["norm_f"], dt), shape.eps), rnd)
    logits = F.linear(x, _t(model["w_lm"], dt))
    top2 = torch.topk(logits, 2, dim=-1).values
    return torch.argmax(logits, dim=-1), top2[:, 0] - top2[:, 1]


def _attn(h, at, cache, pos, rows, dt, eps, rnd):
    """Pre-norm causal attention sublayer with residual; ``cache`` = torch
    float64 tensors [B, L, H], written at pos[b] + i."""
    x = _rb(_norm(h, 1.0, eps), rnd)
    q = F.linear(x, _t(at["w_q"], dt))
    k = F.linear(x, _t(at["w_k"], dt))
    v = F.linear(x, _t(at["w_v"], dt))
    k, v = _rb(k, dt == "bf16"), _rb(v, dt == "bf16")
    B = len(pos)
    H = h.shape[1]
    d = H // HEADS
    o = torch.empty_like(q)
    for b in range(B):
        p0 = int(pos[b])
        cache["k"][b, p0:p0 + rows] = k[b * rows:(b + 1) * rows]
        cache["v"][b, p0:p0 + rows] = v[b * rows:(b + 1) * rows]
        n = p0 + rows
        Q = q[b * rows:(b + 1) * rows].reshape(rows, HEADS, d).transpose(0, 1)
        Kc = cache["k"][b, :n].reshape(n, HEADS, d).transpose(0, 1)
        Vc = cache["v"][b, :n].reshape(n, HEADS, d).transpose(0, 1)
        mask = torch.arange(n)[None, :] <= (p0 + torch.arange(rows))[:, None]
        ob = F.scaled_dot_product_attention(Q, Kc, Vc, attn_mask=mask)
        o[b * rows:(b + 1) * rows] = ob.transpose(0, 1).reshape(rows, H)
    return h + F.linear(_rb(o, rnd), _t(at["w_o"], dt))


def _shape(dtype, n_layers):
    return replace(synth.TINY, dtype=dtype, n_layers=n_layers)


@pytest.fixture(scope="module", params=[("f32", "exact"), ("bf16", "bf16")], ids=["f32", "bf16"])
def tiny3(request):
    """A three-layer tiny model (fp32, or bf16 with the bf16 operand roundings)."""
    dtype, operands = request.param
    shape = _shape(dtype, 3)
    return shape, synth.model_weights(shape), synth.attention_weights(shape), operands


def test_embed_is_a_row_lookup():
    """embed = one-hot(tokens) @ table, for repeated, first and last ids."""
    for dtype in ("f32", "bf16"):
        w = synth.model_weights(_shape(dtype, 1))
        V = synth.TINY.vocab
        tokens = np.array([0, V - 1, 7, 7, 300, 0, 511 % V, 129], np.int64)
        got = oracle.embed(tokens, w["emb"], dtype)
        onehot = F.one_hot(torch.from_numpy(tokens), V).to(torch.float64)
        ref = onehot @ _t(w["emb"], dtype)
        np.testing.assert_array_equal(got, ref.numpy())
        np.testing.assert_array_equal(got, F.embedding(torch.from_numpy(tokens), _t(w["emb"], dtype)).numpy())


def test_multi_layer_decoder_matches_a_dense_composition(tiny3):
    """model_greedy over 3 layers = the torch composition layer by layer
    (every stage's residual, the head's arg max and gap, the smallest router
    gap over the layers)."""
    shape, model, _, operands = tiny3
    rnd = operands == "bf16" and shape.dtype == "bf16"
    tokens = synth.counter_randint(shape.vocab, 9, np.arange(24))
    got = oracle.model_greedy(tokens, model, operands, keep=True)
    h = _t(model["emb"], shape.dtype)[torch.from_numpy(tokens.astype(np.int64))]
    gmin = torch.full((len(tokens),), float("inf"), dtype=torch.float64)
    for layer, st in zip(model["layers"], got["stages"]):
        h, gap = _moe(h, layer, shape, shape.dtype, rnd)
        gmin = torch.minimum(gmin, gap)
        np.testing.assert_allclose(st["h_out"], h.numpy(), rtol=0, atol=TOL)
    arg, hgap = _head(h, model, shape, shape.dtype, rnd)
    clear = hgap.numpy() > 1e-8
    np.testing.assert_array_equal(got["argmax"][clear], arg.numpy()[clear])
    np.testing.assert_allclose(got["gap"], hgap.numpy(), rtol=0, atol=TOL)
    np.testing.assert_allclose(got["router_gap"], gmin.numpy(), rtol=0, atol=TOL)
    np.testing.assert_allclose(got["h"], h.numpy(), rtol=0, atol=TOL)


def test_layers_are_distinct_and_in_order(tiny3):
    """Swapping two layers' weights changes the result (the composition
    above would not detect a loop that ignores the layer index otherwise)."""
    shape, model, _, operands = tiny3
    tokens = synth.counter_randint(shape.vocab, 9, np.arange(8))
    swapped = dict(model, layers=[model["layers"][1], model["layers"][0], model["layers"][2]])
    a = oracle.model_greedy(tokens, model, operands)["h"]
    b = oracle.model_greedy(tokens, swapped, operands)["h"]
    assert np.abs(a - b).max() > 1e-6   # float64 noise is ~1e-15


def test_attention_sublayer_matches_sdpa_with_cache_writes(tiny3):
    """attn_sublayer = RMSNorm, F.linear projections, the rows' keys and values
    written at pos[b] + i, scaled_dot_product_attention under the causal-offset
    mask, W_o and the residual; every cache row is compared, written or not."""
    shape, _, attn, operands = tiny3
    rnd = operands == "bf16" and shape.dtype == "bf16"
    B, rows, L, H = 3, 4, 20, shape.hidden
    pos = np.array([0, 5, 16])
    rng = np.random.default_rng(21)
    h = rng.standard_normal((B * rows, H))
    kc0 = rng.standard_normal((B, L, H)) * 0.7
    vc0 = rng.standard_normal((B, L, H)) * 0.7
    if shape.dtype == "bf16":
        kc0 = _rb(torch.from_numpy(kc0), True).numpy()
        vc0 = _rb(torch.from_numpy(vc0), True).numpy()
    assert _rb(torch.tensor([1 + 2 ** -8 + 2 ** -30], dtype=torch.float64), True).item() == 1 + 2 ** -7   # no double rounding
    cache = {"k": kc0.copy(), "v": vc0.copy()}
    got = oracle.attn_sublayer(h, attn[0], cache, pos, rows, HEADS, shape.dtype, shape.eps, operands)
    tc = {"k": torch.from_numpy(kc0.copy()), "v": torch.from_numpy(vc0.copy())}
    ref = _attn(torch.from_numpy(h), attn[0], tc, pos, rows, shape.dtype, shape.eps, rnd)
    np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=TOL)
    np.testing.assert_allclose(cache["k"], tc["k"].numpy(), rtol=0, atol=TOL)
    np.testing.assert_allclose(cache["v"], tc["v"].numpy(), rtol=0, atol=TOL)
    # rows outside [pos[b], pos[b] + rows) are untouched
    for b in range(B):
        keep = np.ones(L, bool)
        keep[pos[b]:pos[b] + rows] = False
        np.testing.assert_array_equal(cache["k"][b, keep], kc0[b, keep])


def test_cached_decoder_matches_the_composition_over_passes(tiny3):
    """cached_greedy over 3 layers and two successive passes (the second
    reads the first's cache rows) = attention then MoE per layer, then the
    head, composed in torch; caches compared after each pass."""
    shape, model, attn, operands = tiny3
    rnd = operands == "bf16" and shape.dtype == "bf16"
    B, rows, L, H = 3, 3, 12, shape.hidden
    caches = [{"k": np.zeros((B, L, H)), "v": np.zeros((B, L, H))} for _ in attn]
    tcaches = [{"k": torch.zeros(B, L, H, dtype=torch.float64), "v": torch.zeros(B, L, H, dtype=torch.float64)}
               for _ in attn]
    pos = np.array([0, 2, 5])
    for p in range(2):
        tokens = synth.counter_randint(shape.vocab, 10 + p, np.arange(B)[:, None], np.arange(rows)[None, :])
        got = oracle.cached_greedy(tokens, model, attn, caches, pos, HEADS, operands)
        h = _t(model["emb"], shape.dtype)[torch.from_numpy(tokens.reshape(-1).astype(np.int64))]
        gmin = torch.full((B * rows,), float("inf"), dtype=torch.float64)
        for layer, at, tc in zip(model["layers"], attn, tcaches):
            h = _attn(h, at, tc, pos, rows, shape.dtype, shape.eps, rnd)
            h, gap = _moe(h, layer, shape, shape.dtype, rnd)
            gmin = torch.minimum(gmin, gap)
        arg, hgap = _head(h, model, shape, shape.dtype, rnd)
        np.testing.assert_allclose(got["h"], h.numpy(), rtol=0, atol=TOL)
        clear = hgap.numpy() > 1e-8
        np.testing.assert_array_equal(got["argmax"].reshape(-1)[clear], arg.numpy()[clear])
        np.testing.assert_allclose(got["gap"].reshape(-1), hgap.numpy(), rtol=0, atol=TOL)
        np.testing.assert_allclose(got["router_gap"].reshape(-1), gmin.numpy(), rtol=0, atol=TOL)
        for c, tc in zip(caches, tcaches):
            np.testing.assert_allclose(c["k"], tc["k"].numpy(), rtol=0, atol=TOL)
            np.testing.assert_allclose(c["v"], tc["v"].numpy(), rtol=0, atol=TOL)
        pos = pos + rows


@pytest.mark.parametrize("plant", [None, "cache_row", "unnormalised_kv", "no_residual"])
def test_the_composition_catches_planted_mistakes(plant):
    """Each mistake the attention pins target, planted in a copy of the
    oracle's sublayer on the CPU (fp32 tiny model, no roundings), breaks the
    match with the composition; the unplanted copy matches it."""
    shape = _shape("f32", 1)
    at = synth.attention_weights(shape)[0]
    B, rows, L, H = 2, 3, 10, shape.hidden
    pos = np.array([1, 4])
    h = np.random.default_rng(5).standard_normal((B * rows, H))

    def copy_of_sublayer(hh, cache):
        dt = shape.dtype
        x = oracle.rmsnorm(hh, 1.0, shape.eps)
        src = hh if plant == "unnormalised_kv" else x
        q = x @ oracle.to_f64(at["w_q"], dt).T
        k = src @ oracle.to_f64(at["w_k"], dt).T
        v = src @ oracle.to_f64(at["w_v"], dt).T
        shift = 1 if plant == "cache_row" else 0
        for b in range(B):
            for i in range(rows):
                cache["k"][b, pos[b] + i + shift] = k[b * rows + i]
                cache["v"][b, pos[b] + i + shift] = v[b * rows + i]
        o = oracle.attn_decode(q, cache["k"], cache["v"], pos, rows, HEADS, "f64")
        out = o @ oracle.to_f64(at["w_o"], dt).T
        return out if plant == "no_residual" else hh + out

    got = copy_of_sublayer(h, {"k": np.zeros((B, L, H)), "v": np.zeros((B, L, H))})
    tc = {"k": torch.zeros(B, L, H, dtype=torch.float64), "v": torch.zeros(B, L, H, dtype=torch.float64)}
    ref = _attn(torch.from_numpy(h), at, tc, pos, rows, shape.dtype, shape.eps, False).numpy()
    err = np.abs(got - ref).max()
    if plant is None:
        assert err <= TOL
    else:
        assert err > 1e-4
