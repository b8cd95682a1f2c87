"""Pins for the CPU oracle: values and properties fixed by the pages, closed
forms, library routines and brute force -- never the oracle's own formula
retyped.  CPU only."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# number formats

def test_round_bf16_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(11)
    a = rng.standard_normal(200000).astype(np.float32) * np.float32(3.0)
    # exact halfway cases: low 16 bits = 0x8000, both parities of bit 16
    bits = rng.integers(0x3000, 0x5000, size=4000, dtype=np.uint32) << np.uint32(16)
    halves = (bits | np.uint32(0x8000)).view(np.float32)
    a = np.concatenate([a, halves, -halves, np.float32([0.0, 1.0, -2.5, 1e-30, 3e38])])
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_bf16(a.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_bf16_decode_matches_torch():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]   # drop inf/NaN
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.to_f64(bits, "bf16"), ref)


def test_round_bf16_idempotent_and_grid():
    x = np.random.default_rng(3).standard_normal(10000) * 10
    r = oracle.round_bf16(x)
    np.testing.assert_array_equal(oracle.round_bf16(r), r)
    # every rounded value is a bf16 value: its float32 bits have a zero low half
    assert np.all((r.astype(np.float32).view(np.uint32) & 0xFFFF) == 0)
    assert np.all(np.abs(r - x) <= np.abs(x) * 2.0 ** -8 + 1e-300)


# ---------------------------------------------------------------------------
# RMSNorm, SiLU, SwiGLU

def test_rmsnorm_closed_form():
    rng = np.random.default_rng(0)
    h = rng.standard_normal((7, 96)) * rng.uniform(0.1, 10, size=(7, 1))
    eps = 1e-6
    y = oracle.rmsnorm(h, np.ones(96), eps)
    m = np.mean(h * h, axis=1)
    np.testing.assert_allclose(np.mean(y * y, axis=1), m / (m + eps), rtol=1e-12)
    # a constant row c normalises to c / sqrt(c^2 + eps)
    c = np.full((1, 32), -3.0)
    np.testing.assert_allclose(oracle.rmsnorm(c, 1.0, eps), c / math.sqrt(9.0 + eps), rtol=1e-14)
    # gamma scales each channel
    g = rng.uniform(0.5, 2, 96)
    np.testing.assert_allclose(oracle.rmsnorm(h, g, eps), y * g, rtol=1e-14)


def test_silu_against_library():
    z = np.linspace(-40, 40, 2001)
    np.testing.assert_allclose(oracle.silu(z), z * scipy.special.expit(z), rtol=1e-13, atol=1e-300)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert oracle.silu(np.array([-1000.0]))[0] == 0.0


def _torch_swiglu(x, wg, wu, wd):
    x, wg, wu, wd = (torch.from_numpy(np.asarray(a, np.float64)) for a in (x, wg, wu, wd))
    return F.linear(F.silu(F.linear(x, wg)) * F.linear(x, wu), wd).numpy()


# ---------------------------------------------------------------------------
# router

def _rand_layer(rng, H, E, I, ns, dtype="f32", std=0.2):
    G = E + ns
    return {
        "norm": np.ones(H, np.float32),
        "w_router": (rng.standard_normal((E, H)) * std).astype(np.float32),
        "w_gate": (rng.standard_normal((G, I, H)) * std).astype(np.float32),
        "w_up": (rng.standard_normal((G, I, H)) * std).astype(np.float32),
        "w_down": (rng.standard_normal((G, H, I)) * std).astype(np.float32),
        "bias": None,
    }


@pytest.mark.parametrize("E,k", [(8, 2), (6, 3), (5, 1), (7, 7)])
def test_route_brute_force_subset(E, k):
    rng = np.random.default_rng(E * 10 + k)
    x = rng.standard_normal((40, 16))
    wr = rng.standard_normal((E, 16))
    idx, w, logits = oracle.route(x, wr, k)
    p = scipy.special.softmax(x @ wr.T, axis=1)
    for t in range(len(x)):
        best = max(itertools.combinations(range(E), k), key=lambda s: sum(p[t, list(s)]))
        assert set(idx[t]) == set(best)
        assert all(p[t, idx[t, r]] >= p[t, idx[t, r + 1]] for r in range(k - 1))
        np.testing.assert_allclose(w[t], scipy.special.softmax(logits[t, idx[t]]), rtol=1e-12)
        assert abs(w[t].sum() - 1.0) <= 1e-12


def test_route_hand_example_and_ties():
    # logits (0, ln2, ln3): softmax (1/6, 2/6, 3/6); top-2 renormalised (3/5, 2/5)
    x = np.array([[1.0]])
    wr = np.array([[0.0], [math.log(2)], [math.log(3)]])
    idx, w, _ = oracle.route(x, wr, 2)
    assert idx.tolist() == [[2, 1]]
    np.testing.assert_allclose(w, [[0.6, 0.4]], rtol=1e-14)
    # all-equal logits: lowest indices, uniform weights
    idx, w, _ = oracle.route(np.ones((3, 4)), np.zeros((8, 4)), 3)
    assert idx.tolist() == [[0, 1, 2]] * 3
    np.testing.assert_allclose(w, 1 / 3, rtol=1e-14)
    # tie at the boundary: logits (1, 2, 2, 0) -> k=2 picks experts 1, 2; k=1 picks 1
    wr = np.array([[1.0], [2.0], [2.0], [0.0]])
    assert oracle.route(x, wr, 2)[0].tolist() == [[1, 2]]
    assert oracle.route(x, wr, 1)[0].tolist() == [[1]]


def test_route_k_equals_E_is_dense_softmax():
    rng = np.random.default_rng(5)
    x, wr = rng.standard_normal((9, 12)), rng.standard_normal((6, 12))
    idx, w, logits = oracle.route(x, wr, 6)
    p = scipy.special.softmax(x @ wr.T, axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(p, idx.astype(np.int64), 1), rtol=1e-12)


def test_route_bias_shifts_logits():
    rng = np.random.default_rng(6)
    x, wr = rng.standard_normal((20, 8)), rng.standard_normal((6, 8))
    bias = np.array([0, 0, 50.0, 0, 0, 0])  # expert 2 always wins rank 0
    idx, w, logits = oracle.route(x, wr, 2, bias)
    assert np.all(idx[:, 0] == 2)
    np.testing.assert_allclose(logits, x @ wr.T + bias, rtol=1e-14)


def test_route_gap():
    logits = np.array([[3.0, 1.0, 2.0, 0.5], [1.0, 1.0, 1.0, 1.0]])
    np.testing.assert_allclose(oracle.route_gap(logits, 2), [1.0, 0.0])
    assert np.isinf(oracle.route_gap(logits, 4)).all()


# ---------------------------------------------------------------------------
# permute

@pytest.mark.parametrize("T,E,k,ns", [(37, 8, 2, 1), (200, 64, 6, 2), (1, 4, 4, 0), (0, 8, 2, 1)])
def test_permute_matches_stable_argsort(T, E, k, ns):
    rng = np.random.default_rng(T + E)
    idx = np.array([rng.permutation(E)[:k] for _ in range(T)], np.int32).reshape(T, k)
    offsets, src = oracle.permute(idx, E, ns)
    S = k + ns
    groups = np.concatenate([idx, np.tile(np.arange(E, E + ns), (T, 1))], axis=1).reshape(-1)
    groups = groups.astype(np.int64)
    ref_src = np.argsort(groups, kind="stable")
    ref_off = np.concatenate([[0], np.cumsum(np.bincount(groups, minlength=E + ns))])
    np.testing.assert_array_equal(offsets, ref_off)
    np.testing.assert_array_equal(src, ref_src)
    assert sorted(src.tolist()) == list(range(T * S))       # bijection
    for s in range(ns):                                      # shared: all tokens in order
        seg = src[offsets[E + s]:offsets[E + s + 1]]
        np.testing.assert_array_equal(seg, np.arange(T) * S + k + s)


# ---------------------------------------------------------------------------
# MoE layer: sparse dispatch against brute force

def _dense_layer_reference(h, layer, k, E, ns, eps):
    """Every expert on every token through torch; unselected experts get gate 0."""
    x = h / np.sqrt(np.mean(h * h, axis=1, keepdims=True) + eps) * layer["norm"]
    logits = x @ layer["w_router"].astype(np.float64).T
    if layer.get("bias") is not None:
        logits = logits + layer["bias"]
    p = scipy.special.softmax(logits, axis=1)
    top = np.argsort(-p, axis=1, kind="stable")[:, :k]
    gate = np.zeros_like(p)
    for t in range(len(x)):
        gate[t, top[t]] = p[t, top[t]] / p[t, top[t]].sum()
    out = h.copy()
    for e in range(E + ns):
        ye = _torch_swiglu(x, layer["w_gate"][e], layer["w_up"][e], layer["w_down"][e])
        g = gate[:, e:e + 1] if e < E else 1.0
        out = out + g * ye
    return out


@pytest.mark.parametrize("E,k,ns", [(8, 2, 1), (6, 3, 2), (4, 4, 0)])
def test_moe_layer_equals_dense_brute_force(E, k, ns):
    rng = np.random.default_rng(100 + E)
    H, I, T = 24, 16, 33
    layer = _rand_layer(rng, H, E, I, ns)
    h = rng.standard_normal((T, H))
    st = oracle.moe_layer(h, layer, "f32", k, E, ns, 1e-6, operands="exact")
    ref = _dense_layer_reference(h, layer, k, E, ns, 1e-6)
    np.testing.assert_allclose(st["h_out"], ref, rtol=1e-11, atol=1e-12)


def test_single_expert_layer_is_plain_swiglu():
    rng = np.random.default_rng(9)
    H, I, T = 20, 12, 5
    layer = _rand_layer(rng, H, 1, I, 0)
    h = rng.standard_normal((T, H))
    st = oracle.moe_layer(h, layer, "f32", 1, 1, 0, 1e-6, operands="exact")
    np.testing.assert_array_equal(st["w"], np.ones((T, 1)))
    x = h / np.sqrt(np.mean(h * h, axis=1, keepdims=True) + 1e-6)
    ref = h + _torch_swiglu(x, layer["w_gate"][0], layer["w_up"][0], layer["w_down"][0])
    np.testing.assert_allclose(st["h_out"], ref, rtol=1e-12, atol=1e-13)


def test_empty_batch_layer():
    rng = np.random.default_rng(1)
    layer = _rand_layer(rng, 16, 4, 8, 1)
    st = oracle.moe_layer(np.zeros((0, 16)), layer, "f32", 2, 4, 1, 1e-6)
    assert st["h_out"].shape == (0, 16)
    np.testing.assert_array_equal(st["offsets"], np.zeros(6, np.int32))


def test_bf16_operands_mode_close_to_exact():
    shape = synth.ModelShape("mini_bf16", hidden=64, n_routed=8, inter=32, top_k=2,
                             n_shared=2, vocab=300, n_layers=2, dtype="bf16", model_id=7)
    w = synth.model_weights(shape)
    h = np.random.default_rng(2).standard_normal((20, 64))
    a = oracle.moe_layer(h, w["layers"][0], "bf16", 2, 8, 2, 1e-6, operands="exact")
    b = oracle.moe_layer(h, w["layers"][0], "bf16", 2, 8, 2, 1e-6, operands="bf16")
    np.testing.assert_array_equal(b["x_op"], oracle.round_bf16(b["x_op"]))
    np.testing.assert_array_equal(a["idx"], b["idx"])   # router never sees the rounding
    err = np.abs(a["y_slots"] - b["y_slots"]).max()
    assert 0 < err < 2e-3


# ---------------------------------------------------------------------------
# head

def test_first_argmax_library_and_ties():
    rng = np.random.default_rng(4)
    rows = rng.standard_normal((50, 300))
    np.testing.assert_array_equal(oracle.first_argmax(rows), np.argmax(rows, axis=1))
    rows = np.zeros((3, 10))
    rows[0, [3, 7]] = 1.0
    rows[1, [9, 2, 5]] = 2.0
    assert oracle.first_argmax(rows).tolist() == [3, 2, 0]


@pytest.mark.parametrize("chunk", [7, 64, 1000])
def test_lm_head_chunked_against_torch(chunk):
    rng = np.random.default_rng(8)
    T, H, V = 11, 32, 301
    h = rng.standard_normal((T, H))
    w = rng.integers(-2, 3, size=(V, H)).astype(np.float32)
    # token 0: a +-1 row (RMS exactly 1, so normalising with eps=0 leaves it
    # unchanged) aligned with rows 5 and 290, which are equal: an exact tie
    # across chunk boundaries that every summation order reproduces
    sgn = np.where(rng.standard_normal(H) > 0, 1.0, -1.0)
    h[0] = sgn
    w[5] = w[290] = 3 * sgn
    out = oracle.lm_head(h, np.ones(H, np.float32), w, "f32", 0.0, "exact",
                         keep_logits=True, chunk=chunk)
    x = torch.from_numpy(h / np.sqrt(np.mean(h * h, axis=1, keepdims=True)))
    logits = (x @ torch.from_numpy(w.astype(np.float64)).T).numpy()
    np.testing.assert_allclose(out["logits"], logits, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(out["argmax"], np.argmax(logits, axis=1))
    assert out["argmax"][0] == 5 and out["gap"][0] == 0.0 and out["max"][0] == 96.0
    top2 = torch.topk(torch.from_numpy(logits), 2, dim=1).values.numpy()
    np.testing.assert_allclose(out["gap"], top2[:, 0] - top2[:, 1], rtol=1e-9, atol=1e-12)


# ---------------------------------------------------------------------------
# verification

def _verify_by_definition(g, last, drafts):
    """Losslessness characterisation: the commit is the greedy continuation of
    ``last`` cut one past the longest run of drafts that follows it."""
    cont, cur = [], last
    for _ in range(len(drafts) + 1):
        cur = g[cur]
        cont.append(cur)
    m = 0
    while m < len(drafts) and drafts[m] == cont[m]:
        m += 1
    return cont[:m + 1]


@pytest.mark.parametrize("K", [0, 1, 2, 3])
def test_mtp_verify_brute_force_all_maps(K):
    V = 3
    cases = 0
    for gmap in itertools.product(range(V), repeat=V):
        for last in range(V):
            for drafts in itertools.product(range(V), repeat=K):
                tokens = np.array([[last, *drafts]])
                greedy = np.array([[gmap[t] for t in tokens[0]]])
                n, commit, clen, nxt = oracle.mtp_verify(tokens, greedy)
                want = _verify_by_definition(gmap, last, drafts)
                assert commit[0, :clen[0]].tolist() == want
                assert clen[0] == n[0] + 1 == len(want)
                assert (commit[0, clen[0]:] == -1).all()
                assert nxt[0] == want[-1]
                cases += 1
    assert cases == V ** V * V * V ** K


def test_mtp_verify_special_cases():
    g = np.array([[10, 11, 12, 13]])
    # all drafts right -> K accepted + bonus
    n, c, l, nx = oracle.mtp_verify(np.array([[9, 10, 11, 12]]), g)
    assert (n[0], l[0], nx[0]) == (3, 4, 13) and c[0].tolist() == [10, 11, 12, 13]
    # first draft wrong -> only the correction
    n, c, l, nx = oracle.mtp_verify(np.array([[9, 99, 11, 12]]), g)
    assert (n[0], l[0], nx[0]) == (0, 1, 10) and c[0].tolist() == [10, -1, -1, -1]
    # K = 0 -> plain greedy step
    n, c, l, nx = oracle.mtp_verify(np.array([[9]]), np.array([[10]]))
    assert (n[0], l[0], nx[0]) == (0, 1, 10)
    # later drafts right after a miss do not count
    n, c, l, nx = oracle.mtp_verify(np.array([[9, 10, 0, 12]]), g)
    assert (n[0], l[0]) == (1, 2) and c[0].tolist() == [10, 11, -1, -1]


def test_tau_closed_form_matches_table8():
    t8 = _golden("fastmtp_table8.json")
    tau = oracle.expected_tau(t8["conditional_acceptance"])
    # the acceptances are printed to 3 decimals: propagate +-0.0005 into tau
    a1, a2, a3 = t8["conditional_acceptance"]
    slack = 0.0005 * ((1 + a2 + a2 * a3) + a1 * (1 + a3) + a1 * a2)
    assert abs(tau - t8["tau_eager"]) <= 0.005 + slack
    assert round(tau, 2) == t8["tau_eager"]
    # the other readings of the extra-token rule miss the printed value:
    # no extra token (tau = 1.73) and an extra token only when all K match (2.08)
    accepted = sum(np.prod(t8["conditional_acceptance"][:m]) for m in range(1, 4))
    for other in (accepted, accepted + np.prod(t8["conditional_acceptance"])):
        assert abs(other - t8["tau_eager"]) > 0.5


def test_acceptance_rate_matches_result_page():
    res = _golden("fastmtp_result.json")
    t8 = _golden("fastmtp_table8.json")
    rate = oracle.acceptance_rate(oracle.expected_tau(t8["conditional_acceptance"]), res["K"])
    assert abs(rate - res["acceptance_rate"]) <= 0.0005 + 0.0007
    assert abs(oracle.acceptance_rate(res["tau"], res["K"]) - res["acceptance_rate"]) <= 0.0012


def test_tau_statistics_with_synthetic_drafts():
    """32 sequences x 64 steps on a random token map with the Table 8
    acceptances: the mean committed tokens per step must sit within 4 sigma
    (SD of the mean ~0.025) of the closed form the pages print as 2.73."""
    t8 = _golden("fastmtp_table8.json")
    acc = t8["conditional_acceptance"]
    V, B, K, steps = 5000, 32, 3, 64
    gmap = np.random.default_rng(77).integers(0, V, size=V)
    last = synth.initial_tokens(B, V)
    traj = [last.astype(np.int64)]
    for _ in range(steps * (K + 1) + K + 2):
        traj.append(gmap[traj[-1]])
    traj = np.stack(traj, axis=1)            # traj[b, i]: i-th token after start
    pos = np.zeros(B, np.int64)
    total = 0
    for _ in range(steps):
        cont = np.stack([traj[b, pos[b] + 1:pos[b] + 1 + K] for b in range(B)])
        drafts = synth.draft_tokens(cont, pos, acc, V)
        tokens = np.concatenate([traj[np.arange(B), pos][:, None], drafts], axis=1)
        greedy = gmap[tokens]
        n, commit, clen, nxt = oracle.mtp_verify(tokens, greedy)
        for b in range(B):
            np.testing.assert_array_equal(commit[b, :clen[b]], traj[b, pos[b] + 1:pos[b] + 1 + clen[b]])
        pos += clen
        total += clen.sum()
    tau = total / (B * steps)
    assert abs(tau - oracle.expected_tau(acc)) < 0.10
    assert abs(tau - t8["tau_eager"]) < 0.11


# ---------------------------------------------------------------------------
# whole model: losslessness on the tiny fp32 model

@pytest.fixture(scope="module")
def tiny_model():
    return synth.model_weights(synth.TINY)


def test_speculative_commits_equal_greedy_rollout(tiny_model):
    wl = synth.WORKLOADS["tiny_verify_b4k3"]
    B, K, V = wl.batch, wl.drafts, wl.shape.vocab
    last0 = synth.initial_tokens(B, V)
    roll = oracle.greedy_rollout(last0, tiny_model, wl.steps * (K + 1) + K + 1, operands="exact")
    traj = np.concatenate([last0[:, None], roll], axis=1)
    pos = np.zeros(B, np.int64)
    committed = [[] for _ in range(B)]
    last = last0.copy()
    for _ in range(wl.steps):
        cont = np.stack([traj[b, pos[b] + 1:pos[b] + 1 + K] for b in range(B)])
        drafts = synth.draft_tokens(cont, pos, wl.accept, V, mode=wl.draft_mode)
        st = oracle.verify_step(last, drafts, tiny_model, operands="exact")
        for b in range(B):
            committed[b].extend(st["commit"][b, :st["commit_len"][b]].tolist())
        pos += st["commit_len"]
        last = st["next_last"]
    for b in range(B):
        assert committed[b] == roll[b, :len(committed[b])].tolist()
    tau = np.mean([len(c) for c in committed]) / wl.steps
    p = 0.7 + 0.3 / V
    # 4 sequences x 16 steps: loose 4-sigma band (per-step SD ~1.0, /8)
    assert abs(tau - oracle.expected_tau([p] * K)) < 0.5


def test_verify_step_batch_rows_independent(tiny_model):
    """No attention: a token's greedy successor does not depend on its batch."""
    toks = np.array([5, 17, 300, 5, 42], np.int32)
    full = oracle.model_greedy(toks, tiny_model, "exact")["argmax"]
    for i, t in enumerate(toks):
        assert oracle.model_greedy(np.array([t]), tiny_model, "exact")["argmax"][0] == full[i]
    assert full[0] == full[3]


# ---------------------------------------------------------------------------
# shapes against the pages' sizes

def test_decoder_shape_matches_pages():
    d = _golden("decoder_shape.json")
    s = synth.DECODER
    assert (s.n_routed, s.n_shared, s.top_k) == (d["routed_experts"], d["shared_experts"], d["top_k"])
    expert = 3 * s.inter * s.hidden
    per_layer = (s.n_routed + s.n_shared) * expert + s.n_routed * s.hidden
    total = s.n_layers * per_layer + 2 * s.vocab * s.hidden
    active = s.n_layers * ((s.top_k + s.n_shared) * expert + s.n_routed * s.hidden) + s.vocab * s.hidden
    assert 0.8 < total / d["decoder_params"] < 1.2          # "around three billion"
    assert 0.6 < active / d["active_params_per_token"] < 1.2  # attention is not modelled


def test_y_slots_layout_per_slot():
    """Slot r of token t holds w[t, r] times expert idx[t, r]'s output; slot
    k+s holds shared expert s with weight 1 (checked through torch)."""
    rng = np.random.default_rng(21)
    H, I, E, k, ns, T = 16, 8, 6, 2, 2, 9
    layer = _rand_layer(rng, H, E, I, ns)
    h = rng.standard_normal((T, H))
    st = oracle.moe_layer(h, layer, "f32", k, E, ns, 1e-6, operands="exact")
    for t in range(T):
        for r in range(k + ns):
            e = st["idx"][t, r] if r < k else E + (r - k)
            wt = st["w"][t, r] if r < k else 1.0
            ref = wt * _torch_swiglu(st["x"][t:t + 1], layer["w_gate"][e], layer["w_up"][e],
                                     layer["w_down"][e])[0]
            np.testing.assert_allclose(st["y_slots"][t, r], ref, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# FastMTP draft block (oracle.draft_block): closed forms under special weights

def _tiny_draft(model, rng=None, std=0.2):
    """Draft weights for the tiny model (fp32), random or to be overwritten."""
    d = synth.draft_weights(synth.TINY)
    if rng is not None:
        for key in ("w_proj", "w_gate", "w_up", "w_down"):
            d[key] = (rng.standard_normal(d[key].shape) * std).astype(np.float32)
    return d


def _zero_ffn(d):
    d["w_down"] = np.zeros_like(d["w_down"])
    return d


def test_draft_copy_through_is_the_verifier_head(tiny_model):
    """W_p = [I | 0] and no FFN: z_1 = RMSNorm(z_0), so the draft is the
    verifier head's greedy token of z_0 (RMSNorm is idempotent up to eps)."""
    H = synth.TINY.hidden
    d = _zero_ffn(_tiny_draft(tiny_model))
    d["w_proj"] = np.stack([np.eye(H), np.zeros((H, H))]).astype(np.float32)
    d["norm_out"] = np.asarray(tiny_model["norm_f"])
    z0 = synth.draft_states(synth.TINY, 16)
    t0 = np.arange(16) * 7
    out = oracle.draft_block(z0, t0, d, tiny_model, 1, "exact")
    ref = oracle.lm_head(z0, tiny_model["norm_f"], tiny_model["w_lm"], "f32", synth.TINY.eps, "exact")
    assert np.all(ref["gap"] > 1e-6)
    np.testing.assert_array_equal(out["drafts"][:, 0], ref["argmax"])
    ms = np.mean(np.asarray(z0, np.float64) ** 2, axis=1, keepdims=True)
    np.testing.assert_allclose(out["z"], z0 / np.sqrt(ms + synth.TINY.eps), rtol=1e-12)


def test_draft_embedding_echo_repeats_the_token(tiny_model):
    """W_p = [0 | I], no FFN, head tied to an embedding whose rows all have the
    same norm: the draft maximises e_v . e_t over v, which by Cauchy-Schwarz is
    v = t, at every one of the K recursive steps."""
    H, V = synth.TINY.hidden, synth.TINY.vocab
    rng = np.random.default_rng(11)
    emb = rng.standard_normal((V, H))
    emb = (emb / np.linalg.norm(emb, axis=1, keepdims=True)).astype(np.float32)
    model = dict(tiny_model, emb=emb, w_lm=emb)
    d = _zero_ffn(_tiny_draft(model))
    d["w_proj"] = np.stack([np.zeros((H, H)), np.eye(H)]).astype(np.float32)
    # a negative norm_z would flip the echo if it were applied to the embedding half
    d["norm_z"] = np.full(H, -1.0, np.float32)
    d["norm_e"] = np.full(H, 2.0, np.float32)
    t0 = rng.integers(0, V, 24)
    z0 = synth.draft_states(synth.TINY, 24)
    out = oracle.draft_block(z0, t0, d, model, 3, "exact")
    np.testing.assert_array_equal(out["drafts"], np.repeat(t0[:, None], 3, axis=1))


@pytest.mark.parametrize("s,i", [(0, 0), (2, 17), (1, 63)])
def test_draft_single_unit_ffn_closed_form(tiny_model, s, i):
    """Only unit i of slice s of the dense FFN is non-zero (gate row a, up row
    b, down column c): z_1 = z' + c * SiLU(a.x) * (b.x), x = RMSNorm(z'), with
    z' = RMSNorm(z_0) from W_p = [I | 0]."""
    H = synth.TINY.hidden
    rng = np.random.default_rng(5 + s * 100 + i)
    d = _tiny_draft(tiny_model)
    for key in ("w_gate", "w_up", "w_down"):
        d[key] = np.zeros_like(d[key])
    a, b, c = (rng.standard_normal(H) for _ in range(3))
    d["w_gate"][s, i] = a
    d["w_up"][s, i] = b
    d["w_down"][s, :, i] = c
    d["w_proj"] = np.stack([np.eye(H), np.zeros((H, H))]).astype(np.float32)
    gz, gf, ge = (rng.uniform(0.5, 1.5, H).astype(np.float32) for _ in range(3))
    d["norm_z"], d["norm_ffn"], d["norm_e"] = gz, gf, ge
    z0 = synth.draft_states(synth.TINY, 8).astype(np.float64)
    out = oracle.draft_block(z0, np.zeros(8, np.int64), d, tiny_model, 1, "exact")
    eps = synth.TINY.eps
    zp = z0 / np.sqrt(np.mean(z0 ** 2, axis=1, keepdims=True) + eps) * gz
    x = zp / np.sqrt(np.mean(zp ** 2, axis=1, keepdims=True) + eps) * gf
    ga = x @ a.astype(np.float32).astype(np.float64)
    ub = x @ b.astype(np.float32).astype(np.float64)
    want = zp + np.outer(ga / (1 + np.exp(-ga)) * ub, c.astype(np.float32).astype(np.float64))
    np.testing.assert_allclose(out["z"], want, rtol=1e-10, atol=1e-12)


def test_draft_recursion_feeds_state_and_token(tiny_model):
    """K = 3 in one call equals three calls of K = 1, each fed the previous
    call's (z, draft token)."""
    d = _tiny_draft(tiny_model, np.random.default_rng(3))
    z = synth.draft_states(synth.TINY, 12)
    t = np.arange(12) * 31 % synth.TINY.vocab
    full = oracle.draft_block(z, t, d, tiny_model, 3)
    for j in range(3):
        one = oracle.draft_block(z, t, d, tiny_model, 1)
        np.testing.assert_array_equal(one["drafts"][:, 0], full["drafts"][:, j])
        np.testing.assert_array_equal(one["z"], full["zs"][j])
        z, t = one["z"], one["drafts"][:, 0]


def test_draft_dense_slices_layout():
    """The stored slices make up the dense matrices as documented: column
    block g of W_p is w_proj[g]; intermediate rows s*I..(s+1)*I-1 of W_gate are
    w_gate[s]; columns s*I.. of W_down are w_down[s]."""
    d = synth.draft_weights(synth.TINY)
    H, I, n = synth.TINY.hidden, synth.TINY.inter, d["n_slices"]
    dd = oracle.draft_dense(d)
    assert dd["w_p"].shape == (H, 2 * H) and dd["w_gate"].shape == (n * I, H)
    assert dd["w_down"].shape == (H, n * I)
    np.testing.assert_array_equal(dd["w_p"][:, H:], d["w_proj"][1])
    np.testing.assert_array_equal(dd["w_gate"][2 * I:3 * I], d["w_gate"][2])
    np.testing.assert_array_equal(dd["w_up"][I:2 * I], d["w_up"][1])
    np.testing.assert_array_equal(dd["w_down"][:, (n - 1) * I:], d["w_down"][n - 1])
