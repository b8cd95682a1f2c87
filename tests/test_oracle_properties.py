"""Property tests of the CPU oracle over random shapes and values (hypothesis).

Each property is checked against something other than the oracle's own
formula: a closed form, a library routine, a different formulation of the same
definition, or an invariance a plausible indexing mistake would break.  The
fixed pins live in test_oracle_pins.py; these widen them to random inputs.
"""
import numpy as np
import scipy.special
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle

SETTINGS = settings(max_examples=40, deadline=None, suppress_health_check=[HealthCheck.too_slow])


def _rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------ router

@SETTINGS
@given(T=st.integers(1, 6), E=st.integers(1, 16), H=st.integers(1, 24), kfrac=st.floats(0.0, 1.0),
       seed=st.integers(0, 2**31 - 1), biased=st.booleans())
def test_route_properties(T, E, H, kfrac, seed, biased):
    """Routing of random states: the chosen experts are the k largest logits
    in rank order (NumPy's stable sort of the negated logits); the weights are
    positive, non-increasing, sum to 1 and equal scipy's softmax over the
    chosen logits; the pairwise ratio w_i / w_j is exp(l_i - l_j)."""
    k = max(1, min(E, 1 + int(kfrac * E)))
    rng = _rng(seed)
    x = rng.standard_normal((T, H))
    wr = rng.standard_normal((E, H))
    bias = rng.standard_normal(E) if biased else None
    idx, w, logits = oracle.route(x, wr, k, bias)
    ref_logits = x @ wr.T + (bias if biased else 0.0)
    np.testing.assert_allclose(logits, ref_logits, rtol=1e-12, atol=1e-12)
    for t in range(T):
        want = np.argsort(-logits[t], kind="stable")[:k]
        np.testing.assert_array_equal(idx[t], want)
        assert np.all(w[t] > 0)
        assert np.all(np.diff(w[t]) <= 1e-15)
        assert abs(w[t].sum() - 1.0) < 1e-12
        np.testing.assert_allclose(w[t], scipy.special.softmax(logits[t, idx[t]]), rtol=1e-12)
        l_sel = logits[t, idx[t]]
        np.testing.assert_allclose(w[t] / w[t][0], np.exp(l_sel - l_sel[0]), rtol=1e-10)


@SETTINGS
@given(T=st.integers(1, 5), E=st.integers(2, 12), seed=st.integers(0, 2**31 - 1))
def test_route_gap_is_kth_minus_next(T, E, seed):
    """The near-tie gap is the k-th minus the (k+1)-th largest logit, and a
    tie planted at that boundary gives gap 0 with the lower index chosen."""
    rng = _rng(seed)
    k = int(rng.integers(1, E))
    logits = rng.standard_normal((T, E))
    gap = oracle.route_gap(logits, k)
    s = np.sort(logits, axis=1)[:, ::-1]
    np.testing.assert_allclose(gap, s[:, k - 1] - s[:, k])
    # plant: expert b copies expert a's logit, where a is the k-th choice
    order = np.argsort(-logits[0], kind="stable")
    a, b = order[k - 1], order[k]
    logits[0, b] = logits[0, a]
    assert oracle.route_gap(logits, k)[0] == 0.0
    # routing those logits (identity router): of the two tied experts at the
    # boundary, exactly the lower index is chosen
    idx, _, _ = oracle.route(logits[:1], np.eye(E), k)
    assert min(a, b) in idx[0] and max(a, b) not in idx[0]


# ----------------------------------------------------------------- permute

@SETTINGS
@given(T=st.integers(0, 40), E=st.integers(1, 10), ns=st.integers(0, 3), seed=st.integers(0, 2**31 - 1))
def test_permute_is_a_stable_grouping(T, E, ns, seed):
    """sorted_src is a bijection on the pair ids; reading it in order visits
    groups in non-decreasing order and, inside a group, pair ids in
    increasing order (= NumPy's stable argsort of the group ids); offsets are
    the exclusive prefix sums of bincount."""
    rng = _rng(seed)
    k = int(rng.integers(1, E + 1))
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32) if T else np.zeros((0, k), np.int32)
    offsets, src = oracle.permute(idx, E, ns)
    S = k + ns
    P = T * S
    assert sorted(src.tolist()) == list(range(P))
    groups = np.empty(P, np.int64)
    if T:
        groups.reshape(T, S)[:, :k] = idx
        for s in range(ns):
            groups.reshape(T, S)[:, k + s] = E + s
    np.testing.assert_array_equal(src, np.argsort(groups, kind="stable"))
    counts = np.bincount(groups, minlength=E + ns)
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))


# ------------------------------------------------------------------- accept

@SETTINGS
@given(V=st.integers(2, 12), K=st.integers(0, 5), B=st.integers(1, 6), seed=st.integers(0, 2**31 - 1))
def test_accept_commits_follow_the_greedy_rollout(V, K, B, seed):
    """For a model that is a random token map g (greedy[j] = g(tokens[j])),
    the committed tokens are always the next n+1 tokens of the rollout
    last, g(last), g(g(last)), ...: the lossless property, checked against a
    rollout rather than the acceptance rule.  Drafts are planted to be right
    for a random prefix, then arbitrary."""
    rng = _rng(seed)
    g = rng.integers(0, V, size=V)
    last = rng.integers(0, V, size=B)
    roll = np.empty((B, K + 2), np.int64)
    roll[:, 0] = last
    for j in range(K + 1):
        roll[:, j + 1] = g[roll[:, j]]
    drafts = rng.integers(0, V, size=(B, K))
    good = rng.integers(0, K + 1, size=B)
    for b in range(B):
        drafts[b, :good[b]] = roll[b, 1:1 + good[b]]
    tokens = np.concatenate([last[:, None], drafts], axis=1)
    greedy = g[tokens]
    n, commit, clen, nxt = oracle.mtp_verify(tokens, greedy)
    for b in range(B):
        assert n[b] >= good[b]
        assert clen[b] == n[b] + 1
        np.testing.assert_array_equal(commit[b, :clen[b]], roll[b, 1:clen[b] + 1])
        assert np.all(commit[b, clen[b]:] == -1)
        assert nxt[b] == roll[b, clen[b]]


# ----------------------------------------------------------------- RMSNorm

@SETTINGS
@given(T=st.integers(1, 5), H=st.integers(1, 64), scale=st.floats(1e-3, 1e3), seed=st.integers(0, 2**31 - 1))
def test_rmsnorm_closed_forms(T, H, scale, seed):
    """With gain 1: mean(y^2) = m / (m + eps) for m = mean(h^2); scaling h by
    c > 0 with eps = 0 leaves y unchanged; a gain multiplies y elementwise."""
    rng = _rng(seed)
    h = rng.standard_normal((T, H)) + 0.1
    eps = 1e-6
    y = oracle.rmsnorm(h, 1.0, eps)
    m = np.mean(h * h, axis=1)
    np.testing.assert_allclose(np.mean(y * y, axis=1), m / (m + eps), rtol=1e-12)
    np.testing.assert_allclose(oracle.rmsnorm(scale * h, 1.0, 0.0), oracle.rmsnorm(h, 1.0, 0.0), rtol=1e-10)
    gam = rng.standard_normal(H)
    np.testing.assert_allclose(oracle.rmsnorm(h, gam, eps), y * gam, rtol=1e-12, atol=1e-15)


# ------------------------------------------------------------------ arg max

@SETTINGS
@given(T=st.integers(1, 6), V=st.integers(1, 300), seed=st.integers(0, 2**31 - 1))
def test_first_argmax_with_planted_ties(T, V, seed):
    """first_argmax equals np.argmax (which returns the first maximum) on
    rows with several planted copies of the maximum."""
    rng = _rng(seed)
    rows = rng.standard_normal((T, V))
    for t in range(T):
        where = rng.integers(0, V, size=min(V, 3))
        rows[t, where] = rows[t].max() + 1.0
    np.testing.assert_array_equal(oracle.first_argmax(rows), np.argmax(rows, axis=1))


# ------------------------------------------------------- grouped FFN layout

@SETTINGS
@given(T=st.integers(1, 7), seed=st.integers(0, 2**31 - 1))
def test_grouped_ffn_is_token_equivariant(T, seed):
    """Permuting the tokens (their rows, routing and weights) permutes the
    per-slot expert outputs the same way: a token's outputs depend on its own
    row only, whatever its position and companions.  Also checks the slot
    layout against a direct per-token SwiGLU for a few pairs."""
    rng = _rng(seed)
    H, I, E, k, ns = 6, 5, 4, 2, 1
    x = rng.standard_normal((T, H))
    wg = rng.standard_normal((E + ns, I, H)) * 0.3
    wu = rng.standard_normal((E + ns, I, H)) * 0.3
    wd = rng.standard_normal((E + ns, H, I)) * 0.3
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k))
    w /= w.sum(axis=1, keepdims=True)
    off, src = oracle.permute(idx, E, ns)
    y = oracle.grouped_ffn(x, src, off, w, wg, wu, wd, "f32", k, ns)
    perm = rng.permutation(T)
    off2, src2 = oracle.permute(idx[perm], E, ns)
    y2 = oracle.grouped_ffn(x[perm], src2, off2, w[perm], wg, wu, wd, "f32", k, ns)
    np.testing.assert_allclose(y2, y[perm], rtol=1e-12, atol=1e-14)
    t = int(rng.integers(0, T))
    for slot in range(k + ns):
        gidx = idx[t, slot] if slot < k else E + slot - k
        scale = w[t, slot] if slot < k else 1.0
        z = x[t]
        a = (wg[gidx] @ z) * scipy.special.expit(wg[gidx] @ z) * (wu[gidx] @ z)
        np.testing.assert_allclose(y[t, slot], scale * (wd[gidx] @ a), rtol=1e-10, atol=1e-13)
