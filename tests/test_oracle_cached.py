"""Pins of the oracle's decoder with an attention sublayer and per-sequence
caches (oracle.cached_*), on the tiny model, on the CPU."""
import copy

import numpy as np
import pytest

import oracle
import synth

HEADS = 2   # 64-wide heads at H = 128


@pytest.fixture(scope="module")
def tiny():
    return synth.model_weights(synth.TINY), synth.attention_weights(synth.TINY)


def _caches(B, L, H, n_layers):
    return [{"k": np.zeros((B, L, H)), "v": np.zeros((B, L, H))} for _ in range(n_layers)]


def test_zero_output_projection_is_the_moe_only_model(tiny):
    """W_o = 0: the attention sublayer adds nothing, so every row's greedy
    token and final state equal the decoder without attention, exactly."""
    model, attn = tiny
    attn0 = [dict(a, w_o=np.zeros_like(a["w_o"])) for a in attn]
    B, rows, H = 3, 4, synth.TINY.hidden
    tokens = synth.counter_randint(synth.TINY.vocab, 8, np.arange(B)[:, None], np.arange(rows)[None, :])
    got = oracle.cached_greedy(tokens, model, attn0, _caches(B, 16, H, len(attn)), np.array([0, 3, 7]), HEADS,
                               "exact")
    ref = oracle.model_greedy(tokens.reshape(-1), model, "exact")
    np.testing.assert_array_equal(got["argmax"].reshape(-1), ref["argmax"])
    np.testing.assert_array_equal(got["h"], ref["h"])
    np.testing.assert_array_equal(got["router_gap"].reshape(-1), ref["router_gap"])
    np.testing.assert_array_equal(got["gap"].reshape(-1), ref["gap"])


def test_attention_makes_tokens_depend_on_the_prefix(tiny):
    """The same token at the same position gives a different final state
    after a different history (the cache carries it)."""
    model, attn = tiny
    H = synth.TINY.hidden
    outs = []
    for hist in ([5, 9, 11], [200, 3, 77]):
        caches = _caches(1, 8, H, len(attn))
        oracle.cached_greedy(np.array([hist]), model, attn, caches, np.array([0]), HEADS, "exact")
        outs.append(oracle.cached_greedy(np.array([[42]]), model, attn, caches, np.array([3]), HEADS, "exact")["h"])
    assert np.abs(outs[0] - outs[1]).max() > 1e-3


@pytest.mark.parametrize("K", [1, 3])
def test_speculative_commits_equal_the_cached_rollout(tiny, K):
    """Losslessness with attention: verify passes over (last, drafts) with
    drafts right with probability 0.7 commit exactly the tokens of plain
    greedy decoding, although each pass writes cache rows for drafts that are
    later rejected (they are overwritten once the position advances past
    the accepted prefix)."""
    model, attn = tiny
    B, H, V, steps = 4, synth.TINY.hidden, synth.TINY.vocab, 8
    L = steps * (K + 1) + 2
    last0 = synth.initial_tokens(B, V)
    ref = oracle.cached_rollout(last0, model, attn, _caches(B, L, H, len(attn)), np.zeros(B, np.int64), HEADS,
                                steps * (K + 1) + 1, "exact")
    caches = _caches(B, L, H, len(attn))
    pos = np.zeros(B, np.int64)
    last = last0.astype(np.int64)
    done = np.zeros(B, np.int64)
    commits = [[] for _ in range(B)]
    rng = np.random.default_rng(K)
    for _ in range(steps):
        drafts = np.empty((B, K), np.int64)
        for b in range(B):
            for j in range(K):
                right = ref[b, done[b] + j]
                drafts[b, j] = right if rng.random() < 0.7 else rng.integers(0, V)
        st = oracle.cached_verify_step(last, drafts, model, attn, caches, pos, HEADS, "exact")
        for b in range(B):
            commits[b].extend(st["commit"][b, :st["commit_len"][b]].tolist())
        done += st["commit_len"]
        pos = st["pos"]
        last = st["next_last"].astype(np.int64)
    for b in range(B):
        np.testing.assert_array_equal(commits[b], ref[b, :len(commits[b])])
    assert done.min() > steps   # some drafts were accepted
