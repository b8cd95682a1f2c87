"""Verify steps with an attention sublayer in every layer
(moev_verify_step_attn): parity with the oracle's cached decoder, and
losslessness against the GPU's own one-row greedy rollout over the same
caches."""
import copy

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import dev_i32, host, need_gpu, report

pytestmark = pytest.mark.gpu

HEAD_GAP, ROUTE_GAP = 1e-2, 1e-3

# two bf16 layers with the decoder's 128-wide heads
ATTN_BF16 = synth.ModelShape("attn_bf16", hidden=256, n_routed=16, inter=128, top_k=4, n_shared=2,
                             vocab=2048, n_layers=2, dtype="bf16", model_id=5)


@pytest.fixture(scope="module")
def model_mod():
    need_gpu()
    from moe_decoder_greedy_amd import model
    return model


def _prefix_caches(shape, B, rows, L, prefix, seed):
    """Per layer a key and a value cache [B, L, H] with seeded values at every
    position (those at and past pos[b] are overwritten before they are read),
    and the per-sequence prefix lengths pos."""
    out = []
    for layer in range(shape.n_layers):
        a = synth.attention_inputs(B, rows, shape.hidden, L, prefix, seed=seed + layer,
                                   bf16=shape.dtype == "bf16")
        out.append(a)
    return out, out[0]["pos"].astype(np.int64)


def _oracle_caches(raw, dt):
    return [{"k": oracle.to_f64(a["k_cache"], dt), "v": oracle.to_f64(a["v_cache"], dt)} for a in raw]


def _load_caches(dm, raw):
    """The oracle's [B, L, H] caches into the device model's head-major
    [B, heads, L, D] ones."""
    for A, a in zip(dm.attn, raw):
        for key, src in (("k", a["k_cache"]), ("v", a["v_cache"])):
            t = torch.from_numpy(src.view(np.int16)).view(torch.bfloat16) if src.dtype == np.uint16 \
                else torch.from_numpy(src)
            B, heads, L, D = A[key].shape
            A[key].copy_(t.view(B, L, heads, D).permute(0, 2, 1, 3).contiguous().to(A[key].device))


def _gpu_cache(A, key):
    """A device cache back in the oracle's [B, L, H] layout, float64."""
    t = A[key]
    B, heads, L, D = t.shape
    t = t.permute(0, 2, 1, 3).reshape(B, L, heads * D)
    return (t.float() if t.dtype == torch.bfloat16 else t).cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("K", [3, 7, 15])
def test_attn_step_tiny_matches_oracle(model_mod, K):
    """The tiny fp32 model, 3 sequences, K drafts (4, 8 and 16 rows per
    sequence: every row-count build of the attention kernel, whose last split
    merges the states), four passes: unflagged greedy tokens equal the
    oracle's, acceptance follows them, every cache row the passes wrote
    matches the oracle's, and pos advances by commit_len."""
    shape, heads = synth.TINY, 2
    w = synth.model_weights(shape)
    attn = synth.attention_weights(shape)
    B, L = 3, 24 + 4 * (K + 1)
    raw, pos = _prefix_caches(shape, B, K + 1, L, (0, 20), seed=41)
    dm = model_mod.DeviceModel(w)
    dm.attach_attention(attn, heads, B, L)
    _load_caches(dm, raw)
    caches = _oracle_caches(raw, shape.dtype)
    pos_d = dev_i32(pos.astype(np.int32))
    rng = np.random.default_rng(9)
    for step in range(4):
        tokens = rng.integers(0, shape.vocab, size=(B, K + 1)).astype(np.int64)
        if step % 2 == 1:   # the first draft right, so acceptance varies
            probe = oracle.cached_greedy(tokens[:, :1], w, attn, copy.deepcopy(caches), pos, heads, "exact")
            tokens[:, 1] = probe["argmax"][:, 0]
        ref = oracle.cached_greedy(tokens, w, attn, caches, pos, heads, "exact")
        out = dm.verify_step_attn(dev_i32(tokens.astype(np.int32)), pos_d)
        gg = host(out["greedy"])
        flagged = (ref["gap"] < HEAD_GAP) | (ref["router_gap"] < ROUTE_GAP)
        report("attn_step_tiny", step=step, pos=pos.tolist(), flagged=int(flagged.sum()))
        np.testing.assert_array_equal(gg[~flagged], ref["argmax"][~flagged])
        n, c, l, nx = oracle.mtp_verify(tokens, gg)
        np.testing.assert_array_equal(host(out["n_accept"]), n)
        np.testing.assert_array_equal(host(out["commit"]), c)
        np.testing.assert_array_equal(host(out["next_last"]), nx)
        for A, cache in zip(dm.attn, caches):
            for key in ("k", "v"):
                got = _gpu_cache(A, key)
                for b in range(B):
                    rows = slice(int(pos[b]), int(pos[b]) + K + 1)
                    np.testing.assert_allclose(got[b, rows], cache[key][b, rows], rtol=1e-4, atol=1e-5)
        pos = pos + l
        np.testing.assert_array_equal(host(pos_d), pos)


def _rollout(dm, last, pos0, n):
    """n greedy tokens per sequence, one row per pass (K = 0)."""
    cur = torch.from_numpy(last.astype(np.int32)).cuda().reshape(-1, 1)
    pos = dev_i32(pos0.astype(np.int32))
    seq = []
    for _ in range(n):
        out = dm.verify_step_attn(cur, pos)
        cur = out["next_last"].reshape(-1, 1).clone()
        seq.append(host(cur)[:, 0])
    return np.stack(seq, axis=1)


@pytest.mark.parametrize("B,K", [(8, 1), (8, 3), (8, 7), (32, 1), (32, 3)])
def test_attn_step_is_lossless(model_mod, B, K):
    """Speculative passes with drafts right with probability 0.7 commit exactly
    the tokens of one-row greedy decoding from the same caches, bit for bit,
    although every pass writes cache rows for drafts that are then rejected.
    The first pass's unflagged greedy tokens also equal the oracle's (bf16
    operands).  At B = 32 the verify passes (64 or 128 rows) run the dense
    projections split over several 32-row passes with two row tiles per
    workgroup, while the one-row rollout (32 rows) runs them as one pass of
    one row tile: the commits show both give the same bits."""
    shape, heads = ATTN_BF16, 2
    w = synth.model_weights(shape)
    attn = synth.attention_weights(shape)
    steps = 10
    L = 120 + steps * (K + 1) + K + 2
    raw, pos0 = _prefix_caches(shape, B, K + 1, L, (0, 120), seed=51)
    dm = model_mod.DeviceModel(w)
    dm.attach_attention(attn, heads, B, L)
    last0 = synth.initial_tokens(B, shape.vocab).astype(np.int64)
    _load_caches(dm, raw)
    ref = _rollout(dm, last0, pos0, steps * (K + 1) + 1)

    _load_caches(dm, raw)
    rng = np.random.default_rng(K)
    pos_d = dev_i32(pos0.astype(np.int32))
    last = last0.copy()
    done = np.zeros(B, np.int64)
    commits = [[] for _ in range(B)]
    for step in range(steps):
        drafts = np.empty((B, K), np.int64)
        for b in range(B):
            for j in range(K):
                right = ref[b, done[b] + j]
                drafts[b, j] = right if rng.random() < 0.7 else rng.integers(0, shape.vocab)
        tokens = np.concatenate([last[:, None], drafts], axis=1)
        if step == 0:
            orc = oracle.cached_greedy(tokens, w, attn, _oracle_caches(raw, shape.dtype), pos0, heads, "bf16")
        out = dm.verify_step_attn(dev_i32(tokens.astype(np.int32)), pos_d)
        if step == 0:
            flagged = (orc["gap"] < HEAD_GAP) | (orc["router_gap"] < ROUTE_GAP)
            gg = host(out["greedy"])
            report("attn_step_bf16", flagged=int(flagged.sum()), mismatches=int((gg != orc["argmax"]).sum()))
            np.testing.assert_array_equal(gg[~flagged], orc["argmax"][~flagged])
        clen = host(out["commit_len"])
        cm = host(out["commit"])
        for b in range(B):
            commits[b].extend(cm[b, :clen[b]].tolist())
        done += clen
        last = host(out["next_last"]).astype(np.int64)
    np.testing.assert_array_equal(host(pos_d), pos0 + done)
    accepted = 0
    for b in range(B):
        n = len(commits[b])
        accepted += n
        np.testing.assert_array_equal(np.array(commits[b]), ref[b, :n])
    report("attn_step_lossless", K=K, committed=accepted, tau=accepted / (B * steps))
    assert accepted > B * steps   # some drafts were accepted


def test_attn_step_decoder_all_rows(model_mod):
    """The benchmark's shape: the 12-layer decoder with its 129280-token head,
    10 heads of 128, B = 32, K = 3, every layer's caches holding the same
    seeded prefix (100-300 positions).  Every greedy token of all 32
    sequences (128 rows) is recomputed by the oracle from the same caches
    (bf16 operands); unflagged ones must match, and acceptance follows the
    GPU's tokens."""
    shape, heads = synth.DECODER, 10
    report("attn_step_decoder", msg="generating the 12-layer decoder and its attention weights")
    w = synth.model_weights(shape)
    attn = synth.attention_weights(shape)
    B, K, L = 32, 3, 320
    a = synth.attention_inputs(B, K + 1, shape.hidden, L, (100, 300), seed=61)
    dm = model_mod.DeviceModel(w)
    dm.attach_attention(attn, heads, B, L)
    _load_caches(dm, [a] * shape.n_layers)
    pos = a["pos"].astype(np.int64)
    rng = np.random.default_rng(12)
    tokens = rng.integers(0, shape.vocab, size=(B, K + 1)).astype(np.int64)
    out = dm.verify_step_attn(dev_i32(tokens.astype(np.int32)), dev_i32(pos.astype(np.int32)))
    gg = host(out["greedy"])
    sample = list(range(B))
    sub = {key: a[key][sample] for key in ("k_cache", "v_cache")}
    caches = [{"k": oracle.to_f64(sub["k_cache"], "bf16"), "v": oracle.to_f64(sub["v_cache"], "bf16")}
              for _ in range(shape.n_layers)]
    ref = oracle.cached_greedy(tokens[sample], w, attn, caches, pos[sample], heads, "bf16")
    flagged = (ref["gap"] < HEAD_GAP) | (ref["router_gap"] < ROUTE_GAP)
    got = gg[sample]
    report("attn_step_decoder", flagged=int(flagged.sum()), mismatches=int((got != ref["argmax"]).sum()))
    np.testing.assert_array_equal(got[~flagged], ref["argmax"][~flagged])
    n, c, l, nx = oracle.mtp_verify(tokens, gg)
    np.testing.assert_array_equal(host(out["commit"]), c)
    np.testing.assert_array_equal(host(out["next_last"]), nx)


def test_attn_step_graph_replays(model_mod):
    """Three consecutive passes captured as one HIP graph (cache writes,
    attention workspace and the position advance inside it), replayed three
    times from the same restored caches and positions, with eager passes in
    between: every replay reproduces the eager outputs, positions and caches
    bit for bit."""
    shape, heads = ATTN_BF16, 2
    w = synth.model_weights(shape)
    attn = synth.attention_weights(shape)
    B, K, n_steps = 8, 3, 3
    L = 120 + n_steps * (K + 1) + 8
    raw, pos0 = _prefix_caches(shape, B, K + 1, L, (0, 120), seed=71)
    dm = model_mod.DeviceModel(w)
    dm.attach_attention(attn, heads, B, L)
    rng = np.random.default_rng(5)
    toks = [dev_i32(rng.integers(0, shape.vocab, size=(B, K + 1))) for _ in range(n_steps)]
    pos_d = dev_i32(pos0.astype(np.int32))

    def restore():
        _load_caches(dm, raw)
        pos_d.copy_(dev_i32(pos0.astype(np.int32)))
        torch.cuda.synchronize()

    restore()
    eager = [{k: host(v) for k, v in dm.verify_step_attn(t, pos_d).items()} for t in toks]
    eager_pos = host(pos_d)
    eager_k = [_gpu_cache(A, "k") for A in dm.attn]
    outs = [dm.alloc_outputs(B, K) for _ in range(n_steps)]
    restore()
    dm.verify_step_attn(toks[0], pos_d, out=outs[0])   # workspace and code objects ready
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t, o in zip(toks, outs):
            dm.verify_step_attn(t, pos_d, out=o)
    other = dev_i32(rng.integers(0, shape.vocab, size=(B, K + 1)))
    for r in range(3):
        restore()
        for o in outs:
            for v in o.values():
                v.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for s in range(n_steps):
            for k in ("greedy", "n_accept", "commit", "commit_len", "next_last"):
                np.testing.assert_array_equal(host(outs[s][k]), eager[s][k], err_msg=f"replay {r} step {s} {k}")
        np.testing.assert_array_equal(host(pos_d), eager_pos)
        for A, want in zip(dm.attn, eager_k):
            np.testing.assert_array_equal(_gpu_cache(A, "k"), want)
        dm.verify_step_attn(other, pos_d)                # eager work between replays
        torch.cuda.synchronize()
    report("attn_graph", B=B, K=K, steps=n_steps, replays=3)


def test_attn_step_leaves_a_full_cache_alone(model_mod):
    """A sequence whose cache has no room for the pass (pos + K + 1 > max_len)
    commits nothing: commit_len 0, n_accept -1, a commit row of -1, next_last
    its own last token, its position and every row of its caches unchanged.
    The other sequences of the pass, one of them filling its cache exactly,
    match the oracle's cached decoder."""
    shape, heads = synth.TINY, 2
    w = synth.model_weights(shape)
    attn = synth.attention_weights(shape)
    B, K, L = 3, 3, 20
    raw, _ = _prefix_caches(shape, B, K + 1, L, (0, 0), seed=81)
    pos = np.array([0, L - (K + 1), L - K], np.int64)   # fits, fits exactly, one row short
    dm = model_mod.DeviceModel(w)
    dm.attach_attention(attn, heads, B, L)
    _load_caches(dm, raw)
    before = [{key: _gpu_cache(A, key) for key in ("k", "v")} for A in dm.attn]
    tokens = np.random.default_rng(3).integers(0, shape.vocab, size=(B, K + 1)).astype(np.int64)
    pos_d = dev_i32(pos.astype(np.int32))
    out = dm.verify_step_attn(dev_i32(tokens.astype(np.int32)), pos_d)
    torch.cuda.synchronize()
    assert host(out["commit_len"])[2] == 0 and host(out["n_accept"])[2] == -1
    np.testing.assert_array_equal(host(out["commit"])[2], np.full(K + 1, -1))
    assert host(out["next_last"])[2] == tokens[2, 0]
    np.testing.assert_array_equal(host(pos_d), pos + np.append(host(out["commit_len"])[:2], 0))
    for A, b4 in zip(dm.attn, before):
        for key in ("k", "v"):
            np.testing.assert_array_equal(_gpu_cache(A, key)[2], b4[key][2])
    caches = [{"k": c["k"][:2], "v": c["v"][:2]} for c in _oracle_caches(raw, shape.dtype)]
    ref = oracle.cached_greedy(tokens[:2], w, attn, caches, pos[:2], heads, "exact")
    flagged = (ref["gap"] < HEAD_GAP) | (ref["router_gap"] < ROUTE_GAP)
    gg = host(out["greedy"])[:2]
    np.testing.assert_array_equal(gg[~flagged], ref["argmax"][~flagged])
    n, c, l, nx = oracle.mtp_verify(tokens[:2], gg)
    np.testing.assert_array_equal(host(out["commit"])[:2], c)
    np.testing.assert_array_equal(host(out["commit_len"])[:2], l)
    report("attn_full_cache", pos=pos.tolist(), commit_len=host(out["commit_len"]).tolist())
