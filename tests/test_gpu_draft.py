"""FastMTP draft block on the GPU (moev_draft, moev_spec_step) against the
oracle's draft_block, and the whole speculative step against the verify step
and draft call it is made of."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import dev_f32, dev_i32, host, need_gpu, report

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def model_mod():
    need_gpu()
    from moe_decoder_greedy_amd import model
    return model


def _attach(model_mod, shape):
    w = synth.model_weights(shape)
    dw = synth.draft_weights(shape)
    dm = model_mod.DeviceModel(w)
    dm.attach_draft(dw)
    return dm, w, dw


@pytest.fixture(scope="module")
def tiny(model_mod):
    return _attach(model_mod, synth.TINY)


@pytest.fixture(scope="module")
def decoder_head(model_mod):
    # the draft block reads only the decoder's embedding and LM head
    return _attach(model_mod, replace(synth.DECODER, n_layers=0))


@pytest.fixture(scope="module")
def decoder2(model_mod):
    return _attach(model_mod, replace(synth.DECODER, n_layers=2))


def _inputs(shape, B, seed):
    z0 = synth.draft_states(shape, B, seed)
    t0 = synth.counter_randint(shape.vocab, seed, 77, np.arange(B)).astype(np.int32)
    return z0, t0


def _check_draft(dm, w, dw, B, K, operands, head_gap, z_tol, seed=4):
    """Drafts equal the oracle's on every step reached without a near-tie
    (top-2 head logits closer than head_gap at this or an earlier step), and
    z_K matches on rows with no near-tie at all."""
    shape = dm.shape
    z0, t0 = _inputs(shape, B, seed)
    z_out = torch.empty((B, shape.hidden), dtype=torch.float32, device="cuda")
    got = host(dm.draft(dev_f32(z0), dev_i32(t0), K, z_out=z_out))
    ref = oracle.draft_block(z0, t0, dw, w, K, operands)
    clear = np.cumprod(ref["gap"] > head_gap, axis=1).astype(bool)   # no near-tie up to step j
    for j in range(K):
        np.testing.assert_array_equal(got[clear[:, j], j], ref["drafts"][clear[:, j], j])
    rows = clear[:, -1]
    zg = host(z_out)[rows]
    zr = ref["z"][rows]
    err = np.abs(zg - zr).max(axis=1) / np.abs(zr).max(axis=1)
    report("draft", B=B, K=K, operands=operands, clear=int(rows.sum()), z_rel=float(err.max(initial=0)))
    assert rows.mean() > 0.5
    assert err.max(initial=0.0) <= z_tol
    return got, host(z_out)


def test_draft_tiny_fp32_matches_oracle(tiny):
    dm, w, dw = tiny
    _check_draft(dm, w, dw, B=16, K=3, operands="exact", head_gap=1e-4, z_tol=1e-4)


@pytest.mark.parametrize("B,K", [(32, 3), (1, 1), (37, 2)])
def test_draft_decoder_bf16_matches_oracle(decoder_head, B, K):
    dm, w, dw = decoder_head
    _check_draft(dm, w, dw, B=B, K=K, operands="bf16", head_gap=1e-2, z_tol=2e-2)


def test_draft_rows_do_not_depend_on_the_batch(decoder_head):
    """A row's drafts and z_K are the same bits alone, in a small batch and in
    a large one (fixed slice order in every sum)."""
    dm, w, dw = decoder_head
    shape = dm.shape
    z0, t0 = _inputs(shape, 48, seed=9)
    zf = torch.empty((48, shape.hidden), dtype=torch.float32, device="cuda")
    full = host(dm.draft(dev_f32(z0), dev_i32(t0), 3, z_out=zf))
    for rows in ([5], [0, 17, 40], list(range(8, 40))):
        zs = torch.empty((len(rows), shape.hidden), dtype=torch.float32, device="cuda")
        part = host(dm.draft(dev_f32(z0[rows]), dev_i32(t0[rows]), 3, z_out=zs))
        np.testing.assert_array_equal(part, full[rows])
        assert torch.equal(zs, zf[rows])


def test_draft_recursion_equals_single_steps(decoder_head):
    """K = 3 in one call is three K = 1 calls, each fed the previous (z, draft)."""
    dm, w, dw = decoder_head
    shape = dm.shape
    z0, t0 = _inputs(shape, 24, seed=12)
    zf = torch.empty((24, shape.hidden), dtype=torch.float32, device="cuda")
    full = host(dm.draft(dev_f32(z0), dev_i32(t0), 3, z_out=zf))
    z, t = dev_f32(z0), dev_i32(t0)
    for j in range(3):
        zn = torch.empty_like(z)
        d = dm.draft(z, t, 1, z_out=zn)
        np.testing.assert_array_equal(host(d)[:, 0], full[:, j])
        z, t = zn, d[:, 0].contiguous()
    assert torch.equal(z, zf)


def _tokens(shape, B, K, seed=21):
    return synth.counter_randint(shape.vocab, seed, np.arange(B)[:, None], np.arange(K + 1)[None, :]).astype(np.int32)


def test_spec_step_is_verify_then_draft(decoder2):
    """moev_spec_step = moev_verify_step on the same tokens, then moev_draft from
    the final residual row at each sequence's accepted position and next_last;
    its h_final is the residual stream the prefill path computes for the same
    rows."""
    dm, w, dw = decoder2
    shape = dm.shape
    B, K = 32, 3
    T, H = B * (K + 1), shape.hidden
    toks = _tokens(shape, B, K)
    td = dev_i32(toks)
    hf = torch.empty((T, H), dtype=torch.float32, device="cuda")
    out = dm.spec_step(td, h_final=hf)
    ver = dm.verify_step(td)
    for key in ("greedy", "n_accept", "commit", "commit_len"):
        assert torch.equal(out[key], ver[key]), key
    nxt = host(out["next_tokens"])
    np.testing.assert_array_equal(nxt[:, 0], host(ver["next_last"]))
    rows = torch.arange(B, device="cuda") * (K + 1) + ver["n_accept"].long()
    d = host(dm.draft(hf[rows].contiguous(), ver["next_last"].contiguous(), K))
    np.testing.assert_array_equal(nxt[:, 1:], d)
    h_pref = torch.empty((T, H), dtype=torch.float32, device="cuda")
    dm.prefill(td.reshape(1, T), h_out=h_pref)
    assert torch.equal(h_pref, hf)
    # without a caller buffer for h_final, the same tokens come out
    out2 = dm.spec_step(td)
    assert torch.equal(out2["next_tokens"], out["next_tokens"])


def test_spec_loop_graph_replays_match_eager(decoder2):
    """Three chained speculative steps (each fed the previous next_tokens)
    captured in one HIP graph: every replay equals the eager chain."""
    dm, w, dw = decoder2
    shape = dm.shape
    B, K, n = 8, 3, 3
    start = dev_i32(_tokens(shape, B, K, seed=33))

    def chain(tok, outs):
        for i in range(n):
            dm.spec_step(tok if i == 0 else outs[i - 1]["next_tokens"], out=outs[i])

    eager = [dm.alloc_spec_outputs(B, K) for _ in range(n)]
    chain(start, eager)
    torch.cuda.synchronize()
    want = [host(o["next_tokens"]) for o in eager]
    tok_static = start.clone()
    outs = [dm.alloc_spec_outputs(B, K) for _ in range(n)]
    chain(tok_static, outs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain(tok_static, outs)
    for rep in range(3):
        for o in outs:
            o["next_tokens"].fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i in range(n):
            np.testing.assert_array_equal(host(outs[i]["next_tokens"]), want[i])
        torch.cuda.synchronize()
