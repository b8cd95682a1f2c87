"""Verify steps captured as one HIP graph: several consecutive steps per
graph, replayed several times with eager work and synchronisations between
the replays; every replay must reproduce the eager outputs bit for bit.
Covers the token-set step (decode sizes, the router's atomic mask updates and
the embedding kernel's mask reset inside the graph) and the tiled head."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import dev_i32, host, need_gpu, report

pytestmark = pytest.mark.gpu

KEYS = ("greedy", "n_accept", "commit", "commit_len", "next_last")


@pytest.fixture(scope="module")
def model_mod():
    need_gpu()
    from moe_decoder_greedy_amd import model
    return model


def _check_graph(dm, B, K, n_steps, seed, replays=3, weights=None):
    V = dm.shape.vocab
    rng = np.random.default_rng(seed)
    toks = [dev_i32(rng.integers(0, V, size=(B, K + 1))) for _ in range(n_steps)]
    eager = [{k: host(v) for k, v in dm.verify_step(t).items()} for t in toks]
    if weights is not None:
        # the eager outputs the replays must reproduce are themselves the
        # oracle's (fp32 model: exact operands), off near-ties
        for t, e in zip(toks, eager):
            tk = host(t)
            ref = oracle.verify_step(tk[:, 0], tk[:, 1:], weights, operands="exact")
            ok = (ref["gap"] >= 1e-2) & (ref["router_gap"] >= 1e-3)
            np.testing.assert_array_equal(e["greedy"][ok], ref["greedy"][ok])
            clear = ok.all(axis=1)
            np.testing.assert_array_equal(e["commit"][clear], ref["commit"][clear])
            np.testing.assert_array_equal(e["n_accept"][clear], ref["n_accept"][clear])
    outs = [dm.alloc_outputs(B, K) for _ in range(n_steps)]
    dm.verify_step(toks[0], out=outs[0])          # workspace and code objects ready
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t, o in zip(toks, outs):
            dm.verify_step(t, out=o)
    other = dev_i32(rng.integers(0, V, size=(B, K + 1)))
    for r in range(replays):
        for o in outs:
            for v in o.values():
                v.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for s in range(n_steps):
            for k in KEYS:
                np.testing.assert_array_equal(host(outs[s][k]), eager[s][k], err_msg=f"replay {r} step {s} {k}")
        dm.verify_step(other)                      # eager work between replays
        torch.cuda.synchronize()
    report("graph", B=B, K=K, steps=n_steps, replays=replays)


def test_graph_tiny(model_mod):
    """Tiny fp32 model: replays equal the eager steps bit for bit, and those
    equal the oracle's verify (greedy tokens off near-ties, commits)."""
    w = synth.model_weights(synth.TINY)
    dm = model_mod.DeviceModel(w)
    _check_graph(dm, B=4, K=3, n_steps=4, seed=1, weights=w)


@pytest.mark.parametrize("B,K", [(8, 3), (32, 3)])
def test_graph_decoder(model_mod, B, K, request):
    dm = request.getfixturevalue("decoder_model")
    _check_graph(dm, B=B, K=K, n_steps=3, seed=B)


@pytest.fixture(scope="module")
def decoder_model(model_mod):
    return model_mod.DeviceModel(synth.model_weights(synth.DECODER))
