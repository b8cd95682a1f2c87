"""The allocation-free grouped FFN (moe_grouped_ffn_noalloc, for callers that
cannot allocate) against moe_grouped_ffn with a caller workspace, through the
C ABI: two calls in a row on one device, the second smaller, each bit for bit
equal to the workspace entry point's result on the same inputs."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import dev_f32, dev_i32, host, need_gpu, report

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    need_gpu()
    from moe_decoder_greedy_amd import ops as _ops
    return _ops


def _inputs(ops, L, shape, T, seed):
    """bf16 operand rows, a seeded top-k per token (distinct experts, weights
    summing to 1) and the sorted pair order from moe_permute."""
    rng = np.random.default_rng(seed)
    x = torch.from_numpy(synth.hidden_states(shape, T, seed=seed)).cuda().to(torch.bfloat16)
    idx = np.stack([rng.permutation(shape.n_routed)[:shape.top_k] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, shape.top_k)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    off, src = ops.moe_permute(dev_i32(idx), shape.n_routed, shape.n_shared)
    return x, off, src, dev_f32(w)


def test_noalloc_grouped_ffn_matches_workspace_entry_point(ops):
    from moe_decoder_greedy_amd import _lib
    shape = synth.DECODER
    wts = synth.model_weights(shape, layers=[0], head=False)["layers"][0]
    to = lambda a: ops.pack_weights(torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda())
    wg, wu, wd = to(wts["w_gate"]), to(wts["w_up"]), to(wts["w_down"])
    lib = _lib.load()
    S, H, I = shape.top_k + shape.n_shared, shape.hidden, shape.inter
    # 300 tokens takes the tiled GEMMs, 77 the streaming ones
    for T in (300, 77):
        report("noalloc", T=T)
        x, off, src, w = _inputs(ops, wts, shape, T, seed=T)
        ref = ops.moe_grouped_ffn(x, src, off, w, wg, wu, wd, shape.n_routed, shape.top_k, shape.n_shared)
        y = torch.full((T, S, H), float("nan"), dtype=torch.float32, device="cuda")
        st = lib.moe_grouped_ffn_noalloc(ops.ptr(x), ops.ptr(src), ops.ptr(off), ops.ptr(w), ops.ptr(wg),
                                         ops.ptr(wu), ops.ptr(wd), T, H, I, shape.n_routed, shape.top_k,
                                         shape.n_shared, ops.BF16, ops.ptr(y), ops.stream_handle(None))
        assert st == 0, lib.moev_last_error().decode()
        torch.cuda.synchronize()
        a, b = host(y), host(ref)
        assert np.isfinite(a).all()
        np.testing.assert_array_equal(a.view(np.uint64), b.view(np.uint64))
        report("noalloc", T=T, equal=True, scale=float(np.abs(b).max()))
