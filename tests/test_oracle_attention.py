"""Pins of the oracle's decode attention (oracle.attn_decode) against a
library routine and closed forms, on the CPU."""
import numpy as np
import pytest
import torch

import oracle
import synth


def _case(B, rows, H, L, prefix, seed, bf16=False):
    return synth.attention_inputs(B, rows, H, L, prefix, seed=seed, bf16=bf16)


@pytest.mark.parametrize("B,rows,H,heads,L,prefix", [(3, 4, 64, 2, 40, (0, 30)), (2, 1, 32, 4, 9, (0, 8)),
                                                     (1, 5, 48, 3, 70, (60, 65))])
def test_attn_decode_matches_torch_sdpa(B, rows, H, heads, L, prefix):
    """The oracle equals torch's scaled_dot_product_attention (float64) with a
    mask that lets row i of sequence b see positions 0..pos[b]+i."""
    a = _case(B, rows, H, L, prefix, seed=B * 100 + rows)
    got = oracle.attn_decode(a["q"], a["k_cache"], a["v_cache"], a["pos"], rows, heads, a["dtype"])
    d = H // heads
    for b in range(B):
        q = torch.from_numpy(a["q"][b * rows:(b + 1) * rows].astype(np.float64)).view(rows, heads, d).transpose(0, 1)
        k = torch.from_numpy(a["k_cache"][b].astype(np.float64)).view(L, heads, d).transpose(0, 1)
        v = torch.from_numpy(a["v_cache"][b].astype(np.float64)).view(L, heads, d).transpose(0, 1)
        mask = torch.arange(L)[None, :] <= (int(a["pos"][b]) + torch.arange(rows))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(q.contiguous(), k.contiguous(), v.contiguous(),
                                                               attn_mask=mask)
        ref = ref.transpose(0, 1).reshape(rows, H).numpy()
        np.testing.assert_allclose(got[b * rows:(b + 1) * rows], ref, rtol=1e-10, atol=1e-12)


def test_attn_single_key_returns_its_value():
    """With no prefix, the first verify row sees only its own key: the output
    is its own value row exactly (softmax of one score is 1)."""
    a = _case(2, 3, 32, 8, (0, 0), seed=3)
    got = oracle.attn_decode(a["q"], a["k_cache"], a["v_cache"], a["pos"], 3, 4, a["dtype"])
    for b in range(2):
        np.testing.assert_array_equal(got[b * 3], a["v_cache"][b, 0].astype(np.float64))


def test_attn_zero_query_averages_the_visible_values():
    """q = 0 gives equal scores: the output is the mean of the values at
    positions 0..pos[b]+i."""
    a = _case(2, 4, 32, 30, (3, 20), seed=4)
    q = np.zeros_like(a["q"])
    got = oracle.attn_decode(q, a["k_cache"], a["v_cache"], a["pos"], 4, 2, a["dtype"])
    for b in range(2):
        for i in range(4):
            n = int(a["pos"][b]) + i + 1
            np.testing.assert_allclose(got[b * 4 + i], a["v_cache"][b, :n].astype(np.float64).mean(0), rtol=1e-12)


def test_attn_is_causal():
    """Changing keys and values at positions after pos[b]+i leaves row i's
    output unchanged, and changing one it can see changes it."""
    a = _case(1, 4, 32, 30, (10, 10), seed=5)
    base = oracle.attn_decode(a["q"], a["k_cache"], a["v_cache"], a["pos"], 4, 2, a["dtype"])
    k2, v2 = a["k_cache"].copy(), a["v_cache"].copy()
    p = int(a["pos"][0])
    k2[0, p + 2:] += 1.0
    v2[0, p + 2:] -= 3.0
    moved = oracle.attn_decode(a["q"], k2, v2, a["pos"], 4, 2, a["dtype"])
    np.testing.assert_array_equal(moved[:2], base[:2])
    assert np.abs(moved[2:] - base[2:]).max() > 1e-3
