"""Decode attention on the GPU (moev_attn_decode) against the oracle's
attn_decode, on seeded caches."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import dev_f32, dev_i32, host, max_abs, need_gpu, report

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    need_gpu()
    from moe_decoder_greedy_amd import ops as _ops
    return _ops


def _dev_cache(a, heads):
    """The oracle's [B, L, H] caches as the kernel's head-major [B, heads, L, D]."""
    out = []
    for key in ("k_cache", "v_cache"):
        c = a[key]
        B, L, H = c.shape
        t = torch.from_numpy(c.view(np.int16)).view(torch.bfloat16) if a["dtype"] == "bf16" else torch.from_numpy(c)
        out.append(t.view(B, L, heads, H // heads).permute(0, 2, 1, 3).contiguous().cuda())
    return tuple(out)


@pytest.mark.parametrize("B,rows,H,heads,L,prefix,bf16", [
    (8, 4, 1280, 10, 1400, (1100, 1300), True),    # decoder width, page-length prefixes, K = 3
    (5, 1, 256, 4, 300, (0, 299), False),          # greedy rows, fp32 cache, 64-wide heads
    (3, 16, 512, 2, 40, (0, 0), True),             # 256-wide heads, no prefix: row 0 sees only itself
    (4, 2, 256, 4, 90, (88, 88), True),            # 64-wide bf16 heads, the last positions of the cache
])
def test_attn_decode_matches_oracle(ops, B, rows, H, heads, L, prefix, bf16):
    a = synth.attention_inputs(B, rows, H, L, prefix, seed=11 + B, bf16=bf16)
    report("attn_decode", B=B, rows=rows, H=H, heads=heads, L=L, pos=a["pos"].tolist())
    kc, vc = _dev_cache(a, heads)
    out = host(ops.attn_decode(dev_f32(a["q"]), kc, vc, dev_i32(a["pos"]), rows))
    want = oracle.attn_decode(a["q"], a["k_cache"], a["v_cache"], a["pos"], rows, heads, a["dtype"])
    err = max_abs(out, want)
    report("attn_decode", err=err, scale=float(np.abs(want).max()))
    assert err < 2e-5


def test_attn_decode_rows_do_not_depend_on_the_batch(ops):
    """A sequence's outputs are the same bits alone and in a batch."""
    B, rows, H, heads, L = 6, 4, 1280, 10, 600
    a = synth.attention_inputs(B, rows, H, L, (100, 590), seed=21)
    kc, vc = _dev_cache(a, heads)
    q, pos = dev_f32(a["q"]), dev_i32(a["pos"])
    full = host(ops.attn_decode(q, kc, vc, pos, rows))
    for b in (0, 3, 5):
        one = host(ops.attn_decode(q[b * rows:(b + 1) * rows].contiguous(), kc[b:b + 1].contiguous(),
                                   vc[b:b + 1].contiguous(), pos[b:b + 1].contiguous(), rows))
        np.testing.assert_array_equal(one.view(np.uint32), full[b * rows:(b + 1) * rows].view(np.uint32))



@pytest.mark.parametrize("rows", [2, 4, 5, 8, 16])
def test_attn_row_is_the_same_in_a_one_row_pass(ops, rows):
    """Row i of a multi-row pass is the same bits as a one-row pass at
    position pos[b] + i: greedy decoding and a verify pass see the same
    attention.  Row counts cover every instantiation a verify pass of up to
    16 rows selects (2, 4, 8 and 16 rows; 5 runs the 8-row one part full)."""
    B, H, heads, L = 3, 1280, 10, 900
    a = synth.attention_inputs(B, rows, H, L, (100, 880), seed=31)
    kc, vc = _dev_cache(a, heads)
    q, pos = dev_f32(a["q"]), dev_i32(a["pos"])
    full = host(ops.attn_decode(q, kc, vc, pos, rows)).reshape(B, rows, H)
    for i in range(rows):
        qi = q.view(B, rows, H)[:, i].contiguous()
        one = host(ops.attn_decode(qi, kc, vc, (pos + i).contiguous(), 1))
        np.testing.assert_array_equal(one.view(np.uint32), np.ascontiguousarray(full[:, i]).view(np.uint32))
