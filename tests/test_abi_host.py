"""The C-ABI library on the host: it loads, exports every entry point that
include/moev.h declares, and rejects bad arguments before touching the GPU.
No kernel is launched here (CPU only)."""
import ctypes
import os
import re

import pytest

from moe_decoder_greedy_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moev.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
BF16, F32 = 1, 0
FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails validation


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                                 text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libmoev.so not built: run python -m moe_decoder_greedy_amd.build")
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert "moe_route" in names and "mtp_verify" in names and "moev_verify_step" in names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES)


def test_status_strings_and_version(lib):
    assert lib.moev_status_string(0) == b"ok"
    assert lib.moev_status_string(3) == b"workspace missing or too small"
    assert lib.moev_version() == 100


def _err(lib):
    return lib.moev_last_error().decode()


def test_route_validation(lib):
    s = None
    args = dict(h=FAKE, norm=None, eps=1e-6, wr=FAKE, bias=None, T=4, H=1280, E=64, k=6, dt=BF16,
                x=FAKE, idx=FAKE, w=FAKE, logits=None)

    def call(**kw):
        a = dict(args, **kw)
        return lib.moe_route(a["h"], a["norm"], a["eps"], a["wr"], a["bias"], a["T"], a["H"], a["E"],
                             a["k"], a["dt"], a["x"], a["idx"], a["w"], a["logits"], s)
    assert call(h=None) == INVALID and "h must not be NULL" in _err(lib)
    assert call(x=FAKE + 4) == INVALID and "aligned" in _err(lib)
    assert call(k=7, E=6) == UNSUPPORTED
    assert call(E=65) == UNSUPPORTED
    assert call(H=1000) == UNSUPPORTED
    assert call(dt=7) == UNSUPPORTED
    assert call(T=-1) == INVALID
    assert call(T=0, h=None, x=None) == OK          # empty batch: nothing enqueued


def test_permute_validation(lib):
    assert lib.moe_permute(FAKE, 8, 2, 8, 9, FAKE, FAKE, None) == UNSUPPORTED   # ns > 8
    assert lib.moe_permute(FAKE, 8, 0, 8, 1, FAKE, FAKE, None) == UNSUPPORTED   # k = 0
    assert lib.moe_permute(None, 8, 2, 8, 1, FAKE, FAKE, None) == INVALID
    assert lib.moe_permute(FAKE, 8, 2, 8, 1, None, FAKE, None) == INVALID


def test_grouped_ffn_validation_and_workspace(lib):
    need = lib.moe_grouped_ffn_workspace_size(128, 896, 6, 2, BF16)
    assert need >= 128 * 8 * 896 * 2
    call = lambda ws, n, I=896: lib.moe_grouped_ffn(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 128,
                                                    1280, I, 64, 6, 2, BF16, FAKE, ws, n, None)
    assert call(FAKE, need - 1) == WORKSPACE and "needs" in _err(lib)
    assert call(None, need) == WORKSPACE
    assert call(FAKE, need, I=900) == UNSUPPORTED


def test_lmhead_validation(lib):
    need = lib.lmhead_argmax_workspace_size(128, 1280, 129280, BF16)
    assert need > 128 * 1280 * 2
    f = lambda **kw: lib.lmhead_argmax(kw.get("h", FAKE), None, 1e-6, FAKE, 128, 1280, kw.get("V", 129280),
                                       BF16, kw.get("out", FAKE), None, None, FAKE, kw.get("n", need), None)
    assert f(n=need - 1) == WORKSPACE
    assert f(out=None) == INVALID
    assert f(V=0) == INVALID


def test_verify_and_combine_validation(lib):
    assert lib.mtp_verify(FAKE, FAKE, 4, -1, FAKE, FAKE, None, None, None) == INVALID
    assert lib.mtp_verify(FAKE, FAKE, 4, 65, FAKE, FAKE, None, None, None) == UNSUPPORTED
    assert lib.mtp_verify(None, None, 0, 3, None, None, None, None, None) == OK
    assert lib.moe_combine(FAKE, None, 4, 6, 8, FAKE, None) == UNSUPPORTED   # H % 4
    assert lib.moe_combine(None, None, 4, 8, 8, FAKE, None) == INVALID


def test_step_validation(lib):
    layers = (_lib.LayerWeights * 1)(_lib.LayerWeights(None, FAKE, None, FAKE, FAKE, None))
    m = _lib.Model(1280, 64, 896, 6, 2, 129280, 1, BF16, 1e-6, FAKE, None, FAKE, layers)
    ws = lib.moev_verify_step_workspace_size(ctypes.byref(m), 32, 3)
    assert ws > 0
    st = lib.moev_verify_step(ctypes.byref(m), FAKE, 32, 3, FAKE, FAKE, FAKE, None, None, FAKE, ws, None)
    assert st == INVALID and "layer 0" in _err(lib) and "w_down" in _err(lib)
    m.n_layers = 0
    assert lib.moev_verify_step(ctypes.byref(m), FAKE, 32, 3, FAKE, FAKE, FAKE, None, None, FAKE,
                                ws - 1, None) == WORKSPACE
    m.top_k = 65
    assert lib.moev_verify_step(ctypes.byref(m), FAKE, 32, 3, FAKE, FAKE, FAKE, None, None, FAKE,
                                ws, None) == UNSUPPORTED


def test_noalloc_grouped_ffn_rejects_oversize(lib):
    """The allocation-free grouped FFN refuses, before any HIP call, a batch
    whose activations do not fit its static scratch (16 MiB: the decoder's
    I = 896 with k + ns = 8 in bf16 fits up to T = 1170), and passes its
    other checks on to moe_grouped_ffn's (T = 0 is a no-op)."""
    args = lambda T: (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, T, 1280, 896, 64, 6, 2, BF16, FAKE, None)
    assert lib.moe_grouped_ffn_noalloc(*args(1171)) == WORKSPACE
    assert "1171" in _err(lib) and "16777216" in _err(lib)
    assert lib.moe_grouped_ffn_noalloc(*args(0)) == OK
    bad = list(args(16))
    bad[8] = 100                     # H not a multiple of 64
    assert lib.moe_grouped_ffn_noalloc(*bad) == UNSUPPORTED
    bad = list(args(16))
    bad[14] = None                   # y_slots
    assert lib.moe_grouped_ffn_noalloc(*bad) == INVALID


def test_prefill_validation(lib):
    layers = (_lib.LayerWeights * 1)(_lib.LayerWeights(None, FAKE, None, FAKE, FAKE, None))
    m = _lib.Model(1280, 64, 896, 6, 2, 129280, 1, BF16, 1e-6, FAKE, None, FAKE, layers)
    ws = lib.moev_prefill_workspace_size(ctypes.byref(m), 8, 1220)
    # at least the layer loop's activations for 9760 rows
    assert ws > 9760 * 1280 * 4 + 9760 * 8 * 1280 * 4
    assert lib.moev_prefill_workspace_size(ctypes.byref(m), 8, 0) == 0
    call = lambda n_seq=8, seq_len=1220, nt=FAKE, n=ws: lib.moev_prefill(
        ctypes.byref(m), FAKE, n_seq, seq_len, nt, None, FAKE, n, None)
    assert call() == INVALID and "w_down" in _err(lib)     # the layer's missing down weights
    m.n_layers = 0
    assert call(seq_len=0) == INVALID
    assert call(nt=None) == INVALID
    assert call(n=ws - 1) == WORKSPACE
    assert call(n_seq=0) == OK                              # nothing to do
    m.hidden = 1300
    assert call() == UNSUPPORTED


def test_draft_and_spec_step_validation(lib):
    layers = (_lib.LayerWeights * 1)(_lib.LayerWeights(None, FAKE, None, FAKE, FAKE, FAKE))
    m = _lib.Model(1280, 64, 896, 6, 2, 129280, 1, BF16, 1e-6, FAKE, None, FAKE, layers)
    d = _lib.DraftWeights(None, None, FAKE, None, FAKE, FAKE, FAKE, None, 8)
    ws = lib.moev_draft_workspace_size(ctypes.byref(m), ctypes.byref(d), 32)
    # at least the dense FFN's activations and slot outputs for 32 rows
    assert ws > 8 * 32 * 896 * 2 + 32 * 8 * 1280 * 4
    spec = lib.moev_spec_step_workspace_size(ctypes.byref(m), ctypes.byref(d), 32, 3)
    assert spec > ws + lib.moev_verify_step_workspace_size(ctypes.byref(m), 32, 3)
    assert lib.moev_draft_workspace_size(ctypes.byref(m), None, 32) == 0
    draft = lambda dw=ctypes.byref(d), B=32, K=3, z0=FAKE, out=FAKE, n=ws: lib.moev_draft(
        ctypes.byref(m), dw, z0, FAKE, B, K, out, None, FAKE, n, None)
    assert draft(dw=None) == INVALID
    assert draft(K=-1) == INVALID
    assert draft(z0=None) == INVALID
    assert draft(out=None) == INVALID
    assert draft(n=ws - 1) == WORKSPACE
    assert draft(B=0) == OK and draft(K=0) == OK         # nothing to do
    d.w_up = None
    assert draft() == INVALID and "w_up" in _err(lib)
    d.w_up = FAKE
    d.n_slices = 17
    assert draft() == UNSUPPORTED
    d.n_slices = 8
    step = lambda K=3, nt=FAKE, n=spec: lib.moev_spec_step(
        ctypes.byref(m), ctypes.byref(d), FAKE, 32, K, FAKE, FAKE, FAKE, None, nt, None, FAKE, n, None)
    assert step(K=0) == INVALID                         # a speculative step drafts at least one token
    assert step(nt=None) == INVALID
    assert step(n=spec - 1) == WORKSPACE
    m.hidden = 1300
    assert step() == UNSUPPORTED


def test_attn_decode_validation(lib):
    s = None

    need = lib.moev_attn_decode_workspace_size(2, 4, 1280, 10)
    assert need == 2 * 4 * 3 * (1280 + 2 * 10) * 4   # 3 splits x (weighted values + max, sum) per row

    def call(q=FAKE, k=FAKE, v=FAKE, pos=FAKE, B=2, rows=4, L=64, H=1280, heads=10, dt=BF16, out=FAKE,
             ws=FAKE, n=need):
        return lib.moev_attn_decode(q, k, v, pos, B, rows, L, H, heads, dt, out, ws, n, s)

    assert call(rows=0) == UNSUPPORTED and "rows" in _err(lib)
    assert call(rows=17) == UNSUPPORTED
    assert call(H=1280, heads=3) == UNSUPPORTED
    assert call(H=1280, heads=16) == UNSUPPORTED and "head width" in _err(lib)  # 80-wide heads
    assert call(H=1280, heads=40) == UNSUPPORTED                                  # 32-wide heads
    assert call(L=3) == INVALID and "max_len" in _err(lib)
    assert call(dt=7) == UNSUPPORTED
    assert call(B=-1) == INVALID
    assert call(B=0, q=None, k=None, v=None, pos=None, out=None) == OK
    assert call(q=None) == INVALID and "q" in _err(lib)
    assert call(pos=FAKE + 2) == INVALID and "aligned" in _err(lib)
    assert call(ws=None) == WORKSPACE
    assert call(n=need - 1) == WORKSPACE and "needs" in _err(lib)


def test_verify_step_attn_validation(lib):
    layers = (_lib.LayerWeights * 1)(_lib.LayerWeights(None, FAKE, None, FAKE, FAKE, FAKE))
    m = _lib.Model(1280, 64, 896, 6, 2, 129280, 1, BF16, 1e-6, FAKE, None, FAKE, layers)
    al = (_lib.AttnLayer * 1)(_lib.AttnLayer(FAKE, FAKE, FAKE, None))
    a = _lib.Attn(10, 2400, al)
    ws = lib.moev_verify_step_attn_workspace_size(ctypes.byref(m), ctypes.byref(a), 32, 3)
    assert ws > lib.moev_verify_step_workspace_size(ctypes.byref(m), 32, 3)
    assert lib.moev_verify_step_attn_workspace_size(ctypes.byref(m), None, 32, 3) == 0

    def step(attn=ctypes.byref(a), B=32, K=3, pos=FAKE, n=ws):
        return lib.moev_verify_step_attn(ctypes.byref(m), attn, FAKE, B, K, pos, FAKE, FAKE, FAKE, FAKE,
                                         FAKE, FAKE, n, None)

    assert step() == INVALID and "attention layer 0" in _err(lib) and "v_cache" in _err(lib)
    assert step(attn=None) == INVALID
    assert step(K=16) == UNSUPPORTED and "16 rows" in _err(lib)
    assert step(B=200, K=3) == UNSUPPORTED and "exceeds 512" in _err(lib)
    a.n_heads = 16                                    # 80-wide heads
    assert step() == UNSUPPORTED and "head width" in _err(lib)
    a.n_heads, a.max_len = 10, 3
    assert step() == INVALID and "max_len" in _err(lib)
    a.max_len = 2400
    al[0].v_cache = FAKE
    assert step(pos=None) == INVALID and "pos" in _err(lib)
    assert step(n=ws - 1) == WORKSPACE
    assert step(B=0) == OK
