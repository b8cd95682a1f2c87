"""Python binding of the C ABI in include/moev.h, one function per entry point
and with the same names.  Argument marshalling only: tensors must already be
on the GPU, outputs are allocated with torch when not given, and every step of
the computation runs in libmoev's HIP kernels on torch's current stream.
Importing this module loads libmoev.so and raises if it is missing.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _lib

F32, BF16 = 0, 1
_lib.load()  # fail at import when the HIP library is absent
check = _lib.check


def lib():
    return _lib.load()


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"operand dtype must be bfloat16 or float32, got {t.dtype}")


def torch_dtype(code: int) -> torch.dtype:
    return torch.bfloat16 if code == BF16 else torch.float32


def ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def stream_handle(stream: Optional[torch.cuda.Stream] = None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _empty(shape, dtype, like: torch.Tensor):
    return torch.empty(shape, dtype=dtype, device=like.device)


def pack_weights(w: torch.Tensor, stream=None) -> torch.Tensor:
    """Row-major [G, N, K] (or [N, K]) weights -> the fragment-packed layout
    the GEMM entry points take, returned with shape [G, ceil(N/16)*16, K] (or
    [ceil(N/16)*16, K]); the row count keeps the padded tiles."""
    two_d = w.dim() == 2
    G, N, K = (1, *w.shape) if two_d else w.shape
    n = lib().moev_packed_size(G, N, K, dtype_code(w))
    npad = (N + 15) // 16 * 16
    out = torch.empty((G, npad, K), dtype=w.dtype, device=w.device)
    assert out.numel() * out.element_size() == n
    check("moev_pack_weights", lib().moev_pack_weights(ptr(w), ptr(out), G, N, K, dtype_code(w),
                                                       stream_handle(stream)))
    return out[0] if two_d else out


def moe_embed(tokens: torch.Tensor, emb: torch.Tensor, out: Optional[torch.Tensor] = None,
              stream=None) -> torch.Tensor:
    T = tokens.numel()
    V, H = emb.shape
    out = _empty((T, H), torch.float32, emb) if out is None else out
    check("moe_embed", lib().moe_embed(ptr(tokens), ptr(emb), T, H, V, dtype_code(emb), ptr(out),
                                       stream_handle(stream)))
    return out


def moe_route(h: torch.Tensor, norm_w: Optional[torch.Tensor], eps: float, w_router: torch.Tensor,
              bias: Optional[torch.Tensor], k: int, want_logits: bool = False,
              x_out=None, topk_idx=None, topk_w=None, stream=None):
    T, H = h.shape
    E = w_router.shape[0]
    dt = dtype_code(w_router)
    x_out = _empty((T, H), torch_dtype(dt), h) if x_out is None else x_out
    topk_idx = _empty((T, k), torch.int32, h) if topk_idx is None else topk_idx
    topk_w = _empty((T, k), torch.float32, h) if topk_w is None else topk_w
    logits = _empty((T, E), torch.float32, h) if want_logits else None
    check("moe_route", lib().moe_route(ptr(h), ptr(norm_w), eps, ptr(w_router), ptr(bias), T, H, E,
                                       k, dt, ptr(x_out), ptr(topk_idx), ptr(topk_w), ptr(logits),
                                       stream_handle(stream)))
    return x_out, topk_idx, topk_w, logits


def moe_permute(topk_idx: torch.Tensor, n_routed: int, n_shared: int, offsets=None,
                sorted_src=None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    T, k = topk_idx.shape
    offsets = _empty((n_routed + n_shared + 1,), torch.int32, topk_idx) if offsets is None else offsets
    sorted_src = _empty((T * (k + n_shared),), torch.int32, topk_idx) if sorted_src is None else sorted_src
    check("moe_permute", lib().moe_permute(ptr(topk_idx) if T else None, T, k, n_routed, n_shared,
                                           ptr(offsets), ptr(sorted_src) if T else None,
                                           stream_handle(stream)))
    return offsets, sorted_src


def grouped_ffn_workspace(T: int, I: int, k: int, ns: int, dt: int, device) -> torch.Tensor:
    n = lib().moe_grouped_ffn_workspace_size(T, I, k, ns, dt)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def moe_grouped_ffn(x: torch.Tensor, sorted_src: torch.Tensor, offsets: torch.Tensor,
                    topk_w: torch.Tensor, w_gate: torch.Tensor, w_up: torch.Tensor,
                    w_down: torch.Tensor, n_routed: int, k: int, n_shared: int,
                    y_slots=None, ws=None, stream=None) -> torch.Tensor:
    T, H = x.shape
    G, I, _ = w_gate.shape
    dt = dtype_code(w_gate)
    S = k + n_shared
    y_slots = _empty((T, S, H), torch.float32, x) if y_slots is None else y_slots
    ws = grouped_ffn_workspace(T, I, k, n_shared, dt, x.device) if ws is None else ws
    check("moe_grouped_ffn", lib().moe_grouped_ffn(
        ptr(x), ptr(sorted_src), ptr(offsets), ptr(topk_w), ptr(w_gate), ptr(w_up), ptr(w_down),
        T, H, I, n_routed, k, n_shared, dt, ptr(y_slots), ptr(ws), ws.numel(), stream_handle(stream)))
    return y_slots


def moe_ffn_gate_up(x: torch.Tensor, sorted_src: torch.Tensor, offsets: torch.Tensor,
                    w_gate: torch.Tensor, w_up: torch.Tensor, n_routed: int, k: int, n_shared: int,
                    act=None, stream=None) -> torch.Tensor:
    T, H = x.shape
    G, I, _ = w_gate.shape
    dt = dtype_code(w_gate)
    act = _empty((T * (k + n_shared), I), torch_dtype(dt), x) if act is None else act
    check("moe_ffn_gate_up", lib().moe_ffn_gate_up(
        ptr(x), ptr(sorted_src), ptr(offsets), ptr(w_gate), ptr(w_up), T, H, I, n_routed, k,
        n_shared, dt, ptr(act), stream_handle(stream)))
    return act


def moe_ffn_down(act: torch.Tensor, sorted_src: torch.Tensor, offsets: torch.Tensor,
                 topk_w: torch.Tensor, w_down: torch.Tensor, T: int, n_routed: int, k: int,
                 n_shared: int, y_slots=None, stream=None) -> torch.Tensor:
    G, H, I = w_down.shape
    dt = dtype_code(w_down)
    S = k + n_shared
    y_slots = _empty((T, S, H), torch.float32, act) if y_slots is None else y_slots
    check("moe_ffn_down", lib().moe_ffn_down(
        ptr(act), ptr(sorted_src), ptr(offsets), ptr(topk_w), ptr(w_down), T, H, I, n_routed, k,
        n_shared, dt, ptr(y_slots), stream_handle(stream)))
    return y_slots


def moe_combine(y_slots: torch.Tensor, h_in: Optional[torch.Tensor], out=None, stream=None) -> torch.Tensor:
    T, S, H = y_slots.shape
    out = _empty((T, H), torch.float32, y_slots) if out is None else out
    check("moe_combine", lib().moe_combine(ptr(y_slots), ptr(h_in), T, H, S, ptr(out),
                                           stream_handle(stream)))
    return out


def lmhead_workspace(T: int, H: int, V: int, dt: int, device) -> torch.Tensor:
    n = lib().lmhead_argmax_workspace_size(T, H, V, dt)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def lmhead_argmax(h: torch.Tensor, norm_f: Optional[torch.Tensor], eps: float, w_lm: torch.Tensor,
                  want_max: bool = False, want_logits: bool = False, ws=None, argmax_out=None,
                  vocab: Optional[int] = None, stream=None):
    """``w_lm`` is fragment-packed (``pack_weights``); ``vocab`` is the real
    row count when it is not a multiple of 16."""
    T, H = h.shape
    V = w_lm.shape[0] if vocab is None else vocab
    dt = dtype_code(w_lm)
    argmax_out = _empty((T,), torch.int32, h) if argmax_out is None else argmax_out
    mx = _empty((T,), torch.float32, h) if want_max else None
    logits = _empty((T, V), torch.float32, h) if want_logits else None
    ws = lmhead_workspace(T, H, V, dt, h.device) if ws is None else ws
    check("lmhead_argmax", lib().lmhead_argmax(ptr(h), ptr(norm_f), eps, ptr(w_lm), T, H, V, dt,
                                               ptr(argmax_out), ptr(mx), ptr(logits), ptr(ws),
                                               ws.numel(), stream_handle(stream)))
    return argmax_out, mx, logits


def attn_decode_workspace(B: int, rows: int, H: int, n_heads: int, device) -> torch.Tensor:
    n = lib().moev_attn_decode_workspace_size(B, rows, H, n_heads)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def attn_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, pos: torch.Tensor,
                rows: int, out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    """Causal decode attention of each sequence's ``rows`` verify rows (q fp32
    [B*rows, H]) over its head-major cache (k_cache, v_cache [B, n_heads,
    max_len, D], bf16 or fp32; H = n_heads * D); ``pos`` int32 [B] = cached
    positions before each sequence's first row."""
    B, n_heads, L, D = k_cache.shape
    H = n_heads * D
    assert tuple(v_cache.shape) == tuple(k_cache.shape) and q.shape[-1] == H
    out = _empty((B * rows, H), torch.float32, q) if out is None else out
    ws = attn_decode_workspace(B, rows, H, n_heads, q.device) if ws is None else ws
    check("moev_attn_decode", lib().moev_attn_decode(ptr(q), ptr(k_cache), ptr(v_cache), ptr(pos), B, rows, L,
                                                     H, n_heads, dtype_code(k_cache), ptr(out), ptr(ws),
                                                     ws.numel(), stream_handle(stream)))
    return out


def mtp_verify(tokens: torch.Tensor, greedy: torch.Tensor, stream=None):
    B, K1 = tokens.shape
    n_acc = _empty((B,), torch.int32, tokens)
    commit = _empty((B, K1), torch.int32, tokens)
    clen = _empty((B,), torch.int32, tokens)
    nxt = _empty((B,), torch.int32, tokens)
    check("mtp_verify", lib().mtp_verify(ptr(tokens), ptr(greedy), B, K1 - 1, ptr(n_acc),
                                         ptr(commit), ptr(clen), ptr(nxt), stream_handle(stream)))
    return n_acc, commit, clen, nxt
