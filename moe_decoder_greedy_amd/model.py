"""Device-resident synthetic decoder and the whole-step runner.

``DeviceModel`` uploads a weight dict (as produced by ``synth.model_weights``:
bf16 bit patterns as uint16, or float32) to HBM once, keeps it resident, and
exposes ``verify_step`` -- one call into ``moev_verify_step`` that enqueues the
embedding gather, every MoE layer, the greedy head and the prefix accept on
the current stream.  Python only marshals pointers.
"""
from __future__ import annotations

import ctypes
from typing import Dict, Optional

import numpy as np
import torch

from . import _lib
from .ops import BF16, F32, check, lib, pack_weights, ptr, stream_handle


def to_device(a: Optional[np.ndarray], dtype: str, device) -> Optional[torch.Tensor]:
    """numpy -> torch on ``device``; uint16 arrays are bf16 bit patterns."""
    if a is None:
        return None
    if dtype == "bf16" and a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device)


class DeviceModel:
    """A synthetic MoE decoder resident on one GPU."""

    def __init__(self, weights: dict, device="cuda"):
        shape = weights["shape"]
        self.shape = shape
        self.dtype = weights["dtype"]
        self.device = torch.device(device)
        dt = self.dtype
        self.layers = []
        for d in weights["layers"]:
            L = {key: to_device(d[key], dt if key != "bias" else "f32", self.device)
                 for key in ("norm", "w_router", "bias")}
            for key in ("w_gate", "w_up", "w_down"):   # packed on the GPU, row-major copy freed
                L[key] = pack_weights(to_device(d[key], dt, self.device))
            self.layers.append(L)
        self.emb = to_device(weights["emb"], dt, self.device)
        self.norm_f = to_device(weights["norm_f"], dt, self.device)
        self.w_lm = pack_weights(to_device(weights["w_lm"], dt, self.device))
        n = len(self.layers)
        self._c_layers = (_lib.LayerWeights * max(n, 1))()
        for i, L in enumerate(self.layers):
            self._c_layers[i] = _lib.LayerWeights(ptr(L["norm"]), ptr(L["w_router"]), ptr(L["bias"]),
                                                  ptr(L["w_gate"]), ptr(L["w_up"]), ptr(L["w_down"]))
        self._c_model = _lib.Model(
            shape.hidden, shape.n_routed, shape.inter, shape.top_k, shape.n_shared, shape.vocab, n,
            BF16 if dt == "bf16" else F32, shape.eps, ptr(self.emb), ptr(self.norm_f),
            ptr(self.w_lm), self._c_layers)
        self._ws: Dict[tuple, torch.Tensor] = {}

    @property
    def c_model(self):
        return ctypes.byref(self._c_model)

    def weight_bytes(self) -> int:
        n = self.emb.nbytes + self.norm_f.nbytes + self.w_lm.nbytes
        for L in self.layers:
            n += sum(t.nbytes for t in L.values() if t is not None)
        return n

    def workspace(self, B: int, K: int) -> torch.Tensor:
        key = (B, K)
        if key not in self._ws:
            n = lib().moev_verify_step_workspace_size(self.c_model, B, K)
            self._ws[key] = torch.empty(max(n, 256), dtype=torch.uint8, device=self.device)
        return self._ws[key]

    def alloc_outputs(self, B: int, K: int) -> dict:
        d = self.device
        return {"greedy": torch.empty((B, K + 1), dtype=torch.int32, device=d),
                "n_accept": torch.empty((B,), dtype=torch.int32, device=d),
                "commit": torch.empty((B, K + 1), dtype=torch.int32, device=d),
                "commit_len": torch.empty((B,), dtype=torch.int32, device=d),
                "next_last": torch.empty((B,), dtype=torch.int32, device=d)}

    def verify_step(self, tokens: torch.Tensor, out: Optional[dict] = None, stream=None) -> dict:
        """One verify pass; ``tokens`` int32 [B, K+1] on the GPU."""
        B, K1 = tokens.shape
        K = K1 - 1
        out = self.alloc_outputs(B, K) if out is None else out
        ws = self.workspace(B, K)
        check("moev_verify_step", lib().moev_verify_step(
            self.c_model, ptr(tokens), B, K, ptr(out["greedy"]), ptr(out["n_accept"]),
            ptr(out["commit"]), ptr(out["commit_len"]), ptr(out["next_last"]), ptr(ws), ws.numel(),
            stream_handle(stream)))
        return out

    def verify_step_probed(self, tokens: torch.Tensor, stage: str, before, after,
                           out: Optional[dict] = None, stream=None) -> dict:
        """``verify_step`` that also records the torch.cuda.Events ``before[i]``
        / ``after[i]`` around stage ``stage`` of layer i (or of the head)."""
        B, K1 = tokens.shape
        K = K1 - 1
        out = self.alloc_outputs(B, K) if out is None else out
        ws = self.workspace(B, K)
        for e in list(before) + list(after):
            e.record()   # the runtime creates the event on first record
        n = len(before)
        arr_b = (ctypes.c_void_p * n)(*[e.cuda_event for e in before])
        arr_a = (ctypes.c_void_p * n)(*[e.cuda_event for e in after])
        probe = _lib.StepProbe(_lib.STAGES[stage], n, arr_b, arr_a)
        check("moev_verify_step_probed", lib().moev_verify_step_probed(
            self.c_model, ptr(tokens), B, K, ptr(out["greedy"]), ptr(out["n_accept"]),
            ptr(out["commit"]), ptr(out["commit_len"]), ptr(out["next_last"]), ptr(ws), ws.numel(),
            ctypes.byref(probe), stream_handle(stream)))
        return out

    def prefill_workspace(self, n_seq: int, seq_len: int) -> torch.Tensor:
        key = ("prefill", n_seq, seq_len)
        if key not in self._ws:
            n = lib().moev_prefill_workspace_size(self.c_model, n_seq, seq_len)
            self._ws[key] = torch.empty(max(n, 256), dtype=torch.uint8, device=self.device)
        return self._ws[key]

    def prefill(self, tokens: torch.Tensor, next_token: Optional[torch.Tensor] = None,
                h_out: Optional[torch.Tensor] = None, probe=None, stream=None) -> torch.Tensor:
        """``tokens`` int32 [n_seq, seq_len] on the GPU through every layer; the
        greedy token after each sequence's last prompt token.  ``h_out`` (fp32
        [n_seq*seq_len, H], optional) receives the final residual stream.
        ``probe`` = (stage, before_events, after_events) records HIP events
        around that stage's launches."""
        n_seq, seq_len = tokens.shape
        nt = torch.empty((n_seq,), dtype=torch.int32, device=self.device) if next_token is None else next_token
        ws = self.prefill_workspace(n_seq, seq_len)
        if probe is None:
            check("moev_prefill", lib().moev_prefill(
                self.c_model, ptr(tokens), n_seq, seq_len, ptr(nt), ptr(h_out), ptr(ws), ws.numel(),
                stream_handle(stream)))
        else:
            stage, before, after = probe
            for e in list(before) + list(after):
                e.record()
            n = len(before)
            arr_b = (ctypes.c_void_p * n)(*[e.cuda_event for e in before])
            arr_a = (ctypes.c_void_p * n)(*[e.cuda_event for e in after])
            pr = _lib.StepProbe(_lib.STAGES[stage], n, arr_b, arr_a)
            check("moev_prefill_probed", lib().moev_prefill_probed(
                self.c_model, ptr(tokens), n_seq, seq_len, ptr(nt), ptr(h_out), ptr(ws), ws.numel(),
                ctypes.byref(pr), stream_handle(stream)))
        return nt

    # ------------------------------------------------------------ draft block
    def attach_draft(self, draft: dict) -> None:
        """Upload FastMTP draft-block weights (as ``synth.draft_weights``)."""
        dt = self.dtype
        D = {key: to_device(draft[key], dt, self.device)
             for key in ("norm_z", "norm_e", "norm_ffn", "norm_out")}
        for key in ("w_proj", "w_gate", "w_up", "w_down"):
            D[key] = pack_weights(to_device(draft[key], dt, self.device))
        self.draft_w = D
        self._c_draft = _lib.DraftWeights(ptr(D["norm_z"]), ptr(D["norm_e"]), ptr(D["w_proj"]),
                                          ptr(D["norm_ffn"]), ptr(D["w_gate"]), ptr(D["w_up"]),
                                          ptr(D["w_down"]), ptr(D["norm_out"]), int(draft["n_slices"]))

    @property
    def c_draft(self):
        return ctypes.byref(self._c_draft)

    def draft_bytes(self) -> int:
        return sum(t.nbytes for t in self.draft_w.values())

    def _ws_named(self, key, n: int) -> torch.Tensor:
        if key not in self._ws:
            self._ws[key] = torch.empty(max(n, 256), dtype=torch.uint8, device=self.device)
        return self._ws[key]

    def draft(self, z0: torch.Tensor, t0: torch.Tensor, K: int, drafts: Optional[torch.Tensor] = None,
              z_out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        """K draft tokens per row from hidden states ``z0`` (fp32 [B, H]) and
        tokens ``t0`` (int32 [B]); ``z_out`` (optional) receives z_K."""
        B = z0.shape[0]
        d = torch.empty((B, K), dtype=torch.int32, device=self.device) if drafts is None else drafts
        ws = self._ws_named(("draft", B), lib().moev_draft_workspace_size(self.c_model, self.c_draft, B))
        check("moev_draft", lib().moev_draft(self.c_model, self.c_draft, ptr(z0), ptr(t0), B, K, ptr(d),
                                             ptr(z_out), ptr(ws), ws.numel(), stream_handle(stream)))
        return d

    def alloc_spec_outputs(self, B: int, K: int) -> dict:
        out = self.alloc_outputs(B, K)
        del out["next_last"]
        out["next_tokens"] = torch.empty((B, K + 1), dtype=torch.int32, device=self.device)
        return out

    def spec_step(self, tokens: torch.Tensor, out: Optional[dict] = None,
                  h_final: Optional[torch.Tensor] = None, stream=None) -> dict:
        """Verify ``tokens`` (int32 [B, K+1]) and draft the next pass's tokens
        (``out["next_tokens"]``) in one call into ``moev_spec_step``."""
        B, K1 = tokens.shape
        K = K1 - 1
        out = self.alloc_spec_outputs(B, K) if out is None else out
        ws = self._ws_named(("spec", B, K),
                            lib().moev_spec_step_workspace_size(self.c_model, self.c_draft, B, K))
        check("moev_spec_step", lib().moev_spec_step(
            self.c_model, self.c_draft, ptr(tokens), B, K, ptr(out["greedy"]), ptr(out["n_accept"]),
            ptr(out["commit"]), ptr(out["commit_len"]), ptr(out["next_tokens"]), ptr(h_final), ptr(ws),
            ws.numel(), stream_handle(stream)))
        return out

    # ------------------------------------------------------ attention sublayer
    def attach_attention(self, attn: list, n_heads: int, batch: int, max_len: int) -> None:
        """Upload per-layer attention projections (as ``synth.attention_weights``:
        W_q, W_k, W_v, W_o [H, H]; the first three are stacked into one packed
        [3H, H] matrix) and allocate zeroed key/value caches per layer in the
        model dtype, head-major: [batch, n_heads, max_len, H / n_heads]."""
        dt = self.dtype
        H = self.shape.hidden
        D = H // n_heads
        cdt = torch.bfloat16 if dt == "bf16" else torch.float32
        self.attn = []
        for a in attn:
            qkv = np.concatenate([a["w_q"], a["w_k"], a["w_v"]], axis=0)
            self.attn.append({"w_qkv": pack_weights(to_device(qkv, dt, self.device)),
                              "w_o": pack_weights(to_device(a["w_o"], dt, self.device)),
                              "k": torch.zeros((batch, n_heads, max_len, D), dtype=cdt, device=self.device),
                              "v": torch.zeros((batch, n_heads, max_len, D), dtype=cdt, device=self.device)})
        self._c_attn_layers = (_lib.AttnLayer * max(len(self.attn), 1))()
        for i, A in enumerate(self.attn):
            self._c_attn_layers[i] = _lib.AttnLayer(ptr(A["w_qkv"]), ptr(A["w_o"]), ptr(A["k"]), ptr(A["v"]))
        self._c_attn = _lib.Attn(n_heads, max_len, self._c_attn_layers)
        self.attn_batch = batch

    @property
    def c_attn(self):
        return ctypes.byref(self._c_attn)

    def verify_step_attn(self, tokens: torch.Tensor, pos: torch.Tensor, out: Optional[dict] = None,
                         stream=None) -> dict:
        """One verify pass with attention (``moev_verify_step_attn``): tokens
        int32 [B, K+1] at positions pos[b] .. pos[b]+K of the caches; ``pos``
        (int32 [B] on the GPU) advances by commit_len."""
        B, K1 = tokens.shape
        K = K1 - 1
        assert B == self.attn_batch, "the caches were allocated for another batch"
        out = self.alloc_outputs(B, K) if out is None else out
        ws = self._ws_named(("attn", B, K),
                            lib().moev_verify_step_attn_workspace_size(self.c_model, self.c_attn, B, K))
        check("moev_verify_step_attn", lib().moev_verify_step_attn(
            self.c_model, self.c_attn, ptr(tokens), B, K, ptr(pos), ptr(out["greedy"]), ptr(out["n_accept"]),
            ptr(out["commit"]), ptr(out["commit_len"]), ptr(out["next_last"]), ptr(ws), ws.numel(),
            stream_handle(stream)))
        return out

    def greedy(self, tokens: torch.Tensor) -> torch.Tensor:
        """Greedy successor of every token (a K = 0 step)."""
        return self.verify_step(tokens.reshape(-1, 1).to(torch.int32).contiguous())["greedy"].reshape(-1)
