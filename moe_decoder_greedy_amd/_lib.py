"""ctypes loader for libmoev.so, the C-ABI HIP library.

Fails loudly: if the shared library is missing or does not export a symbol
the header declares, importing the binding raises.  There is no fallback
path.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoev.so")

c_int, c_float, c_size_t, c_void_p = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p


class LayerWeights(ctypes.Structure):
    _fields_ = [("norm", c_void_p), ("w_router", c_void_p), ("bias", c_void_p),
                ("w_gate", c_void_p), ("w_up", c_void_p), ("w_down", c_void_p)]


class Model(ctypes.Structure):
    _fields_ = [("hidden", c_int), ("n_routed", c_int), ("inter", c_int), ("top_k", c_int),
                ("n_shared", c_int), ("vocab", c_int), ("n_layers", c_int), ("dtype", c_int),
                ("eps", c_float), ("emb", c_void_p), ("norm_f", c_void_p), ("w_lm", c_void_p),
                ("layers", ctypes.POINTER(LayerWeights))]


class StepProbe(ctypes.Structure):
    _fields_ = [("stage", c_int), ("n", c_int), ("before", ctypes.POINTER(c_void_p)),
                ("after", ctypes.POINTER(c_void_p))]


class DraftWeights(ctypes.Structure):
    _fields_ = [("norm_z", c_void_p), ("norm_e", c_void_p), ("w_proj", c_void_p),
                ("norm_ffn", c_void_p), ("w_gate", c_void_p), ("w_up", c_void_p),
                ("w_down", c_void_p), ("norm_out", c_void_p), ("n_slices", c_int)]


STAGES = {"route": 0, "permute": 1, "gate_up": 2, "down": 3, "combine": 4, "head": 5}

class AttnLayer(ctypes.Structure):
    _fields_ = [("w_qkv", c_void_p), ("w_o", c_void_p), ("k_cache", c_void_p), ("v_cache", c_void_p)]


class Attn(ctypes.Structure):
    _fields_ = [("n_heads", c_int), ("max_len", c_int), ("layers", ctypes.POINTER(AttnLayer))]


# name -> (restype, argtypes); mirrors include/moev.h
SIGNATURES = {
    "moev_status_string": (ctypes.c_char_p, [c_int]),
    "moev_last_error": (ctypes.c_char_p, []),
    "moev_version": (c_int, []),
    "moev_packed_size": (c_size_t, [c_int, c_int, c_int, c_int]),
    "moev_pack_weights": (c_int, [c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_void_p]),
    "moe_embed": (c_int, [c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_void_p, c_void_p]),
    "moe_route": (c_int, [c_void_p, c_void_p, c_float, c_void_p, c_void_p, c_int, c_int, c_int,
                          c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "moe_permute": (c_int, [c_void_p, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p]),
    "moe_grouped_ffn_workspace_size": (c_size_t, [c_int, c_int, c_int, c_int, c_int]),
    "moe_grouped_ffn": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                c_void_p, c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                c_void_p, c_void_p, c_size_t, c_void_p]),
    "moe_grouped_ffn_noalloc": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                        c_void_p, c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                        c_void_p, c_void_p]),
    "moe_ffn_gate_up": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int,
                                c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p]),
    "moe_ffn_down": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int, c_int,
                             c_int, c_int, c_int, c_int, c_void_p, c_void_p]),
    "moe_combine": (c_int, [c_void_p, c_void_p, c_int, c_int, c_int, c_void_p, c_void_p]),
    "lmhead_argmax_workspace_size": (c_size_t, [c_int, c_int, c_int, c_int]),
    "lmhead_argmax": (c_int, [c_void_p, c_void_p, c_float, c_void_p, c_int, c_int, c_int, c_int,
                              c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "mtp_verify": (c_int, [c_void_p, c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p,
                           c_void_p, c_void_p]),
    "moev_verify_step_workspace_size": (c_size_t, [ctypes.POINTER(Model), c_int, c_int]),
    "moev_verify_step": (c_int, [ctypes.POINTER(Model), c_void_p, c_int, c_int, c_void_p,
                                 c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                 c_void_p]),
    "moev_verify_step_probed": (c_int, [ctypes.POINTER(Model), c_void_p, c_int, c_int, c_void_p,
                                        c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                        ctypes.POINTER(StepProbe), c_void_p]),
    "moev_draft_workspace_size": (c_size_t, [ctypes.POINTER(Model), ctypes.POINTER(DraftWeights), c_int]),
    "moev_draft": (c_int, [ctypes.POINTER(Model), ctypes.POINTER(DraftWeights), c_void_p, c_void_p, c_int,
                           c_int, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "moev_spec_step_workspace_size": (c_size_t, [ctypes.POINTER(Model), ctypes.POINTER(DraftWeights), c_int,
                                                 c_int]),
    "moev_spec_step": (c_int, [ctypes.POINTER(Model), ctypes.POINTER(DraftWeights), c_void_p, c_int, c_int,
                               c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                               c_size_t, c_void_p]),
    "moev_verify_step_attn_workspace_size": (c_size_t, [ctypes.POINTER(Model), ctypes.POINTER(Attn), c_int,
                                                         c_int]),
    "moev_verify_step_attn": (c_int, [ctypes.POINTER(Model), ctypes.POINTER(Attn), c_void_p, c_int, c_int,
                                      c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_size_t, c_void_p]),
    "moev_attn_decode_workspace_size": (c_size_t, [c_int, c_int, c_int, c_int]),
    "moev_attn_decode": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_int,
                                 c_int, c_int, c_void_p, c_void_p, c_size_t, c_void_p]),
    "moev_prefill_workspace_size": (c_size_t, [ctypes.POINTER(Model), c_int, c_int]),
    "moev_prefill": (c_int, [ctypes.POINTER(Model), c_void_p, c_int, c_int, c_void_p, c_void_p,
                             c_void_p, c_size_t, c_void_p]),
    "moev_prefill_probed": (c_int, [ctypes.POINTER(Model), c_void_p, c_int, c_int, c_void_p, c_void_p,
                                    c_void_p, c_size_t, ctypes.POINTER(StepProbe), c_void_p]),
}

_lib = None


class MoevError(RuntimeError):
    def __init__(self, fn: str, status: int):
        lib = load()
        detail = lib.moev_last_error().decode()
        super().__init__(f"{fn}: {lib.moev_status_string(status).decode()} ({status}): {detail}")
        self.status = status


def load(path: str = LIB_PATH):
    """Load libmoev.so once and bind every exported entry point."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m moe_decoder_greedy_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)  # AttributeError if the symbol is not exported
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(fn: str, status: int) -> None:
    if status != 0:
        raise MoevError(fn, status)
