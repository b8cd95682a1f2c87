"""Helpers shared by the GPU tests: device transfers, bf16 views, tolerance
checks with near-tie flags.  No arithmetic of the method lives here."""
import dataclasses

import numpy as np
import torch

import synth


def need_gpu():
    import pytest
    if not torch.cuda.is_available():
        pytest.skip("no GPU in this environment")


def dev_bits(a: np.ndarray, dtype: str):
    """numpy weights (uint16 bf16 bits or float32) -> torch on the GPU."""
    if a is None:
        return None
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dev_operand(x: np.ndarray, dtype: str):
    """float64 values exactly representable in ``dtype`` -> torch on the GPU."""
    if dtype == "bf16":
        return dev_bits(synth.f32_to_bf16_bits(x.astype(np.float32)), "bf16")
    return torch.from_numpy(x.astype(np.float32)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy().astype(np.float64 if t.is_floating_point() else np.int64)


def dev_f32(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dev_i32(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def layer_shape(T_dtype="bf16"):
    return dataclasses.replace(synth.DECODER, n_layers=1)


def max_abs(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.abs(a - b).max()) if a.size else 0.0


def report(name, **kw):
    print(f"[{name}] " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)
