"""Host-to-device upload of synthetic workloads (plumbing only)."""
from __future__ import annotations

import numpy as np
import torch

from .inputs import Fp8Inputs, Workload, to_bf16_bits


def tensor(x: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Upload a float32 array holding values of `dtype` ("bf16" or "f32")."""
    if dtype == "bf16":
        bits = to_bf16_bits(x).view(np.int16)
        return torch.from_numpy(bits).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(device)


def upload(w: Workload, device="cuda") -> dict:
    """q, k, v (and beta when fixed) as device tensors."""
    out = {"q": tensor(w.q, w.dtype, device), "k": tensor(w.k, w.dtype, device),
           "v": tensor(w.v, w.dtype, device)}
    if w.beta is not None:
        out["beta"] = torch.from_numpy(np.ascontiguousarray(w.beta, np.float32)).to(device)
    return out


def upload_fp8(f: Fp8Inputs, device="cuda") -> dict:
    """q, k, v as float8_e4m3fn device tensors (the bytes as given)."""
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.uint8)).to(device).view(  # noqa: E731
        torch.float8_e4m3fn)
    return {"q": up(f.q), "k": up(f.k), "v": up(f.v)}
