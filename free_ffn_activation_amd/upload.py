"""Host-array upload and offline packing through the C ABI.

Moves NumPy weight and token arrays (bf16 bit patterns as uint16, or fp32)
onto the device as torch tensors and packs a layer with prox_pack_proxy.
No arithmetic of the method happens here: the packing itself runs in the HIP
library.
"""
from __future__ import annotations

import numpy as np
import torch

from . import prox


def to_device(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """'bf16': uint16 bit patterns -> int16 tensor of the same bits;
    'f32': float32 tensor."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def wdtype_code(dtype: str) -> int:
    return prox.PROX_BF16 if dtype == "bf16" else prox.PROX_F32


def pack_arrays(w_up: np.ndarray, w_gate: np.ndarray, w_down: np.ndarray, dtype: str, device="cuda",
                activation: int = prox.PROX_ACT_SILU) -> prox.ProxLayer:
    """Upload W_up, W_gate ([d_model, d_ff]) and W_down ([d_ff, d_model]) and
    pack them into a new ProxLayer (synchronises the device)."""
    d, f = w_up.shape
    L = prox.ProxLayer(d, f, wdtype_code(dtype), device=device, activation=activation)
    wu = to_device(w_up, dtype, device)
    wg = to_device(w_gate, dtype, device)
    wd = to_device(w_down, dtype, device)
    prox.prox_pack_proxy(wu, wg, wd, L)
    torch.cuda.synchronize()
    del wu, wg, wd
    return L


def pack_layer(layer, device="cuda", activation: int = prox.PROX_ACT_SILU) -> prox.ProxLayer:
    """pack_arrays() for an object with w_up, w_gate, w_down and cfg.dtype
    (a synthetic layer)."""
    return pack_arrays(layer.w_up, layer.w_gate, layer.w_down, layer.cfg.dtype, device, activation)
