"""Helpers shared by the GPU parity tests, the smoke check and the bench.

Moves synthetic layers onto the device, packs them through the library, and
provides the comparison rules: bit-exact integers, the tolerance band for the
channel mask and the float tolerances for y.
"""
from __future__ import annotations

import functools

import numpy as np
import torch

import oracle
import synth

# Tolerances stated for the decode path: masks bit-exact outside a 1e-3
# relative band around tau_s; y within max-abs 2e-2 and relative L2 1e-2.
MASK_BAND_REL = 1e-3
Y_MAX_ABS = 2e-2
Y_REL_L2 = 1e-2


from free_ffn_activation_amd.upload import pack_layer, to_device, wdtype_code  # noqa: F401  (re-exported)


@functools.lru_cache(maxsize=4)
def oracle_layer(cfg_name: str, layer_index: int = 0, n_dec: int = 16, n_cal=None):
    """Oracle-side view of a synthetic layer: fp64 weights and packed proxy."""
    cfg = synth.CONFIGS[cfg_name]
    layer = synth.make_layer(cfg, layer_index, n_dec=n_dec, n_cal=n_cal)
    return layer, oracle_view(layer)


def oracle_view(layer: synth.Layer) -> dict:
    dt = layer.cfg.dtype
    Wu = synth.as_f64(layer.w_up, dt)
    Wg = synth.as_f64(layer.w_gate, dt)
    Wd = synth.as_f64(layer.w_down, dt)
    qu, su = oracle.pack_proxy(Wu)
    qg, sg = oracle.pack_proxy(Wg)
    return {"Wu": Wu, "Wg": Wg, "Wd": Wd, "qu": qu, "su": su, "qg": qg, "sg": sg,
            "x_dec": synth.as_f64(layer.x_dec, dt), "x_cal": synth.as_f64(layer.x_cal, dt)}


def proxy_row_stride(f: int) -> int:
    """Bytes between proxy rows, as documented in prox.h."""
    return f if (f // 128) % 2 == 1 else f + 128


def decode_proxy_bytes(qbytes: np.ndarray, d: int, f: int):
    """Codes of the packed proxy, read per the layout documented in prox.h."""
    rows = np.asarray(qbytes, dtype=np.uint8).reshape(d, proxy_row_stride(f))
    assert np.all(rows[:, f:] == 0), "row padding must be zero"
    q = rows[:, :f].reshape(d, f // 16, 2, 8)
    lo = (q & 0x0F).astype(np.int16) - 8
    hi = (q >> 4).astype(np.int16) - 8
    codes = np.empty((d, f // 16, 2, 16), dtype=np.int16)
    codes[..., 0::2] = lo
    codes[..., 1::2] = hi
    up = codes[:, :, 0, :].reshape(d, f)
    gate = codes[:, :, 1, :].reshape(d, f)
    nib_ok = bool(np.all((q & 0x0F) != 0) and np.all((q >> 4) != 0))
    return up, gate, nib_ok


def band_compare(mask_idx: np.ndarray, count: int, s_oracle: np.ndarray, tau_s: float):
    """Compare a GPU channel list with the oracle's proxy state under the band
    rule.  Returns (out_of_band_mismatches, in_band_disagreements, ascending)."""
    f = s_oracle.size
    J = np.asarray(mask_idx[:count], dtype=np.int64)
    ascending = bool(np.all(np.diff(J) > 0)) and (count == 0 or (J[0] >= 0 and J[-1] < f))
    gpu = np.zeros(f, dtype=bool)
    gpu[J[(J >= 0) & (J < f)]] = True
    ref = oracle.channel_mask(s_oracle, tau_s)
    band = np.abs(np.abs(s_oracle) - tau_s) <= MASK_BAND_REL * tau_s
    diff = gpu != ref
    return int(np.sum(diff & ~band)), int(np.sum(diff & band)), ascending


def band_disagreements(mask_idx: np.ndarray, count: int, s_oracle: np.ndarray, tau_s: float) -> np.ndarray:
    """Distances | |s~_j| - tau_s | (oracle s~) of the channels where the GPU
    list and the oracle mask disagree."""
    f = s_oracle.size
    J = np.asarray(mask_idx[:count], dtype=np.int64)
    gpu = np.zeros(f, dtype=bool)
    gpu[J[(J >= 0) & (J < f)]] = True
    diff = gpu != oracle.channel_mask(s_oracle, tau_s)
    return np.abs(np.abs(s_oracle[diff]) - tau_s)


# A GPU proxy state is within S_TILDE_TOL * max|s~| of the oracle's (the
# proxy-state parity rule), so a channel can only be classified differently
# when its oracle |s~| lies that close to tau_s.
S_TILDE_TOL = 1e-5


def check_in_band(mask_idx: np.ndarray, count: int, s_oracle: np.ndarray, tau_s: float, label: str) -> None:
    """Bound on the in-band disagreements: each must be one the proxy-state
    tolerance explains (oracle |s~| within S_TILDE_TOL * max|s~| of tau_s)."""
    dist = band_disagreements(mask_idx, count, s_oracle, tau_s)
    lim = S_TILDE_TOL * float(np.max(np.abs(s_oracle))) if s_oracle.size else 0.0
    assert np.all(dist <= lim), f"{label}: in-band disagreement {dist.max():.3e} > {lim:.3e}"


def y_errors(y_gpu: np.ndarray, y_ref: np.ndarray):
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    max_abs = float(np.max(np.abs(y_gpu - y_ref))) if y_ref.size else 0.0
    nrm = float(np.linalg.norm(y_ref))
    rel = float(np.linalg.norm(y_gpu - y_ref) / nrm) if nrm > 0 else float(np.linalg.norm(y_gpu))
    return max_abs, rel


def y_ok(y_gpu, y_ref) -> bool:
    m, r = y_errors(y_gpu, y_ref)
    return m <= Y_MAX_ABS and r <= Y_REL_L2
