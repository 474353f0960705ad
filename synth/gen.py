"""Seeded layer and token generators (no method arithmetic here)."""
from __future__ import annotations

import dataclasses
import numpy as np


# --------------------------------------------------------------------------
# bf16 storage helpers (bit-pattern conversions only)
# --------------------------------------------------------------------------
def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def as_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 view of stored values ('bf16' uint16 bits or 'f32')."""
    if dtype == "bf16":
        return f32_from_bf16_bits(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# Workload recipes
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    d_model: int
    d_ff: int
    dtype: str            # 'f32' or 'bf16' (weights and x share it)
    w_std: float          # weight std (i.i.d. normal)
    n_outliers: int       # fixed outlier coordinates of x per layer
    outlier_scale: float  # factor applied to the Laplace value there
    n_cal: int            # calibration tokens
    keep_x: float         # fraction of input coordinates kept (Stage 1)
    sparsity_s: float     # intermediate-channel sparsity (Stage 2)
    batch: int
    base_seed: int


def _nout(d: int) -> int:
    return int(round(0.001 * d))


CONFIGS = {
    "tiny": LayerConfig("tiny", 256, 768, "f32", 0.05, 4, 20.0, 64, 0.5, 0.7, 1, 101),
    "qwen3_8b": LayerConfig("qwen3_8b", 4096, 12288, "bf16", 0.02, _nout(4096), 30.0,
                            256, 0.5, 0.7, 1, 102),
    "qwen3_8b_stack": LayerConfig("qwen3_8b_stack", 4096, 12288, "bf16", 0.02, _nout(4096),
                                  30.0, 256, 0.5, 0.7, 1, 103),
    "qwen3_8b_batch8": LayerConfig("qwen3_8b_batch8", 4096, 12288, "bf16", 0.02, _nout(4096),
                                   30.0, 256, 0.5, 0.7, 8, 104),
    "qwen3_32b": LayerConfig("qwen3_32b", 5120, 25600, "bf16", 0.015, _nout(5120), 30.0,
                             256, 0.5, 0.7, 1, 105),
}


@dataclasses.dataclass
class Layer:
    cfg: LayerConfig
    seed: int
    w_up: np.ndarray      # [d, f]  paper orientation (x @ W_up)
    w_gate: np.ndarray    # [d, f]
    w_down: np.ndarray    # [f, d]
    outlier_pos: np.ndarray  # int64 [n_outliers], sorted
    x_cal: np.ndarray     # [n_cal, d]
    x_dec: np.ndarray     # [n_dec, d]


def _store(a32: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_from_f32(a32) if dtype == "bf16" else np.ascontiguousarray(a32, np.float32)


def make_tokens(rng: np.random.Generator, n: int, d: int, pos: np.ndarray, scale: float,
                dtype: str) -> np.ndarray:
    """Laplace(0,1) tokens; coordinates `pos` multiplied by `scale`."""
    x = rng.laplace(0.0, 1.0, size=(n, d))
    if len(pos):
        x[:, pos] *= scale
    return _store(x.astype(np.float32), dtype)


def make_layer(cfg: LayerConfig, layer_index: int = 0, n_dec: int = 16,
               n_cal: int | None = None, seed: int | None = None) -> Layer:
    """One seeded SwiGLU FFN layer plus calibration and decode tokens.

    Seeding: SeedSequence(seed).spawn(6) gives, in order, the streams for
    W_up, W_gate, W_down, the outlier positions, the calibration tokens and
    the decode tokens (PCG64 each).  seed defaults to base_seed*1000+layer_index.
    """
    if seed is None:
        seed = cfg.base_seed * 1000 + layer_index
    ss = np.random.SeedSequence(seed).spawn(6)
    rngs = [np.random.Generator(np.random.PCG64(s)) for s in ss]
    d, f = cfg.d_model, cfg.d_ff

    def weights(r, shape):
        w = r.standard_normal(size=shape, dtype=np.float32)
        w *= np.float32(cfg.w_std)
        return _store(w, cfg.dtype)

    w_up = weights(rngs[0], (d, f))
    w_gate = weights(rngs[1], (d, f))
    w_down = weights(rngs[2], (f, d))
    pos = np.sort(rngs[3].choice(d, size=cfg.n_outliers, replace=False)).astype(np.int64)
    nc = cfg.n_cal if n_cal is None else n_cal
    x_cal = make_tokens(rngs[4], nc, d, pos, cfg.outlier_scale, cfg.dtype)
    x_dec = make_tokens(rngs[5], n_dec, d, pos, cfg.outlier_scale, cfg.dtype)
    return Layer(cfg, seed, w_up, w_gate, w_down, pos, x_cal, x_dec)
