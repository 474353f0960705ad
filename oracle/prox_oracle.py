"""Plain CPU oracle of the Prox two-stage sparse SwiGLU FFN decode step.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously-correct
reference that the GPU library is checked against.  Only the test suite, the
package smoke check and the benchmark's CPU-baseline leg may import it; the
product path (the HIP library and its Python binding) never does, and the two
share no code.

Arithmetic is NumPy float64 on the exact stored values (bf16 or fp32 weights
and inputs widened exactly), except where a reading below fixes another
precision (the INT4 packer, whose scale is an fp32 value by definition).

Sources, cited by page and section (the pages are the authority):
  [blog]   "Prox 完全拆解：先用便宜代理找通道，再用精确计算守住 SwiGLU 的质量"
           (deep-dive blog post on Prox)
  [paper]  "Prox: 通过近似中间通道显著性实现 LLM 中免训练的 FFN 激活稀疏化"
           (Chinese rendering of arXiv 2607.27591; truncated in section 3.1)
  [gist]   gist.science summaries of arXiv 2607.27591 (Dutch / Portuguese /
           French), section on the hardware implementation.

Readings where the pages are silent (each also listed in the design notes):
  R1  "per-row" INT4 scale = one scale per row of the paper-layout [d, f]
      matrix, i.e. per input coordinate.
  R2  codes in [-7, 7], scale = fp32(absmax / 7), code = round-half-even of
      the fp32 quotient fp32(w / scale), clamped; an all-zero row has scale 0
      and codes 0.
  R4  threshold tests are inclusive (>=), as printed.
  R5  Stage 2 uses the dense x.
  R6  tau_s is calibrated on |proxy state| with input sparsity applied.
  R7  calibration thresholds are exact order statistics; the keep fractions
      are the fp32 values the C ABI receives, so n = ceil(fp32(keep) * N)
      (fp32(0.3) is slightly above 0.3: at N = 1280 that keeps 385, not 384).
  R10 SiLU(z) = z / (1 + exp(-z)).
  R13 empty masks give zero output.
  R14 index lists are ascending.
  R19 the pages' calibration keeps at most 200,000 samples per layer and a
      4,096-bin histogram; read as: an evenly strided subsample (element
      floor(i N / M) of the N pooled magnitudes, i < M), linear bins of width
      w = fp32(max / n_bins) over [0, max], bin = min(n_bins - 1,
      floor(fp32(v / w))), and the threshold is the lower edge fp32(b * w) of
      the bin where the count from the top first reaches the keep count.
  R18 GeGLU layers (the pages evaluate GeGLU-style Gemma-3 as well as SwiGLU
      models) use GELU in its tanh form,
      0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))), in both the proxy
      state and Stage 2; everything else is unchanged.
  R20 the pages' precision ablation swaps the INT4 proxy for an FP16 one at
      the same budget; read as a 16-bit proxy that is the layer's own 16-bit
      weights (bf16 for these layers), so the proxy state is the input-sparse
      projection with the original weights and nothing is quantised.

Parity pins: every function here is pinned by tests that do not route through
itself (dense SwiGLU, brute-force sorts, closed forms, page values); the
proxy-state bits of the GPU are compared under a tolerance band because fp32
summation order is not fixed by the pages.
"""
from __future__ import annotations

import math
import numpy as np


# --------------------------------------------------------------------------
# Elementary definitions
# --------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) (reading R10).  [paper] §2.1 names SiLU as the
    gate non-linearity of SwiGLU."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def gelu_tanh(z: np.ndarray) -> np.ndarray:
    """GELU in its tanh form (reading R18), the gate non-linearity of a GeGLU
    FFN.  [blog] evidence section: GeGLU-style Gemma-3 is among the models the
    method is evaluated on, with the gate activation in place of SiLU."""
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z ** 3)))


ACTIVATIONS = {"silu": silu, "gelu_tanh": gelu_tanh}


def index_set(m: np.ndarray) -> np.ndarray:
    """I(m): ascending positions where the binary mask is 1.  [paper] §2.2."""
    return np.flatnonzero(np.asarray(m, dtype=bool))


def pi_in(x: np.ndarray, W: np.ndarray, m: np.ndarray) -> np.ndarray:
    """Input sparsity: x restricted to I(m) times the rows I(m) of W.
    [paper] §2.2, definition of Pi^in."""
    idx = index_set(m)
    return x[idx] @ W[idx, :]


def pi_out(x: np.ndarray, W: np.ndarray, m: np.ndarray) -> np.ndarray:
    """Output sparsity: x times the columns I(m) of W (only the kept outputs).
    [paper] §2.2, definition of Pi^out."""
    idx = index_set(m)
    return x @ W[:, idx]


# --------------------------------------------------------------------------
# O0: offline INT4 proxy of W_up / W_gate
# --------------------------------------------------------------------------
def pack_proxy(W: np.ndarray):
    """Symmetric per-row INT4 quantisation of one proxy matrix.

    [blog] section "Stage 1": the up and gate proxies are symmetric per-row
    INT4 copies; W_down has none.  Readings R1 (one scale per row of the
    [d_model, d_ff] matrix) and R2 (range, scale, rounding).

    W: [d, f] exact stored values.  Returns (q int8 [d, f], scale float32 [d]).
    """
    W32 = np.asarray(W, dtype=np.float64).astype(np.float32)
    if not np.array_equal(W32.astype(np.float64), np.asarray(W, dtype=np.float64)):
        raise ValueError("weights must be exactly representable in fp32")
    absmax = np.max(np.abs(W32), axis=1)
    scale = (absmax / np.float32(7.0)).astype(np.float32)       # IEEE fp32 division
    q = np.zeros(W32.shape, dtype=np.int8)
    nz = scale > 0
    quot = (W32[nz] / scale[nz, None]).astype(np.float32)       # fp32 quotient
    q[nz] = np.clip(np.rint(quot), -7, 7).astype(np.int8)       # half-to-even
    return q, scale


def dequantize(q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """The proxy matrix W~ = diag(scale) q, in fp64 (exact)."""
    return scale.astype(np.float64)[:, None] * q.astype(np.float64)


# --------------------------------------------------------------------------
# O1-O4: Stage 1, proxy and shared channel mask
# --------------------------------------------------------------------------
def input_mask(x: np.ndarray, tau_x: float) -> np.ndarray:
    """[m_x]_i = 1[|x_i| >= tau_x].  [blog] section "Stage 1", m_x equation."""
    return np.abs(np.asarray(x, dtype=np.float64)) >= np.float64(tau_x)


def proxy_state(x, q_up, sc_up, q_gate, sc_gate, tau_x, act="silu"):
    """Stage-1 proxy state for one token.

    [blog] section "Stage 1": u~ = Pi^in(x, W~_up, m_x),
    h~ = SiLU(Pi^in(x, W~_gate, m_x)), s~ = u~ * h~, with one input mask shared
    by both branches (GELU in place of SiLU for a GeGLU layer, R18).
    Returns dict(u, g, s, m_x).
    """
    x = np.asarray(x, dtype=np.float64)
    m_x = input_mask(x, tau_x)
    idx = index_set(m_x)
    # Pi^in reads only the rows I(m_x) of W~, so only those rows are
    # dequantised: W~[I, :] = diag(scale[I]) q[I, :].
    u = x[idx] @ dequantize(q_up[idx], sc_up[idx])
    g = x[idx] @ dequantize(q_gate[idx], sc_gate[idx])
    s = u * ACTIVATIONS[act](g)
    return {"u": u, "g": g, "s": s, "m_x": m_x}


def proxy_state_w16(x, W_up, W_gate, tau_x, act="silu"):
    """Stage-1 proxy state with the 16-bit proxy of the pages' precision
    ablation ([blog] evidence section, ablation A1; reading R20): the proxy
    matrices are the layer's own 16-bit weights, so
    u~ = Pi^in(x, W_up, m_x), h~ = act(Pi^in(x, W_gate, m_x)), s~ = u~ h~.
    Returns dict(u, g, s, m_x).
    """
    x = np.asarray(x, dtype=np.float64)
    m_x = input_mask(x, tau_x)
    u = pi_in(x, W_up, m_x)
    g = pi_in(x, W_gate, m_x)
    return {"u": u, "g": g, "s": u * ACTIVATIONS[act](g), "m_x": m_x}


def channel_mask(s_tilde: np.ndarray, tau_s: float) -> np.ndarray:
    """[m_s]_j = 1[|s~_j| >= tau_s].  [blog] section "Stage 1", m_s equation."""
    return np.abs(np.asarray(s_tilde, dtype=np.float64)) >= np.float64(tau_s)


# --------------------------------------------------------------------------
# O5-O6: Stage 2, exact compute on the kept channels
# --------------------------------------------------------------------------
def stage2(x, W_up, W_gate, W_down, m_s, act="silu"):
    """Exact sparse SwiGLU (GeGLU with act="gelu_tanh", R18) on the channels
    of m_s.

    [blog] section "Stage 2": u_sp = Pi^out(x, W_up, m_s),
    h_sp = SiLU(Pi^out(x, W_gate, m_s)), s_sp = u_sp * h_sp,
    y = Pi^in(s_sp, W_down, m_s), with the original weights and the dense x
    (reading R5).  s_sp is indexed by the ascending list I(m_s).
    """
    x = np.asarray(x, dtype=np.float64)
    u_sp = pi_out(x, W_up, m_s)
    g_sp = pi_out(x, W_gate, m_s)
    h_sp = ACTIVATIONS[act](g_sp)
    s_sp = u_sp * h_sp
    # Pi^in over the kept rows of W_down; s_sp is already restricted to I(m_s),
    # so scatter it back to a full-length vector before applying the definition.
    s_full = np.zeros(W_down.shape[0], dtype=np.float64)
    s_full[index_set(m_s)] = s_sp
    y = pi_in(s_full, W_down, m_s)
    return {"u": u_sp, "g": g_sp, "s": s_sp, "y": y}


# --------------------------------------------------------------------------
# Whole decode step
# --------------------------------------------------------------------------
def decode(x, W_up, W_gate, W_down, q_up, sc_up, q_gate, sc_gate, tau_x, tau_s, act="silu"):
    """One Prox FFN decode step for one token (batch rows run independently).

    Stage 1 ([blog] "Stage 1") produces the shared channel mask from the INT4
    proxy; Stage 2 ([blog] "Stage 2") computes the kept channels exactly.
    The proxy values never reach y ([blog] "key turn" section: errors stay at
    the mask boundary).
    Returns dict(y, J (ascending int64), k_x, k_s, s_tilde, m_x, m_s, s_sp).
    """
    st = proxy_state(x, q_up, sc_up, q_gate, sc_gate, tau_x, act)
    m_s = channel_mask(st["s"], tau_s)
    out = stage2(x, W_up, W_gate, W_down, m_s, act)
    return {"y": out["y"], "J": index_set(m_s), "k_x": int(st["m_x"].sum()),
            "k_s": int(m_s.sum()), "s_tilde": st["s"], "m_x": st["m_x"], "m_s": m_s,
            "s_sp": out["s"]}


def decode_w16(x, W_up, W_gate, W_down, tau_x, tau_s, act="silu"):
    """decode() with the 16-bit proxy (reading R20) in place of the INT4 one;
    Stage 2 is unchanged."""
    st = proxy_state_w16(x, W_up, W_gate, tau_x, act)
    m_s = channel_mask(st["s"], tau_s)
    out = stage2(x, W_up, W_gate, W_down, m_s, act)
    return {"y": out["y"], "J": index_set(m_s), "k_x": int(st["m_x"].sum()),
            "k_s": int(m_s.sum()), "s_tilde": st["s"], "m_x": st["m_x"], "m_s": m_s,
            "s_sp": out["s"]}


# --------------------------------------------------------------------------
# C1-C2: offline calibration of the per-layer scalar thresholds
# --------------------------------------------------------------------------
def n_keep(keep_fraction: float, n: int) -> int:
    """Number of samples a threshold must keep: ceil(keep * N) in double,
    clamped to [0, N]."""
    k = math.ceil(float(keep_fraction) * n)
    return max(0, min(n, k))


def order_statistic_keep(values: np.ndarray, keep: int) -> float:
    """The keep-th largest value (reading R7); +inf when keep == 0."""
    v = np.sort(np.asarray(values, dtype=np.float64).ravel())
    if keep == 0:
        return math.inf
    return float(v[v.size - keep])


def calibrate(X_cal, q_up, sc_up, q_gate, sc_gate, keep_x: float, sparsity_s: float, act="silu"):
    """Per-layer thresholds (tau_x, tau_s) from calibration tokens.

    [blog] "evidence" section (calibration paragraph): fixed per-layer scalar
    thresholds from activation samples.  tau_x keeps the fraction keep_x of
    the pooled |x| (C1); tau_s keeps 1 - sparsity_s of the pooled |s~|, where
    s~ is the proxy state under tau_x (C2, reading R6).  Both fractions are
    the fp32 values the C ABI receives, widened exactly: n = ceil(fp32(keep_x)
    * N) for tau_x and n = ceil((1 - fp32(sparsity_s)) * N) in double for
    tau_s (reading R7).
    """
    return calibrate_with(X_cal, lambda xt, tx: proxy_state(xt, q_up, sc_up, q_gate, sc_gate, tx, act)["s"],
                          keep_x, sparsity_s)


def calibrate_w16(X_cal, W_up, W_gate, keep_x: float, sparsity_s: float, act="silu"):
    """calibrate() for the 16-bit proxy (reading R20): tau_s is taken over
    the 16-bit proxy state."""
    return calibrate_with(X_cal, lambda xt, tx: proxy_state_w16(xt, W_up, W_gate, tx, act)["s"],
                          keep_x, sparsity_s)


def calibrate_with(X_cal, state_fn, keep_x: float, sparsity_s: float):
    """C1-C2 for a given proxy: state_fn(x_token, tau_x) returns the proxy
    state s~ of one token under the fp32 input threshold tau_x."""
    X = np.asarray(X_cal, dtype=np.float64)
    ax = np.abs(X).ravel()
    # keep fractions arrive as fp32 values (the ABI's type), widened exactly:
    # ceil(keep * N) is taken on that fp32 value (reading R7)
    tau_x = order_statistic_keep(ax, n_keep(float(np.float32(keep_x)), ax.size))
    tau_x32 = float(np.float32(tau_x)) if math.isfinite(tau_x) else math.inf
    s_all = np.concatenate([np.abs(state_fn(X[t], tau_x32)) for t in range(X.shape[0])])
    keep_s = 1.0 - float(np.float32(sparsity_s))
    tau_s = order_statistic_keep(s_all, n_keep(keep_s, s_all.size))
    return tau_x32, tau_s


def strided_sample(values: np.ndarray, max_samples: int) -> np.ndarray:
    """At most max_samples of the pooled values: element floor(i N / M) for
    i < M = min(N, max_samples) (reading R19)."""
    v = np.asarray(values).ravel()
    n = v.size
    m = min(n, int(max_samples))
    idx = np.array([(i * n) // m for i in range(m)], dtype=np.int64) if m else np.zeros(0, np.int64)
    return v[idx]


def histogram_threshold(samples: np.ndarray, keep_fraction: float, n_bins: int) -> float:
    """Threshold from a linear n_bins histogram of the sample magnitudes
    (reading R19): the lower edge of the bin where the count from the top
    first reaches n_keep(keep_fraction, M).  Bin decisions and the edge are
    fp32, the precision the stored threshold has."""
    a = np.abs(np.asarray(samples, dtype=np.float64)).astype(np.float32)
    keep = n_keep(keep_fraction, a.size)
    if keep == 0:
        return math.inf
    vmax = np.float32(a.max())
    w = np.float32(vmax / np.float32(n_bins))
    if w == 0:
        return 0.0
    bins = np.minimum(n_bins - 1, np.floor(a / w).astype(np.int64))
    hist = np.bincount(bins, minlength=n_bins)
    cum = 0
    for b in range(n_bins - 1, -1, -1):
        cum += int(hist[b])
        if cum >= keep:
            return float(np.float32(np.float32(b) * w))
    return 0.0


def calibrate_hist(X_cal, q_up, sc_up, q_gate, sc_gate, keep_x: float, sparsity_s: float,
                   max_samples: int = 200000, n_bins: int = 4096, act="silu"):
    """Per-layer thresholds the way the pages calibrate ([blog] end-to-end
    decoding section, calibration paragraph: at most 200,000 samples per layer
    and a 4,096-bin histogram), with reading R19 for the sampling and binning.
    tau_s is computed on the proxy state under this tau_x (R6)."""
    X = np.asarray(X_cal, dtype=np.float64)
    # keep fractions arrive as fp32 values (the ABI's type), widened exactly
    tau_x = histogram_threshold(strided_sample(np.abs(X), max_samples), float(np.float32(keep_x)), n_bins)
    s_all = np.concatenate([
        np.abs(proxy_state(X[t], q_up, sc_up, q_gate, sc_gate, tau_x, act)["s"])
        for t in range(X.shape[0])])
    keep_s = 1.0 - float(np.float32(sparsity_s))
    tau_s = histogram_threshold(strided_sample(s_all, max_samples), keep_s, n_bins)
    return tau_x, tau_s


# --------------------------------------------------------------------------
# Budget model (host-side planning)
# --------------------------------------------------------------------------
def effective_sparsity(s1: float, s2: float, alpha: float) -> float:
    """e = 1 - C/3 with C = 2 alpha (1 - s1) + 3 (1 - s2).
    [blog] section on the computation budget."""
    cost = 2.0 * alpha * (1.0 - s1) + 3.0 * (1.0 - s2)
    return 1.0 - cost / 3.0


def stage2_sparsity_for_target(e: float, s1: float, alpha: float) -> float:
    """Solve e = s2 - 2 alpha (1 - s1) / 3 for s2.  [blog] budget section."""
    return e + 2.0 * alpha * (1.0 - s1) / 3.0
