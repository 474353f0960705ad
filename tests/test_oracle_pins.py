"""Pins of the CPU oracle against what the pages and mathematics fix.

None of these tests routes through the function it checks: each compares the
oracle with a different computation (dense SwiGLU through torch, brute-force
sorts and loops, closed forms, numbers the pages print).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_values.json")


def _small_layer(d=64, f=96, dtype="f32", seed=7, std=0.05):
    cfg = synth.LayerConfig("small", d, f, dtype, std, 2, 20.0, 16, 0.5, 0.7, 1, seed)
    return synth.make_layer(cfg)


def _f64(layer):
    dt = layer.cfg.dtype
    return (synth.as_f64(layer.w_up, dt), synth.as_f64(layer.w_gate, dt),
            synth.as_f64(layer.w_down, dt), synth.as_f64(layer.x_dec, dt),
            synth.as_f64(layer.x_cal, dt))


def _torch_dense_swiglu(x, Wu, Wg, Wd):
    """Textbook SwiGLU FFN, y = (x W_up * SiLU(x W_gate)) W_down, via torch."""
    xt = torch.from_numpy(x)
    u = xt @ torch.from_numpy(Wu)
    h = torch.nn.functional.silu(xt @ torch.from_numpy(Wg))
    return ((u * h) @ torch.from_numpy(Wd)).numpy(), (u * h).numpy()


# ---------------------------------------------------------------- pack (O0)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_pack_invariants(dtype):
    layer = _small_layer(48, 80, dtype)
    Wu = synth.as_f64(layer.w_up, dtype)
    q, sc = oracle.pack_proxy(Wu)
    assert q.shape == Wu.shape and sc.shape == (Wu.shape[0],)
    assert q.dtype == np.int8 and sc.dtype == np.float32
    assert q.min() >= -7 and q.max() <= 7
    # one scale per row of the [d, f] matrix: every nonzero row reaches |q| = 7
    assert np.all(np.abs(q).max(axis=1) == 7)
    # scale is the fp32 value nearest absmax/7 (checked in exact rational terms)
    a = np.abs(Wu).max(axis=1)
    for r in range(Wu.shape[0]):
        exact = a[r] / 7.0
        assert abs(float(sc[r]) - exact) <= 0.5 * float(np.spacing(np.float32(exact))) * 1.0000001
    # reconstruction error at most half a step (plus the fp32 rounding of w/sc)
    err = np.abs(Wu - sc.astype(np.float64)[:, None] * q)
    bound = sc.astype(np.float64)[:, None] * (0.5 + 2.0 ** -20)
    assert np.all(err <= bound)


def test_pack_zero_row_and_ties():
    W = np.zeros((3, 4), dtype=np.float64)
    # row 1: absmax 7*2^-6 -> scale 2^-6 exactly; 3.5 and 2.5 steps are exact ties
    W[1] = np.array([7.0, 3.5, 2.5, -3.5]) * 2.0 ** -6
    W[2] = np.array([-7.0, 0.5, -0.5, 1.5]) * 2.0 ** -3
    q, sc = oracle.pack_proxy(W)
    assert sc[0] == 0 and np.all(q[0] == 0)
    assert sc[1] == np.float32(2.0 ** -6)
    assert list(q[1]) == [7, 4, 2, -4]          # half to even
    assert list(q[2]) == [-7, 0, 0, 2]


def test_pack_matches_bruteforce_rounding_loop():
    layer = _small_layer(16, 32, "bf16", seed=3)
    W = synth.as_f64(layer.w_gate, "bf16")
    q, sc = oracle.pack_proxy(W)
    for r in range(W.shape[0]):
        s = float(np.float32(float(np.max(np.abs(W[r]))) / 7.0))
        for c in range(W.shape[1]):
            quot = float(np.float32(np.float32(W[r, c]) / np.float32(s)))
            lo = math.floor(quot)
            frac = quot - lo
            if frac > 0.5 or (frac == 0.5 and lo % 2 == 1):
                lo += 1
            assert q[r, c] == max(-7, min(7, lo))


# ---------------------------------------------------------------- masks (O1, O4)
def test_input_mask_bruteforce_and_inclusive():
    rng = np.random.default_rng(0)
    x = rng.laplace(size=200)
    tau = float(np.sort(np.abs(x))[120])
    m = oracle.input_mask(x, tau)
    assert [bool(v) for v in m] == [abs(v) >= tau for v in x]
    assert m[np.argmin(np.abs(np.abs(x) - tau))]          # the tie itself is kept
    assert oracle.input_mask(x, 0.0).all()
    assert not oracle.input_mask(x, math.inf).any()


def test_channel_mask_equals_topk_of_sort():
    layer = _small_layer(32, 64, "f32", seed=11)
    Wu, Wg, Wd, X, _ = _f64(layer)
    qu, su = oracle.pack_proxy(Wu)
    qg, sg = oracle.pack_proxy(Wg)
    st = oracle.proxy_state(X[0], qu, su, qg, sg, 0.5)
    a = np.abs(st["s"])
    for k in (1, 5, 19, 64):
        order = sorted(range(a.size), key=lambda j: -a[j])
        tau = a[order[k - 1]]
        m = oracle.channel_mask(st["s"], tau)
        assert set(np.flatnonzero(m)) == set(order[:k])
        assert int(m.sum()) == k


# ---------------------------------------------------------------- proxy (O2, O3)
def test_proxy_unquantized_all_pass_is_swiglu_intermediate():
    """tau_x = 0 and W~ := W (scale 1, 'codes' = W) must give the textbook s."""
    layer = _small_layer(40, 72, "f32", seed=5)
    Wu, Wg, Wd, X, _ = _f64(layer)
    ones = np.ones(Wu.shape[0], dtype=np.float32)
    st = oracle.proxy_state(X[0], Wu, ones, Wg, ones, 0.0)
    _, s_ref = _torch_dense_swiglu(X[0], Wu, Wg, Wd)
    np.testing.assert_allclose(st["s"], s_ref, rtol=1e-12, atol=1e-14)


def test_proxy_int4_equals_masked_dequant_matmul():
    """s~ equals SwiGLU of (x * m_x) against the dequantised proxy (torch)."""
    layer = _small_layer(48, 64, "bf16", seed=9)
    Wu, Wg, Wd, X, _ = _f64(layer)
    qu, su = oracle.pack_proxy(Wu)
    qg, sg = oracle.pack_proxy(Wg)
    x = X[1]
    tau = float(np.median(np.abs(x)))
    st = oracle.proxy_state(x, qu, su, qg, sg, tau)
    xm = np.where(np.abs(x) >= tau, x, 0.0)
    Du = qu.astype(np.float64) * su.astype(np.float64)[:, None]
    Dg = qg.astype(np.float64) * sg.astype(np.float64)[:, None]
    _, s_ref = _torch_dense_swiglu(xm, Du, Dg, Wd)
    np.testing.assert_allclose(st["s"], s_ref, rtol=1e-12, atol=1e-15)
    assert int(st["m_x"].sum()) == sum(1 for v in x if abs(v) >= tau)


# ---------------------------------------------------------------- stage 2 (O5, O6)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_all_pass_decode_is_dense_swiglu(dtype):
    layer = _small_layer(64, 160, dtype, seed=13)
    Wu, Wg, Wd, X, _ = _f64(layer)
    qu, su = oracle.pack_proxy(Wu)
    qg, sg = oracle.pack_proxy(Wg)
    for t in range(3):
        out = oracle.decode(X[t], Wu, Wg, Wd, qu, su, qg, sg, 0.0, 0.0)
        y_ref, _ = _torch_dense_swiglu(X[t], Wu, Wg, Wd)
        assert out["k_s"] == Wu.shape[1] and out["k_x"] == Wu.shape[0]
        rel = np.linalg.norm(out["y"] - y_ref) / np.linalg.norm(y_ref)
        assert rel <= 1e-12


def test_stage2_weighted_sum_of_down_rows():
    """y = sum_{j in J} s_j W_down[j, :] for any J (row loop, textbook s)."""
    layer = _small_layer(24, 40, "f32", seed=17)
    Wu, Wg, Wd, X, _ = _f64(layer)
    x = X[0]
    _, s_full = _torch_dense_swiglu(x, Wu, Wg, Wd)
    rng = np.random.default_rng(1)
    for trial in range(4):
        m = rng.random(Wu.shape[1]) < 0.3
        out = oracle.stage2(x, Wu, Wg, Wd, m)
        y_ref = np.zeros(Wd.shape[1])
        for j in range(Wu.shape[1]):
            if m[j]:
                y_ref += s_full[j] * Wd[j, :]
        np.testing.assert_allclose(out["y"], y_ref, rtol=1e-12, atol=1e-14)
        u_ref = np.array([sum(x[i] * Wu[i, j] for i in range(x.size))
                          for j in range(Wu.shape[1]) if m[j]])
        np.testing.assert_allclose(out["u"], u_ref, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(out["s"], s_full[m], rtol=1e-12, atol=1e-15)


def test_empty_and_degenerate_masks():
    layer = _small_layer(32, 48, "f32", seed=19)
    Wu, Wg, Wd, X, _ = _f64(layer)
    qu, su = oracle.pack_proxy(Wu)
    qg, sg = oracle.pack_proxy(Wg)
    x = X[0]
    # tau_x above every |x|: s~ = 0, no channel passes a positive tau_s, y = 0
    out = oracle.decode(x, Wu, Wg, Wd, qu, su, qg, sg, math.inf, 1e-6)
    assert out["k_x"] == 0 and out["k_s"] == 0 and np.all(out["y"] == 0)
    # ... but tau_s = 0 then keeps every channel and Stage 2 is dense
    out = oracle.decode(x, Wu, Wg, Wd, qu, su, qg, sg, math.inf, 0.0)
    y_ref, _ = _torch_dense_swiglu(x, Wu, Wg, Wd)
    np.testing.assert_allclose(out["y"], y_ref, rtol=1e-12, atol=1e-14)
    # tau_s = +inf: empty channel mask, y = 0
    out = oracle.decode(x, Wu, Wg, Wd, qu, su, qg, sg, 0.0, math.inf)
    assert out["k_s"] == 0 and np.all(out["y"] == 0) and out["J"].size == 0


def test_index_list_ascending():
    m = np.zeros(100, bool)
    m[[3, 7, 99, 50, 0]] = True
    assert list(oracle.index_set(m)) == [0, 3, 7, 50, 99]


# ---------------------------------------------------------------- l2 bound
def test_l2_residual_identity_and_bound():
    """||xW - x_sp W|| = ||r W|| <= ||r|| ||W||_2 ([blog] key-turn section)."""
    rng = np.random.default_rng(3)
    d, f = 32, 24
    W = rng.standard_normal((d, f)) * 0.1
    x = rng.laplace(size=d)
    k = 12
    keep = np.zeros(d, bool)
    keep[np.argsort(-np.abs(x))[:k]] = True
    full = x @ W
    sp = oracle.pi_in(x, W, keep)
    r = np.where(keep, 0.0, x)
    lhs = np.linalg.norm(full - sp)
    mid = np.linalg.norm(r @ W)
    assert abs(lhs - mid) <= 1e-12 * max(1.0, mid)
    assert lhs <= np.linalg.norm(r) * np.linalg.norm(W, 2) * (1 + 1e-12)


def test_topk_minimises_residual_bruteforce():
    """Top-|x| selection minimises ||r||_2 over every subset of equal size."""
    rng = np.random.default_rng(4)
    n, k = 14, 5
    x = rng.laplace(size=n)
    m = oracle.input_mask(x, float(np.sort(np.abs(x))[n - k]))
    r_top = np.linalg.norm(np.where(m, 0.0, x))
    best = min(np.linalg.norm(np.delete(x, list(c)))
               for c in itertools.combinations(range(n), k))
    assert abs(r_top - best) <= 1e-12


# ---------------------------------------------------------------- calibration
def test_calibration_bruteforce():
    layer = _small_layer(32, 48, "f32", seed=23)
    Wu, Wg, Wd, _, Xc = _f64(layer)
    qu, su = oracle.pack_proxy(Wu)
    qg, sg = oracle.pack_proxy(Wg)
    tau_x, tau_s = oracle.calibrate(Xc, qu, su, qg, sg, 0.5, 0.7)
    vals = sorted(abs(v) for v in Xc.ravel())
    n = len(vals)
    nk = math.ceil(0.5 * n)
    assert tau_x == float(np.float32(vals[n - nk]))
    assert sum(1 for v in vals if v >= tau_x) == nk          # no ties in Laplace draws
    svals = []
    for t in range(Xc.shape[0]):
        st = oracle.proxy_state(Xc[t], qu, su, qg, sg, tau_x)
        svals.extend(abs(v) for v in st["s"])
    svals.sort()
    ns = len(svals)
    nks = math.ceil((1.0 - float(np.float32(0.7))) * ns)
    assert tau_s == svals[ns - nks]
    assert sum(1 for v in svals if v >= tau_s) == nks


def test_calibration_keep_fraction_is_the_fp32_value():
    """keep_x reaches the library as an fp32 value; fp32(0.3) is slightly
    above 0.3, so with N = 1280 pooled values ceil(fp32(0.3) N) = 385 while
    ceil(0.3 N) in double is 384.  The oracle must keep 385 (brute force)."""
    assert math.ceil(0.3 * 1280) == 384
    assert math.ceil(float(np.float32(0.3)) * 1280) == 385
    cfg = synth.LayerConfig("small", 32, 48, "f32", 0.05, 2, 20.0, 40, 0.5, 0.7, 1, 29)
    Wu, Wg, Wd, _, Xc = _f64(synth.make_layer(cfg))   # N = 40 x 32 = 1280 values
    qu, su = oracle.pack_proxy(Wu)
    qg, sg = oracle.pack_proxy(Wg)
    tau_x, _ = oracle.calibrate(Xc, qu, su, qg, sg, 0.3, 0.7)
    vals = sorted(abs(v) for v in Xc.ravel())
    assert len(vals) == 1280
    assert tau_x == float(np.float32(vals[1280 - 385]))
    assert sum(1 for v in vals if v >= tau_x) == 385   # no ties in Laplace draws


def test_n_keep_edges():
    assert oracle.n_keep(0.0, 10) == 0 and oracle.n_keep(1.0, 10) == 10
    assert oracle.n_keep(0.5, 7) == 4
    assert math.isinf(oracle.order_statistic_keep(np.arange(5.0), 0))
    assert oracle.order_statistic_keep(np.arange(5.0), 5) == 0.0


# ---------------------------------------------------------------- page values
def _golden():
    with open(GOLDEN) as fh:
        return json.load(fh)


def test_page_ffn_size():
    g = _golden()["ffn_weights_qwen3_8b"]
    cfg = synth.CONFIGS["qwen3_8b"]
    n = 3 * cfg.d_model * cfg.d_ff
    assert n == 150_994_944
    assert abs(n - g["value"]) <= g["printed_precision"]


def _laplace_energy_closed_form(drop):
    """Fraction of E[x^2] kept when the smallest `drop` fraction of |x| is
    removed from Laplace(0, 1): with q = 1 - drop, t = ln(1/q), the kept mass
    integral of x^2 e^{-x} over x > t is q (t^2 + 2t + 2), out of 2."""
    q = 1.0 - drop
    t = math.log(1.0 / q)
    return q * (t * t + 2 * t + 2) / 2.0


def test_page_laplace_energy_closed_form_and_generator():
    g = _golden()["laplace_energy_kept_drop70"]
    cf = _laplace_energy_closed_form(0.7)
    assert abs(cf - 0.878624) < 5e-7
    assert abs(cf - g["value"]) <= g["printed_precision"]
    assert abs(_laplace_energy_closed_form(0.5) - 0.966687) < 5e-7
    # the synthetic tokens follow that law (outlier-free coordinates)
    cfg = synth.LayerConfig("lap", 1_000_000, 8, "f32", 0.0, 0, 1.0, 1, 0.5, 0.7, 1, 1)
    rng = np.random.Generator(np.random.PCG64(5))
    x = synth.make_tokens(rng, 1, cfg.d_model, np.zeros(0, np.int64), 1.0, "f32")[0]
    x = x.astype(np.float64)
    a = np.abs(x)
    tau = oracle.order_statistic_keep(a, oracle.n_keep(0.3, a.size))
    kept = oracle.input_mask(x, tau)
    frac = float(np.sum(x[kept] ** 2) / np.sum(x ** 2))
    assert abs(frac - cf) < 0.005


def test_page_budget_operating_point():
    g = _golden()
    op = g["budget_operating_point"]
    s2 = oracle.stage2_sparsity_for_target(op["e"], op["s1"], op["alpha"])
    assert abs(s2 - op["s2"]) <= op["printed_precision"]
    assert abs(oracle.effective_sparsity(op["s1"], s2, op["alpha"]) - op["e"]) < 1e-12
    an = g["budget_s2_anchor_forces_full_input_sparsity"]
    # e = s2 - 2 alpha (1 - s1) / 3 with e = s2 forces s1 = 1
    assert abs(oracle.effective_sparsity(an["s1"], an["s2"], an["alpha"]) - an["e"]) < 1e-12
    assert oracle.effective_sparsity(0.99, an["s2"], an["alpha"]) < an["e"]
    # the configs' point (s1 = 0.5, s2 = 0.7) is e = 0.588889
    assert abs(oracle.effective_sparsity(0.5, 0.7, 1 / 3) - 0.5888889) < 1e-6


def test_page_proxy_storage_fraction():
    """Packed INT4 up+gate proxy is d*f bytes: 1/6 of the bf16 FFN bytes."""
    cfg = synth.CONFIGS["qwen3_8b"]
    proxy = cfg.d_model * cfg.d_ff                      # two matrices, 4 bits each
    ffn_bf16 = 3 * cfg.d_model * cfg.d_ff * 2
    assert proxy * 6 == ffn_bf16
    # ~12% of all weights when the FFN is ~70% of the model (page's figure)
    assert abs(proxy / ffn_bf16 * 0.70 - _golden()["proxy_storage_overhead"]["value"]) < 0.005


# ---------------------------------------------------------------- GeGLU (reading R18)
def _torch_dense_geglu(x, Wu, Wg, Wd):
    """GeGLU FFN, y = (x W_up * GELU_tanh(x W_gate)) W_down, via torch."""
    xt = torch.from_numpy(x)
    u = xt @ torch.from_numpy(Wu)
    h = torch.nn.functional.gelu(xt @ torch.from_numpy(Wg), approximate="tanh")
    return ((u * h) @ torch.from_numpy(Wd)).numpy(), (u * h).numpy()


def test_gelu_tanh_matches_library_and_identities():
    z = np.linspace(-12.0, 12.0, 4801)
    ref = torch.nn.functional.gelu(torch.from_numpy(z), approximate="tanh").numpy()
    np.testing.assert_allclose(oracle.gelu_tanh(z), ref, rtol=1e-13, atol=1e-15)
    # gelu(z) - gelu(-z) = z holds exactly for the tanh form
    np.testing.assert_allclose(oracle.gelu_tanh(z) - oracle.gelu_tanh(-z), z, rtol=0, atol=1e-13)
    assert oracle.gelu_tanh(np.array([0.0]))[0] == 0.0


def test_geglu_proxy_and_all_pass_decode():
    layer = _small_layer(48, 96, "bf16", seed=21)
    Wu, Wg, Wd, X, _ = _f64(layer)
    ones = np.ones(Wu.shape[0], dtype=np.float32)
    st = oracle.proxy_state(X[0], Wu, ones, Wg, ones, 0.0, act="gelu_tanh")
    _, s_ref = _torch_dense_geglu(X[0], Wu, Wg, Wd)
    np.testing.assert_allclose(st["s"], s_ref, rtol=1e-12, atol=1e-14)
    qu, su = oracle.pack_proxy(Wu)
    qg, sg = oracle.pack_proxy(Wg)
    for t in range(2):
        out = oracle.decode(X[t], Wu, Wg, Wd, qu, su, qg, sg, 0.0, 0.0, act="gelu_tanh")
        y_ref, _ = _torch_dense_geglu(X[t], Wu, Wg, Wd)
        assert np.linalg.norm(out["y"] - y_ref) / np.linalg.norm(y_ref) <= 1e-12
    # a GeGLU mask differs from the SwiGLU one on the same layer (the
    # activation really is threaded through)
    tau = float(np.median(np.abs(X[2])))
    a = oracle.proxy_state(X[2], qu, su, qg, sg, tau, act="gelu_tanh")["s"]
    b = oracle.proxy_state(X[2], qu, su, qg, sg, tau)["s"]
    assert not np.allclose(a, b)


# ---------------------------------------------------------------- histogram calibration (reading R19)
def test_strided_sample_bruteforce():
    v = np.arange(10) * 1.5
    assert list(oracle.strided_sample(v, 4)) == [v[0], v[2], v[5], v[7]]   # floor(i*10/4)
    assert list(oracle.strided_sample(v, 20)) == list(v)                    # fewer values than M
    big = np.arange(1000)
    s = oracle.strided_sample(big, 7)
    assert list(s) == [(i * 1000) // 7 for i in range(7)]


def test_histogram_threshold_brackets_the_order_statistic():
    """The histogram threshold keeps at least n_keep samples, never more than
    the next bin's worth, and sits within one bin width below the exact
    order statistic."""
    rng = np.random.default_rng(17)
    for trial in range(30):
        a = np.abs(rng.laplace(size=5000)).astype(np.float32)
        keep = float(rng.uniform(0.05, 0.95))
        nb = int(rng.choice([16, 256, 4096]))
        t = oracle.histogram_threshold(a, keep, nb)
        n = oracle.n_keep(keep, a.size)
        exact = oracle.order_statistic_keep(a, n)
        w = np.float32(np.float32(a.max()) / np.float32(nb))
        assert np.sum(a.astype(np.float64) >= t) >= n or t == 0.0
        assert t <= exact + 1e-12 and exact - t <= float(w) * (1 + 1e-6)
    # edges
    a = np.abs(rng.normal(size=100)).astype(np.float32)
    assert math.isinf(oracle.histogram_threshold(a, 0.0, 64))
    assert oracle.histogram_threshold(a, 1.0, 64) == 0.0
    assert oracle.histogram_threshold(np.zeros(10, np.float32), 0.5, 64) == 0.0


def test_calibrate_hist_close_to_exact_calibration():
    layer = _small_layer(64, 128, "f32", seed=23)
    Wu, Wg, Wd, X, Xc = _f64(layer)
    qu, su = oracle.pack_proxy(Wu)
    qg, sg = oracle.pack_proxy(Wg)
    tx_e, ts_e = oracle.calibrate(Xc, qu, su, qg, sg, 0.5, 0.7)
    tx_h, ts_h = oracle.calibrate_hist(Xc, qu, su, qg, sg, 0.5, 0.7, max_samples=200000, n_bins=4096)
    # every sample is kept (N < 200k), so tau_x is within one bin below the exact one
    wx = float(np.float32(np.float32(np.abs(Xc).max()) / np.float32(4096)))
    assert tx_h <= tx_e and tx_e - tx_h <= wx * (1 + 1e-6)
    # tau_s: within one bin below the exact statistic of the same pool (the
    # proxy state under tau_x from the histogram)
    pool = np.concatenate([np.abs(oracle.proxy_state(Xc[t], qu, su, qg, sg, tx_h)["s"])
                           for t in range(Xc.shape[0])])
    exact_s = oracle.order_statistic_keep(pool.astype(np.float32), oracle.n_keep(1.0 - float(np.float32(0.7)), pool.size))
    ws_ = float(np.float32(np.float32(pool.astype(np.float32).max()) / np.float32(4096)))
    assert ts_h <= exact_s and exact_s - ts_h <= ws_ * (1 + 1e-6)


# ---------------------------------------------------------------- 16-bit proxy (ablation A1, reading R20)
def test_proxy_w16_equals_masked_dense_swiglu():
    """The 16-bit proxy state is the SwiGLU intermediate of (x * m_x) against
    the original weights (torch), for bf16 and fp32 layers."""
    for dtype, seed in (("bf16", 41), ("f32", 42)):
        layer = _small_layer(48, 80, dtype, seed=seed)
        Wu, Wg, Wd, X, _ = _f64(layer)
        for t in range(2):
            x = X[t]
            tau = float(np.float32(np.median(np.abs(x))))
            st = oracle.proxy_state_w16(x, Wu, Wg, tau)
            xm = np.where(np.abs(x) >= tau, x, 0.0)
            _, s_ref = _torch_dense_swiglu(xm, Wu, Wg, Wd)
            np.testing.assert_allclose(st["s"], s_ref, rtol=1e-12, atol=1e-15)
            assert int(st["m_x"].sum()) == int(np.sum(np.abs(x) >= tau))


def test_proxy_w16_bruteforce_loops():
    """Tiny case written out as loops over the kept inputs."""
    rng = np.random.default_rng(3)
    d, f = 7, 5
    Wu, Wg = rng.normal(size=(d, f)), rng.normal(size=(d, f))
    x = rng.laplace(size=d)
    tau = float(np.sort(np.abs(x))[3])
    st = oracle.proxy_state_w16(x, Wu, Wg, tau)
    for j in range(f):
        u = sum(x[i] * Wu[i, j] for i in range(d) if abs(x[i]) >= tau)
        g = sum(x[i] * Wg[i, j] for i in range(d) if abs(x[i]) >= tau)
        assert math.isclose(st["s"][j], u * g / (1.0 + math.exp(-g)), rel_tol=1e-12, abs_tol=1e-15)


def test_proxy_w16_with_dequantised_weights_is_the_int4_proxy():
    """Fed the dequantised INT4 matrices, the 16-bit proxy path must give the
    INT4 proxy state (both are Pi^in of the same matrices)."""
    layer = _small_layer(40, 64, "bf16", seed=43)
    Wu, Wg, _, X, _ = _f64(layer)
    qu, su = oracle.pack_proxy(Wu)
    qg, sg = oracle.pack_proxy(Wg)
    tau = float(np.float32(np.median(np.abs(X[0]))))
    a = oracle.proxy_state(X[0], qu, su, qg, sg, tau)
    b = oracle.proxy_state_w16(X[0], oracle.dequantize(qu, su), oracle.dequantize(qg, sg), tau)
    np.testing.assert_allclose(b["s"], a["s"], rtol=1e-12, atol=1e-15)


def test_decode_w16_all_pass_and_empty():
    layer = _small_layer(64, 96, "bf16", seed=44)
    Wu, Wg, Wd, X, _ = _f64(layer)
    out = oracle.decode_w16(X[0], Wu, Wg, Wd, 0.0, 0.0)
    y_ref, _ = _torch_dense_swiglu(X[0], Wu, Wg, Wd)
    assert out["k_s"] == Wu.shape[1] and out["k_x"] == Wu.shape[0]
    assert np.linalg.norm(out["y"] - y_ref) / np.linalg.norm(y_ref) <= 1e-12
    out = oracle.decode_w16(X[1], Wu, Wg, Wd, math.inf, 1e-6)
    assert out["k_x"] == 0 and out["k_s"] == 0 and np.all(out["y"] == 0)


def test_calibration_w16_bruteforce():
    layer = _small_layer(32, 48, "bf16", seed=45)
    Wu, Wg, _, _, Xc = _f64(layer)
    tau_x, tau_s = oracle.calibrate_w16(Xc, Wu, Wg, 0.5, 0.7)
    vals = sorted(abs(v) for v in Xc.ravel())
    n = len(vals)
    assert tau_x == float(np.float32(vals[n - math.ceil(0.5 * n)]))
    svals = []
    for t in range(Xc.shape[0]):
        xm = np.where(np.abs(Xc[t]) >= tau_x, Xc[t], 0.0)
        _, s = _torch_dense_swiglu(xm, Wu, Wg, np.zeros((Wu.shape[1], 1)))
        svals.extend(abs(v) for v in s)
    svals.sort()
    ns = len(svals)
    nks = math.ceil((1.0 - float(np.float32(0.7))) * ns)
    assert math.isclose(tau_s, svals[ns - nks], rel_tol=1e-12)
