"""GPU parity of the 16-bit proxy (the pages' precision ablation A1, reading
R20: the layer's own bf16 weights as the Stage-1 proxy), through the C ABI.

Rules as for the INT4 proxy: packed bytes bit-exact; k_x exact; channel masks
exact outside the 1e-3 tau_s band; y within max-abs 2e-2 / rel-L2 1e-2 of the
oracle's Stage 2 on the GPU's channel list; the proxy state within 1e-5 of its
largest magnitude; tau_x exact and tau_s within 1e-5 relative.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from prox_gpu_util import band_compare, check_in_band, oracle_layer, oracle_view, to_device, y_errors, y_ok

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from free_ffn_activation_amd import prox
    return prox


def _cfg(d, f, seed, n_dec):
    return synth.LayerConfig(f"p16_{d}x{f}", d, f, "bf16", 0.05, max(1, d // 64), 20.0, 16, 0.5, 0.7, n_dec, seed)


def _pack16(P, layer):
    cfg = layer.cfg
    L = P.ProxLayer(cfg.d_model, cfg.d_ff, P.PROX_BF16, proxy16=True)
    wu, wg, wd = (to_device(w, "bf16") for w in (layer.w_up, layer.w_gate, layer.w_down))
    P.prox_pack_proxy(wu, wg, wd, L)
    P.prox_pack_proxy16(wu, wg, L)
    torch.cuda.synchronize()
    return L, L.with_proxy_kind(P.PROX_PROXY_W16)


def _ov16(ov):
    return ov["Wu"], ov["Wg"]


@pytest.mark.parametrize("d,f,seed", [(320, 384, 51), (64, 128, 52), (4096, 12288, None)])
def test_pack16_bit_exact(P, d, f, seed):
    layer = synth.make_layer(synth.CONFIGS["qwen3_8b"], n_dec=1, n_cal=1) if seed is None else \
        synth.make_layer(_cfg(d, f, seed, 1), n_dec=1)
    L, _ = _pack16(P, layer)
    got = L.proxy_w16.cpu().numpy()
    stride = P.prox_proxy16_size(d, f, P.PROX_BF16) // d
    rows = got.reshape(d, stride)
    wu = np.ascontiguousarray(layer.w_up).view(np.uint16).reshape(d, f // 16, 16)
    wg = np.ascontiguousarray(layer.w_gate).view(np.uint16).reshape(d, f // 16, 16)
    expect = np.concatenate([wu, wg], axis=2).reshape(d, 2 * f).view(np.uint8)
    assert np.array_equal(rows[:, : 4 * f], expect)
    assert not rows[:, 4 * f:].any()  # zero padding


def _decode_check(P, L16, layer, ov, tokens, tau_x, tau_s, label):
    x = to_device(layer.x_dec[tokens], "bf16")
    b = len(tokens)
    y = torch.full((b, L16.d_model), math.nan, dtype=torch.float32, device="cuda")
    mi = torch.full((b, L16.d_ff), -7, dtype=torch.int32, device="cuda")
    mc = torch.full((b,), -1, dtype=torch.int32, device="cuda")
    ic = torch.full((b,), -1, dtype=torch.int32, device="cuda")
    ws = P.new_workspace(L16.d_model, L16.d_ff, b)
    P.prox_ffn_decode(L16, x, tau_x, tau_s, y, mi, mc, ic, ws)
    torch.cuda.synchronize()
    y, mi, mc, ic = y.cpu().numpy(), mi.cpu().numpy(), mc.cpu().numpy(), ic.cpu().numpy()
    Wu, Wg = _ov16(ov)
    band = 0
    for k, t in enumerate(tokens):
        ref = oracle.decode_w16(ov["x_dec"][t], Wu, Wg, ov["Wd"], tau_x, tau_s)
        assert ic[k] == ref["k_x"], f"{label} token {t}: k_x"
        oob, inb, asc = band_compare(mi[k], int(mc[k]), ref["s_tilde"], tau_s)
        assert asc and oob == 0, f"{label} token {t}: {oob} channel(s) outside the band disagree"
        check_in_band(mi[k], int(mc[k]), ref["s_tilde"], tau_s, f"{label} token {t}")
        band += inb
        m = np.zeros(L16.d_ff, bool)
        m[mi[k][: mc[k]]] = True
        if not m.any():
            assert np.all(y[k] == 0.0)
            continue
        y_ref = oracle.stage2(ov["x_dec"][t], ov["Wu"], ov["Wg"], ov["Wd"], m)["y"]
        ma, rl = y_errors(y[k], y_ref)
        assert y_ok(y[k], y_ref), f"{label} token {t}: y max-abs {ma:.3e} rel-L2 {rl:.3e}"
    print(f"[{label}] k_x={list(ic)} k_s={list(mc)} in-band={band}")
    return mi, mc


@pytest.mark.parametrize("name", ["small", "qwen3_8b"])
def test_proxy16_state_decode_and_calibration(P, name):
    if name == "small":
        layer = synth.make_layer(_cfg(576, 1152, 53, 4), n_dec=4)
        ov = oracle_view(layer)
        n_cal = None
    else:
        layer, ov = oracle_layer("qwen3_8b")
        n_cal = 16
    L, L16 = _pack16(P, layer)
    Wu, Wg = _ov16(ov)
    xc = ov["x_cal"] if n_cal is None else ov["x_cal"][:n_cal]
    # proxy state of three tokens (batch 3 runs the per-token 16-bit kernel)
    tau_x = float(np.float32(np.median(np.abs(xc))))
    x = to_device(layer.x_dec[:3], "bf16")
    st = torch.empty(3, L.d_ff, dtype=torch.float32, device="cuda")
    ic = torch.empty(3, dtype=torch.int32, device="cuda")
    ws = P.new_workspace(L.d_model, L.d_ff, 3)
    P.prox_proxy_state(L16, x, tau_x, st, ic, ws)
    torch.cuda.synchronize()
    st, ic = st.cpu().numpy(), ic.cpu().numpy()
    for k in range(3):
        ref = oracle.proxy_state_w16(ov["x_dec"][k], Wu, Wg, tau_x)
        assert ic[k] == int(ref["m_x"].sum())
        scale = np.max(np.abs(ref["s"]))
        assert np.max(np.abs(st[k] - ref["s"])) <= 1e-5 * scale, f"{name} token {k}: s~"
    # calibration with the 16-bit proxy
    xcd = to_device(layer.x_cal if n_cal is None else layer.x_cal[:n_cal], "bf16")
    cws = torch.empty(P.prox_calibrate_workspace_size(L.d_model, L.d_ff, xcd.shape[0]), dtype=torch.uint8,
                      device="cuda")
    gx, gs = P.prox_calibrate(L16, xcd, 0.5, 0.7, cws)
    ox, os_ = oracle.calibrate_w16(xc, Wu, Wg, 0.5, 0.7)
    assert gx == ox and abs(gs - os_) <= 1e-5 * os_, f"{name}: tau ({gx}, {gs}) vs ({ox}, {os_})"
    # decode: batch 1 and batch 3, oracle thresholds
    _decode_check(P, L16, layer, ov, [0], ox, os_, f"{name}-w16-b1")
    mi16, mc16 = _decode_check(P, L16, layer, ov, [0, 1, 2], ox, os_, f"{name}-w16-b3")
    # tau_x depends only on the calibration inputs, not on the proxy
    ix, _ = oracle.calibrate(xc, ov["qu"], ov["su"], ov["qg"], ov["sg"], 0.5, 0.7)
    assert ix == ox


def test_proxy16_minimum_shape_and_degenerate(P):
    layer = synth.make_layer(_cfg(64, 128, 54, 2), n_dec=2)
    ov = oracle_view(layer)
    _, L16 = _pack16(P, layer)
    Wu, Wg = _ov16(ov)
    tx, ts = oracle.calibrate_w16(ov["x_cal"], Wu, Wg, 0.5, 0.7)
    _decode_check(P, L16, layer, ov, [0, 1], tx, ts, "64x128-w16")
    mi, mc = _decode_check(P, L16, layer, ov, [0], 0.0, 0.0, "w16-all-pass")
    assert mc[0] == 128
    mi, mc = _decode_check(P, L16, layer, ov, [1], math.inf, 1e-6, "w16-nothing")
    assert mc[0] == 0


def _sweep16(n=4, seed=2031):
    """Seeded bf16 layers and operating points for the 16-bit proxy: d_model a
    multiple of 64 up to 2048, d_ff a multiple of 128 up to 6144, 1 to 9
    tokens, keep_x and s2 off the headline point."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        out.append((64 * int(rng.integers(1, 33)), 128 * int(rng.integers(1, 49)), int(rng.integers(1, 10)),
                    float(rng.choice([0.2, 0.3, 0.5, 0.8])), float(rng.choice([0.4, 0.5, 0.7, 0.9])), 400 + i))
    return out


@pytest.mark.parametrize("d,f,b,keep_x,s2,seed", _sweep16())
def test_proxy16_decode_seeded_shape_sweep(P, d, f, b, keep_x, s2, seed):
    """Decode with the 16-bit proxy on seeded random shapes, batch sizes and
    operating points, thresholds from the oracle's 16-bit calibration."""
    layer = synth.make_layer(_cfg(d, f, seed, b), n_dec=b)
    ov = oracle_view(layer)
    _L, L16 = _pack16(P, layer)
    Wu, Wg = _ov16(ov)
    tau_x, tau_s = oracle.calibrate_w16(ov["x_cal"], Wu, Wg, keep_x, s2)
    _decode_check(P, L16, layer, ov, list(range(b)), tau_x, tau_s, f"w16 {d}x{f}-b{b}-k{keep_x}-s{s2}")
