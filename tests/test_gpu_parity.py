"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Comparison rules: packed codes, scales, input masks and counts bit-exact;
channel masks bit-exact outside a 1e-3 relative band around tau_s (in-band
disagreements are counted and printed); y within max-abs 2e-2 and relative
L2 1e-2 of the oracle, computed from the same channel list.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from prox_gpu_util import (band_compare, check_in_band, decode_proxy_bytes, oracle_layer, oracle_view,
                           pack_layer, to_device, y_errors, y_ok)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from free_ffn_activation_amd import prox
    return prox


def _small_cfg(d, f, dtype, seed, std=0.05, batch=1):
    return synth.LayerConfig(f"s{d}x{f}", d, f, dtype, std, max(1, d // 64), 20.0, 16, 0.5, 0.7,
                             batch, seed)


def _bufs(P, L, b):
    """Output buffers pre-filled with values no correct call leaves behind
    (y is NaN, so a y that was not cleared before accumulation shows)."""
    dev = "cuda"
    return (torch.full((b, L.d_model), math.nan, dtype=torch.float32, device=dev),
            torch.full((b, L.d_ff), -7, dtype=torch.int32, device=dev),
            torch.full((b,), -1, dtype=torch.int32, device=dev),
            torch.full((b,), -1, dtype=torch.int32, device=dev))


def _oracle_taus(ov, keep_x=0.5, sparsity_s=0.7, n_tok=None, act="silu"):
    xc = ov["x_cal"] if n_tok is None else ov["x_cal"][:n_tok]
    return oracle.calibrate(xc, ov["qu"], ov["su"], ov["qg"], ov["sg"], keep_x, sparsity_s, act=act)


def _run_decode(P, L, layer, ov, tokens, tau_x, tau_s, label, act="silu", stages=None):
    dt = layer.cfg.dtype
    x = to_device(layer.x_dec[tokens], dt)
    b = len(tokens)
    y, mi, mc, ic = _bufs(P, L, b)
    ws = P.new_workspace(L.d_model, L.d_ff, b)
    if stages is None:
        P.prox_ffn_decode(L, x, tau_x, tau_s, y, mi, mc, ic, ws)
    else:
        P.prox_ffn_decode_stages(L, x, tau_x, tau_s, y, mi, mc, ic, ws, stages)
    torch.cuda.synchronize()
    y, mi, mc, ic = y.cpu().numpy(), mi.cpu().numpy(), mc.cpu().numpy(), ic.cpu().numpy()
    total_band = 0
    for k, t in enumerate(tokens):
        ref = oracle.decode(ov["x_dec"][t], ov["Wu"], ov["Wg"], ov["Wd"], ov["qu"], ov["su"],
                            ov["qg"], ov["sg"], tau_x, tau_s, act=act)
        assert ic[k] == ref["k_x"], f"{label} token {t}: k_x {ic[k]} != {ref['k_x']}"
        oob, inb, asc = band_compare(mi[k], int(mc[k]), ref["s_tilde"], tau_s)
        assert asc, f"{label} token {t}: index list not ascending / in range"
        assert oob == 0, f"{label} token {t}: {oob} channel(s) outside the band disagree"
        check_in_band(mi[k], int(mc[k]), ref["s_tilde"], tau_s, f"{label} token {t}")
        total_band += inb
        # y against the oracle's Stage 2 on the GPU's own channel list
        m_gpu = np.zeros(L.d_ff, bool)
        m_gpu[mi[k][: mc[k]]] = True
        y_ref = oracle.stage2(ov["x_dec"][t], ov["Wu"], ov["Wg"], ov["Wd"], m_gpu, act=act)["y"]
        if not m_gpu.any():
            assert np.all(y[k] == 0.0)
        else:
            ma, rl = y_errors(y[k], y_ref)
            assert y_ok(y[k], y_ref), f"{label} token {t}: y max-abs {ma:.3e} rel-L2 {rl:.3e}"
    print(f"[{label}] tokens={list(tokens)} k_s={list(mc)} k_x={list(ic)} in-band={total_band}")
    return y, mi, mc, ic


# ------------------------------------------------------------------ packing
@pytest.mark.parametrize("name,d,f,dtype", [("tiny", 256, 768, "f32"),
                                            ("bf16-small", 320, 384, "bf16"),
                                            ("qwen3_8b", 4096, 12288, "bf16")])
def test_pack_bit_exact(P, name, d, f, dtype):
    if name in synth.CONFIGS:
        layer, ov = oracle_layer(name)
    else:
        layer = synth.make_layer(_small_cfg(d, f, dtype, 31))
        ov = oracle_view(layer)
    L = pack_layer(layer)
    q = L.proxy_q.cpu().numpy()
    up, gate, nib_ok = decode_proxy_bytes(q, d, f)
    assert nib_ok, "a nibble of 0 was written"
    assert np.array_equal(up, ov["qu"].astype(np.int16))
    assert np.array_equal(gate, ov["qg"].astype(np.int16))
    sc = L.proxy_scale.cpu().numpy()
    assert np.array_equal(sc[:d].view(np.uint32), ov["su"].view(np.uint32))
    assert np.array_equal(sc[d:].view(np.uint32), ov["sg"].view(np.uint32))
    wt = L.w_upgate_t.cpu().numpy().reshape(f, 2, d)
    wd = L.w_down.cpu().numpy().reshape(f, d)
    src_u = layer.w_up.view(np.int16) if dtype == "bf16" else layer.w_up
    src_g = layer.w_gate.view(np.int16) if dtype == "bf16" else layer.w_gate
    src_d = layer.w_down.view(np.int16) if dtype == "bf16" else layer.w_down
    assert np.array_equal(wt[:, 0, :], src_u.T)
    assert np.array_equal(wt[:, 1, :], src_g.T)
    assert np.array_equal(wd, src_d)


def test_pack_ties_and_zero_rows(P):
    d, f = 64, 128
    W = np.zeros((d, f), dtype=np.float32)
    W[1, :4] = np.array([7.0, 3.5, 2.5, -3.5]) * 2.0 ** -6
    W[2, :4] = np.array([-7.0, 0.5, -0.5, 1.5]) * 2.0 ** -3
    rng = np.random.default_rng(0)
    W[3:] = rng.standard_normal((d - 3, f)).astype(np.float32)
    Wd = rng.standard_normal((f, d)).astype(np.float32)
    L = P.ProxLayer(d, f, P.PROX_F32)
    P.prox_pack_proxy(to_device(W, "f32"), to_device(-W, "f32"), to_device(Wd, "f32"), L)
    torch.cuda.synchronize()
    up, gate, _ = decode_proxy_bytes(L.proxy_q.cpu().numpy(), d, f)
    qu, su = oracle.pack_proxy(W.astype(np.float64))
    qg, sg = oracle.pack_proxy(-W.astype(np.float64))
    assert np.array_equal(up, qu) and np.array_equal(gate, qg)
    assert list(up[1, :4]) == [7, 4, 2, -4] and np.all(up[0] == 0)
    sc = L.proxy_scale.cpu().numpy()
    assert sc[0] == 0 and np.array_equal(sc[:d], su) and np.array_equal(sc[d:], sg)


# ------------------------------------------------------------------ stage 1
@pytest.mark.parametrize("name", ["tiny", "qwen3_8b"])
def test_proxy_state_and_input_mask(P, name):
    layer, ov = oracle_layer(name)
    L = pack_layer(layer)
    cfg = layer.cfg
    tau_x = float(np.float32(np.median(np.abs(ov["x_cal"]))))
    tokens = [0, 1, 2]
    x = to_device(layer.x_dec[tokens], cfg.dtype)
    st = torch.empty(len(tokens), cfg.d_ff, dtype=torch.float32, device="cuda")
    ic = torch.empty(len(tokens), dtype=torch.int32, device="cuda")
    ws = P.new_workspace(cfg.d_model, cfg.d_ff, len(tokens))
    P.prox_proxy_state(L, x, tau_x, st, ic, ws)
    torch.cuda.synchronize()
    st, ic = st.cpu().numpy(), ic.cpu().numpy()
    for k, t in enumerate(tokens):
        ref = oracle.proxy_state(ov["x_dec"][t], ov["qu"], ov["su"], ov["qg"], ov["sg"], tau_x)
        assert ic[k] == int(ref["m_x"].sum())
        scale = np.max(np.abs(ref["s"]))
        err = np.max(np.abs(st[k] - ref["s"]))
        assert err <= 1e-5 * scale, f"token {t}: s~ error {err:.3e} vs scale {scale:.3e}"
    # second call on the same workspace: bit-identical (fixed reduction order)
    st2 = torch.empty(len(tokens), cfg.d_ff, dtype=torch.float32, device="cuda")
    P.prox_proxy_state(L, x, tau_x, st2, None, ws)
    torch.cuda.synchronize()
    assert np.array_equal(st2.cpu().numpy().view(np.uint32), st.view(np.uint32))


# ------------------------------------------------------------------ decode
@pytest.mark.parametrize("name,tokens", [("tiny", [0, 1, 2, 3]), ("qwen3_8b", [0, 1])])
def test_decode_parity(P, name, tokens):
    layer, ov = oracle_layer(name)
    L = pack_layer(layer)
    tau_x, tau_s = _oracle_taus(ov, n_tok=None if name == "tiny" else 16)
    for t in tokens:
        _run_decode(P, L, layer, ov, [t], tau_x, tau_s, f"{name}")


@pytest.fixture(scope="module")
def layer8b(P):
    layer, ov = oracle_layer("qwen3_8b")
    return layer, ov, pack_layer(layer)


# Operating points the benchmark times beside the headline (keep_x 0.5,
# s2 0.7): the 36-layer sweep's s2 = 0.5 and 0.6, the pages' own point from
# the computation-budget section (e = 0.7 at s1 = 0.7 with alpha = 1/3 gives
# s2 = 0.7667, keep_x = 0.3), and the allocator's point for e = 0.7 at s1 = 0.7
# with the alpha measured on MI355X (0.7593: s2 = 0.8519).  Thresholds are the
# oracle's, calibrated on 16 tokens; keep_x 0.3 is not exact in fp32.
@pytest.mark.parametrize("keep_x,s2", [(0.5, 0.5), (0.5, 0.6), (0.3, 0.7667), (0.3, 0.8519)])
def test_decode_operating_points_8b(P, layer8b, keep_x, s2):
    layer, ov, L = layer8b
    if s2 == 0.8519:
        assert abs(oracle.stage2_sparsity_for_target(0.7, 0.7, 0.7593) - s2) < 5e-5
        assert abs(P.prox_budget_s2(0.7, 0.7, 0.7593) - s2) < 5e-5
    if s2 == 0.7667:
        assert abs(oracle.stage2_sparsity_for_target(0.7, 0.7, 1.0 / 3.0) - s2) < 5e-5
    tau_x, tau_s = _oracle_taus(ov, keep_x=keep_x, sparsity_s=s2, n_tok=16)
    _y, _mi, mc, ic = _run_decode(P, L, layer, ov, [0, 1], tau_x, tau_s, f"8b keep_x={keep_x} s2={s2}")
    # the runtime keep fractions land near the calibrated ones (16 tokens)
    assert abs(float(np.mean(ic)) / L.d_model - keep_x) < 0.05
    assert abs(float(np.mean(mc)) / L.d_ff - (1.0 - s2)) < 0.05


def test_calibrate_keep_fraction_fp32(P):
    """keep_x = 0.3 with N a multiple of 10 (320 x 16 = 5120 fp32 values): the
    library counts ceil(fp32(0.3) N) = 1537, as does the oracle; tau_x is
    bit-exact, tau_s within 1e-5."""
    layer = synth.make_layer(_small_cfg(320, 384, "f32", 47), n_dec=1)
    ov = oracle_view(layer)
    L = pack_layer(layer)
    xc = to_device(layer.x_cal, "f32")              # fp32 Laplace draws: no ties
    assert xc.shape[0] * 320 == 5120
    ws = torch.empty(P.prox_calibrate_workspace_size(320, 384, xc.shape[0]), dtype=torch.uint8, device="cuda")
    tx, ts = P.prox_calibrate(L, xc, 0.3, 0.7667, ws)
    rx, rs = _oracle_taus(ov, 0.3, 0.7667)
    assert np.float32(tx) == np.float32(rx)
    assert abs(ts - rs) <= 1e-5 * rs
    assert int(np.sum(np.abs(ov["x_cal"]) >= rx)) == 1537


def test_decode_batch8_per_token_masks(P):
    layer, ov = oracle_layer("qwen3_8b_batch8", n_dec=8, n_cal=16)
    L = pack_layer(layer)
    tau_x, tau_s = _oracle_taus(ov)
    y, mi, mc, ic = _run_decode(P, L, layer, ov, list(range(8)), tau_x, tau_s, "batch8")
    assert len(set(int(v) for v in mc)) > 1  # masks really are per token


def test_decode_qwen3_32b(P):
    cfg = synth.CONFIGS["qwen3_32b"]
    layer = synth.make_layer(cfg, n_dec=2, n_cal=8)
    ov = oracle_view(layer)
    L = pack_layer(layer)
    tau_x, tau_s = _oracle_taus(ov)
    _run_decode(P, L, layer, ov, [0], tau_x, tau_s, "qwen3_32b")


def test_decode_ragged_small_shapes(P):
    """Shapes off the large power-of-two grid: partial column slices (d = 320),
    few panels (f = 384), minimum sizes (64 x 128), bf16 and fp32."""
    for (d, f, dt, seed) in [(320, 384, "bf16", 41), (64, 128, "f32", 42), (576, 1152, "bf16", 43),
                             (192, 640, "f32", 44)]:
        layer = synth.make_layer(_small_cfg(d, f, dt, seed), n_dec=3)
        ov = oracle_view(layer)
        L = pack_layer(layer)
        tau_x, tau_s = _oracle_taus(ov)
        _run_decode(P, L, layer, ov, [0, 1, 2], tau_x, tau_s, f"{d}x{f}-{dt}")


def test_decode_wide_dff_bitmap_chunks(P):
    """d_ff = 33024: the up/gate waves hold the first two 16384-channel chunks
    of the Stage-1 bitmap in registers and read the third from memory when
    they count and select; the all-pass case gives each wave three ordinals
    (the later ones re-read every chunk), and both batch 1 and a group of
    four (grouped kernels, union passes over 1032 bitmap words)."""
    layer = synth.make_layer(_small_cfg(128, 33024, "bf16", 45), n_dec=4)
    ov = oracle_view(layer)
    L = pack_layer(layer)
    tau_x, tau_s = _oracle_taus(ov)
    _run_decode(P, L, layer, ov, [0], tau_x, tau_s, "128x33024")
    _run_decode(P, L, layer, ov, [1, 2, 3, 0], tau_x, tau_s, "128x33024-b4")
    y, mi, mc, ic = _run_decode(P, L, layer, ov, [2], 0.0, 0.0, "128x33024-all-pass")
    assert mc[0] == L.d_ff and np.array_equal(mi[0], np.arange(L.d_ff))


def test_decode_max_d_model(P):
    """d_model = 12288, the largest shape: every up/gate thread stages its six
    16-byte chunks of x, a channel's run takes three 8-step load batches, the
    down kernel covers 24 column slices; batch 1 and a grouped batch of 3."""
    layer = synth.make_layer(_small_cfg(12288, 256, "bf16", 46), n_dec=4)
    ov = oracle_view(layer)
    L = pack_layer(layer)
    tau_x, tau_s = _oracle_taus(ov)
    _run_decode(P, L, layer, ov, [0], tau_x, tau_s, "12288x256")
    _run_decode(P, L, layer, ov, [1, 2, 3], tau_x, tau_s, "12288x256-b3")


def test_decode_max_d_ff(P):
    """d_ff = 65536, the largest: four 16384-channel bitmap chunks (two held
    in registers by every up/gate wave, two re-read), 512 Stage-1 panels, the
    grouped kernels' union scan over 2048 words in 8 passes; batch 1, a
    grouped batch of 3 and the all-pass case."""
    layer = synth.make_layer(_small_cfg(128, 65536, "bf16", 47), n_dec=4)
    ov = oracle_view(layer)
    L = pack_layer(layer)
    tau_x, tau_s = _oracle_taus(ov)
    _run_decode(P, L, layer, ov, [0], tau_x, tau_s, "128x65536")
    _run_decode(P, L, layer, ov, [1, 2, 3], tau_x, tau_s, "128x65536-b3")
    y, mi, mc, ic = _run_decode(P, L, layer, ov, [2], 0.0, 0.0, "128x65536-all-pass")
    assert mc[0] == L.d_ff and np.array_equal(mi[0], np.arange(L.d_ff))


def test_decode_max_d_model_f32(P):
    """d_model = 12288 with fp32 weights: x staged by the up/gate kernel takes
    48 KB of LDS and the down kernel's column slices are 256 wide (48 of
    them); batch 1 and two tokens (per-token kernels: fp32 groups run Stage 2
    per token)."""
    layer = synth.make_layer(_small_cfg(12288, 256, "f32", 48), n_dec=3)
    ov = oracle_view(layer)
    L = pack_layer(layer)
    tau_x, tau_s = _oracle_taus(ov)
    _run_decode(P, L, layer, ov, [0], tau_x, tau_s, "12288x256-f32")
    _run_decode(P, L, layer, ov, [1, 2], tau_x, tau_s, "12288x256-f32-b2")


def _sweep_cases(n=12, seed=2027):
    """Seeded draws of valid layers and operating points: d_model a multiple of
    64 up to 2048, d_ff a multiple of 128 up to 6144, bf16 or fp32, 1 to 9
    tokens (so groups of 1, 2, 3.. 8 and 8 + 1 all occur), keep_x and s2 off
    the headline point."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        d = 64 * int(rng.integers(1, 33))
        f = 128 * int(rng.integers(1, 49))
        dt = "bf16" if rng.random() < 0.7 else "f32"
        b = int(rng.integers(1, 10))
        keep_x = float(rng.choice([0.2, 0.3, 0.5, 0.8]))
        s2 = float(rng.choice([0.4, 0.5, 0.7, 0.9]))
        cases.append((d, f, dt, b, keep_x, s2, 300 + i))
    return cases


@pytest.mark.parametrize("d,f,dt,b,keep_x,s2,seed", _sweep_cases())
def test_decode_seeded_shape_sweep(P, d, f, dt, b, keep_x, s2, seed):
    """Decode parity on seeded random shapes, dtypes, batch sizes and
    operating points (default dispatch: per-token or grouped kernels by group
    size), every token against the oracle under the band rule."""
    layer = synth.make_layer(_small_cfg(d, f, dt, seed), n_dec=b)
    ov = oracle_view(layer)
    L = pack_layer(layer)
    tau_x, tau_s = _oracle_taus(ov, keep_x=keep_x, sparsity_s=s2)
    _run_decode(P, L, layer, ov, list(range(b)), tau_x, tau_s, f"{d}x{f}-{dt}-b{b}-k{keep_x}-s{s2}")


@pytest.mark.parametrize("d,f,dt,b,keep_x,s2,seed", _sweep_cases(n=4, seed=2029))
def test_geglu_decode_seeded_shape_sweep(P, d, f, dt, b, keep_x, s2, seed):
    """The seeded sweep for GeGLU layers (GELU-tanh gate)."""
    layer = synth.make_layer(_small_cfg(d, f, dt, seed), n_dec=b)
    ov = oracle_view(layer)
    L = pack_layer(layer, activation=P.PROX_ACT_GELU_TANH)
    tau_x, tau_s = _oracle_taus(ov, keep_x=keep_x, sparsity_s=s2, act=GELU)
    _run_decode(P, L, layer, ov, list(range(b)), tau_x, tau_s, f"geglu {d}x{f}-{dt}-b{b}", act=GELU)


def test_decode_degenerate_thresholds(P):
    layer, ov = oracle_layer("tiny")
    L = pack_layer(layer)
    d, f = L.d_model, L.d_ff
    # all-pass: dense SwiGLU
    y, mi, mc, ic = _run_decode(P, L, layer, ov, [0], 0.0, 0.0, "all-pass")
    assert mc[0] == f and ic[0] == d and np.array_equal(mi[0], np.arange(f))
    # no input kept and tau_s > 0: empty channel mask, y = 0
    y, mi, mc, ic = _run_decode(P, L, layer, ov, [1], math.inf, 1e-6, "no-input")
    assert ic[0] == 0 and mc[0] == 0 and np.all(y == 0)
    # no input kept but tau_s = 0: every channel, exact dense Stage 2
    y, mi, mc, ic = _run_decode(P, L, layer, ov, [1], math.inf, 0.0, "no-input-all-channels")
    assert mc[0] == f
    # tau_s = +inf: empty channel mask
    y, mi, mc, ic = _run_decode(P, L, layer, ov, [2], 0.0, math.inf, "empty")
    assert mc[0] == 0 and np.all(y == 0)


def test_decode_repeatable_masks(P):
    layer, ov = oracle_layer("qwen3_8b")
    L = pack_layer(layer)
    tau_x, tau_s = _oracle_taus(ov, n_tok=16)
    x = to_device(layer.x_dec[[3]], "bf16")
    ws = P.new_workspace(L.d_model, L.d_ff, 1)
    outs = []
    for _ in range(3):
        y, mi, mc, ic = _bufs(P, L, 1)
        P.prox_ffn_decode(L, x, tau_x, tau_s, y, mi, mc, ic, ws)
        torch.cuda.synchronize()
        outs.append((y.cpu().numpy(), mi.cpu().numpy(), int(mc.item())))
    for y, mi, mc in outs[1:]:
        assert mc == outs[0][2] and np.array_equal(mi[0, :mc], outs[0][1][0, :mc])
        ma, rl = y_errors(y[0], outs[0][0][0].astype(np.float64))
        assert rl < 1e-6


# ------------------------------------------------------------------ stage 2 alone
@pytest.mark.parametrize("name", ["tiny", "qwen3_8b"])
def test_stage2_from_oracle_mask(P, name):
    layer, ov = oracle_layer(name)
    L = pack_layer(layer)
    cfg = layer.cfg
    tau_x, tau_s = _oracle_taus(ov, n_tok=None if name == "tiny" else 16)
    tokens = [4, 5]
    b = len(tokens)
    J = np.zeros((b, cfg.d_ff), dtype=np.int32)
    cnt = np.zeros(b, dtype=np.int32)
    refs = []
    for k, t in enumerate(tokens):
        ref = oracle.decode(ov["x_dec"][t], ov["Wu"], ov["Wg"], ov["Wd"], ov["qu"], ov["su"],
                            ov["qg"], ov["sg"], tau_x, tau_s)
        cnt[k] = ref["k_s"]
        J[k, : ref["k_s"]] = ref["J"]
        refs.append(ref)
    x = to_device(layer.x_dec[tokens], cfg.dtype)
    y = torch.empty(b, cfg.d_model, dtype=torch.float32, device="cuda")
    ws = P.new_workspace(cfg.d_model, cfg.d_ff, b)
    P.prox_ffn_stage2(L, x, torch.from_numpy(J).cuda(), torch.from_numpy(cnt).cuda(), y, ws)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    for k in range(b):
        ma, rl = y_errors(y[k], refs[k]["y"])
        print(f"[stage2 {name}] token {tokens[k]} k_s={cnt[k]} max-abs={ma:.3e} rel-L2={rl:.3e}")
        assert y_ok(y[k], refs[k]["y"])


def test_stage2_skips_out_of_range_indices(P):
    layer, ov = oracle_layer("tiny")
    L = pack_layer(layer)
    f = L.d_ff
    J = np.array([[3, -5, 17, f + 9, 40] + [0] * (f - 5)], dtype=np.int32)
    cnt = np.array([5], dtype=np.int32)
    x = to_device(layer.x_dec[[0]], "f32")
    y = torch.empty(1, L.d_model, dtype=torch.float32, device="cuda")
    ws = P.new_workspace(L.d_model, f, 1)
    P.prox_ffn_stage2(L, x, torch.from_numpy(J).cuda(), torch.from_numpy(cnt).cuda(), y, ws)
    torch.cuda.synchronize()
    m = np.zeros(f, bool)
    m[[3, 17, 40]] = True
    y_ref = oracle.stage2(ov["x_dec"][0], ov["Wu"], ov["Wg"], ov["Wd"], m)["y"]
    assert y_ok(y.cpu().numpy()[0], y_ref)


# ------------------------------------------------------------------ calibration
@pytest.mark.parametrize("name,n_tok", [("tiny", 64), ("qwen3_8b", 16)])
def test_calibrate_parity(P, name, n_tok):
    layer, ov = oracle_layer(name)
    L = pack_layer(layer)
    cfg = layer.cfg
    xc = to_device(layer.x_cal[:n_tok], cfg.dtype)
    ws = torch.empty(P.prox_calibrate_workspace_size(cfg.d_model, cfg.d_ff, n_tok),
                     dtype=torch.uint8, device="cuda")
    tx, ts = P.prox_calibrate(L, xc, cfg.keep_x, cfg.sparsity_s, ws)
    rx, rs = _oracle_taus(ov, cfg.keep_x, cfg.sparsity_s, n_tok=n_tok)
    print(f"[calibrate {name}] tau_x gpu={tx!r} oracle={rx!r}  tau_s gpu={ts!r} oracle={rs!r}")
    assert np.float32(tx) == np.float32(rx)
    assert abs(ts - rs) <= 1e-5 * rs
    # edge fractions: keep everything / nothing
    tx0, ts0 = P.prox_calibrate(L, xc, 1.0, 0.0, ws)
    assert tx0 == float(np.min(np.abs(ov["x_cal"][:n_tok]))) and ts0 >= 0.0
    tx1, ts1 = P.prox_calibrate(L, xc, 0.0, 1.0, ws)
    assert math.isinf(tx1) and math.isinf(ts1)


def _calib_cases(n=8, seed=2035):
    """Seeded layers, calibration-set sizes and keep fractions (n_keep at
    both ends of the range and off round numbers of the fp32 keep value)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = 64 * int(rng.integers(1, 33))
        f = 128 * int(rng.integers(1, 49))
        dt = "bf16" if rng.random() < 0.6 else "f32"
        n_tok = int(rng.integers(1, 25))
        keep_x = float(rng.choice([0.01, 0.1, 0.3, 0.37, 0.5, 0.9, 0.99]))
        s2 = float(rng.choice([0.05, 0.3, 0.7, 0.85, 0.97]))
        out.append((d, f, dt, n_tok, keep_x, s2, 500 + i))
    return out


@pytest.mark.parametrize("d,f,dt,n_tok,keep_x,s2,seed", _calib_cases())
def test_calibrate_seeded_sweep(P, d, f, dt, n_tok, keep_x, s2, seed):
    """prox_calibrate on seeded shapes, calibration-set sizes (1 to 24
    tokens) and keep fractions from 1% to 99%: tau_x bit-exact and tau_s
    within 1e-5 relative of the oracle's order statistics."""
    layer = synth.make_layer(_small_cfg(d, f, dt, seed), n_dec=1, n_cal=24)
    ov = oracle_view(layer)
    L = pack_layer(layer)
    xc = to_device(layer.x_cal[:n_tok], dt)
    ws = torch.empty(P.prox_calibrate_workspace_size(d, f, n_tok), dtype=torch.uint8, device="cuda")
    tx, ts = P.prox_calibrate(L, xc, keep_x, s2, ws)
    rx, rs = _oracle_taus(ov, keep_x, s2, n_tok=n_tok)
    assert np.float32(tx) == np.float32(rx), f"tau_x {tx!r} vs {rx!r}"
    assert abs(ts - rs) <= 1e-5 * abs(rs), f"tau_s {ts!r} vs {rs!r}"


# ------------------------------------------------------------------ graph replay
@pytest.mark.parametrize("name", ["tiny", "qwen3_8b"])
def test_graph_replay_matches_eager(P, name):
    """prox_ffn_decode captured in a HIP graph: every replay (with eager work and
    synchronisations in between) reproduces the eager masks and y."""
    layer, ov = oracle_layer(name)
    L = pack_layer(layer)
    cfg = layer.cfg
    tau_x, tau_s = _oracle_taus(ov, n_tok=None if name == "tiny" else 16)
    toks = [0, 1, 2]
    xs = [to_device(layer.x_dec[[t]], cfg.dtype) for t in toks]
    ws = P.new_workspace(cfg.d_model, cfg.d_ff, 1)
    outs = [_bufs(P, L, 1) for _ in toks]
    eager = []
    for x in xs:
        y, mi, mc, ic = _bufs(P, L, 1)
        P.prox_ffn_decode(L, x, tau_x, tau_s, y, mi, mc, ic, ws)
        torch.cuda.synchronize()
        eager.append((y.cpu().numpy(), mi.cpu().numpy(), int(mc.item()), int(ic.item())))
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for x, (y, mi, mc, ic) in zip(xs, outs):
            P.prox_ffn_decode(L, x, tau_x, tau_s, y, mi, mc, ic, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for x, (y, mi, mc, ic) in zip(xs, outs):
            P.prox_ffn_decode(L, x, tau_x, tau_s, y, mi, mc, ic, ws)
    for rep in range(4):
        for (y, mi, mc, ic) in outs:
            y.fill_(123.0)
            mc.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        for k, (y, mi, mc, ic) in enumerate(outs):
            ey, emi, emc, eic = eager[k]
            assert int(mc.item()) == emc and int(ic.item()) == eic, f"replay {rep} token {k}"
            assert np.array_equal(mi.cpu().numpy()[0, :emc], emi[0, :emc])
            ma, rl = y_errors(y.cpu().numpy()[0], ey[0].astype(np.float64))
            assert rl <= 1e-6, f"replay {rep} token {k}: rel {rl:.2e}"
        # eager work on the same workspace between replays
        yy, mi2, mc2, ic2 = _bufs(P, L, 1)
        P.prox_ffn_decode(L, xs[rep % len(xs)], tau_x, tau_s, yy, mi2, mc2, ic2, ws)
        torch.cuda.synchronize()
        assert int(mc2.item()) == eager[rep % len(xs)][2]
    del g


def test_decode_back_to_back_calls(P):
    """Many stream-ordered calls on one workspace with no host synchronisation
    in between (each call leaves the workspace ready for the next): every
    call's outputs match the same token decoded alone."""
    layer, ov = oracle_layer("qwen3_8b")
    L = pack_layer(layer)
    tau_x, tau_s = _oracle_taus(ov, n_tok=16)
    toks = [0, 1, 2, 3]
    xs = [to_device(layer.x_dec[[t]], "bf16") for t in toks]
    ws = P.new_workspace(L.d_model, L.d_ff, 1)
    alone = []
    for x in xs:
        y, mi, mc, ic = _bufs(P, L, 1)
        P.prox_ffn_decode(L, x, tau_x, tau_s, y, mi, mc, ic, P.new_workspace(L.d_model, L.d_ff, 1))
        torch.cuda.synchronize()
        alone.append((y.cpu().numpy(), mi.cpu().numpy(), int(mc.item()), int(ic.item())))
    n_calls = 48
    outs = [_bufs(P, L, 1) for _ in range(n_calls)]
    for c in range(n_calls):
        y, mi, mc, ic = outs[c]
        P.prox_ffn_decode(L, xs[c % len(xs)], tau_x, tau_s, y, mi, mc, ic, ws)
    torch.cuda.synchronize()
    for c in range(n_calls):
        y, mi, mc, ic = outs[c]
        ey, emi, emc, eic = alone[c % len(xs)]
        assert int(mc.item()) == emc and int(ic.item()) == eic, f"call {c}"
        assert np.array_equal(mi.cpu().numpy()[0, :emc], emi[0, :emc]), f"call {c}"
        ma, rl = y_errors(y.cpu().numpy()[0], ey[0].astype(np.float64))
        assert rl <= 1e-6, f"call {c}: rel {rl:.2e}"


def test_decode_stages_compose(P):
    """Stages run one at a time on the same workspace give prox_ffn_decode."""
    layer, ov = oracle_layer("qwen3_8b")
    L = pack_layer(layer)
    tau_x, tau_s = _oracle_taus(ov, n_tok=16)
    x = to_device(layer.x_dec[[5]], "bf16")
    ws = P.new_workspace(L.d_model, L.d_ff, 1)
    y, mi, mc, ic = _bufs(P, L, 1)
    P.prox_ffn_decode(L, x, tau_x, tau_s, y, mi, mc, ic, ws)
    torch.cuda.synchronize()
    ref = (y.cpu().numpy(), mi.cpu().numpy(), int(mc.item()), int(ic.item()))
    ws2 = P.new_workspace(L.d_model, L.d_ff, 1)
    y2, mi2, mc2, ic2 = _bufs(P, L, 1)
    for bit in (P.PROX_STAGE_PROXY, P.PROX_STAGE_UPGATE, P.PROX_STAGE_DOWN):
        P.prox_ffn_decode_stages(L, x, tau_x, tau_s, y2, mi2, mc2, ic2, ws2, bit)
        torch.cuda.synchronize()
    assert int(mc2.item()) == ref[2] and int(ic2.item()) == ref[3]
    assert np.array_equal(mi2.cpu().numpy()[0, :ref[2]], ref[1][0, :ref[2]])
    ma, rl = y_errors(y2.cpu().numpy()[0], ref[0][0].astype(np.float64))
    assert rl <= 1e-6
    # replaying the up/gate stage alone re-derives the same list from the bitmap
    P.prox_ffn_decode_stages(L, x, tau_x, tau_s, y2, mi2, mc2, ic2, ws2, P.PROX_STAGE_UPGATE)
    torch.cuda.synchronize()
    assert int(mc2.item()) == ref[2] and np.array_equal(mi2.cpu().numpy()[0, :ref[2]], ref[1][0, :ref[2]])


# ------------------------------------------------------------------ GeGLU layers
GELU = "gelu_tanh"


@pytest.mark.parametrize("name,tokens", [("tiny", [0, 1, 2]), ("qwen3_8b", [0, 1])])
def test_geglu_decode_parity(P, name, tokens):
    """A GeGLU layer (GELU-tanh gate) through the same kernels: masks, k_x and
    y against the oracle with the same activation."""
    layer, ov = oracle_layer(name)
    L = pack_layer(layer, activation=P.PROX_ACT_GELU_TANH)
    tau_x, tau_s = _oracle_taus(ov, n_tok=None if name == "tiny" else 16, act=GELU)
    _run_decode(P, L, layer, ov, tokens, tau_x, tau_s, f"geglu {name}", act=GELU)


def test_geglu_proxy_state_stage2_and_calibration(P):
    layer, ov = oracle_layer("tiny")
    L = pack_layer(layer, activation=P.PROX_ACT_GELU_TANH)
    cfg = layer.cfg
    # proxy state
    tau_x = float(np.float32(np.median(np.abs(ov["x_cal"]))))
    x = to_device(layer.x_dec[[0, 1]], cfg.dtype)
    st = torch.empty(2, cfg.d_ff, dtype=torch.float32, device="cuda")
    ws = P.new_workspace(cfg.d_model, cfg.d_ff, 2)
    P.prox_proxy_state(L, x, tau_x, st, None, ws)
    torch.cuda.synchronize()
    for k in range(2):
        ref = oracle.proxy_state(ov["x_dec"][k], ov["qu"], ov["su"], ov["qg"], ov["sg"], tau_x, act=GELU)
        assert np.max(np.abs(st.cpu().numpy()[k] - ref["s"])) <= 1e-5 * np.max(np.abs(ref["s"]))
    # Stage 2 from the oracle's GeGLU channel list
    tau_x, tau_s = _oracle_taus(ov, act=GELU)
    ref = oracle.decode(ov["x_dec"][3], ov["Wu"], ov["Wg"], ov["Wd"], ov["qu"], ov["su"],
                        ov["qg"], ov["sg"], tau_x, tau_s, act=GELU)
    J = np.zeros((1, cfg.d_ff), dtype=np.int32)
    J[0, : ref["k_s"]] = ref["J"]
    cnt = np.array([ref["k_s"]], dtype=np.int32)
    y = torch.empty(1, cfg.d_model, dtype=torch.float32, device="cuda")
    P.prox_ffn_stage2(L, to_device(layer.x_dec[[3]], cfg.dtype), torch.from_numpy(J).cuda(),
                      torch.from_numpy(cnt).cuda(), y, ws)
    torch.cuda.synchronize()
    assert y_ok(y.cpu().numpy()[0], ref["y"])
    # calibration: tau_x is activation-free (bit-exact), tau_s uses GELU
    xc = to_device(layer.x_cal, cfg.dtype)
    cws = torch.empty(P.prox_calibrate_workspace_size(cfg.d_model, cfg.d_ff, xc.shape[0]),
                      dtype=torch.uint8, device="cuda")
    tx, ts = P.prox_calibrate(L, xc, cfg.keep_x, cfg.sparsity_s, cws)
    assert np.float32(tx) == np.float32(tau_x) and abs(ts - tau_s) <= 1e-5 * tau_s
    sw_x, sw_s = _oracle_taus(ov)
    assert abs(sw_s - tau_s) > 1e-3 * tau_s  # the SwiGLU threshold differs


# ------------------------------------------------------------------ histogram calibration
def _bin_width(values, n_bins):
    a = np.abs(np.asarray(values, dtype=np.float64)).astype(np.float32)
    return float(np.float32(np.float32(a.max()) / np.float32(n_bins)))


@pytest.mark.parametrize("name,n_tok,max_samples", [("tiny", 64, 200000), ("qwen3_8b", 16, 50000)])
def test_calibrate_hist_parity(P, name, n_tok, max_samples):
    """tau_x bit-exact (the same strided samples of exact values, fp32 bin
    decisions); tau_s within one bin of the oracle's (its samples are fp32
    GPU proxy states against the oracle's fp64 ones)."""
    layer, ov = oracle_layer(name)
    L = pack_layer(layer)
    cfg = layer.cfg
    nb = 4096
    xc = to_device(layer.x_cal[:n_tok], cfg.dtype)
    ws = torch.empty(P.prox_calibrate_hist_workspace_size(cfg.d_model, cfg.d_ff, n_tok, max_samples, nb),
                     dtype=torch.uint8, device="cuda")
    tx, ts = P.prox_calibrate_hist(L, xc, cfg.keep_x, cfg.sparsity_s, ws, max_samples, nb)
    Xc = ov["x_cal"][:n_tok]
    rx, rs = oracle.calibrate_hist(Xc, ov["qu"], ov["su"], ov["qg"], ov["sg"], cfg.keep_x, cfg.sparsity_s,
                                   max_samples=max_samples, n_bins=nb)
    pool = np.concatenate([oracle.proxy_state(Xc[t], ov["qu"], ov["su"], ov["qg"], ov["sg"], rx)["s"]
                           for t in range(n_tok)])
    ws_bin = _bin_width(oracle.strided_sample(np.abs(pool), max_samples), nb)
    print(f"[calibrate_hist {name}] tau_x gpu={tx!r} oracle={rx!r}  tau_s gpu={ts!r} oracle={rs!r} bin={ws_bin:.3e}")
    assert np.float32(tx) == np.float32(rx)
    assert abs(ts - rs) <= 1.01 * ws_bin
    # edges: keep everything -> 0, keep nothing -> +inf
    tx0, ts0 = P.prox_calibrate_hist(L, xc, 1.0, 0.0, ws, max_samples, nb)
    assert tx0 == 0.0 and ts0 == 0.0
    tx1, ts1 = P.prox_calibrate_hist(L, xc, 0.0, 1.0, ws, max_samples, nb)
    assert math.isinf(tx1) and math.isinf(ts1)


def test_depth_ordered_calibration_on_a_chain(P):
    """The pages calibrate layer by layer in depth order, each on the previous
    layers' sparse outputs.  A chain of three tiny fp32 layers with a residual
    stream, h_{l+1} = h_l + y_l, x_{l+1} = RMSNorm(h_{l+1}): per-layer
    thresholds within one histogram bin of the oracle's chain, the first
    layer's tau_x bit-exact."""
    nb, ms = 4096, 200000
    cfg = synth.CONFIGS["tiny"]
    layers = [synth.make_layer(cfg, l, n_dec=2) for l in range(3)]
    X = synth.as_f64(layers[0].x_cal, "f32")            # the chain's input
    Xg = to_device(layers[0].x_cal, "f32")
    H, Hg = X.copy(), Xg.clone()
    n = X.shape[0]
    ws_cal = torch.empty(P.prox_calibrate_hist_workspace_size(cfg.d_model, cfg.d_ff, n, ms, nb),
                         dtype=torch.uint8, device="cuda")
    ws = P.new_workspace(cfg.d_model, cfg.d_ff, n)
    y = torch.empty(n, cfg.d_model, dtype=torch.float32, device="cuda")
    mi = torch.empty(n, cfg.d_ff, dtype=torch.int32, device="cuda")
    mc = torch.empty(n, dtype=torch.int32, device="cuda")
    for l, lay in enumerate(layers):
        ov = oracle_view(lay)
        L = pack_layer(lay)
        tx, ts = P.prox_calibrate_hist(L, Xg, cfg.keep_x, cfg.sparsity_s, ws_cal, ms, nb)
        rx, rs = oracle.calibrate_hist(X, ov["qu"], ov["su"], ov["qg"], ov["sg"], cfg.keep_x, cfg.sparsity_s,
                                       max_samples=ms, n_bins=nb)
        wx = _bin_width(X, nb)
        pool = np.concatenate([oracle.proxy_state(X[t], ov["qu"], ov["su"], ov["qg"], ov["sg"], rx)["s"]
                               for t in range(n)])
        wsb = _bin_width(pool, nb)
        print(f"[chain layer {l}] tau_x {tx!r}/{rx!r} tau_s {ts!r}/{rs!r}")
        if l == 0:
            assert np.float32(tx) == np.float32(rx)
        assert abs(tx - rx) <= 1.01 * wx and abs(ts - rs) <= 1.01 * wsb
        # this layer's sparse outputs feed the next layer's calibration
        P.prox_ffn_decode(L, Xg, tx, ts, y, mi, mc, None, ws)
        torch.cuda.synchronize()
        Hg = Hg + y
        Xg = (Hg * torch.rsqrt(torch.mean(Hg * Hg, dim=-1, keepdim=True) + 1e-6)).contiguous()
        Y = np.stack([oracle.decode(X[t], ov["Wu"], ov["Wg"], ov["Wd"], ov["qu"], ov["su"], ov["qg"], ov["sg"],
                                    rx, rs)["y"] for t in range(n)])
        H = H + Y
        X = (H / np.sqrt(np.mean(H * H, axis=-1, keepdims=True) + 1e-6)).astype(np.float32).astype(np.float64)


# ------------------------------------------------------------------ fused Stage 2 (batch 1)
def test_fused_and_split_stage2_agree(P, layer8b):
    """Batch 1 runs the up/gate and down kernels as two launches;
    PROX_STAGE_FUSED_STAGE2 runs them as one.  Same masks and counts, y equal
    up to the order of the fp32 atomic additions."""
    layer, ov, L = layer8b
    tau_x, tau_s = _oracle_taus(ov, n_tok=16)
    ws = P.new_workspace(L.d_model, L.d_ff, 1)
    for t in range(4):
        x = to_device(layer.x_dec[[t]], "bf16")
        a, b = _bufs(P, L, 1), _bufs(P, L, 1)
        P.prox_ffn_decode(L, x, tau_x, tau_s, *a, ws)
        P.prox_ffn_decode_stages(L, x, tau_x, tau_s, *b, ws, 7 | P.PROX_STAGE_FUSED_STAGE2)
        torch.cuda.synchronize()
        (ya, mia, mca, ica), (yb, mib, mcb, icb) = ([v.cpu().numpy() for v in o] for o in (a, b))
        n = int(mca[0])
        assert n == int(mcb[0]) and int(ica[0]) == int(icb[0]) and np.array_equal(mia[0, :n], mib[0, :n])
        assert y_errors(ya[0], yb[0].astype(np.float64))[1] <= 1e-6
    P.prox_workspace_check(ws)  # no bounded wait gave up


@pytest.mark.parametrize("d,f,dt,seed", [(256, 768, "f32", 101), (320, 384, "bf16", 41), (12288, 256, "bf16", 46),
                                         (12288, 256, "f32", 48), (128, 33024, "bf16", 45),
                                         (128, 65536, "bf16", 47)])
def test_fused_stage2_parity_shapes(P, d, f, dt, seed):
    """The fused Stage-2 kernel against the oracle on fp32, a partial column
    slice, the largest d_model (bf16 and fp32), a three-chunk bitmap and the
    largest d_ff, plus the degenerate thresholds (all-pass, empty mask)."""
    layer = synth.make_layer(_small_cfg(d, f, dt, seed), n_dec=3)
    ov = oracle_view(layer)
    L = pack_layer(layer)
    tau_x, tau_s = _oracle_taus(ov)
    fused = 7 | P.PROX_STAGE_FUSED_STAGE2
    _run_decode(P, L, layer, ov, [0], tau_x, tau_s, f"{d}x{f} fused", stages=fused)
    _y, mi, mc, _ic = _run_decode(P, L, layer, ov, [1], 0.0, 0.0, f"{d}x{f} fused all-pass", stages=fused)
    assert mc[0] == f
    y, _mi, mc, _ic = _run_decode(P, L, layer, ov, [2], 0.0, math.inf, f"{d}x{f} fused empty", stages=fused)
    assert mc[0] == 0 and np.all(y == 0)


@pytest.mark.parametrize("d,f,dt,b,keep_x,s2,seed", _sweep_cases(n=4, seed=2033))
def test_fused_stage2_seeded_shape_sweep(P, d, f, dt, b, keep_x, s2, seed):
    """The fused Stage-2 kernel on seeded random shapes, dtypes and operating
    points, against the oracle (the kernel serves batch 1: each draw's batch
    size is not used)."""
    layer = synth.make_layer(_small_cfg(d, f, dt, seed), n_dec=1)
    ov = oracle_view(layer)
    L = pack_layer(layer)
    tau_x, tau_s = _oracle_taus(ov, keep_x=keep_x, sparsity_s=s2)
    _run_decode(P, L, layer, ov, [0], tau_x, tau_s, f"fused {d}x{f}-{dt}", stages=7 | P.PROX_STAGE_FUSED_STAGE2)


def test_fused_stage2_items_beyond_the_grid(P):
    """d_model 12288 x d_ff 11264 (bf16): 24 column slices x 11 row groups =
    264 down items for a 256-block grid, so some blocks of the fused Stage-2
    kernel take a second item after the grid barrier; parity against the
    oracle, and the same masks and counts as the two-launch path."""
    layer = synth.make_layer(_small_cfg(12288, 11264, "bf16", 48, std=0.02), n_dec=2, n_cal=4)
    ov = oracle_view(layer)
    L = pack_layer(layer)
    tau_x, tau_s = _oracle_taus(ov)
    _run_decode(P, L, layer, ov, [0, 1], tau_x, tau_s, "12288x11264 fused",
                stages=7 | P.PROX_STAGE_FUSED_STAGE2)
    _run_decode(P, L, layer, ov, [1], tau_x, tau_s, "12288x11264")


def test_fused_stage2_wait_limit_give_up(P, layer8b):
    """The grid barrier's wait is bounded.  With the bound forced to 0 from the
    host, a block that finds the barrier incomplete at its first check gives
    up at once: the call reports mask_count = -1 and the workspace error word
    (PROX_ERR_INTERNAL from prox_workspace_check), and the kernel ends
    normally.  Calls with the default bound on the same workspace are correct
    again afterwards (the barrier's epochs stay consistent)."""
    layer, ov, L = layer8b
    tau_x, tau_s = _oracle_taus(ov, n_tok=16)
    x = to_device(layer.x_dec[[2]], "bf16")
    ws = P.new_workspace(L.d_model, L.d_ff, 1)
    ref = _bufs(P, L, 1)
    P.prox_ffn_decode_stages(L, x, tau_x, tau_s, *ref, ws, 7 | P.PROX_STAGE_FUSED_STAGE2)
    torch.cuda.synchronize()
    P.prox_workspace_check(ws)
    ry, rmi, rmc, ric = (v.cpu().numpy() for v in ref)
    fused = 7 | P.PROX_STAGE_FUSED_STAGE2
    gave_up = 0
    prev = P.prox_set_wait_limit(0)
    try:
        for _ in range(3):
            o = _bufs(P, L, 1)
            P.prox_ffn_decode_stages(L, x, tau_x, tau_s, *o, ws, fused)
            torch.cuda.synchronize()
            try:
                P.prox_workspace_check(ws)
                ok = True
            except P.ProxError as e:
                assert e.status == P.PROX_ERR_INTERNAL
                ok = False
            mc = int(o[2].item())
            if ok:   # every block found the barrier complete: a normal result
                assert mc == int(rmc[0])
            else:
                assert mc == -1
                gave_up += 1
    finally:
        assert P.prox_set_wait_limit(prev) == 0
    assert gave_up >= 1, "no block gave up with a zero wait bound"
    P.prox_workspace_check(ws)  # the error word was cleared
    for _ in range(2):
        o = _bufs(P, L, 1)
        P.prox_ffn_decode_stages(L, x, tau_x, tau_s, *o, ws, fused)
        torch.cuda.synchronize()
        P.prox_workspace_check(ws)
        y, mi, mc, ic = (v.cpu().numpy() for v in o)
        n = int(rmc[0])
        assert int(mc[0]) == n and np.array_equal(mi[0, :n], rmi[0, :n])
        assert y_errors(y[0], ry[0].astype(np.float64))[1] <= 1e-6
