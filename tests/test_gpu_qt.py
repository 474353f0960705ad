"""GPU parity of Stage 1 from the channel-major proxy copy (prox_layer.proxy_qt,
prox_pack_proxy_qt): groups of 2..8 tokens read every proxy row once as
contiguous runs instead of gathering the union of their kept rows.

The copy itself is checked byte for byte against the oracle's INT4 codes laid
out as include/prox.h documents (not against the GPU's own row-major proxy).
Decodes through it are checked per token against the CPU oracle under the same
rules as every decode (k_x exact, masks exact outside the 1e-3 tau_s band, y
within max-abs 2e-2 / rel-L2 1e-2), over shapes that exercise every plan of the
kernel: 1, 2 and 4 parts per channel group, one and two units per streaming
wave, inputs that end inside a 128-row chunk, a single chunk, the largest
d_model (two pre-pass rounds) and the largest d_ff.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from prox_gpu_util import band_compare, check_in_band, oracle_layer, oracle_view, pack_layer, to_device, y_errors, y_ok

pytestmark = pytest.mark.gpu

NIBBLE_POS = (0, 4, 1, 5, 2, 6, 3, 7)  # nibble holding row e of a 4-byte word (prox.h)


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from free_ffn_activation_amd import prox
    return prox


def _cfg(d, f, dtype, seed, n_dec, std=0.05):
    return synth.LayerConfig(f"q{d}x{f}", d, f, dtype, std, max(1, d // 64), 20.0, 16, 0.5, 0.7, n_dec, seed)


def _qt_layer(P, layer, activation=None):
    L = pack_layer(layer) if activation is None else pack_layer(layer, activation=activation)
    L.add_proxy_qt()
    torch.cuda.synchronize()
    return L


def expected_qt(qu: np.ndarray, qg: np.ndarray) -> np.ndarray:
    """The proxy_qt bytes of oracle codes qu, qg ([d][f], -7..7), laid out per
    the prox_layer documentation in include/prox.h."""
    d, f = qu.shape
    nck = -(-d // 128)
    out = np.empty((nck, f // 16, 2, 64, 4), dtype=np.uint32)   # chunk-major
    for pr, q in enumerate((qu, qg)):
        nib = np.full((nck * 128, f), 8, dtype=np.uint32)   # rows past d hold code 0
        nib[:d] = (q.astype(np.int32) + 8).astype(np.uint32)
        # row index of (chunk k, lane l, word s, element e): 128k + 32 (l // 16) + 8s + e
        r = nib.reshape(nck, 4, 4, 8, f // 16, 16)           # [k][l//16][s][e][g][l%16]
        word = np.zeros((nck, 4, 4, f // 16, 16), dtype=np.uint32)
        for e in range(8):
            word |= r[:, :, :, e] << np.uint32(4 * NIBBLE_POS[e])
        # -> [k][g][l][s] with l = 16 (l // 16) + l % 16
        w = word.transpose(0, 3, 1, 4, 2).reshape(nck, f // 16, 64, 4)
        out[:, :, pr] = w
    return out.reshape(-1).view(np.uint8)


@pytest.mark.parametrize("d,f,dtype,seed", [(512, 1024, "bf16", 201), (320, 384, "bf16", 202),
                                            (64, 128, "f32", 203), (4096, 12288, "bf16", 204)])
def test_pack_proxy_qt_layout(P, d, f, dtype, seed):
    layer = synth.make_layer(_cfg(d, f, dtype, seed, 1), n_dec=1)
    ov = oracle_view(layer)
    L = _qt_layer(P, layer)
    assert L.proxy_qt.numel() == P.prox_proxy_qt_size(d, f) == f * 128 * (-(-d // 128))
    got = L.proxy_qt.cpu().numpy()
    exp = expected_qt(ov["qu"], ov["qg"])
    assert got.shape == exp.shape
    bad = np.flatnonzero(got != exp)
    assert bad.size == 0, f"{bad.size} byte(s) differ, first at {bad[:4]}"


def _bufs(L, b):
    dev = "cuda"
    return (torch.full((b, L.d_model), math.nan, dtype=torch.float32, device=dev),
            torch.full((b, L.d_ff), -7, dtype=torch.int32, device=dev),
            torch.full((b,), -1, dtype=torch.int32, device=dev),
            torch.full((b,), -1, dtype=torch.int32, device=dev))


def _taus(ov, act="silu"):
    return oracle.calibrate(ov["x_cal"], ov["qu"], ov["su"], ov["qg"], ov["sg"], 0.5, 0.7, act=act)


def _decode(P, L, x, tau_x, tau_s, ws, stages=None):
    b = x.shape[0]
    y, mi, mc, ic = _bufs(L, b)
    if stages is None:
        P.prox_ffn_decode(L, x, tau_x, tau_s, y, mi, mc, ic, ws)
    else:
        P.prox_ffn_decode_stages(L, x, tau_x, tau_s, y, mi, mc, ic, ws, stages)
    torch.cuda.synchronize()
    return y.cpu().numpy(), mi.cpu().numpy(), mc.cpu().numpy(), ic.cpu().numpy()


def _check_tokens(ov, xs_host, out, tau_x, tau_s, label, act="silu", check_y=True):
    y, mi, mc, ic = out
    band = 0
    for k, xh in enumerate(xs_host):
        ref = oracle.decode(xh, ov["Wu"], ov["Wg"], ov["Wd"], ov["qu"], ov["su"], ov["qg"], ov["sg"],
                            tau_x, tau_s, act=act)
        assert ic[k] == ref["k_x"], f"{label} token {k}: k_x {ic[k]} != {ref['k_x']}"
        oob, inb, asc = band_compare(mi[k], int(mc[k]), ref["s_tilde"], tau_s)
        assert asc, f"{label} token {k}: index list not ascending / in range"
        assert oob == 0, f"{label} token {k}: {oob} channel(s) outside the band disagree"
        check_in_band(mi[k], int(mc[k]), ref["s_tilde"], tau_s, f"{label} token {k}")
        band += inb
        m = np.zeros(len(ref["s_tilde"]), bool)
        m[mi[k][: mc[k]]] = True
        if not m.any():
            assert np.all(y[k] == 0.0), f"{label} token {k}: empty mask but y != 0"
            continue
        if not check_y:
            continue
        y_ref = oracle.stage2(xh, ov["Wu"], ov["Wg"], ov["Wd"], m, act=act)["y"]
        ma, rl = y_errors(y[k], y_ref)
        assert y_ok(y[k], y_ref), f"{label} token {k}: y max-abs {ma:.3e} rel-L2 {rl:.3e}"
    print(f"[{label}] k_x={list(ic)} k_s={list(mc)} in-band={band}")


@pytest.mark.parametrize("d,f,dtype,batch,seed", [
    (512, 1024, "bf16", 2, 211),    # a group of two: per-token kernels, qt Stage 1 when grouping is forced
    (320, 384, "bf16", 3, 212),     # inputs end inside the third 128-row chunk
    (576, 1152, "bf16", 8, 213),    # a full group, 5 chunks in 4 parts of 2 (one short, one empty)
    (512, 1024, "bf16", 11, 214),   # two groups: 8 + 3
    (256, 768, "f32", 5, 215),      # fp32 layer: fp32 x into the operand image
    (64, 128, "bf16", 4, 216),      # minimum shape: one chunk, half of it past d
    (1024, 2560, "bf16", 17, 217),  # three groups: 8 + 8 + 1 (the last one per-token)
    (5120, 25600, "bf16", 3, 218),  # Qwen3-32B shape: 7 groups per block, 2 parts, 20 chunks each
    (128, 65536, "bf16", 3, 219),   # largest d_ff: 16 groups per block, 1 part, two units per wave
    (12288, 256, "f32", 3, 220),    # largest d_model: 24 chunks per part, two pre-pass rounds
])
def test_qt_decode_parity(P, d, f, dtype, batch, seed):
    layer = synth.make_layer(_cfg(d, f, dtype, seed, batch), n_dec=batch)
    ov = oracle_view(layer)
    L = _qt_layer(P, layer)
    tau_x, tau_s = _taus(ov)
    x = to_device(layer.x_dec, dtype)
    ws = P.new_workspace(d, f, batch)
    out = _decode(P, L, x, tau_x, tau_s, ws)
    _check_tokens(ov, ov["x_dec"], out, tau_x, tau_s, f"qt-{d}x{f}-{dtype}-b{batch}")
    if f <= 25600:
        forced = _decode(P, L, x, tau_x, tau_s, ws, stages=7 | P.PROX_STAGE_GROUPED)
        _check_tokens(ov, ov["x_dec"], forced, tau_x, tau_s, f"qt-{d}x{f}-{dtype}-b{batch}-grouped")
    # the union-of-rows Stage 1 (no proxy_qt) on the same inputs: same k_x
    u = _decode(P, L.with_qt(False), x, tau_x, tau_s, ws)
    assert np.array_equal(u[3], out[3])


def test_qt_qwen3_8b_batch8(P):
    """The batch-8 Qwen3-8B-shaped layer through the channel-major Stage 1,
    against the oracle and against the union-of-rows Stage 1."""
    layer, ov = oracle_layer("qwen3_8b_batch8", n_dec=8, n_cal=16)
    L = pack_layer(layer)
    L.add_proxy_qt()
    tau_x, tau_s = _taus(ov)
    x = to_device(layer.x_dec[:8], "bf16")
    ws = P.new_workspace(L.d_model, L.d_ff, 8)
    q = _decode(P, L, x, tau_x, tau_s, ws)
    _check_tokens(ov, ov["x_dec"][:8], q, tau_x, tau_s, "qwen3_8b-b8-qt")
    u = _decode(P, L.with_qt(False), x, tau_x, tau_s, ws)
    assert np.array_equal(q[3], u[3])
    same = sum(int(q[2][k] == u[2][k] and np.array_equal(q[1][k, : q[2][k]], u[1][k, : u[2][k]]))
               for k in range(8))
    assert same >= 4, f"only {same} of 8 tokens have identical masks on both Stage-1 kernels"


def test_qt_geglu(P):
    d, f, batch = 576, 1152, 6
    layer = synth.make_layer(_cfg(d, f, "bf16", 221, batch), n_dec=batch)
    ov = oracle_view(layer)
    L = _qt_layer(P, layer, activation=P.PROX_ACT_GELU_TANH)
    tau_x, tau_s = _taus(ov, act="gelu_tanh")
    x = to_device(layer.x_dec, "bf16")
    ws = P.new_workspace(d, f, batch)
    out = _decode(P, L, x, tau_x, tau_s, ws)
    _check_tokens(ov, ov["x_dec"], out, tau_x, tau_s, f"qt-geglu-{d}x{f}-b{batch}", act="gelu_tanh")


def test_qt_proxy_state(P):
    """prox_proxy_state through the channel-major Stage 1: s~ per token against
    the oracle, and bit-identical on a second call."""
    for name, d, f, dt, batch, seed in [("qwen3_8b_batch8", None, None, "bf16", 8, None),
                                        ("small", 576, 1152, "bf16", 6, 231), ("small32", 320, 384, "f32", 3, 232)]:
        if d is None:
            layer, ov = oracle_layer(name, n_dec=8, n_cal=16)
        else:
            layer = synth.make_layer(_cfg(d, f, dt, seed, batch), n_dec=batch)
            ov = oracle_view(layer)
        L = _qt_layer(P, layer)
        tau_x = float(np.float32(np.median(np.abs(ov["x_cal"]))))
        x = to_device(layer.x_dec[:batch], dt)
        st = torch.empty(batch, L.d_ff, dtype=torch.float32, device="cuda")
        ic = torch.empty(batch, dtype=torch.int32, device="cuda")
        ws = P.new_workspace(L.d_model, L.d_ff, batch)
        P.prox_proxy_state(L, x, tau_x, st, ic, ws)
        torch.cuda.synchronize()
        st_h, ic_h = st.cpu().numpy(), ic.cpu().numpy()
        for k in range(batch):
            ref = oracle.proxy_state(ov["x_dec"][k], ov["qu"], ov["su"], ov["qg"], ov["sg"], tau_x)
            assert ic_h[k] == int(ref["m_x"].sum()), f"{name} token {k}: k_x"
            scale = np.max(np.abs(ref["s"]))
            err = np.max(np.abs(st_h[k] - ref["s"]))
            assert err <= 1e-5 * scale, f"{name} token {k}: s~ error {err:.3e} vs scale {scale:.3e}"
        st2 = torch.empty_like(st)
        P.prox_proxy_state(L, x, tau_x, st2, None, ws)
        torch.cuda.synchronize()
        assert np.array_equal(st2.cpu().numpy().view(np.uint32), st_h.view(np.uint32)), name


def test_qt_degenerate_and_mixed_tokens(P):
    """Thresholds that keep everything or nothing, and a group with an
    all-zero token and an outlier-scaled one (a wide range of per-token
    operand scales in one launch)."""
    d, f, batch = 512, 1024, 4
    layer = synth.make_layer(_cfg(d, f, "bf16", 241, batch), n_dec=batch)
    ov = oracle_view(layer)
    L = _qt_layer(P, layer)
    x = to_device(layer.x_dec, "bf16")
    ws = P.new_workspace(d, f, batch)
    out = _decode(P, L, x, 0.0, 0.0, ws)
    assert np.all(out[2] == f) and np.all(out[3] == d)
    _check_tokens(ov, ov["x_dec"], out, 0.0, 0.0, "qt-all-pass")
    out = _decode(P, L, x, math.inf, 1e-6, ws)
    assert np.all(out[2] == 0) and np.all(out[3] == 0) and np.all(out[0] == 0)
    out = _decode(P, L, x, 0.0, math.inf, ws)
    assert np.all(out[2] == 0) and np.all(out[0] == 0)
    tau_x, tau_s = _taus(ov)
    xb = layer.x_dec.copy()
    xb[1] = 0
    xb[3] = synth.bf16_bits_from_f32((synth.as_f64(xb[0], "bf16") * 8.0).astype(np.float32))  # exact
    xh = synth.as_f64(xb, "bf16")
    out = _decode(P, L, to_device(xb, "bf16"), tau_x, tau_s, ws)
    assert out[3][1] == 0 and out[2][1] == 0 and np.all(out[0][1] == 0)
    _check_tokens(ov, xh, out, tau_x, tau_s, "qt-mixed")
    # a token 1024 times larger than its neighbours (token scales 2^10 apart in
    # one launch): k_x and masks as always; y is ~1e7 here, beyond the
    # decode's absolute y bound, so its y is not compared
    xb[3] = synth.bf16_bits_from_f32((synth.as_f64(xb[0], "bf16") * 1024.0).astype(np.float32))  # exact
    xh = synth.as_f64(xb, "bf16")
    out = _decode(P, L, to_device(xb, "bf16"), tau_x, tau_s, ws)
    _check_tokens(ov, xh, out, tau_x, tau_s, "qt-mixed-x1024", check_y=False)


def test_qt_repeat_and_graph(P):
    """Bit-identical outputs over repeated calls and HIP-graph replays (with
    eager calls of other batch sizes on the same workspace in between)."""
    layer, ov = oracle_layer("qwen3_8b_batch8", n_dec=8, n_cal=16)
    L = pack_layer(layer)
    L.add_proxy_qt()
    tau_x, tau_s = _taus(ov)
    x8 = to_device(layer.x_dec[:8], "bf16")
    x2 = to_device(layer.x_dec[3:5], "bf16")
    ws = P.new_workspace(L.d_model, L.d_ff, 8)
    ref8 = _decode(P, L, x8, tau_x, tau_s, ws)
    ref2 = _decode(P, L, x2, tau_x, tau_s, ws)
    for rep in range(3):
        o8 = _decode(P, L, x8, tau_x, tau_s, ws)
        assert all(np.array_equal(a, b) for a, b in zip(o8, ref8)), f"repeat {rep} (batch 8)"
        o2 = _decode(P, L, x2, tau_x, tau_s, ws)
        assert all(np.array_equal(a, b) for a, b in zip(o2[1:], ref2[1:])), f"repeat {rep} (batch 2)"
    bufs = _bufs(L, 8)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        P.prox_ffn_decode(L, x8, tau_x, tau_s, *bufs, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        P.prox_ffn_decode(L, x8, tau_x, tau_s, *bufs, ws)
    for rep in range(4):
        bufs[0].fill_(123.0)
        bufs[2].fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        got = [t.cpu().numpy() for t in bufs]
        assert all(np.array_equal(a, b) for a, b in zip(got, ref8)), f"graph replay {rep}"
        o2 = _decode(P, L, x2, tau_x, tau_s, ws)
        assert all(np.array_equal(a, b) for a, b in zip(o2[1:], ref2[1:])), f"eager after replay {rep}"
    del g
