"""GPU parity of the grouped batch path (2..8 tokens per group, more tokens in
several groups): Stage 1 over the union of the group's kept rows on the matrix
cores, Stage 2 over the union of the channel lists (bf16 weights).  By default
groups of fewer than 3 tokens run the per-token kernels; PROX_STAGE_GROUPED
forces the grouped ones so that small groups are covered too.

Every token is checked against the CPU oracle run on that token alone (the
batch-1 definition): k_x exact, channel masks exact outside the 1e-3 tau_s
band, y within max-abs 2e-2 / rel-L2 1e-2 of the oracle's Stage 2 on the
GPU's own channel list.  The grouped and the per-token kernels are also
compared with each other, and grouped y is reproducible bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from prox_gpu_util import band_compare, check_in_band, oracle_layer, oracle_view, pack_layer, to_device, y_errors, y_ok

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from free_ffn_activation_amd import prox
    return prox


def _cfg(d, f, dtype, seed, n_dec, std=0.05):
    return synth.LayerConfig(f"g{d}x{f}", d, f, dtype, std, max(1, d // 64), 20.0, 16, 0.5, 0.7, n_dec, seed)


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


def _check_tokens(ov, xs_host, out, tau_x, tau_s, label, act="silu"):
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
        y_ref = oracle.stage2(xh, ov["Wu"], ov["Wg"], ov["Wd"], m, act=act)["y"]
        ma, rl = y_errors(y[k], y_ref)
        assert y_ok(y[k], y_ref), f"{label} token {k}: y max-abs {ma:.3e} rel-L2 {rl:.3e}"
    print(f"[{label}] k_x={list(ic)} k_s={list(mc)} in-band={band}")


@pytest.mark.parametrize("d,f,dtype,batch,seed", [
    (512, 1024, "bf16", 2, 61),     # one group of two
    (320, 384, "bf16", 3, 62),      # partial 512-column slice, 3 panels
    (576, 1152, "bf16", 8, 63),     # one full group, two K-splits of Stage 1
    (512, 1024, "bf16", 11, 64),    # two groups: 8 + 3
    (256, 768, "f32", 5, 65),       # fp32 weights: grouped Stage 1, per-token Stage 2
    (64, 128, "bf16", 4, 66),       # minimum shape
    (1024, 2560, "bf16", 17, 67),   # three groups: 8 + 8 + 1
    (3072, 24576, "bf16", 4, 68),   # 768 rows per Stage-1 split: a full and a ragged 512-row pass
    (5120, 25600, "bf16", 3, 69),   # Qwen3-32B shape: 1280 rows per split, three passes (512, 512, 256)
])
def test_grouped_decode_parity(P, d, f, dtype, batch, seed):
    layer = synth.make_layer(_cfg(d, f, dtype, seed, batch), n_dec=batch)
    ov = oracle_view(layer)
    L = pack_layer(layer)
    tau_x, tau_s = _taus(ov)
    x = to_device(layer.x_dec, dtype)
    ws = P.new_workspace(d, f, batch)
    out = _decode(P, L, x, tau_x, tau_s, ws)
    _check_tokens(ov, ov["x_dec"], out, tau_x, tau_s, f"{d}x{f}-{dtype}-b{batch}")
    forced = _decode(P, L, x, tau_x, tau_s, ws, stages=7 | P.PROX_STAGE_GROUPED)
    _check_tokens(ov, ov["x_dec"], forced, tau_x, tau_s, f"{d}x{f}-{dtype}-b{batch}-grouped")
    if batch < 3:  # the default ran the per-token kernels: same lists as forcing them
        pt = _decode(P, L, x, tau_x, tau_s, ws, stages=7 | P.PROX_STAGE_PER_TOKEN)
        assert all(np.array_equal(a, b) for a, b in zip(out[1:], pt[1:]))
        # y: the per-token down kernel sums with atomics, so only up to fp32 order
        assert y_errors(out[0], pt[0].astype(np.float64))[1] <= 1e-5


@pytest.mark.parametrize("d,f,batch,seed", [(512, 1024, 4, 91), (576, 1152, 8, 92)])
def test_grouped_geglu_parity(P, d, f, batch, seed):
    """A GeGLU layer (GELU-tanh gate) on the grouped kernels: the gate in the
    grouped Stage-1 activation and in the grouped up/gate epilogue."""
    layer = synth.make_layer(_cfg(d, f, "bf16", seed, batch), n_dec=batch)
    ov = oracle_view(layer)
    L = pack_layer(layer, activation=P.PROX_ACT_GELU_TANH)
    tau_x, tau_s = _taus(ov, act="gelu_tanh")
    x = to_device(layer.x_dec, "bf16")
    ws = P.new_workspace(d, f, batch)
    out = _decode(P, L, x, tau_x, tau_s, ws)
    _check_tokens(ov, ov["x_dec"], out, tau_x, tau_s, f"geglu-{d}x{f}-b{batch}", act="gelu_tanh")


def test_many_groups_batch43(P):
    """43 tokens: five grouped groups of 8 and a grouped tail of 3, every
    token against the oracle; the same call with the per-token kernels forced
    gives the same k_x and index lists outside the tau_s band."""
    d, f, batch = 256, 512, 43
    layer = synth.make_layer(_cfg(d, f, "bf16", 93, batch), n_dec=batch)
    ov = oracle_view(layer)
    L = pack_layer(layer)
    tau_x, tau_s = _taus(ov)
    x = to_device(layer.x_dec, "bf16")
    ws = P.new_workspace(d, f, batch)
    out = _decode(P, L, x, tau_x, tau_s, ws)
    _check_tokens(ov, ov["x_dec"], out, tau_x, tau_s, "256x512-b43")
    pt = _decode(P, L, x, tau_x, tau_s, ws, stages=7 | P.PROX_STAGE_PER_TOKEN)
    assert np.array_equal(out[3], pt[3])  # k_x


def test_grouped_qwen3_8b_batch8_and_per_token_kernels(P):
    """The batch-8 Qwen3-8B-shaped layer: grouped path against the oracle, and
    against the per-token kernels on the same inputs."""
    layer, ov = oracle_layer("qwen3_8b_batch8", n_dec=8, n_cal=16)
    L = pack_layer(layer)
    tau_x, tau_s = _taus(ov)
    x = to_device(layer.x_dec[:8], "bf16")
    ws = P.new_workspace(L.d_model, L.d_ff, 8)
    g = _decode(P, L, x, tau_x, tau_s, ws)
    _check_tokens(ov, ov["x_dec"][:8], g, tau_x, tau_s, "qwen3_8b-b8-grouped")
    pt = _decode(P, L, x, tau_x, tau_s, ws, stages=7 | P.PROX_STAGE_PER_TOKEN)
    _check_tokens(ov, ov["x_dec"][:8], pt, tau_x, tau_s, "qwen3_8b-b8-per-token")
    assert np.array_equal(g[3], pt[3])  # k_x
    same = 0
    for k in range(8):
        if g[2][k] == pt[2][k] and np.array_equal(g[1][k, : g[2][k]], pt[1][k, : pt[2][k]]):
            same += 1
            ma, rl = y_errors(g[0][k], pt[0][k].astype(np.float64))
            assert rl <= 1e-4, f"token {k}: grouped vs per-token y rel-L2 {rl:.2e}"
    assert same >= 4, f"only {same} of 8 tokens have identical masks on both paths"
    assert len(set(int(v) for v in g[2])) > 1  # masks really are per token


def test_grouped_proxy_state(P):
    """prox_proxy_state at batch >= 2 (the grouped Stage-1 kernel) against the
    oracle's s~ per token, and bit-identical on a second call."""
    for name, d, f, dt, batch, seed in [("qwen3_8b_batch8", None, None, "bf16", 8, None),
                                        ("small", 576, 1152, "bf16", 6, 71), ("small32", 256, 768, "f32", 3, 72)]:
        if d is None:
            layer, ov = oracle_layer(name, n_dec=8, n_cal=16)
        else:
            layer = synth.make_layer(_cfg(d, f, dt, seed, batch), n_dec=batch)
            ov = oracle_view(layer)
        L = pack_layer(layer)
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


def test_grouped_degenerate_and_mixed_tokens(P):
    """Thresholds that keep everything or nothing, and a group whose tokens
    differ wildly: an all-zero token (no input row kept) next to normal ones."""
    d, f, batch = 512, 1024, 4
    layer = synth.make_layer(_cfg(d, f, "bf16", 81, batch), n_dec=batch)
    ov = oracle_view(layer)
    L = pack_layer(layer)
    x = to_device(layer.x_dec, "bf16")
    ws = P.new_workspace(d, f, batch)
    # all-pass: dense SwiGLU for every token
    out = _decode(P, L, x, 0.0, 0.0, ws)
    assert np.all(out[2] == f) and np.all(out[3] == d)
    assert all(np.array_equal(out[1][k], np.arange(f)) for k in range(batch))
    _check_tokens(ov, ov["x_dec"], out, 0.0, 0.0, "all-pass")
    # nothing kept, tau_s > 0: y = 0
    out = _decode(P, L, x, math.inf, 1e-6, ws)
    assert np.all(out[2] == 0) and np.all(out[3] == 0) and np.all(out[0] == 0)
    # tau_s = +inf: empty channel lists
    out = _decode(P, L, x, 0.0, math.inf, ws)
    assert np.all(out[2] == 0) and np.all(out[0] == 0)
    # mixed: token 1 is all zeros, token 3 an outlier-scaled copy of token 0
    tau_x, tau_s = _taus(ov)
    xb = layer.x_dec.copy()  # bf16 bit patterns
    xb[1] = 0
    xb[3] = synth.bf16_bits_from_f32((synth.as_f64(xb[0], "bf16") * 8.0).astype(np.float32))  # exact
    xh = synth.as_f64(xb, "bf16")
    out = _decode(P, L, to_device(xb, "bf16"), tau_x, tau_s, ws)
    assert out[3][1] == 0 and out[2][1] == 0 and np.all(out[0][1] == 0)
    _check_tokens(ov, xh, out, tau_x, tau_s, "mixed")


def test_grouped_repeat_graph_and_workspace_reuse(P):
    """Grouped y is reproducible bit for bit: repeated calls, HIP-graph replays
    with eager work in between, and calls of other batch sizes on the same
    workspace (tickets and lists left in a consistent state)."""
    layer, ov = oracle_layer("qwen3_8b_batch8", n_dec=8, n_cal=16)
    L = pack_layer(layer)
    tau_x, tau_s = _taus(ov)
    x8 = to_device(layer.x_dec[:8], "bf16")
    x3 = to_device(layer.x_dec[2:5], "bf16")
    ws = P.new_workspace(L.d_model, L.d_ff, 8)
    ref8 = _decode(P, L, x8, tau_x, tau_s, ws)
    G = 7 | P.PROX_STAGE_GROUPED  # three tokens: grouped kernels forced (bit-reproducible y)
    ref3 = _decode(P, L, x3, tau_x, tau_s, ws, stages=G)
    for rep in range(3):
        o8 = _decode(P, L, x8, tau_x, tau_s, ws)
        assert all(np.array_equal(a, b) for a, b in zip(o8, ref8)), f"repeat {rep} (batch 8)"
        o3 = _decode(P, L, x3, tau_x, tau_s, ws, stages=G)
        assert all(np.array_equal(a, b) for a, b in zip(o3, ref3)), f"repeat {rep} (batch 3)"
        p3 = _decode(P, L, x3, tau_x, tau_s, ws)  # per-token kernels on the same workspace
        assert all(np.array_equal(a, b) for a, b in zip(p3[1:], ref3[1:])), f"repeat {rep} (batch 3 per-token)"
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
        o3 = _decode(P, L, x3, tau_x, tau_s, ws, stages=G)  # eager work on the same workspace
        assert all(np.array_equal(a, b) for a, b in zip(o3, ref3)), f"eager after replay {rep}"
    del g
