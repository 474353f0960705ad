"""The allocation-free decode entry point (prox_ffn_decode_noalloc) against
prox_ffn_decode with a caller workspace: the same kernels, so the same masks
and counts bit for bit and y within the decode tolerance, over consecutive
calls of different shapes and batches on the one per-GPU scratch array."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from prox_gpu_util import oracle_layer, pack_layer, to_device, y_errors, y_ok

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from free_ffn_activation_amd import prox
    return prox


def _outs(L, b, fill):
    return (torch.full((b, L.d_model), fill, dtype=torch.float32, device="cuda"),
            torch.full((b, L.d_ff), -7, dtype=torch.int32, device="cuda"),
            torch.full((b,), -1, dtype=torch.int32, device="cuda"),
            torch.full((b,), -1, dtype=torch.int32, device="cuda"))


def _noalloc_raw(P, L, x, tx, ts, outs):
    """The C entry point itself, through ctypes."""
    y, mi, mc, ic = outs
    lib = P.raw_library()
    st = lib.prox_ffn_decode_noalloc(ctypes.byref(L.desc), x.data_ptr(), x.shape[0], tx, ts, y.data_ptr(),
                                     mi.data_ptr(), mc.data_ptr(), ic.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream)
    return st


def _compare(P, L, x, tx, ts, label):
    b = x.shape[0]
    ref = _outs(L, b, 0.0)
    P.prox_ffn_decode(L, x, tx, ts, *ref, P.new_workspace(L.d_model, L.d_ff, b))
    got = _outs(L, b, float("nan"))
    assert _noalloc_raw(P, L, x, tx, ts, got) == P.PROX_OK, P.prox_last_error()
    torch.cuda.synchronize()
    ry, rmi, rmc, ric = (t.cpu().numpy() for t in ref)
    gy, gmi, gmc, gic = (t.cpu().numpy() for t in got)
    assert np.array_equal(gmc, rmc) and np.array_equal(gic, ric), f"{label}: counts differ"
    for k in range(b):
        n = int(rmc[k])
        assert np.array_equal(gmi[k, :n], rmi[k, :n]), f"{label} token {k}: channel list differs"
        ma, rl = y_errors(gy[k], ry[k].astype(np.float64))
        assert y_ok(gy[k], ry[k].astype(np.float64)) and rl <= 1e-5, f"{label} token {k}: y {ma:.2e} / {rl:.2e}"
    print(f"[{label}] batch {b}: k_s {list(gmc)} k_x {list(gic)}")


def _taus(P, L, layer, n_cal):
    xc = to_device(layer.x_cal[:n_cal], layer.cfg.dtype)
    ws = torch.empty(P.prox_calibrate_workspace_size(L.d_model, L.d_ff, n_cal), dtype=torch.uint8, device="cuda")
    return P.prox_calibrate(L, xc, layer.cfg.keep_x, layer.cfg.sparsity_s, ws)


def test_noalloc_matches_workspace_decode(P):
    # call 1: the Qwen3-8B-shaped layer, 2 tokens
    layer8, _ = oracle_layer("qwen3_8b")
    L8 = pack_layer(layer8)
    tx8, ts8 = _taus(P, L8, layer8, 16)
    _compare(P, L8, to_device(layer8.x_dec[[0, 1]], "bf16"), tx8, ts8, "8b b2")
    # call 2: a smaller input (the tiny fp32 layer, 1 token: another shape)
    tiny, _ = oracle_layer("tiny")
    Lt = pack_layer(tiny)
    txt, tst = _taus(P, Lt, tiny, 64)
    _compare(P, Lt, to_device(tiny.x_dec[[3]], "f32"), txt, tst, "tiny b1")
    # back to the 8B shape with one token, then a grouped batch of 8 (the
    # scratch region grows), then one token again on the grown region
    _compare(P, L8, to_device(layer8.x_dec[[2]], "bf16"), tx8, ts8, "8b b1")
    _compare(P, L8, to_device(layer8.x_dec[list(range(8))], "bf16"), tx8, ts8, "8b b8 grouped")
    # the same layer with its channel-major proxy copy: the groups' Stage 1
    # then runs from it (no scratch beyond the masks)
    L8.add_proxy_qt()
    _compare(P, L8, to_device(layer8.x_dec[list(range(8))], "bf16"), tx8, ts8, "8b b8 channel-major")
    _compare(P, L8, to_device(layer8.x_dec[[1, 4, 6]], "bf16"), tx8, ts8, "8b b3 channel-major")
    _compare(P, L8, to_device(layer8.x_dec[[5]], "bf16"), tx8, ts8, "8b b1 again")


def test_noalloc_repeated_calls_one_stream(P):
    """Stream-ordered calls with no host synchronisation in between, on the
    one scratch array: each leaves it ready for the next."""
    layer, _ = oracle_layer("qwen3_8b")
    L = pack_layer(layer)
    tx, ts = _taus(P, L, layer, 16)
    xs = [to_device(layer.x_dec[[t]], "bf16") for t in range(4)]
    refs = []
    for x in xs:
        r = _outs(L, 1, 0.0)
        P.prox_ffn_decode(L, x, tx, ts, *r, P.new_workspace(L.d_model, L.d_ff, 1))
        refs.append(r)
    outs = [_outs(L, 1, float("nan")) for _ in range(12)]
    for c, o in enumerate(outs):
        assert _noalloc_raw(P, L, xs[c % 4], tx, ts, o) == P.PROX_OK
    torch.cuda.synchronize()
    for c, o in enumerate(outs):
        ry, rmi, rmc, _ = (t.cpu().numpy() for t in refs[c % 4])
        gy, gmi, gmc, _ = (t.cpu().numpy() for t in o)
        n = int(rmc[0])
        assert int(gmc[0]) == n and np.array_equal(gmi[0, :n], rmi[0, :n]), f"call {c}"
        assert y_errors(gy[0], ry[0].astype(np.float64))[1] <= 1e-5, f"call {c}"


def test_noalloc_rejects_sizes_beyond_the_scratch(P):
    layer, _ = oracle_layer("qwen3_8b")
    L = pack_layer(layer)
    b = P.PROX_NOALLOC_SCRATCH_BYTES // P.prox_workspace_size(L.d_model, L.d_ff, 1) + 1
    x = torch.zeros(b, L.d_model, dtype=torch.int16, device="cuda")
    outs = _outs(L, b, 0.0)
    assert _noalloc_raw(P, L, x, 0.5, 0.1, outs) == P.PROX_ERR_UNSUPPORTED
    assert "scratch" in P.prox_last_error()
