"""The C-ABI library on the host: it loads, exports every declared symbol and
rejects bad arguments before touching a device (no GPU needed)."""
import ctypes
import math
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "prox.h")

P = pytest.importorskip("free_ffn_activation_amd.prox",
                        reason="libprox.so not built (run __graft_entry__.build())")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(prox_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert "prox_ffn_decode" in names and "prox_pack_proxy" in names and "prox_calibrate" in names
    out = subprocess.run(["nm", "-D", "--defined-only", P.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (prox_[a-z0-9_]+)", out))
    assert set(names) <= exported, f"missing: {set(names) - exported}"
    assert set(names) == set(P.EXPORTED)
    lib = P.raw_library()
    for n in names:
        assert getattr(lib, n) is not None


def test_version_and_sizes():
    assert P.prox_abi_version() == 4
    s = P.prox_layer_sizes(4096, 12288, P.PROX_BF16)
    assert s == (4096 * (12288 + 128), 2 * 4096 * 4, 2 * 12288 * 4096 * 2, 12288 * 4096 * 2)
    assert P.prox_layer_sizes(128, 384, P.PROX_BF16)[0] == 128 * 384     # 384/128 odd: no padding
    s32 = P.prox_layer_sizes(256, 768, P.PROX_F32)
    assert s32[2] == 2 * 256 * 768 * 4
    w1 = P.prox_workspace_size(4096, 12288, 1)
    assert w1 % 256 == 0 and P.prox_workspace_size(4096, 12288, 8) == 8 * w1
    assert P.prox_calibrate_workspace_size(4096, 12288, 256) >= 256 * 12288 * 4


@pytest.mark.parametrize("d,f,dt,status", [(100, 768, 1, P.PROX_ERR_UNSUPPORTED),
                                           (256, 700, 1, P.PROX_ERR_UNSUPPORTED),
                                           (32, 768, 1, P.PROX_ERR_INVALID_ARG),
                                           (256, 768, 7, P.PROX_ERR_INVALID_ARG),
                                           (16384, 768, 0, P.PROX_ERR_UNSUPPORTED),
                                           (4096, 131072, 1, P.PROX_ERR_UNSUPPORTED)])
def test_bad_shapes(d, f, dt, status):
    with pytest.raises(P.ProxError) as ei:
        P.prox_layer_sizes(d, f, dt)
    assert ei.value.status == status
    assert P.prox_last_error() != ""


FAKE = 1 << 40  # a 256-aligned address that is never dereferenced by validation


def _layer(d=256, f=768, dt=0, **kw):
    L = P.prox_layer(d, f, dt, 0, FAKE, FAKE, FAKE, FAKE, 0, 0, None, None)
    for k, v in kw.items():
        setattr(L, k, v)
    return L


def _decode(L, x=FAKE, batch=1, tx=0.5, ts=0.1, y=FAKE, mi=FAKE, mc=FAKE, ic=None, ws=FAKE,
            nbytes=1 << 30):
    lib = P.raw_library()
    return lib.prox_ffn_decode(ctypes.byref(L) if L is not None else None, x, batch, tx, ts, y, mi,
                               mc, ic, ws, nbytes, None)


def test_decode_argument_validation():
    ok_layer = _layer()
    assert _decode(None) == P.PROX_ERR_INVALID_ARG
    assert _decode(_layer(proxy_q=None)) == P.PROX_ERR_INVALID_ARG
    assert _decode(_layer(activation=2)) == P.PROX_ERR_INVALID_ARG
    # proxy kind: unknown kinds, a non-zero reserved field, the 16-bit proxy
    # without its buffer or on an fp32 layer are rejected before any work
    assert _decode(_layer(proxy_kind=2)) == P.PROX_ERR_INVALID_ARG
    assert _decode(_layer(reserved=1)) == P.PROX_ERR_INVALID_ARG
    assert _decode(_layer(dt=P.PROX_BF16, proxy_kind=P.PROX_PROXY_W16)) == P.PROX_ERR_INVALID_ARG
    assert _decode(_layer(proxy_kind=P.PROX_PROXY_W16, proxy_w16=FAKE)) == P.PROX_ERR_UNSUPPORTED
    assert _decode(_layer(dt=P.PROX_BF16, proxy_kind=P.PROX_PROXY_W16, proxy_w16=FAKE + 8)) == P.PROX_ERR_INVALID_ARG
    # the channel-major proxy copy: aligned, and only beside the INT4 proxy
    assert _decode(_layer(proxy_qt=FAKE + 8)) == P.PROX_ERR_INVALID_ARG
    assert _decode(_layer(dt=P.PROX_BF16, proxy_kind=P.PROX_PROXY_W16, proxy_w16=FAKE,
                          proxy_qt=FAKE)) == P.PROX_ERR_INVALID_ARG
    assert _decode(_layer(d=250)) == P.PROX_ERR_UNSUPPORTED
    assert _decode(_layer(w_down=FAKE + 8)) == P.PROX_ERR_INVALID_ARG     # misaligned
    assert _decode(ok_layer, batch=0) == P.PROX_ERR_INVALID_ARG
    assert _decode(ok_layer, batch=257) == P.PROX_ERR_INVALID_ARG
    assert _decode(ok_layer, tx=math.nan) == P.PROX_ERR_INVALID_ARG
    assert _decode(ok_layer, ts=-1.0) == P.PROX_ERR_INVALID_ARG
    assert _decode(ok_layer, x=None) == P.PROX_ERR_INVALID_ARG
    assert _decode(ok_layer, y=FAKE + 4) == P.PROX_ERR_INVALID_ARG
    assert _decode(ok_layer, ws=None) == P.PROX_ERR_INVALID_ARG
    assert _decode(ok_layer, ws=FAKE + 16) == P.PROX_ERR_INVALID_ARG
    need = P.prox_workspace_size(256, 768, 2)
    assert _decode(ok_layer, batch=2, nbytes=need - 1) == P.PROX_ERR_INVALID_ARG
    assert "workspace" in P.prox_last_error()


def test_other_entry_points_validate():
    lib = P.raw_library()
    L = _layer()
    tx, ts = ctypes.c_float(), ctypes.c_float()
    # calibrate: fractions outside [0, 1], tokens out of range, small workspace
    assert lib.prox_calibrate(ctypes.byref(L), FAKE, 64, 1.5, 0.7, ctypes.byref(tx),
                              ctypes.byref(ts), FAKE, 1 << 30, None) == P.PROX_ERR_INVALID_ARG
    assert lib.prox_calibrate(ctypes.byref(L), FAKE, 0, 0.5, 0.7, ctypes.byref(tx),
                              ctypes.byref(ts), FAKE, 1 << 30, None) == P.PROX_ERR_INVALID_ARG
    assert lib.prox_calibrate(ctypes.byref(L), FAKE, 64, 0.5, 0.7, ctypes.byref(tx),
                              ctypes.byref(ts), FAKE, 16, None) == P.PROX_ERR_INVALID_ARG
    assert lib.prox_calibrate(ctypes.byref(L), FAKE, 64, 0.5, 0.7, None, ctypes.byref(ts),
                              FAKE, 1 << 30, None) == P.PROX_ERR_INVALID_ARG
    # pack: NULL / misaligned inputs
    assert lib.prox_pack_proxy(None, FAKE, FAKE, ctypes.byref(L), None) == P.PROX_ERR_INVALID_ARG
    assert lib.prox_pack_proxy(FAKE + 2, FAKE, FAKE, ctypes.byref(L), None) == P.PROX_ERR_INVALID_ARG
    # stage 2 / proxy state
    assert lib.prox_ffn_stage2(ctypes.byref(L), FAKE, 1, None, FAKE, FAKE, FAKE, 1 << 30,
                               None) == P.PROX_ERR_INVALID_ARG
    assert lib.prox_proxy_state(ctypes.byref(L), FAKE, 1, math.nan, FAKE, None, FAKE, 1 << 30,
                                None) == P.PROX_ERR_INVALID_ARG
    # events variant needs the event array
    assert lib.prox_ffn_decode_events(ctypes.byref(L), FAKE, 1, 0.5, 0.1, FAKE, FAKE, FAKE, None,
                                      FAKE, 1 << 30, None, None) == P.PROX_ERR_INVALID_ARG
    assert lib.prox_workspace_init(None, 16, None) == P.PROX_ERR_INVALID_ARG
    # histogram calibration: bins / samples out of range, small workspace, bad fraction
    size = ctypes.c_size_t(0)
    assert lib.prox_calibrate_hist_workspace_size(256, 768, 64, 200000, 4096, ctypes.byref(size)) == P.PROX_OK
    assert size.value >= 64 * 768 * 4 + 200000 * 4 + 4096 * 4
    for ms, nb in ((0, 4096), (200000, 1), (200000, 8193), (1 << 25, 4096)):
        assert lib.prox_calibrate_hist_workspace_size(256, 768, 64, ms, nb, ctypes.byref(size)) == P.PROX_ERR_INVALID_ARG
        assert lib.prox_calibrate_hist(ctypes.byref(L), FAKE, 64, 0.5, 0.7, ms, nb, ctypes.byref(tx),
                                       ctypes.byref(ts), FAKE, 1 << 30, None) == P.PROX_ERR_INVALID_ARG
    assert lib.prox_calibrate_hist(ctypes.byref(L), FAKE, 64, 0.5, 0.7, 200000, 4096, ctypes.byref(tx),
                                   ctypes.byref(ts), FAKE, 16, None) == P.PROX_ERR_INVALID_ARG
    assert lib.prox_calibrate_hist(ctypes.byref(L), FAKE, 64, 0.5, 1.5, 200000, 4096, ctypes.byref(tx),
                                   ctypes.byref(ts), FAKE, 1 << 30, None) == P.PROX_ERR_INVALID_ARG
    # stage subsets: a non-empty subset of the three kernels, plus at most one
    # of the per-token / grouped overrides
    for bad in (0, 8, 16, 24, -1, 32, 7 | 8 | 16, 1 | 8 | 16, 64 | 7, 96):
        assert lib.prox_ffn_decode_stages(ctypes.byref(L), FAKE, 1, 0.5, 0.1, FAKE, FAKE, FAKE,
                                          None, FAKE, 1 << 30, None, bad) == P.PROX_ERR_INVALID_ARG


def test_proxy16_sizes_and_pack_validation():
    # rows of 4 * d_ff bytes, padded to an odd multiple of 128 (d_ff % 128 == 0
    # makes 4 * d_ff / 128 even, so every row carries 128 bytes of padding)
    assert P.prox_proxy16_size(4096, 12288, P.PROX_BF16) == 4096 * (4 * 12288 + 128)
    assert P.prox_proxy16_size(64, 128, P.PROX_BF16) == 64 * (512 + 128)
    assert P.prox_proxy16_size(128, 384, P.PROX_BF16) == 128 * (1536 + 128)
    with pytest.raises(P.ProxError) as ei:
        P.prox_proxy16_size(256, 768, P.PROX_F32)
    assert ei.value.status == P.PROX_ERR_UNSUPPORTED
    # argument checks happen before anything is enqueued (no GPU work here)
    lib = P.raw_library()
    assert lib.prox_pack_proxy16(None, FAKE, ctypes.byref(_layer(dt=P.PROX_BF16, proxy_w16=FAKE)), None) == \
        P.PROX_ERR_INVALID_ARG
    assert lib.prox_pack_proxy16(FAKE, FAKE, None, None) == P.PROX_ERR_INVALID_ARG
    assert lib.prox_pack_proxy16(FAKE, FAKE, ctypes.byref(_layer(dt=P.PROX_BF16)), None) == P.PROX_ERR_INVALID_ARG
    assert lib.prox_pack_proxy16(FAKE, FAKE, ctypes.byref(_layer(proxy_w16=FAKE)), None) == P.PROX_ERR_UNSUPPORTED
    assert lib.prox_pack_proxy16(FAKE + 8, FAKE, ctypes.byref(_layer(dt=P.PROX_BF16, proxy_w16=FAKE)), None) == \
        P.PROX_ERR_INVALID_ARG


def test_noalloc_rejects_before_touching_a_device():
    """The allocation-free entry point validates like prox_ffn_decode and
    refuses a size beyond its scratch array before any device call."""
    lib = P.raw_library()
    L = _layer(4096, 12288, P.PROX_BF16)
    per_token = P.prox_workspace_size(4096, 12288, 1)
    too_many = P.PROX_NOALLOC_SCRATCH_BYTES // per_token + 1
    st = lib.prox_ffn_decode_noalloc(ctypes.byref(L), FAKE, too_many, 0.5, 0.1, FAKE, FAKE, FAKE, None, None)
    assert st == P.PROX_ERR_UNSUPPORTED and "scratch" in P.prox_last_error()
    st = lib.prox_ffn_decode_noalloc(ctypes.byref(L), FAKE, 1, math.nan, 0.1, FAKE, FAKE, FAKE, None, None)
    assert st == P.PROX_ERR_INVALID_ARG
    st = lib.prox_ffn_decode_noalloc(None, FAKE, 1, 0.5, 0.1, FAKE, FAKE, FAKE, None, None)
    assert st == P.PROX_ERR_INVALID_ARG
    assert P.PROX_NOALLOC_SCRATCH_BYTES == 32 << 20


def test_proxy_qt_size_and_pack_validation():
    # d_ff * 128 * ceil(d_model / 128): whole 128-row chunks of every channel
    assert P.prox_proxy_qt_size(4096, 12288) == 4096 * 12288
    assert P.prox_proxy_qt_size(5120, 25600) == 5120 * 25600
    assert P.prox_proxy_qt_size(320, 384) == 384 * 128 * 3
    with pytest.raises(P.ProxError) as ei:
        P.prox_proxy_qt_size(100, 384)
    assert ei.value.status == P.PROX_ERR_UNSUPPORTED
    lib = P.raw_library()
    assert lib.prox_proxy_qt_size(256, 768, None) == P.PROX_ERR_INVALID_ARG
    assert lib.prox_pack_proxy_qt(None, None) == P.PROX_ERR_INVALID_ARG
    assert lib.prox_pack_proxy_qt(ctypes.byref(_layer()), None) == P.PROX_ERR_INVALID_ARG   # no proxy_qt
    assert lib.prox_pack_proxy_qt(ctypes.byref(_layer(proxy_qt=FAKE + 4)), None) == P.PROX_ERR_INVALID_ARG
    assert lib.prox_pack_proxy_qt(ctypes.byref(_layer(dt=P.PROX_BF16, proxy_kind=P.PROX_PROXY_W16,
                                                      proxy_w16=FAKE)), None) == P.PROX_ERR_UNSUPPORTED
