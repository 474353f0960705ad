"""ctypes binding of libprox.so (include/prox.h).

Argument marshalling only: every step of the decode path runs in the HIP
library.  Device buffers are torch tensors (PyTorch provides device memory and
streams); their data pointers and the current HIP stream are passed through.
The functions carry the C names.  If the library is missing this module fails
loudly at import; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# PROX_LIBRARY selects another build of the same library (the host-sanitizer build)
LIB_PATH = os.environ.get("PROX_LIBRARY") or os.path.join(_HERE, "libprox.so")

PROX_OK = 0
PROX_ERR_INVALID_ARG = -1
PROX_ERR_UNSUPPORTED = -2
PROX_ERR_HIP = -3
PROX_ERR_INTERNAL = -4
PROX_F32 = 0
PROX_BF16 = 1
PROX_ACT_SILU = 0
PROX_ACT_GELU_TANH = 1
PROX_PROXY_INT4 = 0
PROX_PROXY_W16 = 1  # the 16-bit proxy of the pages' precision ablation (bf16 layers)
PROX_STAGE_PROXY = 1
PROX_STAGE_UPGATE = 2
PROX_STAGE_DOWN = 4
PROX_STAGE_PER_TOKEN = 8  # batch >= 2: per-token kernels for every group
PROX_STAGE_GROUPED = 16   # batch >= 2: grouped kernels for every group (default: groups of >= 3 tokens)
PROX_STAGE_FUSED_STAGE2 = 32  # batch 1: up/gate and down in one launch joined by a grid barrier (opt-in)
PROX_DEFAULT_WAIT_TICKS = 4000000  # bounded in-kernel waits: 40 ms of the 100 MHz clock

_STATUS_NAMES = {0: "PROX_OK", -1: "PROX_ERR_INVALID_ARG", -2: "PROX_ERR_UNSUPPORTED",
                 -3: "PROX_ERR_HIP", -4: "PROX_ERR_INTERNAL"}

EXPORTED = ("prox_abi_version", "prox_last_error", "prox_layer_sizes", "prox_workspace_size",
            "prox_calibrate_workspace_size", "prox_budget_effective", "prox_budget_s2",
            "prox_workspace_init", "prox_pack_proxy", "prox_proxy16_size", "prox_pack_proxy16",
            "prox_proxy_qt_size", "prox_pack_proxy_qt",
            "prox_calibrate", "prox_calibrate_hist_workspace_size", "prox_calibrate_hist", "prox_ffn_decode", "prox_ffn_decode_noalloc", "prox_ffn_decode_events",
            "prox_ffn_decode_stages", "prox_ffn_stage2", "prox_proxy_state", "prox_workspace_check",
            "prox_set_wait_limit")


class ProxError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                      "(python -m free_ffn_activation_amd.build_lib)")
_lib = ctypes.CDLL(LIB_PATH)

_c_i32, _c_f32, _c_size, _c_vp = ctypes.c_int32, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p


class prox_layer(ctypes.Structure):
    _fields_ = [("d_model", _c_i32), ("d_ff", _c_i32), ("wdtype", _c_i32), ("activation", _c_i32),
                ("proxy_q", _c_vp), ("proxy_scale", _c_vp), ("w_upgate_t", _c_vp),
                ("w_down", _c_vp), ("proxy_kind", _c_i32), ("reserved", _c_i32), ("proxy_w16", _c_vp),
                ("proxy_qt", _c_vp)]


_P = ctypes.POINTER
_sig = {
    "prox_abi_version": (_c_i32, []),
    "prox_last_error": (ctypes.c_char_p, []),
    "prox_layer_sizes": (_c_i32, [_c_i32, _c_i32, _c_i32, _P(_c_size)]),
    "prox_workspace_size": (_c_i32, [_c_i32, _c_i32, _c_i32, _P(_c_size)]),
    "prox_budget_effective": (_c_i32, [_c_f32, _c_f32, _c_f32, _P(_c_f32)]),
    "prox_calibrate_hist_workspace_size": (_c_i32, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _P(_c_size)]),
    "prox_calibrate_hist": (_c_i32, [_P(prox_layer), _c_vp, _c_i32, _c_f32, _c_f32, _c_i32, _c_i32,
                                     _P(_c_f32), _P(_c_f32), _c_vp, _c_size, _c_vp]),
    "prox_budget_s2": (_c_i32, [_c_f32, _c_f32, _c_f32, _P(_c_f32)]),
    "prox_calibrate_workspace_size": (_c_i32, [_c_i32, _c_i32, _c_i32, _P(_c_size)]),
    "prox_workspace_init": (_c_i32, [_c_vp, _c_size, _c_vp]),
    "prox_pack_proxy": (_c_i32, [_c_vp, _c_vp, _c_vp, _P(prox_layer), _c_vp]),
    "prox_proxy16_size": (_c_i32, [_c_i32, _c_i32, _c_i32, _P(_c_size)]),
    "prox_pack_proxy16": (_c_i32, [_c_vp, _c_vp, _P(prox_layer), _c_vp]),
    "prox_proxy_qt_size": (_c_i32, [_c_i32, _c_i32, _P(_c_size)]),
    "prox_pack_proxy_qt": (_c_i32, [_P(prox_layer), _c_vp]),
    "prox_calibrate": (_c_i32, [_P(prox_layer), _c_vp, _c_i32, _c_f32, _c_f32, _P(_c_f32),
                                _P(_c_f32), _c_vp, _c_size, _c_vp]),
    "prox_ffn_decode": (_c_i32, [_P(prox_layer), _c_vp, _c_i32, _c_f32, _c_f32, _c_vp, _c_vp,
                                 _c_vp, _c_vp, _c_vp, _c_size, _c_vp]),
    "prox_ffn_decode_noalloc": (_c_i32, [_P(prox_layer), _c_vp, _c_i32, _c_f32, _c_f32, _c_vp, _c_vp,
                                         _c_vp, _c_vp, _c_vp]),
    "prox_ffn_decode_events": (_c_i32, [_P(prox_layer), _c_vp, _c_i32, _c_f32, _c_f32, _c_vp,
                                        _c_vp, _c_vp, _c_vp, _c_vp, _c_size, _c_vp, _P(_c_vp)]),
    "prox_ffn_decode_stages": (_c_i32, [_P(prox_layer), _c_vp, _c_i32, _c_f32, _c_f32, _c_vp,
                                        _c_vp, _c_vp, _c_vp, _c_vp, _c_size, _c_vp, _c_i32]),
    "prox_ffn_stage2": (_c_i32, [_P(prox_layer), _c_vp, _c_i32, _c_vp, _c_vp, _c_vp, _c_vp,
                                 _c_size, _c_vp]),
    "prox_proxy_state": (_c_i32, [_P(prox_layer), _c_vp, _c_i32, _c_f32, _c_vp, _c_vp, _c_vp,
                                  _c_size, _c_vp]),
    "prox_workspace_check": (_c_i32, [_c_vp, _c_size, _c_vp]),
    "prox_set_wait_limit": (_c_i32, [ctypes.c_uint32, _P(ctypes.c_uint32)]),
}
for _name, (_res, _args) in _sig.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


def raw_library() -> ctypes.CDLL:
    return _lib


def _check(status: int) -> None:
    if status != PROX_OK:
        raise ProxError(status, prox_last_error())


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_contiguous():
        raise ValueError("tensors passed to libprox must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _wdtype_of(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return PROX_F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return PROX_BF16
    raise TypeError(f"unsupported element type {t.dtype} (float32 or bf16 bits)")


# ---------------------------------------------------------------- queries
def prox_abi_version() -> int:
    return int(_lib.prox_abi_version())


def prox_last_error() -> str:
    return _lib.prox_last_error().decode("utf-8", "replace")


def prox_budget_effective(s1: float, s2: float, alpha: float) -> float:
    out = _c_f32(0.0)
    _check(_lib.prox_budget_effective(s1, s2, alpha, ctypes.byref(out)))
    return float(out.value)


def prox_budget_s2(e_target: float, s1: float, alpha: float) -> float:
    out = _c_f32(0.0)
    _check(_lib.prox_budget_s2(e_target, s1, alpha, ctypes.byref(out)))
    return float(out.value)


def prox_layer_sizes(d_model: int, d_ff: int, wdtype: int) -> tuple:
    out = (_c_size * 4)()
    _check(_lib.prox_layer_sizes(d_model, d_ff, wdtype, out))
    return tuple(int(v) for v in out)


def prox_workspace_size(d_model: int, d_ff: int, batch: int) -> int:
    out = _c_size()
    _check(_lib.prox_workspace_size(d_model, d_ff, batch, ctypes.byref(out)))
    return int(out.value)


def prox_calibrate_workspace_size(d_model: int, d_ff: int, n_tokens: int) -> int:
    out = _c_size()
    _check(_lib.prox_calibrate_workspace_size(d_model, d_ff, n_tokens, ctypes.byref(out)))
    return int(out.value)


# ---------------------------------------------------------------- buffers
class ProxLayer:
    """Device buffers of one packed layer (allocated by torch) and their
    prox_layer descriptor."""

    def __init__(self, d_model: int, d_ff: int, wdtype: int, device="cuda", activation: int = 0,
                 proxy16: bool = False):
        """proxy16 also allocates the 16-bit proxy buffer (proxy_w16, bf16 layers);
        the descriptor still selects the INT4 proxy until with_proxy_kind()."""
        sizes = prox_layer_sizes(d_model, d_ff, wdtype)
        self.d_model, self.d_ff, self.wdtype, self.activation = d_model, d_ff, wdtype, activation
        self.proxy_kind = PROX_PROXY_INT4
        wt = torch.float32 if wdtype == PROX_F32 else torch.int16
        es = 4 if wdtype == PROX_F32 else 2
        self.proxy_q = torch.empty(sizes[0], dtype=torch.uint8, device=device)
        self.proxy_scale = torch.empty(sizes[1] // 4, dtype=torch.float32, device=device)
        self.w_upgate_t = torch.empty(sizes[2] // es, dtype=wt, device=device)
        self.w_down = torch.empty(sizes[3] // es, dtype=wt, device=device)
        self.proxy_w16 = (torch.zeros(prox_proxy16_size(d_model, d_ff, wdtype), dtype=torch.uint8, device=device)
                          if proxy16 else None)
        self.proxy_qt = None
        self.use_qt = True
        self.desc = self._make_desc()

    def _make_desc(self) -> prox_layer:
        qt = (self.proxy_qt.data_ptr()
              if (self.proxy_qt is not None and self.use_qt and self.proxy_kind == PROX_PROXY_INT4) else None)
        return prox_layer(self.d_model, self.d_ff, self.wdtype, self.activation, self.proxy_q.data_ptr(),
                          self.proxy_scale.data_ptr(), self.w_upgate_t.data_ptr(), self.w_down.data_ptr(),
                          self.proxy_kind, 0, self.proxy_w16.data_ptr() if self.proxy_w16 is not None else None,
                          qt)

    def add_proxy_qt(self, stream=None, device="cuda") -> None:
        """Allocate the channel-major proxy copy (proxy_qt) and fill it from the
        packed proxy_q (call after prox_pack_proxy)."""
        if self.proxy_qt is None:
            self.proxy_qt = torch.empty(prox_proxy_qt_size(self.d_model, self.d_ff), dtype=torch.uint8,
                                        device=device)
            self.desc = self._make_desc()
        prox_pack_proxy_qt(self, stream)

    def with_qt(self, use: bool) -> "ProxLayer":
        """Another descriptor over the same buffers with proxy_qt passed (True)
        or left out (False, so groups take the union-of-rows Stage 1)."""
        other = object.__new__(ProxLayer)
        other.__dict__.update(self.__dict__)
        other.use_qt = use
        other.desc = other._make_desc()
        return other

    def with_activation(self, activation: int) -> "ProxLayer":
        """Another descriptor over the same packed buffers with a different gate
        activation (the packed data does not depend on it)."""
        other = object.__new__(ProxLayer)
        other.__dict__.update(self.__dict__)
        other.activation = activation
        other.desc = other._make_desc()
        return other

    def add_proxy16(self, device="cuda") -> None:
        """Allocate the 16-bit proxy buffer of an existing layer (fill it with
        prox_pack_proxy16, select it with with_proxy_kind)."""
        if self.proxy_w16 is None:
            self.proxy_w16 = torch.zeros(prox_proxy16_size(self.d_model, self.d_ff, self.wdtype),
                                         dtype=torch.uint8, device=device)
            self.desc = self._make_desc()

    def with_proxy_kind(self, kind: int) -> "ProxLayer":
        """Another descriptor over the same buffers whose Stage 1 reads the given
        proxy (PROX_PROXY_INT4 or PROX_PROXY_W16)."""
        if kind == PROX_PROXY_W16 and self.proxy_w16 is None:
            raise ValueError("this layer has no 16-bit proxy buffer (ProxLayer(..., proxy16=True))")
        other = object.__new__(ProxLayer)
        other.__dict__.update(self.__dict__)
        other.proxy_kind = kind
        other.desc = other._make_desc()
        return other

    @property
    def nbytes(self) -> int:
        bufs = [self.proxy_q, self.proxy_scale, self.w_upgate_t, self.w_down]
        if self.proxy_w16 is not None:
            bufs.append(self.proxy_w16)
        if self.proxy_qt is not None:
            bufs.append(self.proxy_qt)
        return sum(t.numel() * t.element_size() for t in bufs)


def new_workspace(d_model: int, d_ff: int, batch: int, device="cuda") -> torch.Tensor:
    """Zero-filled decode workspace (torch allocation, 256-byte aligned)."""
    n = prox_workspace_size(d_model, d_ff, batch)
    return torch.zeros(n, dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- entry points
def prox_workspace_init(ws: torch.Tensor, stream=None) -> None:
    _check(_lib.prox_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def prox_pack_proxy(W_up: torch.Tensor, W_gate: torch.Tensor, W_down: torch.Tensor,
                    layer: ProxLayer, stream=None) -> None:
    d, f = layer.d_model, layer.d_ff
    for t, shape in ((W_up, (d, f)), (W_gate, (d, f)), (W_down, (f, d))):
        if tuple(t.shape) != shape or _wdtype_of(t) != layer.wdtype:
            raise ValueError(f"weight of shape {tuple(t.shape)} / {t.dtype}, expected {shape}")
    _check(_lib.prox_pack_proxy(_ptr(W_up), _ptr(W_gate), _ptr(W_down), ctypes.byref(layer.desc),
                                _stream(stream)))


def prox_proxy16_size(d_model: int, d_ff: int, wdtype: int) -> int:
    out = _c_size()
    _check(_lib.prox_proxy16_size(d_model, d_ff, wdtype, ctypes.byref(out)))
    return int(out.value)


def prox_pack_proxy16(W_up: torch.Tensor, W_gate: torch.Tensor, layer: ProxLayer, stream=None) -> None:
    d, f = layer.d_model, layer.d_ff
    for t in (W_up, W_gate):
        if tuple(t.shape) != (d, f) or _wdtype_of(t) != layer.wdtype:
            raise ValueError(f"weight of shape {tuple(t.shape)} / {t.dtype}, expected {(d, f)}")
    if layer.proxy_w16 is None:
        raise ValueError("layer has no 16-bit proxy buffer (ProxLayer(..., proxy16=True))")
    _check(_lib.prox_pack_proxy16(_ptr(W_up), _ptr(W_gate), ctypes.byref(layer.desc), _stream(stream)))


def prox_proxy_qt_size(d_model: int, d_ff: int) -> int:
    out = _c_size()
    _check(_lib.prox_proxy_qt_size(d_model, d_ff, ctypes.byref(out)))
    return int(out.value)


def prox_pack_proxy_qt(layer: ProxLayer, stream=None) -> None:
    if layer.proxy_qt is None:
        raise ValueError("layer has no proxy_qt buffer (ProxLayer.add_proxy_qt)")
    desc = layer.desc if layer.use_qt else layer.with_qt(True).desc
    _check(_lib.prox_pack_proxy_qt(ctypes.byref(desc), _stream(stream)))


def prox_calibrate(layer: ProxLayer, X_cal: torch.Tensor, keep_x: float, sparsity_s: float,
                   ws: torch.Tensor, stream=None) -> tuple:
    if X_cal.dim() != 2 or X_cal.shape[1] != layer.d_model or _wdtype_of(X_cal) != layer.wdtype:
        raise ValueError("X_cal must be [n_tokens, d_model] in the layer dtype")
    tx, ts = _c_f32(), _c_f32()
    _check(_lib.prox_calibrate(ctypes.byref(layer.desc), _ptr(X_cal), X_cal.shape[0], keep_x,
                               sparsity_s, ctypes.byref(tx), ctypes.byref(ts), _ptr(ws),
                               ws.numel() * ws.element_size(), _stream(stream)))
    return float(tx.value), float(ts.value)


def prox_calibrate_hist_workspace_size(d_model: int, d_ff: int, n_tokens: int, max_samples: int = 200000,
                                       n_bins: int = 4096) -> int:
    out = _c_size(0)
    _check(_lib.prox_calibrate_hist_workspace_size(d_model, d_ff, n_tokens, max_samples, n_bins,
                                                   ctypes.byref(out)))
    return int(out.value)


def prox_calibrate_hist(layer: ProxLayer, X_cal: torch.Tensor, keep_x: float, sparsity_s: float,
                        ws: torch.Tensor, max_samples: int = 200000, n_bins: int = 4096, stream=None):
    """Histogram calibration (blocking).  Returns (tau_x, tau_s)."""
    if X_cal.dim() != 2 or X_cal.shape[1] != layer.d_model or _wdtype_of(X_cal) != layer.wdtype:
        raise ValueError("X_cal must be [n_tokens, d_model] in the layer dtype")
    tx, ts = _c_f32(0.0), _c_f32(0.0)
    _check(_lib.prox_calibrate_hist(ctypes.byref(layer.desc), _ptr(X_cal), X_cal.shape[0], keep_x, sparsity_s,
                                    max_samples, n_bins, ctypes.byref(tx), ctypes.byref(ts), _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(stream)))
    return float(tx.value), float(ts.value)


def _decode_args(layer, x, y, mask_idx, mask_count, in_count):
    if x.dim() != 2 or x.shape[1] != layer.d_model or _wdtype_of(x) != layer.wdtype:
        raise ValueError("x must be [batch, d_model] in the layer dtype")
    b = x.shape[0]
    if tuple(y.shape) != (b, layer.d_model) or y.dtype != torch.float32:
        raise ValueError("y must be float32 [batch, d_model]")
    if tuple(mask_idx.shape) != (b, layer.d_ff) or mask_idx.dtype != torch.int32:
        raise ValueError("mask_idx must be int32 [batch, d_ff]")
    if tuple(mask_count.shape) != (b,) or mask_count.dtype != torch.int32:
        raise ValueError("mask_count must be int32 [batch]")
    if in_count is not None and (tuple(in_count.shape) != (b,) or in_count.dtype != torch.int32):
        raise ValueError("in_count must be int32 [batch]")
    return b


def prox_ffn_decode(layer: ProxLayer, x: torch.Tensor, tau_x: float, tau_s: float,
                    y: torch.Tensor, mask_idx: torch.Tensor, mask_count: torch.Tensor,
                    in_count: torch.Tensor | None, ws: torch.Tensor, stream=None) -> None:
    b = _decode_args(layer, x, y, mask_idx, mask_count, in_count)
    _check(_lib.prox_ffn_decode(ctypes.byref(layer.desc), _ptr(x), b, tau_x, tau_s, _ptr(y),
                                _ptr(mask_idx), _ptr(mask_count), _ptr(in_count), _ptr(ws),
                                ws.numel() * ws.element_size(), _stream(stream)))


PROX_NOALLOC_SCRATCH_BYTES = 32 << 20


def prox_ffn_decode_noalloc(layer: ProxLayer, x: torch.Tensor, tau_x: float, tau_s: float,
                            y: torch.Tensor, mask_idx: torch.Tensor, mask_count: torch.Tensor,
                            in_count: torch.Tensor | None, stream=None) -> None:
    """prox_ffn_decode on the library's per-GPU scratch array (no workspace)."""
    b = _decode_args(layer, x, y, mask_idx, mask_count, in_count)
    _check(_lib.prox_ffn_decode_noalloc(ctypes.byref(layer.desc), _ptr(x), b, tau_x, tau_s, _ptr(y),
                                        _ptr(mask_idx), _ptr(mask_count), _ptr(in_count), _stream(stream)))


def prox_ffn_decode_events(layer: ProxLayer, x: torch.Tensor, tau_x: float, tau_s: float,
                           y: torch.Tensor, mask_idx: torch.Tensor, mask_count: torch.Tensor,
                           in_count: torch.Tensor | None, ws: torch.Tensor, events,
                           stream=None) -> None:
    """events: four torch.cuda.Event(enable_timing=True) recorded around the
    three kernels (before Stage 1, after Stage 1, after up/gate, after down)."""
    b = _decode_args(layer, x, y, mask_idx, mask_count, in_count)
    handles = (_c_vp * 4)(*[ctypes.c_void_p(ev.cuda_event) for ev in events])
    _check(_lib.prox_ffn_decode_events(ctypes.byref(layer.desc), _ptr(x), b, tau_x, tau_s,
                                       _ptr(y), _ptr(mask_idx), _ptr(mask_count), _ptr(in_count),
                                       _ptr(ws), ws.numel() * ws.element_size(), _stream(stream),
                                       handles))


def prox_ffn_decode_stages(layer: ProxLayer, x: torch.Tensor, tau_x: float, tau_s: float,
                           y: torch.Tensor, mask_idx: torch.Tensor, mask_count: torch.Tensor,
                           in_count: torch.Tensor | None, ws: torch.Tensor, stages: int,
                           stream=None) -> None:
    """Run the decode kernels selected by `stages` (PROX_STAGE_* bits)."""
    b = _decode_args(layer, x, y, mask_idx, mask_count, in_count)
    _check(_lib.prox_ffn_decode_stages(ctypes.byref(layer.desc), _ptr(x), b, tau_x, tau_s, _ptr(y),
                                       _ptr(mask_idx), _ptr(mask_count), _ptr(in_count), _ptr(ws),
                                       ws.numel() * ws.element_size(), _stream(stream), stages))


def prox_ffn_stage2(layer: ProxLayer, x: torch.Tensor, mask_idx: torch.Tensor,
                    mask_count: torch.Tensor, y: torch.Tensor, ws: torch.Tensor,
                    stream=None) -> None:
    b = _decode_args(layer, x, y, mask_idx, mask_count, None)
    _check(_lib.prox_ffn_stage2(ctypes.byref(layer.desc), _ptr(x), b, _ptr(mask_idx),
                                _ptr(mask_count), _ptr(y), _ptr(ws),
                                ws.numel() * ws.element_size(), _stream(stream)))


def prox_proxy_state(layer: ProxLayer, x: torch.Tensor, tau_x: float, s_tilde: torch.Tensor,
                     in_count: torch.Tensor | None, ws: torch.Tensor, stream=None) -> None:
    if x.dim() != 2 or x.shape[1] != layer.d_model or _wdtype_of(x) != layer.wdtype:
        raise ValueError("x must be [batch, d_model] in the layer dtype")
    b = x.shape[0]
    if tuple(s_tilde.shape) != (b, layer.d_ff) or s_tilde.dtype != torch.float32:
        raise ValueError("s_tilde must be float32 [batch, d_ff]")
    _check(_lib.prox_proxy_state(ctypes.byref(layer.desc), _ptr(x), b, tau_x, _ptr(s_tilde),
                                 _ptr(in_count), _ptr(ws), ws.numel() * ws.element_size(),
                                 _stream(stream)))


def prox_workspace_check(ws: torch.Tensor, stream=None) -> None:
    """Raises ProxError(PROX_ERR_INTERNAL) when a decode on ws gave up a
    bounded wait (and clears the error word).  Blocking."""
    _check(_lib.prox_workspace_check(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def prox_set_wait_limit(ticks: int) -> int:
    """Bound of the in-kernel waits (100 MHz clock ticks); returns the old one."""
    prev = ctypes.c_uint32(0)
    _check(_lib.prox_set_wait_limit(int(ticks), ctypes.byref(prev)))
    return int(prev.value)
