"""Python binding of libxlrel.so, the MI355X (gfx950) Transformer-XL relative
attention forward. Argument marshalling only: every step of the computation
runs in the library's HIP kernels. PyTorch supplies device memory and streams.

The names mirror the C ABI in include/xl_rel.h.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
# XL_LIB names another build of the same sources (the host-sanitizer build)
LIB_PATH = os.environ.get("XL_LIB") or os.path.join(_HERE, "libxlrel.so")

XL_OK, XL_NULL_ARG, XL_BAD_SHAPE, XL_UNSUPPORTED, XL_WORKSPACE_TOO_SMALL, XL_HIP_ERROR = range(6)
XL_F32, XL_BF16 = 0, 1
XL_BIAS_CLAMP, XL_BIAS_T5 = 0, 1
XL_T5_BUCKETS = 12
XL_REUSE_TABLE = 1

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


class xl_attn_desc(ctypes.Structure):
    _fields_ = [("batch", _i64), ("d_model", _i64), ("n_head", _i64), ("d_head", _i64),
                ("qlen", _i64), ("mlen", _i64), ("clamp_len", _i64), ("bias_clamp", _i64),
                ("base", ctypes.c_double), ("scale", ctypes.c_float),
                ("dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32), ("attn_splits", ctypes.c_int32),
                ("bias_kind", ctypes.c_int32), ("flags", ctypes.c_int32)]


class xl_attn_weights(ctypes.Structure):
    _fields_ = [(n, _p) for n in ("w_q", "w_k", "w_v", "w_r", "w_o", "u", "v", "bias_table")]


class xl_ws_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("q", "k", "vt", "rel", "r", "attn", "part", "total")] + \
               [("klen", _i64), ("ldv", _i64), ("n_rel", _i64)]


class xl_mem_fifo(ctypes.Structure):
    _fields_ = [("buf", _p), ("mlen_max", _i64), ("len", _i64), ("head", _i64)]


class xl_kv_fifo(ctypes.Structure):
    _fields_ = [("k", _p), ("vt", _p), ("cap", _i64), ("mlen_max", _i64), ("len", _i64), ("head", _i64)]


class XLError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_STATUS.get(status, status)}: {detail}")
        self.status = status


_STATUS = {0: "XL_OK", 1: "XL_NULL_ARG", 2: "XL_BAD_SHAPE", 3: "XL_UNSUPPORTED",
           4: "XL_WORKSPACE_TOO_SMALL", 5: "XL_HIP_ERROR"}

_lib = None

EXPORTS = ("xl_status_string", "xl_last_error", "xl_relpos_embed", "xl_rel_attn_workspace_size",
           "xl_rel_attn_workspace_layout", "xl_rel_attn_fwd", "xl_rel_attn_core_workspace_size", "xl_rel_attn_core",
           "xl_segment_step", "xl_segment_step_kv_workspace_size", "xl_segment_step_kv", "xl_set_core_events",
           "xl_rel_attn_core_bwd_workspace_size", "xl_rel_attn_core_bwd", "xl_decoder_layer_workspace_size", "xl_decoder_layer_fwd", "xl_decoder_stack_workspace_size",
           "xl_decoder_stack_step", "xl_segment_step_noalloc", "xl_decoder_stack_kv_workspace_size",
           "xl_decoder_stack_step_kv")

# bytes of the static scratch of xl_segment_step_noalloc (XL_NOALLOC_SCRATCH_BYTES)
XL_NOALLOC_SCRATCH_BYTES = 64 << 20


def lib():
    """Load libxlrel.so. Fails loudly when it has not been built: there is no
    fallback implementation."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`"
                              " (or transformer_xl_relative_amd/build.py)")
        # One HIP runtime per process: PyTorch ships its own libamdhip64 and
        # loads it under its own file name, so it must be loaded before this
        # library, whose dependency then binds to that same runtime. Loading
        # /opt/rocm's runtime first would leave two runtimes in the process.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        L.xl_status_string.argtypes = [ctypes.c_int]
        L.xl_status_string.restype = ctypes.c_char_p
        L.xl_last_error.argtypes = []
        L.xl_last_error.restype = ctypes.c_char_p
        L.xl_relpos_embed.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_double, ctypes.c_int, _p, _p]
        L.xl_rel_attn_workspace_size.argtypes = [ctypes.POINTER(xl_attn_desc)]
        L.xl_rel_attn_workspace_size.restype = ctypes.c_size_t
        L.xl_rel_attn_workspace_layout.argtypes = [ctypes.POINTER(xl_attn_desc), ctypes.POINTER(xl_ws_layout)]
        L.xl_rel_attn_fwd.argtypes = [ctypes.POINTER(xl_attn_desc), ctypes.POINTER(xl_attn_weights), _p, _p, _p,
                                      _p, ctypes.c_size_t, _p]
        L.xl_rel_attn_core_workspace_size.argtypes = [ctypes.POINTER(xl_attn_desc)]
        L.xl_rel_attn_core_workspace_size.restype = ctypes.c_size_t
        L.xl_rel_attn_core.argtypes = [ctypes.POINTER(xl_attn_desc), _p, _p, _p, _i64, _p, _i64, _p, _p, _p, _p, _p,
                                       ctypes.c_size_t, _p]
        L.xl_segment_step.argtypes = [ctypes.POINTER(xl_attn_desc), ctypes.POINTER(xl_attn_weights), _p,
                                      ctypes.POINTER(xl_mem_fifo), _p, _p, ctypes.c_size_t, _p]
        L.xl_segment_step_noalloc.argtypes = [ctypes.POINTER(xl_attn_desc), ctypes.POINTER(xl_attn_weights), _p,
                                              ctypes.POINTER(xl_mem_fifo), _p, _p]
        L.xl_set_core_events.argtypes = [_p, _p]
        L.xl_segment_step_kv_workspace_size.argtypes = [ctypes.POINTER(xl_attn_desc)]
        L.xl_segment_step_kv_workspace_size.restype = ctypes.c_size_t
        L.xl_segment_step_kv.argtypes = [ctypes.POINTER(xl_attn_desc), ctypes.POINTER(xl_attn_weights), _p,
                                         ctypes.POINTER(xl_kv_fifo), _p, _p, ctypes.c_size_t, _p]
        D = ctypes.POINTER(xl_attn_desc)
        L.xl_rel_attn_core_bwd_workspace_size.argtypes = [D]
        L.xl_rel_attn_core_bwd_workspace_size.restype = ctypes.c_size_t
        L.xl_rel_attn_core_bwd.argtypes = [D, _p, _p, _p, _i64, _p, _i64, _p, _p, _p, _p] + [_p] * 8 + \
            [ctypes.c_size_t, _p]
        L.xl_decoder_layer_workspace_size.argtypes = [D, _i64]
        L.xl_decoder_layer_workspace_size.restype = ctypes.c_size_t
        L.xl_decoder_layer_fwd.argtypes = [D, _i64, ctypes.c_float, ctypes.POINTER(xl_decoder_weights), _p, _p, _p,
                                           _p, ctypes.c_size_t, _p]
        L.xl_decoder_stack_workspace_size.argtypes = [D, _i64]
        L.xl_decoder_stack_workspace_size.restype = ctypes.c_size_t
        L.xl_decoder_stack_step.argtypes = [D, _i64, ctypes.c_float, _i64, ctypes.POINTER(xl_decoder_weights), _p,
                                            ctypes.POINTER(xl_mem_fifo), _p, _p, ctypes.c_size_t, _p]
        L.xl_decoder_stack_kv_workspace_size.argtypes = [D, _i64]
        L.xl_decoder_stack_kv_workspace_size.restype = ctypes.c_size_t
        L.xl_decoder_stack_step_kv.argtypes = [D, _i64, ctypes.c_float, _i64, ctypes.POINTER(xl_decoder_weights), _p,
                                               ctypes.POINTER(xl_kv_fifo), _p, _p, ctypes.c_size_t, _p]
        for f in ("xl_relpos_embed", "xl_rel_attn_workspace_layout", "xl_rel_attn_fwd", "xl_rel_attn_core",
                  "xl_segment_step", "xl_set_core_events", "xl_segment_step_kv", "xl_decoder_layer_fwd",
                  "xl_rel_attn_core_bwd", "xl_segment_step_noalloc",
                  "xl_decoder_stack_step", "xl_decoder_stack_step_kv"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int):
    if status != XL_OK:
        raise XLError(status, lib().xl_last_error().decode())


def _ptr(t) -> Optional[int]:
    """Device address of a tensor (None stays NULL; ints pass through)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to libxlrel must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_desc(*, batch, d_model, n_head, d_head, qlen, mlen=0, clamp_len=-1, bias_clamp=-1, base=10000.0,
              scale=0.0, dtype=XL_BF16, out_dtype=None, attn_splits=0, bias_kind=0, flags=0) -> xl_attn_desc:
    return xl_attn_desc(batch, d_model, n_head, d_head, qlen, mlen, clamp_len, bias_clamp, base, scale,
                        dtype, dtype if out_dtype is None else out_dtype, attn_splits, bias_kind, flags)


@dataclasses.dataclass
class Weights:
    """Layer weights as device tensors ([out, in] projection layout)."""
    w_q: object
    w_k: object
    w_v: object
    w_r: object
    w_o: object
    u: object
    v: object
    bias_table: object = None

    def c(self) -> xl_attn_weights:
        return xl_attn_weights(*[_ptr(getattr(self, f)) for f in
                                 ("w_q", "w_k", "w_v", "w_r", "w_o", "u", "v", "bias_table")])


class xl_decoder_weights(ctypes.Structure):
    _fields_ = [("attn", xl_attn_weights)] + [(n, _p) for n in ("ln1_g", "ln1_b", "ln2_g", "ln2_b", "w1", "b1", "w2",
                                                                "b2")]


@dataclasses.dataclass
class DecoderWeights:
    """Weights of one pre-LN decoder layer as device tensors."""
    attn: Weights
    ln1_g: object
    ln1_b: object
    ln2_g: object
    ln2_b: object
    w1: object
    b1: object
    w2: object
    b2: object

    def c(self) -> xl_decoder_weights:
        return xl_decoder_weights(self.attn.c(), *[_ptr(getattr(self, f)) for f in
                                                   ("ln1_g", "ln1_b", "ln2_g", "ln2_b", "w1", "b1", "w2", "b2")])


def xl_relpos_embed(delta0: int, n_rows: int, d_model: int, clamp_len: int, base: float, out, stream=None):
    dt = XL_BF16 if str(out.dtype) == "torch.bfloat16" else XL_F32
    _check(lib().xl_relpos_embed(delta0, n_rows, d_model, clamp_len, base, dt, _ptr(out), _stream(stream)))
    return out


def xl_rel_attn_workspace_size(desc: xl_attn_desc) -> int:
    return lib().xl_rel_attn_workspace_size(ctypes.byref(desc))


def xl_rel_attn_workspace_layout(desc: xl_attn_desc) -> xl_ws_layout:
    lay = xl_ws_layout()
    _check(lib().xl_rel_attn_workspace_layout(ctypes.byref(desc), ctypes.byref(lay)))
    return lay


def xl_rel_attn_fwd(desc: xl_attn_desc, weights: Weights, h, mem, out, ws, stream=None):
    cw = weights.c() if isinstance(weights, Weights) else weights
    _check(lib().xl_rel_attn_fwd(ctypes.byref(desc), ctypes.byref(cw), _ptr(h), _ptr(mem), _ptr(out), _ptr(ws),
                                 ws.numel() * ws.element_size(), _stream(stream)))
    return out


def xl_rel_attn_core_workspace_size(desc: xl_attn_desc) -> int:
    return lib().xl_rel_attn_core_workspace_size(ctypes.byref(desc))


def xl_rel_attn_core(desc: xl_attn_desc, q, k, vt, ldv: int, r, n_rel: int, u, v, bias_table, attn, ws=None,
                     stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().xl_rel_attn_core(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(vt), ldv, _ptr(r), n_rel, _ptr(u),
                                  _ptr(v), _ptr(bias_table), _ptr(attn), _ptr(ws), nbytes, _stream(stream)))
    return attn


def xl_segment_step(desc: xl_attn_desc, weights: Weights, h, fifo: xl_mem_fifo, out, ws, stream=None):
    cw = weights.c() if isinstance(weights, Weights) else weights
    _check(lib().xl_segment_step(ctypes.byref(desc), ctypes.byref(cw), _ptr(h), ctypes.byref(fifo), _ptr(out),
                                 _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return out


def xl_segment_step_noalloc(desc: xl_attn_desc, weights: Weights, h, fifo: xl_mem_fifo, out, stream=None):
    cw = weights.c() if isinstance(weights, Weights) else weights
    _check(lib().xl_segment_step_noalloc(ctypes.byref(desc), ctypes.byref(cw), _ptr(h), ctypes.byref(fifo),
                                         _ptr(out), _stream(stream)))
    return out


def xl_segment_step_kv_workspace_size(desc: xl_attn_desc) -> int:
    return lib().xl_segment_step_kv_workspace_size(ctypes.byref(desc))


def xl_segment_step_kv(desc: xl_attn_desc, weights: Weights, h, kv: xl_kv_fifo, out, ws, stream=None):
    cw = weights.c() if isinstance(weights, Weights) else weights
    _check(lib().xl_segment_step_kv(ctypes.byref(desc), ctypes.byref(cw), _ptr(h), ctypes.byref(kv), _ptr(out),
                                    _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return out


def xl_set_core_events(ev_begin, ev_end):
    """Record two torch.cuda.Event (or raw hipEvent_t) around the next fused
    attention launches on this thread; None, None turns it off."""
    b = ev_begin.cuda_event if hasattr(ev_begin, "cuda_event") else ev_begin
    e = ev_end.cuda_event if hasattr(ev_end, "cuda_event") else ev_end
    _check(lib().xl_set_core_events(b, e))


class HipEvent:
    """A raw hipEvent_t of the process's HIP runtime (the one torch loaded), for
    timing with xl_set_core_events: hipEventCreate / hipEventElapsedTime."""
    _rt = None

    @classmethod
    def _runtime(cls):
        if cls._rt is None:
            lib()   # torch first, then the runtime libxlrel is bound to
            rt = ctypes.CDLL("libamdhip64.so.7")
            rt.hipEventCreate.argtypes = [ctypes.POINTER(_p)]
            rt.hipEventDestroy.argtypes = [_p]
            rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), _p, _p]
            rt.hipEventRecord.argtypes = [_p, _p]
            cls._rt = rt
        return cls._rt

    def __init__(self):
        self.handle = _p()
        st = self._runtime().hipEventCreate(ctypes.byref(self.handle))
        if st != 0:
            raise XLError(XL_HIP_ERROR, f"hipEventCreate failed ({st})")

    @property
    def cuda_event(self):
        return self.handle.value

    def record(self, stream=None):
        st = self._runtime().hipEventRecord(self.handle, _stream(stream))
        if st != 0:
            raise XLError(XL_HIP_ERROR, f"hipEventRecord failed ({st})")

    def elapsed_ms(self, end: "HipEvent") -> float:
        ms = ctypes.c_float()
        st = self._runtime().hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle)
        if st != 0:
            raise XLError(XL_HIP_ERROR, f"hipEventElapsedTime failed ({st})")
        return ms.value

    def __del__(self):
        if self._rt is not None and self.handle:
            self._rt.hipEventDestroy(self.handle)


def xl_decoder_layer_workspace_size(desc: xl_attn_desc, d_inner: int) -> int:
    return lib().xl_decoder_layer_workspace_size(ctypes.byref(desc), d_inner)


def xl_decoder_layer_fwd(desc: xl_attn_desc, d_inner: int, ln_eps: float, weights, h, mem, out, ws, stream=None):
    cw = weights.c() if isinstance(weights, DecoderWeights) else weights
    _check(lib().xl_decoder_layer_fwd(ctypes.byref(desc), d_inner, ln_eps, ctypes.byref(cw), _ptr(h), _ptr(mem),
                                      _ptr(out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return out


def xl_decoder_stack_workspace_size(desc: xl_attn_desc, d_inner: int) -> int:
    return lib().xl_decoder_stack_workspace_size(ctypes.byref(desc), d_inner)


def xl_decoder_stack_step(desc: xl_attn_desc, d_inner: int, ln_eps: float, weights: list, h, fifos, out, ws,
                          stream=None):
    """weights: one DecoderWeights (or xl_decoder_weights) per layer; fifos: a
    ctypes array of xl_mem_fifo (updated in place)."""
    n = len(weights)
    cw = (xl_decoder_weights * n)(*[w.c() if isinstance(w, DecoderWeights) else w for w in weights])
    if len(fifos) != n:
        raise ValueError("one fifo per layer")
    _check(lib().xl_decoder_stack_step(ctypes.byref(desc), d_inner, ln_eps, n, cw, _ptr(h), fifos, _ptr(out),
                                       _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return out


def xl_decoder_stack_kv_workspace_size(desc: xl_attn_desc, d_inner: int) -> int:
    return lib().xl_decoder_stack_kv_workspace_size(ctypes.byref(desc), d_inner)


def xl_decoder_stack_step_kv(desc: xl_attn_desc, d_inner: int, ln_eps: float, weights: list, h, rings, out, ws,
                             stream=None):
    """weights: one DecoderWeights (or xl_decoder_weights) per layer; rings: a
    ctypes array of xl_kv_fifo (updated in place)."""
    n = len(weights)
    cw = (xl_decoder_weights * n)(*[w.c() if isinstance(w, DecoderWeights) else w for w in weights])
    if len(rings) != n:
        raise ValueError("one ring per layer")
    _check(lib().xl_decoder_stack_step_kv(ctypes.byref(desc), d_inner, ln_eps, n, cw, _ptr(h), rings, _ptr(out),
                                          _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return out


def xl_rel_attn_core_bwd_workspace_size(desc: xl_attn_desc) -> int:
    return lib().xl_rel_attn_core_bwd_workspace_size(ctypes.byref(desc))


def xl_rel_attn_core_bwd(desc: xl_attn_desc, q, k, vt, ldv: int, r, n_rel: int, u, v, bias_table, dout, grads: dict,
                         ws, stream=None):
    """grads: fp32 device tensors dq, dk, dv, dr, du, dv_bias (and dbias with a
    bias table), overwritten."""
    _check(lib().xl_rel_attn_core_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(vt), ldv, _ptr(r), n_rel, _ptr(u),
                                      _ptr(v), _ptr(bias_table), _ptr(dout), _ptr(grads["dq"]), _ptr(grads["dk"]),
                                      _ptr(grads["dv"]), _ptr(grads["dr"]), _ptr(grads["du"]),
                                      _ptr(grads["dv_bias"]), _ptr(grads.get("dbias")), _ptr(ws),
                                      ws.numel() * ws.element_size(), _stream(stream)))
    return grads
