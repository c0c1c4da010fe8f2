"""NumPy front end of the fp64 CPU oracle (oracle/xl_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the GPU library. The C code does all of
the arithmetic; this module only marshals float64 arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# XL_ORACLE_LIB names another build of the same source (the sanitizer build)
_LIB_PATH = os.environ.get("XL_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

_i64 = ctypes.c_int64
_dbl = ctypes.c_double
_p = ctypes.c_void_p


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build
            _build.build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.orc_relpos_embed.argtypes = [_i64, _i64, _i64, _i64, _dbl, _p]
        lib.orc_linear.argtypes = [_p, _i64, _i64, _p, _i64, _p]
        lib.orc_rel_attn_core.argtypes = [_i64] * 5 + [_p, _p, _i64, _i64, _i64, _dbl] + [_p] * 4 + [_i64, _i64] + \
            [_p] * 6
        lib.orc_rel_attn_fwd.argtypes = [_i64] * 9 + [_dbl, _dbl] + [_p] * 15
        lib.orc_t5_bucket.argtypes = [_i64]
        lib.orc_t5_bucket.restype = _i64
        lib.orc_fifo_update.argtypes = [_i64, _i64, _i64, _i64, _p, _i64, _p, _p, ctypes.POINTER(_i64)]
        lib.orc_rel_attn_core_bwd.argtypes = [_i64] * 8 + [_dbl] + [_p] * 4 + [_i64] + [_p] * 11
        lib.orc_rel_attn_core_bwd.restype = ctypes.c_int
        lib.orc_layer_norm.argtypes = [_i64, _i64, _p, _p, _p, _dbl, _p]
        lib.orc_layer_norm.restype = ctypes.c_int
        lib.orc_num_threads.argtypes = []
        lib.orc_num_threads.restype = ctypes.c_int
        for f in ("orc_relpos_embed", "orc_linear", "orc_rel_attn_core", "orc_rel_attn_fwd", "orc_fifo_update"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _i64arr(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int64)


def _ptr(a):
    return None if a is None else a.ctypes.data


class OracleError(RuntimeError):
    pass


def _check(status, what):
    if status != 0:
        raise OracleError(f"{what} returned status {status}")


def t5_bucket(delta: int) -> int:
    """T5 bucket of a relative distance (12 buckets)."""
    return int(_load().orc_t5_bucket(int(delta)))


def num_threads() -> int:
    """OpenMP threads the oracle uses."""
    return int(_load().orc_num_threads())


def relpos_embed(delta0: int, n_rows: int, d_model: int, clamp_len: int = -1, base: float = 10000.0):
    """Rows R_{clamp(delta0+n)} of the sinusoidal relative embedding, [n_rows, d_model]."""
    out = np.empty((n_rows, d_model), np.float64)
    _check(_load().orc_relpos_embed(delta0, n_rows, d_model, clamp_len, base, _ptr(out)), "orc_relpos_embed")
    return out


def linear(x, W):
    """x @ W^T with W stored [out, in]."""
    x = _f64(x)
    W = _f64(W)
    lead = x.shape[:-1]
    x2 = x.reshape(-1, x.shape[-1])
    y = np.empty((x2.shape[0], W.shape[0]), np.float64)
    _check(_load().orc_linear(_ptr(x2), x2.shape[0], x2.shape[1], _ptr(W), W.shape[0], _ptr(y)), "orc_linear")
    return y.reshape(*lead, W.shape[0])


def rel_attn_core(q, k, v, rtab, u, vb, *, scale: float, clamp_len: int = -1, rtab_delta0: int = 0,
                  beta=None, bias_clamp: int = -1, bias_kind: int = 0, qpos=None, kpos=None,
                  want_terms: bool = False, want_probs: bool = False):
    """Attention core on head-major q [B,H,q,dh], k/v [B,H,klen,dh] and a projected
    relative table rtab [H, n, dh] (row n <-> clamped distance rtab_delta0+n).
    beta is the scalar bias table: [2*bias_clamp+1, H] rows by clamped distance
    (bias_kind 0) or [12, H] rows by T5 bucket (bias_kind 1). Returns o [B, q, H*dh] (and optionally the four terms
    [4,B,H,q,klen], probs)."""
    q, k, v, rtab, u, vb, beta = map(_f64, (q, k, v, rtab, u, vb, beta))
    B, H, ql, dh = q.shape
    kl = k.shape[2]
    o = np.empty((B, ql, H * dh), np.float64)
    terms = np.empty((4, B, H, ql, kl), np.float64) if want_terms else None
    probs = np.empty((B, H, ql, kl), np.float64) if want_probs else None
    qpos, kpos = _i64arr(qpos), _i64arr(kpos)
    st = _load().orc_rel_attn_core(B, H, dh, ql, kl, _ptr(qpos), _ptr(kpos), clamp_len, bias_clamp, bias_kind,
                                   scale,
                                   _ptr(q), _ptr(k), _ptr(v), _ptr(rtab), rtab_delta0, rtab.shape[1],
                                   _ptr(u), _ptr(vb), _ptr(beta), _ptr(o), _ptr(terms), _ptr(probs))
    _check(st, "orc_rel_attn_core")
    res = [o]
    if want_terms:
        res.append(terms)
    if want_probs:
        res.append(probs)
    return res[0] if len(res) == 1 else tuple(res)


def rel_attn_core_bwd(q, k, v, rtab, u, vb, dout, *, scale: float, clamp_len: int = -1, beta=None,
                      bias_clamp: int = -1, bias_kind: int = 0):
    """Gradients of the attention core for the upstream gradient dout
    [B, qlen, H*dh] of its output: a dict with dq [B,H,q,dh], dk, dv
    [B,H,klen,dh], dr [H,n,dh] (per table row), du, dv_bias [H,dh] and dbeta
    (or None). Default positions (query i at mlen+i, key j at j)."""
    q, k, v, rtab, u, vb, beta, dout = map(_f64, (q, k, v, rtab, u, vb, beta, dout))
    B, H, ql, dh = q.shape
    kl = k.shape[2]
    out = {"dq": np.empty_like(q), "dk": np.empty_like(k), "dv": np.empty_like(v), "dr": np.empty_like(rtab),
           "du": np.empty_like(u), "dv_bias": np.empty_like(vb),
           "dbeta": np.empty_like(beta) if beta is not None else None}
    st = _load().orc_rel_attn_core_bwd(B, H, dh, ql, kl, clamp_len, bias_clamp, bias_kind, scale, _ptr(q), _ptr(k),
                                       _ptr(v), _ptr(rtab), rtab.shape[1], _ptr(u), _ptr(vb), _ptr(beta),
                                       _ptr(dout), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                                       _ptr(out["dr"]), _ptr(out["du"]), _ptr(out["dv_bias"]), _ptr(out["dbeta"]))
    _check(st, "orc_rel_attn_core_bwd")
    return out


def rel_attn_fwd(h, mem, w_q, w_k, w_v, w_r, w_o, u, vb, *, n_head: int, d_head: int,
                 clamp_len: int = -1, beta=None, bias_clamp: int = -1, bias_kind: int = 0,
                 scale: float | None = None, base: float = 10000.0, qpos=None, kpos=None, want_terms=False, want_probs=False):
    """Full layer: out [B, qlen, D] from h [B, qlen, D] and mem [B, mlen, D]."""
    h = _f64(h)
    B, ql, D = h.shape
    mem = _f64(mem) if mem is not None and mem.shape[1] > 0 else None
    ml = 0 if mem is None else mem.shape[1]
    kl = ql + ml
    w_q, w_k, w_v, w_r, w_o, u, vb, beta = map(_f64, (w_q, w_k, w_v, w_r, w_o, u, vb, beta))
    if scale is None:
        scale = 1.0 / np.sqrt(d_head)
    out = np.empty((B, ql, D), np.float64)
    terms = np.empty((4, B, n_head, ql, kl), np.float64) if want_terms else None
    probs = np.empty((B, n_head, ql, kl), np.float64) if want_probs else None
    qpos, kpos = _i64arr(qpos), _i64arr(kpos)
    st = _load().orc_rel_attn_fwd(B, D, n_head, d_head, ql, ml, clamp_len, bias_clamp, bias_kind, scale, base,
                                  _ptr(qpos), _ptr(kpos), _ptr(h), _ptr(mem),
                                  _ptr(w_q), _ptr(w_k), _ptr(w_v), _ptr(w_r), _ptr(w_o),
                                  _ptr(u), _ptr(vb), _ptr(beta), _ptr(out), _ptr(terms), _ptr(probs))
    _check(st, "orc_rel_attn_fwd")
    res = [out]
    if want_terms:
        res.append(terms)
    if want_probs:
        res.append(probs)
    return res[0] if len(res) == 1 else tuple(res)


def fifo_update(mem, h, mlen_max: int):
    """New memory = last min(len(mem)+len(h), mlen_max) rows of [mem ; h]."""
    h = _f64(h)
    B, ql, D = h.shape
    mem = _f64(mem) if mem is not None else np.zeros((B, 0, D))
    ml = mem.shape[1]
    keep = min(ml + ql, mlen_max)
    out = np.empty((B, keep, D), np.float64)
    n = _i64(0)
    st = _load().orc_fifo_update(B, D, mlen_max, ml, _ptr(mem) if ml else None, ql, _ptr(h), _ptr(out),
                                 ctypes.byref(n))
    _check(st, "orc_fifo_update")
    assert n.value == keep
    return out


def segment_run(stream, n_seg: int, qlen: int, mlen_max: int, weights: dict, *, n_head: int, d_head: int,
                clamp_len: int = -1, bias_clamp: int = -1, bias_kind: int = 0):
    """Segment-recurrent run [felixzhao.cn 118 §2.3.1]: segment t attends over
    [mem_t ; h_t]; afterwards mem_{t+1} = FIFO(mem_t, h_t). The run starts with
    an empty memory. Returns the per-segment outputs and memories."""
    stream = _f64(stream)
    B, _, D = stream.shape
    mem = np.zeros((B, 0, D))
    outs, mems = [], []
    for t in range(n_seg):
        h = stream[:, t * qlen:(t + 1) * qlen]
        out = rel_attn_fwd(h, mem, weights["w_q"], weights["w_k"], weights["w_v"], weights["w_r"],
                           weights["w_o"], weights["u"], weights["v"], n_head=n_head, d_head=d_head,
                           clamp_len=clamp_len, beta=weights.get("beta"), bias_clamp=bias_clamp,
                           bias_kind=bias_kind)
        outs.append(out)
        mem = fifo_update(mem, h, mlen_max)
        mems.append(mem)
    return outs, mems


# --- the decoder layer and stack around the attention -------------------------------------------

def layer_norm(x, gamma=None, beta=None, eps: float = 1e-5):
    """Row-wise layer normalisation over the last axis (population variance)."""
    x = _f64(x)
    D = x.shape[-1]
    x2 = x.reshape(-1, D)
    y = np.empty_like(x2)
    g, bt = _f64(gamma), _f64(beta)
    _check(_load().orc_layer_norm(x2.shape[0], D, _ptr(x2), _ptr(g), _ptr(bt), eps, _ptr(y)), "orc_layer_norm")
    return y.reshape(x.shape)


def ffn(x, w1, b1, w2, b2):
    """Position-wise feed-forward network: two linear layers (with biases)
    around a ReLU [felixzhao.cn 118 §1: two linear layers and a nonlinear
    activation; ReLU is the reading taken]."""
    y1 = linear(x, w1) + _f64(b1)
    y1 = np.maximum(y1, 0.0)
    return linear(y1, w2) + _f64(b2)


def decoder_layer_fwd(h, mem, w: dict, *, n_head: int, d_head: int, clamp_len: int = -1, bias_clamp: int = -1,
                      bias_kind: int = 0, eps: float = 1e-5):
    """One pre-LN decoder layer [felixzhao.cn 118 §2.3.1: N modules of masked
    self-attention and FFN, each feeding the next; 2kiu.com §3.4: the
    attention input is layer-normalised]:
        a   = RelAttn(queries LN1(h), keys and values over [LN1(mem) ; LN1(h)])
        h1  = h + a
        out = h1 + FFN(LN2(h1)).
    The memory holds the previous segment's layer *input* (un-normalised)."""
    h = _f64(h)
    xh = layer_norm(h, w["ln1_g"], w["ln1_b"], eps)
    xm = layer_norm(mem, w["ln1_g"], w["ln1_b"], eps) if mem is not None and mem.shape[1] > 0 else None
    a = rel_attn_fwd(xh, xm, w["w_q"], w["w_k"], w["w_v"], w["w_r"], w["w_o"], w["u"], w["v"], n_head=n_head,
                     d_head=d_head, clamp_len=clamp_len, beta=w.get("beta"), bias_clamp=bias_clamp,
                     bias_kind=bias_kind)
    h1 = h + a
    return h1 + ffn(layer_norm(h1, w["ln2_g"], w["ln2_b"], eps), w["w1"], w["b1"], w["w2"], w["b2"])


def decoder_stack_run(stream, n_seg: int, qlen: int, mlen_max: int, layers: list, *, n_head: int, d_head: int,
                      clamp_len: int = -1, bias_clamp: int = -1, bias_kind: int = 0, eps: float = 1e-5):
    """Segment-recurrent run of an N-layer stack [felixzhao.cn 118 §2.3.1]:
    layer n of segment t attends over [mem_t^n ; h_t^(n-1)] and afterwards
    mem_(t+1)^n = FIFO(mem_t^n, h_t^(n-1)), its own input; h_t^0 is the
    segment of the input stream. Returns the per-segment outputs of the last
    layer and the per-segment lists of per-layer memories."""
    stream = _f64(stream)
    B, _, D = stream.shape
    mems = [np.zeros((B, 0, D)) for _ in layers]
    outs, mem_hist = [], []
    for t in range(n_seg):
        x = stream[:, t * qlen:(t + 1) * qlen]
        for n, w in enumerate(layers):
            y = decoder_layer_fwd(x, mems[n], w, n_head=n_head, d_head=d_head, clamp_len=clamp_len,
                                  bias_clamp=bias_clamp, bias_kind=bias_kind, eps=eps)
            mems[n] = fifo_update(mems[n], x, mlen_max)
            x = y
        outs.append(x)
        mem_hist.append([m.copy() for m in mems])
    return outs, mem_hist
