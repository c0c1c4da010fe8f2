"""Sensitivity guards for the composed-path parity tests.

A parity test can only see a term of the score if leaving that term out
moves the output by more than the tolerance. These helpers rerun the fp64
oracle with one piece of the method altered (a negative control) and report
what fraction of the output elements the altered result would fail under the
same element-wise comparison as the parity tests. Pieces, by the passage
that defines each:
  * u = 0, v = 0, u and v swapped: the global content and position biases of
    the four-term score (qidao123.com thread-401555 §3);
  * W_r = 0: no position term at all (felixzhao.cn article 118 §2.3.2);
  * clamp dropped: distances past C keep their own rows instead of R_C
    (2kiu.com/news/5253360 §2.4);
  * bias table dropped: the per-head scalar bias of jsqmd.com 1364567
    §3.1-§3.4.
CPU only: nothing here touches the GPU library.
"""
from __future__ import annotations

import numpy as np

import oracle

BF16_RTOL, BF16_ATOL = 2e-2, 1e-2   # bf16 inputs, fp32 accumulation
F32_RTOL = 1e-5                     # fp32 workload; atol = 1e-5 * max|ref|


def tolerance(ref, dtype: str):
    ref = np.asarray(ref, np.float64)
    if dtype == "bf16":
        return BF16_RTOL, BF16_ATOL
    return F32_RTOL, F32_RTOL * max(float(np.max(np.abs(ref))), 1e-30)


def fail_fraction(got, ref, dtype: str) -> float:
    """Fraction of elements outside |got - ref| <= atol + rtol |ref|."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rtol, atol = tolerance(ref, dtype)
    return float(np.mean(np.abs(got - ref) > atol + rtol * np.abs(ref)))


def ablations(w, t) -> dict:
    """Altered parameter sets of a layer: name -> overrides of the weight
    dict (f64 arrays, None for a dropped bias table) and of clamp_len."""
    u, v = t["u"].f64, t["v"].f64
    out = {
        "u=0": {"u": np.zeros_like(u)},
        "v=0": {"v": np.zeros_like(v)},
        "u<->v": {"u": v, "v": u},
        "W_r=0": {"w_r": np.zeros_like(t["w_r"].f64)},
    }
    if w.clamp_len >= 0:
        out["no clamp"] = {"clamp_len": -1}
    if w.bias_clamp >= 0:
        out["no bias table"] = {"beta": None}
    return out


def weights64(t, overrides=None) -> dict:
    wts = {k: t[k].f64 for k in ("w_q", "w_k", "w_v", "w_r", "w_o", "u", "v")}
    wts["beta"] = t["beta"].f64 if "beta" in t else None
    for k, val in (overrides or {}).items():
        if k != "clamp_len":
            wts[k] = val
    return wts


def oracle_layer(w, t, overrides=None, bsel=None):
    """The oracle layer forward of t's h and mem, with optional overrides."""
    wts = weights64(t, overrides)
    clamp = (overrides or {}).get("clamp_len", w.clamp_len)
    h, mem = t["h"].f64, t["mem"].f64
    if bsel is not None:
        h, mem = h[bsel], mem[bsel]
    return oracle.rel_attn_fwd(h, mem, wts["w_q"], wts["w_k"], wts["w_v"], wts["w_r"], wts["w_o"], wts["u"],
                               wts["v"], n_head=w.n_head, d_head=w.d_head, clamp_len=clamp, beta=wts["beta"],
                               bias_clamp=w.bias_clamp if wts["beta"] is not None else -1,
                               bias_kind=w.bias_kind)


def oracle_segments(w, t, n_seg, qlen, mlen_max, overrides=None, bsel=None):
    """Per-segment outputs of the oracle's segment-recurrent run."""
    wts = weights64(t, overrides)
    clamp = (overrides or {}).get("clamp_len", w.clamp_len)
    stream = t["h"].f64 if bsel is None else t["h"].f64[bsel]
    outs, _ = oracle.segment_run(stream, n_seg, qlen, mlen_max, wts, n_head=w.n_head, d_head=w.d_head,
                                 clamp_len=clamp, bias_clamp=w.bias_clamp if wts["beta"] is not None else -1,
                                 bias_kind=w.bias_kind)
    return outs


def oracle_core_of_layer(w, t, bsel=None, n_rel=None):
    """The attention core's output (before W_o) of the layer forward, from
    projections the oracle computes itself."""
    h, mem = t["h"].f64, t["mem"].f64
    if bsel is not None:
        h, mem = h[bsel], mem[bsel]
    B, ql, D = h.shape
    H, dh = w.n_head, w.d_head
    x = np.concatenate([mem, h], axis=1)
    kl = x.shape[1]
    q = oracle.linear(h, t["w_q"].f64).reshape(B, ql, H, dh).transpose(0, 2, 1, 3)
    k = oracle.linear(x, t["w_k"].f64).reshape(B, kl, H, dh).transpose(0, 2, 1, 3)
    v = oracle.linear(x, t["w_v"].f64).reshape(B, kl, H, dh).transpose(0, 2, 1, 3)
    rows = kl if n_rel is None else n_rel
    R = oracle.relpos_embed(0, rows, D, w.clamp_len)
    r = oracle.linear(R, t["w_r"].f64).reshape(rows, H, dh).transpose(1, 0, 2)
    return oracle.rel_attn_core(q, k, v, r, t["u"].f64, t["v"].f64, scale=1.0 / np.sqrt(dh),
                                clamp_len=w.clamp_len, beta=t["beta"].f64 if "beta" in t else None,
                                bias_clamp=w.bias_clamp, bias_kind=w.bias_kind)


def distinct_rows(klen: int, clamp_len: int) -> int:
    """Distinct table rows a layer needs: the distances 0..klen-1 of its
    visible pairs, of which those past C share row C (2kiu.com §2.4)."""
    return klen if clamp_len < 0 else min(klen, clamp_len + 1)
