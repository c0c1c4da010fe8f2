"""A second, independent fp64 formulation of the layer, used only to pin the
oracle on tiny inputs. It follows the gather-then-einsum style of the module on
2kiu.com/news/5253360 §3.1 (materialise the relative embedding of every
(query, key) pair, project it, then form the four score terms with einsum),
which shares nothing with the oracle's per-pair loops.
"""
from __future__ import annotations

import numpy as np


def sinusoid_table(deltas: np.ndarray, d_model: int, base: float = 10000.0) -> np.ndarray:
    """[len(deltas), d_model], interleaved sin/cos (qidao123.com thread-401555 §2)."""
    t = np.arange(d_model // 2, dtype=np.float64)
    inv = base ** (-(2.0 * t) / d_model)
    ang = np.asarray(deltas, np.float64)[:, None] * inv[None, :]
    out = np.empty((len(deltas), d_model))
    out[:, 0::2] = np.sin(ang)
    out[:, 1::2] = np.cos(ang)
    return out


def layer(h, mem, w_q, w_k, w_v, w_r, w_o, u, vb, *, n_head, d_head, clamp_len=-1, beta=None,
          bias_clamp=-1, bias_kind=0, scale=None, p1_scaling=False, return_terms=False):
    """Forward of one layer on [mem ; h]. With p1_scaling the 1/sqrt(d) factor
    multiplies only terms (a) and (b), as in the 2kiu.com module; otherwise it
    multiplies the whole sum. bias_kind 1 indexes beta by the T5 bucket, found
    here by a sorted search over the log-scale boundaries 1, 2, 4, ..., 1024."""
    h = np.asarray(h, np.float64)
    B, q, D = h.shape
    mem = np.zeros((B, 0, D)) if mem is None else np.asarray(mem, np.float64)
    m = mem.shape[1]
    kl = m + q
    H, dh = n_head, d_head
    s = 1.0 / np.sqrt(dh) if scale is None else scale
    x = np.concatenate([mem, h], axis=1)
    Q = (h @ np.asarray(w_q, np.float64).T).reshape(B, q, H, dh).transpose(0, 2, 1, 3)
    K = (x @ np.asarray(w_k, np.float64).T).reshape(B, kl, H, dh).transpose(0, 2, 1, 3)
    V = (x @ np.asarray(w_v, np.float64).T).reshape(B, kl, H, dh).transpose(0, 2, 1, 3)
    qi = np.arange(q)[:, None] + m
    kj = np.arange(kl)[None, :]
    delta = qi - kj                                     # [q, kl]
    dc = np.clip(delta, -clamp_len, clamp_len) if clamp_len >= 0 else delta
    R = sinusoid_table(dc.reshape(-1), D).reshape(q, kl, D)   # gathered [q, kl, D]
    rel = (R @ np.asarray(w_r, np.float64).T).reshape(q, kl, H, dh).transpose(2, 0, 1, 3)  # [H,q,kl,dh]
    u = np.asarray(u, np.float64)
    vb = np.asarray(vb, np.float64)
    ta = np.einsum("bhid,bhjd->bhij", Q, K)
    tb = np.einsum("bhid,hijd->bhij", Q, rel)
    tc = np.broadcast_to(np.einsum("hd,bhjd->bhj", u, K)[:, :, None, :], ta.shape)
    td = np.broadcast_to(np.einsum("hd,hijd->hij", vb, rel)[None], ta.shape)
    if p1_scaling:
        score = (ta + tb) * s + tc + td
    else:
        score = (ta + tb + tc + td) * s
    if beta is not None:
        if bias_kind == 1:
            bounds = 2 ** np.arange(11)
            idx = np.searchsorted(bounds, np.maximum(delta, 0), side="left")
        else:
            idx = np.clip(delta, -bias_clamp, bias_clamp) + bias_clamp
        score = score + np.asarray(beta, np.float64)[idx].transpose(2, 0, 1)[None]
    visible = kj <= qi
    score = np.where(visible[None, None], score, -np.inf)
    score = score - score.max(axis=-1, keepdims=True)
    p = np.exp(score)
    p = p / p.sum(axis=-1, keepdims=True)
    o = np.einsum("bhij,bhjd->bhid", p, V).transpose(0, 2, 1, 3).reshape(B, q, H * dh)
    out = o @ np.asarray(w_o, np.float64).T
    if return_terms:
        mask = visible[None, None]
        return out, [np.where(mask, t, 0.0) for t in (ta, tb, tc, td)], p
    return out


def layer_norm(x, gamma, beta, eps):
    """Row-wise layer normalisation with numpy's mean and variance."""
    x = np.asarray(x, np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    var = x.var(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * np.asarray(gamma, np.float64) + np.asarray(beta, np.float64)


def decoder_layer(h, mem, w, *, n_head, d_head, clamp_len=-1, eps=1e-5):
    """Pre-LN decoder layer built from the gather/einsum attention above."""
    h = np.asarray(h, np.float64)
    xm = layer_norm(mem, w["ln1_g"], w["ln1_b"], eps) if mem is not None else None
    xh = layer_norm(h, w["ln1_g"], w["ln1_b"], eps)
    a = layer(xh, xm, w["w_q"], w["w_k"], w["w_v"], w["w_r"], w["w_o"], w["u"], w["v"], n_head=n_head,
              d_head=d_head, clamp_len=clamp_len)
    h1 = h + a
    x2 = layer_norm(h1, w["ln2_g"], w["ln2_b"], eps)
    y = np.maximum(np.einsum("mk,nk->mn", x2.reshape(-1, x2.shape[-1]), np.asarray(w["w1"], np.float64))
                   + np.asarray(w["b1"], np.float64), 0.0)
    y = y @ np.asarray(w["w2"], np.float64).T + np.asarray(w["b2"], np.float64)
    return h1 + y.reshape(h1.shape)
