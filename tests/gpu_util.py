"""Helpers for the GPU parity tests: move seeded inputs to the device, run the
library through its C ABI, compare with the oracle."""
from __future__ import annotations

import numpy as np

import transformer_xl_relative_amd as xl
import xl_inputs
from tests.guards import BF16_ATOL, BF16_RTOL, F32_RTOL, tolerance  # noqa: F401  (one tolerance for all tests)


def torch():
    import torch as _t
    return _t


def dev(t: xl_inputs.Tensor):
    """Device copy holding exactly the stored bits of an input."""
    T = torch()
    if t.dtype == "bf16":
        return T.from_numpy(t.bits.view(np.int16).copy()).view(T.bfloat16).cuda()
    return T.from_numpy(t.f32.copy()).cuda()


def host64(x) -> np.ndarray:
    T = torch()
    return x.detach().float().cpu().numpy().astype(np.float64) if x.dtype != T.float64 else x.cpu().numpy()


def bits_u16(x) -> np.ndarray:
    """uint16 bits of a bf16 device tensor."""
    T = torch()
    return x.detach().cpu().view(T.int16).numpy().view(np.uint16)


def compare(name, got, ref, *, dtype: str, report=None):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values in the GPU result"
    rtol, atol = tolerance(ref, dtype)
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref)
    rel = err / np.maximum(np.abs(ref), atol)
    msg = (f"{name}: max abs err {err.max():.3e}, max rel err {rel.max():.3e}, "
           f"failing {bad.mean() * 100:.4f}% (rtol {rtol}, atol {atol:.2e})")
    if report is not None:
        report.append(msg)
    assert not bad.any(), msg
    return err.max()


class Layer:
    """One layer call's device buffers (inputs, weights, workspace, output)."""

    def __init__(self, w: xl_inputs.Workload, t: dict, *, batch, qlen, mlen, out_f32=True,
                 h_key="h", h_override=None):
        T = torch()
        self.w = w
        self.dt = xl.XL_BF16 if w.dtype == "bf16" else xl.XL_F32
        self.desc = xl.make_desc(batch=batch, d_model=w.d_model, n_head=w.n_head, d_head=w.d_head, qlen=qlen,
                                 mlen=mlen, clamp_len=w.clamp_len, bias_clamp=w.bias_clamp,
                                 bias_kind=w.bias_kind, dtype=self.dt,
                                 out_dtype=xl.XL_F32 if out_f32 else self.dt)
        self.weights = xl.Weights(*(dev(t[k]) for k in ("w_q", "w_k", "w_v", "w_r", "w_o", "u", "v")),
                                  bias_table=dev(t["beta"]) if "beta" in t else None)
        self.ws = T.empty(xl.xl_rel_attn_workspace_size(self.desc), dtype=T.uint8, device="cuda")
        self.layout = xl.xl_rel_attn_workspace_layout(self.desc)
        self.out = T.empty((batch, qlen, w.d_model), dtype=T.float32 if out_f32 else
                           (T.bfloat16 if w.dtype == "bf16" else T.float32), device="cuda")

    def ws_view(self, off, shape):
        T = torch()
        dt = T.bfloat16 if self.w.dtype == "bf16" else T.float32
        n = int(np.prod(shape))
        es = 2 if self.w.dtype == "bf16" else 4
        return self.ws[off:off + n * es].view(dt).view(*shape)


def oracle_layer(t: dict, w: xl_inputs.Workload, h, mem, bsel=None):
    import oracle
    if bsel is not None:
        h = h[bsel]
        mem = mem[bsel]
    return oracle.rel_attn_fwd(h, mem, t["w_q"].f64, t["w_k"].f64, t["w_v"].f64, t["w_r"].f64, t["w_o"].f64,
                               t["u"].f64, t["v"].f64, n_head=w.n_head, d_head=w.d_head, clamp_len=w.clamp_len,
                               beta=t["beta"].f64 if "beta" in t else None, bias_clamp=w.bias_clamp,
                               bias_kind=w.bias_kind)


DEC_KEYS = ("ln1_g", "ln1_b", "ln2_g", "ln2_b", "w1", "b1", "w2", "b2")


def dec_weights(lw: dict):
    """Device weights of one decoder layer from decoder_inputs' per-layer dict."""
    attn = xl.Weights(*(dev(lw[k]) for k in ("w_q", "w_k", "w_v", "w_r", "w_o", "u", "v")),
                      bias_table=dev(lw["beta"]) if "beta" in lw else None)
    return xl.DecoderWeights(attn, *(dev(lw[k]) for k in DEC_KEYS))


def oracle_dec_weights(lw: dict) -> dict:
    return {k: v.f64 for k, v in lw.items()}
