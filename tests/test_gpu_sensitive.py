"""Composed-path parity under the "sensitive" value recipe, with negative
controls.

The workloads' own parameter scales (N(0, 0.02)) leave the layer output
almost blind to u, v, W_r, the clamp and the bias table (see
tests/test_parity_guards.py). Here the same layer, segment-run and decoder
paths run on inputs drawn with larger parameter scales at the workloads' full
qlen and mlen (reduced batch), and each GPU result must
  * match the fp64 oracle within the bf16 tolerance, and
  * FAIL the same comparison against the oracle with one piece altered
    (u = 0, v = 0, u and v swapped, W_r = 0, clamp dropped, bias table
    dropped), so that a wiring mistake in any of them cannot pass.
The attention output before W_o (the workspace's attn region) is compared
with the oracle's core on projections the oracle computes itself, and the
table rows with a row count derived here from the clamp (2kiu.com §2.4).
"""
import dataclasses

import numpy as np
import pytest

import oracle
import xl_inputs
from tests import gpu_util as gu
from tests import guards

pytestmark = pytest.mark.gpu
W = xl_inputs.WORKLOADS
MIN_FAIL = 0.05     # share of the output each control must fail against the GPU result


@pytest.fixture(scope="module")
def T():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import transformer_xl_relative_amd as xl
    xl.lib()
    return torch


def _controls(label, got, w, t, run_oracle):
    for name, ov in guards.ablations(w, t).items():
        frac = guards.fail_fraction(got, run_oracle(ov), w.dtype)
        assert frac >= MIN_FAIL, f"{label}: the GPU output also fits the control '{name}' ({frac:.2%} fail)"


LAYERS = [
    # workload, batch, overrides of the workload
    ("base_bf16", 2, {}),
    ("large_bf16", 1, {}),
    ("longmem_bf16", 2, {}),
    ("longmem_bf16", 1, {"clamp_len": 300, "mlen": 700}),
    ("base_bf16", 1, {"mlen": 1100, "bias_clamp": 0, "bias_kind": 1}),     # T5 buckets past 1024
    ("base_bf16", 1, {"bias_clamp": 128}),                                   # the +-128 table at C1's shape
]


@pytest.mark.parametrize("name,batch,ov", LAYERS, ids=[f"{n}-B{b}-{'-'.join(f'{k}{v}' for k, v in o.items())}"
                                                       for n, b, o in LAYERS])
def test_layer_sensitive(T, name, batch, ov):
    import transformer_xl_relative_amd as xl
    w = dataclasses.replace(W[name], seed=W[name].seed + 100, **ov)
    t = xl_inputs.layer_inputs(w, batch=batch, recipe="sensitive")
    L = gu.Layer(w, t, batch=batch, qlen=w.qlen, mlen=w.mlen)
    xl.xl_rel_attn_fwd(L.desc, L.weights, gu.dev(t["h"]), gu.dev(t["mem"]), L.out, L.ws)
    T.cuda.synchronize()
    got = gu.host64(L.out)
    gu.compare(f"{name} sensitive", got, guards.oracle_layer(w, t), dtype="bf16")
    _controls(name, got, w, t, lambda o: guards.oracle_layer(w, t, o))

    # the attention output before W_o
    lay = L.layout
    H, dh, D, klen = w.n_head, w.d_head, w.d_model, w.qlen + w.mlen
    attn = gu.host64(L.ws_view(lay.attn, (batch, w.qlen, H * dh)))
    gu.compare(f"{name} attn before W_o", attn, guards.oracle_core_of_layer(w, t), dtype="bf16")

    # table rows: the count follows from the clamp, every row against the oracle
    n_rel = guards.distinct_rows(klen, w.clamp_len)
    assert lay.n_rel == n_rel, (lay.n_rel, n_rel)
    R = oracle.relpos_embed(0, n_rel, D, w.clamp_len)
    gu.compare("rel", gu.host64(L.ws_view(lay.rel, (n_rel, D))), R, dtype="bf16")
    r = oracle.linear(R, t["w_r"].f64).reshape(n_rel, H, dh).transpose(1, 0, 2)
    gu.compare("r", gu.host64(L.ws_view(lay.r, (H, n_rel, dh))), r, dtype="bf16")
    if w.clamp_len >= 0 and klen > w.clamp_len + 1:
        # the rows the clamp folds: the distance klen-1 uses row C
        assert np.array_equal(oracle.relpos_embed(klen - 1, 1, D, w.clamp_len), R[-1:])


def _segment_runs(T, w, t, batch, *, kv_ring):
    """Per-segment outputs of the state-FIFO step (and of the key-ring step)."""
    import transformer_xl_relative_amd as xl
    H, dh, D, q, m = w.n_head, w.d_head, w.d_model, w.qlen, w.mlen
    L = gu.Layer(w, t, batch=batch, qlen=q, mlen=m)
    ring = T.zeros((batch, m, D), dtype=T.bfloat16, device="cuda")
    fifo = xl.xl_mem_fifo(ring.data_ptr(), m, 0, 0)
    cap = m + q + 64
    kr = T.full((batch, H, cap, dh), float("nan"), dtype=T.bfloat16, device="cuda")
    vr = T.full((batch, H, dh, cap), float("nan"), dtype=T.bfloat16, device="cuda")
    kv = xl.xl_kv_fifo(kr.data_ptr(), vr.data_ptr(), cap, m, 0, 24)
    kws = T.empty(max(xl.xl_segment_step_kv_workspace_size(L.desc), 1), dtype=T.uint8, device="cuda")
    hs = gu.dev(t["h"])
    outs, ring_outs, mems = [], [], []
    for s in range(w.segments):
        h = hs[:, s * q:(s + 1) * q].contiguous()
        desc = xl.make_desc(batch=batch, d_model=D, n_head=H, d_head=dh, qlen=q, mlen=0, clamp_len=w.clamp_len,
                            bias_clamp=w.bias_clamp, bias_kind=w.bias_kind, dtype=xl.XL_BF16,
                            out_dtype=xl.XL_F32)
        out = T.empty((batch, q, D), dtype=T.float32, device="cuda")
        xl.xl_segment_step(desc, L.weights, h, fifo, out, L.ws)
        if kv_ring:
            out2 = T.empty((batch, q, D), dtype=T.float32, device="cuda")
            xl.xl_segment_step_kv(desc, L.weights, h, kv, out2, kws)
            ring_outs.append(out2)
        T.cuda.synchronize()
        outs.append(gu.host64(out))
        mems.append(gu.bits_u16(ring[:, [(fifo.head + i) % m for i in range(fifo.len)]]))
    return outs, [gu.host64(o) for o in ring_outs], mems


def test_segment_run_sensitive(T):
    # the segmented workload's four segments (qlen = mlen = 512, +-128 bias
    # table), batch 1: state FIFO and key ring against the oracle's run, with
    # every control failing on every segment
    w = dataclasses.replace(W["segments_bf16"], seed=104)
    t = xl_inputs.layer_inputs(w, batch=1, recipe="sensitive")
    outs, ring_outs, mems = _segment_runs(T, w, t, 1, kv_ring=True)
    refs = guards.oracle_segments(w, t, w.segments, w.qlen, w.mlen)
    for s in range(w.segments):
        gu.compare(f"segment {s}", outs[s], refs[s], dtype="bf16")
        assert np.array_equal(ring_outs[s], outs[s]), f"segment {s}: key ring and state FIFO differ"
        keep = min((s + 1) * w.qlen, w.mlen)
        want = xl_inputs.bf16_bits(t["h"].f32[:, (s + 1) * w.qlen - keep:(s + 1) * w.qlen])
        assert np.array_equal(mems[s], want), f"memory after segment {s}"
    for label, ov in guards.ablations(w, t).items():
        alt = guards.oracle_segments(w, t, w.segments, w.qlen, w.mlen, ov)
        for s in range(w.segments):
            frac = guards.fail_fraction(outs[s], alt[s], "bf16")
            assert frac >= MIN_FAIL, f"segment {s} also fits the control '{label}' ({frac:.2%} fail)"


def test_decoder_layer_sensitive(T):
    # the pre-LN decoder layer with the attention weights at the sensitive
    # scales: the attention sublayer stays visible through the residuals
    import transformer_xl_relative_amd as xl
    w = dataclasses.replace(W["base_bf16"], bias_clamp=16, seed=205)
    q, m, d_inner = 128, 128, 512
    t = xl_inputs.decoder_inputs(w, d_inner=d_inner, n_layer=1, batch=1, qlen=q, mlen=m, recipe="sensitive")
    lw = t["layers"][0]
    desc = xl.make_desc(batch=1, d_model=w.d_model, n_head=w.n_head, d_head=w.d_head, qlen=q, mlen=m,
                        clamp_len=w.clamp_len, bias_clamp=w.bias_clamp, bias_kind=w.bias_kind, dtype=xl.XL_BF16,
                        out_dtype=xl.XL_F32)
    ws = T.empty(xl.xl_decoder_layer_workspace_size(desc, d_inner), dtype=T.uint8, device="cuda")
    out = T.empty((1, q, w.d_model), dtype=T.float32, device="cuda")
    xl.xl_decoder_layer_fwd(desc, d_inner, 0.0, gu.dec_weights(lw), gu.dev(t["h"]), gu.dev(t["mem"]), out, ws)
    T.cuda.synchronize()
    got = gu.host64(out)

    def run(ov=None):
        wts = gu.oracle_dec_weights(lw)
        for k, val in (ov or {}).items():
            wts[k] = val
        beta = wts.get("beta")
        if beta is None:
            wts.pop("beta", None)
        return oracle.decoder_layer_fwd(t["h"].f64, t["mem"].f64, wts, n_head=w.n_head, d_head=w.d_head,
                                        clamp_len=w.clamp_len, bias_clamp=w.bias_clamp if beta is not None else -1,
                                        bias_kind=w.bias_kind)

    gu.compare("decoder layer sensitive", got, run(), dtype="bf16")
    _controls("decoder layer", got, w, lw, run)
