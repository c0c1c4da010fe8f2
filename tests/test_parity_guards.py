"""Negative controls of the composed-path parity tests (CPU, oracle only).

Under the "sensitive" value recipe, at the full qlen/mlen of the four bf16
workloads (batch 1; the segmented workload as its four-segment run), the
oracle with any one piece of the score altered -- u or v zeroed, u and v
swapped, W_r zeroed, the clamp dropped, the bias table dropped -- must fail
the bf16 comparison on a large share of the output. A GPU path with the same
wiring mistake would therefore fail the GPU parity tests that use this
recipe (tests/test_gpu_sensitive.py), which repeat the check against the GPU
output itself. Passages: qidao123.com thread-401555 §3 (u, v), felixzhao.cn
article 118 §2.3.2 (W_r), 2kiu.com/news/5253360 §2.4 (clamp), jsqmd.com
1364567 §3.1-§3.4 (bias table).
"""
import pytest

import xl_inputs
from tests import guards

W = xl_inputs.WORKLOADS
MIN_FAIL = 0.10     # each control must fail at least this share of the elements


@pytest.mark.parametrize("name", ["base_bf16", "large_bf16", "longmem_bf16"])
def test_layer_guards_fail(name):
    w = W[name]
    t = xl_inputs.layer_inputs(w, batch=1, recipe="sensitive")
    ref = guards.oracle_layer(w, t)
    abl = guards.ablations(w, t)
    if w.clamp_len >= 0:
        assert "no clamp" in abl
    for label, ov in abl.items():
        frac = guards.fail_fraction(guards.oracle_layer(w, t, ov), ref, "bf16")
        assert frac >= MIN_FAIL, f"{name}: control '{label}' fails only {frac:.2%} of the output"


def test_segment_run_guards_fail():
    w = W["segments_bf16"]
    t = xl_inputs.layer_inputs(w, batch=1, recipe="sensitive")
    refs = guards.oracle_segments(w, t, w.segments, w.qlen, w.mlen)
    abl = guards.ablations(w, t)
    assert "no bias table" in abl
    for label, ov in abl.items():
        outs = guards.oracle_segments(w, t, w.segments, w.qlen, w.mlen, ov)
        for s in range(w.segments):
            frac = guards.fail_fraction(outs[s], refs[s], "bf16")
            assert frac >= MIN_FAIL, f"segment {s}: control '{label}' fails only {frac:.2%}"


def test_config_recipe_is_blind_to_uv_swap():
    # why the second recipe exists: at the configs' own N(0, 0.02) scales the
    # swapped biases hide inside the bf16 tolerance
    w = W["base_bf16"]
    t = xl_inputs.layer_inputs(w, batch=1)
    ref = guards.oracle_layer(w, t)
    frac = guards.fail_fraction(guards.oracle_layer(w, t, guards.ablations(w, t)["u<->v"]), ref, "bf16")
    assert frac < 0.01


def test_decoder_layer_guards_fail():
    # the attention sublayer stays visible through the decoder's residuals
    import dataclasses

    import oracle
    w = dataclasses.replace(W["base_bf16"], bias_clamp=16, seed=205)
    t = xl_inputs.decoder_inputs(w, d_inner=512, n_layer=1, batch=1, qlen=128, mlen=128, recipe="sensitive")
    lw = t["layers"][0]

    def run(ov=None):
        wts = {k: v.f64 for k, v in lw.items()}
        wts.update(ov or {})
        if wts.get("beta") is None:
            wts.pop("beta", None)
        return oracle.decoder_layer_fwd(t["h"].f64, t["mem"].f64, wts, n_head=w.n_head, d_head=w.d_head,
                                        clamp_len=w.clamp_len, bias_clamp=w.bias_clamp if "beta" in wts else -1,
                                        bias_kind=w.bias_kind)

    ref = run()
    for label, ov in guards.ablations(w, lw).items():
        frac = guards.fail_fraction(run(ov), ref, "bf16")
        assert frac >= MIN_FAIL, f"decoder: control '{label}' fails only {frac:.2%}"
