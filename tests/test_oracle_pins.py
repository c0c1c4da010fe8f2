"""Pins of the fp64 CPU oracle against facts that do not come from the oracle
itself: the pages' worked example, trigonometric identities, special cases that
reduce to a library routine, invariances of the method, and an independent
gather/einsum formulation on tiny inputs. Runs on the CPU only.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import xl_inputs
from tests import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tiny(seed=0, B=2, D=16, H=2, dh=8, q=6, m=5, bias_clamp=-1, clamp_len=-1, bias_kind=0):
    rng = np.random.default_rng(seed)
    HD = H * dh
    w = {
        "h": rng.standard_normal((B, q, D)),
        "mem": rng.standard_normal((B, m, D)),
        "w_q": rng.standard_normal((HD, D)) * 0.3,
        "w_k": rng.standard_normal((HD, D)) * 0.3,
        "w_v": rng.standard_normal((HD, D)) * 0.3,
        "w_r": rng.standard_normal((HD, D)) * 0.3,
        "w_o": rng.standard_normal((D, HD)) * 0.3,
        "u": rng.standard_normal((H, dh)) * 0.3,
        "v": rng.standard_normal((H, dh)) * 0.3,
    }
    if bias_clamp >= 0:
        rows = 12 if bias_kind == 1 else 2 * bias_clamp + 1
        w["beta"] = rng.standard_normal((rows, H)) * 0.5
    w.update(n_head=H, d_head=dh, clamp_len=clamp_len, bias_clamp=bias_clamp, bias_kind=bias_kind)
    return w


def _fwd(w, **over):
    a = dict(w)
    a.update(over)
    return oracle.rel_attn_fwd(a["h"], a["mem"], a["w_q"], a["w_k"], a["w_v"], a["w_r"], a["w_o"], a["u"], a["v"],
                               n_head=a["n_head"], d_head=a["d_head"], clamp_len=a["clamp_len"],
                               beta=a.get("beta"), bias_clamp=a["bias_clamp"], bias_kind=a.get("bias_kind", 0),
                               **{k: a[k] for k in ("qpos", "kpos", "want_terms", "want_probs", "scale") if k in a})


def _brute(w, **over):
    a = dict(w)
    a.update(over)
    return brute.layer(a["h"], a["mem"], a["w_q"], a["w_k"], a["w_v"], a["w_r"], a["w_o"], a["u"], a["v"],
                       n_head=a["n_head"], d_head=a["d_head"], clamp_len=a["clamp_len"], beta=a.get("beta"),
                       bias_clamp=a["bias_clamp"], bias_kind=a.get("bias_kind", 0),
                       **{k: a[k] for k in ("p1_scaling", "return_terms", "scale") if k in a})


def _close(a, b, tol=1e-12):
    a = np.asarray(a)
    b = np.asarray(b)
    scale = max(1.0, float(np.max(np.abs(b)))) if b.size else 1.0
    assert a.shape == b.shape
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * scale, f"max abs err {err:.3e} > {tol * scale:.3e}"


# --- relative embedding ------------------------------------------------------

def test_worked_example_r_minus2():
    g = json.load(open(os.path.join(GOLDEN, "worked_example_R_minus2_d4.json")))
    R = oracle.relpos_embed(g["delta"], 1, g["d_model"], -1, g["base"])[0]
    assert np.all(np.abs(R - np.array(g["printed"])) < 1e-3), R
    # and the sign pattern the page prints (sin odd, cos of a small angle ~ 1)
    assert R[0] < 0 and R[1] < 0 and R[2] < 0 and R[3] > 0.999


def test_sinusoid_identities():
    D = 64
    R = oracle.relpos_embed(-40, 81, D)            # distances -40..40
    # sin^2 + cos^2 = 1 for each frequency
    _close(R[:, 0::2] ** 2 + R[:, 1::2] ** 2, np.ones((81, D // 2)), 1e-15)
    # distance 0 is [0, 1, 0, 1, ...]
    z = R[40]
    assert np.all(z[0::2] == 0.0) and np.all(z[1::2] == 1.0)
    # sine part odd, cosine part even in the distance
    _close(R[40 + 7, 0::2], -R[40 - 7, 0::2], 1e-15)
    _close(R[40 + 7, 1::2], R[40 - 7, 1::2], 1e-15)
    # angle addition: the angle is linear in the distance with a per-pair frequency
    a, b = 11, -4
    Ra, Rb, Rab = R[40 + a], R[40 + b], R[40 + a + b]
    _close(Rab[0::2], Ra[0::2] * Rb[1::2] + Ra[1::2] * Rb[0::2], 1e-13)
    _close(Rab[1::2], Ra[1::2] * Rb[1::2] - Ra[0::2] * Rb[0::2], 1e-13)
    # width 2 has the single frequency 1: [sin(delta), cos(delta)] from libm
    R2 = oracle.relpos_embed(-5, 11, 2)
    for n, d in enumerate(range(-5, 6)):
        assert R2[n, 0] == math.sin(d) and R2[n, 1] == math.cos(d)


def test_relpos_clamp_rows():
    R = oracle.relpos_embed(0, 30, 32, clamp_len=10)
    for n in range(11, 30):
        assert np.array_equal(R[n], R[10])
    Rn = oracle.relpos_embed(-30, 30, 32, clamp_len=10)   # negative side clamps to -10
    for n in range(0, 20):
        assert np.array_equal(Rn[n], Rn[20])


def test_bias_table_parameter_count():
    g = json.load(open(os.path.join(GOLDEN, "bias_table_param_count.json")))
    assert (2 * g["k"] + 1) * g["num_heads"] == g["exact"]
    assert abs(g["exact"] - g["printed_approx"]) < 100
    w = xl_inputs.WORKLOADS["segments_bf16"]
    t = xl_inputs.layer_inputs(w, batch=1, qlen=4)
    assert t["beta"].shape == (2 * 128 + 1, 16)


# --- layer: brute force and invariances -------------------------------------------

@pytest.mark.parametrize("seed,q,m,clamp,bias", [(0, 6, 5, -1, -1), (1, 1, 0, -1, -1), (2, 7, 0, 3, -1),
                                                 (3, 4, 9, 2, 3), (4, 5, 3, 0, 1), (5, 8, 8, 16, -1)])
def test_oracle_matches_independent_formulation(seed, q, m, clamp, bias):
    w = _tiny(seed, q=q, m=m, clamp_len=clamp, bias_clamp=bias)
    _close(_fwd(w), _brute(w), 1e-12)


def test_tiny_f32_workload_matches_brute():
    wl = xl_inputs.WORKLOADS["tiny_f32"]
    t = xl_inputs.layer_inputs(wl)
    w = {k: v.f64 for k, v in t.items()}
    w.update(n_head=wl.n_head, d_head=wl.d_head, clamp_len=wl.clamp_len, bias_clamp=-1)
    out = _fwd(w)
    _close(out, _brute(w), 1e-12)
    # the clamp of 16 never bites here (largest distance is klen-1 = 15)
    _close(out, _fwd(w, clamp_len=-1), 0.0)


def test_terms_match_brute_and_ablation():
    w = _tiny(7, q=5, m=4)
    out, terms, probs = _fwd(w, want_terms=True, want_probs=True)
    bout, bterms, bp = _brute(w, return_terms=True)
    for t, bt in zip(terms, bterms):
        _close(t, bt, 1e-12)
    _close(probs, bp, 1e-12)
    # zeroing u removes exactly term (c); zeroing v removes (d); W_r = 0 removes (b) and (d)
    _, t_u, _ = _fwd(w, u=np.zeros_like(w["u"]), want_terms=True, want_probs=True)
    assert np.all(t_u[2] == 0.0)
    _close(t_u[0], terms[0], 0.0)
    _close(t_u[1], terms[1], 0.0)
    _close(t_u[3], terms[3], 0.0)
    _, t_v, _ = _fwd(w, v=np.zeros_like(w["v"]), want_terms=True, want_probs=True)
    assert np.all(t_v[3] == 0.0)
    _close(t_v[2], terms[2], 0.0)
    _, t_r, _ = _fwd(w, w_r=np.zeros_like(w["w_r"]), want_terms=True, want_probs=True)
    assert np.all(t_r[1] == 0.0) and np.all(t_r[3] == 0.0)
    _close(t_r[0], terms[0], 0.0)
    # the logits are scale * (a+b+c+d): recover the probabilities from the terms
    s = 1.0 / math.sqrt(w["d_head"])
    logit = s * terms.sum(axis=0)
    m, q = w["mem"].shape[1], w["h"].shape[1]
    vis = np.arange(q + m)[None, :] <= (np.arange(q)[:, None] + m)
    logit = np.where(vis, logit, -np.inf)
    p = np.exp(logit - logit.max(-1, keepdims=True))
    _close(probs, p / p.sum(-1, keepdims=True), 1e-12)


def test_probs_rows_sum_to_one_and_masked_zero():
    w = _tiny(8, q=6, m=3, bias_clamp=2)
    _, probs = _fwd(w, want_probs=True)
    _close(probs.sum(-1), np.ones(probs.shape[:-1]), 1e-13)
    q, m = 6, 3
    for i in range(q):
        assert np.all(probs[:, :, i, m + i + 1:] == 0.0)
        assert np.all(probs[:, :, i, :m + i + 1] > 0.0)


def test_reduces_to_causal_sdpa():
    torch = pytest.importorskip("torch")
    w = _tiny(9, q=7, m=6)
    zero = dict(u=np.zeros_like(w["u"]), v=np.zeros_like(w["v"]), w_r=np.zeros_like(w["w_r"]))
    out = _fwd(w, **zero)
    B, q, D = w["h"].shape
    m = w["mem"].shape[1]
    H, dh = w["n_head"], w["d_head"]
    x = torch.from_numpy(np.concatenate([w["mem"], w["h"]], 1))
    hq = torch.from_numpy(w["h"])
    Q = torch.nn.functional.linear(hq, torch.from_numpy(w["w_q"])).view(B, q, H, dh).transpose(1, 2)
    K = torch.nn.functional.linear(x, torch.from_numpy(w["w_k"])).view(B, q + m, H, dh).transpose(1, 2)
    V = torch.nn.functional.linear(x, torch.from_numpy(w["w_v"])).view(B, q + m, H, dh).transpose(1, 2)
    mask = torch.arange(q + m)[None, :] <= (torch.arange(q)[:, None] + m)
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask)
    ref = torch.nn.functional.linear(o.transpose(1, 2).reshape(B, q, H * dh), torch.from_numpy(w["w_o"]))
    _close(out, ref.numpy(), 1e-12)


def test_clamp_zero_equals_no_position_term():
    # with C = 0 every distance uses R_0: the position terms are constant along each
    # row of scores and cancel in the softmax, as if W_r were zero
    w = _tiny(10, q=6, m=7)
    _close(_fwd(w, clamp_len=0), _fwd(w, w_r=np.zeros_like(w["w_r"])), 1e-12)
    # a clamp at or beyond the largest distance changes nothing
    _close(_fwd(w, clamp_len=12), _fwd(w, clamp_len=-1), 0.0)
    assert np.max(np.abs(_fwd(w, clamp_len=3) - _fwd(w))) > 1e-6


def test_translation_invariance():
    w = _tiny(11, q=5, m=6)
    q, m = 5, 6
    qpos = np.arange(q) + m
    kpos = np.arange(q + m)
    base = _fwd(w, qpos=qpos, kpos=kpos)
    _close(base, _fwd(w), 0.0)
    for T in (1, 37, 100000):
        _close(_fwd(w, qpos=qpos + T, kpos=kpos + T), base, 0.0)


def test_split_invariance():
    # the output of a position depends on its causal context, not on where the
    # memory/segment split falls
    rng = np.random.default_rng(12)
    w = _tiny(12, q=6, m=5)
    X = rng.standard_normal((2, 11, 16))
    a = _fwd(w, mem=X[:, :5], h=X[:, 5:11])
    b = _fwd(w, mem=X[:, :6], h=X[:, 6:11])
    _close(a[:, 1:], b, 1e-12)


def test_single_query_no_memory_is_value_path():
    w = _tiny(13, q=1, m=0)
    out = _fwd(w, mem=np.zeros((2, 0, 16)))
    ref = (w["h"] @ w["w_v"].T) @ w["w_o"].T
    _close(out, ref, 1e-13)


def test_bias_only_closed_form():
    # with W_q = W_k = W_r = 0 and u = v = 0 the logits are the table entries
    w = _tiny(14, q=4, m=3, bias_clamp=2)
    z = {k: np.zeros_like(w[k]) for k in ("w_q", "w_k", "w_r", "u", "v")}
    _, probs = _fwd(w, want_probs=True, **z)
    beta = w["beta"]
    q, m = 4, 3
    for hh in range(2):
        for i in range(q):
            d = (m + i) - np.arange(m + i + 1)
            logits = beta[np.clip(d, -2, 2) + 2, hh]
            p = np.exp(logits) / np.exp(logits).sum()
            _close(probs[0, hh, i, :m + i + 1], p, 1e-13)


def _t5_golden():
    return json.load(open(os.path.join(GOLDEN, "t5_buckets.json")))


def _t5_from_ranges(d, ranges):
    for i, (lo, hi) in enumerate(ranges):
        if d >= lo and (hi is None or d <= hi):
            return i
    raise AssertionError(f"distance {d} in no range")


def test_t5_bucket_matches_page_ranges():
    g = _t5_golden()
    assert g["num_buckets"] == len(g["boundaries"]) + 1 == len(g["ranges"])
    # the ranges tile [0, inf) and each upper end is the page's boundary
    assert g["ranges"][0][0] == 0
    for (lo, hi), (lo2, _), b in zip(g["ranges"], g["ranges"][1:], g["boundaries"]):
        assert hi == b and lo2 == hi + 1
    for d in list(range(0, 3000)) + [4095, 4096, 1 << 20, (1 << 40) + 3]:
        assert oracle.t5_bucket(d) == _t5_from_ranges(d, g["ranges"]), d
    for d in (-1, -2, -1025):
        assert oracle.t5_bucket(d) == 0


def test_t5_bias_only_closed_form():
    # zero projections and biases: the logits are beta[bucket(distance)]; key
    # positions chosen so that the distances reach every bucket
    g = _t5_golden()
    H = 2
    w = _tiny(17, H=H, q=3, m=13, bias_clamp=0, bias_kind=1)
    z = {k: np.zeros_like(w[k]) for k in ("w_q", "w_k", "w_r", "u", "v")}
    kpos = np.array([0, 1, 500, 1000, 1020, 1500, 1700, 1800, 1900, 1950, 1990, 2005, 2010, 2013, 2015, 2016])
    qpos = np.array([2014, 2016, 2017])
    _, probs = _fwd(w, want_probs=True, qpos=qpos, kpos=kpos, **z)
    beta = w["beta"]
    seen = set()
    for hh in range(H):
        for i, pi in enumerate(qpos):
            vis = kpos <= pi
            b = [_t5_from_ranges(int(pi - pj), g["ranges"]) for pj in kpos[vis]]
            seen.update(b)
            logits = beta[b, hh]
            p = np.exp(logits) / np.exp(logits).sum()
            _close(probs[0, hh, i, vis], p, 1e-13)
            assert np.all(probs[0, hh, i, ~vis] == 0)
    assert seen == set(range(12))


@pytest.mark.parametrize("seed,q,m,clamp", [(18, 6, 5, -1), (19, 9, 40, 8), (20, 1, 0, -1)])
def test_t5_oracle_matches_independent_formulation(seed, q, m, clamp):
    w = _tiny(seed, q=q, m=m, clamp_len=clamp, bias_clamp=0, bias_kind=1)
    _close(_fwd(w), _brute(w), 1e-12)


def test_t5_and_clamp_tables_agree_where_buckets_are_distances():
    # distances 0..2 fall in buckets 0, 0, 1; a clamp table with the same
    # values per distance gives the same layer
    w = _tiny(21, q=2, m=1, bias_clamp=0, bias_kind=1)
    t5 = w["beta"]
    clamp_tab = np.stack([t5[1], t5[0], t5[0], t5[0], t5[1]])   # rows d = -2..2
    _close(_fwd(w), _fwd(w, bias_kind=0, bias_clamp=2, beta=clamp_tab), 1e-14)


def test_p1_scaling_is_rescaled_biases():
    # scaling only (a)+(b), as the 2kiu.com module does, is the same model with
    # u, v divided by the scale
    w = _tiny(15, q=5, m=4)
    s = 1.0 / math.sqrt(w["d_head"])
    p1 = _brute(w, p1_scaling=True)
    _close(_fwd(w, u=w["u"] / s, v=w["v"] / s), p1, 1e-12)


def test_causality_and_masked_keys_ignored():
    w = _tiny(16, q=6, m=4)
    base = _fwd(w)
    h2 = w["h"].copy()
    h2[:, 4:] += 5.0                      # change the last two segment positions
    out2 = _fwd(w, h=h2)
    _close(out2[:, :4], base[:, :4], 0.0)  # earlier queries do not see them
    assert np.max(np.abs(out2[:, 4:] - base[:, 4:])) > 1e-3
    mem2 = w["mem"].copy()
    mem2[:, 0] += 1.0                      # every query sees the memory
    assert np.all(np.max(np.abs(_fwd(w, mem=mem2) - base), axis=-1) > 1e-6)


# --- layer normalisation and the decoder layer ----------------------------------------------

def test_layer_norm_moments_and_invariances():
    rng = np.random.default_rng(30)
    x = rng.standard_normal((7, 48)) * 3.0 + 1.5
    y = oracle.layer_norm(x, eps=0.0)
    _close(y.mean(axis=1), np.zeros(7), 1e-14)
    _close((y * y).mean(axis=1), np.ones(7), 1e-13)           # population variance 1
    _close(oracle.layer_norm(2.5 * x - 4.0, eps=0.0), y, 1e-13)  # affine invariance of the input
    g, bt = rng.standard_normal(48), rng.standard_normal(48)
    _close(oracle.layer_norm(x, g, bt, eps=0.0), y * g + bt, 1e-13)
    # a constant row normalises to beta; eps shrinks the output variance to var/(var+eps)
    c = np.full((2, 48), 3.25)
    _close(oracle.layer_norm(c, g, bt, eps=1e-5), np.broadcast_to(bt, (2, 48)), 0.0)
    v = x.var(axis=1)
    ye = oracle.layer_norm(x, eps=0.5)
    _close((ye * ye).mean(axis=1), v / (v + 0.5), 1e-13)


def _dec_weights(seed, D=16, H=2, dh=8, d_inner=24):
    w = _tiny(seed, D=D, H=H, dh=dh)
    rng = np.random.default_rng(seed + 1000)
    w.update(ln1_g=1.0 + 0.2 * rng.standard_normal(D), ln1_b=0.1 * rng.standard_normal(D),
             ln2_g=1.0 + 0.2 * rng.standard_normal(D), ln2_b=0.1 * rng.standard_normal(D),
             w1=0.3 * rng.standard_normal((d_inner, D)), b1=0.1 * rng.standard_normal(d_inner),
             w2=0.3 * rng.standard_normal((D, d_inner)), b2=0.1 * rng.standard_normal(D))
    return w


def _dec(w, **over):
    a = dict(w)
    a.update(over)
    return oracle.decoder_layer_fwd(a["h"], a["mem"], a, n_head=a["n_head"], d_head=a["d_head"],
                                    clamp_len=a["clamp_len"])


@pytest.mark.parametrize("seed,q,m,clamp", [(31, 6, 5, -1), (32, 1, 0, -1), (33, 7, 9, 3)])
def test_decoder_layer_matches_independent_formulation(seed, q, m, clamp):
    w = _dec_weights(seed)
    rng = np.random.default_rng(seed)
    w["h"] = rng.standard_normal((2, q, 16))
    w["mem"] = rng.standard_normal((2, m, 16))
    w["clamp_len"] = clamp
    ref = brute.decoder_layer(w["h"], w["mem"] if m else None, w, n_head=2, d_head=8, clamp_len=clamp)
    _close(_dec(w), ref, 1e-12)


def test_decoder_layer_identity_and_relu_cut():
    w = _dec_weights(34)
    # both sublayers contribute nothing: the layer is the identity
    z = dict(w_o=np.zeros_like(w["w_o"]), w2=np.zeros_like(w["w2"]), b2=np.zeros_like(w["b2"]))
    _close(_dec(w, **z), w["h"], 0.0)
    # a first-layer bias far below zero switches every ReLU off: the FFN adds b2
    h1 = w["h"] + oracle.rel_attn_fwd(oracle.layer_norm(w["h"], w["ln1_g"], w["ln1_b"]),
                                      oracle.layer_norm(w["mem"], w["ln1_g"], w["ln1_b"]), w["w_q"], w["w_k"],
                                      w["w_v"], w["w_r"], w["w_o"], w["u"], w["v"], n_head=2, d_head=8)
    _close(_dec(w, b1=np.full_like(w["b1"], -1e3)), h1 + w["b2"], 1e-13)


def test_decoder_stack_run_memories_and_identity():
    rng = np.random.default_rng(35)
    layers = [_dec_weights(36 + n) for n in range(3)]
    stream = rng.standard_normal((2, 4 * 5, 16))
    outs, mems = oracle.decoder_stack_run(stream, 4, 5, 7, layers, n_head=2, d_head=8)
    # layer 0's memory is the input stream itself (the last 7 rows seen)
    for t in range(4):
        seen = stream[:, :(t + 1) * 5]
        _close(mems[t][0], seen[:, -7:], 0.0)
    # a one-layer stack is the single-layer segment run with the decoder layer
    outs1, _ = oracle.decoder_stack_run(stream, 4, 5, 7, layers[:1], n_head=2, d_head=8)
    mem = np.zeros((2, 0, 16))
    for t in range(4):
        h = stream[:, t * 5:(t + 1) * 5]
        _close(outs1[t], oracle.decoder_layer_fwd(h, mem, layers[0], n_head=2, d_head=8), 0.0)
        mem = np.concatenate([mem, h], axis=1)[:, -7:]
    # identity layers pass the stream through and every layer remembers it
    ident = [dict(l, w_o=np.zeros_like(l["w_o"]), w2=np.zeros_like(l["w2"]), b2=np.zeros_like(l["b2"]))
             for l in layers]
    outs_i, mems_i = oracle.decoder_stack_run(stream, 4, 5, 7, ident, n_head=2, d_head=8)
    for t in range(4):
        _close(outs_i[t], stream[:, t * 5:(t + 1) * 5], 0.0)
        for n in range(3):
            _close(mems_i[t][n], mems_i[t][0], 0.0)


def test_fifo_update_and_segment_run():
    rng = np.random.default_rng(17)
    B, D, q, mmax = 2, 16, 4, 6
    stream = rng.standard_normal((B, 5 * q, D))
    mem = np.zeros((B, 0, D))
    for t in range(5):
        h = stream[:, t * q:(t + 1) * q]
        mem = oracle.fifo_update(mem, h, mmax)
        seen = stream[:, :(t + 1) * q]
        assert np.array_equal(mem, seen[:, max(0, seen.shape[1] - mmax):])
    w = _tiny(18, D=D, q=q, m=0)
    wts = {k: w[k] for k in ("w_q", "w_k", "w_v", "w_r", "w_o", "u", "v")}
    outs, mems = oracle.segment_run(stream, 5, q, mmax, wts, n_head=2, d_head=8)
    for t in range(5):
        prev = np.zeros((B, 0, D)) if t == 0 else mems[t - 1]
        _close(outs[t], _fwd(w, h=stream[:, t * q:(t + 1) * q], mem=prev), 0.0)
    # a long memory equals attending over the whole prefix
    outs_long, _ = oracle.segment_run(stream, 3, q, 100, wts, n_head=2, d_head=8)
    _close(outs_long[2], _fwd(w, h=stream[:, 2 * q:3 * q], mem=stream[:, :2 * q]), 0.0)


# --- the backward of the attention core --------------------------------------------------------

def _core_case(seed, B=2, H=2, dh=4, q=3, m=2, clamp=-1, bias=-1, kind=0):
    rng = np.random.default_rng(seed)
    kl = q + m
    n_rel = kl if clamp < 0 else min(kl, clamp + 1)
    c = dict(q=rng.standard_normal((B, H, q, dh)), k=rng.standard_normal((B, H, kl, dh)),
             v=rng.standard_normal((B, H, kl, dh)), r=rng.standard_normal((H, n_rel, dh)),
             u=0.5 * rng.standard_normal((H, dh)), vb=0.5 * rng.standard_normal((H, dh)),
             dout=rng.standard_normal((B, q, H * dh)), clamp=clamp, bias=bias, kind=kind, scale=0.7)
    c["beta"] = rng.standard_normal(((12 if kind else 2 * bias + 1), H)) * 0.5 if bias >= 0 else None
    return c


def _core_loss(c, **over):
    a = dict(c)
    a.update(over)
    o = oracle.rel_attn_core(a["q"], a["k"], a["v"], a["r"], a["u"], a["vb"], scale=a["scale"], clamp_len=a["clamp"],
                             beta=a["beta"], bias_clamp=a["bias"], bias_kind=a["kind"])
    return float(np.sum(o * a["dout"]))


def _core_grads(c):
    return oracle.rel_attn_core_bwd(c["q"], c["k"], c["v"], c["r"], c["u"], c["vb"], c["dout"], scale=c["scale"],
                                    clamp_len=c["clamp"], beta=c["beta"], bias_clamp=c["bias"], bias_kind=c["kind"])


@pytest.mark.parametrize("seed,q,m,clamp,bias,kind", [(40, 3, 2, -1, -1, 0), (41, 4, 3, 2, 1, 0), (42, 2, 0, -1, -1, 0),
                                                       (43, 3, 4, 1, 0, 1)])
def test_core_backward_matches_finite_differences(seed, q, m, clamp, bias, kind):
    c = _core_case(seed, q=q, m=m, clamp=clamp, bias=bias, kind=kind)
    g = _core_grads(c)
    eps = 1e-6
    for name, key in [("q", "dq"), ("k", "dk"), ("v", "dv"), ("r", "dr"), ("u", "du"), ("vb", "dv_bias"),
                      ("beta", "dbeta")]:
        if c[name] is None:
            assert g[key] is None
            continue
        x = c[name]
        fd = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            fd[idx] = (_core_loss(c, **{name: xp}) - _core_loss(c, **{name: xm})) / (2 * eps)
        _close(g[key], fd, 1e-7)


def test_core_backward_invariants():
    c = _core_case(44, B=2, H=3, dh=5, q=6, m=4, bias=2)
    g = _core_grads(c)
    # shifting every key of a head moves each query's logits by a constant
    _close(g["dk"].sum(axis=2), np.zeros((2, 3, 5)), 1e-12)
    # shifting every value shifts every output: sum_j dv_j = sum_i dout_i
    dsum = c["dout"].reshape(2, 6, 3, 5).sum(axis=1)
    _close(g["dv"].sum(axis=2), dsum, 1e-12)
    # a constant added to a head's whole bias table changes nothing
    _close(g["dbeta"].sum(axis=0), np.zeros(3), 1e-12)
    # q_i enters as q_i + u and q_i + v: du + dv_bias = sum over (b, i) of dq
    _close(g["du"] + g["dv_bias"], g["dq"].sum(axis=(0, 2)), 1e-12)
    z = _core_grads(dict(c, dout=np.zeros_like(c["dout"])))
    for key in ("dq", "dk", "dv", "dr", "du", "dv_bias", "dbeta"):
        assert np.all(z[key] == 0.0)
