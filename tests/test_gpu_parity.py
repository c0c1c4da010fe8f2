"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle.

Sizes: reduced batches the oracle finishes in seconds (several query/key tiles
and ragged tails), the full workload sizes in the benchmark's launch
configuration compared on sampled batch elements, and edge cases. Tolerances:
bf16 inputs with fp32 accumulation |g-o| <= 1e-2 + 2e-2|o|; the fp32 workload
|g-o| <= 1e-5 (|o| + max|o|).
"""
import zlib

import numpy as np
import pytest

import oracle
import xl_inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

W = xl_inputs.WORKLOADS


@pytest.fixture(scope="module")
def T():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import transformer_xl_relative_amd as xl
    xl.lib()
    return torch


def _run_layer(T, w, t, *, batch, qlen, mlen, out_f32=True):
    import transformer_xl_relative_amd as xl
    L = gu.Layer(w, t, batch=batch, qlen=qlen, mlen=mlen, out_f32=out_f32)
    h = gu.dev(t["h"])
    mem = gu.dev(t["mem"]) if mlen > 0 else None
    xl.xl_rel_attn_fwd(L.desc, L.weights, h, mem, L.out, L.ws)
    T.cuda.synchronize()
    return L


# --- relative embedding ---------------------------------------------------------

def test_relpos_worked_example(T):
    import transformer_xl_relative_amd as xl
    out = T.empty((1, 4), dtype=T.float32, device="cuda")
    xl.xl_relpos_embed(-2, 1, 4, -1, 10000.0, out)
    T.cuda.synchronize()
    got = out.cpu().numpy()[0]
    assert np.all(np.abs(got - np.array([-0.909, -0.416, -0.020, 0.999])) < 1e-3), got


@pytest.mark.parametrize("delta0,n,D,clamp", [(-40, 81, 64, -1), (0, 1664, 512, 1000), (-7, 300, 1024, 128),
                                              (0, 768, 1024, -1), (3, 5, 16, 16)])
def test_relpos_vs_oracle(T, delta0, n, D, clamp):
    import transformer_xl_relative_amd as xl
    ref = oracle.relpos_embed(delta0, n, D, clamp)
    o32 = T.empty((n, D), dtype=T.float32, device="cuda")
    obf = T.empty((n, D), dtype=T.bfloat16, device="cuda")
    xl.xl_relpos_embed(delta0, n, D, clamp, 10000.0, o32)
    xl.xl_relpos_embed(delta0, n, D, clamp, 10000.0, obf)
    T.cuda.synchronize()
    g32 = o32.cpu().numpy().astype(np.float64)
    # fp64 evaluation rounded once: within half an ulp of float32 (device and host
    # libm may differ in the last fp64 bit, hence the small slack)
    assert np.all(np.abs(g32 - ref) <= 2.0 ** -24 * np.abs(ref) * (1 + 1e-6) + 1e-45)
    gbf = gu.host64(obf)
    # bfloat16 keeps 8 significant bits: half an ulp is at most 2^-8 relative
    assert np.all(np.abs(gbf - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)
    # exactly the nearest bfloat16 of the oracle value except at rounding ties of libm differences
    want = xl_inputs.bf16_to_f32(xl_inputs.bf16_bits(ref.astype(np.float32))).astype(np.float64)
    assert np.mean(gbf != want) < 1e-3


# --- whole layer at reduced batch: output and every intermediate ---------------------

def _check_intermediates(T, L, w, t, batch, qlen, mlen):
    lay = L.layout
    H, dh, D = w.n_head, w.d_head, w.d_model
    h = t["h"].f64[:batch, :qlen]
    mem = t["mem"].f64[:batch, :mlen]
    x = np.concatenate([mem, h], axis=1)
    klen = qlen + mlen
    q = oracle.linear(h, t["w_q"].f64).reshape(batch, qlen, H, dh).transpose(0, 2, 1, 3)
    k = oracle.linear(x, t["w_k"].f64).reshape(batch, klen, H, dh).transpose(0, 2, 1, 3)
    v = oracle.linear(x, t["w_v"].f64).reshape(batch, klen, H, dh).transpose(0, 2, 1, 3)
    R = oracle.relpos_embed(0, lay.n_rel, D)
    r = oracle.linear(R, t["w_r"].f64).reshape(lay.n_rel, H, dh).transpose(1, 0, 2)
    gu.compare("q", gu.host64(L.ws_view(lay.q, (batch, H, qlen, dh))), q, dtype=w.dtype)
    gu.compare("k", gu.host64(L.ws_view(lay.k, (batch, H, klen, dh))), k, dtype=w.dtype)
    vt = gu.host64(L.ws_view(lay.vt, (batch, H, dh, lay.ldv)))[..., :klen]
    gu.compare("vt", vt, v.transpose(0, 1, 3, 2), dtype=w.dtype)
    gu.compare("rel", gu.host64(L.ws_view(lay.rel, (lay.n_rel, D))), R, dtype=w.dtype)
    gu.compare("r", gu.host64(L.ws_view(lay.r, (H, lay.n_rel, dh))), r, dtype=w.dtype)


@pytest.mark.parametrize("name,batch,qlen,mlen", [
    ("tiny_f32", 1, 8, 8),
    ("base_bf16", 2, 128, 128),
    ("large_bf16", 1, 384, 384),
    ("longmem_bf16", 1, 64, 1600),
])
def test_layer_reduced(T, name, batch, qlen, mlen):
    w = W[name]
    t = xl_inputs.layer_inputs(w, batch=batch, qlen=qlen, mlen=mlen)
    L = _run_layer(T, w, t, batch=batch, qlen=qlen, mlen=mlen)
    ref = gu.oracle_layer(t, w, t["h"].f64, t["mem"].f64)
    gu.compare(f"{name} out", gu.host64(L.out), ref, dtype=w.dtype)
    _check_intermediates(T, L, w, t, batch, qlen, mlen)


def test_layer_bf16_output(T):
    w = W["base_bf16"]
    t = xl_inputs.layer_inputs(w, batch=1, qlen=96, mlen=40)
    L = _run_layer(T, w, t, batch=1, qlen=96, mlen=40, out_f32=False)
    ref = gu.oracle_layer(t, w, t["h"].f64, t["mem"].f64)
    gu.compare("bf16 out", gu.host64(L.out), ref, dtype="bf16")


# --- full workload sizes, sampled batch elements ------------------------------------------

@pytest.mark.parametrize("name", ["tiny_f32", "base_bf16", "large_bf16", "longmem_bf16"])
def test_layer_full_size_sampled(T, name):
    w = W[name]
    t = xl_inputs.layer_inputs(w)
    L = _run_layer(T, w, t, batch=w.batch, qlen=w.qlen, mlen=w.mlen)
    out = gu.host64(L.out)
    bsel = sorted({0, w.batch - 1})
    ref = gu.oracle_layer(t, w, t["h"].f64, t["mem"].f64, bsel=bsel)
    gu.compare(f"{name} full (batches {bsel})", out[bsel], ref, dtype=w.dtype)


# --- edge cases -------------------------------------------------------------------------------

EDGE = [
    # (label, dtype workload, qlen, mlen, clamp_len, bias_clamp)
    ("q1_m0", "base_bf16", 1, 0, -1, -1),
    ("q1_m1600", "longmem_bf16", 1, 1600, 1000, -1),
    ("ragged_q37_m91", "base_bf16", 37, 91, -1, -1),
    ("klen_lt_tile", "base_bf16", 5, 3, -1, -1),
    ("two_qtiles_ragged", "base_bf16", 200, 17, -1, -1),
    ("mlen0_q130", "base_bf16", 130, 0, -1, -1),
    ("clamp0", "base_bf16", 40, 30, 0, -1),
    ("clamp3", "base_bf16", 40, 30, 3, -1),
    ("clamp_klen_minus1", "base_bf16", 40, 30, 69, -1),
    ("bias_on", "base_bf16", 70, 50, -1, 16),
    ("bias_and_clamp", "base_bf16", 70, 50, 20, 8),
    ("f32_ragged", "tiny_f32", 13, 29, 5, -1),
    ("f32_bias", "tiny_f32", 9, 4, -1, 3),
]


@pytest.mark.parametrize("label,base,qlen,mlen,clamp,bias", EDGE, ids=[e[0] for e in EDGE])
def test_edge_cases(T, label, base, qlen, mlen, clamp, bias):
    import dataclasses
    w = dataclasses.replace(W[base], clamp_len=clamp, bias_clamp=bias, seed=zlib.crc32(label.encode()) % 1000)
    t = xl_inputs.layer_inputs(w, batch=2, qlen=qlen, mlen=mlen)
    L = _run_layer(T, w, t, batch=2, qlen=qlen, mlen=mlen)
    ref = gu.oracle_layer(t, w, t["h"].f64, t["mem"].f64)
    gu.compare(label, gu.host64(L.out), ref, dtype=w.dtype)


@pytest.mark.parametrize("d_model,n_head", [(32, 1), (96, 2), (160, 3), (544, 8)])
def test_layer_model_width(T, d_model, n_head):
    # d_model a multiple of 32 but not of 64: the projections end on a K stage
    # of half width; also output widths that leave ragged column tiles
    import dataclasses
    w = dataclasses.replace(W["base_bf16"], d_model=d_model, n_head=n_head, seed=d_model + n_head)
    t = xl_inputs.layer_inputs(w, batch=2, qlen=70, mlen=45)
    L = _run_layer(T, w, t, batch=2, qlen=70, mlen=45)
    ref = gu.oracle_layer(t, w, t["h"].f64, t["mem"].f64)
    gu.compare(f"d_model {d_model}", gu.host64(L.out), ref, dtype=w.dtype)
    _check_intermediates(T, L, w, t, 2, 70, 45)


def test_layer_projection_tall_tiles(T):
    # batch 8, qlen 608, mlen 544 at d_model 512: the grouped projection makes
    # 192 tiles of 256 x 256 and 256 of 192 x 256, so it runs on the latter;
    # query tiles cross batch boundaries (608 rows is not a multiple of 192)
    # and the key, transposed value and R epilogues see 192-row tiles
    w = W["base_bf16"]
    t = xl_inputs.layer_inputs(w, batch=8, qlen=608, mlen=544)
    L = _run_layer(T, w, t, batch=8, qlen=608, mlen=544)
    _check_intermediates(T, L, w, t, 8, 608, 544)
    bsel = [0, 5, 7]
    ref = gu.oracle_layer(t, w, t["h"].f64, t["mem"].f64, bsel=bsel)
    gu.compare(f"tall projection (batches {bsel})", gu.host64(L.out)[bsel], ref, dtype=w.dtype)


@pytest.mark.parametrize("base,qlen,mlen,clamp", [("base_bf16", 70, 1000, -1), ("base_bf16", 130, 0, -1),
                                                  ("longmem_bf16", 64, 1600, 1000), ("tiny_f32", 9, 1030, 5)])
def test_layer_t5_bias(T, base, qlen, mlen, clamp):
    # the whole layer with the T5 bucket table
    import dataclasses
    w = dataclasses.replace(W[base], clamp_len=clamp, bias_clamp=0, bias_kind=1, seed=qlen + mlen)
    t = xl_inputs.layer_inputs(w, batch=2, qlen=qlen, mlen=mlen)
    assert t["beta"].f32.shape == (12, w.n_head)
    L = _run_layer(T, w, t, batch=2, qlen=qlen, mlen=mlen)
    ref = gu.oracle_layer(t, w, t["h"].f64, t["mem"].f64)
    gu.compare(f"t5 {base} q{qlen} m{mlen}", gu.host64(L.out), ref, dtype=w.dtype)


def test_split_invariance_gpu(T):
    # the output of a position does not depend on where the memory/segment split falls
    import dataclasses
    w = dataclasses.replace(W["base_bf16"], seed=77)
    t = xl_inputs.layer_inputs(w, batch=1, qlen=100, mlen=60)
    X = np.concatenate([t["mem"].f32, t["h"].f32], axis=1)
    outs = []
    for m in (60, 61):
        t2 = dict(t)
        t2["mem"] = xl_inputs.Tensor(X[:, :m], "bf16")
        t2["h"] = xl_inputs.Tensor(X[:, m:], "bf16")
        L = _run_layer(T, w, t2, batch=1, qlen=160 - m, mlen=m)
        outs.append(gu.host64(L.out))
    np.testing.assert_allclose(outs[0][:, 1:], outs[1], rtol=2e-2, atol=1e-2)


# --- the fused attention kernel alone ----------------------------------------------------------

CORE = [
    # dtype, B, H, qlen, mlen, clamp, bias, attn_splits (0: the library's choice)
    ("bf16", 2, 3, 200, 75, -1, -1, 0),
    ("bf16", 1, 2, 64, 1600, 1000, -1, 0),     # long memory: split by the library
    ("bf16", 2, 2, 129, 128, -1, 128, 0),
    ("f32", 2, 2, 20, 11, 7, -1, 0),
    # forced key splits: uneven boundaries, empty splits (the first query tile
    # has only three fully visible steps), the diagonal tile, decode-like q = 1
    ("bf16", 2, 3, 200, 75, -1, -1, 3),
    ("bf16", 2, 2, 129, 128, -1, 128, 16),
    ("bf16", 1, 2, 1, 1600, 1000, -1, 7),
    ("bf16", 1, 1, 300, 0, -1, -1, 2),
    ("bf16", 2, 2, 64, 700, 300, 40, 64),
]


@pytest.mark.parametrize("dtype,B,H,qlen,mlen,clamp,bias,splits", CORE,
                         ids=[f"{c[0]}-B{c[1]}H{c[2]}-q{c[3]}m{c[4]}-c{c[5]}b{c[6]}-s{c[7]}" for c in CORE])
def test_core_alone(T, dtype, B, H, qlen, mlen, clamp, bias, splits):
    _core_case(T, dtype, B, H, qlen, mlen, clamp, bias, splits)


CORE_T5 = [
    # T5 bucket rows: distances past 1024 reach the last bucket; with key
    # splits; a tile whose distances stay in the first buckets; fp32
    ("bf16", 2, 2, 129, 1000, -1, 0),
    ("bf16", 1, 3, 64, 1600, 1000, 7),
    ("bf16", 2, 2, 40, 0, -1, 0),
    ("f32", 2, 2, 40, 1100, -1, 0),
]


@pytest.mark.parametrize("dtype,B,H,qlen,mlen,clamp,splits", CORE_T5,
                         ids=[f"{c[0]}-B{c[1]}H{c[2]}-q{c[3]}m{c[4]}-c{c[5]}-s{c[6]}" for c in CORE_T5])
def test_core_t5_bias(T, dtype, B, H, qlen, mlen, clamp, splits):
    _core_case(T, dtype, B, H, qlen, mlen, clamp, 0, splits, bias_kind=1)


def _core_case(T, dtype, B, H, qlen, mlen, clamp, bias, splits, bias_kind=0):
    import transformer_xl_relative_amd as xl
    dh = 64 if dtype == "bf16" else 8
    klen = qlen + mlen
    n_rel = klen if clamp < 0 else min(klen, clamp + 1)
    ci = xl_inputs.core_inputs(batch=B, n_head=H, d_head=dh, qlen=qlen, mlen=mlen, n_rows=n_rel, dtype=dtype,
                               seed=B * 100 + qlen + 7 * bias_kind, bias_clamp=bias, bias_kind=bias_kind)
    s = 1.0 / np.sqrt(dh)
    # operands in the kernel's layout: transposed values
    ldv = (klen + 7) // 8 * 8 + 8
    vt = np.zeros((B, H, dh, ldv), np.float32)
    vt[..., :klen] = ci["v"].f32.transpose(0, 1, 3, 2)
    vt = xl_inputs.Tensor(vt, dtype)
    desc = xl.make_desc(batch=B, d_model=2, n_head=H, d_head=dh, qlen=qlen, mlen=mlen, clamp_len=clamp,
                        bias_clamp=bias, dtype=xl.XL_BF16 if dtype == "bf16" else xl.XL_F32, attn_splits=splits,
                        bias_kind=bias_kind)
    attn = T.empty((B, qlen, H * dh), dtype=T.bfloat16 if dtype == "bf16" else T.float32, device="cuda")
    beta = gu.dev(ci["beta"]) if bias >= 0 else None
    nws = xl.xl_rel_attn_core_workspace_size(desc)
    if splits > 1 or (dtype == "bf16" and mlen >= 1600):
        assert nws > 0
    ws = T.empty(nws, dtype=T.uint8, device="cuda") if nws else None
    xl.xl_rel_attn_core(desc, gu.dev(ci["q"]), gu.dev(ci["k"]), gu.dev(vt), ldv, gu.dev(ci["r"]), n_rel,
                        gu.dev(ci["u"]), gu.dev(ci["vb"]), beta, attn, ws)
    T.cuda.synchronize()
    ref = oracle.rel_attn_core(ci["q"].f64, ci["k"].f64, ci["v"].f64, ci["r"].f64, ci["u"].f64, ci["vb"].f64,
                               scale=s, clamp_len=clamp, beta=ci["beta"].f64 if bias >= 0 else None,
                               bias_clamp=bias, bias_kind=bias_kind)
    gu.compare("core", gu.host64(attn), ref, dtype=dtype)


# --- segment-recurrent run with the FIFO memory -------------------------------------------------

def _segment_run_gpu(T, w, t, *, batch, qlen, n_seg, mlen_max, head0=0):
    import transformer_xl_relative_amd as xl
    stream = t["h"]
    D = w.d_model
    dt = xl.XL_BF16 if w.dtype == "bf16" else xl.XL_F32
    tdt = T.bfloat16 if w.dtype == "bf16" else T.float32
    L = gu.Layer(w, t, batch=batch, qlen=qlen, mlen=mlen_max)   # workspace for the largest memory
    ring = T.zeros((batch, mlen_max, D), dtype=tdt, device="cuda")
    fifo = xl.xl_mem_fifo(ring.data_ptr(), mlen_max, 0, head0)
    hs = gu.dev(stream)
    outs, mems = [], []
    for s in range(n_seg):
        h = hs[:, s * qlen:(s + 1) * qlen].contiguous()
        out = T.empty((batch, qlen, D), dtype=T.float32, device="cuda")
        desc = xl.make_desc(batch=batch, d_model=D, n_head=w.n_head, d_head=w.d_head, qlen=qlen, mlen=0,
                            clamp_len=w.clamp_len, bias_clamp=w.bias_clamp, bias_kind=w.bias_kind, dtype=dt,
                            out_dtype=xl.XL_F32)
        xl.xl_segment_step(desc, L.weights, h, fifo, out, L.ws)
        T.cuda.synchronize()
        outs.append(gu.host64(out))
        # logical memory order from the ring
        idx = [(fifo.head + i) % mlen_max for i in range(fifo.len)]
        mems.append(ring[:, idx].clone())
        assert fifo.len == min((s + 1) * qlen, mlen_max)
    return outs, mems


@pytest.mark.parametrize("qlen,n_seg,mlen_max,head0", [(128, 4, 128, 0), (96, 4, 200, 0), (64, 3, 50, 7),
                                                       (40, 5, 100, 99)])
def test_segment_run_reduced(T, qlen, n_seg, mlen_max, head0):
    import dataclasses
    w = dataclasses.replace(W["segments_bf16"], qlen=qlen, mlen=mlen_max, segments=n_seg)
    t = xl_inputs.layer_inputs(w, batch=1, qlen=qlen)
    outs, mems = _segment_run_gpu(T, w, t, batch=1, qlen=qlen, n_seg=n_seg, mlen_max=mlen_max, head0=head0)
    wts = {k: t[k].f64 for k in ("w_q", "w_k", "w_v", "w_r", "w_o", "u", "v", "beta")}
    routs, rmems = oracle.segment_run(t["h"].f64, n_seg, qlen, mlen_max, wts, n_head=w.n_head, d_head=w.d_head,
                                      clamp_len=w.clamp_len, bias_clamp=w.bias_clamp, bias_kind=w.bias_kind)
    for s in range(n_seg):
        gu.compare(f"segment {s}", outs[s], routs[s], dtype="bf16")
        # the memory holds copies of the input states: bit-exact
        want = xl_inputs.bf16_bits(rmems[s].astype(np.float32))
        assert np.array_equal(gu.bits_u16(mems[s]), want), f"memory after segment {s} differs"


def test_segment_run_full_size_sampled(T):
    w = W["segments_bf16"]
    t = xl_inputs.layer_inputs(w)
    outs, mems = _segment_run_gpu(T, w, t, batch=w.batch, qlen=w.qlen, n_seg=w.segments, mlen_max=w.mlen)
    wts = {k: t[k].f64 for k in ("w_q", "w_k", "w_v", "w_r", "w_o", "u", "v", "beta")}
    routs, rmems = oracle.segment_run(t["h"].f64[:1], w.segments, w.qlen, w.mlen, wts, n_head=w.n_head,
                                      d_head=w.d_head, clamp_len=w.clamp_len, bias_clamp=w.bias_clamp,
                                      bias_kind=w.bias_kind)
    for s in range(w.segments):
        gu.compare(f"segment {s} (batch 0)", outs[s][:1], routs[s], dtype="bf16")
        want = xl_inputs.bf16_bits(rmems[s].astype(np.float32))
        assert np.array_equal(gu.bits_u16(mems[s][:1]), want)


# --- the same run on a key ring of projected keys and values ----------------------------------

def _segment_run_kv(T, w, t, *, batch, qlen, n_seg, mlen_max, cap, head0=0):
    import transformer_xl_relative_amd as xl
    L = gu.Layer(w, t, batch=batch, qlen=qlen, mlen=mlen_max)
    H, dh, D = w.n_head, w.d_head, w.d_model
    kr = T.empty((batch, H, cap, dh), dtype=T.bfloat16, device="cuda")
    vr = T.empty((batch, H, dh, cap), dtype=T.bfloat16, device="cuda")
    kr.fill_(float("nan"))     # never read before written
    vr.fill_(float("nan"))
    kv = xl.xl_kv_fifo(kr.data_ptr(), vr.data_ptr(), cap, mlen_max, 0, head0)
    ws = T.empty(max(xl.xl_segment_step_kv_workspace_size(L.desc), 1), dtype=T.uint8, device="cuda")
    hs = gu.dev(t["h"])
    outs = []
    for s in range(n_seg):
        h = hs[:, s * qlen:(s + 1) * qlen].contiguous()
        out = T.empty((batch, qlen, D), dtype=T.float32, device="cuda")
        desc = xl.make_desc(batch=batch, d_model=D, n_head=H, d_head=dh, qlen=qlen, mlen=0,
                            clamp_len=w.clamp_len, bias_clamp=w.bias_clamp, bias_kind=w.bias_kind,
                            dtype=xl.XL_BF16, out_dtype=xl.XL_F32)
        xl.xl_segment_step_kv(desc, L.weights, h, kv, out, ws)
        T.cuda.synchronize()
        outs.append(out.clone())
        assert kv.len == min((s + 1) * qlen, mlen_max)
    return outs


@pytest.mark.parametrize("qlen,n_seg,mlen_max,cap,head0", [(128, 4, 128, 256, 0), (64, 5, 200, 272, 16),
                                                           (40, 6, 96, 144, 136), (64, 6, 256, 320, 0)])
def test_segment_run_kv_ring(T, qlen, n_seg, mlen_max, cap, head0):
    # the key ring holds the keys and values the state FIFO path computes from
    # the stored states, so both runs give the same bits; and both match the oracle
    import dataclasses
    w = dataclasses.replace(W["segments_bf16"], qlen=qlen, mlen=mlen_max, segments=n_seg)
    t = xl_inputs.layer_inputs(w, batch=1, qlen=qlen)
    ring_outs = _segment_run_kv(T, w, t, batch=1, qlen=qlen, n_seg=n_seg, mlen_max=mlen_max, cap=cap,
                                head0=head0)
    outs, _ = _segment_run_gpu(T, w, t, batch=1, qlen=qlen, n_seg=n_seg, mlen_max=mlen_max)
    wts = {k: t[k].f64 for k in ("w_q", "w_k", "w_v", "w_r", "w_o", "u", "v", "beta")}
    routs, _ = oracle.segment_run(t["h"].f64, n_seg, qlen, mlen_max, wts, n_head=w.n_head, d_head=w.d_head,
                                  clamp_len=w.clamp_len, bias_clamp=w.bias_clamp, bias_kind=w.bias_kind)
    for s in range(n_seg):
        got = gu.host64(ring_outs[s])
        assert np.array_equal(got, outs[s]), f"segment {s}: key ring and state FIFO differ"
        gu.compare(f"key ring segment {s}", got, routs[s], dtype="bf16")


def test_segment_run_kv_ring_t5(T):
    # the segment step on the key ring with the T5 bucket table: memory grows
    # past 1024 positions, so every bucket is used
    import dataclasses
    qlen, n_seg, mlen_max, cap = 256, 6, 1024, 1280
    w = dataclasses.replace(W["segments_bf16"], n_head=4, qlen=qlen, mlen=mlen_max, segments=n_seg, bias_clamp=0,
                            bias_kind=1)
    t = xl_inputs.layer_inputs(w, batch=1, qlen=qlen)
    ring_outs = _segment_run_kv(T, w, t, batch=1, qlen=qlen, n_seg=n_seg, mlen_max=mlen_max, cap=cap, head0=8)
    wts = {k: t[k].f64 for k in ("w_q", "w_k", "w_v", "w_r", "w_o", "u", "v", "beta")}
    routs, _ = oracle.segment_run(t["h"].f64, n_seg, qlen, mlen_max, wts, n_head=w.n_head, d_head=w.d_head,
                                  clamp_len=w.clamp_len, bias_clamp=w.bias_clamp, bias_kind=w.bias_kind)
    for s in range(n_seg):
        gu.compare(f"t5 key ring segment {s}", gu.host64(ring_outs[s]), routs[s], dtype="bf16")


def test_segment_run_kv_ring_tall_tiles(T):
    # batch 8, qlen 480, 192 memory rows at d_model 1024: the second segment's
    # grouped projection (R, the queries and the segment's keys and values)
    # makes 192 tiles of 256 x 256 and 256 of 192 x 256, so its key and value
    # rows go into the wrapped ring from 192-row tiles that cross batch elements
    import dataclasses
    qlen, n_seg, mlen_max, cap, batch = 480, 2, 192, 704, 8
    w = dataclasses.replace(W["segments_bf16"], qlen=qlen, mlen=mlen_max, segments=n_seg, seed=480)
    t = xl_inputs.layer_inputs(w, batch=batch, qlen=qlen)
    ring_outs = _segment_run_kv(T, w, t, batch=batch, qlen=qlen, n_seg=n_seg, mlen_max=mlen_max, cap=cap,
                                head0=600)
    bsel = [0, 3, 7]
    wts = {k: t[k].f64 for k in ("w_q", "w_k", "w_v", "w_r", "w_o", "u", "v", "beta") if k in t}
    routs, _ = oracle.segment_run(t["h"].f64[bsel], n_seg, qlen, mlen_max, wts, n_head=w.n_head, d_head=w.d_head,
                                  clamp_len=w.clamp_len, bias_clamp=w.bias_clamp, bias_kind=w.bias_kind)
    for s in range(n_seg):
        gu.compare(f"tall key ring segment {s} (batches {bsel})", gu.host64(ring_outs[s])[bsel], routs[s],
                   dtype="bf16")


def test_segment_run_kv_ring_full_size(T):
    # the segmented workload at full size (batch 4, 16 heads, qlen = mlen = 512),
    # key ring against the state FIFO path, bit for bit
    w = W["segments_bf16"]
    t = xl_inputs.layer_inputs(w)
    ring_outs = _segment_run_kv(T, w, t, batch=w.batch, qlen=w.qlen, n_seg=w.segments, mlen_max=w.mlen,
                                cap=w.mlen + w.qlen + 64, head0=24)
    outs, _ = _segment_run_gpu(T, w, t, batch=w.batch, qlen=w.qlen, n_seg=w.segments, mlen_max=w.mlen)
    for s in range(w.segments):
        assert np.array_equal(gu.host64(ring_outs[s]), outs[s]), f"segment {s} differs"


# --- the table of a full-memory segment run, computed once -----------------------------------

@pytest.mark.parametrize("kv_ring", [False, True])
def test_reuse_table_bit_identical(T, kv_ring):
    # once the memory is full the table rows no longer change (they depend on
    # the distance alone); steps that skip the sinusoid and the R projection
    # (XL_REUSE_TABLE) give the same bits as steps that recompute them
    import dataclasses
    import transformer_xl_relative_amd as xl
    qlen, n_seg, mlen_max = 64, 6, 128
    w = dataclasses.replace(W["segments_bf16"], n_head=4, qlen=qlen, mlen=mlen_max, segments=n_seg, bias_clamp=16,
                            clamp_len=150, seed=61)
    t = xl_inputs.layer_inputs(w, batch=2, qlen=qlen, recipe="sensitive")
    L = gu.Layer(w, t, batch=2, qlen=qlen, mlen=mlen_max)
    H, dh, D = w.n_head, w.d_head, w.d_model
    hs = gu.dev(t["h"])
    runs = []
    for reuse in (False, True):
        ring = T.zeros((2, mlen_max, D), dtype=T.bfloat16, device="cuda")
        fifo = xl.xl_mem_fifo(ring.data_ptr(), mlen_max, 0, 0)
        cap = mlen_max + qlen + 8
        kr = T.zeros((2, H, cap, dh), dtype=T.bfloat16, device="cuda")
        vr = T.zeros((2, H, dh, cap), dtype=T.bfloat16, device="cuda")
        kv = xl.xl_kv_fifo(kr.data_ptr(), vr.data_ptr(), cap, mlen_max, 0, 0)
        ws = T.empty(L.ws.numel(), dtype=T.uint8, device="cuda")
        outs = []
        for s in range(n_seg):
            full = (fifo.len if not kv_ring else kv.len) == mlen_max
            flags = xl.XL_REUSE_TABLE if reuse and full and s >= 3 else 0
            desc = xl.make_desc(batch=2, d_model=D, n_head=H, d_head=dh, qlen=qlen, mlen=0, clamp_len=w.clamp_len,
                                bias_clamp=w.bias_clamp, dtype=xl.XL_BF16, out_dtype=xl.XL_F32, flags=flags)
            out = T.empty((2, qlen, D), dtype=T.float32, device="cuda")
            h = hs[:, s * qlen:(s + 1) * qlen].contiguous()
            if kv_ring:
                xl.xl_segment_step_kv(desc, L.weights, h, kv, out, ws)
            else:
                xl.xl_segment_step(desc, L.weights, h, fifo, out, ws)
            T.cuda.synchronize()
            outs.append(gu.host64(out))
        runs.append(outs)
    for s in range(n_seg):
        assert np.array_equal(runs[0][s], runs[1][s]), f"segment {s}"
