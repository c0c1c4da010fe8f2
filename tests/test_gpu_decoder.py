"""GPU parity of the pre-LN decoder layer and the segment-recurrent decoder
stack against the fp64 oracle, through the C ABI."""
import dataclasses

import numpy as np
import pytest

import oracle
import transformer_xl_relative_amd as xl
import xl_inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
W = xl_inputs.WORKLOADS


@pytest.fixture(scope="module")
def T():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    xl.lib()
    return torch


def _desc(w, *, batch, qlen, mlen, out_f32=True):
    dt = xl.XL_BF16 if w.dtype == "bf16" else xl.XL_F32
    return xl.make_desc(batch=batch, d_model=w.d_model, n_head=w.n_head, d_head=w.d_head, qlen=qlen, mlen=mlen,
                        clamp_len=w.clamp_len, bias_clamp=w.bias_clamp, bias_kind=w.bias_kind, dtype=dt,
                        out_dtype=xl.XL_F32 if out_f32 else dt)


def _oracle_layer(t, w, lw, h, mem):
    return oracle.decoder_layer_fwd(h, mem, gu.oracle_dec_weights(lw), n_head=w.n_head, d_head=w.d_head,
                                    clamp_len=w.clamp_len, bias_clamp=w.bias_clamp, bias_kind=w.bias_kind)


def _run_layer(T, w, t, *, batch, qlen, mlen, d_inner):
    desc = _desc(w, batch=batch, qlen=qlen, mlen=mlen)
    ws = T.empty(xl.xl_decoder_layer_workspace_size(desc, d_inner), dtype=T.uint8, device="cuda")
    out = T.empty((batch, qlen, w.d_model), dtype=T.float32, device="cuda")
    xl.xl_decoder_layer_fwd(desc, d_inner, 0.0, gu.dec_weights(t["layers"][0]), gu.dev(t["h"]),
                            gu.dev(t["mem"]) if mlen else None, out, ws)
    T.cuda.synchronize()
    return gu.host64(out)


# (the last two: rows longer than the layer norm keeps in registers; kind 1: the T5 log-bucket table)
@pytest.mark.parametrize("base,qlen,mlen,d_inner,bias,wide,kind", [
    ("base_bf16", 70, 45, 256, -1, 0, 0), ("base_bf16", 128, 0, 512, -1, 0, 0), ("base_bf16", 37, 91, 96, 16, 0, 0),
    ("tiny_f32", 9, 13, 32, -1, 0, 0), ("tiny_f32", 8, 8, 64, 3, 0, 0), ("base_bf16", 20, 12, 64, -1, 2560, 0),
    ("tiny_f32", 6, 5, 32, -1, 1040, 0), ("base_bf16", 48, 1100, 128, 0, 0, 1), ("tiny_f32", 7, 40, 32, 0, 0, 1)])
def test_decoder_layer(T, base, qlen, mlen, d_inner, bias, wide, kind):
    w = dataclasses.replace(W[base], bias_clamp=bias, bias_kind=kind, seed=qlen * 7 + mlen)
    if wide:
        w = dataclasses.replace(w, d_model=wide, n_head=2)
    t = xl_inputs.decoder_inputs(w, d_inner=d_inner, n_layer=1, batch=2, qlen=qlen, mlen=mlen)
    got = _run_layer(T, w, t, batch=2, qlen=qlen, mlen=mlen, d_inner=d_inner)
    ref = _oracle_layer(t, w, t["layers"][0], t["h"].f64, t["mem"].f64)
    gu.compare(f"decoder layer {base} q{qlen} m{mlen}", got, ref, dtype=w.dtype)


def test_decoder_layer_large_sampled(T):
    # the large workload's shape with a 4096-wide feed-forward network; batch 0 checked
    w = W["large_bf16"]
    t = xl_inputs.decoder_inputs(w, d_inner=4096, n_layer=1)
    got = _run_layer(T, w, t, batch=w.batch, qlen=w.qlen, mlen=w.mlen, d_inner=4096)
    ref = _oracle_layer(t, w, t["layers"][0], t["h"].f64[:1], t["mem"].f64[:1])
    gu.compare("decoder layer large (batch 0)", got[:1], ref, dtype="bf16")


def test_decoder_layer_ragged_tall_tiles(T):
    # the first feed-forward product, 1520 x 8000 x 1056, makes 6 x 32 = 192 tiles of
    # 256 x 256 and 8 x 32 = 256 of 192 x 256, so it runs on the latter, with ragged
    # row and column tiles (1520 = 7 x 192 + 176, 8000 = 31 x 256 + 64) and a K of
    # 32 mod 64 (a half-width last stage); batch 0 checked
    w = dataclasses.replace(W["base_bf16"], d_model=1056, n_head=2, seed=1056)
    t = xl_inputs.decoder_inputs(w, d_inner=8000, n_layer=1, batch=2, qlen=760, mlen=24)
    got = _run_layer(T, w, t, batch=2, qlen=760, mlen=24, d_inner=8000)
    ref = _oracle_layer(t, w, t["layers"][0], t["h"].f64[:1], t["mem"].f64[:1])
    gu.compare("decoder layer ragged 192 x 256 tiles (batch 0)", got[:1], ref, dtype="bf16")


def _stack_run(T, w, t, *, batch, qlen, n_seg, mlen_max, d_inner, n_layer, head0=0):
    D = w.d_model
    dt = T.bfloat16 if w.dtype == "bf16" else T.float32
    rings = [T.zeros((batch, mlen_max, D), dtype=dt, device="cuda") for _ in range(n_layer)]
    fifos = (xl.xl_mem_fifo * n_layer)(*[xl.xl_mem_fifo(r.data_ptr(), mlen_max, 0, head0) for r in rings])
    weights = [gu.dec_weights(lw) for lw in t["layers"]]
    hs = gu.dev(t["h"])
    outs, mems = [], []
    for s in range(n_seg):
        desc = _desc(w, batch=batch, qlen=qlen, mlen=fifos[0].len)
        ws = T.empty(xl.xl_decoder_stack_workspace_size(desc, d_inner), dtype=T.uint8, device="cuda")
        h = hs[:, s * qlen:(s + 1) * qlen].contiguous()
        out = T.empty((batch, qlen, D), dtype=T.float32, device="cuda")
        xl.xl_decoder_stack_step(desc, d_inner, 0.0, weights, h, fifos, out, ws)
        T.cuda.synchronize()
        outs.append(gu.host64(out))
        # each ring in age order (oldest first)
        cur = []
        for n in range(n_layer):
            f = fifos[n]
            idx = [(f.head + i) % mlen_max for i in range(f.len)]
            cur.append(rings[n][:, idx].clone())
        mems.append(cur)
    return outs, mems


# (bias, kind: the scalar bias table, clamped (0) or T5 buckets (1); -1: none)
@pytest.mark.parametrize("base,qlen,n_seg,mlen_max,d_inner,n_layer,head0,bias,kind",
                         [("base_bf16", 64, 4, 96, 256, 3, 0, -1, 0), ("base_bf16", 40, 3, 100, 128, 2, 37, -1, 0),
                          ("tiny_f32", 8, 4, 12, 32, 3, 5, -1, 0), ("base_bf16", 32, 3, 80, 128, 2, 11, 8, 0),
                          ("tiny_f32", 8, 4, 12, 32, 2, 3, 0, 1)])
def test_decoder_stack_run(T, base, qlen, n_seg, mlen_max, d_inner, n_layer, head0, bias, kind):
    w = dataclasses.replace(W[base], segments=n_seg, qlen=qlen, mlen=mlen_max, seed=n_layer * 10 + qlen,
                            bias_clamp=bias, bias_kind=kind)
    t = xl_inputs.decoder_inputs(w, d_inner=d_inner, n_layer=n_layer, batch=2, qlen=qlen)
    outs, mems = _stack_run(T, w, t, batch=2, qlen=qlen, n_seg=n_seg, mlen_max=mlen_max, d_inner=d_inner,
                            n_layer=n_layer, head0=head0)
    routs, rmems = oracle.decoder_stack_run(t["h"].f64, n_seg, qlen, mlen_max,
                                            [gu.oracle_dec_weights(lw) for lw in t["layers"]], n_head=w.n_head,
                                            d_head=w.d_head, clamp_len=w.clamp_len, bias_clamp=w.bias_clamp,
                                            bias_kind=w.bias_kind)
    for s in range(n_seg):
        gu.compare(f"stack segment {s}", outs[s], routs[s], dtype=w.dtype)
        # layer 0 keeps the input stream itself: bit for bit
        if w.dtype == "bf16":
            want = xl_inputs.bf16_bits(rmems[s][0].astype(np.float32))
            assert np.array_equal(gu.bits_u16(mems[s][0]), want), f"layer 0 memory after segment {s}"
        else:
            assert np.array_equal(gu.host64(mems[s][0]), rmems[s][0]), f"layer 0 memory after segment {s}"
        for n in range(1, n_layer):
            gu.compare(f"layer {n} memory after segment {s}", gu.host64(mems[s][n]), rmems[s][n], dtype=w.dtype)


def _stack_run_kv(T, w, t, *, batch, qlen, n_seg, mlen_max, cap, d_inner, n_layer, head0=0):
    D, H, dh = w.d_model, w.n_head, w.d_head
    kr = [T.full((batch, H, cap, dh), float("nan"), dtype=T.bfloat16, device="cuda") for _ in range(n_layer)]
    vr = [T.full((batch, H, dh, cap), float("nan"), dtype=T.bfloat16, device="cuda") for _ in range(n_layer)]
    rings = (xl.xl_kv_fifo * n_layer)(*[xl.xl_kv_fifo(k.data_ptr(), v.data_ptr(), cap, mlen_max, 0, head0)
                                        for k, v in zip(kr, vr)])
    weights = [gu.dec_weights(lw) for lw in t["layers"]]
    hs = gu.dev(t["h"])
    outs = []
    for s in range(n_seg):
        desc = _desc(w, batch=batch, qlen=qlen, mlen=rings[0].len)
        ws = T.empty(xl.xl_decoder_stack_kv_workspace_size(desc, d_inner), dtype=T.uint8, device="cuda")
        h = hs[:, s * qlen:(s + 1) * qlen].contiguous()
        out = T.empty((batch, qlen, D), dtype=T.float32, device="cuda")
        xl.xl_decoder_stack_step_kv(desc, d_inner, 0.0, weights, h, rings, out, ws)
        T.cuda.synchronize()
        outs.append(gu.host64(out))
        for n in range(n_layer):
            assert rings[n].len == min((s + 1) * qlen, mlen_max)
    return outs


# the stack on key rings of projected keys and values: bit for bit the state-FIFO stack's
# outputs (the memory's rows were normalised and projected with the same code when they were the
# segment), and the oracle's; rings start anywhere and wrap
@pytest.mark.parametrize("qlen,n_seg,mlen_max,cap,n_layer,head0,bias,kind",
                         [(64, 4, 96, 160, 3, 0, -1, 0), (40, 3, 80, 128, 2, 56, 8, 0), (32, 4, 64, 104, 2, 24, 0, 1)])
def test_decoder_stack_kv_matches_fifo(T, qlen, n_seg, mlen_max, cap, n_layer, head0, bias, kind):
    d_inner = 256
    w = dataclasses.replace(W["base_bf16"], segments=n_seg, qlen=qlen, mlen=mlen_max, seed=n_layer * 7 + qlen,
                            bias_clamp=bias, bias_kind=kind)
    t = xl_inputs.decoder_inputs(w, d_inner=d_inner, n_layer=n_layer, batch=2, qlen=qlen)
    outs, _ = _stack_run(T, w, t, batch=2, qlen=qlen, n_seg=n_seg, mlen_max=mlen_max, d_inner=d_inner,
                         n_layer=n_layer)
    kouts = _stack_run_kv(T, w, t, batch=2, qlen=qlen, n_seg=n_seg, mlen_max=mlen_max, cap=cap, d_inner=d_inner,
                          n_layer=n_layer, head0=head0)
    routs, _ = oracle.decoder_stack_run(t["h"].f64, n_seg, qlen, mlen_max,
                                        [gu.oracle_dec_weights(lw) for lw in t["layers"]], n_head=w.n_head,
                                        d_head=w.d_head, clamp_len=w.clamp_len, bias_clamp=w.bias_clamp,
                                        bias_kind=w.bias_kind)
    for s in range(n_seg):
        assert np.array_equal(kouts[s], outs[s]), f"segment {s}: key-ring stack differs from the state-FIFO stack"
        gu.compare(f"key-ring stack segment {s}", kouts[s], routs[s], dtype=w.dtype)


def _random_layer(idx):
    # a seeded random bf16 decoder layer: widths in multiples of 32 (half-width last K
    # stages when 32 mod 64), several heads, ragged segment and memory lengths, any FFN
    # width, bias kinds; the GEMM launches land on the 64 x 64 and both 128 x 128 tiles
    rng = np.random.default_rng(5100 + idx)
    n_head = int(rng.integers(1, 5))
    d_model = 32 * int(rng.integers(2, 33))
    d_inner = 32 * int(rng.integers(1, 65))
    batch, qlen = int(rng.integers(1, 4)), int(rng.integers(1, 301))
    mlen = 0 if idx % 4 == 0 else int(rng.integers(1, 401))
    bias = -1 if rng.random() < 0.5 else int(rng.integers(0, 65))
    kind = int(rng.integers(0, 2)) if bias >= 0 else 0
    return n_head, d_model, d_inner, batch, qlen, mlen, bias, kind


@pytest.mark.parametrize("idx", range(8))
def test_decoder_layer_random(T, idx):
    n_head, d_model, d_inner, batch, qlen, mlen, bias, kind = _random_layer(idx)
    print(f"decoder random {idx}: H{n_head} D{d_model} di{d_inner} B{batch} q{qlen} m{mlen} bias {bias} kind {kind}",
          flush=True)
    w = dataclasses.replace(W["base_bf16"], d_model=d_model, n_head=n_head, bias_clamp=bias, bias_kind=kind,
                            seed=700 + idx)
    t = xl_inputs.decoder_inputs(w, d_inner=d_inner, n_layer=1, batch=batch, qlen=qlen, mlen=mlen)
    got = _run_layer(T, w, t, batch=batch, qlen=qlen, mlen=mlen, d_inner=d_inner)
    ref = _oracle_layer(t, w, t["layers"][0], t["h"].f64, t["mem"].f64)
    gu.compare(f"decoder random {idx}", got, ref, dtype="bf16")
