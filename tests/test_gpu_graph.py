"""The layer forward captured in a HIP graph.

xl_rel_attn_fwd issues only kernel launches on the caller's stream (no
allocation, copy, fill or synchronisation), so a caller can capture it. Every
replay must give the bits of the eager call; the replays are separated by
eager work of the program and a synchronisation, and the output buffer is
overwritten before each one, so that a replay that skipped a node or read a
stale argument shows.
"""
import numpy as np
import pytest

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


# large_bf16 at batch 2 (one attention launch), longmem_bf16 at batch 2 (its
# keys split: the attention and the merge kernel)
@pytest.mark.parametrize("name,batch,qlen,mlen", [("large_bf16", 2, 384, 384), ("longmem_bf16", 2, 64, 1600)])
def test_layer_graph_replay(T, name, batch, qlen, mlen):
    import transformer_xl_relative_amd as xl
    w = W[name]
    t = xl_inputs.layer_inputs(w, batch=batch, qlen=qlen, mlen=mlen)
    L = gu.Layer(w, t, batch=batch, qlen=qlen, mlen=mlen, out_f32=True)
    h = gu.dev(t["h"])
    mem = gu.dev(t["mem"])
    print(f"graph replay: {name} batch {batch} qlen {qlen} mlen {mlen}", flush=True)
    xl.xl_rel_attn_fwd(L.desc, L.weights, h, mem, L.out, L.ws)
    T.cuda.synchronize()
    eager = L.out.clone()
    ref = gu.oracle_layer(t, w, t["h"].f64, t["mem"].f64, bsel=[0])
    gu.compare(f"{name} eager", gu.host64(eager)[:1], ref, dtype=w.dtype)

    out = T.empty_like(L.out)
    side = T.cuda.Stream()
    graph = T.cuda.CUDAGraph()
    with T.cuda.graph(graph, stream=side):
        xl.xl_rel_attn_fwd(L.desc, L.weights, h, mem, out, L.ws)
    scratch = T.empty(1 << 20, dtype=T.float32, device="cuda")
    for rep in range(4):
        out.fill_(float("nan"))
        scratch.normal_()                      # eager work between the replays
        _ = scratch.sum().item()
        graph.replay()
        T.cuda.synchronize()
        assert T.equal(out, eager), f"replay {rep}: differs from the eager call"
    # and the eager call after the replays still gives the same bits
    L.out.fill_(float("nan"))
    xl.xl_rel_attn_fwd(L.desc, L.weights, h, mem, L.out, L.ws)
    T.cuda.synchronize()
    assert np.array_equal(gu.host64(L.out), gu.host64(eager))


def test_decoder_layer_graph_replay(T):
    # the pre-LN decoder layer (layer norms, attention, feed-forward network
    # with its residuals) at the large workload's width with a long memory
    # (its keys split), captured and replayed
    import transformer_xl_relative_amd as xl
    w = W["large_bf16"]
    batch, qlen, mlen, d_inner = 2, 64, 1200, 4096
    t = xl_inputs.decoder_inputs(w, d_inner=d_inner, n_layer=1, batch=batch, qlen=qlen, mlen=mlen)
    desc = xl.make_desc(batch=batch, d_model=w.d_model, n_head=w.n_head, d_head=w.d_head, qlen=qlen, mlen=mlen,
                        clamp_len=w.clamp_len, bias_clamp=w.bias_clamp, bias_kind=w.bias_kind, dtype=xl.XL_BF16,
                        out_dtype=xl.XL_F32)
    ws = T.empty(xl.xl_decoder_layer_workspace_size(desc, d_inner), dtype=T.uint8, device="cuda")
    weights = gu.dec_weights(t["layers"][0])
    h = gu.dev(t["h"])
    mem = gu.dev(t["mem"])
    eager = T.empty((batch, qlen, w.d_model), dtype=T.float32, device="cuda")
    print(f"graph replay: decoder layer batch {batch} qlen {qlen} mlen {mlen} d_inner {d_inner}", flush=True)
    xl.xl_decoder_layer_fwd(desc, d_inner, 0.0, weights, h, mem, eager, ws)
    T.cuda.synchronize()
    import oracle
    ref = oracle.decoder_layer_fwd(t["h"].f64[:1], t["mem"].f64[:1], gu.oracle_dec_weights(t["layers"][0]),
                                   n_head=w.n_head, d_head=w.d_head, clamp_len=w.clamp_len,
                                   bias_clamp=w.bias_clamp, bias_kind=w.bias_kind)
    gu.compare("decoder layer eager", gu.host64(eager)[:1], ref, dtype="bf16")

    out = T.empty_like(eager)
    side = T.cuda.Stream()
    graph = T.cuda.CUDAGraph()
    with T.cuda.graph(graph, stream=side):
        xl.xl_decoder_layer_fwd(desc, d_inner, 0.0, weights, h, mem, out, ws)
    scratch = T.empty(1 << 20, dtype=T.float32, device="cuda")
    for rep in range(4):
        out.fill_(float("nan"))
        scratch.normal_()
        _ = scratch.sum().item()
        graph.replay()
        T.cuda.synchronize()
        assert T.equal(out, eager), f"replay {rep}: differs from the eager call"


def test_core_backward_graph_replay(T):
    # the attention-core gradients (every output written by one thread, no
    # atomics) with a bias table, captured and replayed: each replay rewrites
    # every gradient with the eager bits
    import transformer_xl_relative_amd as xl
    B, H, qlen, mlen, dh, bias = 2, 3, 200, 75, 64, 40
    klen = qlen + mlen
    n_rel = klen
    ci = xl_inputs.core_inputs(batch=B, n_head=H, d_head=dh, qlen=qlen, mlen=mlen, n_rows=n_rel, dtype="bf16",
                               seed=11, bias_clamp=bias, bias_kind=0)
    rng = np.random.default_rng(12)
    dout = xl_inputs.Tensor(rng.standard_normal((B, qlen, H * dh)).astype(np.float32), "bf16")
    ldv = (klen + 7) // 8 * 8 + 8
    vt = np.zeros((B, H, dh, ldv), np.float32)
    vt[..., :klen] = ci["v"].f32.transpose(0, 1, 3, 2)
    vt = xl_inputs.Tensor(vt, "bf16")
    desc = xl.make_desc(batch=B, d_model=2, n_head=H, d_head=dh, qlen=qlen, mlen=mlen, clamp_len=-1,
                        bias_clamp=bias, bias_kind=0, dtype=xl.XL_BF16)
    shapes = {"dq": (B, H, qlen, dh), "dk": (B, H, klen, dh), "dv": (B, H, klen, dh), "dr": (H, n_rel, dh),
              "du": (H, dh), "dv_bias": (H, dh), "dbias": tuple(ci["beta"].shape)}
    grads = lambda: {k: T.full(s, float("nan"), dtype=T.float32, device="cuda") for k, s in shapes.items()}
    ops = (gu.dev(ci["q"]), gu.dev(ci["k"]), gu.dev(vt), ldv, gu.dev(ci["r"]), n_rel, gu.dev(ci["u"]),
           gu.dev(ci["vb"]), gu.dev(ci["beta"]), gu.dev(dout))
    ws = T.empty(xl.xl_rel_attn_core_bwd_workspace_size(desc), dtype=T.uint8, device="cuda")
    print(f"graph replay: core backward B {B} H {H} qlen {qlen} mlen {mlen} bias {bias}", flush=True)
    eager = grads()
    xl.xl_rel_attn_core_bwd(desc, *ops, eager, ws)
    T.cuda.synchronize()
    for k, g in eager.items():
        assert bool(T.isfinite(g).all()), k

    out = grads()
    side = T.cuda.Stream()
    graph = T.cuda.CUDAGraph()
    with T.cuda.graph(graph, stream=side):
        xl.xl_rel_attn_core_bwd(desc, *ops, out, ws)
    scratch = T.empty(1 << 20, dtype=T.float32, device="cuda")
    for rep in range(4):
        for g in out.values():
            g.fill_(float("nan"))
        scratch.normal_()
        _ = scratch.sum().item()
        graph.replay()
        T.cuda.synchronize()
        for k in shapes:
            assert T.equal(out[k], eager[k]), f"replay {rep}: {k} differs from the eager call"
