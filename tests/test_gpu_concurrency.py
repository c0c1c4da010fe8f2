"""The library under concurrent use: it keeps no global state between calls
(caller-owned workspaces and FIFOs, a thread-local error string, launch
attributes set once), so independent calls on different streams, or from
different host threads, must give exactly the results they give alone.

* two layer forwards with different inputs, their launches interleaved on two
  streams, against each run alone on one stream (bit for bit);
* two host threads, each running a segment-recurrent run on its own stream
  with its own FIFO and workspace, against the same runs done one after the
  other (bit for bit).
"""
import threading

import pytest

import xl_inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def T():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import transformer_xl_relative_amd as xl
    xl.lib()
    return torch


def _layer(T, w, seed):
    t = xl_inputs.layer_inputs(w, seed=seed)
    L = gu.Layer(w, t, batch=w.batch, qlen=w.qlen, mlen=w.mlen)
    return L, gu.dev(t["h"]), gu.dev(t["mem"])


def test_two_streams_interleaved(T):
    import dataclasses
    import transformer_xl_relative_amd as xl
    w = dataclasses.replace(xl_inputs.WORKLOADS["base_bf16"], batch=8)
    runs = [_layer(T, w, seed) for seed in (3, 4)]
    alone = []
    for L, h, mem in runs:
        xl.xl_rel_attn_fwd(L.desc, L.weights, h, mem, L.out, L.ws)
        T.cuda.synchronize()
        alone.append(L.out.clone())
        L.out.fill_(float("nan"))
    streams = [T.cuda.Stream(), T.cuda.Stream()]
    for st in streams:
        st.wait_stream(T.cuda.current_stream())   # the inputs' uploads
    for _ in range(3):   # several rounds of launches alternating between the streams
        for (L, h, mem), st in zip(runs, streams):
            xl.xl_rel_attn_fwd(L.desc, L.weights, h, mem, L.out, L.ws, stream=st)
    T.cuda.synchronize()
    for k, (L, _, _) in enumerate(runs):
        assert T.equal(L.out, alone[k]), f"run {k} differs when interleaved with the other stream"


def _segment_run(T, w, t, stream, n_seg, out_list, err):
    import transformer_xl_relative_amd as xl
    try:
        B, q, D = w.batch, w.qlen, w.d_model
        L = gu.Layer(w, t, batch=B, qlen=q, mlen=w.mlen)
        ring = T.zeros((B, w.mlen, D), dtype=T.bfloat16, device="cuda")
        fifo = xl.xl_mem_fifo(ring.data_ptr(), w.mlen, 0, 0)
        hs = gu.dev(t["h"])
        stream.wait_stream(T.cuda.current_stream())   # the uploads of this thread's inputs
        with T.cuda.stream(stream):
            for s in range(n_seg):
                h = hs[:, s * q:(s + 1) * q].contiguous()
                out = T.empty((B, q, D), dtype=T.float32, device="cuda")
                desc = xl.make_desc(batch=B, d_model=D, n_head=w.n_head, d_head=w.d_head, qlen=q, mlen=0,
                                    clamp_len=w.clamp_len, bias_clamp=w.bias_clamp, bias_kind=w.bias_kind,
                                    dtype=xl.XL_BF16, out_dtype=xl.XL_F32)
                xl.xl_segment_step(desc, L.weights, h, fifo, out, L.ws, stream=stream)
                out_list.append(out)
        stream.synchronize()
        out_list[:] = [o.cpu() for o in out_list] + [ring.view(T.int16).cpu()]
    except Exception as e:   # reported by the main thread
        err.append(e)


def test_two_threads_segment_runs(T):
    import dataclasses
    w = dataclasses.replace(xl_inputs.WORKLOADS["segments_bf16"], batch=2, qlen=128, mlen=256, segments=4)
    inputs = [xl_inputs.layer_inputs(w, seed=seed) for seed in (5, 6)]
    seq = []
    for t in inputs:
        res, err = [], []
        _segment_run(T, w, t, T.cuda.Stream(), 4, res, err)
        assert not err, err
        seq.append(res)
    results, errors = [[], []], []
    threads = [threading.Thread(target=_segment_run, args=(T, w, inputs[k], T.cuda.Stream(), 4, results[k], errors))
               for k in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a thread did not finish"
    assert not errors, errors
    for k in range(2):
        assert len(results[k]) == len(seq[k])
        for a, b in zip(results[k], seq[k]):
            assert T.equal(a, b), f"thread {k}: results differ from the sequential run"
