"""The allocation-free segment step (xl_segment_step_noalloc) against the
workspace-taking xl_segment_step, through the C ABI: the same inputs and
memory give the same output and the same memory, bit for bit, on two calls
in a row (the second smaller, so it runs on the first's leftover scratch),
and the first also matches the fp64 oracle."""
import dataclasses

import numpy as np
import pytest

import xl_inputs
from tests import gpu_util as gu
from tests import guards

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


def _pair(T, w, t, batch, qlen, mlen, head):
    """Run both entry points on identical copies of a full memory ring; return
    (out, ring) of the workspace step, then of the allocation-free step."""
    import transformer_xl_relative_amd as xl
    D = w.d_model
    L = gu.Layer(w, t, batch=batch, qlen=qlen, mlen=mlen)
    mem = gu.dev(t["mem"])
    ring0 = T.empty((batch, mlen, D), dtype=T.bfloat16, device="cuda")
    ring0[:, head:] = mem[:, :mlen - head]      # logical row i at ring row (head + i) % mlen
    ring0[:, :head] = mem[:, mlen - head:]
    h = gu.dev(t["h"])
    res = []
    for noalloc in (False, True):
        ring = ring0.clone()
        fifo = xl.xl_mem_fifo(ring.data_ptr(), mlen, mlen, head)
        desc = xl.make_desc(batch=batch, d_model=D, n_head=w.n_head, d_head=w.d_head, qlen=qlen, mlen=0,
                            clamp_len=w.clamp_len, bias_clamp=w.bias_clamp, bias_kind=w.bias_kind,
                            dtype=xl.XL_BF16, out_dtype=xl.XL_F32)
        out = T.full((batch, qlen, D), float("nan"), dtype=T.float32, device="cuda")
        if noalloc:
            xl.xl_segment_step_noalloc(desc, L.weights, h, fifo, out)
        else:
            xl.xl_segment_step(desc, L.weights, h, fifo, out, L.ws)
        T.cuda.synchronize()
        assert (fifo.len, fifo.head) == (mlen, (head + qlen) % mlen)
        res.append((gu.host64(out), gu.bits_u16(ring)))
    return res


def test_noalloc_matches_segment_step_twice(T):
    # first call: the large workload's shape at batch 2 (41 MB of scratch at
    # batch 8; here about 10 MB); second call: smaller, with a clamp and a
    # bias table, reusing the scratch the first one left behind
    cases = [
        (dataclasses.replace(W["large_bf16"], seed=301), 2, 384, 384, 40),
        (dataclasses.replace(W["base_bf16"], clamp_len=50, bias_clamp=16, seed=302), 1, 72, 136, 8),
    ]
    for i, (w, batch, qlen, mlen, head) in enumerate(cases):
        t = xl_inputs.layer_inputs(w, batch=batch, qlen=qlen, mlen=mlen, recipe="sensitive")
        (o_ws, r_ws), (o_na, r_na) = _pair(T, w, t, batch, qlen, mlen, head)
        assert np.array_equal(o_na, o_ws), f"call {i}: outputs differ"
        assert np.array_equal(r_na, r_ws), f"call {i}: memories differ"
        if i == 0:
            gu.compare("noalloc vs oracle", o_na, guards.oracle_layer(w, t), dtype="bf16")


def test_noalloc_rejects_oversize(T):
    import transformer_xl_relative_amd as xl
    w = W["large_bf16"]
    t = xl_inputs.layer_inputs(w, batch=1, qlen=8, mlen=8)
    L = gu.Layer(w, t, batch=1, qlen=8, mlen=8)
    desc = xl.make_desc(batch=64, d_model=1024, n_head=16, d_head=64, qlen=1024, mlen=0, dtype=xl.XL_BF16)
    ring = T.empty((64, 1024, 1024), dtype=T.bfloat16, device="cuda")
    fifo = xl.xl_mem_fifo(ring.data_ptr(), 1024, 1024, 0)
    h = T.empty((64, 1024, 1024), dtype=T.bfloat16, device="cuda")
    out = T.empty((64, 1024, 1024), dtype=T.float32, device="cuda")
    with pytest.raises(xl.XLError) as ei:
        xl.xl_segment_step_noalloc(desc, L.weights, h, fifo, out)
    assert ei.value.status == xl.XL_WORKSPACE_TOO_SMALL
    assert (fifo.len, fifo.head) == (1024, 0)
