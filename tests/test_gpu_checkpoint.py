"""Checkpoint and resume of a segment-recurrent run across processes.

The segmented workload (batch 4, d_model 1024, 16 heads, qlen = mlen = 512,
the +-128 bias table, 4 segments) runs once without interruption in this
process, and once split over two child processes: the first runs segments 0
and 1 from an empty memory and saves the memory (transformer_xl_relative_amd.
checkpoint); the second loads it and runs segments 2 and 3. Every kernel of a
segment step is deterministic, so the resumed outputs and the final memory
must equal the uninterrupted run's bit for bit. Both memory forms are
covered: the FIFO of layer input states and the key ring of projected keys
and values; and a 2-layer decoder stack on key rings (base_bf16 widths,
qlen 64, 128 memory keys, d_inner 256), one checkpoint file per layer.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import xl_inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEAD0 = 200          # first physical row of the memory: the run wraps the ring
CAP_EXTRA = 64       # key-ring rows beyond mlen + qlen


def _segments(kind, first, last, ckpt_in=None, ckpt_out=None):
    """Run segments first..last-1 on the GPU; returns their outputs (fp32, host) and the final state."""
    import torch
    import transformer_xl_relative_amd as xl
    from transformer_xl_relative_amd import checkpoint
    w = xl_inputs.WORKLOADS["segments_bf16"]
    t = xl_inputs.layer_inputs(w)
    B, q, D, H, dh = w.batch, w.qlen, w.d_model, w.n_head, w.d_head
    L = gu.Layer(w, t, batch=B, qlen=q, mlen=w.mlen)
    hs = gu.dev(t["h"])
    if kind == "state":
        if ckpt_in:
            ring, fifo = checkpoint.load_fifo(ckpt_in)
        else:
            ring = torch.zeros((B, w.mlen, D), dtype=torch.bfloat16, device="cuda")
            fifo = xl.xl_mem_fifo(ring.data_ptr(), w.mlen, 0, HEAD0)
        ws = L.ws
    else:
        cap = w.mlen + q + CAP_EXTRA
        if ckpt_in:
            kr, vr, fifo = checkpoint.load_kv_fifo(ckpt_in)
        else:
            kr = torch.full((B, H, cap, dh), float("nan"), dtype=torch.bfloat16, device="cuda")
            vr = torch.full((B, H, dh, cap), float("nan"), dtype=torch.bfloat16, device="cuda")
            fifo = xl.xl_kv_fifo(kr.data_ptr(), vr.data_ptr(), cap, w.mlen, 0, HEAD0)
        ws = torch.empty(xl.xl_segment_step_kv_workspace_size(L.desc), dtype=torch.uint8, device="cuda")
    outs = []
    for s in range(first, last):
        h = hs[:, s * q:(s + 1) * q].contiguous()
        out = torch.empty((B, q, D), dtype=torch.float32, device="cuda")
        desc = xl.make_desc(batch=B, d_model=D, n_head=H, d_head=dh, qlen=q, mlen=0, clamp_len=w.clamp_len,
                            bias_clamp=w.bias_clamp, bias_kind=w.bias_kind, dtype=xl.XL_BF16, out_dtype=xl.XL_F32)
        if kind == "state":
            xl.xl_segment_step(desc, L.weights, h, fifo, out, ws)
        else:
            xl.xl_segment_step_kv(desc, L.weights, h, fifo, out, ws)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    if ckpt_out:
        if kind == "state":
            checkpoint.save_fifo(ckpt_out, fifo, ring)
        else:
            checkpoint.save_kv_fifo(ckpt_out, fifo, kr, vr)
    state = [fifo.len, fifo.head]
    if kind == "state":
        mem = ring.view(torch.uint16).cpu().numpy()
    else:
        mem = np.concatenate([kr.view(torch.uint16).cpu().numpy().reshape(-1),
                              vr.view(torch.uint16).cpu().numpy().reshape(-1)])
    return outs, state, mem


def _stack_segments(first, last, ckpt_in=None, ckpt_out=None):
    """The same for a 2-layer decoder stack on key rings (xl_decoder_stack_step_kv): each layer's
    ring is checkpointed in a file of its own."""
    import dataclasses
    import torch
    import transformer_xl_relative_amd as xl
    from transformer_xl_relative_amd import checkpoint
    NL, DI, B, q = 2, 256, 2, 64
    w = dataclasses.replace(xl_inputs.WORKLOADS["base_bf16"], segments=4, qlen=q, mlen=128, seed=77)
    t = xl_inputs.decoder_inputs(w, d_inner=DI, n_layer=NL, batch=B, qlen=q)
    D, H, dh = w.d_model, w.n_head, w.d_head
    cap = w.mlen + q + CAP_EXTRA
    if ckpt_in:
        rings = [checkpoint.load_kv_fifo(f"{ckpt_in}.{n}.npz") for n in range(NL)]
    else:
        rings = []
        for _ in range(NL):
            kr = torch.full((B, H, cap, dh), float("nan"), dtype=torch.bfloat16, device="cuda")
            vr = torch.full((B, H, dh, cap), float("nan"), dtype=torch.bfloat16, device="cuda")
            rings.append((kr, vr, xl.xl_kv_fifo(kr.data_ptr(), vr.data_ptr(), cap, w.mlen, 0, HEAD0)))
    # the ctypes array holds the rings' state from here on (the library updates it in place)
    kvs = (xl.xl_kv_fifo * NL)(*[f for _, _, f in rings])
    weights = [gu.dec_weights(lw) for lw in t["layers"]]
    hs = gu.dev(t["h"])
    outs = []
    for s in range(first, last):
        h = hs[:, s * q:(s + 1) * q].contiguous()
        out = torch.empty((B, q, D), dtype=torch.float32, device="cuda")
        desc = xl.make_desc(batch=B, d_model=D, n_head=H, d_head=dh, qlen=q, mlen=kvs[0].len,
                            clamp_len=w.clamp_len, bias_clamp=w.bias_clamp, bias_kind=w.bias_kind,
                            dtype=xl.XL_BF16, out_dtype=xl.XL_F32)
        ws = torch.empty(xl.xl_decoder_stack_kv_workspace_size(desc, DI), dtype=torch.uint8, device="cuda")
        xl.xl_decoder_stack_step_kv(desc, DI, 0.0, weights, h, kvs, out, ws)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    if ckpt_out:
        for n, (kr, vr, _) in enumerate(rings):
            checkpoint.save_kv_fifo(f"{ckpt_out}.{n}.npz", kvs[n], kr, vr)
    state = [x for n in range(NL) for x in (kvs[n].len, kvs[n].head)]
    mem = np.concatenate([a.view(torch.uint16).cpu().numpy().reshape(-1) for kr, vr, _ in rings for a in (kr, vr)])
    return outs, state, mem


def _child(kind, first, last, ckpt_in, ckpt_out, result):
    """Entry point of a child process: runs the segments and stores what the parent compares."""
    run = _stack_segments if kind == "stack_keys" else lambda *a: _segments(kind, *a)
    outs, state, mem = run(first, last, ckpt_in or None, ckpt_out or None)
    np.savez(result, outs=np.stack(outs), state=np.array(state, np.int64), mem=mem)


def _spawn(kind, first, last, ckpt_in, ckpt_out, result):
    code = ("import sys; sys.path.insert(0, '.'); from tests import test_gpu_checkpoint as m; "
            f"m._child({kind!r}, {first}, {last}, {ckpt_in!r}, {ckpt_out!r}, {result!r})")
    print(f"child: {kind} segments {first}..{last - 1}", flush=True)
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]


@pytest.fixture(scope="module")
def T():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import transformer_xl_relative_amd as xl
    xl.lib()
    return torch


@pytest.mark.parametrize("kind", ["state", "keys", "stack_keys"])
def test_resume_in_another_process(T, kind, tmp_path):
    ref_outs, ref_state, ref_mem = _stack_segments(0, 4) if kind == "stack_keys" else _segments(kind, 0, 4)
    ckpt = str(tmp_path / f"{kind}_after_2.npz")
    _spawn(kind, 0, 2, "", ckpt, str(tmp_path / "a.npz"))
    _spawn(kind, 2, 4, ckpt, "", str(tmp_path / "b.npz"))
    with np.load(tmp_path / "a.npz", allow_pickle=False) as a, np.load(tmp_path / "b.npz", allow_pickle=False) as b:
        for s in range(2):
            assert np.array_equal(a["outs"][s], ref_outs[s]), f"segment {s} differs before the checkpoint"
            assert np.array_equal(b["outs"][s], ref_outs[2 + s]), f"segment {2 + s} differs after the resume"
        assert list(b["state"]) == ref_state
        assert np.array_equal(b["mem"], ref_mem), "memory after the resumed run differs"
