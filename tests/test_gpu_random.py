"""Randomised-shape parity: seeded draws of shapes and options, each compared
element-wise with the fp64 oracle through the C ABI.

The fixed cases elsewhere pin the known edges; these draws vary everything at
once (batch, heads, qlen down to 1, memory from empty to several key tiles,
clamp, the bias table and its kind, the key-split count; for the key-ring
segment step also the ring capacity and its starting row), so that a tiling,
LDS-slot or ring-offset mistake that only some combination reaches shows up
as a parity failure. The draws are fixed by the seed: every run tests the
same cases, and a failing case is named by its parameters.
"""
import dataclasses

import numpy as np
import pytest

import oracle
import xl_inputs
from tests import gpu_util as gu
from tests.test_gpu_parity import _core_case, _segment_run_kv

pytestmark = pytest.mark.gpu


def _core_draws(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        dtype = "bf16" if rng.random() < 0.8 else "f32"
        B = int(rng.integers(1, 4))
        H = int(rng.integers(1, 5)) if dtype == "bf16" else int(rng.choice([2, 4]))
        qlen = int(rng.choice([1, 7, 31, 32, 33])) if rng.random() < 0.25 else int(rng.integers(1, 330))
        mlen = 0 if rng.random() < 0.2 else int(rng.integers(1, 900))
        klen = qlen + mlen
        clamp = -1 if rng.random() < 0.5 else int(rng.integers(0, klen + 1))
        kind, bias = 0, -1
        u = rng.random()
        if u < 0.2:
            kind, bias = 1, 0
        elif u < 0.5:
            bias = int(rng.integers(0, 200))
        splits = 0
        if dtype == "bf16":
            v = rng.random()
            splits = 1 if v < 0.1 else (int(rng.integers(2, 9)) if v < 0.4 else 0)
        out.append((dtype, B, H, qlen, mlen, clamp, bias, kind, splits))
    return out


CORE_DRAWS = _core_draws(32, 20261202)


@pytest.fixture(scope="module")
def T():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import transformer_xl_relative_amd as xl
    xl.lib()
    return torch


@pytest.mark.parametrize("dtype,B,H,qlen,mlen,clamp,bias,kind,splits", CORE_DRAWS,
                         ids=[f"{c[0]}-B{c[1]}H{c[2]}-q{c[3]}m{c[4]}-c{c[5]}b{c[6]}k{c[7]}-s{c[8]}"
                              for c in CORE_DRAWS])
def test_core_random(T, dtype, B, H, qlen, mlen, clamp, bias, kind, splits):
    _core_case(T, dtype, B, H, qlen, mlen, clamp, bias, splits, bias_kind=kind)


def _ring_draws(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        qlen = 8 * int(rng.integers(1, 25))
        mlen_max = 8 * int(rng.integers(1, 50))
        cap = mlen_max + qlen + 8 * int(rng.integers(0, 20))
        head0 = 8 * int(rng.integers(0, cap // 8))
        n_seg = int(rng.integers(2, 5))
        bias = -1 if rng.random() < 0.5 else int(rng.integers(0, 160))
        clamp = -1 if rng.random() < 0.6 else int(rng.integers(0, mlen_max + qlen))
        out.append((qlen, n_seg, mlen_max, cap, head0, bias, clamp))
    return out


RING_DRAWS = _ring_draws(8, 7)


@pytest.mark.parametrize("qlen,n_seg,mlen_max,cap,head0,bias,clamp", RING_DRAWS,
                         ids=[f"q{c[0]}x{c[1]}-m{c[2]}-cap{c[3]}-h{c[4]}-b{c[5]}-c{c[6]}" for c in RING_DRAWS])
def test_segment_run_kv_ring_random(T, qlen, n_seg, mlen_max, cap, head0, bias, clamp):
    # a narrower layer (d_model 256, 4 heads) keeps the oracle's runs short
    w = dataclasses.replace(xl_inputs.WORKLOADS["segments_bf16"], d_model=256, n_head=4, qlen=qlen, mlen=mlen_max,
                            segments=n_seg, bias_clamp=bias, clamp_len=clamp, seed=qlen + mlen_max + cap)
    t = xl_inputs.layer_inputs(w, batch=1, qlen=qlen)
    outs = _segment_run_kv(T, w, t, batch=1, qlen=qlen, n_seg=n_seg, mlen_max=mlen_max, cap=cap, head0=head0)
    wts = {k: t[k].f64 for k in ("w_q", "w_k", "w_v", "w_r", "w_o", "u", "v", "beta") if k in t}
    routs, _ = oracle.segment_run(t["h"].f64, n_seg, qlen, mlen_max, wts, n_head=w.n_head, d_head=w.d_head,
                                  clamp_len=w.clamp_len, bias_clamp=w.bias_clamp, bias_kind=w.bias_kind)
    for s in range(n_seg):
        gu.compare(f"key ring segment {s}", gu.host64(outs[s]), routs[s], dtype="bf16")
