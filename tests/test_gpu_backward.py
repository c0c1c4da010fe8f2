"""GPU parity of the attention-core gradients (xl_rel_attn_core_bwd) against
the fp64 oracle's, on the same seeded operands, through the C ABI.

Tolerance: the GPU accumulates every gradient in fp32 from the stored input
values (bf16 or fp32); on the bf16 path its products take fp32 operands
(softmax terms, q + u, q + v) as a high and a low bf16 part, about 16 bits of
mantissa, so each product carries a relative error near 2^-16 and the sums
over at most klen (or B*qlen) terms add fp32 rounding: each gradient tensor
must agree elementwise within 1e-3 * |ref| + 1e-3 * max|ref|."""
import numpy as np
import pytest

import oracle
import transformer_xl_relative_amd as xl
import xl_inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
RTOL = 1e-3


@pytest.fixture(scope="module")
def T():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    xl.lib()
    return torch


def _close(name, got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite"
    atol = RTOL * max(float(np.max(np.abs(ref))), 1e-30)
    err = np.abs(got - ref)
    bad = err > atol + RTOL * np.abs(ref)
    assert not bad.any(), f"{name}: max abs err {err.max():.3e} (atol {atol:.3e}), failing {bad.mean() * 100:.3f}%"


def _run(T, dtype, B, H, qlen, mlen, clamp, bias, kind=0, seed=0, extra_rows=0):
    dh = 64 if dtype == "bf16" else 8
    klen = qlen + mlen
    need = klen if clamp < 0 else min(klen, clamp + 1)
    n_rel = need + extra_rows
    ci = xl_inputs.core_inputs(batch=B, n_head=H, d_head=dh, qlen=qlen, mlen=mlen, n_rows=n_rel, dtype=dtype,
                               seed=seed, bias_clamp=bias, bias_kind=kind)
    rng = np.random.default_rng(seed + 1)
    dout = xl_inputs.Tensor(rng.standard_normal((B, qlen, H * dh)).astype(np.float32), dtype)
    ldv = (klen + 7) // 8 * 8 + 8
    vt = np.zeros((B, H, dh, ldv), np.float32)
    vt[..., :klen] = ci["v"].f32.transpose(0, 1, 3, 2)
    vt = xl_inputs.Tensor(vt, dtype)
    desc = xl.make_desc(batch=B, d_model=2, n_head=H, d_head=dh, qlen=qlen, mlen=mlen, clamp_len=clamp,
                        bias_clamp=bias, bias_kind=kind, dtype=xl.XL_BF16 if dtype == "bf16" else xl.XL_F32)
    f32 = lambda *s: T.full(s, float("nan"), dtype=T.float32, device="cuda")
    g = {"dq": f32(B, H, qlen, dh), "dk": f32(B, H, klen, dh), "dv": f32(B, H, klen, dh), "dr": f32(H, n_rel, dh),
         "du": f32(H, dh), "dv_bias": f32(H, dh)}
    if bias >= 0:
        g["dbias"] = f32(*ci["beta"].shape)
    ws = T.empty(xl.xl_rel_attn_core_bwd_workspace_size(desc), dtype=T.uint8, device="cuda")
    xl.xl_rel_attn_core_bwd(desc, gu.dev(ci["q"]), gu.dev(ci["k"]), gu.dev(vt), ldv, gu.dev(ci["r"]), n_rel,
                            gu.dev(ci["u"]), gu.dev(ci["vb"]), gu.dev(ci["beta"]) if bias >= 0 else None,
                            gu.dev(dout), g, ws)
    T.cuda.synchronize()
    ref = oracle.rel_attn_core_bwd(ci["q"].f64, ci["k"].f64, ci["v"].f64, ci["r"].f64, ci["u"].f64, ci["vb"].f64,
                                   dout.f64, scale=1.0 / np.sqrt(dh), clamp_len=clamp,
                                   beta=ci["beta"].f64 if bias >= 0 else None, bias_clamp=bias, bias_kind=kind)
    for key, rkey in [("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dr", "dr"), ("du", "du"), ("dv_bias", "dv_bias")] + \
            ([("dbias", "dbeta")] if bias >= 0 else []):
        _close(key, gu.host64(g[key]), ref[rkey])


BWD = [
    # dtype, B, H, qlen, mlen, clamp, bias, bias kind
    ("bf16", 2, 3, 200, 75, -1, -1, 0),        # several query rows per wave of keys, ragged
    ("bf16", 1, 2, 64, 700, 300, 40, 0),       # clamped distances share the last table row
    ("bf16", 2, 2, 40, 1100, -1, 0, 1),        # T5 buckets past 1024
    ("bf16", 1, 1, 1, 0, -1, -1, 0),           # a single key
    ("f32", 2, 2, 20, 11, 7, -1, 0),
    ("f32", 1, 2, 9, 4, -1, 3, 0),
    ("f32", 2, 2, 11, 40, -1, 0, 1),           # fp32 path with the T5 buckets
    ("bf16", 3, 2, 13, 60, 20, 5, 0),          # query blocks of 8 with a ragged last block
    ("bf16", 1, 1, 70, 1, -1, -1, 0),          # key chunks of 64 with a ragged last chunk
]


@pytest.mark.parametrize("dtype,B,H,qlen,mlen,clamp,bias,kind", BWD,
                         ids=[f"{c[0]}-B{c[1]}H{c[2]}-q{c[3]}m{c[4]}-c{c[5]}b{c[6]}k{c[7]}" for c in BWD])
def test_core_backward(T, dtype, B, H, qlen, mlen, clamp, bias, kind):
    _run(T, dtype, B, H, qlen, mlen, clamp, bias, kind, seed=qlen + mlen + bias)


def test_core_backward_extra_table_rows(T):
    # table rows beyond those any distance uses get a zero gradient
    _run(T, "bf16", 1, 2, 33, 20, 10, -1, seed=5, extra_rows=9)


def test_core_backward_large(T):
    # the large workload's shape (batch 8, 16 heads, qlen = mlen = 384), all gradients
    _run(T, "bf16", 8, 16, 384, 384, -1, -1, seed=11)


def test_core_backward_longmem(T):
    # the long-memory workload's shape: batch 4, 8 heads, qlen 64, 1600 memory keys, clamp 1000 (the
    # last table row takes the 600 clamped distances)
    _run(T, "bf16", 4, 8, 64, 1600, 1000, -1, seed=13)


def test_core_backward_segment_bias(T):
    # a steady-state segment of the segment workload (qlen = mlen = 512) with the +-128 bias table, one
    # batch element of 4
    _run(T, "bf16", 1, 16, 512, 512, -1, 128, seed=17)


def _random_shape(idx):
    # a seeded random bf16 shape: ragged query blocks, any klen mod 4 (the logits kernel's scalar
    # store path), no memory (whole quarters of the first key block see no key), clamp and bias kinds
    rng = np.random.default_rng(4200 + idx)
    B, H = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    qlen = int(rng.integers(1, 261))
    mlen = 0 if idx % 3 == 0 else int(rng.integers(1, 401))
    klen = qlen + mlen
    clamp = -1 if rng.random() < 0.5 else int(rng.integers(1, klen + 1))
    bias = -1 if rng.random() < 0.5 else int(rng.integers(0, 65))
    kind = int(rng.integers(0, 2)) if bias >= 0 else 0
    return B, H, qlen, mlen, clamp, bias, kind


@pytest.mark.parametrize("idx", range(8))
def test_core_backward_random(T, idx):
    B, H, qlen, mlen, clamp, bias, kind = _random_shape(idx)
    print(f"backward random {idx}: B{B} H{H} q{qlen} m{mlen} clamp {clamp} bias {bias} kind {kind}", flush=True)
    _run(T, "bf16", B, H, qlen, mlen, clamp, bias, kind, seed=900 + idx)
