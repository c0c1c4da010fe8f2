"""The path at the largest key count per head that the library accepts:
klen = (2^31 - 1) // 128 = 16,777,215, so that a head's K rows of 128 bytes
stay within 32-bit offsets.

The fused attention alone, with V^T rows of 16,777,224 columns, whose byte
offsets pass 2^31: one batch element and head, 64 queries, the clamped
distance table of the long-memory workload, the library's own key split (64
workgroups of 8192 steps).

Keys and values come from seeded pools (xl_inputs.long_key_core_inputs)
with one dominant probe key per sampled query row, placed where an offset
error would first show: the first key, both sides of the first key-split
boundary, both sides of 2^23, near 2^24, the last two keys (the last one in
the ragged final tile) and one key just past a row's causal limit, which
must get no weight. The sampled rows are compared with the oracle, which
sums over every key.

One key-ring segment step on a full ring of the largest capacity under that
limit (16,777,208 slots, a multiple of 8), starting mid-buffer and wrapping:
the memory keys and values are the probe construction above, the layer's
query and output projections the identity (d_model 64, one head), so the
sampled outputs are the probed attention rows, checked against the oracle
over every key; and the segment's projected keys and values land in the
ring at the wrapped rows.

The fused attention with a bias table at the longest context that the
kernel's LDS copy of the table allows (20,096 keys), for both kinds of
table, element-wise against the oracle.

The layer at the widest shapes accepted: d_model 65,536 with one head
(projections with a K of 65,536, an output projection of 65,536 columns,
32,768 sinusoid frequencies) and 1,024 heads (n_head * d_head = 65,536) at
d_model 64, under the sensitive recipe, element-wise against the oracle.

One segment step on a full FIFO of that many memory rows (d_model 32: one
head, projections with a K of 32), whose ring starts mid-buffer and wraps:
the projected keys and values at the rows where an offset error would first
show against the oracle's projection of those rows, the FIFO update bit for
bit, and a finite output.
"""
import time

import numpy as np
import pytest

import oracle
import xl_inputs
from tests import gpu_util as gu
from tests.test_gpu_parity import W, _core_case, _run_layer

pytestmark = pytest.mark.gpu

KLEN = (2 ** 31 - 1) // 128
QLEN = 64
MLEN = KLEN - QLEN
CLAMP = 1000
PROBES = {0: 0, 1: 262143, 2: 262144, 5: MLEN + 6, 31: 2 ** 23 - 1, 32: 2 ** 23, 33: 2 ** 24 - 1024,
          62: KLEN - 2, 63: KLEN - 1}


@pytest.fixture(scope="module")
def T():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import transformer_xl_relative_amd as xl
    xl.lib()
    return torch


@pytest.mark.timeout(600)
def test_core_max_key_count(T):
    import transformer_xl_relative_amd as xl
    t0 = time.time()
    ci = xl_inputs.long_key_core_inputs(qlen=QLEN, mlen=MLEN, n_rows=CLAMP + 1, seed=23, probes=PROBES)
    ldv = (KLEN + 7) // 8 * 8 + 8
    vt = np.zeros((64, ldv), np.uint16)
    vt[:, :KLEN] = ci["v_bits"].T
    print(f"\n  inputs drawn in {time.time() - t0:.1f} s", flush=True)
    up = lambda bits: T.from_numpy(bits.view(np.int16)).cuda().view(T.bfloat16)
    k = up(ci["k_bits"])
    vtd = up(vt)
    del vt
    desc = xl.make_desc(batch=1, d_model=2, n_head=1, d_head=64, qlen=QLEN, mlen=MLEN, clamp_len=CLAMP,
                        dtype=xl.XL_BF16)
    attn = T.empty((1, QLEN, 64), dtype=T.bfloat16, device="cuda")
    nws = xl.xl_rel_attn_core_workspace_size(desc)
    assert nws > 0   # the library splits the keys
    ws = T.empty(nws, dtype=T.uint8, device="cuda")
    xl.xl_rel_attn_core(desc, gu.dev(ci["q"]), k, vtd, ldv, gu.dev(ci["r"]), CLAMP + 1, gu.dev(ci["u"]),
                        gu.dev(ci["vb"]), None, attn, ws)
    T.cuda.synchronize()
    print(f"  GPU done at {time.time() - t0:.1f} s", flush=True)
    rows = sorted(PROBES)
    got = gu.host64(attn)[:, rows]
    ref = oracle.rel_attn_core(ci["q"].f64[:, :, rows], ci["k"], ci["v"], ci["r"].f64, ci["u"].f64, ci["vb"].f64,
                               scale=0.125, clamp_len=CLAMP, qpos=[MLEN + i for i in rows])
    print(f"  oracle done at {time.time() - t0:.1f} s", flush=True)
    gu.compare("max key count, sampled rows", got, ref, dtype="bf16")


@pytest.mark.timeout(600)
def test_segment_step_max_memory(T):
    import transformer_xl_relative_amd as xl
    D = 32
    t0 = time.time()
    li = xl_inputs.long_memory_layer_inputs(d_model=D, n_head=1, qlen=QLEN, mlen=MLEN, seed=29)
    head0 = 1_000_003
    ring_np = np.roll(li["mem_bits"], head0, axis=1)   # logical row j at physical row (head0 + j) % MLEN
    ring = T.from_numpy(ring_np.view(np.int16)).cuda().view(T.bfloat16)
    del ring_np
    print(f"\n  inputs drawn in {time.time() - t0:.1f} s", flush=True)
    fifo = xl.xl_mem_fifo(ring.data_ptr(), MLEN, MLEN, head0)
    desc = xl.make_desc(batch=1, d_model=D, n_head=1, d_head=64, qlen=QLEN, mlen=MLEN, clamp_len=CLAMP,
                        dtype=xl.XL_BF16, out_dtype=xl.XL_F32)
    ws = T.empty(xl.xl_rel_attn_workspace_size(desc), dtype=T.uint8, device="cuda")
    lay = xl.xl_rel_attn_workspace_layout(desc)
    w = xl.Weights(*(gu.dev(li[k]) for k in ("w_q", "w_k", "w_v", "w_r", "w_o", "u", "v")), bias_table=None)
    out = T.empty((1, QLEN, D), dtype=T.float32, device="cuda")
    xl.xl_segment_step(desc, w, gu.dev(li["h"]), fifo, out, ws)
    T.cuda.synchronize()
    print(f"  GPU done at {time.time() - t0:.1f} s", flush=True)
    assert (fifo.len, fifo.head) == (MLEN, (head0 + QLEN) % MLEN)
    assert bool(T.isfinite(out).all())
    # keys and values as projected, at the rows where an offset error would first show
    rows = [0, 1, 2 ** 23 - 1, 2 ** 23, MLEN - 1, MLEN, KLEN - 1]
    x = np.stack([li["mem_pool"].f64[li["mem_idx"][j]] if j < MLEN else li["h"].f64[0, j - MLEN] for j in rows])
    kview = ws[lay.k:lay.k + KLEN * 64 * 2].view(T.bfloat16).view(KLEN, 64)
    vview = ws[lay.vt:lay.vt + 64 * lay.ldv * 2].view(T.bfloat16).view(64, lay.ldv)
    gu.compare("max memory: projected keys", gu.host64(kview[rows]), oracle.linear(x, li["w_k"].f64), dtype="bf16")
    gu.compare("max memory: projected values", gu.host64(vview[:, rows].T), oracle.linear(x, li["w_v"].f64),
               dtype="bf16")
    # the FIFO: the segment's rows replaced the oldest QLEN rows, bit for bit; the others stay
    h_bits = li["h"].bits[0]
    new = [(head0 + t) % MLEN for t in range(QLEN)]
    assert np.array_equal(gu.bits_u16(ring[0, new]), h_bits)
    kept = [QLEN, QLEN + 2 ** 23, MLEN - 1]
    got_kept = gu.bits_u16(ring[0, [(head0 + j) % MLEN for j in kept]])
    assert np.array_equal(got_kept, li["mem_bits"][0, kept])


@pytest.mark.timeout(600)
def test_segment_step_kv_max_ring(T):
    import transformer_xl_relative_amd as xl
    cap = KLEN // 8 * 8
    mem = cap - QLEN                 # the memory is full: len = mlen_max
    head0 = 1_000_008
    probes = {0: 0, 1: 262143, 2: 262144, 31: 2 ** 23 - 1, 32: 2 ** 23, 33: mem - 1024, 63: mem - 1}
    t0 = time.time()
    ci = xl_inputs.long_key_core_inputs(qlen=QLEN, mlen=mem, n_rows=2, seed=31, probes=probes)
    wt = xl_inputs.identity_head_weights(seed=37)
    nan = np.full((QLEN, 64), 0x7FC0, np.uint16)          # ring slots the step writes before reading
    kr = np.roll(np.concatenate([ci["k_bits"][:mem], nan]), head0, axis=0)
    vr = np.roll(np.concatenate([ci["v_bits"][:mem], nan]).T, head0, axis=1)
    up = lambda bits: T.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(T.bfloat16)
    kr_d, vr_d = up(kr), up(vr)
    del kr, vr
    print(f"\n  inputs drawn in {time.time() - t0:.1f} s", flush=True)
    kv = xl.xl_kv_fifo(kr_d.data_ptr(), vr_d.data_ptr(), cap, mem, mem, head0)
    desc = xl.make_desc(batch=1, d_model=64, n_head=1, d_head=64, qlen=QLEN, mlen=0, clamp_len=CLAMP,
                        dtype=xl.XL_BF16, out_dtype=xl.XL_F32)
    dd = xl.make_desc(batch=1, d_model=64, n_head=1, d_head=64, qlen=QLEN, mlen=mem, clamp_len=CLAMP,
                      dtype=xl.XL_BF16, out_dtype=xl.XL_F32)
    ws = T.empty(xl.xl_segment_step_kv_workspace_size(dd), dtype=T.uint8, device="cuda")
    w = xl.Weights(*(gu.dev(x) for x in (wt["w_q"], wt["w_k"], wt["w_v"], wt["w_r"], wt["w_o"], ci["u"], ci["vb"])),
                   bias_table=None)
    h = gu.dev(ci["q"]).view(1, QLEN, 64)
    out = T.empty((1, QLEN, 64), dtype=T.float32, device="cuda")
    xl.xl_segment_step_kv(desc, w, h, kv, out, ws)
    T.cuda.synchronize()
    print(f"  GPU done at {time.time() - t0:.1f} s", flush=True)
    assert (kv.len, kv.head) == (mem, (head0 + QLEN) % cap)
    # the segment's keys and values, projected into the ring at the wrapped rows
    h64 = ci["q"].f64[0, 0]
    k_seg, v_seg = oracle.linear(h64, wt["w_k"].f64), oracle.linear(h64, wt["w_v"].f64)
    slots = [(head0 + mem + t) % cap for t in range(QLEN)]
    gu.compare("max ring: segment keys", gu.host64(kr_d[slots]), k_seg, dtype="bf16")
    gu.compare("max ring: segment values", gu.host64(vr_d[:, slots].T), v_seg, dtype="bf16")
    # the probed rows of the output against the oracle over every key
    k_all, v_all = ci["k"], ci["v"]
    k_all[0, 0, mem:] = k_seg
    v_all[0, 0, mem:] = v_seg
    n_rel = CLAMP + 1
    r_tab = oracle.linear(oracle.relpos_embed(0, n_rel, 64, CLAMP), wt["w_r"].f64)[None]
    rows = sorted(probes)
    ref = oracle.rel_attn_core(h64[None, None, rows], k_all, v_all, r_tab, ci["u"].f64, ci["vb"].f64, scale=0.125,
                               clamp_len=CLAMP, qpos=[mem + i for i in rows])
    print(f"  oracle done at {time.time() - t0:.1f} s", flush=True)
    gu.compare("max ring: probed rows", gu.host64(out)[:, rows], ref, dtype="bf16")


# (80 KB of tiles and rings plus 4 bytes per table entry, mlen + qlen + 384
# entries, within the 160 KB of LDS)
BIAS_KLEN_MAX = 80 * 1024 // 4 - 384


# qlen 1 and 129 leave a last query tile of one query, where the table (which
# covers the tile's 128 rows) fills the LDS exactly
@pytest.mark.parametrize("qlen,bias_kind,bias", [(1, 0, 128), (64, 1, 0), (129, 0, 16)])
def test_core_bias_table_max_context(T, qlen, bias_kind, bias):
    _core_case(T, "bf16", 1, 2, qlen, BIAS_KLEN_MAX - qlen, -1, bias, 0, bias_kind=bias_kind)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("d_model,n_head", [(65536, 1), (64, 1024)])
def test_layer_max_width(T, d_model, n_head):
    import dataclasses
    w = dataclasses.replace(W["base_bf16"], d_model=d_model, n_head=n_head, seed=41)
    t = xl_inputs.layer_inputs(w, batch=1, qlen=QLEN, mlen=QLEN, recipe="sensitive")
    L = _run_layer(T, w, t, batch=1, qlen=QLEN, mlen=QLEN)
    ref = gu.oracle_layer(t, w, t["h"].f64, t["mem"].f64)
    gu.compare(f"d_model {d_model}, {n_head} heads", gu.host64(L.out), ref, dtype="bf16")
