"""The fused attention at the largest key count per head that the library
accepts: klen = (2^31 - 1) // 128 = 16,777,215, so that a head's K rows of
128 bytes stay within 32-bit offsets, and V^T rows of 16,777,224 columns,
whose byte offsets pass 2^31. One batch element and head, 64 queries, the
clamped distance table of the long-memory workload, the library's own key
split (64 workgroups of 8192 steps).

Keys and values come from seeded pools (xl_inputs.long_key_core_inputs)
with one dominant probe key per sampled query row, placed where an offset
error would first show: the first key, both sides of the first key-split
boundary, both sides of 2^23, near 2^24, the last two keys (the last one in
the ragged final tile) and one key just past a row's causal limit, which
must get no weight. The sampled rows are compared with the oracle, which
sums over every key.
"""
import time

import numpy as np
import pytest

import oracle
import xl_inputs
from tests import gpu_util as gu

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
