"""The long-key-range input recipe (xl_inputs.long_key_core_inputs) that the
maximum-size GPU test relies on, checked on the CPU at 2^14 keys with the
oracle: each probed query row takes almost all of its output from its probe's
value, the probe past a row's causal limit gets none, and moving one probe
key (what a wrong address would read instead) changes that row's output by
far more than the bf16 tolerance, so the sampled comparison can see it."""
import numpy as np

import oracle
import xl_inputs
from tests.guards import tolerance

QLEN, KLEN = 64, 1 << 14
MLEN = KLEN - QLEN
PROBES = {0: 0, 1: 4095, 2: 4096, 5: MLEN + 6, 31: (1 << 13) - 1, 32: 1 << 13, 62: KLEN - 2, 63: KLEN - 1}
ROWS = sorted(PROBES)


def _core(ci):
    return oracle.rel_attn_core(ci["q"].f64[:, :, ROWS], ci["k"], ci["v"], ci["r"].f64, ci["u"].f64, ci["vb"].f64,
                                scale=0.125, clamp_len=1000, qpos=[MLEN + i for i in ROWS])[0]


def test_probes_dominate_their_rows():
    ci = xl_inputs.long_key_core_inputs(qlen=QLEN, mlen=MLEN, n_rows=1001, seed=23, probes=PROBES)
    o = _core(ci)
    for n, i in enumerate(ROWS):
        pv = ci["v"][0, 0, PROBES[i]]
        share = float(o[n] @ pv / (pv @ pv))
        if i == 5:   # the probe sits one key past this row's last visible key
            assert abs(share) < 0.2, (i, share)
        else:
            assert share > 0.9, (i, share)


def test_moved_probe_is_visible():
    ci = xl_inputs.long_key_core_inputs(qlen=QLEN, mlen=MLEN, n_rows=1001, seed=23, probes=PROBES)
    ref = _core(ci)
    rtol, atol = tolerance(ref, "bf16")
    for i in (2, 63):
        j = PROBES[i]
        k_saved = ci["k"][0, 0, j].copy()
        ci["k"][0, 0, j] = ci["k"][0, 0, j - 1]      # the key a one-row address slip would read
        got = _core(ci)
        ci["k"][0, 0, j] = k_saved
        n = ROWS.index(i)
        err = np.abs(got[n] - ref[n])
        assert (err > atol + rtol * np.abs(ref[n])).mean() > 0.5, i
