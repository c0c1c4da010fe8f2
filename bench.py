"""Benchmark of the Transformer-XL relative attention hot path on one MI355X.

One step = one xl_segment_step of the large-like workload (batch 8, d_model
1024, 16 heads of 64, qlen = mlen = 384, causal over [memory ; segment]): the
sinusoid rows, the R/Q/K/V projections, the fused relative attention, the
output projection and the FIFO memory update, on synthetic seeded inputs that
are resident in HBM before the timed region starts. The memory FIFO is full,
so every step attends over 384 memory rows + 384 segment rows.

Prints one JSON line. value is the metric: the fused relative attention's
algorithmic TFLOP/s (6 d_head flops per visible query-key pair) over that
kernel's own time, from HIP events that the runtime timestamps at the
kernel's start and end, over K further steps so that the events do not
perturb the timed ones (the merge of key splits is inside the bracket when
the keys are split). ms_per_step is the whole step's time over the K timed
steps, and layer_tflops the layer's algorithmic rate over it. The roofline
object is the fused attention's against the bf16 MFMA peak (the metric's
denominator), with its HBM rate and fraction beside it; cpu_baseline is the
oracle's attention core on a bounded sample of the same workload (the same
flop count), cpu_baseline_layer the oracle's whole layer.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
                  [--copy-calib-mib M]        # also run a plain device copy of M MiB (counter calibration)
  python bench.py --core base_bf16,large_bf16,...  [--launches N]
                  # the fused attention alone (xl_rel_attn_core) per workload, warm and
                  # cold (1 GiB written between launches to evict the caches): one JSON
                  # line per workload with the median, p10 and p90 kernel times; NAME/tpN
                  # is one GPU's share (n_head / N heads) under head sharding, NAME@mM the
                  # workload with M memory rows
  python bench.py --summarize DIR [--copy-calib-mib M]   # markdown summary of rocprofv3 output under DIR
  python bench.py --decoder N [--d-inner F] [--workload NAME] [--steps K] [--warmup W] [--no-cpu]
                  # one segment step of an N-layer pre-LN decoder stack (xl_decoder_stack_step),
                  # every layer's memory full: one JSON line (a separate measurement, not the
                  # headline); F defaults to 4 * d_model
  python bench.py --backward [--workload NAME] [--steps K] [--warmup W] [--no-cpu]
                  # the attention-core gradients (xl_rel_attn_core_bwd) on the workload's
                  # shape: one JSON line with the kernel sequence's time and its rate
  python bench.py --vendor-gemm [--workload NAME] [--launches N]
                  # the layer's projection shapes as plain torch.matmul GEMMs (the ROCm
                  # BLAS library): the platform's own rate on them, for context

HBM traffic of the attention kernel comes from two rocprofv3 --pmc passes
(FETCH_SIZE, then WRITE_SIZE) over this script with --copy-calib-mib, each
counter scaled by known bytes / counted KiB of the plain copy in the same
run. The scaled figures are recorded in TRAFFIC below together with the
SHA-256 of the kernel sources they were taken on; when the sources differ,
the reported traffic is null.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0

# Sources that make up the fused attention kernel; the traffic record below is
# valid only for this exact text.
ATTN_SOURCES = ("transformer_xl_relative_amd/csrc/attn_bf16.hip", "transformer_xl_relative_amd/csrc/attn.hip",
                "transformer_xl_relative_amd/csrc/xl_common.hpp", "transformer_xl_relative_amd/csrc/xl_internal.hpp",
                "transformer_xl_relative_amd/build.py")

# HBM bytes per launch of the fused attention kernel (calibrated FETCH_SIZE and
# WRITE_SIZE, see profiles/attn_bf16_kernel_<workload>_pmc_traffic.md).
TRAFFIC = {
    "large_bf16": {"sha256": "db195e5eb6ab7cb1535eed1060ff7fd41d77c01d824cc560574d1227235bfc8f",
                   "bytes": 39642961, "fetch_bytes": 33351505, "write_bytes": 6291456},
}


def attn_sources_sha():
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def layer_flops(w, mlen, kv_ring=False):
    """Algorithmic FLOPs of one layer step: projections + fused attention
    (kv_ring: the keys and values of the memory are kept, so only the
    segment's rows are projected)."""
    B, D, H, dh, q = w.batch, w.d_model, w.n_head, w.d_head, w.qlen
    HD = H * dh
    klen = q + mlen
    n_rel = klen if w.clamp_len < 0 else min(klen, w.clamp_len + 1)
    attn = 6.0 * dh * B * H * w.n_valid_pairs(mlen)          # (q+u).k, (q+v).r, P.V
    kv_rows = B * q if kv_ring else B * klen
    proj = 2.0 * D * HD * (n_rel + B * q + 2 * kv_rows + B * q)   # r, q, k+v, o
    return attn + proj, attn


def attn_min_bytes(w, mlen):
    """Algorithmic (minimum) HBM bytes of the fused attention: the queries, keys,
    values and projected table r read once, the output written once (the
    biases u and v, H*d_head each, are not counted)."""
    B, H, dh, q = w.batch, w.n_head, w.d_head, w.qlen
    klen = q + mlen
    n_rel = klen if w.clamp_len < 0 else min(klen, w.clamp_len + 1)
    es = 2
    return es * (B * H * q * dh + 2 * B * H * klen * dh + H * n_rel * dh + B * q * H * dh)


def host_cpu_model():
    """The host CPU's model name (lscpu's 'Model name', from /proc/cpuinfo),
    with its family, model and stepping numbers (a virtualised host may give
    only a short name)."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                k, _, v = line.partition(":")
                k = k.strip()
                if k in ("model name", "cpu family", "model", "stepping") and k not in fields:
                    fields[k] = v.strip()
                if not line.strip() and fields:
                    break
    except OSError:
        pass
    name = fields.get("model name", "unknown")
    nums = [f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping") if k in fields]
    return f"{name} ({', '.join(nums)})" if nums else name


def roofline(flops, nbytes, seconds, bound=None):
    """Bound, achieved rate and fraction for one kernel time. The bound is
    chosen by arithmetic intensity against the ridge point unless given."""
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    tf = flops / seconds / 1e12
    gbs = nbytes / seconds / 1e9
    if bound is None:
        bound = "hbm" if flops / nbytes < ridge else "mfma"
    if bound == "hbm":
        return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "mfma_tflops": round(tf, 3),
                "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
    return {"bound": "mfma", "achieved": round(tf, 3), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "mfma_tflops": round(tf, 3),
            "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "hbm_gbs": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def cpu_baseline(w, t, min_seconds=10.0):
    """The oracle (as it stands) on a bounded sample: whole layer forwards of
    single batch elements of the same workload, repeated until min_seconds."""
    import oracle
    n, t0 = 0, time.perf_counter()
    while True:
        b = n % w.batch
        oracle.rel_attn_fwd(t["h"].f64[b:b + 1], t["mem"].f64[b:b + 1], t["w_q"].f64, t["w_k"].f64,
                            t["w_v"].f64, t["w_r"].f64, t["w_o"].f64, t["u"].f64, t["v"].f64,
                            n_head=w.n_head, d_head=w.d_head, clamp_len=w.clamp_len,
                            beta=t["beta"].f64 if "beta" in t else None, bias_clamp=w.bias_clamp,
                            bias_kind=w.bias_kind)
        n += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    flops, _ = layer_flops(w, w.mlen)
    per_elem = flops / w.batch
    return {"value": round(per_elem * n / el / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "cpu_model": host_cpu_model(),
            "sample": f"{n} full-layer forwards of one batch element (of {w.batch}) of {w.name}, "
                      f"fp64, {el:.1f} s wall"}


def cpu_baseline_core(w, t, min_seconds=10.0):
    """The oracle's attention core alone (the four dots per pair, softmax, P.V)
    on one batch element's projected operands, repeated until min_seconds; the
    projections are computed once, outside the timing."""
    import numpy as np
    import oracle
    H, dh, q, m = w.n_head, w.d_head, w.qlen, w.mlen
    h, mem = t["h"].f64[:1], t["mem"].f64[:1]
    x = np.concatenate([mem, h], axis=1)
    heads = lambda a, n: a.reshape(1, n, H, dh).transpose(0, 2, 1, 3).copy()
    qh = heads(oracle.linear(h, t["w_q"].f64), q)
    kh = heads(oracle.linear(x, t["w_k"].f64), m + q)
    vh = heads(oracle.linear(x, t["w_v"].f64), m + q)
    n_rel = (m + q) if w.clamp_len < 0 else min(m + q, w.clamp_len + 1)
    rt = oracle.linear(oracle.relpos_embed(0, n_rel, w.d_model), t["w_r"].f64).reshape(n_rel, H, dh)
    rt = rt.transpose(1, 0, 2).copy()
    beta = t["beta"].f64 if "beta" in t else None
    n, t0 = 0, time.perf_counter()
    while True:
        oracle.rel_attn_core(qh, kh, vh, rt, t["u"].f64, t["v"].f64, scale=1.0 / np.sqrt(dh),
                             clamp_len=w.clamp_len, beta=beta, bias_clamp=w.bias_clamp, bias_kind=w.bias_kind)
        n += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    flops = 6.0 * dh * H * w.n_valid_pairs()
    return {"value": round(flops * n / el / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "cpu_model": host_cpu_model(),
            "sample": f"{n} attention cores (four explicit dots per pair, softmax, P.V) of one batch element "
                      f"(of {w.batch}) of {w.name}, fp64, {el:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="large_bf16")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="before warm-up, run a plain device-to-device copy of this many MiB three times")
    ap.add_argument("--summarize", metavar="DIR", help="print a summary of the rocprofv3 databases under DIR")
    ap.add_argument("--core", metavar="WORKLOADS",
                    help="comma-separated workloads: time the fused attention alone; a name may carry @mM (M "
                         "memory rows), @bB (batch B), @sS (at most S workgroups per query tile, as the "
                         "descriptor's attn_splits) and /tpN (one GPU's heads under N-way head sharding)")
    ap.add_argument("--launches", type=int, default=100, help="timed launches per --core measurement")
    ap.add_argument("--decoder", type=int, default=0, metavar="N",
                    help="time one segment step of an N-layer decoder stack instead of the attention layer")
    ap.add_argument("--d-inner", type=int, default=0, help="feed-forward width of --decoder (0: 4 * d_model)")
    ap.add_argument("--backward", action="store_true", help="time the attention-core gradients instead")
    ap.add_argument("--kv-ring", action="store_true",
                    help="step with xl_segment_step_kv (projected keys and values of the memory kept in a ring); "
                         "with --decoder, xl_decoder_stack_step_kv")
    ap.add_argument("--reuse-table", action="store_true",
                    help="steps after the first skip the sinusoid and the R projection (XL_REUSE_TABLE; the "
                         "memory is full, so the table is that of the first step): a separate measurement, "
                         "the default step computes every row of the path")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="time the layer's projection shapes as plain torch.matmul (the ROCm BLAS library): "
                         "context for the projection kernels' rates, not a path of the library")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize, args.copy_calib_mib)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the relative attention forward is "
              "built and measured on a single MI355X", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import transformer_xl_relative_amd as xl
    import xl_inputs
    from tests import gpu_util as gu

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.core:
        core_bench(args.core.split(","), args.launches, args.warmup)
        return
    if args.vendor_gemm:
        vendor_gemm_bench(xl_inputs.WORKLOADS[args.workload], args.launches, args.warmup)
        return
    w = xl_inputs.WORKLOADS[args.workload]
    if w.dtype != "bf16":
        raise SystemExit("bench.py measures the bf16 workloads")
    if args.backward:
        backward_bench(w, args.steps, args.warmup, args.no_cpu)
        return
    if args.decoder > 0:
        decoder_bench(w, args.decoder, args.d_inner or 4 * w.d_model, args.steps, args.warmup, args.no_cpu,
                      args.kv_ring)
        return
    t = xl_inputs.layer_inputs(w) if w.segments == 1 else None
    if t is None:
        # segment workload: bench one steady-state segment (full memory)
        t = xl_inputs.layer_inputs(dataclass_replace(w, segments=1))
    D = w.d_model
    L = gu.Layer(w, t, batch=w.batch, qlen=w.qlen, mlen=w.mlen, out_f32=False)
    h = gu.dev(t["h"])
    ring = gu.dev(t["mem"]).contiguous()
    fifo = xl.xl_mem_fifo(ring.data_ptr(), w.mlen, w.mlen, 0)   # full memory, oldest row first
    desc = xl.make_desc(batch=w.batch, d_model=D, n_head=w.n_head, d_head=w.d_head, qlen=w.qlen, mlen=0,
                        clamp_len=w.clamp_len, bias_clamp=w.bias_clamp, bias_kind=w.bias_kind, dtype=xl.XL_BF16,
                        out_dtype=xl.XL_BF16)
    stream = torch.cuda.current_stream()

    def step():
        xl.xl_segment_step(desc, L.weights, h, fifo, L.out, L.ws, stream)

    if args.kv_ring:
        # the key ring starts empty and fills with the first steps' keys (a
        # memory of mlen keys after ceil(mlen / qlen) steps, before the warm-up)
        if w.qlen % 8 or w.mlen % 8:
            raise SystemExit("--kv-ring needs qlen and mlen multiples of 8")
        cap = (w.mlen + w.qlen + 7) // 8 * 8
        kr = torch.zeros((w.batch, w.n_head, cap, w.d_head), dtype=torch.bfloat16, device="cuda")
        vr = torch.zeros((w.batch, w.n_head, w.d_head, cap), dtype=torch.bfloat16, device="cuda")
        kv = xl.xl_kv_fifo(kr.data_ptr(), vr.data_ptr(), cap, w.mlen, 0, 0)
        kdesc = xl.make_desc(batch=w.batch, d_model=D, n_head=w.n_head, d_head=w.d_head, qlen=w.qlen, mlen=w.mlen,
                             clamp_len=w.clamp_len, bias_clamp=w.bias_clamp, bias_kind=w.bias_kind, dtype=xl.XL_BF16,
                             out_dtype=xl.XL_BF16)
        kws = torch.empty(xl.xl_segment_step_kv_workspace_size(kdesc), dtype=torch.uint8, device="cuda")

        def step():
            xl.xl_segment_step_kv(desc, L.weights, h, kv, L.out, kws, stream)

        while kv.len < w.mlen:
            step()

    if args.reuse_table:
        step()                       # a full-memory step computes the table; the next ones reuse it
        desc.flags = xl.XL_REUSE_TABLE

    if args.copy_calib_mib > 0:
        # a plain elementwise copy kernel (int32 -> float32 conversion: reads and
        # writes 4 bytes per element); the runtime's blit copy is not used because
        # its non-temporal accesses are undercounted by FETCH_SIZE / WRITE_SIZE
        n = (args.copy_calib_mib << 20) // 4
        src = torch.ones(n, dtype=torch.int32, device="cuda")
        dst = torch.empty(n, dtype=torch.float32, device="cuda")
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    # the timed steps: nothing but the steps between the two events
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(K):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = e0.elapsed_time(e1)
    ms_per_step = gpu_ms / K
    # then K more steps with the attention kernel's own start and end timestamps
    evs = [(xl.HipEvent(), xl.HipEvent()) for _ in range(K)]
    for i in range(K):
        xl.xl_set_core_events(*evs[i])
        step()
    torch.cuda.synchronize()
    xl.xl_set_core_events(None, None)
    core_ms = np.array([a.elapsed_ms(b) for a, b in evs])
    core_avg_ms = float(core_ms.mean())
    assert (kv.len if args.kv_ring else fifo.len) == w.mlen

    flops, attn_flops = layer_flops(w, w.mlen, args.kv_ring)
    # the metric: the fused relative attention's algorithmic TFLOP/s over its
    # own kernel time (the merge of key splits included); the whole step's
    # rate is reported beside it as layer_tflops
    value = attn_flops / (core_avg_ms * 1e-3) / 1e12
    layer_tflops = flops / (ms_per_step * 1e-3) / 1e12
    rec = TRAFFIC.get(w.name)
    traffic = rec["bytes"] if rec is not None and rec["sha256"] == attn_sources_sha() else None
    res = {
        "metric": "rel-attn fwd TFLOP/s (4-term+rel_shift) and % bf16 MFMA peak, 1 GPU",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations and memory, N(0,0.02) weights; resident in HBM)",
        "config": {"workload": (f"{w.name}: one segment step (sinusoid, R/Q/K/V projections, fused relative "
                                f"attention, output projection, FIFO update), batch {w.batch}, d_model {D}, "
                                f"{w.n_head} heads x {w.d_head}, qlen {w.qlen}, mlen {w.mlen}, causal")
                               if not args.kv_ring else
                               (f"{w.name}: one segment step on a key ring (sinusoid, R/Q projections, K/V "
                                f"projection of the segment's rows only, fused relative attention over the ring, "
                                f"output projection), batch {w.batch}, d_model {D}, {w.n_head} heads x {w.d_head}, "
                                f"qlen {w.qlen}, mlen {w.mlen}, causal"),
                   "batch": w.batch, "qlen": w.qlen, "mlen": w.mlen, "d_model": D, "n_head": w.n_head,
                   "d_head": w.d_head, "clamp_len": w.clamp_len, "bias_clamp": w.bias_clamp,
                   "reuse_table": bool(args.reuse_table)},
        "roofline": {"kernel": "attn_bf16_kernel (fused relative attention)",
                     **roofline(attn_flops, attn_min_bytes(w, w.mlen), core_avg_ms * 1e-3, bound="mfma"),
                     "traffic": traffic,
                     "algorithmic_flops": attn_flops, "algorithmic_bytes": attn_min_bytes(w, w.mlen),
                     "avg_kernel_us": round(core_avg_ms * 1e3, 3)},
        "layer_tflops": round(layer_tflops, 3),
        "layer_flops_per_step": flops,
        "wall_s_timed_region": round(wall, 4),
    }
    if not args.no_cpu:
        # the metric's own scope: the oracle's attention core against the fused attention
        res["cpu_baseline"] = cpu_baseline_core(w, t)
        res["gpu_over_cpu"] = round(value / res["cpu_baseline"]["value"], 1)
        # and the whole layer against the step
        res["cpu_baseline_layer"] = cpu_baseline(w, t)
        res["gpu_over_cpu_layer"] = round(layer_tflops / res["cpu_baseline_layer"]["value"], 1)
    print(json.dumps(res), flush=True)


FP32_PEAK_TFLOPS = 157.3   # MI355X fp32 peak: dense matrix cores and packed vector alike


def backward_flops(w):
    """Algorithmic FLOPs of the core gradients: per valid pair the two logit
    dots recomputed (4 dh), dP (2 dh), dq from k and r (4 dh), dk, dv and dr
    (2 dh each): 16 dh per pair."""
    return 16.0 * w.d_head * w.batch * w.n_head * w.n_valid_pairs()


def backward_bench(w, K, warmup, no_cpu):
    import numpy as np
    import torch
    import transformer_xl_relative_amd as xl
    import xl_inputs
    from tests import gpu_util as gu
    B, H, dh, q, m = w.batch, w.n_head, w.d_head, w.qlen, w.mlen
    klen = q + m
    n_rel = klen if w.clamp_len < 0 else min(klen, w.clamp_len + 1)
    ci = xl_inputs.core_inputs(batch=B, n_head=H, d_head=dh, qlen=q, mlen=m, n_rows=n_rel, dtype="bf16", seed=w.seed,
                               bias_clamp=w.bias_clamp, bias_kind=w.bias_kind)
    rng = np.random.default_rng(w.seed + 1)
    dout = xl_inputs.Tensor(rng.standard_normal((B, q, H * dh)).astype(np.float32), "bf16")
    ldv = (klen + 63) // 64 * 64
    vt = np.zeros((B, H, dh, ldv), np.float32)
    vt[..., :klen] = ci["v"].f32.transpose(0, 1, 3, 2)
    vt = gu.dev(xl_inputs.Tensor(vt, "bf16"))
    desc = xl.make_desc(batch=B, d_model=H * dh, n_head=H, d_head=dh, qlen=q, mlen=m, clamp_len=w.clamp_len,
                        bias_clamp=w.bias_clamp, bias_kind=w.bias_kind)
    f32 = lambda *sh: torch.empty(sh, dtype=torch.float32, device="cuda")
    g = {"dq": f32(B, H, q, dh), "dk": f32(B, H, klen, dh), "dv": f32(B, H, klen, dh), "dr": f32(H, n_rel, dh),
         "du": f32(H, dh), "dv_bias": f32(H, dh)}
    if w.bias_clamp >= 0:
        g["dbias"] = f32(*ci["beta"].shape)
    ws = torch.empty(xl.xl_rel_attn_core_bwd_workspace_size(desc), dtype=torch.uint8, device="cuda")
    args = [gu.dev(ci[k]) for k in ("q", "k")] + [vt, ldv, gu.dev(ci["r"]), n_rel, gu.dev(ci["u"]), gu.dev(ci["vb"]),
                                                  gu.dev(ci["beta"]) if w.bias_clamp >= 0 else None, gu.dev(dout)]
    stream = torch.cuda.current_stream()

    def run():
        xl.xl_rel_attn_core_bwd(desc, *args, g, ws, stream)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(K):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    flops = backward_flops(w)
    tf = flops / (ms * 1e-3) / 1e12
    res = {"metric": "rel-attn core backward TFLOP/s (dq, dk, dv, dr, du, dv), 1 GPU", "value": round(tf, 3),
           "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": warmup, "ms_per_step": round(ms, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32 (bf16 operands)",
           "data": "synthetic (seeded projected operands of the workload's shape)",
           "config": {"workload": f"{w.name}: gradients of the fused attention core, batch {B}, {H} heads x {dh}, "
                                  f"qlen {q}, mlen {m}", "batch": B, "qlen": q, "mlen": m, "n_head": H, "d_head": dh},
           "roofline": {"kernel": "the backward kernel sequence (bf16 matrix-core products of split fp32 operands)",
                        "bound": "mfma", "achieved": round(tf, 3), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "fp32_peak_frac": round(tf / FP32_PEAK_TFLOPS, 4),
                        "traffic": None, "algorithmic_flops": flops}}
    if not no_cpu:
        import oracle
        n, t0 = 0, time.perf_counter()
        while True:
            b = n % B
            oracle.rel_attn_core_bwd(ci["q"].f64[b:b + 1], ci["k"].f64[b:b + 1], ci["v"].f64[b:b + 1], ci["r"].f64,
                                     ci["u"].f64, ci["vb"].f64, dout.f64[b:b + 1], scale=1.0 / np.sqrt(dh),
                                     clamp_len=w.clamp_len, beta=ci["beta"].f64 if w.bias_clamp >= 0 else None,
                                     bias_clamp=w.bias_clamp, bias_kind=w.bias_kind)
            n += 1
            el = time.perf_counter() - t0
            if el >= 10.0:
                break
        cpu = flops / B * n / el / 1e12
        res["cpu_baseline"] = {"value": round(cpu, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
                               "kind": "oracle", "sample": f"{n} core backwards of one batch element (of {B}) of "
                                                           f"{w.name}, fp64, {el:.1f} s wall"}
        res["gpu_over_cpu"] = round(tf / cpu, 1)
    print(json.dumps(res), flush=True)


def decoder_flops(w, d_inner, kv_ring=False):
    """Algorithmic FLOPs of one decoder layer step: the attention layer and the
    two feed-forward GEMMs (layer norms, biases, ReLU and residuals are
    elementwise and not counted); with key rings only the segment's keys and
    values are projected."""
    flops, _ = layer_flops(w, w.mlen, kv_ring)
    return flops + 2.0 * 2.0 * w.batch * w.qlen * w.d_model * d_inner


def decoder_bench(w, n_layer, d_inner, K, warmup, no_cpu, kv_ring=False):
    import numpy as np
    import torch
    import transformer_xl_relative_amd as xl
    import xl_inputs
    from tests import gpu_util as gu
    if w.segments > 1:
        w = dataclass_replace(w, segments=1)
    t = xl_inputs.decoder_inputs(w, d_inner=d_inner, n_layer=n_layer)
    D = w.d_model
    weights = [gu.dec_weights(lw) for lw in t["layers"]]
    # every layer's memory full (the drawn memory rows, oldest first)
    rings = [gu.dev(t["mem"]).contiguous() for _ in range(n_layer)]
    fifos = (xl.xl_mem_fifo * n_layer)(*[xl.xl_mem_fifo(r.data_ptr(), w.mlen, w.mlen, 0) for r in rings])
    desc = xl.make_desc(batch=w.batch, d_model=D, n_head=w.n_head, d_head=w.d_head, qlen=w.qlen, mlen=w.mlen,
                        clamp_len=w.clamp_len, bias_clamp=w.bias_clamp, bias_kind=w.bias_kind, dtype=xl.XL_BF16,
                        out_dtype=xl.XL_BF16)
    ws = torch.empty(xl.xl_decoder_stack_workspace_size(desc, d_inner), dtype=torch.uint8, device="cuda")
    h = gu.dev(t["h"])
    out = torch.empty((w.batch, w.qlen, D), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        xl.xl_decoder_stack_step(desc, d_inner, 0.0, weights, h, fifos, out, ws, stream)

    if kv_ring:
        # each layer's memory as a full key ring: one step over the drawn memory
        # rows (qlen = mlen) from empty rings projects them in, then every timed
        # step runs with len = mlen and moves the ring by qlen
        if w.qlen % 8 or w.mlen % 8:
            raise SystemExit("--kv-ring needs qlen and mlen multiples of 8")
        H, dh, cap = w.n_head, w.d_head, w.mlen + w.qlen
        kr = [torch.empty((w.batch, H, cap, dh), dtype=torch.bfloat16, device="cuda") for _ in range(n_layer)]
        vr = [torch.empty((w.batch, H, dh, cap), dtype=torch.bfloat16, device="cuda") for _ in range(n_layer)]
        kvs = (xl.xl_kv_fifo * n_layer)(*[xl.xl_kv_fifo(k.data_ptr(), v.data_ptr(), cap, w.mlen, 0, 0)
                                          for k, v in zip(kr, vr)])
        d0 = xl.make_desc(batch=w.batch, d_model=D, n_head=H, d_head=dh, qlen=w.mlen, mlen=0, clamp_len=w.clamp_len,
                          bias_clamp=w.bias_clamp, bias_kind=w.bias_kind, dtype=xl.XL_BF16, out_dtype=xl.XL_BF16)
        ws0 = torch.empty(xl.xl_decoder_stack_kv_workspace_size(d0, d_inner), dtype=torch.uint8, device="cuda")
        out0 = torch.empty((w.batch, w.mlen, D), dtype=torch.bfloat16, device="cuda")
        xl.xl_decoder_stack_step_kv(d0, d_inner, 0.0, weights, gu.dev(t["mem"]).contiguous(), kvs, out0, ws0, stream)
        del ws0, out0
        ws = torch.empty(xl.xl_decoder_stack_kv_workspace_size(desc, d_inner), dtype=torch.uint8, device="cuda")

        def step():
            xl.xl_decoder_stack_step_kv(desc, d_inner, 0.0, weights, h, kvs, out, ws, stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(K):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    if kv_ring:
        assert all(r.len == w.mlen for r in kvs)
    flops = n_layer * decoder_flops(w, d_inner, kv_ring)
    value = flops / (ms * 1e-3) / 1e12
    res = {
        "metric": "decoder stack fwd TFLOP/s (pre-LN layers: relative attention + FFN), 1 GPU",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations and memories, N(0,0.02) weights, LN gains 1+N(0,0.02))",
        "config": {"workload": (f"{w.name} decoder stack: one segment step of {n_layer} pre-LN layers (LN1 over "
                                f"[memory ; segment], relative attention + residual, LN2, FFN {D}->{d_inner}->{D} "
                                f"+ residual, per-layer FIFO update), batch {w.batch}, qlen {w.qlen}, mlen {w.mlen}"
                                if not kv_ring else
                                f"{w.name} decoder stack on key rings: one segment step of {n_layer} pre-LN layers "
                                f"(LN1 over the segment, its keys and values projected into the layer's ring of "
                                f"projected memory keys, relative attention + residual, LN2, FFN {D}->{d_inner}->{D} "
                                f"+ residual), batch {w.batch}, qlen {w.qlen}, mlen {w.mlen}"),
                   "n_layer": n_layer, "d_inner": d_inner, "batch": w.batch, "qlen": w.qlen, "mlen": w.mlen,
                   "d_model": D, "n_head": w.n_head, "d_head": w.d_head},
        "flops_per_step": flops,
    }
    if not no_cpu:
        import oracle
        lw = gu.oracle_dec_weights(t["layers"][0])
        n, t0 = 0, time.perf_counter()
        while True:
            b = n % w.batch
            oracle.decoder_layer_fwd(t["h"].f64[b:b + 1], t["mem"].f64[b:b + 1], lw, n_head=w.n_head,
                                     d_head=w.d_head, clamp_len=w.clamp_len, bias_clamp=w.bias_clamp,
                                     bias_kind=w.bias_kind)
            n += 1
            el = time.perf_counter() - t0
            if el >= 10.0:
                break
        # (the same algorithmic count as the GPU figure: one layer step's work)
        cpu = decoder_flops(w, d_inner, kv_ring) / w.batch * n / el / 1e12
        res["cpu_baseline"] = {"value": round(cpu, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
                               "kind": "oracle",
                               "sample": f"{n} decoder-layer forwards of one batch element (of {w.batch}) of "
                                         f"{w.name}, fp64, {el:.1f} s wall"}
        res["gpu_over_cpu"] = round(value / cpu, 1)
    print(json.dumps(res), flush=True)


def vendor_gemm_bench(w, launches, warmup):
    """The layer's four projection products as plain row-major GEMMs through
    torch.matmul (hipBLASLt on ROCm), `launches` calls each replayed from a
    captured graph and timed with events: the rate the platform's own GEMM
    reaches on these shapes, printed as one JSON line. No epilogue (head layout, V^T, ring) and no grouping: a
    reference point for the projection kernels, whose times come from the
    kernel traces of the layer step."""
    import torch
    D, HD = w.d_model, w.n_head * w.d_head
    klen = w.qlen + w.mlen
    n_rel = klen if w.clamp_len < 0 else min(klen, w.clamp_len + 1)
    shapes = {"r": (n_rel, HD, D), "q": (w.batch * w.qlen, HD, D), "kv": (w.batch * klen, 2 * HD, D),
              "o": (w.batch * w.qlen, D, HD)}
    out = {"workload": w.name, "library": "torch.matmul (bf16 in, bf16 out), graph replay", "launches": launches}
    g = torch.Generator(device="cuda").manual_seed(0)
    for name, (M, N, K) in shapes.items():
        a = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16)
        b = torch.randn(N, K, device="cuda", generator=g).to(torch.bfloat16)
        bt = b.t()
        c = torch.empty(M, N, device="cuda", dtype=torch.bfloat16)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(max(warmup, 3)):
                torch.matmul(a, bt, out=c)
        torch.cuda.current_stream().wait_stream(side)
        # the calls replayed from a captured graph, so that the host's
        # per-call cost does not pace the GPU
        per_graph = 20
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(per_graph):
                torch.matmul(a, bt, out=c)
        replays = max(launches // per_graph, 1)
        graph.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(replays):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (replays * per_graph)
        tf = 2.0 * M * N * K / (us * 1e-6) / 1e12
        out[name] = {"M": M, "N": N, "K": K, "us": round(us, 3), "tflops": round(tf, 1),
                     "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
    print(json.dumps(out), flush=True)


def core_bench(names, launches, warmup):
    """The fused attention alone on each workload's projected operands (taken
    from the workspace of one layer forward): per-launch kernel times from
    runtime-timestamped HIP events, warm (operands as the projections left
    them) and cold (1 GiB written between launches, more than the 256 MB
    last-level cache holds)."""
    import numpy as np
    import torch
    import transformer_xl_relative_amd as xl
    import xl_inputs
    from tests import gpu_util as gu

    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    for name in names:
        # "NAME/tpN": one GPU's share when the heads are sharded over N GPUs;
        # "@mM": M memory rows (a sweep of the key count); "@bB": batch B (every
        # compute unit with two workgroups, for instance); "@sS": the key-split
        # cap S of the descriptor (a sweep of the split count)
        base, _, tp = name.partition("/tp")
        base, *mods = base.split("@")
        w = xl_inputs.WORKLOADS[base]
        splits = 0
        for mod in mods:
            key, val = mod[:1], int(mod[1:])
            if key == "m":
                w = dataclass_replace(w, mlen=val)
            elif key == "b":
                w = dataclass_replace(w, batch=val)
            elif key == "s":
                splits = val
            else:
                raise SystemExit(f"{name}: unknown modifier @{mod}")
        if tp:
            if w.n_head % int(tp):
                raise SystemExit(f"{name}: {w.n_head} heads do not split over {tp} GPUs")
            w = dataclass_replace(w, n_head=w.n_head // int(tp))
        if w.dtype != "bf16":
            raise SystemExit("--core measures the bf16 workloads")
        if w.segments > 1:
            w = dataclass_replace(w, segments=1)   # one steady-state segment (full memory)
        t = xl_inputs.layer_inputs(w)
        L = gu.Layer(w, t, batch=w.batch, qlen=w.qlen, mlen=w.mlen, out_f32=False)
        xl.xl_rel_attn_fwd(L.desc, L.weights, gu.dev(t["h"]), gu.dev(t["mem"]), L.out, L.ws)
        lay = L.layout
        B, H, dh, q = w.batch, w.n_head, w.d_head, w.qlen
        qd = L.ws_view(lay.q, (B, H, q, dh))
        k, vt = L.ws_view(lay.k, (B, H, lay.klen, dh)), L.ws_view(lay.vt, (B, H, dh, lay.ldv))
        r = L.ws_view(lay.r, (H, lay.n_rel, dh))
        attn = torch.empty((B, q, H * dh), dtype=torch.bfloat16, device="cuda")
        L.desc.attn_splits = splits
        nws = xl.xl_rel_attn_core_workspace_size(L.desc)
        cws = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws else None
        beta = L.weights.bias_table

        def run():
            xl.xl_rel_attn_core(L.desc, qd, k, vt, lay.ldv, r, lay.n_rel, L.weights.u, L.weights.v, beta, attn, cws)

        out = {"workload": name, "key_split_workspace": nws > 0}
        flops = 6.0 * dh * B * H * w.n_valid_pairs()
        nbytes = attn_min_bytes(w, w.mlen)
        for mode in ("warm", "cold"):
            for _ in range(warmup):
                run()
            evs = [(xl.HipEvent(), xl.HipEvent()) for _ in range(launches)]
            torch.cuda.synchronize()
            for i in range(launches):
                if mode == "cold":
                    scratch.fill_(i & 255)
                xl.xl_set_core_events(*evs[i])
                run()
            torch.cuda.synchronize()
            xl.xl_set_core_events(None, None)
            us = np.array([a.elapsed_ms(b) for a, b in evs]) * 1e3
            med = float(np.median(us))
            out[mode] = {"median_us": round(med, 3), "p10_us": round(float(np.percentile(us, 10)), 3),
                         "p90_us": round(float(np.percentile(us, 90)), 3),
                         **roofline(flops, nbytes, med * 1e-6)}
        out["algorithmic_flops"] = flops
        out["algorithmic_bytes"] = nbytes
        print(json.dumps(out), flush=True)


def summarize(d, copy_mib):
    """Markdown tables from the rocprofv3 SQLite output under d: per-kernel
    launch count and average duration, and for counter runs the average
    counter value per dispatch (with the copy-kernel scale factor when the
    run held a plain copy of copy_mib MiB)."""
    import collections
    import sqlite3
    dbs = sorted(glob.glob(os.path.join(d, "**", "*.db"), recursive=True))
    if not dbs:
        raise SystemExit(f"no rocprofv3 database under {d}")

    def short(name):
        return name.replace("void ", "").replace("xl::(anonymous namespace)::", "").split("(")[0]

    for db in dbs:
        c = sqlite3.connect(db)
        tabs = {r[0] for r in c.execute("select name from sqlite_master")}
        print(f"### {os.path.relpath(db, d)}\n")
        if "kernels" in tabs:
            dur = collections.defaultdict(list)
            for name, gx, gy, gz, wx, wy, wz, st, en in c.execute(
                    "select name, grid_x, grid_y, grid_z, workgroup_x, workgroup_y, workgroup_z, start, end "
                    "from kernels"):
                wgs = (gx // max(wx, 1)) * (gy // max(wy, 1)) * (gz // max(wz, 1))
                dur[(short(name), wgs)].append((en - st) / 1e3)
            if dur:
                print("| kernel | workgroups | launches | avg us | min us | max us |")
                print("|---|---|---|---|---|---|")
                for (k, wg), v in sorted(dur.items(), key=lambda kv: -sum(kv[1])):
                    print(f"| {k} | {wg} | {len(v)} | {sum(v) / len(v):.3f} | {min(v):.3f} | {max(v):.3f} |")
                print()
        if "counters_collection" in tabs:
            agg = collections.defaultdict(list)
            for kname, cname, val in c.execute("select kernel_name, counter_name, value from counters_collection"):
                agg[(short(kname), cname)].append(val)
            if agg:
                print("| kernel | counter | dispatches | avg per dispatch |")
                print("|---|---|---|---|")
                for (k, cn), v in sorted(agg.items()):
                    print(f"| {k} | {cn} | {len(v)} | {sum(v) / len(v):.1f} |")
                print()
                if copy_mib:
                    kib = copy_mib * 1024
                    for (k, cn), v in sorted(agg.items()):
                        if "copy_kernel" in k and cn in ("FETCH_SIZE", "WRITE_SIZE"):
                            avg = sum(v) / len(v)
                            print(f"copy calibration {cn}: {kib} KiB moved, {avg:.1f} KiB counted, "
                                  f"scale {kib / avg:.4f}\n")


def dataclass_replace(w, **kw):
    import dataclasses
    return dataclasses.replace(w, **kw)


if __name__ == "__main__":
    main()
