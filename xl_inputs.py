"""Seeded synthetic inputs for the Transformer-XL relative attention forward.

This module is shared by the GPU library's tests/bench and by the CPU oracle's
tests. It holds no arithmetic of the method itself: it only draws random
numbers, rounds them to the storage precision, and describes the five
workload shapes.

Workloads (value recipe, applied to every one):
  * hidden states h and memory N(0, 1);
  * projection weights W_q, W_k, W_v, W_r (each [n_head*d_head, d_model]) and
    W_o ([d_model, n_head*d_head]) N(0, 0.02) -- the nn.Linear [out, in]
    layout, so a projection is y = x @ W^T;
  * global biases u, v ([n_head, d_head]) N(0, 0.02);
  * the optional per-head scalar bias table beta ([2*bias_clamp+1, n_head],
    or [12, n_head] for the T5 buckets) N(0, 0.02).
Draws are float32 from numpy.random.default_rng(seed) in the order
h, mem, W_q, W_k, W_v, W_r, W_o, u, v, beta; bf16 workloads round every draw
once to bfloat16 (round to nearest even) and both sides consume those bits.
A second recipe ("sensitive", see RECIPES) draws the same shapes in the same
order with larger parameter scales, for parity tests that must see every
term of the score in the layer output.
"""
from __future__ import annotations

import dataclasses
import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    d_model: int
    n_head: int
    d_head: int
    qlen: int
    mlen: int
    clamp_len: int = -1     # < 0: no clamp of the relative distance
    bias_clamp: int = -1    # < 0: no scalar bias table
    bias_kind: int = 0      # 0: rows by clamped distance, 1: twelve T5 bucket rows
    dtype: str = "bf16"     # "f32" or "bf16"
    segments: int = 1       # > 1: segment-recurrent run with FIFO memory
    seed: int = 0

    @property
    def klen(self) -> int:
        return self.qlen + self.mlen

    def n_valid_pairs(self, mlen: int | None = None) -> int:
        """Causal (query, key) pairs per (batch, head): query i sees j <= mlen+i."""
        m = self.mlen if mlen is None else mlen
        q = self.qlen
        return q * m + q * (q + 1) // 2


# The five workloads: tiny fp32, base-like, large-like (the throughput
# target, qlen = mlen = 384), long-memory evaluation, and the 4-segment
# recurrent run with a +-128 scalar bias table.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 16, 2, 8, 8, 8, clamp_len=16, dtype="f32", seed=0),
    "base_bf16": Workload("base_bf16", 32, 512, 8, 64, 128, 128, seed=1),
    "large_bf16": Workload("large_bf16", 8, 1024, 16, 64, 384, 384, seed=2),
    "longmem_bf16": Workload("longmem_bf16", 4, 512, 8, 64, 64, 1600, clamp_len=1000, seed=3),
    "segments_bf16": Workload("segments_bf16", 4, 1024, 16, 64, 512, 512, bias_clamp=128,
                              segments=4, seed=4),
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to float32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


class Tensor:
    """One input: the exact stored values (float64 view) and the storage bits."""

    def __init__(self, f32: np.ndarray, dtype: str):
        self.dtype = dtype
        if dtype == "bf16":
            self.bits = bf16_bits(f32)
            self.f32 = bf16_to_f32(self.bits)
        elif dtype == "f32":
            self.f32 = np.ascontiguousarray(f32, dtype=np.float32)
            self.bits = self.f32
        else:
            raise ValueError(dtype)
        self.f64 = self.f32.astype(np.float64)

    @property
    def shape(self):
        return self.f32.shape


def _normal(rng, shape, std):
    return (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def bias_rows(bias_clamp: int, bias_kind: int) -> int:
    """Rows of the scalar bias table: 2k+1 clamped distances, or 12 buckets."""
    return 12 if bias_kind == 1 else 2 * bias_clamp + 1


# Standard deviations of the drawn parameters. "config" is the workloads' own
# recipe. "sensitive" is a second recipe for parity tests of the composed
# layer: projections N(0, 1/fan_in) (so that projected queries, keys, values
# and table rows are of unit size), u and v N(0, 0.5), the bias table N(0, 1).
# Under it every term of the score moves the layer output by much more than
# the bf16 tolerance, which the config recipe's tiny weights do not.
RECIPES = ("config", "sensitive")


def _std(recipe: str, name: str, fan_in: int) -> float:
    if recipe == "config":
        return 0.02
    if recipe == "sensitive":
        if name in ("w_q", "w_k", "w_v", "w_r", "w_o"):
            return float(1.0 / np.sqrt(fan_in))
        return {"u": 0.5, "v": 0.5, "beta": 1.0}[name]
    raise ValueError(recipe)


def layer_inputs(w: Workload, *, batch: int | None = None, qlen: int | None = None,
                 mlen: int | None = None, seed: int | None = None, recipe: str = "config") -> dict:
    """Draw one layer call's inputs. Sizes default to the workload's.

    For a segment-recurrent workload, 'h' is the whole input stream
    [batch, segments*qlen, d_model] and 'mem' is empty (the run starts with
    no memory). recipe selects the parameter scales (RECIPES); the draw order
    is the same for both.
    """
    B = w.batch if batch is None else batch
    q = w.qlen if qlen is None else qlen
    m = w.mlen if mlen is None else mlen
    rng = np.random.default_rng(w.seed if seed is None else seed)
    HD = w.n_head * w.d_head
    D = w.d_model
    if w.segments > 1:
        h = _normal(rng, (B, w.segments * q, D), 1.0)
        mem = np.zeros((B, 0, D), np.float32)
    else:
        h = _normal(rng, (B, q, D), 1.0)
        mem = _normal(rng, (B, m, D), 1.0)
    sd = lambda name, fan_in=0: _std(recipe, name, fan_in)
    out = {
        "h": h, "mem": mem,
        "w_q": _normal(rng, (HD, D), sd("w_q", D)),
        "w_k": _normal(rng, (HD, D), sd("w_k", D)),
        "w_v": _normal(rng, (HD, D), sd("w_v", D)),
        "w_r": _normal(rng, (HD, D), sd("w_r", D)),
        "w_o": _normal(rng, (D, HD), sd("w_o", HD)),
        "u": _normal(rng, (w.n_head, w.d_head), sd("u")),
        "v": _normal(rng, (w.n_head, w.d_head), sd("v")),
    }
    if w.bias_clamp >= 0:
        out["beta"] = _normal(rng, (bias_rows(w.bias_clamp, w.bias_kind), w.n_head), sd("beta"))
    return {k: Tensor(a, w.dtype) for k, a in out.items()}


def decoder_inputs(w: Workload, *, d_inner: int, n_layer: int, batch: int | None = None, qlen: int | None = None,
                   mlen: int | None = None, seed: int | None = None, recipe: str = "config") -> dict:
    """Inputs of a decoder stack: 'h' (or the whole stream of a
    segment-recurrent workload) and 'mem' as layer_inputs draws them, then per
    layer, in order, the attention weights (the same recipe as layer_inputs),
    LN1 gain 1 + N(0, 0.02) and shift N(0, 0.02), the same for LN2, W1
    [d_inner, D], b1 [d_inner], W2 [D, d_inner], b2 [D], all N(0, 0.02).
    recipe scales the attention weights as layer_inputs does (RECIPES).
    Returns {'h', 'mem', 'layers': [dict per layer]}."""
    B = w.batch if batch is None else batch
    q = w.qlen if qlen is None else qlen
    m = w.mlen if mlen is None else mlen
    rng = np.random.default_rng(w.seed if seed is None else seed)
    HD, D = w.n_head * w.d_head, w.d_model
    if w.segments > 1:
        h = _normal(rng, (B, w.segments * q, D), 1.0)
        mem = np.zeros((B, 0, D), np.float32)
    else:
        h = _normal(rng, (B, q, D), 1.0)
        mem = _normal(rng, (B, m, D), 1.0)
    layers = []
    for _ in range(n_layer):
        sd = lambda name, fan_in=0: _std(recipe, name, fan_in)
        lw = {
            "w_q": _normal(rng, (HD, D), sd("w_q", D)), "w_k": _normal(rng, (HD, D), sd("w_k", D)),
            "w_v": _normal(rng, (HD, D), sd("w_v", D)), "w_r": _normal(rng, (HD, D), sd("w_r", D)),
            "w_o": _normal(rng, (D, HD), sd("w_o", HD)),
            "u": _normal(rng, (w.n_head, w.d_head), sd("u")), "v": _normal(rng, (w.n_head, w.d_head), sd("v")),
        }
        if w.bias_clamp >= 0:
            lw["beta"] = _normal(rng, (bias_rows(w.bias_clamp, w.bias_kind), w.n_head), sd("beta"))
        lw["ln1_g"] = (1.0 + _normal(rng, (D,), 0.02)).astype(np.float32)
        lw["ln1_b"] = _normal(rng, (D,), 0.02)
        lw["ln2_g"] = (1.0 + _normal(rng, (D,), 0.02)).astype(np.float32)
        lw["ln2_b"] = _normal(rng, (D,), 0.02)
        lw["w1"] = _normal(rng, (d_inner, D), 0.02)
        lw["b1"] = _normal(rng, (d_inner,), 0.02)
        lw["w2"] = _normal(rng, (D, d_inner), 0.02)
        lw["b2"] = _normal(rng, (D,), 0.02)
        layers.append({k: Tensor(a, w.dtype) for k, a in lw.items()})
    return {"h": Tensor(h, w.dtype), "mem": Tensor(mem, w.dtype), "layers": layers}


def core_inputs(*, batch: int, n_head: int, d_head: int, qlen: int, mlen: int, n_rows: int,
                dtype: str, seed: int, bias_clamp: int = -1, bias_kind: int = 0) -> dict:
    """Inputs for the attention core alone: head-major q, k, v, a projected
    relative table r ([n_head, n_rows, d_head], row n <-> distance n) and the
    biases u, v. Magnitudes are those of projected N(0,1) activations."""
    rng = np.random.default_rng(seed)
    k_len = qlen + mlen
    out = {
        "q": _normal(rng, (batch, n_head, qlen, d_head), 0.6),
        "k": _normal(rng, (batch, n_head, k_len, d_head), 0.6),
        "v": _normal(rng, (batch, n_head, k_len, d_head), 0.6),
        "r": _normal(rng, (n_head, n_rows, d_head), 0.6),
        "u": _normal(rng, (n_head, d_head), 0.3),
        "vb": _normal(rng, (n_head, d_head), 0.3),
    }
    if bias_clamp >= 0:
        out["beta"] = _normal(rng, (bias_rows(bias_clamp, bias_kind), n_head), 0.3)
    return {k: Tensor(a, dtype) for k, a in out.items()}


def long_key_core_inputs(*, qlen: int, mlen: int, n_rows: int, seed: int, probes: dict, pool: int = 4096) -> dict:
    """Inputs for the attention core over a very long key range (one batch
    element, one head, d_head 64, bf16), drawn in seconds even for tens of
    millions of keys, and built so that a sampled output shows a key or value
    read from the wrong place:

    * a shared direction c and one direction w_i per probed query row i:
      seeded, orthonormal;
    * query row i: 3 c + 3 w_i (probed rows only) + N(0, 0.3);
    * keys and values: rows of two seeded pools of `pool` N(0, 0.6) rows, one
      seeded index per key; every key then has 55 c subtracted, so its scaled
      content score is near -20 for every query and all of them together weigh
      little against one probe;
    * probes {query row i: key j}: key j is 20 w_i and its value a seeded N(0, 1)
      row, so that query row i, when it sees key j, puts almost all of its
      weight there (scaled score about 7.5, against about 0 for the other
      probes), and none when the causal mask hides key j from it;
    * r (n_rows distance rows) N(0, 0.6); u and v N(0, 0.3).

    Draw order: c and the directions, q noise, the two pools, the key index, the
    value index, the probe values, r, u, v. Returns Tensor objects for q, r, u
    and vb, and for k and v the bf16 bits [k_len, 64] ("k_bits", "v_bits") and
    their exact values [1, 1, k_len, 64] as float64 ("k", "v")."""
    dh = 64
    k_len = qlen + mlen
    rows = sorted(probes)
    assert all(0 <= i < qlen for i in rows) and all(0 <= probes[i] < k_len for i in rows)
    rng = np.random.default_rng(seed)
    basis, _ = np.linalg.qr(rng.standard_normal((dh, len(rows) + 1)))
    c, w = basis[:, 0], {i: basis[:, 1 + n] for n, i in enumerate(rows)}
    q = 3.0 * c[None, :] + rng.standard_normal((qlen, dh)) * 0.3
    for i in rows:
        q[i] += 3.0 * w[i]
    pools = [bf16_bits(_normal(rng, (pool, dh), 0.6) - (55.0 * c[None, :] if n == 0 else 0.0)) for n in range(2)]
    out = {}
    for name, bits in (("k", pools[0]), ("v", pools[1])):
        idx = rng.integers(0, pool, size=k_len)
        out[name + "_bits"] = bits[idx]
        out[name] = bf16_to_f32(bits).astype(np.float64)[idx][None, None]
    vals = bf16_bits(rng.standard_normal((len(rows), dh)).astype(np.float32))
    for n, i in enumerate(rows):
        j = probes[i]
        kb = bf16_bits((20.0 * w[i]).astype(np.float32))
        out["k_bits"][j] = kb
        out["k"][0, 0, j] = bf16_to_f32(kb)
        out["v_bits"][j] = vals[n]
        out["v"][0, 0, j] = bf16_to_f32(vals[n])
    out["q"] = Tensor(q.astype(np.float32)[None, None], "bf16")
    out["r"] = Tensor(_normal(rng, (1, n_rows, dh), 0.6), "bf16")
    out["u"] = Tensor(_normal(rng, (1, dh), 0.3), "bf16")
    out["vb"] = Tensor(_normal(rng, (1, dh), 0.3), "bf16")
    return out


def long_memory_layer_inputs(*, d_model: int, n_head: int, qlen: int, mlen: int, seed: int, pool: int = 4096) -> dict:
    """Layer inputs (one batch element, bf16, d_head 64) with a memory of tens
    of millions of rows, drawn in seconds: each memory row is a row of a seeded
    pool of `pool` N(0, 1) rows, picked by a seeded index per memory row; h
    N(0, 1); W_q, W_k, W_v, W_r, W_o and u, v N(0, 0.02), the workloads' recipe.
    Draw order: h, the pool, the index, W_q, W_k, W_v, W_r, W_o, u, v. Returns
    Tensor objects for h, the pool ("mem_pool") and the weights, the index
    ("mem_idx") and the memory's bf16 bits [1, mlen, d_model] ("mem_bits")."""
    rng = np.random.default_rng(seed)
    hd = n_head * 64
    out = {"h": Tensor(_normal(rng, (1, qlen, d_model), 1.0), "bf16")}
    out["mem_pool"] = Tensor(_normal(rng, (pool, d_model), 1.0), "bf16")
    out["mem_idx"] = rng.integers(0, pool, size=mlen)
    out["mem_bits"] = out["mem_pool"].bits[out["mem_idx"]][None]
    for name, shape in (("w_q", (hd, d_model)), ("w_k", (hd, d_model)), ("w_v", (hd, d_model)),
                        ("w_r", (hd, d_model)), ("w_o", (d_model, hd))):
        out[name] = Tensor(_normal(rng, shape, 0.02), "bf16")
    out["u"] = Tensor(_normal(rng, (n_head, 64), 0.02), "bf16")
    out["v"] = Tensor(_normal(rng, (n_head, 64), 0.02), "bf16")
    return out


def identity_head_weights(*, seed: int) -> dict:
    """Layer weights of one head (d_head 64) at d_model 64 whose query and
    output projections are the identity, so that the layer's queries are its
    input rows and its output is the attention output; W_k, W_v, W_r
    N(0, 0.02), drawn in that order."""
    rng = np.random.default_rng(seed)
    eye = np.eye(64, dtype=np.float32)
    out = {"w_q": Tensor(eye, "bf16"), "w_o": Tensor(eye, "bf16")}
    for name in ("w_k", "w_v", "w_r"):
        out[name] = Tensor(_normal(rng, (64, 64), 0.02), "bf16")
    return out
