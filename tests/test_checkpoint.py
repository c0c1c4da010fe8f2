"""Host-side checks of the memory checkpoint files (CPU tensors, no GPU): the
ring bytes, len and head survive a save and load bit for bit, files load
without unpickling, and inconsistent or foreign files are refused."""
import numpy as np
import pytest
import torch

import transformer_xl_relative_amd as xl
from transformer_xl_relative_amd import checkpoint


def _bits(shape, seed):
    g = np.random.default_rng(seed)
    return torch.from_numpy(g.integers(0, 1 << 16, size=shape, dtype=np.uint16).astype(np.int16)).view(torch.bfloat16)


def test_state_fifo_round_trip(tmp_path):
    ring = _bits((3, 40, 16), 1)
    fifo = xl.xl_mem_fifo(ring.data_ptr(), 40, 33, 37)
    p = tmp_path / "f.npz"
    checkpoint.save_fifo(p, fifo, ring)
    buf, f2 = checkpoint.load_fifo(p, device="cpu")
    assert buf.dtype == torch.bfloat16 and buf.shape == ring.shape
    assert torch.equal(buf.view(torch.int16), ring.view(torch.int16))
    assert (f2.mlen_max, f2.len, f2.head) == (40, 33, 37) and f2.buf == buf.data_ptr()
    with np.load(p, allow_pickle=False) as z:      # plain arrays only
        assert set(z.files) == {"format", "kind", "buf", "dtype", "shape", "ints"}


def test_key_ring_round_trip(tmp_path):
    k, vt = _bits((2, 4, 48, 8), 2), _bits((2, 4, 8, 48), 3)
    kv = xl.xl_kv_fifo(k.data_ptr(), vt.data_ptr(), 48, 32, 24, 40)
    p = tmp_path / "k.npz"
    checkpoint.save_kv_fifo(p, kv, k, vt)
    k2, vt2, kv2 = checkpoint.load_kv_fifo(p, device="cpu")
    assert torch.equal(k2.view(torch.int16), k.view(torch.int16))
    assert torch.equal(vt2.view(torch.int16), vt.view(torch.int16))
    assert (kv2.cap, kv2.mlen_max, kv2.len, kv2.head) == (48, 32, 24, 40)
    assert (kv2.k, kv2.vt) == (k2.data_ptr(), vt2.data_ptr())


def test_refusals(tmp_path):
    ring = _bits((1, 8, 4), 4)
    with pytest.raises(ValueError):                 # the FIFO does not point at this tensor
        checkpoint.save_fifo(tmp_path / "x.npz", xl.xl_mem_fifo(0, 8, 0, 0), ring)
    p = tmp_path / "s.npz"
    checkpoint.save_fifo(p, xl.xl_mem_fifo(ring.data_ptr(), 8, 5, 2), ring)
    with pytest.raises(ValueError):                 # a state FIFO file is not a key ring
        checkpoint.load_kv_fifo(p, device="cpu")
    bad = tmp_path / "bad.npz"
    with np.load(p, allow_pickle=False) as z:
        d = {n: z[n] for n in z.files}
    d["ints"] = np.array([8, 9, 2], np.int64)       # len beyond mlen_max
    np.savez(bad, **d)
    with pytest.raises(ValueError):
        checkpoint.load_fifo(bad, device="cpu")
