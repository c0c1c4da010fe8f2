"""Checkpoint and resume of a segment-recurrent run's state.

The only state a segment-recurrent run carries from one segment to the next
is the memory (felixzhao.cn article 118 §2.3.1: the cached states of the
previous segment; intelliparadigm.com 2238855 §3.2: the cache reused at
evaluation). Here it is caller-owned: the FIFO ring of layer input states
(xl_mem_fifo: ring bytes, len, head) or the key ring of projected keys and
values (xl_kv_fifo: two rings, cap, len, head). Resuming in another process
therefore means restoring those bytes and integers exactly; the next segment
step then computes what the uninterrupted run computes.

The files are numpy .npz archives of plain arrays (no pickled objects: they
load with allow_pickle=False). Device buffers are copied through host memory
as raw bytes, so bf16 contents survive bit for bit.
"""
import numpy as np
import torch

from . import xl_kv_fifo, xl_mem_fifo

_FORMAT = "xl-fifo-1"


def _bytes_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.uint8).cpu().numpy().reshape(-1)


def _tensor_of(raw: np.ndarray, dtype: str, shape, device) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(raw)).to(device)
    return t.view(getattr(torch, dtype)).reshape(tuple(int(s) for s in shape))


def save_fifo(path, fifo: xl_mem_fifo, buf: torch.Tensor) -> None:
    """Write the state FIFO (its ring `buf`, whose data pointer fifo.buf holds) to `path`."""
    if buf.data_ptr() != fifo.buf:
        raise ValueError("buf is not the FIFO's ring")
    np.savez(path, format=np.array(_FORMAT), kind=np.array("state"), buf=_bytes_of(buf),
             dtype=np.array(str(buf.dtype).replace("torch.", "")), shape=np.array(buf.shape, np.int64),
             ints=np.array([fifo.mlen_max, fifo.len, fifo.head], np.int64))


def load_fifo(path, device="cuda"):
    """Read a state FIFO written by save_fifo: returns (ring tensor on `device`, xl_mem_fifo over it)."""
    with np.load(path, allow_pickle=False) as z:
        if str(z["format"]) != _FORMAT or str(z["kind"]) != "state":
            raise ValueError(f"{path} is not a state FIFO checkpoint")
        buf = _tensor_of(z["buf"], str(z["dtype"]), z["shape"], device)
        mlen_max, ln, head = (int(x) for x in z["ints"])
    if buf.shape[1] != mlen_max or not (0 <= ln <= mlen_max and 0 <= head < mlen_max):
        raise ValueError(f"{path}: inconsistent FIFO state")
    return buf, xl_mem_fifo(buf.data_ptr(), mlen_max, ln, head)


def save_kv_fifo(path, kv: xl_kv_fifo, k: torch.Tensor, vt: torch.Tensor) -> None:
    """Write the key ring (tensors k and vt, whose data pointers kv holds) to `path`."""
    if k.data_ptr() != kv.k or vt.data_ptr() != kv.vt:
        raise ValueError("k, vt are not the key ring's buffers")
    np.savez(path, format=np.array(_FORMAT), kind=np.array("keys"), k=_bytes_of(k), vt=_bytes_of(vt),
             dtype=np.array(str(k.dtype).replace("torch.", "")), k_shape=np.array(k.shape, np.int64),
             vt_shape=np.array(vt.shape, np.int64), ints=np.array([kv.cap, kv.mlen_max, kv.len, kv.head], np.int64))


def load_kv_fifo(path, device="cuda"):
    """Read a key ring written by save_kv_fifo: returns (k, vt on `device`, xl_kv_fifo over them)."""
    with np.load(path, allow_pickle=False) as z:
        if str(z["format"]) != _FORMAT or str(z["kind"]) != "keys":
            raise ValueError(f"{path} is not a key-ring checkpoint")
        dt = str(z["dtype"])
        k = _tensor_of(z["k"], dt, z["k_shape"], device)
        vt = _tensor_of(z["vt"], dt, z["vt_shape"], device)
        cap, mlen_max, ln, head = (int(x) for x in z["ints"])
    if k.shape[2] != cap or vt.shape[3] != cap or not (0 <= ln <= mlen_max and 0 <= head < cap):
        raise ValueError(f"{path}: inconsistent key-ring state")
    return k, vt, xl_kv_fifo(k.data_ptr(), vt.data_ptr(), cap, mlen_max, ln, head)
