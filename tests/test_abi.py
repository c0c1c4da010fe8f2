"""The C ABI on the CPU: the library loads, exports every entry point the
header declares, and rejects invalid arguments on the host before anything is
launched (no GPU needed: every call below fails validation)."""
import ctypes
import os
import re
import subprocess

import pytest

import transformer_xl_relative_amd as xl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "xl_rel.h")

FAKE = [0x7F0000000000 + i * 0x100000000 for i in range(16)]   # distinct, never dereferenced


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(xl_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_expected_entry_points():
    fns = header_functions()
    for f in ("xl_relpos_embed", "xl_rel_attn_fwd", "xl_rel_attn_core", "xl_segment_step"):
        assert f in fns
    assert set(fns) == set(xl.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = xl.lib()
    for f in header_functions():
        assert hasattr(lib, f), f
    nm = subprocess.run(["nm", "-D", "--defined-only", xl.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r" T (xl_\w+)", nm))
    assert set(header_functions()) <= exported


def test_status_strings():
    lib = xl.lib()
    assert lib.xl_status_string(0) == b"ok"
    assert lib.xl_status_string(4) == b"workspace too small"
    assert lib.xl_status_string(99) == b"unknown status"


def _desc(**over):
    kw = dict(batch=2, d_model=512, n_head=8, d_head=64, qlen=128, mlen=128, dtype=xl.XL_BF16)
    kw.update(over)
    return xl.make_desc(**kw)


def _weights(bias=False):
    return xl.xl_attn_weights(*FAKE[:7], FAKE[7] if bias else None)


def _fwd(desc, w=None, h=FAKE[8], mem=FAKE[9], out=FAKE[10], ws=FAKE[11], ws_bytes=1 << 40):
    w = _weights() if w is None else w
    return xl.lib().xl_rel_attn_fwd(ctypes.byref(desc) if desc is not None else None, ctypes.byref(w), h, mem, out,
                                    ws, ws_bytes, None)


@pytest.mark.parametrize("over,status", [
    (dict(d_head=32), xl.XL_UNSUPPORTED),
    (dict(dtype=xl.XL_F32), xl.XL_UNSUPPORTED),          # f32 supports d_head 8 only
    (dict(d_model=511), xl.XL_BAD_SHAPE),
    (dict(d_model=40), xl.XL_UNSUPPORTED),               # bf16 needs a multiple of 32
    (dict(qlen=0), xl.XL_BAD_SHAPE),
    (dict(batch=0), xl.XL_BAD_SHAPE),
    (dict(mlen=-1), xl.XL_BAD_SHAPE),
    (dict(dtype=7), xl.XL_BAD_SHAPE),
    (dict(out_dtype=9), xl.XL_BAD_SHAPE),
    (dict(base=-1.0), xl.XL_BAD_SHAPE),
    (dict(scale=float("inf")), xl.XL_BAD_SHAPE),
    (dict(qlen=1 << 30), xl.XL_UNSUPPORTED),
    (dict(bias_clamp=128, mlen=20000, qlen=200), xl.XL_UNSUPPORTED),   # LDS bias table limit
    (dict(attn_splits=-1), xl.XL_BAD_SHAPE),
    (dict(attn_splits=65), xl.XL_BAD_SHAPE),
    (dict(bias_kind=2), xl.XL_BAD_SHAPE),
    (dict(bias_kind=-1, bias_clamp=4), xl.XL_BAD_SHAPE),
    (dict(flags=2), xl.XL_BAD_SHAPE),                    # unknown flag bit
])
def test_fwd_rejects_bad_descriptors(over, status):
    assert _fwd(_desc(**over)) == status
    assert xl.lib().xl_last_error() != b""


def test_fwd_rejects_null_and_alias_and_small_workspace():
    lib = xl.lib()
    assert _fwd(None) == xl.XL_NULL_ARG
    assert _fwd(_desc(), mem=None) == xl.XL_NULL_ARG                       # mlen > 0 needs mem
    assert _fwd(_desc(bias_clamp=16)) == xl.XL_NULL_ARG                    # table missing
    w = _weights()
    w.w_o = None
    assert _fwd(_desc(), w=w) == xl.XL_NULL_ARG
    assert _fwd(_desc(), out=FAKE[8]) == xl.XL_BAD_SHAPE                   # out aliases h
    d = _desc()
    need = xl.xl_rel_attn_workspace_size(d)
    assert _fwd(d, ws_bytes=need - 1) == xl.XL_WORKSPACE_TOO_SMALL
    assert b"needs" in lib.xl_last_error()
    assert _fwd(d, ws=FAKE[11] + 8, ws_bytes=need + 8) == xl.XL_UNSUPPORTED  # misaligned workspace


def test_workspace_size_formula():
    for kw in (dict(), dict(clamp_len=100), dict(mlen=0, qlen=37), dict(dtype=xl.XL_F32, d_head=8, d_model=16)):
        d = _desc(**kw)
        lay = xl.xl_rel_attn_workspace_layout(d)
        B, H, dh, q, m, D = d.batch, d.n_head, d.d_head, d.qlen, d.mlen, d.d_model
        es = 2 if d.dtype == xl.XL_BF16 else 4
        klen = q + m
        ldv = (klen + 63) // 64 * 64
        n_rel = klen if d.clamp_len < 0 else min(klen, d.clamp_len + 1)
        a = lambda x: (x + 255) // 256 * 256
        sizes = [B * H * q * dh, B * H * klen * dh, B * H * dh * ldv, n_rel * D, H * n_rel * dh, B * q * H * dh]
        # the split attention's partials come last (none for f32 and for the shapes that are not split)
        part = xl.xl_rel_attn_core_workspace_size(d)
        assert lay.part == sum(a(s * es) for s in sizes)
        assert lay.total == lay.part + a(part)
        if d.dtype == xl.XL_F32:
            assert part == 0
        assert (lay.klen, lay.ldv, lay.n_rel) == (klen, ldv, n_rel)
        assert xl.xl_rel_attn_workspace_size(d) == lay.total
        offs = [lay.q, lay.k, lay.vt, lay.rel, lay.r, lay.attn]
        assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert xl.xl_rel_attn_workspace_size(_desc(d_head=16)) == 0


def test_split_workspace():
    # long memory, one query tile per head: the library splits the keys and
    # needs S * B*H*qlen * (d_head + 2) floats of partials, S in [2, 64]
    d = _desc(batch=1, n_head=2, qlen=64, mlen=1600)
    per = d.batch * d.n_head * d.qlen * (d.d_head + 2) * 4
    need = xl.xl_rel_attn_core_workspace_size(d)
    assert need % per == 0 and 2 <= need // per <= 64
    lay = xl.xl_rel_attn_workspace_layout(d)
    assert lay.part % 256 == 0 and lay.total == lay.part + (need + 255) // 256 * 256
    # a forced count, and no split at all
    assert xl.xl_rel_attn_core_workspace_size(_desc(batch=1, n_head=2, qlen=64, mlen=1600, attn_splits=5)) == 5 * per
    assert xl.xl_rel_attn_core_workspace_size(_desc(attn_splits=1)) == 0
    # f32 never splits
    assert xl.xl_rel_attn_core_workspace_size(_desc(dtype=xl.XL_F32, d_head=8, d_model=16, attn_splits=7)) == 0
    assert xl.xl_rel_attn_core_workspace_size(_desc(attn_splits=99)) == 0      # invalid descriptor


def test_workspace_grows_with_memory():
    # a workspace sized for the longest memory serves every shorter one: the
    # split partials are sized for any memory length
    for kw in (dict(batch=4, n_head=8, qlen=64, d_model=512), dict(batch=1, n_head=2, qlen=64, d_model=128)):
        sizes = [xl.xl_rel_attn_workspace_size(_desc(mlen=m, **kw)) for m in range(0, 2100, 8)]
        assert all(a <= b for a, b in zip(sizes, sizes[1:])), kw
        core = [xl.xl_rel_attn_core_workspace_size(_desc(mlen=m, **kw)) for m in range(0, 2100, 8)]
        assert all(a <= b for a, b in zip(core, core[1:])), kw
    dec = [xl.xl_decoder_stack_workspace_size(_desc(batch=2, n_head=8, qlen=64, d_model=256, mlen=m), 1024)
           for m in range(1800, 2100, 8)]
    assert all(a <= b for a, b in zip(dec, dec[1:]))
    # the key-ring stack and step likewise (their memory lengths are the rings' lens)
    for fn in (lambda d: xl.xl_decoder_stack_kv_workspace_size(d, 1024), xl.xl_segment_step_kv_workspace_size):
        kv = [fn(_desc(batch=2, n_head=8, qlen=64, d_model=256, mlen=m)) for m in range(0, 2100, 8)]
        assert all(0 < a <= b for a, b in zip(kv, kv[1:]))


def test_core_rejects_bad_arguments():
    lib = xl.lib()
    d = _desc()
    klen = d.qlen + d.mlen
    call = lambda ldv, n_rel, bias=None, desc=d, ws=None, nb=0: lib.xl_rel_attn_core(
        ctypes.byref(desc), *FAKE[:3], ldv, FAKE[5], n_rel, FAKE[13], FAKE[14], bias, FAKE[6], ws, nb, None)
    assert call(klen - 8, klen) == xl.XL_BAD_SHAPE            # ldv < klen
    assert call(klen + 4, klen) == xl.XL_BAD_SHAPE            # ldv not a multiple of 8
    assert call(klen, klen - 1) == xl.XL_BAD_SHAPE            # r too short
    assert call(klen, klen, desc=_desc(bias_clamp=4)) == xl.XL_NULL_ARG
    assert lib.xl_rel_attn_core(ctypes.byref(d), None, *FAKE[1:3], klen, FAKE[5], klen, FAKE[13], FAKE[14], None,
                                FAKE[6], None, 0, None) == xl.XL_NULL_ARG
    assert lib.xl_rel_attn_core(ctypes.byref(d), *FAKE[:3], klen, FAKE[5], klen, None, FAKE[14], None,
                                FAKE[6], None, 0, None) == xl.XL_NULL_ARG      # u missing
    # a split needs its workspace: missing, too small, misaligned, aliasing the output
    ds = _desc(attn_splits=3)
    need = xl.xl_rel_attn_core_workspace_size(ds)
    assert need > 0
    assert call(klen, klen, desc=ds) == xl.XL_NULL_ARG
    assert call(klen, klen, desc=ds, ws=FAKE[12], nb=need - 1) == xl.XL_WORKSPACE_TOO_SMALL
    assert call(klen, klen, desc=ds, ws=FAKE[12] + 16, nb=need) == xl.XL_UNSUPPORTED
    assert call(klen, klen, desc=ds, ws=FAKE[6], nb=need) == xl.XL_BAD_SHAPE


def test_segment_step_rejects_bad_fifo():
    lib = xl.lib()
    d = _desc(mlen=0)
    w = _weights()
    step = lambda fifo, h=FAKE[8]: lib.xl_segment_step(ctypes.byref(d), ctypes.byref(w), h,
                                                       ctypes.byref(fifo) if fifo is not None else None,
                                                       FAKE[10], FAKE[11], 1 << 40, None)
    assert step(None) == xl.XL_NULL_ARG
    assert step(xl.xl_mem_fifo(None, 128, 0, 0)) == xl.XL_NULL_ARG
    assert step(xl.xl_mem_fifo(FAKE[12], 128, 129, 0)) == xl.XL_BAD_SHAPE     # len > mlen_max
    assert step(xl.xl_mem_fifo(FAKE[12], 128, 0, 128)) == xl.XL_BAD_SHAPE     # head out of range
    assert step(xl.xl_mem_fifo(FAKE[12], 0, 0, 0)) == xl.XL_BAD_SHAPE
    assert step(xl.xl_mem_fifo(FAKE[12], 128, 10, 3), h=FAKE[12] + 64) == xl.XL_BAD_SHAPE  # h inside the ring
    f = xl.xl_mem_fifo(FAKE[12], 128, 10, 3)
    assert lib.xl_segment_step(ctypes.byref(d), ctypes.byref(w), FAKE[8], ctypes.byref(f), FAKE[10], FAKE[11],
                               16, None) == xl.XL_WORKSPACE_TOO_SMALL
    assert (f.len, f.head) == (10, 3)                                           # untouched on error


def test_segment_step_noalloc_rejects_before_any_launch():
    # host checks of the allocation-free step: bad fifo, bad shapes, and a step
    # whose workspace would exceed the static scratch; the fifo stays untouched
    lib = xl.lib()
    w = _weights()
    step = lambda d, fifo: lib.xl_segment_step_noalloc(ctypes.byref(d), ctypes.byref(w), FAKE[8],
                                                       ctypes.byref(fifo) if fifo is not None else None,
                                                       FAKE[10], None)
    d = _desc(mlen=0)
    assert step(d, None) == xl.XL_NULL_ARG
    assert step(d, xl.xl_mem_fifo(FAKE[12], 128, 129, 0)) == xl.XL_BAD_SHAPE
    big = _desc(mlen=0, batch=64, d_model=1024, n_head=16, qlen=1024)
    f = xl.xl_mem_fifo(FAKE[12], 1024, 1024, 5)
    ws_need = lib.xl_rel_attn_workspace_size(ctypes.byref(_desc(mlen=1024, batch=64, d_model=1024, n_head=16,
                                                                qlen=1024)))
    assert ws_need > xl.XL_NOALLOC_SCRATCH_BYTES
    assert step(big, f) == xl.XL_WORKSPACE_TOO_SMALL
    assert b"allocation-free" in lib.xl_last_error()
    assert (f.len, f.head) == (1024, 5)


def test_segment_step_kv_rejects_bad_ring():
    lib = xl.lib()
    d = _desc(mlen=0)                       # qlen 128
    w = _weights()
    K, VT = FAKE[12], FAKE[13]

    def step(kv, desc=d, h=FAKE[8], out=FAKE[10], nb=1 << 40):
        return lib.xl_segment_step_kv(ctypes.byref(desc), ctypes.byref(w), h,
                                      ctypes.byref(kv) if kv is not None else None, out, FAKE[11], nb, None)
    ok = lambda **kw: xl.xl_kv_fifo(**{**dict(k=K, vt=VT, cap=256, mlen_max=128, len=64, head=8), **kw})
    assert step(None) == xl.XL_NULL_ARG
    assert step(ok(k=None)) == xl.XL_NULL_ARG
    assert step(ok(cap=200)) == xl.XL_BAD_SHAPE                 # cap < mlen_max + qlen
    assert step(ok(len=136)) == xl.XL_BAD_SHAPE                 # len > mlen_max
    assert step(ok(head=256)) == xl.XL_BAD_SHAPE                # head out of range
    assert step(ok(head=4)) == xl.XL_UNSUPPORTED                # not a multiple of 8
    assert step(ok(cap=260)) == xl.XL_UNSUPPORTED
    assert step(ok(), desc=_desc(mlen=0, qlen=100)) == xl.XL_UNSUPPORTED     # qlen not a multiple of 8
    assert step(ok(), desc=_desc(mlen=0, dtype=xl.XL_F32, d_head=8, d_model=16)) == xl.XL_UNSUPPORTED
    assert step(ok(), h=K + 64) == xl.XL_BAD_SHAPE              # h inside the key ring
    assert step(ok(vt=K + 4096)) == xl.XL_BAD_SHAPE             # the two rings overlap
    kv = ok()
    assert step(kv, nb=16) == xl.XL_WORKSPACE_TOO_SMALL
    assert (kv.len, kv.head) == (64, 8)                          # untouched on error
    # the ring workspace drops the k and v^T regions of the layer workspace
    dl = _desc(mlen=64)
    full, lay = xl.xl_rel_attn_workspace_size(dl), xl.xl_rel_attn_workspace_layout(dl)
    assert xl.xl_segment_step_kv_workspace_size(dl) == full - (lay.rel - lay.k)
    assert xl.xl_segment_step_kv_workspace_size(_desc(dtype=xl.XL_F32, d_head=8, d_model=16)) == 0


def test_relpos_rejects_bad_arguments():
    lib = xl.lib()
    assert lib.xl_relpos_embed(0, 4, 7, -1, 10000.0, xl.XL_F32, FAKE[0], None) == xl.XL_BAD_SHAPE
    assert lib.xl_relpos_embed(0, -1, 8, -1, 10000.0, xl.XL_F32, FAKE[0], None) == xl.XL_BAD_SHAPE
    assert lib.xl_relpos_embed(0, 4, 8, -1, -2.0, xl.XL_F32, FAKE[0], None) == xl.XL_BAD_SHAPE
    assert lib.xl_relpos_embed(0, 4, 8, -1, 10000.0, 5, FAKE[0], None) == xl.XL_BAD_SHAPE
    assert lib.xl_relpos_embed(0, 4, 8, -1, 10000.0, xl.XL_F32, None, None) == xl.XL_NULL_ARG
    assert lib.xl_relpos_embed(0, 0, 8, -1, 10000.0, xl.XL_F32, None, None) == xl.XL_OK   # nothing to do


def _dec_weights(bias=False, **over):
    f = dict(ln1_g=FAKE[1], ln1_b=FAKE[2], ln2_g=FAKE[3], ln2_b=FAKE[4], w1=FAKE[5], b1=FAKE[6], w2=FAKE[7],
             b2=FAKE[13])
    f.update(over)
    return xl.xl_decoder_weights(_weights(bias), *[f[k] for k in ("ln1_g", "ln1_b", "ln2_g", "ln2_b", "w1", "b1",
                                                                  "w2", "b2")])


def test_decoder_layer_rejects_bad_arguments():
    lib = xl.lib()

    def call(desc=None, d_inner=2048, eps=0.0, w=None, h=FAKE[8], mem=FAKE[9], out=FAKE[10], ws=FAKE[11],
             nb=1 << 40):
        desc = _desc() if desc is None else desc
        w = _dec_weights() if w is None else w
        return lib.xl_decoder_layer_fwd(ctypes.byref(desc), d_inner, eps, ctypes.byref(w), h, mem, out, ws, nb,
                                        None)
    assert call(w=_dec_weights(w2=None)) == xl.XL_NULL_ARG
    assert call(w=_dec_weights(ln1_g=None)) == xl.XL_NULL_ARG
    assert call(desc=_desc(flags=xl.XL_REUSE_TABLE)) == xl.XL_UNSUPPORTED   # layers share the workspace
    assert call(d_inner=0) == xl.XL_BAD_SHAPE
    assert call(d_inner=100) == xl.XL_BAD_SHAPE                  # not a multiple of 32
    assert call(eps=-1.0) == xl.XL_BAD_SHAPE
    assert call(eps=float("nan")) == xl.XL_BAD_SHAPE
    assert call(w=_dec_weights(b1=FAKE[6] + 8)) == xl.XL_UNSUPPORTED   # misaligned bias
    assert call(h=FAKE[8] + 2) == xl.XL_UNSUPPORTED
    assert call(out=FAKE[8]) == xl.XL_BAD_SHAPE                  # out aliases h
    assert call(h=None) == xl.XL_NULL_ARG
    assert call(nb=16) == xl.XL_WORKSPACE_TOO_SMALL
    assert call(ws=FAKE[11] + 16) == xl.XL_UNSUPPORTED           # workspace alignment
    d = _desc()
    need = xl.xl_decoder_layer_workspace_size(d, 2048)
    assert need > xl.xl_rel_attn_workspace_size(d)
    assert call(nb=need - 1) == xl.XL_WORKSPACE_TOO_SMALL
    assert xl.xl_decoder_layer_workspace_size(_desc(qlen=0), 2048) == 0


def test_decoder_stack_rejects_bad_arguments():
    lib = xl.lib()
    d = _desc(mlen=128)

    def call(n=2, fifos=None, w=None, h=FAKE[8], out=FAKE[10], nb=1 << 40, d_inner=2048):
        fifos = fifos if fifos is not None else (xl.xl_mem_fifo * 2)(xl.xl_mem_fifo(FAKE[12], 128, 64, 0),
                                                                     xl.xl_mem_fifo(FAKE[14], 128, 64, 0))
        w = w if w is not None else (xl.xl_decoder_weights * 2)(*[_dec_weights() for _ in range(2)])
        return lib.xl_decoder_stack_step(ctypes.byref(d), d_inner, 0.0, n, w, h, fifos, out, FAKE[11], nb, None)
    assert call(n=0) == xl.XL_BAD_SHAPE
    two = lambda a, b: (xl.xl_mem_fifo * 2)(a, b)
    assert call(fifos=two(xl.xl_mem_fifo(FAKE[12], 128, 129, 0), xl.xl_mem_fifo(FAKE[14], 128, 0, 0))) == \
        xl.XL_BAD_SHAPE                                              # len > mlen_max
    assert call(fifos=two(xl.xl_mem_fifo(FAKE[12], 256, 200, 0), xl.xl_mem_fifo(FAKE[14], 256, 0, 0))) == \
        xl.XL_BAD_SHAPE                                              # len > desc->mlen
    assert call(fifos=two(xl.xl_mem_fifo(FAKE[12], 128, 64, 0), xl.xl_mem_fifo(FAKE[12] + 4096, 128, 64, 0))) == \
        xl.XL_BAD_SHAPE                                              # rings overlap
    assert call(h=FAKE[14] + 64) == xl.XL_BAD_SHAPE                  # h inside a ring
    assert call(out=FAKE[8]) == xl.XL_BAD_SHAPE                      # out aliases h
    assert call(d_inner=48) == xl.XL_BAD_SHAPE
    fifos = two(xl.xl_mem_fifo(FAKE[12], 128, 64, 5), xl.xl_mem_fifo(FAKE[14], 128, 64, 7))
    assert call(fifos=fifos, nb=16) == xl.XL_WORKSPACE_TOO_SMALL
    assert [(f.len, f.head) for f in fifos] == [(64, 5), (64, 7)]    # untouched on error
    need = xl.xl_decoder_stack_workspace_size(d, 2048)
    assert need > xl.xl_decoder_layer_workspace_size(d, 2048)
    assert call(fifos=fifos, nb=need - 1) == xl.XL_WORKSPACE_TOO_SMALL


def test_decoder_stack_kv_rejects_bad_arguments():
    lib = xl.lib()
    d = _desc(mlen=128)
    MIB = 1 << 20
    ring = lambda base, **kw: xl.xl_kv_fifo(**{**dict(k=base, vt=base + MIB, cap=256, mlen_max=128, len=64, head=8),
                                               **kw})
    two = lambda a, b: (xl.xl_kv_fifo * 2)(a, b)

    def call(n=2, rings=None, h=FAKE[8], out=FAKE[10], nb=1 << 40, d_inner=2048, desc=d):
        rings = rings if rings is not None else two(ring(FAKE[12]), ring(FAKE[14]))
        w = (xl.xl_decoder_weights * 2)(*[_dec_weights() for _ in range(2)])
        return lib.xl_decoder_stack_step_kv(ctypes.byref(desc), d_inner, 0.0, n, w, h, rings, out, FAKE[11], nb, None)
    assert call(n=0) == xl.XL_BAD_SHAPE
    assert call(desc=_desc(mlen=128, dtype=xl.XL_F32, d_head=8)) == xl.XL_UNSUPPORTED       # bf16 only
    assert call(rings=two(ring(FAKE[12], len=136), ring(FAKE[14]))) == xl.XL_BAD_SHAPE      # len > mlen_max
    assert call(rings=two(ring(FAKE[12], mlen_max=256, cap=512, len=200), ring(FAKE[14]))) == \
        xl.XL_BAD_SHAPE                                                                     # len > desc->mlen
    assert call(rings=two(ring(FAKE[12], cap=160), ring(FAKE[14]))) == xl.XL_BAD_SHAPE      # cap < mlen_max + qlen
    assert call(rings=two(ring(FAKE[12], head=4), ring(FAKE[14]))) == xl.XL_UNSUPPORTED     # head not a multiple of 8
    assert call(rings=two(ring(FAKE[12]), ring(FAKE[12] + 4096))) == xl.XL_BAD_SHAPE        # rings overlap
    assert call(rings=two(ring(FAKE[12], vt=FAKE[12] + 4096), ring(FAKE[14]))) == xl.XL_BAD_SHAPE   # k aliases vt
    assert call(h=FAKE[14] + 64) == xl.XL_BAD_SHAPE                                          # h inside a ring
    assert call(out=FAKE[8]) == xl.XL_BAD_SHAPE                                              # out aliases h
    assert call(d_inner=48) == xl.XL_BAD_SHAPE
    rings = two(ring(FAKE[12], head=16), ring(FAKE[14], head=24))
    assert call(rings=rings, nb=16) == xl.XL_WORKSPACE_TOO_SMALL
    assert [(r.len, r.head) for r in rings] == [(64, 16), (64, 24)]                          # untouched on error
    need = xl.xl_decoder_stack_kv_workspace_size(d, 2048)
    # no normalised memory rows and no k or vt regions: smaller than the state-FIFO stack's
    assert 0 < need < xl.xl_decoder_stack_workspace_size(d, 2048)
    assert call(rings=rings, nb=need - 1) == xl.XL_WORKSPACE_TOO_SMALL
    assert xl.xl_decoder_stack_kv_workspace_size(_desc(dtype=xl.XL_F32, d_head=8), 2048) == 0


def test_core_backward_rejects_bad_arguments():
    lib = xl.lib()
    d = _desc(mlen=64, qlen=64)
    klen = 128
    need = xl.xl_rel_attn_core_bwd_workspace_size(d)
    rows = 2 * 8 * 64   # batch x heads x qlen
    # P and dS, dq_u and dq_v, the dr partials (batch x heads x (klen - 1) rows), the row stats
    assert need == 2 * (rows * klen * 4) + 2 * (rows * 64 * 4) + 2 * 8 * (klen - 1) * 64 * 4 + rows * 3 * 4

    def call(ldv=klen, n_rel=klen, bias=None, dbias=None, desc=d, ws=FAKE[15], nb=need, dq=FAKE[9], dk=FAKE[10]):
        return lib.xl_rel_attn_core_bwd(ctypes.byref(desc), FAKE[0], FAKE[1], FAKE[2], ldv, FAKE[3], n_rel, FAKE[4],
                                        FAKE[5], bias, FAKE[6], dq, dk, FAKE[11], FAKE[12], FAKE[13], FAKE[14], dbias,
                                        ws, nb, None)
    assert call(ldv=klen - 8) == xl.XL_BAD_SHAPE
    assert call(ldv=klen + 4) == xl.XL_BAD_SHAPE          # not a multiple of 8
    assert call(n_rel=klen - 1) == xl.XL_BAD_SHAPE
    assert call(dq=None) == xl.XL_NULL_ARG
    assert call(desc=_desc(mlen=64, qlen=64, bias_clamp=4), bias=FAKE[7]) == xl.XL_NULL_ARG   # no dbias
    assert call(nb=need - 1) == xl.XL_WORKSPACE_TOO_SMALL
    assert call(ws=None) == xl.XL_WORKSPACE_TOO_SMALL
    assert call(ws=FAKE[15] + 16) == xl.XL_UNSUPPORTED
    assert call(dq=FAKE[0]) == xl.XL_BAD_SHAPE            # dq aliases q
    assert call(dk=FAKE[9] + 64) == xl.XL_BAD_SHAPE       # dk overlaps dq
    assert xl.xl_rel_attn_core_bwd_workspace_size(_desc(qlen=0)) == 0


BIG = 1 << 62   # a product of two such sizes overflows int64


@pytest.mark.parametrize("field", ["batch", "n_head", "qlen", "mlen", "d_model"])
def test_huge_sizes_rejected_without_overflow(field):
    # every caller size is bounded on its own before any product of sizes is
    # formed; the sanitizer run of this file catches a product that overflows
    lib = xl.lib()
    d = _desc(**{field: BIG})
    assert _fwd(d) == xl.XL_UNSUPPORTED
    assert xl.xl_rel_attn_workspace_size(d) == 0
    assert xl.xl_rel_attn_core_workspace_size(d) == (0 if field != "d_model" else
                                                    xl.xl_rel_attn_core_workspace_size(_desc()))
    assert xl.xl_rel_attn_core_bwd_workspace_size(d) == (0 if field != "d_model" else
                                                        xl.xl_rel_attn_core_bwd_workspace_size(_desc()))
    assert xl.xl_decoder_layer_workspace_size(d, 2048) == 0
    assert xl.xl_decoder_stack_workspace_size(d, 2048) == 0
    if field != "mlen":   # the segment step takes its memory length from the FIFO
        ds = _desc(mlen=0, **{field: BIG})
        f = xl.xl_mem_fifo(FAKE[12], 128, 0, 0)
        assert lib.xl_segment_step(ctypes.byref(ds), ctypes.byref(_weights()), FAKE[8], ctypes.byref(f), FAKE[10],
                                   FAKE[11], 1 << 40, None) == xl.XL_UNSUPPORTED


def test_huge_fifo_and_ring_rejected_without_overflow():
    lib = xl.lib()
    w = _weights()
    d = _desc(mlen=0, batch=1 << 20)
    # batch x mlen_max rows beyond the 32-bit row range
    f = xl.xl_mem_fifo(FAKE[12], 1 << 20, 0, 0)
    assert lib.xl_segment_step(ctypes.byref(d), ctypes.byref(w), FAKE[8], ctypes.byref(f), FAKE[10], FAKE[11],
                               1 << 40, None) == xl.XL_UNSUPPORTED
    assert b"mlen_max" in lib.xl_last_error()
    f = xl.xl_mem_fifo(FAKE[12], BIG, 0, 0)
    assert lib.xl_segment_step(ctypes.byref(d), ctypes.byref(w), FAKE[8], ctypes.byref(f), FAKE[10], FAKE[11],
                               1 << 40, None) == xl.XL_UNSUPPORTED
    # key ring: mlen_max + qlen would overflow; batch x cap beyond the row range
    for kw in (dict(mlen_max=(1 << 63) - 8, cap=256), dict(mlen_max=128, cap=BIG)):
        kv = xl.xl_kv_fifo(**{**dict(k=FAKE[12], vt=FAKE[13], len=0, head=0), **kw})
        assert lib.xl_segment_step_kv(ctypes.byref(_desc(mlen=0)), ctypes.byref(w), FAKE[8], ctypes.byref(kv),
                                      FAKE[10], FAKE[11], 1 << 40, None) == xl.XL_UNSUPPORTED
    kv = xl.xl_kv_fifo(k=FAKE[12], vt=FAKE[13], cap=1 << 16, mlen_max=128, len=0, head=0)
    assert lib.xl_segment_step_kv(ctypes.byref(d), ctypes.byref(w), FAKE[8], ctypes.byref(kv), FAKE[10], FAKE[11],
                                  1 << 40, None) == xl.XL_UNSUPPORTED
    # decoder: d_inner far beyond the feed-forward's limit
    assert xl.xl_decoder_layer_workspace_size(_desc(), BIG) == 0
    assert xl.xl_decoder_stack_workspace_size(_desc(), BIG) == 0
    # the plain backward's score matrix beyond 2^40 elements
    db = _desc(batch=4096, n_head=16, qlen=8192, mlen=0)   # 2^42 scores
    assert xl.xl_rel_attn_core_bwd_workspace_size(db) == 0


def test_key_count_limit_boundary():
    # the largest key count per head the kernels' 32-bit K offsets allow is
    # accepted, one more key is refused
    klen_max = (2 ** 31 - 1) // 128
    ok = _desc(batch=1, n_head=1, qlen=64, mlen=klen_max - 64)
    assert xl.xl_rel_attn_core_workspace_size(ok) > 0
    assert xl.xl_rel_attn_core_workspace_size(_desc(batch=1, n_head=1, qlen=64, mlen=klen_max - 63)) == 0


def test_bias_table_context_boundary():
    # with a bias table the kernel keeps one value per distance in LDS: the
    # longest context it takes is accepted, one more key is refused
    kmax = 80 * 1024 // 4 - 384
    assert xl.xl_rel_attn_core_workspace_size(_desc(batch=1, n_head=1, qlen=64, mlen=kmax - 64, bias_clamp=8)) > 0
    assert xl.xl_rel_attn_core_workspace_size(_desc(batch=1, n_head=1, qlen=64, mlen=kmax - 63, bias_clamp=8)) == 0


def test_width_limit_boundaries():
    # d_model and n_head * d_head up to 65536 are accepted, one step more is refused
    size = lambda **kw: xl.xl_rel_attn_workspace_size(_desc(batch=1, qlen=64, mlen=64, **kw))
    assert size(d_model=65536, n_head=1) > 0
    assert size(d_model=65536 + 32, n_head=1) == 0
    assert size(d_model=64, n_head=1024) > 0
    assert size(d_model=64, n_head=1025) == 0


def test_tensor_size_bound():
    # within every per-size limit, but with 2^45 key elements: refused before
    # any product of sizes could overflow the projection launches' tile counts
    d = _desc(batch=32, n_head=1024, d_model=64, qlen=64, mlen=(2 ** 31 - 1) // 128 - 64)
    assert _fwd(d) == xl.XL_UNSUPPORTED
    assert b"2^40" in xl.lib().xl_last_error()
    assert xl.xl_rel_attn_core_workspace_size(d) == 0
