"""The C ABI on the host: the library loads, exports every function include/sdm.h
declares, and rejects malformed calls with the documented code before any device work
(no GPU needed: rejected calls never touch a HIP API)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdm.h")
LIB = os.path.join(ROOT, "chunked_sparse_delta_amd", "libsdm.so")

OK, DTYPE, SHAPE, RANGE, NULL, ALIGN, WORKSPACE, UNSUPPORTED, HIP = 0, -1, -2, -3, -4, -5, -6, -7, -8


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sdm_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from chunked_sparse_delta_amd import build
        build.build()
    return ctypes.CDLL(LIB)


def test_header_declares_the_boundary():
    assert declared_functions() == ["sdm_bwd", "sdm_bwd_workspace_bytes", "sdm_chunk_mats", "sdm_chunk_records",
                                    "sdm_error_string",
                                    "sdm_fwd", "sdm_fwd_noalloc", "sdm_fwd_phase1", "sdm_fwd_phase2", "sdm_fwd_plan",
                                    "sdm_fwd_workspace_bytes", "sdm_last_error", "sdm_product_key_topk",
                                    "sdm_product_key_topk_backward", "sdm_wy_solve"]


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_error_strings(lib):
    lib.sdm_error_string.restype = ctypes.c_char_p
    for code in (OK, DTYPE, SHAPE, RANGE, NULL, ALIGN, WORKSPACE, UNSUPPORTED, HIP):
        assert lib.sdm_error_string(code) and lib.sdm_error_string(code) != b"unknown error"
    assert lib.sdm_error_string(-99) == b"unknown error"


def test_workspace_bytes(lib):
    f = lib.sdm_fwd_workspace_bytes
    f.restype = ctypes.c_size_t
    one = f(8, 2048, 64, 8, 8, 64, 1)
    step = f(8, 2048, 64, 8, 8, 64, 2) - one             # one step of chunks
    assert one == step > 0 and step % 256 == 0
    assert f(8, 2048, 64, 8, 8, 64, 0) == one + 31 * step    # Nt = 32 steps
    assert f(8, 2048, 64, 8, 8, 64, 5) == one + 4 * step
    assert f(8, 2048, 64, 8, 8, 64, 999) == one + 31 * step
    assert f(8, 2048, 8, 8, 8, 64, 0) == 0                # chunk out of range
    assert f(8, 2048, 64, 0, 8, 64, 0) == 0               # W < 1
    assert f(8, 2048, 64, 8, 257, 64, 0) == 0             # R > 256
    # 112 B per write entry, 24 B per read entry, 16 B per chunk-matrix element, a slot
    # search index of about one word per write entry (a power of two, at most 2^14), 20 B
    # per possible group of >= 16 members, the three dense hot operands [C][HCAP]
    # (HCAP = that count rounded up to 16, at most 512), 64 words of counts and team words,
    # and the Phase-2 team exchange of u and inter, 2 x C x head_dim (rounded up to 64)
    # floats (+ alignment)
    per_chunk = step / 8
    E, F, C2, C, hd = 64 * 8, 64 * 8, 64 * 64, 64, 64
    NB = 512
    hmax = E // 16 + 1
    hcap = min(512, (hmax + 15) // 16 * 16)
    base = (112 * E + 24 * F + 16 * C2 + 4 * (NB + 1) + 20 * hmax + 12 * C * hcap + 4 * 64
            + 8 * C * ((hd + 63) // 64 * 64))
    assert base <= per_chunk <= base + 40 * 256


class Call:
    """A well-formed sdm_fwd call on fake (never dereferenced) aligned pointers."""

    FAKE = 0x7f0000000000

    def __init__(self, lib):
        self.lib = lib
        lib.sdm_last_error.restype = ctypes.c_char_p
        self.P, self.T, self.C, self.W, self.R, self.G, self.hd, self.M = 2, 100, 32, 4, 3, 4, 64, 50
        self.dtype = 0
        self.ws_bytes = None
        self.kb, self.qb, self.shared, self.rep = 4, 4, 0, None
        self.ptr = {k: self.FAKE + (i << 32) for i, k in enumerate(
            ["kidx", "qidx", "kval", "qval", "beta", "g", "v", "bank", "out", "ws", "valid"])}

    def run(self):
        from chunked_sparse_delta_amd import _Bank, _Exec, _Slots, _Weights
        lib = self.lib
        lib.sdm_fwd.argtypes = [ctypes.c_int32] * 3 + [ctypes.c_void_p] * 4 + [ctypes.c_int32] + [ctypes.c_void_p] * 5
        slots = _Slots(self.ptr["kidx"], self.ptr["qidx"], self.W, self.R, self.kb, self.qb)
        weights = _Weights(self.ptr["kval"], self.ptr["qval"])
        bank = _Bank(self.ptr["bank"], self.M, self.hd, self.dtype, self.shared)
        lib.sdm_fwd_workspace_bytes.restype = ctypes.c_size_t
        need = lib.sdm_fwd_workspace_bytes(self.P, self.T, self.C, self.W, self.R, self.hd, 0)
        ex = _Exec(None, self.ptr["ws"], need if self.ws_bytes is None else self.ws_bytes, None, 0, self.rep)
        rc = lib.sdm_fwd(self.P, self.T, self.C, ctypes.byref(slots), ctypes.byref(weights), self.ptr["beta"],
                         self.ptr["g"], self.G, self.ptr["v"], ctypes.byref(bank), self.ptr["valid"],
                         self.ptr["out"], ctypes.byref(ex))
        return rc, lib.sdm_last_error().decode()


@pytest.mark.parametrize("field,value,code", [
    ("P", 0, SHAPE), ("T", 0, SHAPE), ("C", 15, RANGE), ("C", 257, RANGE), ("W", 0, SHAPE), ("W", 257, SHAPE),
    ("R", 0, SHAPE), ("R", 300, SHAPE), ("G", 2, SHAPE), ("hd", 0, SHAPE), ("hd", (1 << 20) + 1, RANGE),
    ("M", 0, SHAPE), ("M", 1 << 30, RANGE), ("dtype", 2, DTYPE), ("ws_bytes", 1024, WORKSPACE),
    ("kb", 2, DTYPE), ("qb", 16, DTYPE), ("shared", 2, SHAPE),
])
def test_fwd_rejects_before_any_work(lib, field, value, code):
    c = Call(lib)
    setattr(c, field, value)
    rc, msg = c.run()
    assert rc == code, msg
    assert msg


@pytest.mark.parametrize("name", ["kidx", "qidx", "kval", "qval", "beta", "g", "v", "bank", "out", "ws"])
def test_fwd_rejects_null(lib, name):
    c = Call(lib)
    c.ptr[name] = None
    rc, msg = c.run()
    assert rc == (WORKSPACE if name == "ws" else NULL), msg


@pytest.mark.parametrize("name,off,dtype", [("kidx", 2, 0), ("beta", 1, 0), ("bank", 2, 0), ("v", 1, 1),
                                           ("ws", 16, 0), ("valid", 2, 0)])
def test_fwd_rejects_misaligned(lib, name, off, dtype):
    c = Call(lib)
    c.dtype = dtype
    c.ptr[name] += off
    rc, msg = c.run()
    assert rc == ALIGN, msg


@pytest.mark.parametrize("name,off,kb", [("kidx", 4, 8), ("qidx", 4, 8)])
def test_fwd_rejects_misaligned_int64_ids(lib, name, off, kb):
    c = Call(lib)
    c.kb = c.qb = kb
    c.ptr[name] += off
    rc, msg = c.run()
    assert rc == ALIGN, msg


def test_fwd_rejects_misaligned_repeat_counter(lib):
    c = Call(lib)
    c.rep = Call.FAKE + 4
    rc, msg = c.run()
    assert rc == ALIGN, msg


def test_fwd_rejects_out_overlapping_bank(lib):
    c = Call(lib)
    c.ptr["out"] = c.ptr["bank"] + 256
    rc, msg = c.run()
    assert rc == SHAPE and "overlap" in msg


def test_noalloc_rejects_before_any_work(lib):
    """sdm_fwd_noalloc takes no workspace (a non-NULL one is refused) and refuses shapes
    whose single step needs more than its static scratch, both before any HIP call."""
    from chunked_sparse_delta_amd import NOALLOC_SCRATCH_BYTES, _Bank, _Exec, _Slots, _Weights
    lib.sdm_fwd_noalloc.argtypes = [ctypes.c_int32] * 3 + [ctypes.c_void_p] * 4 + [ctypes.c_int32] + \
        [ctypes.c_void_p] * 5
    lib.sdm_fwd_workspace_bytes.restype = ctypes.c_size_t
    c = Call(lib)

    def call(P, T, C, W, R, ws, ws_bytes):
        slots = _Slots(c.ptr["kidx"], c.ptr["qidx"], W, R, 4, 4)
        weights = _Weights(c.ptr["kval"], c.ptr["qval"])
        bank = _Bank(c.ptr["bank"], c.M, c.hd, 0, 0)
        ex = _Exec(None, ws, ws_bytes, None, 0, None)
        rc = lib.sdm_fwd_noalloc(P, T, C, ctypes.byref(slots), ctypes.byref(weights), c.ptr["beta"], c.ptr["g"], W,
                                 c.ptr["v"], ctypes.byref(bank), c.ptr["valid"], c.ptr["out"], ctypes.byref(ex))
        return rc, lib.sdm_last_error().decode()

    rc, msg = call(2, 100, 32, 4, 3, c.ptr["ws"], 1 << 20)
    assert rc == WORKSPACE and "static scratch" in msg
    assert lib.sdm_fwd_workspace_bytes(8, 256, 256, 256, 256, 64, 1) > NOALLOC_SCRATCH_BYTES
    rc, msg = call(8, 256, 256, 256, 256, None, 0)
    assert rc == WORKSPACE and "static scratch" in msg
    rc, msg = call(2, 100, 32, 0, 3, None, 0)
    assert rc == SHAPE, msg


def test_fwd_rejects_too_many_token_rows(lib):
    c = Call(lib)
    c.P, c.T, c.C = 4096, 1 << 20, 256
    rc, _ = c.run()
    assert rc == RANGE


def test_wy_solve_rejects(lib):
    from chunked_sparse_delta_amd import _Exec
    f = lib.sdm_wy_solve
    f.argtypes = [ctypes.c_int64, ctypes.c_int32] + [ctypes.c_void_p] * 6
    ex = _Exec(None, None, 0, None, 0)
    fake = Call.FAKE
    assert f(4, 0, fake, fake, fake, fake, fake, ctypes.byref(ex)) == RANGE
    assert f(4, 257, fake, fake, fake, fake, fake, ctypes.byref(ex)) == RANGE
    assert f(-1, 16, fake, fake, fake, fake, fake, ctypes.byref(ex)) == SHAPE
    assert f(4, 16, None, fake, fake, fake, fake, ctypes.byref(ex)) == NULL
    assert f(4, 16, fake + 2, fake, fake, fake, fake, ctypes.byref(ex)) == ALIGN
    assert f(0, 16, None, None, None, None, None, ctypes.byref(ex)) == OK   # nothing to do
    assert f(4, 16, fake, fake, fake, fake, fake, None) == NULL


def test_plan_rejects_before_any_device_query(lib):
    from chunked_sparse_delta_amd import _Plan
    f = lib.sdm_fwd_plan
    f.argtypes = [ctypes.c_int32] * 6 + [ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p]
    pl = _Plan()
    assert f(8, 2048, 64, 8, 8, 64, 4096, 1, None) == NULL
    assert f(0, 2048, 64, 8, 8, 64, 4096, 1, ctypes.byref(pl)) == SHAPE
    assert f(8, 2048, 8, 8, 8, 64, 4096, 1, ctypes.byref(pl)) == RANGE
    assert f(8, 2048, 64, 8, 8, 64, 4096, 7, ctypes.byref(pl)) == DTYPE
    assert f(8, 2048, 64, 8, 8, 64, 0, 1, ctypes.byref(pl)) == RANGE


def test_topk_rejects_before_any_launch(lib):
    from chunked_sparse_delta_amd import _Exec
    f = lib.sdm_product_key_topk
    f.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    ex = _Exec(None, None, 0, None, 0, None)
    fake = Call.FAKE

    def call(rows=4, dtype=0, factors=(16, 16), k=8, raw=fake, val=fake, lin=fake, e=ex):
        fa = (ctypes.c_int32 * len(factors))(*factors)
        return f(rows, raw, dtype, fa, len(factors), k, val, lin, None if e is None else ctypes.byref(e))

    assert call(e=None) == NULL
    assert call(dtype=3) == DTYPE
    assert call(rows=-1) == SHAPE
    assert call(factors=()) == SHAPE and call(factors=(2,) * 9) == SHAPE
    assert call(factors=(16, 0)) == SHAPE
    assert call(k=0) == SHAPE and call(k=257) == SHAPE
    assert call(factors=(65536, 2)) == UNSUPPORTED
    assert call(factors=(4096,) * 5) == UNSUPPORTED         # 2^60 slots
    assert call(raw=None) == NULL and call(lin=None) == NULL
    assert call(raw=fake + 2) == ALIGN and call(dtype=1, raw=fake + 1) == ALIGN and call(lin=fake + 4) == ALIGN
    assert call(rows=0, raw=None, val=None, lin=None) == OK


def test_topk_backward_rejects_before_any_launch(lib):
    from chunked_sparse_delta_amd import _Exec
    f = lib.sdm_product_key_topk_backward
    f.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                  ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    ex = _Exec(None, None, 0, None, 0, None)
    fake = Call.FAKE

    def call(rows=4, lin=fake, g=fake, dtype=0, factors=(16, 16), kk=8, out=fake, e=ex):
        fa = (ctypes.c_int32 * len(factors))(*factors)
        return f(rows, lin, g, dtype, fa, len(factors), kk, out, None if e is None else ctypes.byref(e))

    assert call(e=None) == NULL and call(dtype=5) == DTYPE and call(rows=-1) == SHAPE
    assert call(kk=0) == SHAPE and call(kk=257) == SHAPE and call(factors=(2, 3), kk=7) == SHAPE
    assert call(factors=(65536,)) == UNSUPPORTED and call(lin=None) == NULL
    assert call(lin=fake + 4) == ALIGN and call(dtype=1, g=fake + 1) == ALIGN
    assert call(rows=0, lin=None, g=None, out=None) == OK


def test_bwd_workspace_bytes(lib):
    """Saved rows (4 * W * hd bytes per token), folded read slots (8 * R per token), the
    per-slice dots (4 * (2W + R + 1) per token and column slice), a flag per token pair,
    each 256-byte aligned, and for a bfloat16 bank its float32 working rows. Config 1's shapes take 4-column slices
    (8 streams x 16 slices = 128 workgroups)."""
    f = lib.sdm_bwd_workspace_bytes
    f.restype = ctypes.c_size_t
    f.argtypes = [ctypes.c_int32] * 5 + [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    snap, lead, part, pairs = 8 * 16 * 4 * 2048 * 8 * 4, 8 * 2048 * 8 * 8, 8 * 16 * 2048 * 25 * 4, 8 * 1024 * 4
    base = snap + lead + part + pairs
    NONE, FP8, INT4, BF16 = 0, 1, 2, 3
    assert f(8, 2048, 8, 8, 64, 4096, 0, 0, NONE) == base
    assert f(8, 2048, 8, 8, 64, 4096, 1, 0, NONE) == base + 8 * 4096 * 64 * 4
    assert f(8, 2048, 8, 8, 64, 4096, 1, 1, NONE) == base + 4096 * 64 * 4
    # bfloat16 snapshot rows halve the saved rows of a float32 bank; a bfloat16 bank runs it as none
    assert f(8, 2048, 8, 8, 64, 4096, 0, 0, BF16) == base - snap // 2
    assert f(8, 2048, 8, 8, 64, 4096, 1, 0, BF16) == f(8, 2048, 8, 8, 64, 4096, 1, 0, NONE)
    assert f(8, 2048, 8, 8, 64, 4096, 0, 0, FP8) == 0 and f(8, 2048, 8, 8, 64, 4096, 0, 0, INT4) == 0
    assert f(8, 2048, 8, 8, 64, 4096, 0, 0, 4) == 0 and f(8, 2048, 8, 8, 64, 4096, 0, 0, -1) == 0
    assert f(0, 2048, 8, 8, 64, 4096, 0, 0, NONE) == 0 and f(8, 2048, 0, 8, 64, 4096, 0, 0, NONE) == 0
    assert f(8, 2048, 8, 257, 64, 4096, 0, 0, NONE) == 0 and f(8, 2048, 8, 8, 64, 0, 0, 0, NONE) == 0
    assert f(8, 2048, 8, 8, 64, 4096, 2, 0, NONE) == 0 and f(8, 2048, 8, 8, 64, 4096, 0, 2, NONE) == 0


def test_bwd_rejects_before_any_work(lib):
    from chunked_sparse_delta_amd import _Bank, _Exec, _Grads, _Slots, _Weights
    lib.sdm_last_error.restype = ctypes.c_char_p
    f = lib.sdm_bwd
    f.argtypes = [ctypes.c_int32, ctypes.c_int32] + [ctypes.c_void_p] * 4 + [ctypes.c_int32] + [ctypes.c_void_p] * 5 + \
        [ctypes.c_int32, ctypes.c_void_p]
    lib.sdm_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.sdm_bwd_workspace_bytes.argtypes = [ctypes.c_int32] * 5 + [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                                                   ctypes.c_int32]
    fake = Call.FAKE
    P, T, W, R, hd, M = 2, 100, 4, 3, 64, 50
    ptr = {k: fake + (i << 32) for i, k in enumerate(["kidx", "qidx", "kval", "qval", "beta", "g", "v", "bank", "go",
                                                      "ws", "gbank", "gv", "gbeta", "gg", "gk", "gq"])}

    def call(dtype=0, shared=0, ws=None, gbank=None, gv=None, G=W, kb=4, go=None, snap=0):
        need = lib.sdm_bwd_workspace_bytes(P, T, W, R, hd, M, dtype if dtype in (0, 1) else 0, shared & 1,
                                           snap if snap in (0, 3) else 0)
        slots = _Slots(ptr["kidx"], ptr["qidx"], W, R, kb, 4)
        weights = _Weights(ptr["kval"], ptr["qval"])
        bank = _Bank(ptr["bank"], M, hd, dtype, shared)
        grads = _Grads(ptr["gbank"] if gbank is None else gbank, ptr["gv"] if gv is None else gv, ptr["gbeta"],
                       ptr["gg"], ptr["gk"], ptr["gq"])
        ex = _Exec(None, ptr["ws"], need if ws is None else ws(need), None, 0, None)
        return f(P, T, ctypes.byref(slots), ctypes.byref(weights), ptr["beta"], ptr["g"], G, ptr["v"],
                 ctypes.byref(bank), None, ptr["go"] if go is None else go, ctypes.byref(grads), snap, ctypes.byref(ex))

    assert call(dtype=2) == DTYPE and call(shared=2) == SHAPE
    assert call(ws=lambda n: n - 1) == WORKSPACE and call(dtype=1, ws=lambda n: n - 256) == WORKSPACE
    assert call(gv=0) == NULL and call(gv=ptr["gv"] + 2) == ALIGN
    assert call(gbank=ptr["bank"] + 64) == SHAPE and call(go=ptr["bank"] + 64) == SHAPE
    assert call(dtype=1, go=ptr["go"] + 1) == ALIGN
    assert call(G=2) == SHAPE and call(kb=3) == DTYPE
    # snapshot modes: fp8 and int4 refused, unknown values are bad arguments; bf16 rows take
    # half the saved-row bytes of a float32 bank (a workspace one byte short is refused)
    assert call(snap=1) == UNSUPPORTED and call(snap=2) == UNSUPPORTED
    assert call(snap=4) == SHAPE and call(snap=-1) == SHAPE
    assert call(snap=3, ws=lambda n: n - 1) == WORKSPACE
