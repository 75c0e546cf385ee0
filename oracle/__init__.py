"""CPU oracle of the SDM write/read forward. TEST INFRASTRUCTURE, NOT PRODUCT.

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may import or
run anything here. The product path (chunked_sparse_delta_amd) never does, and this
package shares no code with it; both take their inputs from ``workloads``.

  O1  token_loop.c      the per-token recurrence in fp64 (the definition)
  O1b token_loop.c      the same recurrence under the bfloat16 storage contract: written
                        rows rounded to bfloat16 once per chunk, readings rounded to
                        bfloat16 (token_loop(..., bf16_chunk=C))
  O2  chunk_algebra.py  the chunked three-part form in fp64, for tiny inputs
  token_loop over a [M, hd] bank: one bank shared by every stream (slot sets disjoint,
                        checked); repeated_write_slots: the pages' count of write entries
                        repeating a slot of their own token

Pins: tests/test_oracle.py checks O1 against O2 (two independent derivations),
against closed forms (decay-only, scalar EMA, one-token delta update, overwrite
under a large negative log-decay, a hand-worked rational example in tests/golden/)
and against invariants (padding, chunk-size, stream and column independence). O1b is
pinned by its rounding (ties to even, no double rounding, against an independent
float32 bit-level rounding), by its reduction to O1 with one rounding when one chunk
spans the stream, and by its equality with O1 when every value is bfloat16-exact. The
shared-bank loop is pinned to the per-stream loop on interleaved relabeled slots (equal
bit for bit, O1 and O1b), the repeat count to hand-counted tokens.
Parity unpinned: none.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import chunk_algebra  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "token_loop.c")
_LIB = os.path.join(_HERE, "libsdm_oracle.so")
_lock = threading.Lock()
_lib = None

ERRORS = {-1: "slot id out of range", -2: "write slot repeated within a token",
          -3: "bad argument", -4: "out of memory"}


def build(force: bool = False) -> str:
    """Compile token_loop.c with gcc into oracle/libsdm_oracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-fno-fast-math", "-o", tmp, _SRC, "-lm"],
                       check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            f = lib.sdm_oracle_token_loop
            i64, p = ctypes.c_int64, ctypes.c_void_p
            f.argtypes = [i64, i64, i64, i64, i64, i64, i64, i64] + [p] * 10
            f.restype = ctypes.c_int
            fb = lib.sdm_oracle_token_loop_bf16
            fb.argtypes = [i64, i64, i64, i64, i64, i64, i64, i64, i64] + [p] * 10
            fb.restype = ctypes.c_int
            fs = lib.sdm_oracle_token_loop_shared
            fs.argtypes = [i64, i64, i64, i64, i64, i64, i64, i64, i64] + [p] * 10
            fs.restype = ctypes.c_int
            lib.sdm_oracle_round_bf16.argtypes = [ctypes.c_double]
            lib.sdm_oracle_round_bf16.restype = ctypes.c_double
            _lib = lib
    return _lib


def as_f64_inputs(inputs: dict) -> dict:
    """fp64 copies of a ``workloads.generate`` dict (bank-dtype arrays widened exactly)."""
    from workloads import to_float
    dt = inputs["dtype"]
    return dict(
        bank=to_float(inputs["bank"], dt),
        k_idx=np.ascontiguousarray(inputs["k_idx"], dtype=np.int32),
        k_val=to_float(inputs["k_val"], dt),
        v=to_float(inputs["v"], dt),
        beta=np.asarray(inputs["beta"], dtype=np.float64),
        g=np.asarray(inputs["log_decay"], dtype=np.float64),
        q_idx=np.ascontiguousarray(inputs["q_idx"], dtype=np.int32),
        q_val=to_float(inputs["q_val"], dt),
        valid=np.ascontiguousarray(inputs["valid"], dtype=np.int32),
    )


def round_bf16(x) -> np.ndarray:
    """Nearest bfloat16 of each finite double (ties to even), as doubles."""
    lib = _load()
    x = np.asarray(x, dtype=np.float64)
    return np.vectorize(lib.sdm_oracle_round_bf16, otypes=[np.float64])(x) if x.size else x.copy()


def token_loop(f64: dict, threads: int = 1, streams=None, bf16_chunk: int | None = None):
    """O1 over the streams of fp64 inputs (``as_f64_inputs``). Returns (readings
    [P, T, hd], final bank) in fp64; ``streams`` restricts the work to a subset (the other
    streams' outputs are left zero / unchanged). With ``bf16_chunk`` = C it runs O1b, the
    loop under the bfloat16 storage contract for chunks of C.

    The bank is [P, M, hd] (one bank per stream) or [M, hd]: one bank for every stream
    (page 21, memory_ops.py, sdm_write_read with shared_bank=True), whose streams must
    select disjoint slots over the whole call; that contract is checked here."""
    lib = _load()
    bank = np.array(f64["bank"], dtype=np.float64, copy=True, order="C")
    shared = bank.ndim == 2
    k_idx = np.ascontiguousarray(f64["k_idx"], dtype=np.int32)
    P, T, W = k_idx.shape
    M, hd = bank.shape[-2], bank.shape[-1]
    if shared:
        _check_disjoint_streams(k_idx, f64["q_idx"], f64.get("valid"))
    R = f64["q_idx"].shape[2]
    g = np.ascontiguousarray(f64["g"], dtype=np.float64)
    G = g.shape[2]
    arrs = dict(k_val=np.ascontiguousarray(f64["k_val"], dtype=np.float64),
                v=np.ascontiguousarray(f64["v"], dtype=np.float64),
                beta=np.ascontiguousarray(f64["beta"], dtype=np.float64),
                q_idx=np.ascontiguousarray(f64["q_idx"], dtype=np.int32),
                q_val=np.ascontiguousarray(f64["q_val"], dtype=np.float64))
    valid = f64.get("valid")
    valid = None if valid is None else np.ascontiguousarray(valid, dtype=np.int32)
    out = np.zeros((P, T, hd), dtype=np.float64)
    ptr = lambda a: None if a is None else a.ctypes.data  # noqa: E731

    def run(p):
        args = (ptr(k_idx), ptr(arrs["k_val"]), ptr(arrs["v"]), ptr(arrs["beta"]), ptr(g), ptr(arrs["q_idx"]),
                ptr(arrs["q_val"]), ptr(valid), ptr(bank), ptr(out))
        if shared:
            rc = lib.sdm_oracle_token_loop_shared(p, p + 1, T, W, R, G, hd, M, int(bf16_chunk or 0), *args)
        elif bf16_chunk is None:
            rc = lib.sdm_oracle_token_loop(p, p + 1, T, W, R, G, hd, M, *args)
        else:
            rc = lib.sdm_oracle_token_loop_bf16(p, p + 1, T, W, R, G, hd, M, int(bf16_chunk), *args)
        if rc:
            raise ValueError(f"oracle: stream {p}: {ERRORS.get(rc, rc)}")

    todo = list(range(P)) if streams is None else [int(p) for p in streams]
    if threads <= 1:
        for p in todo:
            run(p)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(run, todo))
    return out, bank


def _check_disjoint_streams(k_idx, q_idx, valid) -> None:
    """Raise unless no slot is selected (written or read) by two streams over their live
    tokens: the shared-bank contract."""
    P, T = k_idx.shape[0], k_idx.shape[1]
    owner = {}
    for p in range(P):
        n = T if valid is None else int(valid[p])
        for s in set(np.asarray(k_idx[p, :n]).ravel().tolist()) | set(np.asarray(q_idx[p, :n]).ravel().tolist()):
            if owner.setdefault(int(s), p) != p:
                raise ValueError(f"oracle: slot {s} is selected by streams {owner[int(s)]} and {p} of a shared bank")


def repeated_write_slots(k_idx, valid=None) -> int:
    """The number of live write entries that repeat a slot of their own token (page 21,
    memory_ops.py, repeated_write_slots): for each live token, its W entries minus its
    distinct slots. Plain loops over the tokens."""
    k_idx = np.asarray(k_idx)
    P, T, W = k_idx.shape
    total = 0
    for p in range(P):
        n = T if valid is None else int(valid[p])
        for t in range(n):
            total += W - len(set(k_idx[p, t].tolist()))
    return total
