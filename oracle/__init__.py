"""CPU oracle of the SDM write/read forward. TEST INFRASTRUCTURE, NOT PRODUCT.

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may import or
run anything here. The product path (chunked_sparse_delta_amd) never does, and this
package shares no code with it; both take their inputs from ``workloads``.

  O1  token_loop.c      the per-token recurrence in fp64 (the definition)
  O1b token_loop.c      the same recurrence under the bfloat16 storage contract: written
                        rows rounded to bfloat16 once per chunk, readings rounded to
                        bfloat16 (token_loop(..., bf16_chunk=C))
  O2  chunk_algebra.py  the chunked three-part form in fp64, for tiny inputs
  O3  token_loop_backward.c  the gradient of O1's loop (its statements in reverse, chain
                        rule on each), fp64: token_loop_backward
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
bit for bit, O1 and O1b), the repeat count to hand-counted tokens. O3
(tests/test_backward_oracle.py) is pinned by central finite differences of O1 for every
input element, a one-token closed form, linearity in the output gradients, zero gradients
of padding tokens and the gate-width reduction (G = 1 equals the sum of G = W).
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
_SRCS = [os.path.join(_HERE, "token_loop.c"), os.path.join(_HERE, "token_loop_backward.c")]
_LIB = os.path.join(_HERE, "libsdm_oracle.so")
_lock = threading.Lock()
_lib = None

ERRORS = {-1: "slot id out of range", -2: "write slot repeated within a token",
          -3: "bad argument", -4: "out of memory"}


def build(force: bool = False) -> str:
    """Compile token_loop.c and token_loop_backward.c with gcc into oracle/libsdm_oracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < max(map(os.path.getmtime, _SRCS)):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-fno-fast-math", "-o", tmp, *_SRCS, "-lm"],
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
            fbw = lib.sdm_oracle_token_loop_backward
            fbw.argtypes = [i64, i64, i64, i64, i64, i64, i64, i64] + [p] * 17
            fbw.restype = ctypes.c_int
            fbs = lib.sdm_oracle_token_loop_backward_snap
            fbs.argtypes = [i64, i64, i64, i64, i64, i64, i64, i64] + [p] * 17 + [i64]
            fbs.restype = ctypes.c_int
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


def token_loop_backward(f64: dict, grad_out, grad_bank_final=None, threads: int = 1, streams=None,
                        snapshot_quant: str = "none") -> dict:
    """O3: the gradient of J = sum(grad_out * readings) + sum(grad_bank_final * final bank)
    through O1's loop, for fp64 inputs (``as_f64_inputs``, one bank per stream, [P, M, hd]).
    grad_out [P, T, hd]; grad_bank_final [P, M, hd] or None (zeros). Returns a dict of fp64
    gradients named like the inputs: bank [P, M, hd] (with respect to the bank the forward
    started from), k_val, v, beta, g, q_val. ``streams`` restricts the work (other streams'
    gradients stay zero). ``snapshot_quant="bf16"``: the saved rows are kept rounded to
    bfloat16 and the reverse pass works from them (the pages' bf16 snapshot of a float32
    bank)."""
    if snapshot_quant not in ("none", "bf16"):
        raise ValueError(f"oracle: snapshot_quant must be 'none' or 'bf16', got {snapshot_quant!r}")
    lib = _load()
    bank0 = np.ascontiguousarray(f64["bank"], dtype=np.float64)
    if bank0.ndim != 3:
        raise ValueError("oracle: the backward takes one bank per stream")
    k_idx = np.ascontiguousarray(f64["k_idx"], dtype=np.int32)
    P, T, W = k_idx.shape
    M, hd = bank0.shape[1], bank0.shape[2]
    q_idx = np.ascontiguousarray(f64["q_idx"], dtype=np.int32)
    R = q_idx.shape[2]
    g = np.ascontiguousarray(f64["g"], dtype=np.float64)
    G = g.shape[2]
    k_val = np.ascontiguousarray(f64["k_val"], dtype=np.float64)
    v = np.ascontiguousarray(f64["v"], dtype=np.float64)
    beta = np.ascontiguousarray(f64["beta"], dtype=np.float64)
    q_val = np.ascontiguousarray(f64["q_val"], dtype=np.float64)
    valid = f64.get("valid")
    valid = None if valid is None else np.ascontiguousarray(valid, dtype=np.int32)
    go = np.ascontiguousarray(grad_out, dtype=np.float64)
    gbf = None if grad_bank_final is None else np.ascontiguousarray(grad_bank_final, dtype=np.float64)
    if go.shape != (P, T, hd) or (gbf is not None and gbf.shape != bank0.shape):
        raise ValueError("oracle: gradient shapes do not match the inputs")
    out = dict(bank=np.zeros_like(bank0), k_val=np.zeros((P, T, W)), v=np.zeros((P, T, hd)),
               beta=np.zeros((P, T)), g=np.zeros((P, T, G)), q_val=np.zeros((P, T, R)))
    ptr = lambda a: None if a is None else a.ctypes.data  # noqa: E731

    def run(p):
        rc = lib.sdm_oracle_token_loop_backward_snap(
            p, p + 1, T, W, R, G, hd, M, ptr(k_idx), ptr(k_val), ptr(v), ptr(beta), ptr(g), ptr(q_idx),
            ptr(q_val), ptr(valid), ptr(bank0), ptr(go), ptr(gbf), ptr(out["bank"]), ptr(out["k_val"]),
            ptr(out["v"]), ptr(out["beta"]), ptr(out["g"]), ptr(out["q_val"]), 1 if snapshot_quant == "bf16" else 0)
        if rc:
            raise ValueError(f"oracle: stream {p}: {ERRORS.get(rc, rc)}")

    todo = list(range(P)) if streams is None else [int(p) for p in streams]
    if threads <= 1:
        for p in todo:
            run(p)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(run, todo))
    return out


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
