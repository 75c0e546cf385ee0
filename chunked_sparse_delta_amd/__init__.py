"""MI355X-native forward of the chunked sparse-delta-memory write/read op.

A thin ctypes binding of libsdm.so (include/sdm.h). This module marshals torch tensors
into the C ABI: it checks that shapes, dtypes and devices agree (so that the library's
pointer arguments describe the tensors it is handed), allocates the output and the
workspace with torch, and passes the current HIP stream. Every step of the computation
runs in the library's HIP kernels; there is no other path. If libsdm.so is missing or
cannot be loaded, every call raises.

    out = sdm_fwd(bank, k_idx, k_val, v, beta, log_decay, q_idx, q_val, chunk=64)

mirrors sdm_write_read's no-grad forward (memory_ops.py, sparse-delta-memory 2.0.0
wheel, diffend page 21) with per-stream banks: bank [P, M, hd] is advanced in place and
the readings [P, T, hd] are returned.

    grads = sdm_bwd(bank0, k_idx, k_val, v, beta, log_decay, q_idx, q_val, grad_out)

is the backward: the float32 gradients of sum(grad_out * readings) (plus
sum(grad_bank * final bank) when given) with respect to the bank the forward started
from and every float input.
"""

from __future__ import annotations

import ctypes
import math
import os
import threading

import torch

__all__ = ["SdmError", "sdm_fwd", "sdm_fwd_noalloc", "sdm_fwd_phase1", "sdm_fwd_phase2", "sdm_bwd", "sdm_write_read", "bwd_workspace_bytes", "chunk_mats", "chunk_records", "wy_solve", "product_key_topk", "product_key_topk_backward",
           "workspace_bytes", "plan",
           "library_path",
           "SDM_ERRORS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.environ.get("SDM_LIBRARY", os.path.join(_HERE, "libsdm.so"))

SDM_ERRORS = {0: "SDM_OK", -1: "SDM_ERR_DTYPE", -2: "SDM_ERR_SHAPE", -3: "SDM_ERR_RANGE", -4: "SDM_ERR_NULL",
              -5: "SDM_ERR_ALIGN", -6: "SDM_ERR_WORKSPACE", -7: "SDM_ERR_UNSUPPORTED", -8: "SDM_ERR_HIP"}
_DTYPES = {torch.float32: 0, torch.bfloat16: 1}


class SdmError(RuntimeError):
    """A negative return code of libsdm; ``code`` holds it, the message holds sdm_last_error()."""

    def __init__(self, code: int, msg: str):
        super().__init__(f"{SDM_ERRORS.get(code, code)}: {msg}")
        self.code = code


class _Slots(ctypes.Structure):
    _fields_ = [("write", ctypes.c_void_p), ("read", ctypes.c_void_p), ("W", ctypes.c_int32), ("R", ctypes.c_int32),
                ("write_id_bytes", ctypes.c_int32), ("read_id_bytes", ctypes.c_int32)]


class _Weights(ctypes.Structure):
    _fields_ = [("write", ctypes.c_void_p), ("read", ctypes.c_void_p)]


class _Bank(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("rows", ctypes.c_int64), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("shared", ctypes.c_int32)]


class _Exec(ctypes.Structure):
    _fields_ = [("stream", ctypes.c_void_p), ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("events", ctypes.c_void_p), ("num_events", ctypes.c_int32), ("repeated_writes", ctypes.c_void_p),
                ("phase2_cus", ctypes.c_int32)]


_ID_BYTES = {torch.int32: 4, torch.int64: 8}


TIMING_EVENTS = 8   # SDM_TIMING_EVENTS
BWD_TIMING_EVENTS = 4   # SDM_BWD_TIMING_EVENTS


_lock = threading.Lock()
_lib = None


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise RuntimeError(f"libsdm.so not found at {_LIB_PATH}: build it first "
                                   "(python -m chunked_sparse_delta_amd.build)")
            lib = ctypes.CDLL(_LIB_PATH)
            i32, i64, p, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
            lib.sdm_fwd_workspace_bytes.argtypes = [i32] * 7
            lib.sdm_fwd_workspace_bytes.restype = sz
            lib.sdm_fwd.argtypes = [i32, i32, i32, p, p, p, p, i32, p, p, p, p, p]
            for fn in (lib.sdm_fwd_phase1, lib.sdm_fwd_phase2, lib.sdm_fwd_noalloc):
                fn.argtypes = [i32, i32, i32, p, p, p, p, i32, p, p, p, p, p]
                fn.restype = ctypes.c_int
            lib.sdm_fwd.restype = ctypes.c_int
            lib.sdm_chunk_mats.argtypes = [i32, i32, i32, p, p, p, p, i32, i64, i32, i32, p, p, p, p, p, p, p, p]
            lib.sdm_chunk_mats.restype = ctypes.c_int
            lib.sdm_chunk_records.argtypes = [i32, i32, i32, p, p, p, p, i32, i64, i32, i32, p, p, p, p, p, p, p]
            lib.sdm_chunk_records.restype = ctypes.c_int
            lib.sdm_wy_solve.argtypes = [i64, i32, p, p, p, p, p, p]
            lib.sdm_wy_solve.restype = ctypes.c_int
            lib.sdm_fwd_plan.argtypes = [i32, i32, i32, i32, i32, i32, i64, i32, p]
            lib.sdm_fwd_plan.restype = ctypes.c_int
            lib.sdm_product_key_topk.argtypes = [i64, p, i32, p, i32, i32, p, p, p]
            lib.sdm_product_key_topk.restype = ctypes.c_int
            lib.sdm_product_key_topk_backward.argtypes = [i64, p, p, i32, p, i32, i32, p, p]
            lib.sdm_product_key_topk_backward.restype = ctypes.c_int
            lib.sdm_bwd_workspace_bytes.argtypes = [i32] * 5 + [i64, i32, i32, i32]
            lib.sdm_bwd_workspace_bytes.restype = ctypes.c_size_t
            lib.sdm_bwd.argtypes = [i32, i32, p, p, p, p, i32, p, p, p, p, p, i32, p]
            lib.sdm_bwd.restype = ctypes.c_int
            lib.sdm_error_string.argtypes = [ctypes.c_int]
            lib.sdm_error_string.restype = ctypes.c_char_p
            lib.sdm_last_error.argtypes = []
            lib.sdm_last_error.restype = ctypes.c_char_p
            _lib = lib
    return _lib


def _check_rc(lib, rc: int) -> None:
    if rc != 0:
        raise SdmError(rc, lib.sdm_last_error().decode(errors="replace"))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_ptr(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _expect(t: torch.Tensor, name: str, shape, dtype, device) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the bank on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def workspace_bytes(P: int, T: int, C: int, W: int, R: int, hd: int, slab_steps: int = 0) -> int:
    """Bytes of scratch sdm_fwd needs for slabs of ``slab_steps`` steps (0: all steps)."""
    return int(_load().sdm_fwd_workspace_bytes(P, T, C, W, R, hd, slab_steps))


class _Plan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("vec", "slice_vectors", "slices", "phase2_mode",
                                               "phase2_lds_bytes", "phase1_fused", "phase1_partitions_log2",
                                               "lds_limit", "lds_default", "phase2_team")]


PHASE2_MODES = ("memory", "staged", "resident")


def plan(P: int, T: int, C: int, W: int, R: int, hd: int, M: int, dtype: torch.dtype) -> dict:
    """The launch plan sdm_fwd takes for these shapes on the current device (sdm_fwd_plan)."""
    lib = _load()
    if dtype not in _DTYPES:
        raise TypeError(f"bank dtype must be float32 or bfloat16, got {dtype}")
    out = _Plan()
    _check_rc(lib, lib.sdm_fwd_plan(P, T, C, W, R, hd, M, _DTYPES[dtype], ctypes.byref(out)))
    d = {n: int(getattr(out, n)) for n, _ in _Plan._fields_}
    d["phase2_mode"] = PHASE2_MODES[d["phase2_mode"]]
    return d


def _workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator returns blocks aligned to at least 512 bytes.
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    if ws.data_ptr() % 256:
        raise RuntimeError("workspace allocation is not 256-byte aligned")
    return ws


DEFAULT_WORKSPACE_CAP = 8 << 30


def _inputs(bank, k_idx, k_val, v, beta, log_decay, q_idx, q_val, valid_tokens, shared_bank=False):
    if bank.dtype not in _DTYPES:
        raise TypeError(f"bank must be float32 or bfloat16, got {bank.dtype}")
    if k_idx.dim() != 3 or q_idx.dim() != 3:
        raise ValueError("k_idx and q_idx must be [P, T, W] and [P, T, R]")
    P, T, W = k_idx.shape
    if bank.dim() == 2:   # one bank for every stream
        if P > 1 and not shared_bank:
            raise ValueError(f"{P} streams over one bank of {bank.shape[0]} slots: pass shared_bank=True to assert "
                             "that the streams select disjoint slots for the whole call (not checked), or give "
                             "each stream its own bank [P, M, head_dim]")
        M, hd = bank.shape
        shape = (M, hd)
    elif bank.dim() == 3:
        _, M, hd = bank.shape
        shape = (P, M, hd)
    else:
        raise ValueError(f"bank must be [P, M, head_dim] or a shared [M, head_dim], got shape {tuple(bank.shape)}")
    R = q_idx.shape[2]
    G = log_decay.shape[-1] if log_decay.dim() == 3 else -1
    dev = bank.device
    if dev.type != "cuda":
        raise ValueError("bank must be a GPU tensor")
    _expect(bank, "bank", shape, bank.dtype, dev)
    for t, name, shp in ((k_idx, "k_idx", (P, T, W)), (q_idx, "q_idx", (P, T, R))):
        if t.dtype not in _ID_BYTES:
            raise TypeError(f"{name} must be int32 or int64, got {t.dtype}")
        _expect(t, name, shp, t.dtype, dev)
    _expect(k_val, "k_val", (P, T, W), bank.dtype, dev)
    _expect(q_val, "q_val", (P, T, R), bank.dtype, dev)
    _expect(v, "v", (P, T, hd), bank.dtype, dev)
    _expect(beta, "beta", (P, T), torch.float32, dev)
    _expect(log_decay, "log_decay", (P, T, G), torch.float32, dev)
    if valid_tokens is not None:
        _expect(valid_tokens, "valid_tokens", (P,), torch.int32, dev)
    slots = _Slots(k_idx.data_ptr(), q_idx.data_ptr(), W, R, _ID_BYTES[k_idx.dtype], _ID_BYTES[q_idx.dtype])
    weights = _Weights(k_val.data_ptr(), q_val.data_ptr())
    return P, M, hd, T, W, R, G, slots, weights


def sdm_fwd(bank: torch.Tensor, k_idx: torch.Tensor, k_val: torch.Tensor, v: torch.Tensor, beta: torch.Tensor,
            log_decay: torch.Tensor, q_idx: torch.Tensor, q_val: torch.Tensor, *, chunk: int = 64,
            valid_tokens: torch.Tensor | None = None, out: torch.Tensor | None = None,
            workspace: torch.Tensor | None = None, max_workspace_bytes: int = DEFAULT_WORKSPACE_CAP,
            stream=None, events=None, shared_bank: bool = False,
            repeated_writes: torch.Tensor | None = None) -> torch.Tensor:
    """SDM forward on the GPU. Returns the readings [P, T, hd] (bank dtype); ``bank``
    [P, M, hd] (one bank per stream) or [M, hd] (one bank for all streams; with P > 1 it
    needs ``shared_bank=True``, asserting disjoint slot sets) is advanced in place. Slot
    ids are int32 or int64. ``valid_tokens`` (int32 [P], on the GPU) marks the tokens at
    and past each stream's end as padding. ``workspace`` (uint8, GPU) is used if given,
    else one of at most ``max_workspace_bytes`` (at least one step) is allocated.
    ``events``: optional ctypes array of TIMING_EVENTS hipEvent_t handles recorded at the
    kernel boundaries of the first slab (see sdm_exec in include/sdm.h).
    ``repeated_writes``: optional int64 [1] GPU tensor; the call adds the number of write
    entries repeating a slot of their own token."""
    lib = _load()
    P, M, hd, T, W, R, G, slots, weights = _inputs(bank, k_idx, k_val, v, beta, log_decay, q_idx, q_val,
                                                   valid_tokens, shared_bank)
    if repeated_writes is not None:
        _expect(repeated_writes, "repeated_writes", (1,), torch.int64, bank.device)
    if out is None:
        out = torch.empty((P, T, hd), dtype=bank.dtype, device=bank.device)
    else:
        _expect(out, "out", (P, T, hd), bank.dtype, bank.device)
    if workspace is None:
        need_all = workspace_bytes(P, T, chunk, W, R, hd, 0)
        need_one = workspace_bytes(P, T, chunk, W, R, hd, 1)
        nbytes = need_all if need_all <= max_workspace_bytes else max(need_one,
                                                                      max_workspace_bytes // need_one * need_one)
        workspace = _workspace(nbytes, bank.device)
    bk = _Bank(bank.data_ptr(), M, hd, _DTYPES[bank.dtype], 1 if bank.dim() == 2 else 0)
    ex = _Exec(_stream_ptr(stream), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
               None if events is None else ctypes.cast(events, ctypes.c_void_p), 0 if events is None else len(events),
               None if repeated_writes is None else repeated_writes.data_ptr())
    rc = lib.sdm_fwd(P, T, chunk, ctypes.byref(slots), ctypes.byref(weights), _ptr(beta), _ptr(log_decay), G,
                     _ptr(v), ctypes.byref(bk), _ptr(valid_tokens), _ptr(out), ctypes.byref(ex))
    _check_rc(lib, rc)
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20   # SDM_NOALLOC_SCRATCH_BYTES


def sdm_fwd_noalloc(bank: torch.Tensor, k_idx: torch.Tensor, k_val: torch.Tensor, v: torch.Tensor,
                    beta: torch.Tensor, log_decay: torch.Tensor, q_idx: torch.Tensor, q_val: torch.Tensor, *,
                    chunk: int = 64, valid_tokens: torch.Tensor | None = None, out: torch.Tensor | None = None,
                    stream=None, events=None, shared_bank: bool = False,
                    repeated_writes: torch.Tensor | None = None) -> torch.Tensor:
    """sdm_fwd on the library's static scratch (sdm_fwd_noalloc): no workspace is allocated
    or passed; shapes whose single step needs more than NOALLOC_SCRATCH_BYTES are refused.
    ``out`` is allocated here when omitted (pass it to allocate nothing at all). Calls that
    overlap on one GPU share its scratch and race."""
    lib = _load()
    P, M, hd, T, W, R, G, slots, weights = _inputs(bank, k_idx, k_val, v, beta, log_decay, q_idx, q_val,
                                                   valid_tokens, shared_bank)
    if repeated_writes is not None:
        _expect(repeated_writes, "repeated_writes", (1,), torch.int64, bank.device)
    if out is None:
        out = torch.empty((P, T, hd), dtype=bank.dtype, device=bank.device)
    else:
        _expect(out, "out", (P, T, hd), bank.dtype, bank.device)
    bk = _Bank(bank.data_ptr(), M, hd, _DTYPES[bank.dtype], 1 if bank.dim() == 2 else 0)
    ex = _Exec(_stream_ptr(stream), None, 0,
               None if events is None else ctypes.cast(events, ctypes.c_void_p), 0 if events is None else len(events),
               None if repeated_writes is None else repeated_writes.data_ptr())
    rc = lib.sdm_fwd_noalloc(P, T, chunk, ctypes.byref(slots), ctypes.byref(weights), _ptr(beta), _ptr(log_decay),
                             G, _ptr(v), ctypes.byref(bk), _ptr(valid_tokens), _ptr(out), ctypes.byref(ex))
    _check_rc(lib, rc)
    return out


class _Grads(ctypes.Structure):
    _fields_ = [("bank", ctypes.c_void_p), ("v", ctypes.c_void_p), ("beta", ctypes.c_void_p),
                ("log_decay", ctypes.c_void_p), ("write", ctypes.c_void_p), ("read", ctypes.c_void_p)]


# snapshot_quant modes of sdm_write_read (page 21, memory_ops.py): SDM_SNAP_* of include/sdm.h
SNAPSHOT_QUANT = {"none": 0, "fp8": 1, "int4": 2, "bf16": 3}


def _snap_mode(snapshot_quant: str) -> int:
    if snapshot_quant not in SNAPSHOT_QUANT:
        raise ValueError(f"snapshot_quant must be one of {tuple(SNAPSHOT_QUANT)}, got {snapshot_quant!r}")
    return SNAPSHOT_QUANT[snapshot_quant]


def bwd_workspace_bytes(P: int, T: int, W: int, R: int, hd: int, M: int, dtype: torch.dtype = torch.float32,
                        shared_bank: bool = False, snapshot_quant: str = "none") -> int:
    """Workspace bytes sdm_bwd needs (0 for rejected shapes or snapshot modes)."""
    return int(_load().sdm_bwd_workspace_bytes(P, T, W, R, hd, M, _DTYPES.get(dtype, -1), 1 if shared_bank else 0,
                                               _snap_mode(snapshot_quant)))


def sdm_bwd(bank: torch.Tensor, k_idx: torch.Tensor, k_val: torch.Tensor, v: torch.Tensor, beta: torch.Tensor,
            log_decay: torch.Tensor, q_idx: torch.Tensor, q_val: torch.Tensor, grad_out: torch.Tensor, *,
            grad_bank: torch.Tensor | None = None, valid_tokens: torch.Tensor | None = None,
            workspace: torch.Tensor | None = None, stream=None, events=None, shared_bank: bool = False,
            snapshot_quant: str = "none") -> dict:
    """Backward of sdm_fwd. ``bank`` (float32 or bfloat16; [P, M, hd], or a shared [M, hd]
    with ``shared_bank=True``) holds the bank the forward STARTED from; a float32 bank is
    replayed and restored (exactly with ``snapshot_quant="none"``; with "bf16" its saved rows
    are bfloat16, the reverse sweep works from them, and the rows the forward wrote come back
    rounded to bfloat16), a bfloat16 one only read. "fp8" and "int4" are refused (SdmError,
    SDM_ERR_UNSUPPORTED). ``grad_out`` [P, T, hd] (bank
    dtype) is the gradient of the readings; ``grad_bank`` (float32, the bank's shape,
    optional) that of the final bank, overwritten in place with the gradient with respect
    to the initial bank (a zero tensor is allocated if omitted). ``events``: optional ctypes
    array of BWD_TIMING_EVENTS hipEvent_t recorded at the kernel boundaries. Returns
    dict(bank, v, beta, log_decay, k_val, q_val) of float32 gradients."""
    lib = _load()
    P, M, hd, T, W, R, G, slots, weights = _inputs(bank, k_idx, k_val, v, beta, log_decay, q_idx, q_val,
                                                   valid_tokens, shared_bank)
    dev = bank.device
    _expect(grad_out, "grad_out", (P, T, hd), bank.dtype, dev)
    if grad_bank is None:
        grad_bank = torch.zeros(bank.shape, dtype=torch.float32, device=dev)
    else:
        _expect(grad_bank, "grad_bank", tuple(bank.shape), torch.float32, dev)
    out = dict(bank=grad_bank, v=torch.empty((P, T, hd), dtype=torch.float32, device=dev),
               beta=torch.empty((P, T), dtype=torch.float32, device=dev),
               log_decay=torch.empty((P, T, G), dtype=torch.float32, device=dev),
               k_val=torch.empty((P, T, W), dtype=torch.float32, device=dev),
               q_val=torch.empty((P, T, R), dtype=torch.float32, device=dev))
    mode = _snap_mode(snapshot_quant)
    if workspace is None:
        need = bwd_workspace_bytes(P, T, W, R, hd, M, bank.dtype, bank.dim() == 2, snapshot_quant)
        workspace = _workspace(need if need else 256, dev)   # 0: the call itself reports why
    gr = _Grads(*(out[k].data_ptr() for k in ("bank", "v", "beta", "log_decay", "k_val", "q_val")))
    bk = _Bank(bank.data_ptr(), M, hd, _DTYPES[bank.dtype], 1 if bank.dim() == 2 else 0)
    ex = _Exec(_stream_ptr(stream), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
               None if events is None else ctypes.cast(events, ctypes.c_void_p), 0 if events is None else len(events),
               None)
    rc = lib.sdm_bwd(P, T, ctypes.byref(slots), ctypes.byref(weights), _ptr(beta), _ptr(log_decay), G, _ptr(v),
                     ctypes.byref(bk), _ptr(valid_tokens), _ptr(grad_out), ctypes.byref(gr), mode, ctypes.byref(ex))
    _check_rc(lib, rc)
    return out


class _SDMWriteRead(torch.autograd.Function):
    """sdm_fwd with sdm_bwd as its backward: the bank is state (advanced in place, no
    gradient); the float inputs get gradients. The forward keeps a copy of the bank as it
    was, which the backward replays from."""

    @staticmethod
    def forward(ctx, bank, k_val, v, beta, log_decay, q_val, k_idx, q_idx, chunk, valid_tokens, shared_bank,
                snapshot_quant):
        bank0 = bank.detach().clone()
        out = sdm_fwd(bank, k_idx, k_val.detach(), v.detach(), beta.detach(), log_decay.detach(), q_idx,
                      q_val.detach(), chunk=chunk, valid_tokens=valid_tokens, shared_bank=shared_bank)
        ctx.save_for_backward(bank0, k_val, v, beta, log_decay, q_val, k_idx, q_idx)
        ctx.valid_tokens, ctx.shared_bank, ctx.snapshot_quant = valid_tokens, shared_bank, snapshot_quant
        return out

    @staticmethod
    def backward(ctx, grad_out):
        bank0, k_val, v, beta, log_decay, q_val, k_idx, q_idx = ctx.saved_tensors
        go = grad_out.to(bank0.dtype).contiguous()
        g = sdm_bwd(bank0, k_idx, k_val.detach(), v.detach(), beta.detach(), log_decay.detach(), q_idx,
                    q_val.detach(), go, valid_tokens=ctx.valid_tokens, shared_bank=ctx.shared_bank,
                    snapshot_quant=ctx.snapshot_quant)
        need = ctx.needs_input_grad   # (bank, k_val, v, beta, log_decay, q_val, ...)
        out = [None] * 12
        for i, (name, like) in enumerate((("k_val", k_val), ("v", v), ("beta", beta), ("log_decay", log_decay),
                                          ("q_val", q_val)), start=1):
            if need[i]:
                out[i] = g[name].to(like.dtype)
        return tuple(out)


def sdm_write_read(bank: torch.Tensor, k_idx: torch.Tensor, k_val: torch.Tensor, v: torch.Tensor,
                   beta: torch.Tensor, log_decay: torch.Tensor, q_idx: torch.Tensor, q_val: torch.Tensor, *,
                   chunk: int = 64, valid_tokens: torch.Tensor | None = None,
                   shared_bank: bool = False, snapshot_quant: str = "none") -> torch.Tensor:
    """The memory op for autograd: returns the readings and advances ``bank`` in place, as
    sdm_fwd does; when grad mode is on and k_val, v, beta, log_decay or q_val requires grad,
    the readings' backward is sdm_bwd (gradients cast to the inputs' dtypes; its saved rows
    stored as ``snapshot_quant``, "none" or "bf16"). The bank is state: it receives no
    gradient here (it must not require grad); sdm_bwd gives the gradient of the initial bank
    to callers that need it. For a bfloat16 bank the backward is the derivative of the
    per-token loop at the given inputs, the forward's roundings to bfloat16 taken as the
    identity (their derivative almost everywhere in the sense that matters for training:
    the rounding is a storage format, not part of the function the loop defines)."""
    _snap_mode(snapshot_quant)
    needs = torch.is_grad_enabled() and any(t.requires_grad for t in (k_val, v, beta, log_decay, q_val))
    if bank.requires_grad:
        raise ValueError("sdm_write_read advances the bank in place: the bank must not require grad "
                         "(use sdm_bwd for the gradient of the initial bank)")
    if not needs:
        return sdm_fwd(bank, k_idx, k_val, v, beta, log_decay, q_idx, q_val, chunk=chunk,
                       valid_tokens=valid_tokens, shared_bank=shared_bank)
    return _SDMWriteRead.apply(bank, k_val, v, beta, log_decay, q_val, k_idx, q_idx, chunk, valid_tokens,
                               shared_bank, snapshot_quant)


def _fwd_part(part: int, bank, k_idx, k_val, v, beta, log_decay, q_idx, q_val, *, chunk, valid_tokens, out,
              workspace, stream, shared_bank, repeated_writes, phase2_cus=0):
    lib = _load()
    P, M, hd, T, W, R, G, slots, weights = _inputs(bank, k_idx, k_val, v, beta, log_decay, q_idx, q_val,
                                                   valid_tokens, shared_bank)
    if repeated_writes is not None:
        _expect(repeated_writes, "repeated_writes", (1,), torch.int64, bank.device)
    if out is not None:
        _expect(out, "out", (P, T, hd), bank.dtype, bank.device)
    bk = _Bank(bank.data_ptr(), M, hd, _DTYPES[bank.dtype], 1 if bank.dim() == 2 else 0)
    ex = _Exec(_stream_ptr(stream), workspace.data_ptr(), workspace.numel() * workspace.element_size(), None, 0,
               None if repeated_writes is None else repeated_writes.data_ptr(), int(phase2_cus))
    fn = lib.sdm_fwd_phase1 if part == 1 else lib.sdm_fwd_phase2
    rc = fn(P, T, chunk, ctypes.byref(slots), ctypes.byref(weights), _ptr(beta), _ptr(log_decay), G, _ptr(v),
            ctypes.byref(bk), _ptr(valid_tokens), _ptr(out), ctypes.byref(ex))
    _check_rc(lib, rc)


def sdm_fwd_phase1(bank, k_idx, k_val, v, beta, log_decay, q_idx, q_val, *, workspace: torch.Tensor, chunk: int = 64,
                   valid_tokens=None, stream=None, shared_bank: bool = False, repeated_writes=None) -> None:
    """The forward's Phase 1 and solve for every chunk into ``workspace`` (uint8, at least
    workspace_bytes(..., slab_steps=0)): reads the slot ids, weights, gates, beta and
    valid_tokens only (the bank gives its shape and dtype). Pair with sdm_fwd_phase2."""
    _fwd_part(1, bank, k_idx, k_val, v, beta, log_decay, q_idx, q_val, chunk=chunk, valid_tokens=valid_tokens,
              out=None, workspace=workspace, stream=stream, shared_bank=shared_bank, repeated_writes=repeated_writes)


def sdm_fwd_phase2(bank, k_idx, k_val, v, beta, log_decay, q_idx, q_val, *, workspace: torch.Tensor, out: torch.Tensor,
                   chunk: int = 64, valid_tokens=None, stream=None, shared_bank: bool = False,
                   phase2_cus: int = 0) -> torch.Tensor:
    """The forward's Phase 2 from a ``workspace`` filled by sdm_fwd_phase1 with the same
    arguments (ordered before this call): advances ``bank`` in place and writes ``out``;
    with the phase-1 call it gives exactly sdm_fwd's result. ``phase2_cus`` (0: all) caps
    the CUs its slice geometry plans for, leaving the rest to a Phase 1 run beside it."""
    _fwd_part(2, bank, k_idx, k_val, v, beta, log_decay, q_idx, q_val, chunk=chunk, valid_tokens=valid_tokens,
              out=out, workspace=workspace, stream=stream, shared_bank=shared_bank, repeated_writes=None,
              phase2_cus=phase2_cus)
    return out


def chunk_mats(k_idx, k_val, beta, log_decay, q_idx, q_val, *, rows: int, head_dim: int, chunk: int,
               valid_tokens=None, stream=None) -> dict:
    """Phase-1 and solve intermediates of every chunk (chunk n = p * Nt + ti): A, QK, X,
    QX float32 [P * Nt, C, C]; gw [P * Nt, C, W]; gr [P * Nt, C, R]."""
    lib = _load()
    if k_val.dtype not in _DTYPES:
        raise TypeError(f"k_val must be float32 or bfloat16, got {k_val.dtype}")
    P, T, W = k_idx.shape
    R = q_idx.shape[2]
    dev = k_idx.device
    dummy = torch.empty((P, 1, head_dim), dtype=k_val.dtype, device=dev)
    _, _, _, _, W, R, G, slots, weights = _inputs(dummy, k_idx, k_val, torch.empty((P, T, head_dim),
                                                  dtype=k_val.dtype, device=dev), beta, log_decay, q_idx, q_val,
                                                  valid_tokens)
    Nt = -(-T // chunk)
    N = P * Nt
    f = dict(dtype=torch.float32, device=dev)
    res = dict(A=torch.empty((N, chunk, chunk), **f), QK=torch.empty((N, chunk, chunk), **f),
               X=torch.empty((N, chunk, chunk), **f), QX=torch.empty((N, chunk, chunk), **f),
               gw=torch.empty((N, chunk, W), **f), gr=torch.empty((N, chunk, R), **f))
    ws = _workspace(workspace_bytes(P, T, chunk, W, R, head_dim, 1), dev)
    ex = _Exec(_stream_ptr(stream), ws.data_ptr(), ws.numel(), None, 0, None)
    rc = lib.sdm_chunk_mats(P, T, chunk, ctypes.byref(slots), ctypes.byref(weights), _ptr(beta), _ptr(log_decay), G,
                            rows, head_dim, _DTYPES[k_val.dtype], _ptr(valid_tokens), _ptr(res["A"]), _ptr(res["QK"]),
                            _ptr(res["X"]), _ptr(res["QX"]), _ptr(res["gw"]), _ptr(res["gr"]), ctypes.byref(ex))
    _check_rc(lib, rc)
    return res


def chunk_records(k_idx, k_val, beta, log_decay, q_idx, q_val, *, rows: int, head_dim: int, chunk: int,
                  valid_tokens=None, stream=None) -> dict:
    """Phase 1's integer records of every chunk (sdm_chunk_records; chunk n = p * Nt + ti):
    meta int32 [N, 8], spk and grec int32 [N, C * W, 4], ecr int32 [N, C, W, 4], rcr int32
    [N, C, R, 4] (formats in include/sdm.h)."""
    lib = _load()
    if k_val.dtype not in _DTYPES:
        raise TypeError(f"k_val must be float32 or bfloat16, got {k_val.dtype}")
    P, T, W = k_idx.shape
    R = q_idx.shape[2]
    dev = k_idx.device
    dummy = torch.empty((P, 1, head_dim), dtype=k_val.dtype, device=dev)
    _, _, _, _, W, R, G, slots, weights = _inputs(dummy, k_idx, k_val, torch.empty((P, T, head_dim),
                                                  dtype=k_val.dtype, device=dev), beta, log_decay, q_idx, q_val,
                                                  valid_tokens)
    N = P * (-(-T // chunk))
    i = dict(dtype=torch.int32, device=dev)
    res = dict(meta=torch.empty((N, 8), **i), spk=torch.empty((N, chunk * W, 4), **i),
               grec=torch.empty((N, chunk * W, 4), **i), ecr=torch.empty((N, chunk, W, 4), **i),
               rcr=torch.empty((N, chunk, R, 4), **i))
    ws = _workspace(workspace_bytes(P, T, chunk, W, R, head_dim, 1), dev)
    ex = _Exec(_stream_ptr(stream), ws.data_ptr(), ws.numel(), None, 0, None)
    rc = lib.sdm_chunk_records(P, T, chunk, ctypes.byref(slots), ctypes.byref(weights), _ptr(beta), _ptr(log_decay),
                               G, rows, head_dim, _DTYPES[k_val.dtype], _ptr(valid_tokens), _ptr(res["meta"]),
                               _ptr(res["spk"]), _ptr(res["grec"]), _ptr(res["ecr"]), _ptr(res["rcr"]),
                               ctypes.byref(ex))
    _check_rc(lib, rc)
    return res


def wy_solve(A: torch.Tensor, beta: torch.Tensor, QK: torch.Tensor, stream=None):
    """X = (I + tril(beta[:, None] * A, -1))^-1 and QX = QK @ X per chunk (A, QK [n, C, C]
    float32, beta [n, C] float32, all on the GPU)."""
    lib = _load()
    if A.dim() != 3 or A.shape[1] != A.shape[2] or QK.shape != A.shape:
        raise ValueError(f"A and QK must be [n, C, C], got {tuple(A.shape)} and {tuple(QK.shape)}")
    n, C, _ = A.shape
    for t, name, shape in ((A, "A", (n, C, C)), (QK, "QK", (n, C, C)), (beta, "beta", (n, C))):
        _expect(t, name, shape, torch.float32, A.device)
    X = torch.empty_like(A)
    QX = torch.empty_like(A)
    ex = _Exec(_stream_ptr(stream), None, 0, None, 0, None)
    rc = lib.sdm_wy_solve(n, C, _ptr(A), _ptr(beta), _ptr(QK), _ptr(X), _ptr(QX), ctypes.byref(ex))
    _check_rc(lib, rc)
    return X, QX


def product_key_topk(raw: torch.Tensor, factors, k: int, stream=None):
    """Exact top-k over all sums of one value from each product-key factor
    (sdm_product_key_topk). raw [..., sum(factors)] float32 or bfloat16 on the GPU.
    Returns (val [..., kk] in raw's dtype, lin [..., kk] int64 ascending),
    kk = min(k, prod(factors))."""
    lib = _load()
    if raw.dtype not in _DTYPES:
        raise TypeError(f"raw must be float32 or bfloat16, got {raw.dtype}")
    factors = [int(f) for f in factors]
    D = sum(factors)
    if raw.dim() < 1 or raw.shape[-1] != D:
        raise ValueError(f"raw must be [..., {D}] for factors {factors}, got {tuple(raw.shape)}")
    if raw.device.type != "cuda" or not raw.is_contiguous():
        raise ValueError("raw must be a contiguous GPU tensor")
    kk = min(int(k), math.prod(factors)) if factors else 0
    lead = tuple(raw.shape[:-1])
    rows = math.prod(lead) if lead else 1
    val = torch.empty(lead + (max(kk, 0),), dtype=raw.dtype, device=raw.device)
    lin = torch.empty(lead + (max(kk, 0),), dtype=torch.int64, device=raw.device)
    fac = (ctypes.c_int32 * max(1, len(factors)))(*factors)
    ex = _Exec(_stream_ptr(stream), None, 0, None, 0, None)
    _check_rc(lib, lib.sdm_product_key_topk(rows, _ptr(raw), _DTYPES[raw.dtype], fac, len(factors), int(k), _ptr(val),
                                            _ptr(lin), ctypes.byref(ex)))
    return val, lin


def product_key_topk_backward(lin: torch.Tensor, grad_val: torch.Tensor, factors, stream=None) -> torch.Tensor:
    """The gradient with respect to raw of product_key_topk's values
    (sdm_product_key_topk_backward): lin [..., kk] int64 and grad_val [..., kk] (float32 or
    bfloat16) on the GPU. Returns grad_raw [..., sum(factors)] in grad_val's dtype."""
    lib = _load()
    if grad_val.dtype not in _DTYPES:
        raise TypeError(f"grad_val must be float32 or bfloat16, got {grad_val.dtype}")
    factors = [int(f) for f in factors]
    if lin.dtype != torch.int64 or lin.shape != grad_val.shape or lin.device != grad_val.device:
        raise ValueError("lin must be int64 with grad_val's shape and device")
    if grad_val.device.type != "cuda" or not (lin.is_contiguous() and grad_val.is_contiguous()):
        raise ValueError("lin and grad_val must be contiguous GPU tensors")
    lead, kk = tuple(lin.shape[:-1]), int(lin.shape[-1])
    rows = math.prod(lead) if lead else 1
    graw = torch.empty(lead + (sum(factors),), dtype=grad_val.dtype, device=grad_val.device)
    fac = (ctypes.c_int32 * max(1, len(factors)))(*factors)
    ex = _Exec(_stream_ptr(stream), None, 0, None, 0, None)
    _check_rc(lib, lib.sdm_product_key_topk_backward(rows, _ptr(lin), _ptr(grad_val), _DTYPES[grad_val.dtype], fac,
                                                     len(factors), kk, _ptr(graw), ctypes.byref(ex)))
    return graw
