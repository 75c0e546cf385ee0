"""A float32 evaluation of the bfloat16 storage contract: a noise model for the bf16 bars.

Not an oracle and not an expected value: the tests compare the HIP path with the fp64
oracle (O1, and O1b = O1 under the contract). This module answers a different question:
how far from O1b may a *correct* float32 evaluation of the contract land, row by row?
It runs the per-token loop of the SDMWriteRead docstring (memory_ops.py, sparse-delta-
memory 2.0.0 wheel, diffend page 21) in float32 arithmetic, keeping the bank in float32
inside a chunk and rounding every row written in the chunk to bfloat16 (nearest, ties to
even) at the chunk's end and at the stream's last live token, with each reading rounded to
bfloat16 (the storage contract of phase2_kernels.py's docstring, page 23). Its per-row
distance from O1b measures how much one-ulp bfloat16 rounding flips, which any float32
implementation makes somewhere, grow into by the end of the call.

Vectorized across streams (one numpy step per token), so that a whole workload of tens
of streams runs in seconds.
"""

from __future__ import annotations

import numpy as np


def _round_bf16_f32(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 of each float32 (ties to even), as float32; NaN and inf kept."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32)
    return np.where(np.isfinite(x), out, x).astype(np.float32)


def token_loop_contract_f32(inp: dict, C: int):
    """Readings [P, T, hd] and final bank [P, M, hd] (float32) of ``workloads.generate``
    inputs with a bfloat16 bank, per-stream banks, distinct write slots per token."""
    from workloads import to_float
    dt = inp["dtype"]
    B = to_float(inp["bank"], dt, np.float32).copy()
    P, M, hd = B.shape
    k_idx = np.asarray(inp["k_idx"], dtype=np.int64)
    q_idx = np.asarray(inp["q_idx"], dtype=np.int64)
    T, W = k_idx.shape[1], k_idx.shape[2]
    kv = to_float(inp["k_val"], dt, np.float32)
    qv = to_float(inp["q_val"], dt, np.float32)
    v = to_float(inp["v"], dt, np.float32)
    beta = np.asarray(inp["beta"], dtype=np.float32)
    g = np.asarray(inp["log_decay"], dtype=np.float32)
    G = g.shape[2]
    valid = np.asarray(inp["valid"], dtype=np.int64)
    out = np.zeros((P, T, hd), dtype=np.float32)
    pr = np.arange(P)[:, None]
    touched = np.zeros((P, M), dtype=bool)
    for t in range(T):
        live = t < valid
        if not live.any():
            break
        lp = np.nonzero(live)[0]
        ks = k_idx[lp, t]                                   # [p, W]
        gam = np.exp(g[lp, t] if G == W else np.repeat(g[lp, t], W, axis=1)).astype(np.float32)
        read = B[lp[:, None], ks] * gam[..., None]          # [p, W, hd]
        ret = np.einsum("pw,pwh->ph", kv[lp, t], read, dtype=np.float32)
        delta = beta[lp, t, None] * (v[lp, t] - ret)
        B[lp[:, None], ks] = read + kv[lp, t][..., None] * delta[:, None, :]
        touched[lp[:, None], ks] = True
        rows = B[lp[:, None], q_idx[lp, t]]
        out[lp, t] = _round_bf16_f32(np.einsum("pr,prh->ph", qv[lp, t], rows, dtype=np.float32))
        # chunk end (or a stream's last live token): round the rows written in the chunk
        end = ((t + 1) % C == 0) | (t + 1 == valid)
        for p in np.nonzero(end & live)[0]:
            s = np.nonzero(touched[p])[0]
            B[p, s] = _round_bf16_f32(B[p, s])
            touched[p, s] = False
    del pr
    return out, B


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per row (last axis) infinity-norm relative error, for rows of ref that are not all
    zero; shape = the leading axes flattened, restricted to those rows."""
    g = got.reshape(-1, got.shape[-1]).astype(np.float64)
    r = ref.reshape(-1, ref.shape[-1]).astype(np.float64)
    scale = np.max(np.abs(r), axis=1)
    keep = scale > 0
    return np.max(np.abs(g[keep] - r[keep]), axis=1) / scale[keep]
