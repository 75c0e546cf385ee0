"""Seeded synthetic inputs for the chunked sparse-delta-memory (SDM) forward.

This module draws the inputs of the write/read op and nothing else: bank rows,
write/read slot ids, slot weights, write strengths, log-decays, values and the
per-stream valid-token counts. It computes no part of the op. Both sides of every
parity check (the CPU oracle and the HIP path), the benchmark and the smoke check
take their inputs from here.

Workload shapes follow the five configurations the op is specified on (one stream
up to 64 streams, chunk 16..256, head_dim 32..256, 2..256 slots per token), plus
"4p", config 4 with weights scaled by 1/sqrt(width) so that its bank stays finite
(config 4 as literally drawn grows past 1e30 within a few chunks; its timing runs
on the literal draw, its parity on 4p).

Draw recipe (numpy PCG64). Stream p of a workload takes its own child of
``SeedSequence(20261202 + index)`` (index 0..4; "4p" uses 4), and that child
spawns one generator per array in the fixed order bank, k_idx, q_idx, k_val,
q_val, beta, log_decay, v, valid. Any single stream can therefore be regenerated
alone, bit for bit.

  bank       N(0, 1) rounded to the bank dtype (round to nearest even)
  ids        W (R) distinct slots per token: i.i.d. draws with repeats discarded,
             the first W distinct values in draw order; uniform over [0, M), or a
             truncated Zipf(s) with p(i) ~ (i + 1)^-s (rank i is slot i), or half
             Zipf then half uniform (the uniform half avoids the Zipf half)
  k_val      U(0, 1) (times scale), rounded to the bank dtype; q_val likewise
  beta       sigmoid(N(0, 1)), float32, one per token
  log_decay  -a * softplus(N(mu, 1)), float32, one per write slot
  v          N(0, 1) rounded to the bank dtype
  valid      T, or uniform over the integers T/2 .. T (ragged tails)

bf16 arrays are held as their uint16 bit patterns (numpy has no bfloat16);
``to_float`` widens them.
"""

from __future__ import annotations

import dataclasses
import hashlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np

MASTER_SEED = 20261202
ARRAY_ORDER = ("bank", "k_idx", "q_idx", "k_val", "q_val", "beta", "log_decay", "v", "valid")


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int          # seed offset
    P: int              # streams
    T: int              # tokens per stream
    C: int              # chunk size
    hd: int             # head_dim
    M: int              # bank rows per stream
    dtype: str          # "f32" or "bf16"
    W: int              # write slots per token
    R: int              # read slots per token
    ids: str            # "uniform", "zipf", "mixed"
    zipf_s: float = 0.0
    decay_scale: float = 0.1    # log_decay = -decay_scale * softplus(N(decay_mu, 1))
    decay_mu: float = 0.0
    ragged: bool = False        # valid ~ U{T/2..T} per stream
    weight_scale: float = 1.0   # k_val ~ U(0,1) * scale_w / sqrt(W) when < 0 (see scales())
    gate_width: int = 0         # 0: one gate per write slot (G = W); 1: one per token

    @property
    def G(self) -> int:
        return self.W if self.gate_width == 0 else 1

    @property
    def Nt(self) -> int:
        return -(-self.T // self.C)

    def scales(self) -> tuple[float, float]:
        """(write, read) weight multipliers."""
        if self.weight_scale < 0:
            return 1.0 / np.sqrt(self.W), 1.0 / np.sqrt(self.R)
        return self.weight_scale, self.weight_scale

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "0": Workload("0", 0, P=1, T=128, C=16, hd=32, M=256, dtype="f32", W=2, R=2, ids="uniform"),
    "1": Workload("1", 1, P=8, T=2048, C=64, hd=64, M=4096, dtype="bf16", W=8, R=8, ids="uniform"),
    "2": Workload("2", 2, P=32, T=4096, C=64, hd=128, M=16384, dtype="bf16", W=32, R=32,
                  ids="zipf", zipf_s=1.1, decay_scale=1.0, decay_mu=-2.0),
    "3": Workload("3", 3, P=16, T=8192, C=128, hd=128, M=65536, dtype="f32", W=64, R=64,
                  ids="uniform", ragged=True),
    "4": Workload("4", 4, P=64, T=4096, C=256, hd=256, M=131072, dtype="bf16", W=256, R=256,
                  ids="mixed", zipf_s=1.2, decay_scale=1.0, decay_mu=-3.0),
}
CONFIGS["4p"] = CONFIGS["4"].replace(name="4p", weight_scale=-1.0)


def workload_name(wl: Workload) -> str:
    return (f"sdm_fwd_cfg{wl.name}_P{wl.P}_T{wl.T}_C{wl.C}_hd{wl.hd}_M{wl.M}_{wl.dtype}"
            f"_W{wl.W}_R{wl.R}_{wl.ids}")


# ----------------------------------------------------------------------------
# Element conversions (bf16 as uint16 bit patterns)
# ----------------------------------------------------------------------------

def round_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_float(arr: np.ndarray, dtype: str, out_dtype=np.float64) -> np.ndarray:
    """Widen a bank-dtype array (float32, or bf16 bits) to ``out_dtype``."""
    if dtype == "bf16":
        return bf16_bits_to_f32(arr).astype(out_dtype, copy=False)
    return np.asarray(arr, dtype=np.float32).astype(out_dtype, copy=False)


def _to_bank_dtype(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16_bits(x32)
    return np.ascontiguousarray(x32, dtype=np.float32)


# ----------------------------------------------------------------------------
# Slot ids
# ----------------------------------------------------------------------------

def _first_distinct(cand: np.ndarray, need: int) -> tuple[np.ndarray, np.ndarray]:
    """Per row of ``cand``, the first ``need`` distinct values in draw order.
    Returns (values [rows, need], ok [rows]); rows with too few distinct values are
    not ok (their values are garbage)."""
    rows, k = cand.shape
    order = np.argsort(cand, axis=1, kind="stable")
    srt = np.take_along_axis(cand, order, axis=1)
    dup_sorted = np.zeros((rows, k), dtype=bool)
    dup_sorted[:, 1:] = srt[:, 1:] == srt[:, :-1]
    dup = np.empty_like(dup_sorted)
    np.put_along_axis(dup, order, dup_sorted, axis=1)
    first = ~dup
    ok = first.sum(axis=1) >= need
    # position of each first occurrence among the first occurrences, in draw order
    rank = np.cumsum(first, axis=1) - 1
    take = first & (rank < need)
    vals = np.zeros((rows, need), dtype=cand.dtype)
    r_idx, c_idx = np.nonzero(take & ok[:, None])
    vals[r_idx, rank[r_idx, c_idx]] = cand[r_idx, c_idx]
    return vals, ok


def _zipf_cdf(M: int, s: float) -> np.ndarray:
    w = np.arange(1, M + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(w)
    return cdf / cdf[-1]


def _distinct_ids(rng: np.random.Generator, rows: int, width: int, M: int, kind: str,
                  zipf_s: float, cdf: np.ndarray | None) -> np.ndarray:
    if width > M:
        raise ValueError(f"{width} distinct slots per token need M >= {width}, got {M}")
    n_zipf = {"uniform": 0, "zipf": width, "mixed": width // 2}[kind]

    def draw_uniform(n, k):
        return rng.integers(0, M, size=(n, k), dtype=np.int64)

    def draw_zipf(n, k):
        u = rng.random((n, k))
        return np.minimum(np.searchsorted(cdf, u, side="right"), M - 1).astype(np.int64)

    def distinct(prefix: np.ndarray | None, need: int, draw) -> np.ndarray:
        """``need`` distinct values per row after the (already distinct) prefix columns."""
        n = rows
        pre = 0 if prefix is None else prefix.shape[1]
        out = np.empty((n, need), dtype=np.int64)
        pending = np.arange(n)
        k = need + max(4, need // 4)
        while pending.size:
            cand = draw(pending.size, k)
            if prefix is not None:
                cand = np.concatenate([prefix[pending], cand], axis=1)
            vals, ok = _first_distinct(cand, pre + need)
            out[pending[ok]] = vals[ok, pre:]
            pending = pending[~ok]
            k *= 2
        return out

    zipf_part = distinct(None, n_zipf, draw_zipf) if n_zipf else None
    if n_zipf == width:
        ids = zipf_part
    else:
        uni = distinct(zipf_part, width - n_zipf, draw_uniform)
        ids = uni if zipf_part is None else np.concatenate([zipf_part, uni], axis=1)
    return ids.astype(np.int32)


# ----------------------------------------------------------------------------
# Generator
# ----------------------------------------------------------------------------

def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def _stream_rngs(wl: Workload, p: int) -> dict:
    ss = np.random.SeedSequence(MASTER_SEED + wl.index).spawn(wl.P)[p]
    return {name: np.random.Generator(np.random.PCG64(child))
            for name, child in zip(ARRAY_ORDER, ss.spawn(len(ARRAY_ORDER)))}


def _gen_stream(wl: Workload, p: int, cdf, with_bank: bool) -> dict:
    rng = _stream_rngs(wl, p)
    T, W, R = wl.T, wl.W, wl.R
    sw, sr = wl.scales()
    out = {}
    if with_bank:
        out["bank"] = _to_bank_dtype(
            rng["bank"].standard_normal((wl.M, wl.hd), dtype=np.float32), wl.dtype)
    out["k_idx"] = _distinct_ids(rng["k_idx"], T, W, wl.M, wl.ids, wl.zipf_s, cdf)
    out["q_idx"] = _distinct_ids(rng["q_idx"], T, R, wl.M, wl.ids, wl.zipf_s, cdf)
    out["k_val"] = _to_bank_dtype((rng["k_val"].random((T, W)) * sw).astype(np.float32), wl.dtype)
    out["q_val"] = _to_bank_dtype((rng["q_val"].random((T, R)) * sr).astype(np.float32), wl.dtype)
    z = rng["beta"].standard_normal(T)
    out["beta"] = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    z = rng["log_decay"].standard_normal((T, wl.G)) + wl.decay_mu
    out["log_decay"] = (-wl.decay_scale * _softplus(z)).astype(np.float32)
    out["v"] = _to_bank_dtype(rng["v"].standard_normal((T, wl.hd), dtype=np.float32), wl.dtype)
    if wl.ragged:
        out["valid"] = np.int32(rng["valid"].integers(T // 2, T + 1))
    else:
        out["valid"] = np.int32(T)
    return out


def generate(wl: Workload, streams=None, with_bank: bool = True, threads: int = 8) -> dict:
    """Inputs of ``wl`` for ``streams`` (default: all), stacked along a leading stream axis.

    Returns a dict with bank [S, M, hd], k_idx/q_idx int32 [S, T, W|R], k_val/q_val
    [S, T, W|R], beta float32 [S, T], log_decay float32 [S, T, G], v [S, T, hd],
    valid int32 [S], plus "dtype" and "streams". Bank-dtype arrays are float32, or
    uint16 bf16 bit patterns when dtype is "bf16".
    """
    streams = list(range(wl.P)) if streams is None else [int(p) for p in streams]
    cdf = _zipf_cdf(wl.M, wl.zipf_s) if wl.ids in ("zipf", "mixed") else None
    with ThreadPoolExecutor(max_workers=max(1, min(threads, len(streams)))) as ex:
        parts = list(ex.map(lambda p: _gen_stream(wl, p, cdf, with_bank), streams))
    out = {k: np.stack([d[k] for d in parts]) for k in parts[0]}
    out["dtype"] = wl.dtype
    out["streams"] = np.asarray(streams, dtype=np.int64)
    return out


def digest(inputs: dict) -> dict:
    """sha256 of every array (for recording which inputs a run used)."""
    return {k: hashlib.sha256(np.ascontiguousarray(v).tobytes()).hexdigest()[:16]
            for k, v in inputs.items() if isinstance(v, np.ndarray)}


def small(name: str = "tiny", *, P=2, T=37, C=16, hd=8, M=24, dtype="f32", W=3, R=2,
          ids="uniform", zipf_s=1.1, decay_scale=0.1, decay_mu=0.0, ragged=False,
          weight_scale=1.0, gate_width=0, index=7) -> Workload:
    """A small workload of the same recipe for parity and edge-case tests."""
    return Workload(name, index, P=P, T=T, C=C, hd=hd, M=M, dtype=dtype, W=W, R=R, ids=ids,
                    zipf_s=zipf_s, decay_scale=decay_scale, decay_mu=decay_mu, ragged=ragged,
                    weight_scale=weight_scale, gate_width=gate_width)


def shared_bank_inputs(inputs: dict) -> dict:
    """The same work over one bank shared by every stream: local slot s of stream p becomes
    row s * P + p of a [P * M, hd] bank (streams interleaved, slot sets disjoint), ids
    relabeled to match. A pure relabeling of ``inputs`` (any dict with ``bank`` [P, M, hd],
    ``k_idx`` and ``q_idx``); the other arrays are shared, not copied."""
    bank = np.asarray(inputs["bank"])
    P, M, hd = bank.shape
    shared = np.empty((M * P, hd), dtype=bank.dtype)
    for p in range(P):
        shared[np.arange(M) * P + p] = bank[p]
    off = np.arange(P, dtype=np.int64)[:, None, None]
    out = dict(inputs)
    out["bank"] = shared
    out["k_idx"] = (np.asarray(inputs["k_idx"], dtype=np.int64) * P + off).astype(np.int32)
    out["q_idx"] = (np.asarray(inputs["q_idx"], dtype=np.int64) * P + off).astype(np.int32)
    return out


def per_stream_bank(shared: np.ndarray, P: int) -> np.ndarray:
    """[P, M, hd] view order of a bank interleaved by ``shared_bank_inputs``."""
    MP, hd = shared.shape
    return shared.reshape(MP // P, P, hd).transpose(1, 0, 2)


def grad_inputs(wl: Workload, seed: int = 0, bank_grad: bool = True) -> dict:
    """Seeded gradients to push through the backward: grad_out [P, T, hd] ~ N(0, 1) and,
    with ``bank_grad``, grad_bank [P, M, hd] ~ N(0, 1) (else None), float32."""
    rng = np.random.default_rng([wl.index, 7919, seed])
    go = rng.standard_normal((wl.P, wl.T, wl.hd), dtype=np.float32)
    gb = rng.standard_normal((wl.P, wl.M, wl.hd), dtype=np.float32) if bank_grad else None
    return dict(grad_out=go, grad_bank=gb)
