"""Helpers of the GPU tests: move generator inputs to the GPU, run the HIP path through
the C ABI binding, compare against the oracle."""

from __future__ import annotations

import numpy as np
import torch

import workloads

TOL = {"f32": 1e-4, "bf16": 2e-2}   # infinity-norm relative error per output tensor, vs O1
# bf16 banks are also compared with O1b, the token loop under the bfloat16 storage
# contract (rows rounded once per chunk, readings rounded). The GPU must stay within
# bar = max(TOL, SLACK x |O1b - O1|) of O1: the contract itself can exceed TOL on a bank
# that grows by many orders of magnitude. Against O1b: within TOL_CONTRACT where the
# contract meets TOL (SLACK x |O1b - O1| <= TOL); where it does not, one-ulp bf16 rounding
# differences between two correct evaluations of the contract (fp32 chunked on the GPU,
# fp64 token loop in O1b) compound to the contract's own error, and the bound is the
# triangle inequality through the exact result, bar + |O1b - O1|.
TOL_CONTRACT = 2e-2
SLACK = 1.25


def to_torch(inp: dict, device) -> dict:
    dt = inp["dtype"]

    def bank_dtype(a):
        if dt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)

    return dict(
        bank=bank_dtype(inp["bank"]), k_idx=torch.from_numpy(inp["k_idx"]).to(device),
        q_idx=torch.from_numpy(inp["q_idx"]).to(device), k_val=bank_dtype(inp["k_val"]),
        q_val=bank_dtype(inp["q_val"]), v=bank_dtype(inp["v"]),
        beta=torch.from_numpy(inp["beta"]).to(device), log_decay=torch.from_numpy(inp["log_decay"]).to(device),
        valid=torch.from_numpy(np.ascontiguousarray(inp["valid"], dtype=np.int32)).to(device))


def run(t: dict, C: int, bank=None, **kw):
    """One sdm_fwd call on a copy of t["bank"] (or on ``bank``). Returns (out, bank)."""
    from chunked_sparse_delta_amd import sdm_fwd
    b = t["bank"].clone() if bank is None else bank
    out = sdm_fwd(b, t["k_idx"], t["k_val"], t["v"], t["beta"], t["log_decay"], t["q_idx"], t["q_val"],
                  chunk=C, valid_tokens=t["valid"], **kw)
    torch.cuda.synchronize()
    return out, b


def f64(x: torch.Tensor) -> np.ndarray:
    return x.detach().float().cpu().numpy().astype(np.float64)


def bits(x: torch.Tensor) -> np.ndarray:
    y = x.detach().cpu()
    return (y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32)).numpy()


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    if scale == 0.0:
        return float(np.max(np.abs(got))) if got.size else 0.0
    return float(np.max(np.abs(got - ref)) / scale)


def oracle_ref(inp: dict, threads: int = 8, bf16_chunk=None):
    import oracle
    return oracle.token_loop(oracle.as_f64_inputs(inp), threads=threads, bf16_chunk=bf16_chunk)


def parity(out, bank, inp: dict, C: int, what: str = "", threads: int = 8, streams=None):
    """Check GPU readings and bank against O1 (and, for bf16 banks, O1b) on the given
    streams of ``inp`` (all by default; ``out``/``bank`` hold exactly those streams)."""
    ref = oracle_ref(inp, threads)
    con = oracle_ref(inp, threads, bf16_chunk=C) if inp["dtype"] == "bf16" else None
    check(out, bank, ref, con, inp["dtype"], what)


def check(out, bank, ref, con, dtype: str, what: str = ""):
    got = [f64(x) if isinstance(x, torch.Tensor) else x for x in (out, bank)]
    tol = TOL[dtype]
    msg, checks = [], []
    for name, g, r, c in zip(("readings", "bank"), got, ref, con if con is not None else (None, None)):
        e = rel_err(g, r)
        bar = tol
        line = f"{name} vs O1 {e:.3e}"
        if c is not None:
            e_c, e_m = rel_err(g, c), rel_err(c, r)
            bar = max(tol, SLACK * e_m)
            line += f", vs O1b {e_c:.3e} (O1b vs O1 {e_m:.3e})"
            checks.append((e_c, TOL_CONTRACT if SLACK * e_m <= tol else bar + e_m, name + " vs O1b"))
        checks.append((e, bar, name + " vs O1"))
        msg.append(line)
    print(f"{what}: " + "; ".join(msg) + f" (tol {tol})", flush=True)
    for e, bar, label in checks:
        assert np.isfinite(e) and e <= bar, (what, label, e, bar)


def assert_parity(out, bank, ref_out, ref_bank, dtype: str, what: str = "", con=None):
    check(out, bank, (ref_out, ref_bank), con, dtype, what)


def generate(wl, streams=None):
    return workloads.generate(wl, streams=streams)
