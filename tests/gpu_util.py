"""Helpers of the GPU tests: move generator inputs to the GPU, run the HIP path through
the C ABI binding, compare against the oracle."""

from __future__ import annotations

import numpy as np
import torch

import workloads

TOL = {"f32": 1e-4, "bf16": 2e-2}   # infinity-norm relative error per output tensor


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


def oracle_ref(inp: dict, threads: int = 8):
    import oracle
    return oracle.token_loop(oracle.as_f64_inputs(inp), threads=threads)


def assert_parity(out, bank, ref_out, ref_bank, dtype: str, what: str = ""):
    tol = TOL[dtype]
    e_out = rel_err(f64(out) if isinstance(out, torch.Tensor) else out, ref_out)
    e_bank = rel_err(f64(bank) if isinstance(bank, torch.Tensor) else bank, ref_bank)
    print(f"{what}: readings rel err {e_out:.3e}, bank rel err {e_bank:.3e} (tol {tol})", flush=True)
    assert np.isfinite(e_out) and e_out <= tol, (what, "readings", e_out)
    assert np.isfinite(e_bank) and e_bank <= tol, (what, "bank", e_bank)


def generate(wl, streams=None):
    return workloads.generate(wl, streams=streams)
