"""Product-key exact top-k on the GPU (sdm_product_key_topk through the C ABI) against the
oracle (oracle/product_key_topk.py): the selected slots and their scores bit for bit,
including exact ties (integer-valued rows), -0 / +0, infinities and NaN."""

import numpy as np
import pytest
import torch

import workloads
from oracle import product_key_topk as pk

pytestmark = pytest.mark.gpu


def _raw(kind, rows, D, seed):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        x = rng.normal(size=(rows, D))
    elif kind == "ties":               # few distinct values: exact ties everywhere
        x = rng.integers(-3, 4, size=(rows, D)).astype(np.float64)
    else:                              # signed zeros, infinities and NaN among normals
        x = rng.normal(size=(rows, D))
        pick = rng.random((rows, D))
        x[pick < 0.05] = 0.0
        x[(pick >= 0.05) & (pick < 0.10)] = -0.0
        x[(pick >= 0.10) & (pick < 0.12)] = np.inf
        x[(pick >= 0.12) & (pick < 0.14)] = -np.inf
        x[(pick >= 0.14) & (pick < 0.16)] = np.nan
    return x.astype(np.float32)


def _to_dtype(x32, dtype, device):
    if dtype == "bf16":
        bits = workloads.round_bf16_bits(x32)
        t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)
        return t, workloads.bf16_bits_to_f32(bits)
    return torch.from_numpy(x32).to(device), x32


def _bits(t):
    y = t.detach().cpu()
    return (y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32)).numpy()


def _oracle_val_bits(val, dtype):
    if dtype == "bf16":
        return (val.view(np.uint32) >> 16).astype(np.uint16).view(np.int16)
    return val.view(np.int32)


CASES = [("f32", (16, 16), 8), ("f32", (33, 70), 40), ("bf16", (64, 64), 32), ("bf16", (5, 7, 9), 20),
         ("bf16", (4, 3, 5, 2), 50), ("f32", (300,), 17), ("f32", (2, 3), 10), ("bf16", (512, 512), 256),
         ("f32", (1000, 4096), 64), ("f32", (3, 3, 3), 27), ("f32", (7, 5, 3, 2, 2), 33),
         # factors wider than one LDS sort (ranked in pieces), up to the pages' 65535 columns
         ("f32", (16384, 8), 64), ("bf16", (65535, 65535), 256), ("f32", (5000, 3, 7), 100), ("bf16", (65535,), 200)]


@pytest.mark.parametrize("path", ["auto", "block"])
@pytest.mark.parametrize("kind", ["normal", "ties", "special"])
@pytest.mark.parametrize("dtype,factors,k", CASES, ids=[f"{d}-{'x'.join(map(str, f))}-k{k}" for d, f, k in CASES])
def test_topk_matches_oracle(gpu, dtype, factors, k, kind, path, monkeypatch):
    """auto: rows of factors <= 256 columns with k <= 64 run one row per wavefront (sorts in
    registers), the others one row per workgroup; block: every row on the workgroup kernel."""
    from chunked_sparse_delta_amd import product_key_topk
    if path == "block":
        monkeypatch.setenv("SDM_TOPK_PATH", "block")
    else:
        monkeypatch.delenv("SDM_TOPK_PATH", raising=False)
    rows = 13   # not a multiple of the four rows of a wavefront workgroup
    x32 = _raw(kind, rows, sum(factors), seed=sum(factors) + 7 * k + len(kind))
    t, exact = _to_dtype(x32, dtype, gpu)
    val, lin = product_key_topk(t, factors, k)
    torch.cuda.synchronize()
    ov, ol = pk.product_key_topk(exact, factors, k, bf16=dtype == "bf16")
    assert lin.shape == ol.shape and val.dtype == t.dtype
    assert np.array_equal(lin.cpu().numpy(), ol), kind
    got, want = _bits(val), _oracle_val_bits(ov, dtype)
    both_nan = np.isnan(val.float().cpu().numpy()) & np.isnan(ov)
    assert np.array_equal(np.where(both_nan, 0, got), np.where(both_nan, 0, want)), kind


def test_topk_leading_dims_and_empty(gpu):
    from chunked_sparse_delta_amd import product_key_topk
    x = torch.randn(2, 3, 40, device=gpu)
    val, lin = product_key_topk(x, (8, 32), 12)
    assert val.shape == (2, 3, 12) and lin.shape == (2, 3, 12)
    v2, l2 = product_key_topk(x.reshape(6, 40), (8, 32), 12)
    assert torch.equal(lin.reshape(6, 12), l2) and torch.equal(val.reshape(6, 12), v2)
    v0, l0 = product_key_topk(torch.empty(0, 40, device=gpu), (8, 32), 12)
    assert v0.shape == (0, 12) and l0.shape == (0, 12)


@pytest.mark.parametrize("dtype,factors,k", [("f32", (16, 16), 8), ("bf16", (64, 64), 32), ("bf16", (5, 7, 9), 20),
                                             ("f32", (300,), 17), ("f32", (33, 70), 40), ("bf16", (512, 512), 256),
                                             ("f32", (16384, 8), 64), ("bf16", (65535, 65535), 256)])
def test_topk_backward_matches_oracle(gpu, dtype, factors, k):
    """The sparse backward: each raw column's gradient is the sum, in output order, of the
    gradients of the selected slots that use it (oracle_topk_backward), bit for bit."""
    from chunked_sparse_delta_amd import product_key_topk, product_key_topk_backward
    rows = 13
    x32 = _raw("normal", rows, sum(factors), seed=k + 3)
    t, _ = _to_dtype(x32, dtype, gpu)
    _, lin = product_key_topk(t, factors, k)
    g32 = _raw("ties" if dtype == "f32" else "normal", rows, lin.shape[1], seed=k + 5)
    gt, gexact = _to_dtype(g32, dtype, gpu)
    graw = product_key_topk_backward(lin, gt, factors)
    torch.cuda.synchronize()
    want = pk.product_key_topk_backward(lin.cpu().numpy(), gexact, factors, bf16=dtype == "bf16")
    assert graw.shape == (rows, sum(factors)) and graw.dtype == gt.dtype
    assert np.array_equal(_bits(graw), _oracle_val_bits(want, dtype))


def test_random_factor_shapes(gpu, monkeypatch):
    """30 random shapes (a fixed seed) within the documented limits: 1 to 8 factors of 1 to
    65535 columns (product below 2^55), k from 1 to 256, 1 to 39 rows, both dtypes, normal,
    tied and special values, either kernel; the forward and the sparse backward bit for bit."""
    from chunked_sparse_delta_amd import product_key_topk, product_key_topk_backward
    rng = np.random.default_rng(20261205)
    for i in range(30):
        F = int(rng.choice([1, 2, 2, 2, 3, 3, 4, 4, 5, 6, 8]))
        while True:
            f = tuple(max(1, min(65535, int(np.exp(rng.uniform(0, np.log(65535 if F <= 2 else 2000))))))
                      for _ in range(F))
            if np.prod([float(x) for x in f]) < 2.0 ** 55:
                break
        k = int(rng.choice([1, 2, 7, 16, 32, 64, 100, 200, 256]))
        rows = int(rng.integers(1, 40))
        rows = min(rows, max(1, int(4e5 / sum(f))))   # keeps the oracle to a second or so
        dtype = str(rng.choice(["f32", "bf16"]))
        kind = str(rng.choice(["normal", "ties", "special"]))
        path = str(rng.choice(["auto", "block"]))
        tag = f"factors {f} k{k} rows{rows} {dtype} {kind} {path}"
        print(tag, flush=True)
        if path == "block":
            monkeypatch.setenv("SDM_TOPK_PATH", "block")
        else:
            monkeypatch.delenv("SDM_TOPK_PATH", raising=False)
        x32 = _raw(kind, rows, sum(f), seed=9000 + i)
        t, exact = _to_dtype(x32, dtype, gpu)
        val, lin = product_key_topk(t, f, k)
        torch.cuda.synchronize()
        ov, ol = pk.product_key_topk(exact, f, k, bf16=dtype == "bf16")
        assert lin.shape == ol.shape and np.array_equal(lin.cpu().numpy(), ol), tag
        got, want = _bits(val), _oracle_val_bits(ov, dtype)
        both_nan = np.isnan(val.float().cpu().numpy()) & np.isnan(ov)
        assert np.array_equal(np.where(both_nan, 0, got), np.where(both_nan, 0, want)), tag
        g32 = _raw("normal", rows, lin.shape[1], seed=9500 + i)
        gt, gexact = _to_dtype(g32, dtype, gpu)
        graw = product_key_topk_backward(lin, gt, f)
        torch.cuda.synchronize()
        wantb = pk.product_key_topk_backward(lin.cpu().numpy(), gexact, f, bf16=dtype == "bf16")
        assert np.array_equal(_bits(graw), _oracle_val_bits(wantb, dtype)), tag
    monkeypatch.delenv("SDM_TOPK_PATH", raising=False)
