"""Pins of the product-key top-k oracle (oracle/product_key_topk.py) against what the rule
of page 23 (product_key_topk.py, product_key_topk docstring) fixes: the brute-force top-k
over every slot where no scores tie, hand-worked tie cases, the -0 / NaN order, one factor,
k at and above the slot count, and bfloat16 rounding of partial sums."""

import math

import numpy as np
import pytest

from oracle import product_key_topk as pk


@pytest.mark.parametrize("factors,k", [
    ((5, 7), 1), ((5, 7), 3), ((5, 7), 10), ((5, 7), 35), ((5, 7), 200),
    ((4, 3, 5), 7), ((4, 3, 5), 60), ((3, 3, 2, 4), 11), ((9,), 4), ((2, 17), 16), ((16, 16), 40),
])
def test_staged_rule_equals_brute_force_without_ties(factors, k):
    rng = np.random.default_rng(sum(factors) * 131 + k)
    raw = rng.normal(size=(6, sum(factors))).astype(np.float32)
    val, lin = pk.product_key_topk(raw, factors, k)
    kk = min(k, math.prod(factors))
    assert val.shape == (6, kk) and lin.shape == (6, kk)
    starts = np.cumsum([0] + list(factors))[:-1]
    for r in range(6):
        assert set(lin[r].tolist()) == pk.brute_force_topk(raw[r], factors, k)
        assert np.all(np.diff(lin[r]) > 0)
        for x, l in zip(val[r], lin[r]):   # the score of the slot, summed in factor order
            cols = np.unravel_index(int(l), factors)
            s = np.float32(raw[r, starts[0] + cols[0]])
            for f in range(1, len(factors)):
                s = np.float32(s + raw[r, starts[f] + cols[f]])
            assert x == s


def test_wide_factor_equals_brute_force_without_ties():
    """A factor of 16384 columns (the pages' two- to four-factor kernels take up to 65535)
    with a factor of 8: the staged rule against all 131072 slots."""
    factors, k = (16384, 8), 64
    rng = np.random.default_rng(16384)
    raw = rng.normal(size=(2, sum(factors))).astype(np.float32)
    val, lin = pk.product_key_topk(raw, factors, k)
    for r in range(2):
        a, b = raw[r, :16384], raw[r, 16384:]
        sums = (a[:, None] + b[None, :]).astype(np.float32).ravel()   # two terms: exact float32 sums
        order = np.argsort(-sums, kind="stable")
        assert sums[order[k - 1]] != sums[order[k]]   # no tie at the boundary
        assert set(lin[r].tolist()) == set(order[:k].tolist())


def test_ties_follow_the_stated_order():
    """factors (2, 2), k = 2, all four scores 1: factor ranks put the larger column first
    (col 1, col 0); stage 1 keeps c = 2 of the pairs (0,0), (0,1), (1,0) by the larger
    i + j, then the larger i: (1,0) -> slot (0, 1) = lin 1, then (0,1) -> slot (1, 0) = lin 2."""
    val, lin = pk.product_key_topk(np.array([[1, 1, 0, 0]], np.float32), (2, 2), 2)
    assert lin.tolist() == [[1, 2]] and val.tolist() == [[1.0, 1.0]]


def test_signed_zero_and_nan_order():
    val, lin = pk.product_key_topk(np.array([[-0.0, 0.0, -1.0]], np.float32), (3,), 1)
    assert lin.tolist() == [[1]] and math.copysign(1.0, float(val[0, 0])) > 0
    # NaN counts as -inf and ties with it: larger column first
    val, lin = pk.product_key_topk(np.array([[np.nan, -np.inf, -5.0]], np.float32), (3,), 2)
    assert lin.tolist() == [[1, 2]] and val[0, 0] == -np.inf and val[0, 1] == -5.0


def test_one_factor_and_k_beyond_the_slots():
    raw = np.array([[0.5, -2.0, 3.0, 0.25, 3.0]], np.float32)
    val, lin = pk.product_key_topk(raw, (5,), 3)
    assert lin.tolist() == [[0, 2, 4]]                       # 3.0 (col 4), 3.0 (col 2), 0.5
    val, lin = pk.product_key_topk(np.arange(5, dtype=np.float32)[None], (2, 3), 10)
    assert lin.tolist() == [list(range(6))]                  # kk = 6: every slot


def test_bf16_partial_sums_round_before_the_next_factor():
    """1 + 2^-8 is a bfloat16 tie that rounds to 1 (even): with three bfloat16 factors the
    partial sum 1 + 2^-8 becomes 1 before the third 2^-8 is added; float32 keeps it."""
    row = np.array([1.0, 2.0 ** -8, 2.0 ** -8], np.float32)
    v, _ = pk.topk_row(row, (1, 1, 1), 1, bf16=True)
    assert v == [np.float32(1.0 + 2.0 ** -8)]
    v, _ = pk.topk_row(row, (1, 1, 1), 1, bf16=False)
    assert v == [np.float32(1.0 + 2.0 ** -7)]
    assert pk.round_bf16(np.float32(1.0 + 2.0 ** -8)) == np.float32(1.0)
    assert pk.round_bf16(np.float32(1.0 + 3 * 2.0 ** -8)) == np.float32(1.0 + 2.0 ** -6)
    # two factors: no partial rounding
    v, _ = pk.topk_row(np.array([1.0, 2.0 ** -8], np.float32), (1, 1), 1, bf16=True)
    assert v == [np.float32(1.0 + 2.0 ** -8)]


def test_backward_scatters_each_slot_gradient_to_its_columns():
    """Integer gradients sum exactly: each factor's columns receive every selected slot's
    gradient once (so each factor's column sums equal the total), at the columns of the
    slot; unselected columns get zero."""
    factors = (4, 3, 5)
    lin = np.array([[0, 7, 59], [5, 6, 30]], np.int64)        # slots (0,0,0) (0,1,2) (3,2,4) ...
    g = np.array([[1, 2, 4], [8, 16, 32]], np.float32)
    out = pk.product_key_topk_backward(lin, g, factors)
    assert out.shape == (2, 12)
    starts = [0, 4, 7]
    for r in range(2):
        for f, w in enumerate(factors):
            assert out[r, starts[f]:starts[f] + w].sum() == g[r].sum()
    # row 0: slots (0,0,0), (0,1,2), (3,2,4)
    assert out[0].tolist() == [3, 0, 0, 4, 1, 2, 4, 1, 0, 2, 0, 4]
    # row 1: slots (0,1,0) -> 5, (0,1,1) -> 6, (2,0,0) -> 30
    assert out[1].tolist() == [24, 0, 32, 0, 32, 24, 0, 40, 16, 0, 0, 0]


def test_backward_rounds_to_bf16_once():
    lin = np.array([[0, 1]], np.int64)                          # both slots use column 0 of factor 0
    g = np.array([[1.0, 2.0 ** -8]], np.float32)
    out = pk.product_key_topk_backward(lin, g, (1, 2), bf16=True)
    assert out[0, 0] == np.float32(1.0)                         # 1 + 2^-8 rounds to 1 (even)
    assert out[0, 1] == np.float32(1.0) and out[0, 2] == np.float32(2.0 ** -8)
