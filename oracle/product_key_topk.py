"""Product-key exact top-k, forward, on the CPU. TEST INFRASTRUCTURE, NOT PRODUCT.

The selection rule of ``product_key_topk`` (page 23, product_key_topk.py, the function's
docstring), restated as numbered conditions and taken step by step in plain Python:

  1. A slot chooses one column per factor. Its score is the float32 total of the chosen
     values, added in factor order; for bfloat16 input with three or more factors the running
     total is brought to bfloat16 each time before another factor's value joins it.
  2. Scores are compared as float32 numbers, except that negative zero ranks beneath
     positive zero and a NaN ranks as negative infinity.
  3. Inside one factor the columns are ordered by value, highest first, equal values putting
     the higher column index first; the first stage keeps min(k, width) of them.
  4. Each further stage f pairs a surviving rank i (i < n) of the previous stage with one of
     factor f's leading m = min(k, width_f) ranks j, only where (i + 1)(j + 1) <= c for
     c = min(k, n m), and keeps the c best pairs by score; an exact score tie is won by the
     pair with the greater i + j, and then by the greater i.
  5. The survivors come out by ascending linear index lin = (..(c_0 f_1 + c_1) ..) f_{F-1} +
     c_{F-1}, each with its score rounded to the input dtype.

Readings where the text leaves a step open (also listed in the design doc): the stage that adds
a factor other than the last one ranks its pairs by the partial sum it carries forward (the
bfloat16-rounded one when rounding applies); the last stage ranks by the float32 sum.

Pins (tests/test_topk_oracle.py): the brute-force top-k over every slot on tie-free inputs,
hand-worked tie cases, one factor, k at and above the slot count, the -0 / NaN order, and the
rounding of partial sums.
"""

from __future__ import annotations

import math

import numpy as np

MAX_K = 256


def order_key(x: float) -> tuple:
    """The float32 comparison of the rule as a sortable key: NaN as -inf, -0 below +0."""
    x = float(np.float32(x))
    if math.isnan(x):
        x = -math.inf
    return (x, 0 if (x == 0.0 and math.copysign(1.0, x) < 0) else 1)


def round_bf16(x: np.float32) -> np.float32:
    """Nearest bfloat16 of a float32 (ties to even), as a float32."""
    u = np.array([x], dtype=np.float32).view(np.uint32)[0]
    if (u & 0x7F800000) == 0x7F800000:   # inf or NaN: keep (NaN stays NaN)
        return np.float32(x)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return np.array([r], dtype=np.uint32).view(np.float32)[0]


def topk_row(row: np.ndarray, factors, k: int, bf16: bool):
    """One row: ``row`` float32 values of the factors side by side (exact copies of the
    input, bfloat16 inputs widened). Returns (val list of float32, lin list of int), lin
    ascending; val not yet rounded to the input dtype."""
    F = len(factors)
    assert F >= 1 and 1 <= k <= MAX_K and len(row) == sum(factors)
    starts = np.cumsum([0] + list(factors))[:-1]
    ranks = []
    for f, w in enumerate(factors):
        vals = [np.float32(row[starts[f] + c]) for c in range(w)]
        # descending by value; among equal values the higher column index comes first
        order = sorted(range(w), key=lambda c: (order_key(vals[c]), c), reverse=True)
        ranks.append([(vals[c], c) for c in order])
    kk = min(k, math.prod(factors))
    # stage 0: the first ranks of factor 0
    n = min(k, factors[0])
    cur = [(ranks[0][i][0], ranks[0][i][1]) for i in range(n)]   # (score, lin) in rank order
    for f in range(1, F):
        m = min(k, factors[f])
        c = min(k, len(cur) * m)
        pairs = []
        for i in range(len(cur)):
            for j in range(m):
                if (i + 1) * (j + 1) > c:
                    break
                with np.errstate(invalid="ignore", over="ignore"):   # inf - inf is NaN, as on the GPU
                    s = np.float32(cur[i][0] + ranks[f][j][0])
                if bf16 and F > 2 and f < F - 1:
                    s = round_bf16(s)
                pairs.append((s, i, j))
        # descending by score; equal scores: the higher i + j first, then the higher i
        pairs.sort(key=lambda q: (order_key(q[0]), q[1] + q[2], q[1]), reverse=True)
        cur = [(s, cur[i][1] * factors[f] + ranks[f][j][1]) for s, i, j in pairs[:c]]
    assert len(cur) == kk
    cur.sort(key=lambda q: q[1])
    return [s for s, _ in cur], [lin for _, lin in cur]


def product_key_topk(raw: np.ndarray, factors, k: int, bf16: bool = False):
    """raw [N, sum(factors)] float32 (bfloat16 inputs widened exactly, ``bf16`` set).
    Returns (val [N, kk] float32 holding the scores rounded to the input dtype, lin [N, kk]
    int64)."""
    raw = np.asarray(raw, dtype=np.float32)
    N = raw.shape[0]
    kk = min(k, math.prod(factors))
    val = np.zeros((N, kk), dtype=np.float32)
    lin = np.zeros((N, kk), dtype=np.int64)
    for r in range(N):
        v, l = topk_row(raw[r], factors, k, bf16)
        val[r] = [round_bf16(x) if bf16 else x for x in v]
        lin[r] = l
    return val, lin


def brute_force_topk(row: np.ndarray, factors, k: int):
    """The kk best slots of one row over every slot (float32 sums in factor order, no
    rounding), as a set of lin. Only meaningful where no two scores tie."""
    starts = np.cumsum([0] + list(factors))[:-1]
    scores = []
    for idx in np.ndindex(*factors):
        s = np.float32(0.0)
        for f, c in enumerate(idx):
            s = np.float32(s + np.float32(row[starts[f] + c])) if f else np.float32(row[starts[f] + c])
        lin = 0
        for f, c in enumerate(idx):
            lin = lin * factors[f] + c
        scores.append((order_key(s), lin))
    scores.sort(reverse=True)
    kk = min(k, math.prod(factors))
    return {lin for _, lin in scores[:kk]}


def product_key_topk_backward(lin: np.ndarray, grad_val: np.ndarray, factors, bf16: bool = False) -> np.ndarray:
    """The sparse backward of the top-k: d(val)/d(raw) is 1 at each factor column of a
    selected slot (roundings of the score pass the gradient through), so the gradient of a
    raw column is the sum of grad_val over the selected slots that use it. Sums run in
    float32 over the slots in output (ascending slot index) order; the result is rounded to
    the input dtype. lin, grad_val [N, kk] (grad_val exact float32 copies). Returns [N, D]
    float32 (bfloat16 values when ``bf16``)."""
    lin = np.asarray(lin, dtype=np.int64)
    grad_val = np.asarray(grad_val, dtype=np.float32)
    N, kk = lin.shape
    starts = np.cumsum([0] + list(factors))[:-1]
    out = np.zeros((N, sum(factors)), dtype=np.float32)
    for r in range(N):
        for s in range(kk):
            cols = np.unravel_index(int(lin[r, s]), factors)
            for f, c in enumerate(cols):
                j = starts[f] + c
                out[r, j] = np.float32(out[r, j] + grad_val[r, s])
    if bf16:
        out = np.vectorize(round_bf16, otypes=[np.float32])(out) if out.size else out
    return out
