"""Pins of the CPU oracle (O1 token loop, O2 chunk algebra) against facts fixed by the
pages and by the mathematics, not against itself. CPU only."""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import chunk_algebra
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_example.json")


def _rel(a, b):
    scale = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / scale)


def _frac(a):
    return np.vectorize(lambda s: float(Fraction(s)))(np.asarray(a, dtype=object)).astype(np.float64)


def _hand_inputs(valid=3):
    d = json.load(open(GOLDEN))
    g = np.where(np.asarray(d["gate_is_minus_ln2"]), -math.log(2.0), 0.0)
    return d, dict(
        bank=_frac(d["bank"])[None], k_idx=np.asarray(d["k_idx"], np.int32)[None],
        k_val=_frac(d["k_val"])[None], v=_frac(d["v"])[None], beta=_frac(d["beta"])[None],
        g=g[None], q_idx=np.asarray(d["q_idx"], np.int32)[None], q_val=_frac(d["q_val"])[None],
        valid=np.asarray([valid], np.int32))


def tiny_inputs(seed=0, P=2, T=23, W=3, R=2, hd=4, M=9, G=None, ragged=True, gpos=False):
    """fp64 random inputs with many repeated slots across tokens (M small)."""
    rng = np.random.default_rng(seed)
    G = W if G is None else G
    k_idx = np.stack([np.stack([rng.choice(M, W, replace=False) for _ in range(T)]) for _ in range(P)])
    q_idx = rng.integers(0, M, size=(P, T, R))
    g = -0.3 * rng.random((P, T, G))
    if gpos:
        g = rng.normal(0.0, 0.3, (P, T, G))
    return dict(
        bank=rng.normal(size=(P, M, hd)), k_idx=k_idx.astype(np.int32),
        k_val=rng.random((P, T, W)), v=rng.normal(size=(P, T, hd)),
        beta=1 / (1 + np.exp(-rng.normal(size=(P, T)))), g=g, q_idx=q_idx.astype(np.int32),
        q_val=rng.random((P, T, R)),
        valid=(rng.integers(T // 2, T + 1, size=P) if ragged else np.full(P, T)).astype(np.int32))


# ---------------------------------------------------------------- worked example

@pytest.mark.parametrize("valid", [3, 2])
def test_hand_example_token_loop(valid):
    d, inp = _hand_inputs(valid)
    out, bank = oracle.token_loop(inp)
    ref = d if valid == 3 else d["valid_2"]
    assert _rel(out[0], _frac(ref["readings"])) < 1e-15
    assert _rel(bank[0], _frac(ref["final_bank"])) < 1e-15


@pytest.mark.parametrize("C", [1, 2, 3, 4])
@pytest.mark.parametrize("valid", [3, 2])
def test_hand_example_chunked(C, valid):
    d, inp = _hand_inputs(valid)
    out, bank, _ = chunk_algebra.forward(inp, C)
    ref = d if valid == 3 else d["valid_2"]
    assert _rel(out[0], _frac(ref["readings"])) < 1e-14
    assert _rel(bank[0], _frac(ref["final_bank"])) < 1e-14


# ---------------------------------------------------------------- two derivations agree

@pytest.mark.parametrize("seed,kw,C", [
    (0, {}, 4), (1, {}, 1), (2, {}, 7), (3, dict(G=1), 5), (4, dict(gpos=True), 6),
    (5, dict(W=1, R=1, M=3), 8), (6, dict(W=4, R=5, M=6, T=17), 17), (7, dict(ragged=False), 23),
    (8, dict(T=9, M=4, W=2, R=3), 3),
])
def test_token_loop_equals_chunk_algebra(seed, kw, C):
    inp = tiny_inputs(seed, **kw)
    o1, b1 = oracle.token_loop(inp)
    o2, b2, _ = chunk_algebra.forward(inp, C)
    assert _rel(o2, o1) < 1e-12
    assert _rel(b2, b1) < 1e-12


def test_generated_small_workload_both_oracles():
    wl = workloads.small(P=2, T=40, C=16, hd=4, M=12, W=3, R=2, ragged=True, ids="zipf")
    inp = oracle.as_f64_inputs(workloads.generate(wl))
    o1, b1 = oracle.token_loop(inp, threads=2)
    o2, b2, _ = chunk_algebra.forward(inp, wl.C)
    assert _rel(o2, o1) < 1e-12 and _rel(b2, b1) < 1e-12


# ---------------------------------------------------------------- closed forms

def test_beta_zero_rows_only_decay():
    inp = tiny_inputs(11, ragged=False)
    inp["beta"][:] = 0.0
    out, bank = oracle.token_loop(inp)
    P, T, W = inp["k_idx"].shape
    for p in range(P):
        total = np.zeros(inp["bank"].shape[1])
        for t in range(T):
            for w in range(W):
                total[inp["k_idx"][p, t, w]] += inp["g"][p, t, w]
            # reading at t: sum_r q exp(sum of gates on that slot so far) B0
            ref = sum(inp["q_val"][p, t, r] * math.exp(total[inp["q_idx"][p, t, r]])
                      * inp["bank"][p, inp["q_idx"][p, t, r]] for r in range(inp["q_idx"].shape[2]))
            assert np.allclose(out[p, t], ref, rtol=1e-13, atol=1e-13)
        assert np.allclose(bank[p], np.exp(total)[:, None] * inp["bank"][p], rtol=1e-13, atol=1e-13)


def test_scalar_ema():
    """W = R = 1 on one row with k = q = 1 and g = 0: the bank is an EMA of v."""
    T = 50
    rng = np.random.default_rng(3)
    beta = rng.random(T)
    v = rng.normal(size=T)
    b0 = 0.7
    inp = dict(bank=np.full((1, 1, 1), b0), k_idx=np.zeros((1, T, 1), np.int32), k_val=np.ones((1, T, 1)),
               v=v[None, :, None], beta=beta[None], g=np.zeros((1, T, 1)),
               q_idx=np.zeros((1, T, 1), np.int32), q_val=np.ones((1, T, 1)), valid=np.array([T], np.int32))
    out, bank = oracle.token_loop(inp)
    # closed form: b_t = prod_{s<=t}(1-beta_s) b0 + sum_{s<=t} beta_s v_s prod_{s<r<=t}(1-beta_r)
    for t in range(T):
        keep = np.prod(1 - beta[:t + 1])
        acc = sum(beta[s] * v[s] * np.prod(1 - beta[s + 1:t + 1]) for s in range(t + 1))
        assert abs(out[0, t, 0] - (keep * b0 + acc)) < 1e-12
    for C in (1, 4, 16):
        o2, _, _ = chunk_algebra.forward(inp, C)
        assert _rel(o2, out) < 1e-12


def test_single_token_is_plain_delta_update():
    inp = tiny_inputs(21, P=1, T=1, W=4, R=3, hd=5, M=10, ragged=False)
    out, bank = oracle.token_loop(inp)
    B0 = inp["bank"][0]
    s, k, g = inp["k_idx"][0, 0], inp["k_val"][0, 0], inp["g"][0, 0]
    decayed = np.exp(g)[:, None] * B0[s]
    delta = inp["beta"][0, 0] * (inp["v"][0, 0] - k @ decayed)
    ref_bank = B0.copy()
    ref_bank[s] = decayed + k[:, None] * delta[None, :]
    assert np.allclose(bank[0], ref_bank, rtol=1e-14, atol=1e-14)
    ref_out = inp["q_val"][0, 0] @ ref_bank[inp["q_idx"][0, 0]]
    assert np.allclose(out[0, 0], ref_out, rtol=1e-14, atol=1e-14)
    o2, b2, _ = chunk_algebra.forward(inp, 1)
    assert _rel(o2, out) < 1e-14 and _rel(b2, bank) < 1e-14


def test_large_negative_decay_overwrites():
    """exp(-80) ~ 1.8e-35: each write replaces its row by k * beta * v."""
    inp = tiny_inputs(5, P=1, T=12, W=1, R=1, hd=3, M=4, ragged=False)
    inp["g"][:] = -80.0
    inp["q_idx"][...] = inp["k_idx"]
    out, bank = oracle.token_loop(inp)
    k, b, v = inp["k_val"][0, :, 0], inp["beta"][0], inp["v"][0]
    ref = (inp["q_val"][0, :, 0] * k * b)[:, None] * v
    assert np.allclose(out[0], ref, rtol=1e-12, atol=1e-30)
    o2, _, _ = chunk_algebra.forward(inp, 4)
    assert np.allclose(o2, out, rtol=1e-12, atol=1e-30)


# ---------------------------------------------------------------- chunk-algebra structure

def test_no_repeat_in_chunk_gives_identity_solve():
    """Slots written at most once per chunk: A = 0, so X = I and QX = QK."""
    T, M, W = 8, 64, 3
    inp = tiny_inputs(9, P=1, T=T, W=W, R=2, M=M, ragged=False)
    inp["k_idx"][0] = np.arange(T * W).reshape(T, W)
    _, _, inter = chunk_algebra.forward(inp, T, emit=True)
    c = inter[0][0]
    assert np.all(c["A"] == 0.0)
    assert np.array_equal(c["X"], np.eye(T))
    assert np.allclose(c["QX"], np.tril(c["QK"]), rtol=0, atol=0)


def test_X_unit_lower_and_leading_block():
    inp = tiny_inputs(13, P=1, T=16, W=3, R=2, M=5, ragged=False)
    _, _, inter = chunk_algebra.forward(inp, 16, emit=True)
    c = inter[0][0]
    X = c["X"]
    assert np.all(np.diag(X) == 1.0) or np.allclose(np.diag(X), 1.0, atol=1e-14)
    assert np.all(np.triu(X, 1) == 0.0)
    assert not np.signbit(np.triu(X, 1)).any()
    Lm = np.tril(c["beta"][:, None] * c["A"], -1)
    for k in (1, 5, 9):
        lead = np.linalg.inv(np.eye(k) + Lm[:k, :k])
        assert np.allclose(X[:k, :k], lead, rtol=1e-12, atol=1e-12)
    # X is the inverse
    assert np.allclose(X @ (np.eye(16) + Lm), np.eye(16), atol=1e-12)


# ---------------------------------------------------------------- invariants

def test_padding_is_inert():
    inp = tiny_inputs(17, P=2, T=30, ragged=False)
    inp["valid"] = np.array([30, 19], np.int32)
    out, bank = oracle.token_loop(inp)
    assert np.all(out[1, 19:] == 0.0)
    trunc = {k: (v[1:2, :19] if k not in ("bank", "valid") else v[1:2]) for k, v in inp.items()}
    trunc["valid"] = np.array([19], np.int32)
    o_t, b_t = oracle.token_loop(trunc)
    assert np.array_equal(out[1, :19], o_t[0])
    assert np.array_equal(bank[1], b_t[0])
    for C in (4, 16):
        o2, b2, _ = chunk_algebra.forward(inp, C)
        assert np.all(o2[1, 19:] == 0.0)
        assert _rel(o2, out) < 1e-12 and _rel(b2, bank) < 1e-12


@pytest.mark.parametrize("C", [1, 2, 3, 5, 8, 16, 29, 64])
def test_chunk_size_independence(C):
    inp = tiny_inputs(19, P=1, T=29, W=3, R=3, M=6)
    o1, b1 = oracle.token_loop(inp)
    o2, b2, _ = chunk_algebra.forward(inp, C)
    assert _rel(o2, o1) < 1e-12 and _rel(b2, b1) < 1e-12


def test_stream_independence():
    inp = tiny_inputs(23, P=3, T=20)
    out, bank = oracle.token_loop(inp)
    for p in range(3):
        one = {k: v[p:p + 1] for k, v in inp.items()}
        o, b = oracle.token_loop(one)
        assert np.array_equal(o[0], out[p]) and np.array_equal(b[0], bank[p])
    o2, b2, _ = chunk_algebra.forward({k: v[::-1].copy() for k, v in inp.items()}, 4)
    assert _rel(o2[::-1], out) < 1e-12 and _rel(b2[::-1], bank) < 1e-12


def test_columns_evolve_independently():
    inp = tiny_inputs(29, P=2, T=25, hd=6)
    out, bank = oracle.token_loop(inp)
    perm = np.array([3, 0, 5, 1, 4, 2])
    pin = dict(inp, bank=inp["bank"][:, :, perm], v=inp["v"][:, :, perm])
    o, b = oracle.token_loop(pin)
    assert np.array_equal(o, out[:, :, perm]) and np.array_equal(b, bank[:, :, perm])


def test_permuting_slot_ids_permutes_bank_rows():
    inp = tiny_inputs(31, P=1, T=20, M=9)
    out, bank = oracle.token_loop(inp)
    perm = np.random.default_rng(0).permutation(9)   # new id of old row i is perm[i]
    pin = dict(inp, k_idx=perm[inp["k_idx"]].astype(np.int32), q_idx=perm[inp["q_idx"]].astype(np.int32))
    newbank = np.empty_like(inp["bank"])
    newbank[:, perm] = inp["bank"]
    pin["bank"] = newbank
    o, b = oracle.token_loop(pin)
    assert np.allclose(o, out, rtol=1e-13, atol=1e-13)
    assert np.allclose(b[:, perm], bank, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- caller contract

def test_token_loop_rejects_repeated_write_slot():
    inp = tiny_inputs(37, P=1, T=4, W=2, M=5, ragged=False)
    inp["k_idx"][0, 2] = [3, 3]
    with pytest.raises(ValueError, match="repeated"):
        oracle.token_loop(inp)


def test_token_loop_rejects_out_of_range_slot():
    inp = tiny_inputs(41, P=1, T=4, W=2, M=5, ragged=False)
    inp["q_idx"][0, 1, 0] = 5
    with pytest.raises(ValueError, match="range"):
        oracle.token_loop(inp)


# ---------------------------------------------------------------- a planted mistake is caught

def test_pins_catch_a_dropped_decay(monkeypatch):
    """Plant a plausible mistake in the chunk algebra (forget the decay inside A) and
    check that the token-loop comparison rejects it."""
    inp = tiny_inputs(43, P=1, T=20, M=5)
    o1, _ = oracle.token_loop(inp)
    real = chunk_algebra.phase1

    def wrong(*a, **k):
        d = real(*a, **k)
        k_idx, k_val, g = a[0], a[1], a[2]
        A = np.zeros_like(d["A"])
        C, W = k_idx.shape
        for i in range(C):
            for j in range(i):
                for w in range(W):
                    for w2 in range(W):
                        if k_idx[i, w] == k_idx[j, w2] and i < a[6]:
                            A[i, j] += k_val[i, w] * k_val[j, w2]
        d["A"] = A
        return d
    monkeypatch.setattr(chunk_algebra, "phase1", wrong)
    o2, _, _ = chunk_algebra.forward(inp, 5)
    assert _rel(o2, o1) > 1e-6


# ---------------------------------------------------------------- O1b: the bfloat16 storage contract

def test_round_bf16_ties_to_even_without_double_rounding():
    one = 1.0
    assert oracle.round_bf16(one + 2 ** -8) == one                   # tie -> even
    assert oracle.round_bf16(one + 3 * 2 ** -8) == one + 2 ** -6     # tie -> even (up)
    assert oracle.round_bf16(one + 2 ** -8 + 2 ** -40) == one + 2 ** -7   # just above the tie: up
    assert oracle.round_bf16(-(one + 2 ** -8 + 2 ** -40)) == -(one + 2 ** -7)
    assert oracle.round_bf16(0.0) == 0.0 and oracle.round_bf16(3.0) == 3.0


def test_round_bf16_matches_float32_bit_rounding():
    """On float32 inputs (no double rounding possible) it equals the bit-level
    float32 -> bfloat16 rounding of the input generator, an independent routine."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(4000) * np.exp(rng.uniform(-20, 20, 4000))).astype(np.float32)
    ref = workloads.bf16_bits_to_f32(workloads.round_bf16_bits(x)).astype(np.float64)
    assert np.array_equal(oracle.round_bf16(x.astype(np.float64)), ref)


def test_bf16_loop_with_one_chunk_is_rounded_o1():
    """With one chunk spanning the stream, no row is rounded before the end: readings
    are O1's rounded, written rows are O1's rounded, other rows are untouched."""
    inp = tiny_inputs(47, P=2, T=20, W=3, R=2, M=12, ragged=True)
    o1, b1 = oracle.token_loop(inp)
    ob, bb = oracle.token_loop(inp, bf16_chunk=64)
    assert np.array_equal(ob, oracle.round_bf16(o1))
    for p in range(2):
        written = np.unique(inp["k_idx"][p, :inp["valid"][p]])
        assert np.array_equal(bb[p, written], oracle.round_bf16(b1[p, written]))
        rest = np.setdiff1d(np.arange(12), written)
        assert np.array_equal(bb[p, rest], inp["bank"][p, rest])


@pytest.mark.parametrize("C", [1, 2, 4])
def test_bf16_loop_equals_o1_on_bf16_exact_values(C):
    """Small integers, k = 1, no decay and beta = 1/2 keep every value a short dyadic
    fraction: rounding is the identity and O1b equals O1 exactly."""
    T, M, hd = 4, 2, 2
    rng = np.random.default_rng(2)
    inp = dict(bank=rng.integers(-4, 5, (1, M, hd)).astype(np.float64),
               k_idx=rng.integers(0, M, (1, T, 1)).astype(np.int32), k_val=np.ones((1, T, 1)),
               v=rng.integers(-4, 5, (1, T, hd)).astype(np.float64), beta=np.full((1, T), 0.5),
               g=np.zeros((1, T, 1)), q_idx=rng.integers(0, M, (1, T, 1)).astype(np.int32),
               q_val=np.ones((1, T, 1)), valid=np.array([T], np.int32))
    o1, b1 = oracle.token_loop(inp)
    ob, bb = oracle.token_loop(inp, bf16_chunk=C)
    assert np.array_equal(o1, oracle.round_bf16(o1)) and np.array_equal(b1, oracle.round_bf16(b1))
    assert np.array_equal(ob, o1) and np.array_equal(bb, b1)


def test_bf16_loop_rounds_at_chunk_ends():
    """Rounding a row at a chunk end changes what later chunks read: with a value that
    is not bfloat16-exact, chunk size 1 and chunk size T disagree."""
    inp = tiny_inputs(53, P=1, T=12, W=2, R=2, M=4, ragged=False)
    o_a, _ = oracle.token_loop(inp, bf16_chunk=1)
    o_b, _ = oracle.token_loop(inp, bf16_chunk=12)
    assert not np.array_equal(o_a, o_b)
    assert _rel(o_a, o_b) < 5e-2


# ---------------------------------------------------------------- shared bank, repeated writes

@pytest.mark.parametrize("bf16_chunk", [None, 4])
def test_shared_bank_equals_per_stream_banks(bf16_chunk):
    """One bank shared by streams with disjoint slots (page 21, sdm_write_read with
    shared_bank=True) computes what per-stream banks compute, row for row."""
    inp = tiny_inputs(41, P=3, T=30, M=7)
    out, bank = oracle.token_loop(inp, bf16_chunk=bf16_chunk)
    sh = workloads.shared_bank_inputs(inp)
    o2, b2 = oracle.token_loop(sh, bf16_chunk=bf16_chunk)
    assert b2.shape == (21, 4)
    assert np.array_equal(o2, out)
    assert np.array_equal(workloads.per_stream_bank(b2, 3), bank)


def test_shared_bank_rejects_streams_sharing_a_slot():
    sh = workloads.shared_bank_inputs(tiny_inputs(43, P=2, T=10, M=5))
    sh["q_idx"] = sh["q_idx"].copy()
    sh["q_idx"][1, 0, 0] = sh["k_idx"][0, 0, 0]   # stream 1 reads a slot stream 0 writes
    with pytest.raises(ValueError, match="selected by streams"):
        oracle.token_loop(sh)


def test_repeated_write_slots_hand_count():
    """Entries that repeat a slot of their own token (page 21, repeated_write_slots):
    [3, 5, 3, 3] repeats twice, [7, 7, 8, 9] once, distinct tokens never."""
    k = np.array([[[3, 5, 3, 3], [1, 2, 3, 4], [7, 7, 8, 9]],
                  [[0, 1, 2, 3], [6, 6, 6, 6], [5, 4, 3, 2]]], np.int32)
    assert oracle.repeated_write_slots(k) == 2 + 1 + 3
    assert oracle.repeated_write_slots(k, valid=[1, 2]) == 2 + 3
    assert oracle.repeated_write_slots(k, valid=[0, 0]) == 0
    inp = tiny_inputs(47, P=2, T=30)
    assert oracle.repeated_write_slots(inp["k_idx"], inp["valid"]) == 0
