"""Pins of the backward oracle O3 (oracle/token_loop_backward.c) against what the forward
fixes, not against itself: central finite differences of the forward oracle O1 for every
input element, a one-token closed form, linearity in the output gradients, padding tokens,
untouched rows and the reduction of a per-token gate to per-slot gates. CPU only."""

import math

import numpy as np
import pytest

import oracle


def _inputs(seed, P=2, T=7, W=2, R=3, hd=3, M=5, G=None, ragged=True, dup_reads=False):
    """fp64 inputs with slots repeating across tokens (M small); distinct writes per token."""
    rng = np.random.default_rng(seed)
    G = W if G is None else G
    k_idx = np.stack([np.stack([rng.choice(M, W, replace=False) for _ in range(T)]) for _ in range(P)])
    q_idx = rng.integers(0, M, size=(P, T, R))
    if dup_reads:
        q_idx[:, :, -1] = q_idx[:, :, 0]
    return dict(
        bank=rng.normal(size=(P, M, hd)), k_idx=k_idx.astype(np.int32), k_val=rng.normal(size=(P, T, W)),
        v=rng.normal(size=(P, T, hd)), beta=1 / (1 + np.exp(-rng.normal(size=(P, T)))),
        g=rng.normal(-0.4, 0.3, (P, T, G)), q_idx=q_idx.astype(np.int32), q_val=rng.normal(size=(P, T, R)),
        valid=(np.array([T, T - 2][:P] + [T] * max(0, P - 2)) if ragged else np.full(P, T)).astype(np.int32))


def _objective(inp, go, gbf):
    out, bank = oracle.token_loop(inp)
    return float(np.sum(go * out) + np.sum(gbf * bank))


FD_NAMES = ("bank", "k_val", "v", "beta", "g", "q_val")


@pytest.mark.parametrize("seed,G,dup", [(0, None, False), (1, 1, False), (2, None, True), (3, 1, True)])
def test_gradients_equal_central_differences_of_the_forward(seed, G, dup):
    """Every partial derivative of J = <grad_out, readings> + <grad_bank_final, final bank>,
    taken by central differences of O1 (h = 1e-5, truncation error ~ h^2), against O3."""
    inp = _inputs(seed, G=G, dup_reads=dup)
    rng = np.random.default_rng(100 + seed)
    go = rng.normal(size=inp["v"].shape)
    gbf = rng.normal(size=inp["bank"].shape)
    got = oracle.token_loop_backward(inp, go, gbf)
    h = 1e-5
    for name in FD_NAMES:
        x = inp[name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            plus = {**inp, name: x.copy()}
            plus[name][idx] += h
            minus = {**inp, name: x.copy()}
            minus[name][idx] -= h
            fd[idx] = (_objective(plus, go, gbf) - _objective(minus, go, gbf)) / (2 * h)
        scale = max(1.0, float(np.max(np.abs(fd))))
        assert np.max(np.abs(got[name] - fd)) <= 1e-7 * scale, name


def test_one_token_closed_form():
    """One token, one write and one read of the same row b: new = e^g b (1 - beta k^2) + k beta v
    and out = q new, so dJ/dv = q k beta go, dJ/dq = <go, new>, dJ/dbeta = q k <go, v - k e^g b>,
    dJ/db = q e^g (1 - beta k^2) go, dJ/dk = q <go, beta v - 2 k beta e^g b>,
    dJ/dg = q (1 - beta k^2) e^g <go, b>."""
    b = np.array([0.5, -1.25, 2.0])
    v = np.array([1.0, 0.25, -0.5])
    k, q, beta, g = 0.75, -1.5, 0.6, -0.3
    go = np.array([0.3, -0.7, 1.1])
    inp = dict(bank=b[None, None], k_idx=np.array([[[1]]], np.int32), k_val=np.array([[[k]]]), v=v[None, None],
               beta=np.array([[beta]]), g=np.array([[[g]]]), q_idx=np.array([[[1]]], np.int32),
               q_val=np.array([[[q]]]), valid=np.array([1], np.int32))
    inp["bank"] = np.stack([np.zeros(3), b, np.zeros(3)])[None]           # M = 3, row 1 is b
    got = oracle.token_loop_backward(inp, go[None, None])
    e = math.exp(g)
    new = e * b * (1 - beta * k * k) + k * beta * v
    np.testing.assert_allclose(got["v"][0, 0], q * k * beta * go, rtol=1e-14)
    np.testing.assert_allclose(got["q_val"][0, 0, 0], go @ new, rtol=1e-14)
    np.testing.assert_allclose(got["beta"][0, 0], q * k * go @ (v - k * e * b), rtol=1e-14)
    np.testing.assert_allclose(got["bank"][0, 1], q * e * (1 - beta * k * k) * go, rtol=1e-14)
    np.testing.assert_allclose(got["k_val"][0, 0, 0], q * go @ (beta * v - 2 * k * beta * e * b), rtol=1e-14)
    np.testing.assert_allclose(got["g"][0, 0, 0], q * (1 - beta * k * k) * e * (go @ b), rtol=1e-14)
    assert not got["bank"][0, 0].any() and not got["bank"][0, 2].any()


def test_linear_in_the_output_gradients():
    inp = _inputs(5, P=1, T=9, W=3, R=2, hd=4, M=7)
    rng = np.random.default_rng(7)
    go1, go2 = rng.normal(size=(2,) + inp["v"].shape)
    gb1, gb2 = rng.normal(size=(2,) + inp["bank"].shape)
    a = oracle.token_loop_backward(inp, go1, gb1)
    b = oracle.token_loop_backward(inp, go2, gb2)
    c = oracle.token_loop_backward(inp, 2 * go1 - 3 * go2, 2 * gb1 - 3 * gb2)
    for name in FD_NAMES:
        np.testing.assert_allclose(c[name], 2 * a[name] - 3 * b[name], rtol=1e-10, atol=1e-12)


def test_padding_tokens_and_untouched_rows():
    """Padding tokens get zero gradients (they take part in nothing), and the gradient of a
    row no live token selects is the final-bank gradient of that row."""
    inp = _inputs(9, P=2, T=8, W=2, R=2, hd=3, M=12)
    inp["valid"] = np.array([5, 0], np.int32)
    rng = np.random.default_rng(11)
    go, gbf = rng.normal(size=inp["v"].shape), rng.normal(size=inp["bank"].shape)
    got = oracle.token_loop_backward(inp, go, gbf)
    for name in ("k_val", "v", "beta", "g", "q_val"):
        assert not got[name][0, 5:].any() and not got[name][1].any()
    np.testing.assert_array_equal(got["bank"][1], gbf[1])
    used = set(inp["k_idx"][0, :5].ravel().tolist()) | set(inp["q_idx"][0, :5].ravel().tolist())
    for s in set(range(12)) - used:
        np.testing.assert_array_equal(got["bank"][0, s], gbf[0, s])


def test_per_token_gate_is_the_sum_of_per_slot_gates():
    """G = 1 applies one log-decay to each write of a token: its gradient is the sum of the
    per-slot gradients of the same loop run with that value repeated W times."""
    inp1 = _inputs(13, P=2, T=9, W=3, R=2, hd=4, M=6, G=1)
    inpw = {**inp1, "g": np.repeat(inp1["g"], 3, axis=2)}
    rng = np.random.default_rng(17)
    go, gbf = rng.normal(size=inp1["v"].shape), rng.normal(size=inp1["bank"].shape)
    a = oracle.token_loop_backward(inp1, go, gbf)
    b = oracle.token_loop_backward(inpw, go, gbf)
    np.testing.assert_allclose(a["g"][..., 0], b["g"].sum(axis=2), rtol=1e-12, atol=1e-14)
    for name in ("bank", "k_val", "v", "beta", "q_val"):
        np.testing.assert_allclose(a[name], b[name], rtol=1e-12, atol=1e-14)


def test_rejects_repeated_write_slots():
    inp = _inputs(21, P=1, T=3, W=2)
    inp["k_idx"][0, 1, 1] = inp["k_idx"][0, 1, 0]
    with pytest.raises(ValueError, match="repeated"):
        oracle.token_loop_backward(inp, np.zeros_like(inp["v"]))


# ------------------------------------------------------------------ bfloat16 snapshot rows

def _write_once_inputs(seed, P=2, T=6, W=3, R=3, hd=4):
    """fp64 inputs in which every slot is written by at most one token of its stream (slot
    ids of token t are t * W .. t * W + W - 1, shuffled), so that each saved row is the row
    the forward started from."""
    rng = np.random.default_rng(seed)
    M = T * W + 3
    k_idx = np.stack([np.stack([rng.permutation(np.arange(t * W, t * W + W)) for t in range(T)])
                      for _ in range(P)]).astype(np.int32)
    return dict(
        bank=rng.normal(size=(P, M, hd)), k_idx=k_idx, k_val=rng.normal(size=(P, T, W)),
        v=rng.normal(size=(P, T, hd)), beta=1 / (1 + np.exp(-rng.normal(size=(P, T)))),
        g=rng.normal(-0.4, 0.3, (P, T, W)), q_idx=rng.integers(0, M, size=(P, T, R)).astype(np.int32),
        q_val=rng.normal(size=(P, T, R)), valid=np.array([T, T - 1][:P], dtype=np.int32))


SNAP_NAMES = ("bank", "k_val", "v", "beta", "g")   # every gradient but the read weights'


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_bf16_snapshot_is_the_gradient_from_rounded_saved_rows(seed):
    """With every slot written at most once, each saved row is the initial bank row, so
    keeping the snapshot as bfloat16 rows means working backwards from the bank rounded to
    bfloat16: every gradient except the read weights' equals plain O3 run on the rounded bank,
    bit for bit. A read weight's gradient is a dot product with the row read: a slot that a
    later token writes has been restored from its rounded saved row by then (O3 on the rounded
    bank reads the same value); any other row read is the forward's own (plain O3)."""
    inp = _write_once_inputs(seed)
    rng = np.random.default_rng(50 + seed)
    go = rng.normal(size=inp["v"].shape)
    gbf = rng.normal(size=inp["bank"].shape)
    got = oracle.token_loop_backward(inp, go, gbf, snapshot_quant="bf16")
    rounded = dict(inp, bank=oracle.round_bf16(inp["bank"]))
    want = oracle.token_loop_backward(rounded, go, gbf)
    plain = oracle.token_loop_backward(inp, go, gbf)
    assert not np.array_equal(rounded["bank"], inp["bank"])
    for name in SNAP_NAMES:
        assert np.array_equal(got[name], want[name]), name
    P, T, R = inp["q_idx"].shape
    for p in range(P):
        for t in range(int(inp["valid"][p])):
            later = set(inp["k_idx"][p, t + 1:int(inp["valid"][p])].ravel().tolist())
            for r in range(R):
                ref = want if int(inp["q_idx"][p, t, r]) in later else plain
                assert got["q_val"][p, t, r] == ref["q_val"][p, t, r], (p, t, r)
    assert any(not np.array_equal(got[n], plain[n]) for n in SNAP_NAMES)


def test_bf16_snapshot_of_a_bf16_exact_bank_reduces_to_o3():
    """Saved rows that are bfloat16 already (every slot written at most once, bank rows
    bfloat16-exact) are stored unchanged: the bf16 snapshot gives plain O3's gradients."""
    inp = _write_once_inputs(7)
    inp["bank"] = oracle.round_bf16(inp["bank"])
    rng = np.random.default_rng(57)
    go = rng.normal(size=inp["v"].shape)
    gbf = rng.normal(size=inp["bank"].shape)
    got = oracle.token_loop_backward(inp, go, gbf, snapshot_quant="bf16")
    want = oracle.token_loop_backward(inp, go, gbf)
    for name in FD_NAMES:
        assert np.array_equal(got[name], want[name]), name


def test_bf16_snapshot_changes_gradients_by_rounding_only():
    """Slots rewritten many times (M small): the rounded saved rows differ from the exact ones,
    so the gradients differ, by about the bfloat16 rounding of the rows (2^-8 relative)."""
    inp = _inputs(11, T=9, M=4)
    rng = np.random.default_rng(61)
    go = rng.normal(size=inp["v"].shape)
    gbf = rng.normal(size=inp["bank"].shape)
    got = oracle.token_loop_backward(inp, go, gbf, snapshot_quant="bf16")
    want = oracle.token_loop_backward(inp, go, gbf)
    diff = [np.max(np.abs(got[n] - want[n])) / max(np.max(np.abs(want[n])), 1e-300) for n in FD_NAMES]
    assert max(diff) > 0 and max(diff) < 3e-2, diff
