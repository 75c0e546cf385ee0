"""The backward (sdm_bwd through the C ABI) against the backward oracle O3 (the fp64
adjoint of the token loop, pinned by finite differences of the forward oracle).

Bar: infinity-norm relative error per gradient tensor within 1e-4 (the float32 bar of the
forward; the emulated float32 error of these sizes is ~1e-6), padding tokens exactly 0,
the bank restored bit for bit, bitwise-identical reruns."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import small
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

TOL = 1e-4
NAMES = {"bank": "bank", "v": "v", "beta": "beta", "log_decay": "g", "k_val": "k_val", "q_val": "q_val"}


def _grad_out(gr, dtype, gpu):
    """grad_out in the bank dtype on the GPU; gr["grad_out"] becomes its exact float32 value."""
    if dtype == "bf16":
        bits = workloads.round_bf16_bits(gr["grad_out"])
        gr["grad_out"] = workloads.bf16_bits_to_f32(bits)
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(gpu)
    return torch.from_numpy(gr["grad_out"]).to(gpu)


def _run(wl, gpu, seed=0, bank_grad=True, dup_reads=False, id64=False, snapshot_quant="none", write_once=False):
    inp = gu.generate(wl)
    if dup_reads and wl.R > 1:
        inp["q_idx"][:, ::2, -1] = inp["q_idx"][:, ::2, 0]
    if write_once:   # token t writes slots t W .. t W + W - 1 (shuffled): each row written at most once
        assert wl.M >= wl.T * wl.W
        rng = np.random.default_rng(wl.index)
        inp["k_idx"] = np.stack([np.stack([rng.permutation(np.arange(t * wl.W, (t + 1) * wl.W)) for t in range(wl.T)])
                                 for _ in range(wl.P)]).astype(np.int32)
    gr = workloads.grad_inputs(wl, seed, bank_grad)
    t = gu.to_torch(inp, gpu)
    if id64:
        t["k_idx"], t["q_idx"] = t["k_idx"].long(), t["q_idx"].long()
    from chunked_sparse_delta_amd import sdm_bwd
    bank = t["bank"].clone()
    gb = None if gr["grad_bank"] is None else torch.from_numpy(gr["grad_bank"]).to(gpu)
    got = sdm_bwd(bank, t["k_idx"], t["k_val"], t["v"], t["beta"], t["log_decay"], t["q_idx"], t["q_val"],
                  _grad_out(gr, wl.dtype, gpu), grad_bank=gb, valid_tokens=t["valid"], snapshot_quant=snapshot_quant)
    torch.cuda.synchronize()
    return inp, gr, t, bank, got


def _check(inp, gr, got, streams=None, snapshot_quant="none", tol=TOL):
    f = oracle.as_f64_inputs(inp)
    want = oracle.token_loop_backward(f, gr["grad_out"], gr["grad_bank"], threads=8, streams=streams,
                                      snapshot_quant=snapshot_quant)
    if streams is not None:
        want = {k: v[list(streams)] for k, v in want.items()}
    for k, ok in NAMES.items():
        g = gu.f64(got[k] if streams is None else got[k][list(streams)])
        w = want[ok]
        assert g.shape == w.shape, k
        assert gu.rel_err(g, w) <= tol, (k, gu.rel_err(g, w))
    valid = inp["valid"]
    for p in (range(inp["valid"].shape[0]) if streams is None else streams):
        n = int(valid[p])
        for k in ("v", "beta", "log_decay", "k_val", "q_val"):
            assert not gu.f64(got[k][p, n:]).any(), (k, p)


CASES = [
    small(P=2, T=37, C=16, hd=8, M=24, W=3, R=2),
    small(P=3, T=50, C=16, hd=10, M=9, W=4, R=5, ragged=True, index=11),               # ragged hd, many repeats
    small(P=2, T=40, C=16, hd=70, M=30, W=5, R=3, gate_width=1, index=12),             # G = 1, several slices
    small(P=1, T=64, C=16, hd=16, M=6, W=3, R=4, decay_scale=1.5, index=13),           # strong decays
    small(P=2, T=30, C=16, hd=33, M=300, W=40, R=70, ids="zipf", index=14),            # W, R above one pass
    small(P=4, T=20, C=16, hd=1, M=5, W=2, R=1, index=15),                             # one column
    small(P=2, T=25, C=16, hd=64, M=512, W=256, R=256, index=16),                      # widest entries
    small(P=2, T=40, C=16, hd=12, M=300, W=20, R=30, ragged=True, index=20),           # 2 entries per lane
    small(P=1, T=30, C=16, hd=20, M=400, W=50, R=64, index=21),                        # 4 entries per lane
    small(P=2, T=37, C=16, hd=24, M=30, W=3, R=4, dtype="bf16", ragged=True, index=23),  # bfloat16 bank
    small(P=3, T=30, C=16, hd=16, M=200, W=20, R=6, dtype="bf16", ids="zipf", gate_width=1, index=24),
    small(P=1, T=1, C=16, hd=8, M=1, W=1, R=1, index=27),                                # one token, one row
    small(P=1, T=20, C=16, hd=1024, M=30, W=3, R=3, dtype="bf16", index=28),             # wide head
]


@pytest.fixture(params=["pair", "lds", "memory", "block"])
def residency(request, monkeypatch):
    """pair: the default (slices in LDS where they fit, tokens in pairs where a token's entries
    fill at most half the entry groups); lds: slices in LDS, one token per step
    (SDM_BWD_PAIR=0); memory: one wavefront per slice on rows in memory where a lane covers
    its entries in at most 8, else the 256-thread sweep (SDM_BWD_RES=0); block: always the
    256-thread sweep (SDM_BWD_RES=0, SDM_BWD_WAVE=0)."""
    for var in ("SDM_BWD_RES", "SDM_BWD_PAIR", "SDM_BWD_WAVE"):
        monkeypatch.delenv(var, raising=False)
    if request.param in ("memory", "block"):
        monkeypatch.setenv("SDM_BWD_RES", "0")
    if request.param == "block":
        monkeypatch.setenv("SDM_BWD_WAVE", "0")
    elif request.param == "lds":
        monkeypatch.setenv("SDM_BWD_PAIR", "0")
    return request.param


@pytest.mark.parametrize("wl", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_backward_matches_oracle(gpu, wl, residency):
    inp, gr, t, bank, got = _run(wl, gpu, dup_reads=True)
    _check(inp, gr, got)
    assert np.array_equal(gu.bits(bank), gu.bits(t["bank"])), "bank not restored bit for bit"


def test_backward_without_bank_gradient_int64_ids(gpu):
    wl = small(P=2, T=45, C=16, hd=12, M=20, W=3, R=3, ragged=True, index=17)
    inp, gr, t, bank, got = _run(wl, gpu, bank_grad=False, id64=True)
    _check(inp, gr, got)


def test_backward_all_padding_stream(gpu):
    wl = small(P=3, T=20, C=16, hd=8, M=10, W=2, R=2, index=18)
    inp = gu.generate(wl)
    inp["valid"] = np.array([20, 0, 7], np.int32)
    gr = workloads.grad_inputs(wl, 1)
    t = gu.to_torch(inp, gpu)
    from chunked_sparse_delta_amd import sdm_bwd
    got = sdm_bwd(t["bank"].clone(), t["k_idx"], t["k_val"], t["v"], t["beta"], t["log_decay"], t["q_idx"],
                  t["q_val"], torch.from_numpy(gr["grad_out"]).to(gpu),
                  grad_bank=torch.from_numpy(gr["grad_bank"]).to(gpu), valid_tokens=t["valid"])
    torch.cuda.synchronize()
    _check(inp, gr, got)
    assert np.array_equal(gu.f64(got["bank"])[1], gr["grad_bank"][1].astype(np.float64))


def test_backward_reruns_are_bitwise_and_slices_agree(gpu, monkeypatch):
    wl = small(P=2, T=60, C=16, hd=96, M=40, W=6, R=5, ragged=True, index=19)
    runs = []
    for sl, res in ((None, None), (None, None), ("64", None), ("4", None), (None, "0")):
        for var, val in (("SDM_BWD_SLICE", sl), ("SDM_BWD_RES", res)):
            if val is None:
                monkeypatch.delenv(var, raising=False)
            else:
                monkeypatch.setenv(var, val)
        runs.append(_run(wl, gpu, seed=3)[4])
    for k in NAMES:
        assert np.array_equal(gu.bits(runs[0][k]), gu.bits(runs[1][k])), k
        for r in runs[2:]:
            assert gu.rel_err(gu.f64(r[k]), gu.f64(runs[0][k])) <= 1e-5, k


@pytest.mark.parametrize("cfg,streams", [("2", (0, 17, 31)), ("3", (0, 9, 15))])
def test_backward_full_size_sampled_streams(gpu, cfg, streams):
    """Configs 2 (bfloat16 bank, Zipf slots, 32 + 32 per token) and 3 (float32, ragged, 64 + 64
    per token) at full size through the one-wavefront sweep on rows in memory; every gradient
    of sampled streams against O3 (each stream's gradients depend on that stream alone)."""
    wl = workloads.CONFIGS[cfg]
    inp, gr, t, bank, got = _run(wl, gpu)
    _check(inp, gr, got, streams=streams)
    assert np.array_equal(gu.bits(bank), gu.bits(t["bank"]))


def test_backward_config1_shape_full_size(gpu, residency):
    """The benchmarked backward workload: config 1's shapes (8 streams x 2048 tokens, head 64,
    4096 rows, 8 + 8 slots) with a float32 bank, every gradient against O3 (the bench runs
    the LDS-resident sweep)."""
    wl = workloads.CONFIGS["1"].replace(dtype="f32")
    inp, gr, t, bank, got = _run(wl, gpu)
    _check(inp, gr, got)
    assert np.array_equal(gu.bits(bank), gu.bits(t["bank"]))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_shared_bank_matches_per_stream_banks(gpu, dtype, monkeypatch):
    """One bank shared by every stream, the streams' slots interleaved and disjoint (the
    forward's shared-bank contract): every gradient equals that of per-stream banks bit for
    bit (the sweep in memory on both sides; a shared bank never takes the resident sweep,
    whose whole-slice write-back would overwrite the other streams' rows)."""
    from chunked_sparse_delta_amd import sdm_bwd
    monkeypatch.setenv("SDM_BWD_RES", "0")
    wl = small(P=3, T=40, C=16, hd=20, M=25, W=3, R=4, dtype=dtype, ragged=True, index=25)
    inp, gr, t, bank, got = _run(wl, gpu, dup_reads=True)
    _check(inp, gr, got)
    sh = gu.to_torch(dict(workloads.shared_bank_inputs(inp), dtype=dtype), gpu)
    P, M, hd = wl.P, wl.M, wl.hd
    gbs = torch.from_numpy(np.ascontiguousarray(
        workloads.shared_bank_inputs(dict(inp, bank=gr["grad_bank"]))["bank"])).to(gpu)
    bank_sh = sh["bank"].clone()
    got2 = sdm_bwd(bank_sh, sh["k_idx"], sh["k_val"], sh["v"], sh["beta"], sh["log_decay"], sh["q_idx"], sh["q_val"],
                   _grad_out(dict(gr), dtype, gpu), grad_bank=gbs, valid_tokens=sh["valid"], shared_bank=True)
    torch.cuda.synchronize()
    assert got2["bank"].shape == (M * P, hd)
    assert np.array_equal(gu.bits(got2["bank"].reshape(M, P, hd).permute(1, 0, 2).contiguous()),
                          gu.bits(got["bank"]))
    for k in ("v", "beta", "log_decay", "k_val", "q_val"):
        assert np.array_equal(gu.bits(got2[k]), gu.bits(got[k])), k
    assert np.array_equal(gu.bits(bank_sh), gu.bits(sh["bank"]))


@pytest.mark.parametrize("S", ["8", "16", "32", "64"])
def test_backward_wide_slices(gpu, S, monkeypatch):
    """Slices of 8..64 columns: the resident sweep's column sums take every lane-exchange
    width (quad swaps, half-row and row mirrors, 16- and 32-lane shuffles); the sweep in
    memory runs the same shapes."""
    wl = small(P=2, T=33, C=16, hd=100, M=60, W=3, R=4, ragged=True, index=22)
    monkeypatch.setenv("SDM_BWD_SLICE", S)
    for res, wave in ((None, None), ("0", None), ("0", "0")):
        for var, val in (("SDM_BWD_RES", res), ("SDM_BWD_WAVE", wave)):
            if val is None:
                monkeypatch.delenv(var, raising=False)
            else:
                monkeypatch.setenv(var, val)
        inp, gr, t, bank, got = _run(wl, gpu, seed=int(S), dup_reads=True)
        _check(inp, gr, got)
        assert np.array_equal(gu.bits(bank), gu.bits(t["bank"]))


@pytest.mark.parametrize("T,M,dtype", [(37, 12, "f32"), (64, 2000, "f32"), (63, 40, "bf16"), (70, 9, "f32"),
                                       (2, 30, "f32"), (1, 30, "f32")])
def test_backward_token_pairs_give_the_same_bits(gpu, T, M, dtype, monkeypatch):
    """Tokens taken in pairs (one step for a pair selecting disjoint rows, two masked steps
    otherwise; a small bank makes many pairs dependent) give exactly the bits of the resident
    sweep taking one token per step, for every remainder of pairs modulo the prefetch depth
    and odd, ragged and single-token streams; both match the oracle."""
    wl = small(P=3, T=T, C=16, hd=12, M=M, W=4, R=3, dtype=dtype, ragged=T > 2, index=26)
    runs = []
    for pair in (None, "0"):
        monkeypatch.delenv("SDM_BWD_RES", raising=False)
        if pair is None:
            monkeypatch.delenv("SDM_BWD_PAIR", raising=False)
        else:
            monkeypatch.setenv("SDM_BWD_PAIR", pair)
        inp, gr, t, bank, got = _run(wl, gpu, seed=T, dup_reads=True)
        _check(inp, gr, got)
        runs.append(got)
    for k in NAMES:
        assert np.array_equal(gu.bits(runs[0][k]), gu.bits(runs[1][k])), k


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_sdm_write_read_autograd(gpu, dtype):
    """sdm_write_read under autograd: the readings equal sdm_fwd's bit for bit, the bank is
    advanced in place the same way, and torch.autograd.grad gives sdm_bwd's gradients (cast
    to the inputs' dtypes) for the float inputs that require grad."""
    from chunked_sparse_delta_amd import sdm_bwd, sdm_fwd, sdm_write_read
    wl = small(P=2, T=45, C=16, hd=16, M=20, W=3, R=4, dtype=dtype, ragged=True, index=29)
    inp = gu.generate(wl)
    gr = workloads.grad_inputs(wl, 2, bank_grad=False)
    t = gu.to_torch(inp, gpu)
    go = _grad_out(gr, dtype, gpu)
    leaves = {k: t[k].clone().requires_grad_(True) for k in ("k_val", "v", "beta", "log_decay", "q_val")}
    bank_a, bank_b, bank_c = t["bank"].clone(), t["bank"].clone(), t["bank"].clone()
    out = sdm_write_read(bank_a, t["k_idx"], leaves["k_val"], leaves["v"], leaves["beta"], leaves["log_decay"],
                         t["q_idx"], leaves["q_val"], chunk=16, valid_tokens=t["valid"])
    grads = torch.autograd.grad(out, [leaves[k] for k in ("k_val", "v", "beta", "log_decay")], grad_outputs=go)
    ref = sdm_fwd(bank_b, t["k_idx"], t["k_val"], t["v"], t["beta"], t["log_decay"], t["q_idx"], t["q_val"],
                  chunk=16, valid_tokens=t["valid"])
    want = sdm_bwd(bank_c, t["k_idx"], t["k_val"], t["v"], t["beta"], t["log_decay"], t["q_idx"], t["q_val"], go,
                   valid_tokens=t["valid"])
    torch.cuda.synchronize()
    assert np.array_equal(gu.bits(out), gu.bits(ref)) and np.array_equal(gu.bits(bank_a), gu.bits(bank_b))
    for g, k in zip(grads, ("k_val", "v", "beta", "log_decay")):
        assert g.dtype == leaves[k].dtype
        assert np.array_equal(gu.bits(g), gu.bits(want[k].to(g.dtype))), k
    with pytest.raises(ValueError, match="must not require grad"):
        sdm_write_read(t["bank"].clone().requires_grad_(True), t["k_idx"], leaves["k_val"], leaves["v"],
                       leaves["beta"], leaves["log_decay"], t["q_idx"], leaves["q_val"], chunk=16)


# ------------------------------------------------------------------ bfloat16 snapshot rows

# Where a saved row is the result of arithmetic (a row written before), the kernel rounds
# its float32 value to bfloat16 and the oracle its fp64 value: the two sides can land on
# neighbouring bfloat16 values when the exact row sits within float32 error of a rounding
# boundary, so a restored element may differ by one bfloat16 ulp (2^-8 relative). Rows
# written once are saved as the bank's own rows (no arithmetic): both sides round the same
# value, and the float32 bar holds.
TOL_SNAP = 2.0 ** -8

SNAP_CASES = [
    small(P=3, T=50, C=16, hd=10, M=9, W=4, R=5, ragged=True, index=11),               # rows rewritten often
    small(P=2, T=40, C=16, hd=70, M=30, W=5, R=3, gate_width=1, index=12),             # several slices
    small(P=2, T=30, C=16, hd=33, M=300, W=40, R=70, ids="zipf", index=14),            # W, R above one pass
    small(P=2, T=40, C=16, hd=12, M=300, W=20, R=30, ragged=True, index=20),           # 2 entries per lane
]
ONCE_CASES = [
    small(P=2, T=40, C=16, hd=24, M=200, W=4, R=5, ragged=True, index=31),
    small(P=2, T=12, C=16, hd=33, M=500, W=40, R=70, index=32),
]


def _check_restored_bank(inp, wl, bank):
    """The bank comes back with the rows the forward wrote rounded to bfloat16 (nearest
    even) and the others bit for bit."""
    b0 = np.ascontiguousarray(inp["bank"], dtype=np.float32)
    want = b0.copy()
    for p in range(wl.P):
        rows = np.unique(inp["k_idx"][p, :int(inp["valid"][p])])
        want[p, rows] = workloads.bf16_bits_to_f32(workloads.round_bf16_bits(b0[p, rows]))
    assert np.array_equal(gu.bits(bank), want.view(np.int32)), "bank not restored to the rounded snapshot rows"


@pytest.mark.parametrize("wl", SNAP_CASES, ids=[f"c{i}" for i in range(len(SNAP_CASES))])
def test_backward_bf16_snapshot_matches_oracle(gpu, wl, residency):
    """snapshot_quant="bf16" on a float32 bank (sdm_write_read's argument, page 21): the saved
    rows are bfloat16, the gradients match the oracle's bf16-snapshot mode within one
    bfloat16 ulp of the saved rows, the bank comes back with the written rows rounded, and a
    rerun gives the same bits."""
    inp, gr, t, bank, got = _run(wl, gpu, dup_reads=True, snapshot_quant="bf16")
    _check(inp, gr, got, snapshot_quant="bf16", tol=TOL_SNAP)
    _check_restored_bank(inp, wl, bank)
    inp2, gr2, t2, bank2, got2 = _run(wl, gpu, dup_reads=True, snapshot_quant="bf16")
    for k in NAMES:
        assert np.array_equal(gu.bits(got[k]), gu.bits(got2[k])), k


@pytest.mark.parametrize("wl", ONCE_CASES, ids=[f"c{i}" for i in range(len(ONCE_CASES))])
def test_backward_bf16_snapshot_write_once_at_the_float32_bar(gpu, wl, residency):
    """Every row written at most once: the saved rows are the bank's rows, rounded the same way
    on both sides, and the bf16-snapshot gradients meet the float32 bar (1e-4)."""
    inp, gr, t, bank, got = _run(wl, gpu, dup_reads=True, snapshot_quant="bf16", write_once=True)
    _check(inp, gr, got, snapshot_quant="bf16")
    _check_restored_bank(inp, wl, bank)


def test_backward_bf16_snapshot_of_a_bf16_bank_is_none(gpu):
    """A bfloat16 bank runs snapshot_quant="bf16" as "none" (the pages' effective snapshot
    mode: its rows are bfloat16 already): the same bits."""
    wl = small(P=2, T=37, C=16, hd=24, M=30, W=3, R=4, dtype="bf16", ragged=True, index=23)
    _, _, _, _, a = _run(wl, gpu, snapshot_quant="none")
    _, _, _, _, b = _run(wl, gpu, snapshot_quant="bf16")
    for k in NAMES:
        assert np.array_equal(gu.bits(a[k]), gu.bits(b[k])), k


@pytest.mark.parametrize("mode", ["fp8", "int4"])
def test_backward_refuses_unscaled_snapshot_modes(gpu, mode):
    """fp8 and int4 snapshot rows are refused before any work (the pages give their row
    widths, not how values are scaled into them)."""
    from chunked_sparse_delta_amd import SdmError
    wl = small(P=1, T=10, C=16, hd=8, M=10, W=2, R=2, index=30)
    inp = gu.generate(wl)
    t = gu.to_torch(inp, gpu)
    from chunked_sparse_delta_amd import sdm_bwd
    bank = t["bank"].clone()
    go = torch.ones_like(t["v"])
    with pytest.raises(SdmError) as ei:
        sdm_bwd(bank, t["k_idx"], t["k_val"], t["v"], t["beta"], t["log_decay"], t["q_idx"], t["q_val"], go,
                valid_tokens=t["valid"], snapshot_quant=mode)
    assert ei.value.code == -7
    assert np.array_equal(gu.bits(bank), gu.bits(t["bank"]))
