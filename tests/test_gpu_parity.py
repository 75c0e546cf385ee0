"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the GPU.

Bar: infinity-norm relative error per output tensor (readings, final bank) within 1e-4
for float32 banks and 2e-2 for bfloat16 banks; padding rows exactly +0; bitwise-identical
reruns."""

import numpy as np
import pytest
import torch

import workloads
from workloads import small
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ the solve on its own

@pytest.mark.parametrize("C", [1, 16, 37, 64, 65, 128, 200, 256])
def test_wy_solve_matches_inverse(gpu, C):
    from chunked_sparse_delta_amd import wy_solve
    rng = np.random.default_rng(C)
    n = 3
    A = rng.uniform(0.0, 2.0 / np.sqrt(C), (n, C, C)).astype(np.float32)
    A[:, np.triu_indices(C)[0], np.triu_indices(C)[1]] = np.nan   # never read
    QK = rng.normal(size=(n, C, C)).astype(np.float32)
    QK[:, np.triu_indices(C, 1)[0], np.triu_indices(C, 1)[1]] = np.nan
    beta = rng.uniform(0, 1, (n, C)).astype(np.float32)
    X, QX = wy_solve(torch.from_numpy(A).to(gpu), torch.from_numpy(beta).to(gpu), torch.from_numpy(QK).to(gpu))
    X, QX = X.cpu().numpy(), QX.cpu().numpy()
    for k in range(n):
        Lm = np.tril(beta[k, :, None].astype(np.float64) * np.nan_to_num(A[k].astype(np.float64)), -1)
        Xr = np.linalg.inv(np.eye(C) + Lm)
        QXr = np.tril(np.nan_to_num(QK[k].astype(np.float64))) @ Xr
        assert gu.rel_err(X[k].astype(np.float64), np.tril(Xr)) < 1e-5
        assert gu.rel_err(QX[k].astype(np.float64), np.tril(QXr)) < 1e-5
        up = np.triu_indices(C, 1)
        assert np.all(X[k][up] == 0) and not np.signbit(X[k][up]).any()
        assert np.all(QX[k][up] == 0) and not np.signbit(QX[k][up]).any()
        assert np.all(np.diag(X[k]) == 1.0)


# ------------------------------------------------------------------ Phase 1 and the solve vs the chunk algebra

@pytest.mark.parametrize("wl", [
    small(P=2, T=37, C=16, hd=8, M=12, W=3, R=2),
    small(P=1, T=40, C=20, hd=8, M=9, W=4, R=3, gate_width=1, ragged=True, index=3),
    small(P=2, T=33, C=32, hd=8, M=30, W=5, R=4, dtype="bf16", ids="zipf", index=4),
    # every slot written ~30 times per chunk: all groups hot (dense Gram on the matrix cores)
    small(P=2, T=70, C=64, hd=8, M=6, W=3, R=3, index=5),
    # Zipf: hot head, cold tail, in one chunk
    small(P=1, T=96, C=48, hd=8, M=40, W=5, R=4, ids="zipf", zipf_s=1.3, ragged=True, index=6),
    # large log-decays: big groups whose decay span exceeds the dense path's bound stay cold
    small(P=1, T=64, C=64, hd=8, M=5, W=2, R=2, decay_scale=4.0, index=8),
    # chunks of more than 1024 entries: Phase 1 in slot partitions (or by sorting)
    small(P=1, T=60, C=32, hd=8, M=300, W=40, R=36, ids="zipf", ragged=True, index=43),
    small(P=1, T=48, C=48, hd=8, M=500, W=24, R=24, ids="mixed", weight_scale=-1.0, index=44),
    small(P=1, T=64, C=32, hd=8, M=60, W=40, R=40, index=45),
], ids=["tiny", "gate1", "bf16zipf", "allhot", "mixed", "bigdecay", "part_zipf", "part_mixed", "part_fewslots"])
@pytest.mark.parametrize("part", ["1", "1:3", "0"])
def test_chunk_intermediates_match_chunk_algebra(gpu, wl, part, monkeypatch):
    """Phase 1 and the solve against O2's chunk algebra, on every Phase-1 path: fused (small
    chunks), in slot partitions (default count, or 8), and by sorting."""
    monkeypatch.setenv("SDM_P1_PART", part[0])
    if ":" in part:
        monkeypatch.setenv("SDM_P1_NP_LOG", part.split(":")[1])
    else:
        monkeypatch.delenv("SDM_P1_NP_LOG", raising=False)
    import oracle
    from oracle import chunk_algebra
    from chunked_sparse_delta_amd import chunk_mats
    inp = gu.generate(wl)
    f = oracle.as_f64_inputs(inp)
    _, _, inter = chunk_algebra.forward(f, wl.C, emit=True)
    t = gu.to_torch(inp, gpu)
    res = chunk_mats(t["k_idx"], t["k_val"], t["beta"], t["log_decay"], t["q_idx"], t["q_val"], rows=wl.M,
                     head_dim=wl.hd, chunk=wl.C, valid_tokens=t["valid"])
    res = {k: v.cpu().numpy().astype(np.float64) for k, v in res.items()}
    Nt = wl.Nt
    for p in range(wl.P):
        for ti in range(Nt):
            c = inter[p][ti]
            n = p * Nt + ti
            for key, ref in (("A", np.tril(c["A"], -1)), ("QK", np.tril(c["QK"])), ("X", c["X"]), ("QX", c["QX"]),
                             ("gw", c["gw"]), ("gr", c["gr"])):
                got = res[key][n]
                assert gu.rel_err(got, ref) < 2e-5, (p, ti, key, gu.rel_err(got, ref))
            up = np.triu_indices(wl.C, 1)
            for key in ("QK", "X", "QX"):
                assert np.all(res[key][n][up] == 0), (p, ti, key)
            assert np.all(res["A"][n][np.triu_indices(wl.C)] == 0)


def _check_records(rec, n, kc, qc, nl, want_groups, want_only, what):
    """Phase 1's integer records of chunk n against the definition: the write groups (each
    slot's write entries in token order), the single-member flags, each write entry's place
    and group, and each read's latest write of its slot at or before its token, exactly."""
    C, W = kc.shape
    R = qc.shape[1]
    meta = rec["meta"][n]
    El = nl * W
    assert meta[0] == nl and meta[1] == El and meta[2] == len(want_groups), (what, meta)
    spk = rec["spk"][n][:El]
    grec = rec["grec"][n][:meta[2]]
    got, first_of, size_of, covered = {}, {}, {}, np.zeros(El, dtype=np.int64)
    for r in grec:
        slot, y = int(r[0]), int(r[1])
        first, cnt, t0 = y & 0xFFFF, ((y >> 16) & 0xFF) + 1, (y >> 24) & 0xFF
        mem = spk[first:first + cnt]
        assert np.all(mem[:, 0] == slot) and int(mem[0, 1]) == t0, (what, slot)
        got[slot] = [int(t) for t in mem[:, 1]]
        first_of[slot], size_of[slot] = first, cnt
        covered[first:first + cnt] += 1
    assert np.all(covered == 1), what   # the groups tile the sorted positions
    assert got == {s: [t for t, _ in m] for s, m in want_groups.items()}, what
    hot = set()
    for t in range(nl):
        for w in range(W):
            slot = int(kc[t, w])
            assert (size_of[slot] == 1) == bool(want_only[t, w]), (what, t, w)
            e = rec["ecr"][n][t, w]
            m = int(e[1])
            assert int(spk[m, 0]) == slot and int(spk[m, 1]) == t, (what, t, w)
            if int(e[0]) == m and int(e[2]) == 0 and int(e[3]) == 0:
                hot.add(slot)
            else:
                assert int(e[0]) == first_of[slot] and slot not in hot, (what, t, w)
    assert len(hot) == meta[3] and all(size_of[s] >= 16 for s in hot), what
    for t in range(C):
        for r in range(R):
            e = rec["rcr"][n][t, r]
            if t >= nl:
                assert not e.any(), (what, t, r)
                continue
            q = int(qc[t, r])
            latest = max([tt for tt, _ in want_groups.get(q, []) if tt <= t], default=None)
            if e.any():
                assert latest is not None and q not in hot, (what, t, r)
                assert int(e[0]) == first_of[q], (what, t, r)
                assert int(spk[int(e[1]) - 1, 0]) == q and int(spk[int(e[1]) - 1, 1]) == latest, (what, t, r)
            else:
                assert latest is None or q in hot, (what, t, r)


@pytest.mark.parametrize("wl", [
    small(P=2, T=37, C=16, hd=8, M=12, W=3, R=2),
    small(P=2, T=33, C=32, hd=8, M=30, W=5, R=4, dtype="bf16", ids="zipf", index=4),
    small(P=2, T=70, C=64, hd=8, M=6, W=3, R=3, index=5),
    small(P=1, T=96, C=48, hd=8, M=40, W=5, R=4, ids="zipf", zipf_s=1.3, ragged=True, index=6),
    small(P=1, T=60, C=32, hd=8, M=300, W=40, R=36, ids="zipf", ragged=True, index=43),
    small(P=1, T=64, C=32, hd=8, M=60, W=40, R=40, index=45),
], ids=["tiny", "bf16zipf", "allhot", "mixed", "part_zipf", "part_fewslots"])
@pytest.mark.parametrize("part", ["1", "1:3", "0"])
def test_phase1_records_match_the_chunk_algebra(gpu, wl, part, monkeypatch):
    """Phase 1's integer outputs bit-exactly against O2's groups and single-member flags, on
    every Phase-1 path (fused small chunks, slot partitions, sorting)."""
    import oracle
    from oracle import chunk_algebra
    from chunked_sparse_delta_amd import chunk_records
    monkeypatch.setenv("SDM_P1_PART", part[0])
    if ":" in part:
        monkeypatch.setenv("SDM_P1_NP_LOG", part.split(":")[1])
    else:
        monkeypatch.delenv("SDM_P1_NP_LOG", raising=False)
    inp = gu.generate(wl)
    f = oracle.as_f64_inputs(inp)
    _, _, inter = chunk_algebra.forward(f, wl.C, emit=True)
    t = gu.to_torch(inp, gpu)
    rec = chunk_records(t["k_idx"], t["k_val"], t["beta"], t["log_decay"], t["q_idx"], t["q_val"], rows=wl.M,
                        head_dim=wl.hd, chunk=wl.C, valid_tokens=t["valid"])
    rec = {k: v.cpu().numpy() for k, v in rec.items()}
    for p in range(wl.P):
        nv = int(inp["valid"][p])
        for ti in range(wl.Nt):
            nl = max(0, min(wl.C, nv - ti * wl.C))
            kc = np.zeros((wl.C, wl.W), np.int64)
            qc = np.zeros((wl.C, wl.R), np.int64)
            kc[:nl] = inp["k_idx"][p, ti * wl.C:ti * wl.C + nl]
            qc[:nl] = inp["q_idx"][p, ti * wl.C:ti * wl.C + nl]
            c = inter[p][ti]
            _check_records(rec, p * wl.Nt + ti, kc, qc, nl, c["groups"], c["is_only"], (p, ti))


def test_phase1_records_of_a_full_size_config_4p_stream(gpu):
    """Config 4's shapes (chunk 256, 256 write and 256 read slots per token, half Zipf): the
    records of every chunk of one stream against the grouping computed from the ids directly."""
    from chunked_sparse_delta_amd import chunk_records
    wl = workloads.CONFIGS["4p"]
    inp = gu.generate(wl, streams=[0])
    t = gu.to_torch(inp, gpu)
    rec = chunk_records(t["k_idx"], t["k_val"], t["beta"], t["log_decay"], t["q_idx"], t["q_val"], rows=wl.M,
                        head_dim=wl.hd, chunk=wl.C, valid_tokens=t["valid"])
    rec = {k: v.cpu().numpy() for k, v in rec.items()}
    assert rec["meta"][:, 7].max() == 0   # every chunk ran in LDS slot partitions
    for ti in (0, 7, wl.Nt - 1):
        kc = inp["k_idx"][0, ti * wl.C:(ti + 1) * wl.C].astype(np.int64)
        qc = inp["q_idx"][0, ti * wl.C:(ti + 1) * wl.C].astype(np.int64)
        groups = {}
        for tt in range(wl.C):
            for w in range(wl.W):
                groups.setdefault(int(kc[tt, w]), []).append((tt, w))
        only = np.vectorize(lambda s: len(groups[int(s)]) == 1)(kc)
        _check_records(rec, ti, kc, qc, wl.C, groups, only, ("4p", ti))


# ------------------------------------------------------------------ end to end, small shapes

SMALL = [
    small(P=2, T=37, C=16, hd=8, M=24, W=3, R=2, index=10),                                  # ragged last chunk
    small(P=3, T=100, C=32, hd=64, M=40, W=5, R=4, dtype="bf16", ids="zipf", index=11),
    small(P=2, T=64, C=64, hd=3, M=20, W=2, R=3, index=12),                                  # scalar path, f32
    small(P=2, T=70, C=17, hd=5, M=30, W=4, R=4, dtype="bf16", ragged=True, index=13),       # odd C, scalar bf16
    small(P=1, T=300, C=128, hd=16, M=300, W=16, R=8, ids="zipf", ragged=True, weight_scale=-1.0, index=14),
    small(P=2, T=513, C=256, hd=32, M=1000, W=32, R=32, ids="mixed", weight_scale=-1.0, index=15),
    small(P=2, T=50, C=16, hd=8, M=30, W=3, R=3, gate_width=1, index=16),                    # one gate per token
    small(P=8, T=130, C=100, hd=8, M=60, W=4, R=4, index=17, ragged=True),                   # P % 8 == 0 layout
    small(P=16, T=96, C=48, hd=24, M=100, W=6, R=6, dtype="bf16", index=18),
    small(P=1, T=16, C=16, hd=4, M=2, W=1, R=1, index=19),                                   # one chunk, tiny bank
    small(P=2, T=200, C=64, hd=256, M=300, W=256, R=256, dtype="bf16", weight_scale=-1.0, index=20),  # max width
    small(P=1, T=1, C=16, hd=8, M=1, W=1, R=1, index=40),                                     # one token, one row
    small(P=2, T=5, C=64, hd=16, M=10, W=2, R=2, ragged=True, index=41),                     # shorter than a chunk
    small(P=1, T=40, C=16, hd=1024, M=30, W=3, R=3, dtype="bf16", index=42),                 # wide head
    # bfloat16 rows of one column: one reading rounded to the neighbouring bfloat16 value is
    # a whole row's error, one ulp (up to 2^-7 of the value)
    small(P=1, T=259, C=16, hd=1, M=834, W=128, R=48, dtype="bf16", ids="mixed", gate_width=1, weight_scale=-1.0,
          index=1020),
    # one-column rows again, one reading cancelling to -4e-6 (its float32 noise 2 % of it)
    small(P=2, T=376, C=100, hd=1, M=1668, W=40, R=256, dtype="bf16", gate_width=1, weight_scale=-1.0, index=1011),
]


@pytest.mark.parametrize("wl", SMALL, ids=[f"P{w.P}T{w.T}C{w.C}hd{w.hd}W{w.W}{w.dtype}{w.ids}G{w.G}" for w in SMALL])
def test_forward_small(gpu, wl):
    inp = gu.generate(wl)
    t = gu.to_torch(inp, gpu)
    out, bank = gu.run(t, wl.C)
    gu.parity(out, bank, inp, wl.C, wl.name)
    o = gu.f64(out)
    for p in range(wl.P):
        pad = o[p, int(inp["valid"][p]):]
        assert np.all(pad == 0) and not np.signbit(pad).any()


def test_forward_g_positive(gpu):
    """Positive log-decays (rows grow between writes) take the same path."""
    wl = small(P=2, T=60, C=16, hd=8, M=10, W=2, R=2, decay_scale=-0.05, index=21)
    inp = gu.generate(wl)
    assert (inp["log_decay"] > 0).all()
    out, bank = gu.run(gu.to_torch(inp, gpu), wl.C)
    gu.parity(out, bank, inp, wl.C, "g>0")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_degenerate_values(gpu, dtype):
    """Inputs at the method's degenerate values, mixed in one call: beta = 0 (a token that
    only decays its rows), beta = 1 with one unit write weight (the row replaced by v),
    zero write or read weights, zero log-decays (no decay), v = 0, and a bank of zeros in
    one stream. The oracle decides every case."""
    wl = small(P=3, T=90, C=32, hd=16, M=24, W=4, R=3, dtype=dtype, index=46)
    inp = gu.generate(wl)
    one = 0x3F80 if dtype == "bf16" else 1.0    # bfloat16 arrays hold bit patterns
    beta = inp["beta"]
    beta[:, 0::7] = 0.0
    beta[:, 3::11] = 1.0
    kv = inp["k_val"]
    kv[:, 3::11, :] = 0
    kv[:, 3::11, 0] = one
    kv[:, 5::9, 1] = 0
    qv = inp["q_val"]
    qv[:, 2::5, :] = 0
    qv[:, 4::13, 1] = 0
    g = inp["log_decay"]
    g[:, 10:40] = 0.0
    g[1] = 0.0
    v = inp["v"]
    v[:, 6::8] = 0
    inp["bank"][2] = 0
    out, bank = gu.run(gu.to_torch(inp, gpu), wl.C)
    gu.parity(out, bank, inp, wl.C, f"degenerate {dtype}")


def test_all_padding_and_zero_valid(gpu):
    wl = small(P=3, T=40, C=16, hd=8, M=16, W=2, R=2, index=22)
    inp = gu.generate(wl)
    inp["valid"] = np.array([0, 40, 17], np.int32)
    t = gu.to_torch(inp, gpu)
    out, bank = gu.run(t, wl.C)
    gu.parity(out, bank, inp, wl.C, "valid 0/40/17")
    assert torch.equal(bank[0], t["bank"][0])          # stream 0 untouched
    assert (gu.f64(out[0]) == 0).all()


@pytest.mark.parametrize("C", [16, 32, 64, 128, 256])
def test_result_does_not_depend_on_chunk_size(gpu, C):
    wl = small(P=2, T=300, C=C, hd=16, M=50, W=4, R=4, ragged=True, index=23)
    inp = gu.generate(wl)
    out, bank = gu.run(gu.to_torch(inp, gpu), C)
    gu.parity(out, bank, inp, C, f"C={C}")


# ------------------------------------------------------------------ determinism and independence

def test_bitwise_reruns_workspace_and_stream_independence(gpu):
    wl = small(P=8, T=256, C=64, hd=64, M=200, W=8, R=8, dtype="bf16", ids="zipf", ragged=True, index=24)
    inp = gu.generate(wl)
    t = gu.to_torch(inp, gpu)
    o1, b1 = gu.run(t, wl.C)
    o2, b2 = gu.run(t, wl.C)
    assert np.array_equal(gu.bits(o1), gu.bits(o2)) and np.array_equal(gu.bits(b1), gu.bits(b2))
    # smallest workspace (one step per slab) gives the same bits
    from chunked_sparse_delta_amd import workspace_bytes
    one = workspace_bytes(wl.P, wl.T, wl.C, wl.W, wl.R, wl.hd, 1)
    o3, b3 = gu.run(t, wl.C, max_workspace_bytes=one)
    assert np.array_equal(gu.bits(o1), gu.bits(o3)) and np.array_equal(gu.bits(b1), gu.bits(b3))
    # stream 5 alone gives the same bits as inside the batch
    t5 = {k: v[5:6].contiguous() for k, v in t.items()}
    o5, b5 = gu.run(t5, wl.C)
    assert np.array_equal(gu.bits(o5[0]), gu.bits(o1[5])) and np.array_equal(gu.bits(b5[0]), gu.bits(b1[5]))


@pytest.mark.parametrize("wl,part", [
    (small(P=2, T=90, C=32, hd=32, M=40, W=4, R=4, ragged=True, index=25), "1"),                  # fused
    (small(P=1, T=300, C=128, hd=16, M=300, W=16, R=8, ids="zipf", ragged=True, weight_scale=-1.0,
           index=14), "1"),                                                                          # partitions
    (small(P=1, T=300, C=128, hd=16, M=300, W=16, R=8, ids="zipf", ragged=True, weight_scale=-1.0,
           index=14), "0"),                                                                          # sorting
    (small(P=3, T=150, C=64, hd=64, M=200, W=24, R=24, dtype="bf16", ids="zipf", ragged=True, index=53), "1"),
], ids=["fused", "partitioned", "sorting", "bf16_partitioned"])
def test_poisoned_output_and_workspace(gpu, wl, part, monkeypatch):
    """A workspace of 0xFF bytes (NaN words, -1 ints) and a NaN-filled output give the bits
    of a zeroed workspace, on every Phase-1 path: nothing reads workspace memory the call did
    not write first (padding tokens included)."""
    monkeypatch.setenv("SDM_P1_PART", part)
    inp = gu.generate(wl)
    t = gu.to_torch(inp, gpu)
    from chunked_sparse_delta_amd import workspace_bytes
    n = workspace_bytes(wl.P, wl.T, wl.C, wl.W, wl.R, wl.hd, 0)
    o1, b1 = gu.run(t, wl.C, workspace=torch.zeros((n,), dtype=torch.uint8, device=gpu))
    gu.parity(o1, b1, inp, wl.C, f"poison baseline {part}")
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device=gpu)
    out = torch.full((wl.P, wl.T, wl.hd), float("nan"), dtype=t["bank"].dtype, device=gpu)
    o2, b2 = gu.run(t, wl.C, out=out, workspace=ws)
    assert np.array_equal(gu.bits(o1), gu.bits(o2)) and np.array_equal(gu.bits(b1), gu.bits(b2))


# ------------------------------------------------------------------ the five workloads at full size

@pytest.mark.parametrize("name", ["0", "1", "2", "3"])
def test_workload_full_size(gpu, name):
    wl = workloads.CONFIGS[name]
    inp = gu.generate(wl)
    t = gu.to_torch(inp, gpu)
    out, bank = gu.run(t, wl.C)
    gu.parity(out, bank, inp, wl.C, f"config {name}", threads=16)
    o2, b2 = gu.run(t, wl.C)
    assert np.array_equal(gu.bits(out), gu.bits(o2)) and np.array_equal(gu.bits(bank), gu.bits(b2))


def test_workload_4p_sampled_streams(gpu):
    """Config 4's shapes (timed literally) at full size; the oracle checks eight sampled
    streams of the finite twin 4p (weights / sqrt(256)) computed in the full launch, one on
    each XCD (stream p runs on XCD p mod 8)."""
    wl = workloads.CONFIGS["4p"]
    inp = gu.generate(wl)
    t = gu.to_torch(inp, gpu)
    del inp
    out, bank = gu.run(t, wl.C)
    sample = [0, 9, 18, 27, 36, 45, 54, 63]
    sub = gu.generate(wl, streams=sample)
    gu.parity(out[sample], bank[sample], sub, wl.C, f"config 4p streams {sample}", threads=8)
    o2, b2 = gu.run(t, wl.C)
    assert np.array_equal(gu.bits(out), gu.bits(o2)) and np.array_equal(gu.bits(bank), gu.bits(b2))


def test_workload_4_literal_properties(gpu):
    """Config 4 as drawn (the timed workload: weights U(0,1) over 256 slots, so the bank
    overflows to inf and NaN within a few chunks and no oracle value is meaningful), at full
    size in the launch bench.py times, checked by properties that hold at any size: a rerun
    gives the same bits, rows that no token writes keep their input bits, and a stream run
    alone (one stream per launch: another plan, other slices) gives the bits it gets inside
    the batch of 64 (NaN for NaN: which NaN an operation on two NaNs returns depends on the
    instruction the compiler picked, and the slicing of another plan picks other ones)."""
    wl = workloads.CONFIGS["4"]
    inp = gu.generate(wl)
    t = gu.to_torch(inp, gpu)
    out, bank = gu.run(t, wl.C)
    gu.check_untouched_rows(bank, inp, "config 4")
    del inp
    o2, b2 = gu.run(t, wl.C)
    assert np.array_equal(gu.bits(out), gu.bits(o2)) and np.array_equal(gu.bits(bank), gu.bits(b2))
    del o2, b2
    for p in (0, 63):
        one = gu.to_torch(gu.generate(wl, streams=[p]), gpu)
        o1, b1 = gu.run(one, wl.C)
        for name, x, y in (("readings", o1[0], out[p]), ("bank", b1[0], bank[p])):
            bx, by = gu.bits(x), gu.bits(y)
            nan = torch.isnan(x).cpu().numpy() & torch.isnan(y).cpu().numpy()
            bad = (bx != by) & ~nan
            print(f"stream {p} {name}: {int(nan.sum())} NaN in both, {int(bad.sum())} other elements differ",
                  flush=True)
            assert not bad.any(), (name, p, np.argwhere(bad)[:4])


@pytest.mark.parametrize("wl", [
    small(P=8, T=300, C=64, hd=64, M=200, W=8, R=8, dtype="bf16", ids="zipf", ragged=True, index=26),
    small(P=3, T=260, C=128, hd=32, M=300, W=16, R=16, ragged=True, index=27),
    small(P=2, T=100, C=48, hd=40, M=80, W=5, R=3, ids="zipf", index=28),
    # 16 writes per token over 160 Zipf rows: write groups of every size, from one member to the
    # whole chunk (the DW's member windows, its four-at-a-time loop and its whole-wavefront
    # groups in every slice width)
    small(P=8, T=256, C=64, hd=64, M=160, W=16, R=16, dtype="bf16", ids="zipf", ragged=True, index=31),
], ids=["bf16_P8", "f32_P3", "f32_partial_slice", "bf16_groups_of_every_size"])
def test_phase2_geometry_does_not_change_bits(gpu, wl, monkeypatch):
    """The column slicing, the LDS staging and the LDS-resident bank slice change only the schedule:
    every geometry gives the same bits (the gather, matmul and DW sums run in orders fixed by W, R
    and C, and a resident bank row is held in the bank dtype, rounded where memory would round it)."""
    inp = gu.generate(wl)
    t = gu.to_torch(inp, gpu)
    results = []
    for geom in (None, "1", "2", "4", "8", "1,1", "2,1", "4,1", "8,1", "1,0", "2,0", "4,0", "8,0"):
        if geom is None:
            monkeypatch.delenv("SDM_P2_GEOM", raising=False)
        else:
            monkeypatch.setenv("SDM_P2_GEOM", geom)
        o, b = gu.run(t, wl.C)
        results.append((geom, gu.bits(o), gu.bits(b)))
    gu.parity(o, b, inp, wl.C, "geometry")
    for geom, ob, bb in results[1:]:
        assert np.array_equal(ob, results[0][1]) and np.array_equal(bb, results[0][2]), geom


def test_plan_reports_phase2_modes(gpu, monkeypatch):
    """The plan query follows the mode cap of the tuning override, and the headline shape
    (C=64, hd=64 bf16, 4096 rows, W=R=8) keeps its bank slice resident in LDS, in slices of
    one 8-byte vector (4 columns: 16 slices per stream) since 8-column slices would leave
    more than half of the CUs idle; a shape with enough streams keeps 16-byte vectors."""
    from chunked_sparse_delta_amd import plan
    monkeypatch.delenv("SDM_P2_GEOM", raising=False)
    p = plan(8, 2048, 64, 8, 8, 64, 4096, torch.bfloat16)
    assert p["phase2_mode"] == "resident" and p["phase2_lds_bytes"] <= p["lds_limit"], p
    assert p["vec"] == 4 and p["slice_vectors"] == 1 and p["slices"] == 16, p
    wide = plan(64, 256, 64, 8, 8, 64, 4096, torch.bfloat16)
    assert wide["vec"] == 8, wide
    for cap, mode in (("1,1", "staged"), ("1,0", "memory")):
        monkeypatch.setenv("SDM_P2_GEOM", cap)
        q = plan(8, 2048, 64, 8, 8, 64, 4096, torch.bfloat16)
        assert q["phase2_mode"] == mode and q["slice_vectors"] == 1 and q["vec"] == 8, q


@pytest.mark.parametrize("wl", [
    small(P=8, T=300, C=64, hd=64, M=200, W=8, R=8, dtype="bf16", ids="zipf", ragged=True, index=29),
    small(P=3, T=260, C=48, hd=32, M=60, W=16, R=16, ids="zipf", zipf_s=1.3, ragged=True, index=30),
], ids=["bf16_P8", "f32_hot"])
def test_phase1_fusion_does_not_change_bits(gpu, wl, monkeypatch):
    """Phase 1 and the solve fused into one workgroup per chunk give the same bits as the
    separate sorting kernels (the per-chunk arithmetic is the same; only the launch differs)."""
    inp = gu.generate(wl)
    t = gu.to_torch(inp, gpu)
    monkeypatch.setenv("SDM_P1_PART", "0")
    results = []
    for fused in ("0", "1"):
        monkeypatch.setenv("SDM_P1_FUSED", fused)
        o, b = gu.run(t, wl.C)
        results.append((gu.bits(o), gu.bits(b)))
    gu.parity(o, b, inp, wl.C, "fused phase 1")
    assert np.array_equal(results[0][0], results[1][0]) and np.array_equal(results[0][1], results[1][1])


PART = [
    small(P=3, T=300, C=128, hd=32, M=2000, W=24, R=24, ids="zipf", ragged=True, index=46),
    small(P=2, T=600, C=256, hd=16, M=4000, W=64, R=48, dtype="bf16", ids="mixed", weight_scale=-1.0, index=47),
    small(P=4, T=200, C=64, hd=24, M=50, W=48, R=40, ragged=True, weight_scale=-1.0, index=48),  # long groups
    small(P=2, T=130, C=64, hd=8, M=300, W=32, R=32, gate_width=1, index=49),
]


@pytest.mark.parametrize("wl", PART, ids=["zipf_C128", "mixed_C256_bf16", "fewslots", "gate1"])
def test_phase1_paths_match_the_oracle(gpu, wl, monkeypatch):
    """Chunks of more than 1024 entries run Phase 1 in slot partitions held in LDS, one
    partition after another; any partition count (1 to 64) and the sorting path (also the
    fallback for a partition larger than the LDS holds: one partition for every slot of a big
    chunk forces it) give results within the oracle's bar, each bitwise reproducible."""
    inp = gu.generate(wl)
    t = gu.to_torch(inp, gpu)
    for part, nplog in (("1", None), ("1", "0"), ("1", "3"), ("1", "6"), ("0", None)):
        monkeypatch.setenv("SDM_P1_PART", part)
        if nplog is None:
            monkeypatch.delenv("SDM_P1_NP_LOG", raising=False)
        else:
            monkeypatch.setenv("SDM_P1_NP_LOG", nplog)
        o, b = gu.run(t, wl.C)
        gu.parity(o, b, inp, wl.C, f"phase 1 part={part} np_log={nplog}")
        o2, b2 = gu.run(t, wl.C)
        assert np.array_equal(gu.bits(o), gu.bits(o2)) and np.array_equal(gu.bits(b), gu.bits(b2)), (part, nplog)


def test_phase1_partition_overflow_takes_the_sorting_path(gpu, monkeypatch):
    """A chunk with a partition of more entries than the LDS holds (3072) is left to the
    sorting kernels by the partitioned kernel: the result is then bit for bit the sorting
    path's (one partition forced on chunks of 256 x (16 + 16) = 8192 entries)."""
    wl = small(P=2, T=512, C=256, hd=16, M=3000, W=16, R=16, ids="zipf", index=50)
    inp = gu.generate(wl)
    t = gu.to_torch(inp, gpu)
    monkeypatch.setenv("SDM_P1_PART", "0")
    o0, b0 = gu.run(t, wl.C)
    monkeypatch.setenv("SDM_P1_PART", "1")
    monkeypatch.setenv("SDM_P1_NP_LOG", "0")
    o1, b1 = gu.run(t, wl.C)
    gu.parity(o1, b1, inp, wl.C, "overflow")
    assert np.array_equal(gu.bits(o0), gu.bits(o1)) and np.array_equal(gu.bits(b0), gu.bits(b1))


# ------------------------------------------------------------------ forward variants

@pytest.mark.parametrize("wl", [
    small(P=3, T=150, C=32, hd=24, M=40, W=5, R=4, dtype="bf16", ids="zipf", ragged=True, index=33),
    small(P=2, T=130, C=64, hd=16, M=300, W=32, R=32, index=34),
], ids=["bf16_zipf", "f32_w32"])
def test_int64_ids_give_the_same_bits(gpu, wl):
    """Slot ids may be int32 or int64 (page 21, memory_ops.py, _layout): the values are the
    same rows, so every combination gives the same bits."""
    inp = gu.generate(wl)
    t = gu.to_torch(inp, gpu)
    o, b = gu.run(t, wl.C)
    gu.parity(o, b, inp, wl.C, "int32 ids")
    for kd, qd in ((torch.int64, torch.int64), (torch.int64, torch.int32), (torch.int32, torch.int64)):
        t2 = dict(t, k_idx=t["k_idx"].to(kd), q_idx=t["q_idx"].to(qd))
        o2, b2 = gu.run(t2, wl.C)
        assert np.array_equal(gu.bits(o2), gu.bits(o)) and np.array_equal(gu.bits(b2), gu.bits(b)), (kd, qd)


@pytest.mark.parametrize("wl", [
    small(P=4, T=200, C=64, hd=64, M=64, W=8, R=8, dtype="bf16", ids="zipf", ragged=True, index=35),
    small(P=3, T=100, C=32, hd=20, M=50, W=4, R=3, ragged=True, index=36),
    small(P=2, T=300, C=128, hd=32, M=700, W=16, R=16, index=37),
], ids=["bf16_staged", "f32_partial", "f32_memory"])
def test_shared_bank_matches_per_stream_banks(gpu, wl, monkeypatch):
    """One bank shared by every stream (sdm_write_read with shared_bank=True, page 21,
    memory_ops.py docstring), the streams' slots interleaved and disjoint: the readings and
    each stream's rows equal those of per-stream banks bit for bit when Phase 1 sorts every
    chunk (relabeling slot s of stream p as s * P + p keeps each chunk's slot order), and are
    within the oracle's bar on the default path, whose slot partitions (slot mod 2^k) the
    relabeling reshuffles. (A workgroup writing a whole slice back, as the resident mode
    does, would overwrite the other streams' rows.)"""
    inp = gu.generate(wl)
    t = gu.to_torch(inp, gpu)
    sh = gu.to_torch(dict(workloads.shared_bank_inputs(inp), dtype=inp["dtype"]), gpu)
    assert sh["bank"].shape == (wl.P * wl.M, wl.hd)
    P, M, hd = wl.P, wl.M, wl.hd
    o2, b2 = gu.run(sh, wl.C, shared_bank=True)
    gu.parity(o2, b2.reshape(M, P, hd).permute(1, 0, 2).contiguous(), inp, wl.C, "shared bank")
    monkeypatch.setenv("SDM_P1_PART", "0")
    o, b = gu.run(t, wl.C)
    gu.parity(o, b, inp, wl.C, "per-stream banks")
    o2, b2 = gu.run(sh, wl.C, shared_bank=True)
    assert np.array_equal(gu.bits(o2), gu.bits(o))
    assert np.array_equal(gu.bits(b2.reshape(M, P, hd).permute(1, 0, 2).contiguous()), gu.bits(b))


def test_shared_bank_needs_the_opt_in(gpu):
    from chunked_sparse_delta_amd import sdm_fwd
    wl = small(P=2, T=40, C=16, hd=8, M=20, W=2, R=2, index=38)
    sh = gu.to_torch(dict(workloads.shared_bank_inputs(gu.generate(wl)), dtype="f32"), gpu)
    with pytest.raises(ValueError, match="shared_bank=True"):
        sdm_fwd(sh["bank"], sh["k_idx"], sh["k_val"], sh["v"], sh["beta"], sh["log_decay"], sh["q_idx"],
                sh["q_val"], chunk=16)


@pytest.mark.parametrize("fused", ["1", "0"])
def test_repeated_write_counter(gpu, fused, monkeypatch):
    """The device counter of write entries repeating a slot of their own token (page 21,
    memory_ops.py, repeated_write_slots) equals the oracle's count, and accumulates over
    calls. Such calls break the distinct-slots contract, so only the count is checked."""
    import oracle
    monkeypatch.setenv("SDM_P1_FUSED", fused)
    wl = small(P=3, T=70, C=32, hd=8, M=30, W=4, R=2, ragged=True, index=39)
    inp = gu.generate(wl)
    k = inp["k_idx"].copy()
    k[0, 3, 1] = k[0, 3, 0]               # one repeat
    k[1, 10, 1:] = k[1, 10, 0]            # three repeats in one token
    k[2, 40, 2] = k[2, 40, 3]             # one repeat (counted only if token 40 is live)
    k[0, 69, 3] = k[0, 69, 0]             # last token of stream 0 (counted only if live)
    inp["k_idx"] = k
    want = oracle.repeated_write_slots(k, inp["valid"])
    assert want >= 4
    t = gu.to_torch(inp, gpu)
    cnt = torch.zeros(1, dtype=torch.int64, device=gpu)
    gu.run(t, wl.C, repeated_writes=cnt)
    assert int(cnt.item()) == want
    gu.run(t, wl.C, repeated_writes=cnt)
    assert int(cnt.item()) == 2 * want
    gen = gu.generate(wl)                 # distinct slots: nothing counted
    cnt.zero_()
    gu.run(gu.to_torch(gen, gpu), wl.C, repeated_writes=cnt)
    assert int(cnt.item()) == 0


@pytest.mark.parametrize("wl", [
    small(P=3, T=150, C=32, hd=24, M=40, W=5, R=4, dtype="bf16", ids="zipf", ragged=True, index=43),
    small(P=2, T=130, C=64, hd=16, M=300, W=32, R=32, index=44),
], ids=["bf16zipf", "w32"])
def test_split_forward_gives_the_same_bits(gpu, wl):
    """sdm_fwd_phase1 then sdm_fwd_phase2 (here on two streams ordered by an event, with
    another call's Phase 2 between them on the second stream) equals sdm_fwd bit for bit;
    a split call needs the workspace of every step."""
    from chunked_sparse_delta_amd import SdmError, sdm_fwd_phase1, sdm_fwd_phase2, workspace_bytes
    t = gu.to_torch(gu.generate(wl), gpu)
    o_ref, b_ref = gu.run(t, wl.C)
    ws = torch.empty(workspace_bytes(wl.P, wl.T, wl.C, wl.W, wl.R, wl.hd, 0), dtype=torch.uint8, device=gpu)
    bank = t["bank"].clone()
    out = torch.empty_like(o_ref)
    args = (t["k_idx"], t["k_val"], t["v"], t["beta"], t["log_decay"], t["q_idx"], t["q_val"])
    s1 = torch.cuda.Stream()
    ev = torch.cuda.Event()
    with torch.cuda.stream(s1):
        sdm_fwd_phase1(bank, *args, workspace=ws, chunk=wl.C, valid_tokens=t["valid"], stream=s1)
        ev.record(s1)
    torch.cuda.current_stream().wait_event(ev)
    sdm_fwd_phase2(bank, *args, workspace=ws, out=out, chunk=wl.C, valid_tokens=t["valid"])
    torch.cuda.synchronize()
    assert np.array_equal(gu.bits(out), gu.bits(o_ref)) and np.array_equal(gu.bits(bank), gu.bits(b_ref))
    small_ws = torch.empty(workspace_bytes(wl.P, wl.T, wl.C, wl.W, wl.R, wl.hd, 1), dtype=torch.uint8, device=gpu)
    with pytest.raises(SdmError, match="all"):
        sdm_fwd_phase1(bank, *args, workspace=small_ws, chunk=wl.C, valid_tokens=t["valid"])


@pytest.mark.gpu
def test_overlapped_batches_give_the_same_bits(gpu):
    """Batches run back to back with batch k+1's Phase 1 on a second stream (and workspace)
    overlapping batch k's Phase 2 give, batch by batch, sdm_fwd's readings and bank bits."""
    from chunked_sparse_delta_amd import sdm_fwd_phase1, sdm_fwd_phase2, workspace_bytes
    base = small(P=3, T=150, C=32, hd=24, M=40, W=5, R=4, dtype="bf16", ids="zipf", ragged=True, index=45)
    batches = [gu.to_torch(gu.generate(base.replace(index=45 + k)), gpu) for k in range(3)]
    keys = ("k_idx", "k_val", "v", "beta", "log_decay", "q_idx", "q_val")
    bank_ref = batches[0]["bank"].clone()
    refs = []
    for t in batches:
        o, _ = gu.run(t, base.C, bank=bank_ref)
        refs.append((gu.bits(o), gu.bits(bank_ref)))
    nb = workspace_bytes(base.P, base.T, base.C, base.W, base.R, base.hd, 0)
    ws = [torch.empty(nb, dtype=torch.uint8, device=gpu) for _ in range(2)]
    bank = batches[0]["bank"].clone()
    outs = [torch.empty((base.P, base.T, base.hd), dtype=bank.dtype, device=gpu) for _ in batches]
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    p1_done = [torch.cuda.Event() for _ in batches]
    p2_done = [torch.cuda.Event() for _ in batches]
    side.wait_stream(main)
    # Phase 1 of batch 0, then for each k: Phase 2 of k on main, Phase 1 of k+1 on side
    with torch.cuda.stream(side):
        sdm_fwd_phase1(bank, *(batches[0][x] for x in keys), workspace=ws[0], chunk=base.C,
                       valid_tokens=batches[0]["valid"], stream=side)
        p1_done[0].record(side)
    for k, t in enumerate(batches):
        main.wait_event(p1_done[k])
        sdm_fwd_phase2(bank, *(t[x] for x in keys), workspace=ws[k % 2], out=outs[k], chunk=base.C,
                       valid_tokens=t["valid"], stream=main)
        p2_done[k].record(main)
        if k + 1 < len(batches):
            nxt = batches[k + 1]
            with torch.cuda.stream(side):
                if k >= 1:
                    side.wait_event(p2_done[k - 1])
                sdm_fwd_phase1(bank, *(nxt[x] for x in keys), workspace=ws[(k + 1) % 2], chunk=base.C,
                               valid_tokens=nxt["valid"], stream=side)
                p1_done[k + 1].record(side)
    torch.cuda.synchronize()
    for k, (o_bits, b_bits) in enumerate(refs):
        assert np.array_equal(gu.bits(outs[k]), o_bits), f"readings of batch {k}"
    assert np.array_equal(gu.bits(bank), refs[-1][1])


@pytest.mark.gpu
@pytest.mark.parametrize("wl", [
    small(P=8, T=200, C=64, hd=128, M=300, W=8, R=8, dtype="bf16", ids="zipf", ragged=True, index=47),
    # bank slices too large for LDS: staged blocks (bf16, config 2's widths) and memory mode (f32)
    small(P=8, T=200, C=64, hd=128, M=16384, W=32, R=32, dtype="bf16", ids="zipf", index=51),
    small(P=4, T=300, C=128, hd=128, M=4000, W=24, R=24, ragged=True, index=52),
], ids=["resident", "staged", "memory"])
def test_phase2_cu_budget_does_not_change_bits(gpu, wl):
    """sdm_fwd_phase2's phase2_cus (the CUs its slice geometry plans for) changes only the
    schedule: every budget gives sdm_fwd's bits (resident, staged and memory geometries); a
    negative budget is rejected."""
    from chunked_sparse_delta_amd import SdmError, sdm_fwd_phase1, sdm_fwd_phase2, workspace_bytes
    t = gu.to_torch(gu.generate(wl), gpu)
    o_ref, b_ref = gu.run(t, wl.C)
    args = (t["k_idx"], t["k_val"], t["v"], t["beta"], t["log_decay"], t["q_idx"], t["q_val"])
    ws = torch.empty(workspace_bytes(wl.P, wl.T, wl.C, wl.W, wl.R, wl.hd, 0), dtype=torch.uint8, device=gpu)
    for cus in (1, 16, 64, 128, 100000):
        bank = t["bank"].clone()
        out = torch.empty_like(o_ref)
        sdm_fwd_phase1(bank, *args, workspace=ws, chunk=wl.C, valid_tokens=t["valid"])
        sdm_fwd_phase2(bank, *args, workspace=ws, out=out, chunk=wl.C, valid_tokens=t["valid"], phase2_cus=cus)
        torch.cuda.synchronize()
        assert np.array_equal(gu.bits(out), gu.bits(o_ref)) and np.array_equal(gu.bits(bank), gu.bits(b_ref)), cus
    with pytest.raises(SdmError, match="phase2_cus"):
        sdm_fwd_phase2(t["bank"].clone(), *args, workspace=ws, out=torch.empty_like(o_ref), chunk=wl.C,
                       valid_tokens=t["valid"], phase2_cus=-1)


@pytest.mark.parametrize("wl", [
    small(P=2, T=256, C=128, hd=8, M=40, W=24, R=24, ids="zipf", ragged=True, index=80),
    small(P=2, T=130, C=64, hd=8, M=12, W=6, R=5, index=81),
    # nine tiles per wavefront (three interleaved groups), hot columns over several blocks
    small(P=1, T=512, C=256, hd=8, M=400, W=32, R=32, ids="zipf", index=82),
    # a ragged tile count (C = 200: 91 tiles, five or six per wavefront)
    small(P=2, T=300, C=200, hd=8, M=300, W=16, R=16, ids="mixed", ragged=True, index=83),
], ids=["C128_zipf", "C64_allhot", "C256_zipf", "C200_mixed"])
def test_hot_gram_kernels_give_the_same_bits(gpu, wl, monkeypatch):
    """The hot Gram staged in LDS (one workgroup per chunk and matrix) and the per-tile kernel
    (operands from memory) run the same MFMA chains: identical A and QK."""
    from chunked_sparse_delta_amd import chunk_mats
    monkeypatch.setenv("SDM_P1_FUSED", "0")
    t = gu.to_torch(gu.generate(wl), gpu)
    res = {}
    for mode in ("1", "0"):
        monkeypatch.setenv("SDM_P1_HOT_LDS", mode)
        r = chunk_mats(t["k_idx"], t["k_val"], t["beta"], t["log_decay"], t["q_idx"], t["q_val"], rows=wl.M,
                       head_dim=wl.hd, chunk=wl.C, valid_tokens=t["valid"])
        res[mode] = {k: gu.bits(v) for k, v in r.items()}
    for k in res["1"]:
        assert np.array_equal(res["1"][k], res["0"][k]), k


@pytest.mark.parametrize("wl", [
    small(P=8, T=300, C=128, hd=64, M=3000, W=32, R=32, ids="mixed", weight_scale=-1.0, ragged=True, index=90),
    small(P=8, T=256, C=64, hd=128, M=5000, W=64, R=32, dtype="bf16", ids="zipf", weight_scale=-1.0, index=91),
], ids=["f32_mixed", "bf16_zipf"])
def test_non_temporal_gather_gives_the_same_bits(gpu, wl, monkeypatch):
    """Rows that one entry of a chunk alone reads (marked by the partitioned Phase 1) load with
    the non-temporal hint on large workloads: the same bits with it on and off, in memory mode
    with one workgroup per slice and with teams, and the oracle agrees."""
    from chunked_sparse_delta_amd import plan
    inp = gu.generate(wl)
    t = gu.to_torch(inp, gpu)
    for k in ("SDM_P2_TEAM", "SDM_P2_NT"):
        monkeypatch.delenv(k, raising=False)
    monkeypatch.setenv("SDM_P2_GEOM", "8,0")
    assert plan(wl.P, wl.T, wl.C, wl.W, wl.R, wl.hd, wl.M, t["bank"].dtype)["phase2_mode"] == "memory"
    runs = {}
    for team in ("0", "4"):
        monkeypatch.setenv("SDM_P2_TEAM", team)
        for nt in ("0", "1"):
            monkeypatch.setenv("SDM_P2_NT", nt)
            runs[(team, nt)] = gu.run(t, wl.C)
    o_ref, b_ref = runs[("0", "0")]
    for key, (o, b) in runs.items():
        assert np.array_equal(gu.bits(o), gu.bits(o_ref)) and np.array_equal(gu.bits(b), gu.bits(b_ref)), key
    gu.parity(*runs[("0", "1")], inp, wl.C, "non-temporal gather")
