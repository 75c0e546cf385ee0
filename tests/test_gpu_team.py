"""Phase-2 teams on the GPU: several workgroups sharing one (stream, column slice) give the
bits of one workgroup per (stream, slice), whatever the team size and whichever workgroup
runs which piece (every unclaimed piece claimed at once, with SDM_P2_TEAM_STEAL=0)."""

import numpy as np
import pytest
import torch

import workloads
from workloads import small
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

CASES = [
    # float32, ids and weights one at a time (W, R not multiples of 32), ragged streams
    small(P=8, T=300, C=64, hd=64, M=512, W=8, R=8, ragged=True, index=60),
    # float32, a partial last slice (head_dim 40: slices of 8 and 2 vectors), Zipf repeats
    small(P=8, T=200, C=64, hd=40, M=300, W=32, R=32, ids="zipf", ragged=True, index=61),
    # bfloat16, 16 streams, groups with many members
    small(P=16, T=200, C=64, hd=128, M=2000, W=32, R=32, dtype="bf16", ids="mixed", ragged=True, index=62),
    # the largest chunk: pieces of 64 tokens (team of 4) or 128 (team of 2)
    small(P=8, T=600, C=256, hd=32, M=5000, W=16, R=8, ids="zipf", ragged=True, index=63),
]
IDS = ["f32_narrow", "f32_partial_slice", "bf16_P16", "f32_C256"]


def _diff(got, ref) -> str:
    """'' when the bit patterns agree, else a short account of where they do not."""
    g, r = gu.bits(got), gu.bits(ref)
    if np.array_equal(g, r):
        return ""
    bad = np.argwhere(g != r)
    d = np.abs(gu.f64(got) - gu.f64(ref))
    return f"{len(bad)} of {g.size} differ, first at {tuple(bad[0])}, largest |diff| {d.max():.3e}"


def _run_env(monkeypatch, t, C, **env):
    for k in ("SDM_P2_TEAM", "SDM_P2_TEAM_STEAL", "SDM_P2_GEOM"):
        monkeypatch.delenv(k, raising=False)
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    return gu.run(t, C)


@pytest.mark.parametrize("wl", CASES, ids=IDS)
def test_teams_give_the_bits_of_one_workgroup(gpu, wl, monkeypatch):
    from chunked_sparse_delta_amd import plan
    inp = gu.generate(wl)
    t = gu.to_torch(inp, gpu)
    o_ref, b_ref = _run_env(monkeypatch, t, wl.C, SDM_P2_TEAM="0")
    dt = t["bank"].dtype
    bad = []
    for env in ({"SDM_P2_TEAM": "2"}, {"SDM_P2_TEAM": "4"},
                {"SDM_P2_TEAM": "4", "SDM_P2_TEAM_STEAL": "0"}, {"SDM_P2_TEAM": "2", "SDM_P2_TEAM_STEAL": "0"}):
        o, b = _run_env(monkeypatch, t, wl.C, **env)
        p = plan(wl.P, wl.T, wl.C, wl.W, wl.R, wl.hd, wl.M, dt)
        assert p["phase2_team"] == int(env["SDM_P2_TEAM"]) and p["phase2_mode"] == "memory", (env, p)
        assert p["slice_vectors"] == 8 and p["slices"] == (wl.hd // p["vec"] + 7) // 8, (env, p)
        do, db = _diff(o, o_ref), _diff(b, b_ref)
        print(f"{env}: readings {do or 'same bits'}; bank {db or 'same bits'}", flush=True)
        if do or db:
            bad.append(env)
    assert not bad, bad
    gu.parity(o, b, inp, wl.C, "team of 2, pieces claimed at once")


def test_team_sizes_the_kernel_cannot_take_are_not_planned(gpu, monkeypatch):
    """Streams not in whole groups of 8, or pieces that are not whole 16-token tiles, fall
    back to one workgroup per slice (same bits)."""
    from chunked_sparse_delta_amd import plan
    monkeypatch.setenv("SDM_P2_TEAM", "4")
    assert plan(4, 256, 64, 8, 8, 64, 512, torch.float32)["phase2_team"] == 1       # P % 8 != 0
    assert plan(8, 256, 32, 8, 8, 64, 512, torch.float32)["phase2_team"] == 1       # 32 / 4 = 8 tokens
    assert plan(8, 256, 32, 8, 8, 64, 512, torch.float32)["slice_vectors"] >= 1
    monkeypatch.setenv("SDM_P2_TEAM", "2")
    assert plan(8, 256, 32, 8, 8, 64, 512, torch.float32)["phase2_team"] == 2
    assert plan(8, 256, 48, 8, 8, 64, 512, torch.float32)["phase2_team"] == 1       # 24-token pieces


def test_full_size_config_3_teams(gpu, monkeypatch):
    """Config 3 (16 float32 streams, 128-column rows: 4 slices of one 128-byte line) is
    planned with teams of 4 on a 256-CU device; its bits equal those of 32-byte slices
    (one workgroup each), and the oracle agrees (the full-size parity test checks the
    default plan against O1 too)."""
    from chunked_sparse_delta_amd import plan
    wl = workloads.CONFIGS["3"]
    monkeypatch.delenv("SDM_P2_TEAM", raising=False)
    monkeypatch.delenv("SDM_P2_GEOM", raising=False)
    p = plan(wl.P, wl.T, wl.C, wl.W, wl.R, wl.hd, wl.M, torch.float32)
    if torch.cuda.get_device_properties(0).multi_processor_count >= 256:
        assert p["phase2_team"] == 4 and p["slices"] == 4 and p["slice_vectors"] == 8, p
    inp = gu.generate(wl)
    t = gu.to_torch(inp, gpu)
    o_def, b_def = _run_env(monkeypatch, t, wl.C)
    o_one, b_one = _run_env(monkeypatch, t, wl.C, SDM_P2_TEAM="0")
    assert np.array_equal(gu.bits(o_def), gu.bits(o_one)) and np.array_equal(gu.bits(b_def), gu.bits(b_one))
    o_st, b_st = _run_env(monkeypatch, t, wl.C, SDM_P2_TEAM_STEAL="0")
    assert np.array_equal(gu.bits(o_st), gu.bits(o_one)) and np.array_equal(gu.bits(b_st), gu.bits(b_one))


def test_teams_only_replace_narrow_memory_mode_slices(gpu, monkeypatch):
    """Unasked, teams stand in only for narrow slices that would read the bank from memory:
    config 2's shapes (narrow slices stage the chunk's arrays in LDS) keep one workgroup
    per slice."""
    from chunked_sparse_delta_amd import plan
    monkeypatch.delenv("SDM_P2_TEAM", raising=False)
    monkeypatch.delenv("SDM_P2_GEOM", raising=False)
    wl = workloads.CONFIGS["2"]
    p = plan(wl.P, wl.T, wl.C, wl.W, wl.R, wl.hd, wl.M, torch.bfloat16)
    assert p["phase2_team"] == 1 and p["phase2_mode"] != "memory", p


def test_two_team_launches_at_once_give_their_own_bits(gpu, monkeypatch):
    """Two calls planned with teams of 4 on two streams at once (2 x 256 workgroups for 256
    CUs, so some teams are not all on CUs together; waiting workgroups claim the absent
    members' pieces): each call gives the bits it gives alone."""
    from chunked_sparse_delta_amd import plan, sdm_fwd
    monkeypatch.setenv("SDM_P2_TEAM", "4")
    wls = [small(P=16, T=1024, C=128, hd=128, M=20000, W=64, R=64, ragged=True, index=70 + i) for i in range(2)]
    ts = [gu.to_torch(gu.generate(wl), gpu) for wl in wls]
    assert plan(16, 1024, 128, 64, 64, 128, 20000, torch.float32)["phase2_team"] == 4
    alone = [gu.run(t, wl.C) for t, wl in zip(ts, wls)]
    banks = [t["bank"].clone() for t in ts]
    outs = [None, None]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for i, (t, wl) in enumerate(zip(ts, wls)):
        with torch.cuda.stream(streams[i]):
            outs[i] = sdm_fwd(banks[i], t["k_idx"], t["k_val"], t["v"], t["beta"], t["log_decay"], t["q_idx"],
                              t["q_val"], chunk=wl.C, valid_tokens=t["valid"], stream=streams[i])
    torch.cuda.synchronize()
    for i in range(2):
        assert np.array_equal(gu.bits(outs[i]), gu.bits(alone[i][0])), i
        assert np.array_equal(gu.bits(banks[i]), gu.bits(alone[i][1])), i
