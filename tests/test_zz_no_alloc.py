"""sdm_fwd_noalloc, the entry point for callers that cannot allocate: through the C ABI it
gives sdm_fwd's bits (same arguments, the workspace taken from the library's static
scratch), on two calls in a row the second with a smaller problem (the scratch keeps the
first call's contents, which the second must not depend on), and it refuses shapes whose
single step would not fit the scratch before doing any work."""

import numpy as np
import pytest
import torch

from workloads import small
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _noalloc(t, C, bank, out=None):
    from chunked_sparse_delta_amd import sdm_fwd_noalloc
    o = sdm_fwd_noalloc(bank, t["k_idx"], t["k_val"], t["v"], t["beta"], t["log_decay"], t["q_idx"], t["q_val"],
                        chunk=C, valid_tokens=t["valid"], out=out)
    torch.cuda.synchronize()
    return o, bank


def test_noalloc_matches_sdm_fwd_twice_shrinking(gpu):
    big = small(P=8, T=700, C=64, hd=64, M=4096, W=16, R=16, dtype="bf16", ids="zipf", ragged=True, index=61)
    little = small(P=3, T=90, C=32, hd=24, M=50, W=5, R=4, ragged=True, index=62)
    for wl in (big, little):
        inp = gu.generate(wl)
        t = gu.to_torch(inp, gpu)
        o_ref, b_ref = gu.run(t, wl.C)
        out = torch.full_like(o_ref, float("nan"))
        o, b = _noalloc(t, wl.C, t["bank"].clone(), out=out)
        assert o.data_ptr() == out.data_ptr()
        assert np.array_equal(gu.bits(o), gu.bits(o_ref)) and np.array_equal(gu.bits(b), gu.bits(b_ref)), wl.name
        gu.parity(o, b, inp, wl.C, f"noalloc {wl.name}")


def test_noalloc_slabs_when_the_scratch_holds_fewer_steps(gpu):
    """A problem whose steps do not all fit the scratch runs in slabs; results never depend on
    the slab size, so the bits still equal sdm_fwd's with a workspace for every step."""
    from chunked_sparse_delta_amd import NOALLOC_SCRATCH_BYTES, workspace_bytes
    wl = small(P=32, T=1024, C=64, hd=32, M=2048, W=32, R=32, dtype="bf16", ids="zipf", index=63)
    assert workspace_bytes(wl.P, wl.T, wl.C, wl.W, wl.R, wl.hd, 0) > NOALLOC_SCRATCH_BYTES
    assert workspace_bytes(wl.P, wl.T, wl.C, wl.W, wl.R, wl.hd, 1) <= NOALLOC_SCRATCH_BYTES
    inp = gu.generate(wl)
    t = gu.to_torch(inp, gpu)
    o_ref, b_ref = gu.run(t, wl.C)
    o, b = _noalloc(t, wl.C, t["bank"].clone())
    assert np.array_equal(gu.bits(o), gu.bits(o_ref)) and np.array_equal(gu.bits(b), gu.bits(b_ref))


def test_noalloc_refuses_a_step_larger_than_the_scratch(gpu):
    from chunked_sparse_delta_amd import NOALLOC_SCRATCH_BYTES, SdmError, workspace_bytes
    P, T, C, W, R, hd, M = 8, 256, 256, 256, 256, 8, 64
    assert workspace_bytes(P, T, C, W, R, hd, 1) > NOALLOC_SCRATCH_BYTES
    dev = gpu
    bank = torch.zeros((P, M, hd), dtype=torch.float32, device=dev)
    ids = torch.arange(W, dtype=torch.int32, device=dev).remainder(M).expand(P, T, W).contiguous()
    ones = torch.ones((P, T, W), dtype=torch.float32, device=dev)
    v = torch.ones((P, T, hd), dtype=torch.float32, device=dev)
    out = torch.full((P, T, hd), 7.0, device=dev)
    t = dict(k_idx=ids, k_val=ones, v=v, beta=torch.ones((P, T), device=dev), log_decay=-ones, q_idx=ids,
             q_val=ones, valid=None)
    with pytest.raises(SdmError) as ei:
        _noalloc(t, C, bank, out=out)
    assert ei.value.code == -6 and "static scratch" in str(ei.value)
    assert bool((out == 7.0).all()) and bool((bank == 0).all())
