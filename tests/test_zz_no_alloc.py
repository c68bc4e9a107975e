"""kda_chunk_fwd_noalloc (static device scratch, no workspace) against kda_chunk_fwd
(caller workspace) on the GPU: two calls in a row, the second smaller, each
bit-identical to the workspace entry point's result on the same inputs (same
kernels, same arithmetic), for bf16 and fp32 inputs; and a call beyond the
scratch's limit refused."""
import pytest
import torch

import channel_gated_delta_amd as kda
from channel_gated_delta_amd import workloads
from gpu_helpers import Guarded, note

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def reference(inp, spec):
    """kda_chunk_fwd with a caller workspace, outputs poisoned beforehand."""
    T, H, DK, DV, N = spec.total_tokens, spec.heads, spec.dk, spec.dv, len(spec.lengths)
    o = torch.full((T, H, DV), float("nan"), device=DEV)
    hT = torch.full((N, H, DK, DV), float("nan"), device=DEV)
    kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                  cu_seqlens=inp["cu_seqlens"], scale=spec.read_scale,
                  gate_lower_bound=spec.gate_lb, initial_state=inp["h0"], out=o, final_state=hT)
    return o, hT


def no_alloc(inp, spec):
    T, H, DK, DV, N = spec.total_tokens, spec.heads, spec.dk, spec.dv, len(spec.lengths)
    o = Guarded((T, H, DV), torch.float32, DEV, "o")
    hT = Guarded((N, H, DK, DV), torch.float32, DEV, "final state")
    kda.chunk_fwd_noalloc(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], o.t, hT.t,
                          cu_seqlens=inp["cu_seqlens"], scale=spec.read_scale,
                          gate_lower_bound=spec.gate_lb, initial_state=inp["h0"])
    return o, hT


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_no_alloc_matches_workspace_entry_point(dtype):
    big = workloads.PrefillSpec("big", [2048, 1000, 1048], heads=96, conv=False, h0_std=0.05,
                                dtype=dtype, seed=91)
    small = workloads.PrefillSpec("small", [37, 200], heads=8, conv=False, h0_std=0.05,
                                  dtype=dtype, seed=92)
    for spec in (big, small):
        note("no-alloc chunk call: %d tokens x %d heads" % (spec.total_tokens, spec.heads))
        inp = workloads.make_prefill(spec, DEV)
        got_o, got_h = no_alloc(inp, spec)
        ref_o, ref_h = reference(inp, spec)
        torch.cuda.synchronize()
        got_o.check()
        got_h.check()
        assert bool(torch.isfinite(got_o.t).all()) and bool(torch.isfinite(got_h.t).all())
        assert torch.equal(got_o.t, ref_o), "o differs from kda_chunk_fwd's"
        assert torch.equal(got_h.t, ref_h), "final state differs from kda_chunk_fwd's"


def test_no_alloc_refuses_beyond_the_scratch():
    # Tb / P rows of 5462 x 96 = 524352 token-heads: above the scratch's 524288
    spec = workloads.PrefillSpec("over", [5462], heads=96, conv=False, dtype=torch.float32,
                                 seed=93)
    inp = workloads.make_prefill(spec, DEV)
    o = torch.full((spec.total_tokens, 96, 128), float("nan"), device=DEV)
    with pytest.raises(kda.KdaError) as e:
        kda.chunk_fwd_noalloc(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], o, None,
                              scale=spec.read_scale)
    assert e.value.status == kda.KDA_ERR_UNSUPPORTED and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool(torch.isnan(o).all()), "a refused call wrote its output"
