"""The five workloads at full size, HIP path vs the fp64 oracle (needs an MI355X).

The GPU runs every head at the full shape, in the launch configuration that
bench.py times; the oracle recomputes a sample of heads (or of (sequence, head)
pairs for decode) from the same seeded inputs, one by one.  Every other output
is checked for finiteness.  Bar: max|gpu - oracle| / rms(oracle) <= 2e-2 (bf16
inputs) or 1e-4 (fp32 inputs) on outputs and final states.
"""
import numpy as np
import pytest
import torch

import channel_gated_delta_amd as kda
import oracle
from channel_gated_delta_amd import workloads
from gpu_helpers import (assert_parity, assert_prologue, gpu_prefill, note, oracle_prefill, to64,
                         tol_for)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_prefill_workload(name, heads, fused_gate=False):
    spec = workloads.standard_specs()[name]
    note("workload %s%s: %d tokens, sampled heads %s" %
         (spec.name, " (fused gate)" if fused_gate else "", spec.total_tokens, heads))
    inp = workloads.make_prefill(spec, DEV)
    gate = workloads.make_gate(spec, DEV) if fused_gate else None
    got = gpu_prefill(inp, spec, gate=gate)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(got["o"]).all()) and bool(torch.isfinite(got["hT"]).all())
    go = to64(got["o"][:, heads])
    gh = to64(got["hT"][:, heads])
    gp = {name: to64(got[name][:, heads]) for name in ("q", "k", "v")} if spec.conv else None
    del got
    ref = oracle_prefill(inp, spec, heads, gate=gate)
    tol = tol_for(spec.dtype)
    if gp is not None:
        assert_prologue(gp, ref, spec.dtype)
    assert_parity("o (sampled heads)", go, ref["o"], tol)
    assert_parity("final state (sampled heads)", gh, ref["hT"], tol)
    return spec


def test_tiny_fp32_workload_full():
    """B=1, H=1, T=64, d=16, chunk 16, fp32: every output against the oracle."""
    run_prefill_workload("tiny_fp32", [0])


@pytest.mark.timeout(600)
def test_prefill_workload():
    """B=1, T=4096, H=96, d=128, chunk 64, bf16, conv4+SiLU+L2 prologue, zero h0."""
    run_prefill_workload("prefill", [0, 41, 95])


@pytest.mark.timeout(600)
def test_prefill_workload_fused_gate():
    """The prefill workload with the bounded gate formed in the kernels from bf16 z."""
    run_prefill_workload("prefill", [5, 60], fused_gate=True)


@pytest.mark.timeout(600)
def test_prefill_workload_output_epilogue():
    """The prefill read-out (fp32 o) through the per-head RMSNorm and sigmoid output gate
    (bf16 y), in the configuration bench.py times; sampled heads element by element."""
    spec = workloads.standard_specs()["prefill"]
    inp = workloads.make_prefill(spec, DEV)
    ep = workloads.make_epilogue(spec, DEV)
    got = gpu_prefill(inp, spec)
    y = kda.output_norm_gate(got["o"], ep["gate"], ep["weight"], eps=1e-6)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y.float()).all())
    heads = [2, 50, 93]
    ref = oracle.output_norm_gate(to64(got["o"][:, heads]), to64(ep["gate"][:, heads]),
                                  to64(ep["weight"]), 1e-6)
    g = to64(y[:, heads])
    bound = 2.0 ** -8 * np.abs(ref) + 1e-6 * float(np.sqrt(np.mean(ref * ref)))
    excess = np.abs(g - ref) - bound
    note("  epilogue: max |y - ref| / rms(ref) = %.3e" %
         (float(np.max(np.abs(g - ref))) / float(np.sqrt(np.mean(ref * ref)))))
    assert np.all(excess <= 0), "max excess %.3e" % float(np.max(excess))


@pytest.mark.timeout(600)
def test_prefill_workload_gdn():
    """The prefill workload (conv prologue on the GPU) with one decay per (token, head)."""
    spec = workloads.standard_specs()["prefill"]
    inp = workloads.make_prefill(spec, DEV)
    gh = workloads.make_head_gate(spec, DEV)
    H, DK, DV = spec.heads, spec.dk, spec.dv
    q, _ = kda.short_conv(inp["q_raw"], inp["w_q"], num_heads=H, head_dim=DK, l2_normalize=True)
    k, _ = kda.short_conv(inp["k_raw"], inp["w_k"], num_heads=H, head_dim=DK, l2_normalize=True)
    v, _ = kda.short_conv(inp["v_raw"], inp["w_v"], num_heads=H, head_dim=DV)
    o, hT = kda.gdn_chunk_fwd(q, k, v, gh, inp["beta"], scale=spec.read_scale,
                              gate_lower_bound=spec.gate_lb, chunk_size=spec.chunk)
    torch.cuda.synchronize()
    heads = [1, 47, 94]
    cu = inp["cu_seqlens"].cpu().numpy()
    g = np.repeat(to64(gh[:, heads])[:, :, None], DK, axis=2)
    ro, rh = oracle.recurrent(to64(q[:, heads]), to64(k[:, heads]), to64(v[:, heads]), g,
                              to64(inp["beta"][:, heads]), cu, spec.read_scale)
    assert_parity("o (GDN, sampled heads)", to64(o[:, heads]), ro, 2e-2)
    assert_parity("final state (GDN, sampled heads)", to64(hT[:, heads]), rh, 2e-2)


@pytest.mark.timeout(600)
def test_decode_conv_workload():
    """64 sequences x 96 heads, 8 fused steps (conv + SiLU + L2 + the recurrent step) from
    raw projections and conv caches; every (sequence, head) against the oracle."""
    spec = workloads.standard_specs()["decode"]
    B, H, DK, DV, steps = spec.batch, spec.heads, spec.dk, spec.dv, 8
    note("decode+conv workload %d x %d heads, %d steps" % (B, H, steps))
    state = workloads.make_decode_state(spec, DEV)
    cv = workloads.make_decode_conv(spec, DEV)
    s0 = to64(state)
    c0 = {n: to64(cv["conv_" + n]) for n in "qkv"}
    ins, outs = [], []
    for t in range(steps):
        d = workloads.make_decode_conv_step(spec, t, DEV)
        outs.append(kda.decode_step_conv(d["q_raw"], d["k_raw"], d["v_raw"], cv["w_q"], cv["w_k"],
                                         cv["w_v"], cv["conv_q"], cv["conv_k"], cv["conv_v"],
                                         d["g"], d["beta"], state, scale=spec.dk ** -0.5))
        ins.append({key: val.cpu() for key, val in d.items()})
    torch.cuda.synchronize()
    got_o = to64(torch.stack(outs, dim=1).reshape(B * steps, H, DV))
    del outs

    def packed(key):
        x = torch.stack([i[key] for i in ins], dim=1)
        return x.double().numpy().reshape(B * steps, *x.shape[2:])

    cu = np.arange(B + 1) * steps
    q = oracle.prologue(packed("q_raw"), to64(cv["w_q"]), H, DK, cu, state_in=c0["q"],
                        normalize=True)
    k = oracle.prologue(packed("k_raw"), to64(cv["w_k"]), H, DK, cu, state_in=c0["k"],
                        normalize=True)
    v = oracle.prologue(packed("v_raw"), to64(cv["w_v"]), H, DV, cu, state_in=c0["v"])
    o, hT = oracle.recurrent(q, k, v, packed("g"), packed("beta"), cu, spec.dk ** -0.5, s0)
    assert_parity("o (all pairs, all steps)", got_o, o, 2e-2)
    assert_parity("final state", to64(state), hT, 2e-2)


@pytest.mark.timeout(600)
def test_varlen_workload():
    """8 packed sequences (32768 tokens), random h0 per sequence, conv reset per sequence."""
    run_prefill_workload("varlen", [7, 64])


@pytest.mark.timeout(900)
def test_long_workload():
    """B=1, T=131072, H=96, g = -8 sigmoid(N(0, 2)); oracle over the whole sequence."""
    run_prefill_workload("long", [3, 90])


@pytest.mark.timeout(600)
def test_decode_workload():
    """64 sequences x 96 heads, 256 in-place steps; sampled (sequence, head) pairs."""
    spec = workloads.standard_specs()["decode"]
    B, H, DK, DV, steps = spec.batch, spec.heads, spec.dk, spec.dv, spec.steps
    pairs = [(0, 0), (5, 17), (31, 48), (40, 95), (63, 7), (63, 95)]
    note("decode workload: %d x %d heads, %d steps, pairs %s" % (B, H, steps, pairs))
    state = workloads.make_decode_state(spec, DEV)
    bi = torch.tensor([p[0] for p in pairs], device=DEV)
    hi = torch.tensor([p[1] for p in pairs], device=DEV)
    s0 = state[bi, hi].clone()
    o = torch.empty((B, H, DV), dtype=torch.float32, device=DEV)
    keep = {key: [] for key in ("q", "k", "v", "g", "beta")}
    outs = []
    for t in range(steps):
        d = workloads.make_decode_step(spec, t, DEV)
        kda.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state, out=o)
        outs.append(o[bi, hi].clone())
        for key in keep:
            keep[key].append(d[key][bi, hi])
        assert bool(torch.isfinite(o).all())
    torch.cuda.synchronize()
    assert bool(torch.isfinite(state).all())
    P = len(pairs)

    def seq(key):
        x = torch.stack(keep[key], dim=1)          # [P, steps, ...]
        return to64(x.reshape(P * steps, 1, *x.shape[2:]))

    ro, rh = oracle.recurrent(seq("q"), seq("k"), seq("v"), seq("g"),
                              seq("beta").reshape(P * steps, 1), np.arange(P + 1) * steps,
                              DK ** -0.5, to64(s0).reshape(P, 1, DK, DV))
    go = to64(torch.stack(outs, dim=1).reshape(P * steps, 1, DV))
    assert_parity("decode o (sampled pairs)", go, ro, 2e-2)
    assert_parity("decode state (sampled pairs)", to64(state[bi, hi]).reshape(P, 1, DK, DV), rh,
                  2e-2)
