"""The five workloads at full size, HIP path vs the fp64 oracle (needs an MI355X).

The GPU runs every head at the full shape, in the launch configuration that
bench.py times, with every output poisoned (NaN) and guarded beforehand.  The
oracle then recomputes every head (every (sequence, head) pair for decode) from
the same seeded inputs, a batch of heads at a time to bound host memory, and
every element is compared.  Bar: max|gpu - oracle| / rms(oracle) <= 2e-2 (bf16
inputs) or 1e-4 (fp32 inputs) over each whole output and final state; the bf16
prologue outputs must equal the oracle's correctly rounded values bit for bit.
"""
import numpy as np
import pytest
import torch

import channel_gated_delta_amd as kda
import oracle
from channel_gated_delta_amd import workloads
from gpu_helpers import (Parity, assert_prologue, check_written, gpu_prefill, guarded, note,
                         oracle_prefill, to64, tol_for)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def head_batches(H, size):
    return [list(range(h, min(h + size, H))) for h in range(0, H, size)]


def compare_all_heads(inp, spec, got, gate=None, g_head=None, head_batch=16, label=""):
    """Every head of o and of the final states against the oracle, batch by batch."""
    tol = tol_for(spec.dtype)
    po, ph = Parity("o%s (all heads)" % label), Parity("final state%s (all heads)" % label)
    for heads in head_batches(spec.heads, head_batch):
        ref = oracle_prefill(inp, spec, heads, gate=gate, g_head=g_head)
        if spec.conv and gate is None and g_head is None:
            gp = {n: to64(got[n][:, heads]) for n in ("q", "k", "v")}
            assert_prologue(gp, ref, spec.dtype)
        po.add(to64(got["o"][:, heads]), ref["o"], where="heads %d-%d" % (heads[0], heads[-1]))
        ph.add(to64(got["hT"][:, heads]), ref["hT"], where="heads %d-%d" % (heads[0], heads[-1]))
        note("  heads %d-%d: o err so far %.3e, state %.3e" %
             (heads[0], heads[-1], po.err(), ph.err()))
        del ref
    po.check(tol)
    ph.check(tol)


def run_prefill_workload(name, fused_gate=False, head_batch=16):
    spec = workloads.standard_specs()[name]
    note("workload %s%s: %d tokens, all %d heads" %
         (spec.name, " (fused gate)" if fused_gate else "", spec.total_tokens, spec.heads))
    inp = workloads.make_prefill(spec, DEV)
    gate = workloads.make_gate(spec, DEV) if fused_gate else None
    got = gpu_prefill(inp, spec, gate=gate)
    check_written(got)
    compare_all_heads(inp, spec, got, gate=gate, head_batch=head_batch)
    return spec


def test_tiny_fp32_workload_full():
    """B=1, H=1, T=64, d=16, chunk 16, fp32: every output against the oracle."""
    run_prefill_workload("tiny_fp32")


@pytest.mark.timeout(600)
def test_prefill_workload():
    """B=1, T=4096, H=96, d=128, bf16, conv4+SiLU+L2 prologue, zero h0: all heads."""
    run_prefill_workload("prefill", head_batch=48)


@pytest.mark.timeout(600)
def test_prefill_workload_fused_gate():
    """The prefill workload with the bounded gate formed in the kernels from bf16 z."""
    run_prefill_workload("prefill", fused_gate=True, head_batch=48)


@pytest.mark.timeout(600)
def test_prefill_workload_output_epilogue():
    """The prefill read-out (fp32 o) through the per-head RMSNorm and sigmoid output gate
    (bf16 y), in the configuration bench.py times; every element."""
    spec = workloads.standard_specs()["prefill"]
    inp = workloads.make_prefill(spec, DEV)
    ep = workloads.make_epilogue(spec, DEV)
    got = gpu_prefill(inp, spec)
    reg = []
    y = guarded(tuple(ep["gate"].shape), ep["gate"].dtype, DEV, "y", reg)
    kda.output_norm_gate(got["o"], ep["gate"], ep["weight"], eps=1e-6, out=y)
    check_written(got)
    reg[0].check()
    assert bool(torch.isfinite(y.float()).all())
    worst, rms = 0.0, 0.0
    for heads in head_batches(spec.heads, 48):
        ref = oracle.output_norm_gate(to64(got["o"][:, heads]), to64(ep["gate"][:, heads]),
                                      to64(ep["weight"]), 1e-6)
        g = to64(y[:, heads])
        r = float(np.sqrt(np.mean(ref * ref)))
        bound = 2.0 ** -8 * np.abs(ref) + 1e-6 * r
        excess = np.abs(g - ref) - bound
        worst = max(worst, float(np.max(np.abs(g - ref))) / r)
        assert np.all(excess <= 0), "heads %s: max excess %.3e" % (heads, float(np.max(excess)))
    note("  epilogue: max |y - ref| / rms(ref) = %.3e (all heads)" % worst)


@pytest.mark.timeout(600)
def test_prefill_workload_gdn():
    """The prefill workload (conv prologue on the GPU) with one decay per (token, head)."""
    spec = workloads.standard_specs()["prefill"]
    inp = workloads.make_prefill(spec, DEV)
    gh = workloads.make_head_gate(spec, DEV)
    H, DK, DV, T = spec.heads, spec.dk, spec.dv, spec.total_tokens
    reg = []
    q = guarded((T, H, DK), spec.dtype, DEV, "q", reg)
    k = guarded((T, H, DK), spec.dtype, DEV, "k", reg)
    v = guarded((T, H, DV), spec.dtype, DEV, "v", reg)
    o = guarded((T, H, DV), torch.float32, DEV, "o", reg)
    hT = guarded((1, H, DK, DV), torch.float32, DEV, "final state", reg)
    ws = guarded((kda.chunk_workspace_bytes(T, H, DK, DV),), torch.uint8, DEV, "workspace", reg)
    kda.short_conv(inp["q_raw"], inp["w_q"], num_heads=H, head_dim=DK, l2_normalize=True, out=q)
    kda.short_conv(inp["k_raw"], inp["w_k"], num_heads=H, head_dim=DK, l2_normalize=True, out=k)
    kda.short_conv(inp["v_raw"], inp["w_v"], num_heads=H, head_dim=DV, out=v)
    kda.gdn_chunk_fwd(q, k, v, gh, inp["beta"], scale=spec.read_scale,
                      gate_lower_bound=spec.gate_lb, chunk_size=spec.chunk, out=o,
                      final_state=hT, workspace=ws)
    got = dict(q=q, k=k, v=v, o=o, hT=hT, _guards=reg)
    check_written(got)
    compare_all_heads(inp, spec, got, g_head=gh, head_batch=48, label=" (GDN)")


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
        o = torch.full((B, H, DV), float("nan"), device=DEV)
        outs.append(kda.decode_step_conv(d["q_raw"], d["k_raw"], d["v_raw"], cv["w_q"], cv["w_k"],
                                         cv["w_v"], cv["conv_q"], cv["conv_k"], cv["conv_v"],
                                         d["g"], d["beta"], state, scale=spec.dk ** -0.5,
                                         out=o))
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
    po, ph = Parity("o (all pairs, all steps)"), Parity("final state (all pairs)")
    po.add(got_o, o)
    ph.add(to64(state), hT)
    po.check(2e-2)
    ph.check(2e-2)


@pytest.mark.timeout(600)
def test_varlen_workload():
    """8 packed sequences (32768 tokens), random h0 per sequence, conv reset per sequence."""
    run_prefill_workload("varlen", head_batch=16)


@pytest.mark.timeout(1200)
def test_long_workload():
    """B=1, T=131072, H=96, g = -8 sigmoid(N(0, 2)); the oracle runs the whole sequence for
    every head (16 heads at a time); every o and the final states are compared."""
    run_prefill_workload("long", head_batch=16)


@pytest.mark.timeout(900)
def test_decode_workload():
    """64 sequences x 96 heads, 256 in-place steps; every (sequence, head) pair and every
    step's o, a batch of sequences at a time on the oracle."""
    spec = workloads.standard_specs()["decode"]
    B, H, DK, DV, steps = spec.batch, spec.heads, spec.dk, spec.dv, spec.steps
    note("decode workload: %d x %d heads, %d steps, all pairs" % (B, H, steps))
    state = workloads.make_decode_state(spec, DEV)
    s0 = state.cpu()
    o = torch.empty((steps, B, H, DV), dtype=torch.float32, device=DEV)
    o.fill_(float("nan"))
    keep = {key: [] for key in ("q", "k", "v", "g", "beta")}
    for t in range(steps):
        d = workloads.make_decode_step(spec, t, DEV)
        kda.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state, out=o[t])
        for key in keep:
            keep[key].append(d[key].cpu())
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(state).all())
    got_o = o.cpu()
    got_s = state.cpu()
    del o
    po, ph = Parity("decode o (all pairs, all steps)"), Parity("decode state (all pairs)")
    SB = 16
    for b0 in range(0, B, SB):
        b1 = min(b0 + SB, B)
        nb = b1 - b0

        def seq(key):   # steps x [B, H, ...] -> sequence-major [nb * steps, H, ...]
            x = torch.stack([s[b0:b1] for s in keep[key]], dim=1)
            return x.double().numpy().reshape(nb * steps, *x.shape[2:])

        ro, rh = oracle.recurrent(seq("q"), seq("k"), seq("v"), seq("g"), seq("beta"),
                                  np.arange(nb + 1) * steps, DK ** -0.5,
                                  s0[b0:b1].double().numpy())
        go = got_o[:, b0:b1].permute(1, 0, 2, 3).double().numpy().reshape(nb * steps, H, DV)
        po.add(go, ro, where="sequences %d-%d" % (b0, b1 - 1))
        ph.add(got_s[b0:b1].double().numpy(), rh, where="sequences %d-%d" % (b0, b1 - 1))
        note("  sequences %d-%d: o err so far %.3e, state %.3e" % (b0, b1 - 1, po.err(), ph.err()))
    po.check(2e-2)
    ph.check(2e-2)
