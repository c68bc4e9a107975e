"""Shared plumbing of the GPU parity tests: run the HIP path through the binding,
run the oracle on the same inputs (optionally on a sample of heads), compare."""
from __future__ import annotations

import sys

import numpy as np
import torch

import channel_gated_delta_amd as kda
import oracle
from channel_gated_delta_amd import workloads

TOL_BF16 = 2e-2   # max|gpu - oracle| / rms(oracle), bf16 inputs
TOL_F32 = 1e-4    # same, fp32 inputs


def tol_for(dtype) -> float:
    return TOL_BF16 if dtype == torch.bfloat16 else TOL_F32


def note(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().double().cpu().numpy()


def gpu_prefill(inp, spec, chunk=None, out=None, gate=None):
    """HIP path: prologue (if the workload has raw projections) then chunk_fwd, or
    chunk_fwd_gated when ``gate`` (workloads.make_gate's z, a_log, dt_bias; the
    last two may be None) is given."""
    H, DK, DV = spec.heads, spec.dk, spec.dv
    cu = inp["cu_seqlens"]
    if spec.conv:
        q, _ = kda.short_conv(inp["q_raw"], inp["w_q"], num_heads=H, head_dim=DK, cu_seqlens=cu,
                              l2_normalize=True)
        k, _ = kda.short_conv(inp["k_raw"], inp["w_k"], num_heads=H, head_dim=DK, cu_seqlens=cu,
                              l2_normalize=True)
        v, _ = kda.short_conv(inp["v_raw"], inp["w_v"], num_heads=H, head_dim=DV, cu_seqlens=cu)
    else:
        q, k, v = inp["q"], inp["k"], inp["v"]
    if gate is None:
        o, hT = kda.chunk_fwd(q, k, v, inp["g"], inp["beta"], cu_seqlens=cu,
                              scale=spec.read_scale, gate_lower_bound=spec.gate_lb,
                              chunk_size=chunk or spec.chunk, initial_state=inp["h0"], out=out)
    else:
        o, hT = kda.chunk_fwd_gated(q, k, v, gate["z"], inp["beta"], a_log=gate.get("a_log"),
                                    dt_bias=gate.get("dt_bias"), lower_bound=spec.gate_lb,
                                    cu_seqlens=cu, scale=spec.read_scale,
                                    chunk_size=chunk or spec.chunk, initial_state=inp["h0"],
                                    out=out)
    return dict(q=q, k=k, v=v, o=o, hT=hT)


def oracle_prefill(inp, spec, heads, gate=None):
    """Oracle on the sampled heads: fp64 prologue (conv + SiLU + L2), the bounded
    gate from ``gate``'s inputs if given (else the workload's g), the recurrence."""
    H, DK, DV = spec.heads, spec.dk, spec.dv
    cu = inp["cu_seqlens"].cpu().numpy()
    heads = list(heads)

    def chans(x, D):
        x = x.view(x.shape[0], H, D)[:, heads, :]
        return to64(x.reshape(x.shape[0], len(heads) * D))

    def wch(w, D):
        return to64(w.view(H, D, -1)[heads].reshape(len(heads) * D, -1))

    if spec.conv:
        # q, k, v reach the recurrence as tensors of the activation dtype (O1c)
        rb = spec.dtype == torch.bfloat16
        q = oracle.prologue(chans(inp["q_raw"], DK), wch(inp["w_q"], DK), len(heads), DK, cu,
                            normalize=True, out_bf16=rb)
        k = oracle.prologue(chans(inp["k_raw"], DK), wch(inp["w_k"], DK), len(heads), DK, cu,
                            normalize=True, out_bf16=rb)
        v = oracle.prologue(chans(inp["v_raw"], DV), wch(inp["w_v"], DV), len(heads), DV, cu,
                            out_bf16=rb)
    else:
        q = to64(inp["q"][:, heads])
        k = to64(inp["k"][:, heads])
        v = to64(inp["v"][:, heads])
    if gate is None:
        g = to64(inp["g"][:, heads])
    else:
        al, dt = gate.get("a_log"), gate.get("dt_bias")
        g = oracle.bounded_gate(to64(gate["z"][:, heads]), None if al is None else to64(al[heads]),
                                None if dt is None else to64(dt[heads]), spec.gate_lb)
    beta = to64(inp["beta"][:, heads])
    h0 = None if inp["h0"] is None else to64(inp["h0"][:, heads])
    o, hT = oracle.recurrent(q, k, v, g, beta, cu_seqlens=cu, scale=spec.read_scale, h0=h0)
    return dict(q=q, k=k, v=v, o=o, hT=hT)


def assert_prologue(got, ref, dtype):
    """The prologue's q, k, v against the oracle's: bf16 outputs are the correctly
    rounded values, so they must be identical; fp32 outputs agree to 1e-5 relative."""
    for name in ("q", "k", "v"):
        g, r = np.asarray(got[name], dtype=np.float64), np.asarray(ref[name], dtype=np.float64)
        if dtype == torch.bfloat16:
            bad = int(np.sum(g != r))
            note("  prologue %s: %d of %d bf16 values differ" % (name, bad, g.size))
            assert bad == 0, "prologue %s: %d values differ from the oracle" % (name, bad)
        else:
            err = float(np.max(np.abs(g - r) / (np.abs(r) + 1e-30)))
            note("  prologue %s: max rel err %.3e" % (name, err))
            assert err <= 1e-5, "prologue %s: rel err %.3e" % (name, err)


def assert_parity(name, got, ref, tol):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = oracle.rel_err(got, ref)
    note("  %-28s rel err %.3e (tol %.0e)" % (name, err, tol))
    if not (np.isfinite(err) and err <= tol):
        d = np.abs(got - ref)
        d[~np.isfinite(d)] = np.inf
        idx = np.unravel_index(int(np.argmax(d)), d.shape)
        note("  worst element %s: got %r ref %r (rms ref %.3e, nonfinite %d)" %
             (idx, got[idx], ref[idx], float(np.sqrt(np.mean(ref * ref))),
              int(np.sum(~np.isfinite(got)))))
    assert np.isfinite(err) and err <= tol, "%s: rel err %.3e > %.0e" % (name, err, tol)
    return err
