"""Shared plumbing of the GPU parity tests: run the HIP path through the binding,
run the oracle on the same inputs (in batches of heads for the full-size
workloads), compare.

Every output the HIP path writes lands in a buffer that was filled with NaN
before the call and sits between two guard bands of a sentinel value: after the
call no NaN may remain (every element was written) and the guard bands must be
untouched (nothing was written outside the buffer).  The chunk workspace is
filled with 0xFF bytes (fp32 NaN) the same way, so stale Tb / P rows from an
earlier call cannot stand in for rows a kernel failed to write.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import channel_gated_delta_amd as kda
import oracle

TOL_BF16 = 2e-2   # max|gpu - oracle| / rms(oracle), bf16 inputs
TOL_F32 = 1e-4    # same, fp32 inputs

GUARD_BYTES = 4096         # guard band on each side of an output buffer
SENTINEL = -7.75           # exact in bf16 and fp32
SENTINEL_BYTE = 0xA5


def tol_for(dtype) -> float:
    return TOL_BF16 if dtype == torch.bfloat16 else TOL_F32


def note(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().double().cpu().numpy()


class Guarded:
    """An output tensor filled with NaN (0xFF bytes for uint8), placed between two
    guard bands of a sentinel; ``check`` verifies the bands after the calls."""

    def __init__(self, shape, dtype, device, name):
        self.name = name
        esz = torch.empty(0, dtype=dtype).element_size()
        self.g = GUARD_BYTES // esz
        self.n = int(np.prod(shape)) if len(shape) else 1
        self.buf = torch.empty(self.n + 2 * self.g, dtype=dtype, device=device)
        self.fill = SENTINEL if dtype.is_floating_point else SENTINEL_BYTE
        self.buf.fill_(self.fill)
        self.t = self.buf[self.g:self.g + self.n].view(tuple(shape))
        self.t.fill_(float("nan") if dtype.is_floating_point else 0xFF)

    def check(self):
        head, tail = self.buf[:self.g], self.buf[self.g + self.n:]
        assert bool((head == self.fill).all()) and bool((tail == self.fill).all()), \
            "%s: a kernel wrote outside the buffer" % self.name


def guarded(shape, dtype, device, name, registry):
    g = Guarded(shape, dtype, device, name)
    registry.append(g)
    return g.t


def check_written(got):
    """After the calls of gpu_prefill: synchronise, check the guard bands, and check
    that no NaN is left in an output (every element was written)."""
    torch.cuda.synchronize()
    for g in got["_guards"]:
        g.check()
    for name in ("q", "k", "v", "o", "hT"):
        t = got.get(name)
        if t is not None and t.is_floating_point() and t.numel():
            bad = int((~torch.isfinite(t)).sum())
            assert bad == 0, "%s: %d elements not finite (unwritten or overflow)" % (name, bad)


def gpu_prefill(inp, spec, chunk=None, gate=None, out_dtype=torch.float32):
    """HIP path: prologue (if the workload has raw projections) then chunk_fwd, or
    chunk_fwd_gated when ``gate`` (workloads.make_gate's z, a_log, dt_bias; the
    last two may be None) is given.  Outputs and the workspace are poisoned and
    guarded (see the module docstring); call check_written() afterwards."""
    H, DK, DV = spec.heads, spec.dk, spec.dv
    T, N = spec.total_tokens, len(spec.lengths)
    dev = inp["beta"].device
    cu = inp["cu_seqlens"]
    reg = []
    if spec.conv:
        q = guarded((T, H, DK), spec.dtype, dev, "q", reg)
        k = guarded((T, H, DK), spec.dtype, dev, "k", reg)
        v = guarded((T, H, DV), spec.dtype, dev, "v", reg)
        kda.short_conv(inp["q_raw"], inp["w_q"], num_heads=H, head_dim=DK, cu_seqlens=cu,
                       l2_normalize=True, out=q)
        kda.short_conv(inp["k_raw"], inp["w_k"], num_heads=H, head_dim=DK, cu_seqlens=cu,
                       l2_normalize=True, out=k)
        kda.short_conv(inp["v_raw"], inp["w_v"], num_heads=H, head_dim=DV, cu_seqlens=cu, out=v)
    else:
        q, k, v = inp["q"], inp["k"], inp["v"]
    o = guarded((T, H, DV), out_dtype, dev, "o", reg)
    hT = guarded((N, H, DK, DV), torch.float32, dev, "final state", reg)
    ws_bytes = kda.chunk_workspace_bytes(T, H, DK, DV, chunk or spec.chunk, spec.dtype, out_dtype)
    ws = guarded((max(ws_bytes, 1),), torch.uint8, dev, "workspace", reg)
    if gate is None:
        kda.chunk_fwd(q, k, v, inp["g"], inp["beta"], cu_seqlens=cu, scale=spec.read_scale,
                      gate_lower_bound=spec.gate_lb, chunk_size=chunk or spec.chunk,
                      initial_state=inp["h0"], out=o, final_state=hT, workspace=ws)
    else:
        kda.chunk_fwd_gated(q, k, v, gate["z"], inp["beta"], a_log=gate.get("a_log"),
                            dt_bias=gate.get("dt_bias"), lower_bound=spec.gate_lb,
                            cu_seqlens=cu, scale=spec.read_scale,
                            chunk_size=chunk or spec.chunk, initial_state=inp["h0"], out=o,
                            final_state=hT, workspace=ws)
    return dict(q=q, k=k, v=v, o=o, hT=hT, _guards=reg)


def oracle_prefill(inp, spec, heads, gate=None, g_head=None):
    """Oracle on the given heads: fp64 prologue (conv + SiLU + L2), the bounded gate
    from ``gate``'s inputs if given (else the per-head decay ``g_head`` [T, H] if
    given, else the workload's g), the recurrence."""
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
    if gate is not None:
        al, dt = gate.get("a_log"), gate.get("dt_bias")
        g = oracle.bounded_gate(to64(gate["z"][:, heads]), None if al is None else to64(al[heads]),
                                None if dt is None else to64(dt[heads]), spec.gate_lb)
    elif g_head is not None:
        g = np.repeat(to64(g_head[:, heads])[:, :, None], DK, axis=2)
    else:
        g = to64(inp["g"][:, heads])
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
            if bad:
                note("  prologue %s: %d of %d bf16 values differ" % (name, bad, g.size))
            assert bad == 0, "prologue %s: %d values differ from the oracle" % (name, bad)
        else:
            err = float(np.max(np.abs(g - r) / (np.abs(r) + 1e-30)))
            note("  prologue %s: max rel err %.3e" % (name, err))
            assert err <= 1e-5, "prologue %s: rel err %.3e" % (name, err)


class Parity:
    """max|got - ref| / rms(ref) over a tensor compared in pieces (the same value
    oracle.rel_err gives on the whole tensor)."""

    def __init__(self, name):
        self.name, self.maxd, self.ss, self.n = name, 0.0, 0.0, 0
        self.worst = None

    def add(self, got, ref, where=""):
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        d = np.abs(got - ref)
        d[~np.isfinite(d)] = np.inf
        if d.size:
            i = np.unravel_index(int(np.argmax(d)), d.shape)
            if float(d[i]) > self.maxd or self.worst is None:
                self.maxd = max(self.maxd, float(d[i]))
                self.worst = (where, i, got[i], ref[i])
        self.ss += float(np.sum(ref * ref))
        self.n += ref.size

    def err(self) -> float:
        rms = float(np.sqrt(self.ss / self.n)) if self.n else 0.0
        return self.maxd / rms if rms > 0 else self.maxd

    def check(self, tol):
        err = self.err()
        note("  %-36s rel err %.3e (tol %.0e, %d elements)" % (self.name, err, tol, self.n))
        if not (np.isfinite(err) and err <= tol):
            note("  worst element %s" % (self.worst,))
        assert np.isfinite(err) and err <= tol, "%s: rel err %.3e > %.0e" % (self.name, err, tol)
        return err


def assert_parity(name, got, ref, tol):
    p = Parity(name)
    p.add(got, ref)
    return p.check(tol)
