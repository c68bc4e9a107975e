"""Benchmark of the KDA forward hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill|varlen|long]

A step is one pass of the prefill path over one batch of synthetic input resident
in HBM: the conv4 + SiLU (+ q/k L2) prologue on q, k, v followed by the
chunkwise KDA call (B=1, T=4096, H=96, dk=dv=128, bf16; chunk 64 requested, the
kernels walk 16-token chunks; final state written).  ``value`` is prefill
tokens/s.  The same JSON line carries:

* ``roofline``: the chunk call's algorithmic HBM bytes per launch (q, k, v bf16,
  g fp32, beta, o counted as bf16: 1540 B per token and head, plus the states)
  divided by its average launch duration, timed with HIP events on the stream it
  runs on, against the 8 TB/s HBM peak.  The call writes o in fp32 (1796 B per
  token and head); ``frac_fp32_o`` is the fraction on those bytes.  ``traffic``
  is the measured HBM traffic per launch from the committed rocprofv3 counter
  summary when it was taken on the current kernel source, else null;
* ``mfma``: the call's useful bf16 MFMA work (the chunk algorithm's product
  flops, split terms not counted) per second against the 2.5 PFLOP/s dense peak;
* ``hbm_copy``: a plain device-to-device copy of 1 GiB timed the same way (the
  bandwidth this GPU attains on a streaming copy, beside the 8 TB/s spec);
* ``varlen``, ``long``: the same step on the packed variable-length workload
  (8 sequences, 32768 tokens, random h0) and the long-context workload
  (131072 tokens, gates down to -8), with their chunk calls' rooflines;
* ``decode``: 256 in-place decode steps of 64 sequences x 96 heads (steps/s) and
  the decode kernel's roofline;
* ``fused_gate``: the prefill step with the bounded gate formed inside the chunk
  kernels from bf16 pre-activations (kda_chunk_fwd_gated) instead of a
  precomputed fp32 g, and that call's roofline;
* ``output_epilogue``: the per-head RMSNorm and sigmoid output gate applied to the
  step's fp32 read-out (bf16 gate in, bf16 y out), timed alone, and its roofline;
* ``decode_conv``: the same 256 decode steps from raw projections with the conv,
  SiLU and q/k L2 fused in (kda_decode_step_conv; conv caches updated in place);
* ``gdn``: the prefill step with one decay per (token, head) (kda_gdn_chunk_fwd,
  g [T, H]) and that call's roofline;
* ``cpu_baseline``: the fp64 oracle (prologue + recurrence) timed on this host's
  cores over the same workload, repeated for at least ten seconds.

Only one GPU is used; ``--gpus`` above 1 is refused.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "KDA prefill tokens/s (H=96, d=128) + decode steps/s; % of roofline"


KERNEL_SOURCES = {
    "chunk": ("kda_device.cuh", "kda_chunk_common.cuh", "kda_chunk_prep.cuh", "kda_chunk_state.cuh",
              "kda_chunk_dispatch.cuh", "kda_chunk_bf16.hip"),
    "decode": ("kda_device.cuh", "kda_decode.hip"),
    "decodeconv": ("kda_device.cuh", "kda_decode.hip"),
    "gated": ("kda_device.cuh", "kda_chunk_common.cuh", "kda_chunk_prep.cuh",
              "kda_chunk_state.cuh", "kda_chunk_dispatch.cuh", "kda_chunk_bf16_gz.hip"),
    "epilogue": ("kda_device.cuh", "kda_epilogue.hip"),
    "gdn": ("kda_device.cuh", "kda_chunk_common.cuh", "kda_chunk_prep.cuh",
            "kda_chunk_state.cuh", "kda_chunk_dispatch.cuh", "kda_chunk_bf16_gdn.hip"),
}


def code_text(src: str) -> str:
    """C/C++ source without comments and with whitespace runs collapsed: what the
    compiler sees, so that editing a comment does not date a counter summary."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def kernel_source_digest(kind: str) -> str:
    """Hash of the code (comments and layout excluded) of the sources a kernel is built
    from, to date counter summaries."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "channel_gated_delta_amd", "csrc")
    for name in KERNEL_SOURCES[kind]:
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kind: str, workload: str):
    """HBM bytes per launch from profiles/<kind>_<workload>_traffic.md, if that summary was
    taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "%s_%s_traffic.md" % (kind, workload))
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source_digest:\s*([0-9a-f]+)", text)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != kernel_source_digest(kind):
        return None
    return float(t.group(1))


def prefill_step_bytes(T: int, H: int, dk: int, dv: int, N: int, h0: bool,
                       o_bytes: int = 2) -> float:
    """Algorithmic HBM bytes of one chunk call: every tensor once.

    per token per head: q, k (bf16) 2*2*dk + v (bf16) 2*dv + g (fp32) 4*dk + beta 4
    + o (o_bytes per element: 2 counts it as bf16, 1540 B in all for d = 128; the
    call's fp32 o is 4); plus the final state (and the initial state when given).
    """
    per_tok_head = 2 * dk + 2 * dk + 2 * dv + 4 * dk + 4 + o_bytes * dv
    states = N * H * dk * dv * 4 * (2 if h0 else 1)
    return float(T * H * per_tok_head + states)


def prefill_useful_flops(T: int, H: int, dk: int, dv: int, C: int = 64) -> float:
    """The chunk algorithm's useful product flops per call, per token and head
    2 * [3 dk dv + (C / 2) (3 dk + 2 dv)] (the in-chunk triangles counted as half,
    the O(C^2) solve left out), at the 64-token chunk the workload names."""
    return float(T * H * 2 * (3 * dk * dv + (C // 2) * (3 * dk + 2 * dv)))


def gdn_step_bytes(T: int, H: int, dk: int, dv: int, N: int, h0: bool,
                   o_bytes: int = 2) -> float:
    """As prefill_step_bytes with one fp32 decay per (token, head) in place of g."""
    return prefill_step_bytes(T, H, dk, dv, N, h0, o_bytes) - float(T * H * (4 * dk - 4))


def gated_step_bytes(T: int, H: int, dk: int, dv: int, N: int, h0: bool,
                     o_bytes: int = 2) -> float:
    """As prefill_step_bytes with the gate's bf16 pre-activation z (2*dk per token and
    head) in place of the fp32 g; A_log and dt_bias are negligible."""
    return prefill_step_bytes(T, H, dk, dv, N, h0, o_bytes) - float(T * H * 2 * dk)


def decode_conv_step_bytes(B: int, H: int, dk: int, dv: int) -> float:
    """decode_step_bytes with raw q, k, v in place of the processed ones, plus the conv
    caches read and written (3 bf16 tokens per channel) and the conv weights once."""
    C = 2 * dk + dv
    return float(decode_step_bytes(B, H, dk, dv) + B * H * 2 * 3 * C * 2 + H * C * 4 * 2)


def run_decode_conv(torch, kda, workloads, steps=256, warmup=16):
    spec = workloads.standard_specs()["decode"]
    dev = "cuda:0"
    B, H, DK, DV = spec.batch, spec.heads, spec.dk, spec.dv
    state = workloads.make_decode_state(spec, dev)
    cv = workloads.make_decode_conv(spec, dev)
    ins = [workloads.make_decode_conv_step(spec, t, dev) for t in range(steps)]
    o = torch.empty((B, H, DV), dtype=torch.float32, device=dev)

    def call(d, st):
        kda.decode_step_conv(d["q_raw"], d["k_raw"], d["v_raw"], cv["w_q"], cv["w_k"], cv["w_v"],
                             cv["conv_q"], cv["conv_k"], cv["conv_v"], d["g"], d["beta"], st,
                             out=o)

    scratch = state.clone()
    for t in range(warmup):
        call(ins[t % steps], scratch)
    del scratch
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for t in range(steps):
        call(ins[t], state)
    b.record(stream)
    torch.cuda.synchronize()
    return dict(spec=spec, steps=steps, ms=a.elapsed_time(b), B=B, H=H, DK=DK, DV=DV)


def epilogue_bytes(T: int, H: int, dv: int) -> float:
    """Output epilogue: read o (fp32) and the gate (bf16), write y (bf16)."""
    return float(T * H * dv * (4 + 2 + 2))


def run_epilogue(args, torch, kda, workloads, o):
    spec = workloads.standard_specs()[args.workload]
    ep = workloads.make_epilogue(spec, "cuda:0")
    y = torch.empty_like(ep["gate"])
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        kda.output_norm_gate(o, ep["gate"], ep["weight"], out=y)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(args.steps):
        kda.output_norm_gate(o, ep["gate"], ep["weight"], out=y)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / args.steps


def prologue_bytes(T: int, H: int, d: int) -> float:
    """conv4+SiLU(+L2): read x and write y (bf16) for q, k, v; weights are negligible."""
    return float(3 * T * H * d * 2 * 2)


def decode_step_bytes(B: int, H: int, dk: int, dv: int) -> float:
    """State read + write (fp32) plus q, k, v (bf16), g (fp32), beta, o (fp32) per (seq, head)."""
    return float(B * H * (2 * dk * dv * 4 + 2 * dk * 2 + dv * 2 + 4 * dk + 4 + 4 * dv))


def run_prefill(args, torch, kda, workloads, gated=False, gdn=False, workload=None, steps=None,
                overlap=False):
    """Time the prefill step (3 conv calls + the chunk call) on one workload.

    With ``overlap`` (plain g only) the step runs the v conv on a second stream
    beside the q and k convs and the chunk call's prep (kda_chunk_fwd_phases: the
    prep does not read v), and the walk waits for it; the chunk call's own time is
    then not separable, so ``chunk_ms`` is only meaningful without overlap."""
    specs = workloads.standard_specs()
    spec = specs[workload or args.workload]
    nsteps = steps or args.steps
    dev = "cuda:0"
    inp = workloads.make_prefill(spec, dev)
    gate = workloads.make_gate(spec, dev) if gated else None
    ghead = workloads.make_head_gate(spec, dev) if gdn else None
    H, DK, DV = spec.heads, spec.dk, spec.dv
    T, N = spec.total_tokens, len(spec.lengths)
    cu = inp["cu_seqlens"] if N > 1 else None
    qb = torch.empty((T, H, DK), dtype=spec.dtype, device=dev)
    kb = torch.empty_like(qb)
    vb = torch.empty((T, H, DV), dtype=spec.dtype, device=dev)
    ob = torch.empty((T, H, DV), dtype=torch.float32, device=dev)
    hT = torch.empty((N, H, DK, DV), dtype=torch.float32, device=dev)
    ws = torch.empty(kda.chunk_workspace_bytes(T, H, DK, DV, spec.chunk, spec.dtype),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream() if overlap else None
    chunk_kw = dict(cu_seqlens=cu, scale=spec.read_scale, gate_lower_bound=spec.gate_lb,
                    chunk_size=spec.chunk, initial_state=inp["h0"], out=ob, final_state=hT,
                    workspace=ws)

    def step_overlap(ev=None):
        side.wait_stream(stream)          # the previous step's walk reads vb
        with torch.cuda.stream(side):
            kda.short_conv(inp["v_raw"], inp["w_v"], num_heads=H, head_dim=DV, cu_seqlens=cu,
                           out=vb)
            v_done = torch.cuda.Event()
            v_done.record(side)
        kda.short_conv(inp["q_raw"], inp["w_q"], num_heads=H, head_dim=DK, cu_seqlens=cu,
                       l2_normalize=True, out=qb)
        kda.short_conv(inp["k_raw"], inp["w_k"], num_heads=H, head_dim=DK, cu_seqlens=cu,
                       l2_normalize=True, out=kb)
        kda.chunk_fwd(qb, kb, vb, inp["g"], inp["beta"], **chunk_kw, phases=kda.PHASE_PREP)
        stream.wait_event(v_done)
        kda.chunk_fwd(qb, kb, vb, inp["g"], inp["beta"], **chunk_kw, phases=kda.PHASE_WALK)

    def step(ev=None):
        if overlap:
            return step_overlap(ev)
        kda.short_conv(inp["q_raw"], inp["w_q"], num_heads=H, head_dim=DK, cu_seqlens=cu,
                       l2_normalize=True, out=qb)
        kda.short_conv(inp["k_raw"], inp["w_k"], num_heads=H, head_dim=DK, cu_seqlens=cu,
                       l2_normalize=True, out=kb)
        kda.short_conv(inp["v_raw"], inp["w_v"], num_heads=H, head_dim=DV, cu_seqlens=cu, out=vb)
        if ev is not None:
            ev[0].record(stream)
        if ghead is not None:
            kda.gdn_chunk_fwd(qb, kb, vb, ghead, inp["beta"], cu_seqlens=cu,
                              scale=spec.read_scale, gate_lower_bound=spec.gate_lb,
                              chunk_size=spec.chunk, initial_state=inp["h0"], out=ob,
                              final_state=hT, workspace=ws)
        elif gate is None:
            kda.chunk_fwd(qb, kb, vb, inp["g"], inp["beta"], **chunk_kw)
        else:
            kda.chunk_fwd_gated(qb, kb, vb, gate["z"], inp["beta"], a_log=gate["a_log"],
                                dt_bias=gate["dt_bias"], lower_bound=spec.gate_lb, cu_seqlens=cu,
                                scale=spec.read_scale, chunk_size=spec.chunk,
                                initial_state=inp["h0"], out=ob, final_state=hT, workspace=ws)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(nsteps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(nsteps):
        step(events[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    chunk_ms = None if overlap else sum(a.elapsed_time(b) for a, b in events) / nsteps
    ms_step = total_ms / nsteps
    return dict(spec=spec, T=T, N=N, ms_step=ms_step, chunk_ms=chunk_ms, inp=inp, o=ob,
                steps=nsteps)


def run_decode(torch, kda, workloads, steps=256, warmup=16):
    spec = workloads.standard_specs()["decode"]
    dev = "cuda:0"
    B, H, DK, DV = spec.batch, spec.heads, spec.dk, spec.dv
    state = workloads.make_decode_state(spec, dev)
    ins = [workloads.make_decode_step(spec, t, dev) for t in range(steps)]
    o = torch.empty((B, H, DV), dtype=torch.float32, device=dev)
    scratch = state.clone()
    for t in range(warmup):
        d = ins[t % steps]
        kda.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], scratch, out=o)
    del scratch
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for t in range(steps):
        d = ins[t]
        kda.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state, out=o)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b)
    return dict(spec=spec, steps=steps, ms=ms, B=B, H=H, DK=DK, DV=DV)


def cpu_baseline(res, workloads, min_s=10.0, max_passes=20):
    """The oracle (fp64 prologue + recurrence) over the workload's heads (all by default),
    repeated until at least ``min_s`` seconds of wall time have been spent."""
    import numpy as np
    import oracle
    spec, inp = res["spec"], res["inp"]
    H, DK, DV = spec.heads, spec.dk, spec.dv
    n_heads = max(1, min(H, int(os.environ.get("KDA_CPU_SAMPLE_HEADS", str(H)))))
    heads = list(range(n_heads))
    f64 = lambda t: t.detach().double().cpu().numpy()  # noqa: E731

    def chans(x, D):
        return f64(x.view(x.shape[0], H, D)[:, heads, :].reshape(x.shape[0], n_heads * D))

    def wch(w, D):
        return f64(w.view(H, D, -1)[heads].reshape(n_heads * D, -1))

    cu = inp["cu_seqlens"].cpu().numpy()
    xq, xk, xv = chans(inp["q_raw"], DK), chans(inp["k_raw"], DK), chans(inp["v_raw"], DV)
    wq, wk, wv = wch(inp["w_q"], DK), wch(inp["w_k"], DK), wch(inp["w_v"], DV)
    g = f64(inp["g"][:, heads])
    beta = f64(inp["beta"][:, heads])
    h0 = None if inp["h0"] is None else f64(inp["h0"][:, heads])
    oracle.default()
    passes, dt = 0, 0.0
    while passes < max_passes and (passes == 0 or dt < min_s):
        t0 = time.perf_counter()
        q = oracle.prologue(xq, wq, n_heads, DK, cu, normalize=True, out_bf16=True)
        k = oracle.prologue(xk, wk, n_heads, DK, cu, normalize=True, out_bf16=True)
        v = oracle.prologue(xv, wv, n_heads, DV, cu, out_bf16=True)
        oracle.recurrent(q, k, v, g, beta, cu, spec.read_scale, h0)
        dt += time.perf_counter() - t0
        passes += 1
    # tokens/s of the whole workload: each pass covers n_heads of H heads
    value = res["T"] * passes / (dt * H / n_heads)
    return {"value": value, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "%d of %d heads x all %d tokens (fp64 conv+SiLU+L2 prologue and token-by-"
                      "token recurrence), %d passes in %.1f s wall%s" %
                      (n_heads, H, res["T"], passes, dt,
                       "" if n_heads == H else ", scaled by %d/%d" % (H, n_heads))}


def copy_calibration(torch, nbytes=1 << 30, reps=3):
    """A plain copy of known size: every byte read once and written once.  Under a
    counter profiler its FETCH_SIZE / WRITE_SIZE per dispatch, divided by nbytes,
    give the factor that turns those counters into bytes."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "dispatches": reps}))


def timed_copy(torch, nbytes=1 << 30, reps=20):
    """GB/s of a plain device-to-device copy (1 GiB read + 1 GiB written per call),
    timed with HIP events over ``reps`` back-to-back calls after two warm-ups."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, dst
    return {"gbs": round(2 * nbytes / (ms / 1e3) / 1e9, 1), "bytes_per_call": 2 * nbytes,
            "ms_per_call": round(ms, 4), "peak_spec_gbs": HBM_PEAK_GBS,
            "what": "torch copy_ of 1 GiB fp32 (read + write), 20 calls"}


def chunk_roofline(spec, res, kernel, bytes_fn, traffic_kind):
    """Roofline of a chunk call: algorithmic bytes (o counted as bf16) over the call's
    HIP-event time; the same with the fp32 o the call writes; measured traffic."""
    H, DK, DV, T, N = spec.heads, spec.dk, spec.dv, res["T"], res["N"]
    h0 = spec.h0_std is not None
    alg = bytes_fn(T, H, DK, DV, N, h0, 2)
    alg32 = bytes_fn(T, H, DK, DV, N, h0, 4)
    sec = res["chunk_ms"] / 1e3
    ach = alg / sec / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(traffic_kind, spec_key(spec)),
            "kernel": kernel, "algorithmic_bytes_per_launch": alg,
            "bytes_accounting": "q,k,v bf16 + g fp32 + beta + o as bf16 per token-head, + states",
            "frac_fp32_o": round(alg32 / sec / 1e9 / HBM_PEAK_GBS, 4),
            "algorithmic_bytes_fp32_o": alg32,
            "avg_launch_ms": round(res["chunk_ms"], 4)}


def spec_key(spec) -> str:
    return spec.name.split()[0]


def sub_line(args, torch, kda, workloads, name, steps):
    """The prefill step on another workload: tokens/s (the v conv beside the chunk prep,
    as in the main line) and the chunk call's roofline (timed in the one-stream step)."""
    res = run_prefill(args, torch, kda, workloads, workload=name, steps=steps)
    ores = run_prefill(args, torch, kda, workloads, workload=name, steps=steps, overlap=True)
    spec = res["spec"]
    out = {"workload": spec.name, "value": round(res["T"] / (ores["ms_step"] / 1e3), 1),
           "unit": "tokens/s", "tokens": res["T"], "sequences": res["N"],
           "ms_per_step": round(ores["ms_step"], 4),
           "serial_ms_per_step": round(res["ms_step"], 4), "steps": res["steps"],
           "chunk_tokens_per_s": round(res["T"] / (res["chunk_ms"] / 1e3), 1),
           "roofline": chunk_roofline(spec, res, "kda_chunk_fwd (chunk_prep16_kernel + "
                                      "chunk_state_kernel)", prefill_step_bytes, "chunk")}
    del res, ores
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill", choices=["prefill", "varlen", "long"])
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-gate", action="store_true")
    ap.add_argument("--no-epilogue", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-sub", action="store_true",
                    help="skip the varlen and long-context sub-lines")
    ap.add_argument("--no-copy", action="store_true", help="skip the timed 1 GiB copy")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (torch elementwise kernel), the "
                         "reference for scaling HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this build runs on exactly one GPU; --gpus %d is not supported "
              "(no multi-GPU path exists)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import channel_gated_delta_amd as kda
    from channel_gated_delta_amd import workloads
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if not os.path.exists(kda.LIB_PATH):
        from channel_gated_delta_amd import build
        build.build()
    kda.library()
    if args.copy_calibration:
        copy_calibration(torch)
        return

    res = run_prefill(args, torch, kda, workloads)                 # the chunk call's own time
    ores = run_prefill(args, torch, kda, workloads, overlap=True)  # the step as it runs best
    spec = res["spec"]
    H, DK, DV, T, N = spec.heads, spec.dk, spec.dv, res["T"], res["N"]
    tok_s = T / (ores["ms_step"] / 1e3)
    roof = chunk_roofline(spec, res, "kda_chunk_fwd (chunk_prep16_kernel + chunk_state_kernel)",
                          prefill_step_bytes, "chunk")
    useful = prefill_useful_flops(T, H, DK, DV, spec.chunk)
    ut = useful / (res["chunk_ms"] / 1e3) / 1e12
    out = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ores["ms_step"], 4),
        "serial_ms_per_step": round(res["ms_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; no weights or datasets)",
        "config": {"workload": spec.name, "batch": N, "seq_len": T, "heads": H, "dk": DK,
                   "dv": DV, "chunk_requested": spec.chunk, "chunk_internal": 16,
                   "path": "3x short_conv (conv4+SiLU, q/k L2) + chunk_fwd (fp32 o); the v "
                           "conv on a second stream beside the q/k convs and the chunk prep "
                           "(kda_chunk_fwd_phases), the walk after both"},
        "roofline": roof,
        "mfma": {"useful_gflop_per_launch": round(useful / 1e9, 2),
                 "useful_tflops": round(ut, 1), "peak_tflops": 2500.0,
                 "frac_of_bf16_peak": round(ut / 2500.0, 4),
                 "what": "chunk algorithm's product flops (64-token chunk, triangles halved, "
                         "split-bf16 terms not counted) / the call's event time"},
    }
    if not args.no_copy:
        out["hbm_copy"] = timed_copy(torch)
    keep_o = res["o"] if not args.no_epilogue else None
    keep_res = {"spec": spec, "inp": res["inp"], "T": T} if not args.no_cpu else None
    del res
    torch.cuda.empty_cache()
    if not args.no_sub and args.workload == "prefill":
        out["varlen"] = sub_line(args, torch, kda, workloads, "varlen", args.steps)
        out["long"] = sub_line(args, torch, kda, workloads, "long", min(args.steps, 10))
    if not args.no_decode:
        d = run_decode(torch, kda, workloads)
        ms_dec = d["ms"] / d["steps"]
        dbytes = decode_step_bytes(d["B"], d["H"], d["DK"], d["DV"])
        dach = dbytes / (ms_dec / 1e3) / 1e9
        out["decode"] = {"value": round(d["steps"] / (d["ms"] / 1e3), 1), "unit": "steps/s",
                         "workload": d["spec"].name, "ms_per_step": round(ms_dec, 4),
                         "roofline": {"bound": "hbm", "achieved": round(dach, 1),
                                      "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": round(dach / HBM_PEAK_GBS, 4),
                                      "traffic": measured_traffic("decode", "decode"),
                                      "algorithmic_bytes_per_launch": dbytes}}
    if not args.no_decode:
        d = run_decode_conv(torch, kda, workloads)
        ms_dec = d["ms"] / d["steps"]
        dbytes = decode_conv_step_bytes(d["B"], d["H"], d["DK"], d["DV"])
        dach = dbytes / (ms_dec / 1e3) / 1e9
        out["decode_conv"] = {"value": round(d["steps"] / (d["ms"] / 1e3), 1), "unit": "steps/s",
                              "workload": d["spec"].name + ", conv+SiLU+L2 fused",
                              "ms_per_step": round(ms_dec, 4),
                              "roofline": {"bound": "hbm", "achieved": round(dach, 1),
                                           "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                           "frac": round(dach / HBM_PEAK_GBS, 4),
                                           "traffic": measured_traffic("decodeconv", "decode"),
                                           "algorithmic_bytes_per_launch": dbytes}}
    if not args.no_gate:
        gres = run_prefill(args, torch, kda, workloads, gated=True)
        out["fused_gate"] = {
            "value": round(T / (gres["ms_step"] / 1e3), 1), "unit": "tokens/s",
            "ms_per_step": round(gres["ms_step"], 4),
            "path": "3x short_conv + chunk_fwd_gated (g = lb sigmoid(e^A_log (z + dt_bias)) "
                    "in-kernel, z bf16)",
            "roofline": chunk_roofline(spec, gres, "kda_chunk_fwd_gated", gated_step_bytes,
                                       "gated")}
        del gres
    if not args.no_gate:
        hres = run_prefill(args, torch, kda, workloads, gdn=True)
        out["gdn"] = {
            "value": round(T / (hres["ms_step"] / 1e3), 1), "unit": "tokens/s",
            "ms_per_step": round(hres["ms_step"], 4),
            "path": "3x short_conv + gdn_chunk_fwd (one decay per token and head)",
            "roofline": chunk_roofline(spec, hres, "kda_gdn_chunk_fwd", gdn_step_bytes, "gdn")}
        del hres
    if not args.no_epilogue:
        ems = run_epilogue(args, torch, kda, workloads, keep_o)
        ebytes = epilogue_bytes(T, H, DV)
        each = ebytes / (ems / 1e3) / 1e9
        out["output_epilogue"] = {
            "ms_per_call": round(ems, 4),
            "path": "kda_output_norm_gate: y = o / sqrt(mean(o^2) + eps) * w * sigmoid(gate), "
                    "fp32 o, bf16 gate and y",
            "roofline": {"bound": "hbm", "achieved": round(each, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(each / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("epilogue", args.workload),
                         "kernel": "norm_gate_kernel", "algorithmic_bytes_per_launch": ebytes}}
    out["prologue_ms_per_step"] = round(out["serial_ms_per_step"] - roof["avg_launch_ms"], 4)
    out["prologue_bytes_per_step"] = prologue_bytes(T, H, DK)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(keep_res, workloads)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
