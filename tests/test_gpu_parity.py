"""HIP path vs the fp64 oracle, element by element, on seeded inputs (needs an MI355X).

Sizes the oracle finishes in seconds, spanning several 16-token tiles, several
chunks and ragged tails, plus edge cases; the full workload shapes live in
test_gpu_workloads.py.  Bar: max|gpu - oracle| / rms(oracle) <= 2e-2 for bf16
inputs and <= 1e-4 for fp32 inputs (outputs and final states); the prologue is
held to one rounding of its output dtype, element by element.
"""
import numpy as np
import pytest
import torch

import channel_gated_delta_amd as kda
import oracle
from channel_gated_delta_amd import workloads
from gpu_helpers import (assert_parity, check_written, gpu_prefill, note, oracle_prefill, to64,
                         tol_for)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
RAGGED = [1, 3, 15, 17, 63, 65, 130]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kda.library()


def spec_of(lengths, H=3, dk=128, dv=128, chunk=64, dtype=torch.bfloat16, conv=False, lb=-5.0,
            gate_std=1.0, h0=None, seed=0):
    return workloads.PrefillSpec("t", list(lengths), heads=H, dk=dk, dv=dv, chunk=chunk,
                                 dtype=dtype, conv=conv, gate_lb=lb, gate_std=gate_std,
                                 h0_std=h0, seed=seed)


def check_prefill(spec, heads=None, chunk=None):
    inp = workloads.make_prefill(spec, DEV)
    got = gpu_prefill(inp, spec, chunk=chunk)
    check_written(got)
    heads = list(range(spec.heads)) if heads is None else list(heads)
    ref = oracle_prefill(inp, spec, heads)
    tol = tol_for(spec.dtype)
    assert_parity("o", to64(got["o"][:, heads]), ref["o"], tol)
    assert_parity("final state", to64(got["hT"][:, heads]), ref["hT"], tol)
    return inp, got, ref


def test_tiny_fp32_workload():
    """B=1, H=1, T=64, d=16, chunk 16, fp32, q/k unit length, scale 1: tolerance 1e-4."""
    check_prefill(workloads.standard_specs()["tiny_fp32"])


@pytest.mark.parametrize("lengths", [RAGGED, [16, 17, 31, 32, 33, 2, 500]], ids=["a", "b"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_ragged_varlen_with_h0(lengths, dtype):
    note("ragged varlen %s lengths %s" % (dtype, lengths))
    check_prefill(spec_of(lengths, H=2, dtype=dtype, h0=0.05, seed=len(lengths) + sum(lengths)))


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (64, 64), (128, 16), (16, 128)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_head_dims(dk, dv, dtype):
    note("dims dk=%d dv=%d %s" % (dk, dv, dtype))
    check_prefill(spec_of([200, 37], H=3, dk=dk, dv=dv, dtype=dtype, h0=0.1, seed=dk + dv))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_prologue_pipeline_varlen(dtype):
    """conv + SiLU + L2 prologue feeding the chunk kernel, several sequences."""
    check_prefill(spec_of([300, 5, 129, 64], H=4, dtype=dtype, conv=True, h0=0.05, seed=11))


@pytest.mark.parametrize("lb,std", [(-8.0, 2.0), (-9.0, 3.0)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_strong_decay(lb, std, dtype):
    """Gate floors below -5 (16-token decay span down to e^-144): finite and accurate."""
    check_prefill(spec_of([256, 77], H=2, lb=lb, gate_std=std, h0=0.05, seed=int(-lb),
                          dtype=dtype))


@pytest.mark.parametrize("lengths", [[130, 64], [130, 64] * 40], ids=["narrow", "wide"])
def test_bf16_output_is_rounded_fp32_output(lengths):
    """With bf16 inputs, a bf16 o is exactly the fp32 o rounded to nearest even (also
    in the 128-column workgroups: 80 sequences x 2 heads)."""
    spec = spec_of(lengths, H=2, h0=0.05, seed=21)
    inp = workloads.make_prefill(spec, DEV)
    o32, h32 = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                             cu_seqlens=inp["cu_seqlens"], initial_state=inp["h0"])
    o16, h16 = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                             cu_seqlens=inp["cu_seqlens"], initial_state=inp["h0"],
                             out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert o16.dtype == torch.bfloat16
    assert torch.equal(o16, o32.to(torch.bfloat16)) and torch.equal(h16, h32)


def test_identity_gate_keeps_state():
    """g = 0, beta = 0: the final state equals h0 and o = scale * S0^T q."""
    spec = spec_of([96, 40], H=2, h0=0.1, seed=5)
    inp = workloads.make_prefill(spec, DEV)
    inp["g"].zero_()
    inp["beta"].zero_()
    got = gpu_prefill(inp, spec)
    check_written(got)
    assert torch.equal(got["hT"], inp["h0"])
    ref = oracle_prefill(inp, spec, [0, 1])
    assert_parity("o", to64(got["o"]), ref["o"], 2e-2)


def test_empty_and_single_token_sequences():
    spec = spec_of([0, 1, 0, 70, 0], H=2, h0=0.05, seed=6)
    check_prefill(spec)


@pytest.mark.parametrize("nseq", [300, 1100])
def test_many_packed_sequences(nseq):
    """Hundreds of packed sequences with ties and empty ones: 300 are walked longest
    first (the order kernel spans two blocks), 1100 exceed the ordered batches' cap
    and keep their packed order.  Random h0 checks that every sequence's state
    lands in its own slot."""
    rng = np.random.default_rng(nseq)
    lengths = [int(x) for x in rng.integers(0, 40, size=nseq)]
    lengths[nseq // 2] = 200                      # the longest sits in the middle
    note("%d packed sequences, %d tokens" % (nseq, sum(lengths)))
    check_prefill(spec_of(lengths, H=2, h0=0.05, seed=nseq))


WIDE_LENGTHS = [1, 3, 15, 16, 17, 31, 33, 63, 64, 65, 130, 7, 0, 40, 200] * 5   # 75 sequences


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_wide_slices_many_units(dtype):
    """More (sequence, head) units than half the CUs: the state kernel takes all 128
    value columns of a head in one workgroup (8 consumer waves) instead of two
    64-column slices.  Ragged lengths, an empty sequence, h0."""
    assert len(WIDE_LENGTHS) * 2 * 2 > torch.cuda.get_device_properties(0).multi_processor_count
    note("wide slices: %d sequences x 2 heads %s" % (len(WIDE_LENGTHS), dtype))
    check_prefill(spec_of(WIDE_LENGTHS, H=2, dtype=dtype, h0=0.05, seed=75))


@pytest.mark.parametrize("lengths", [[4096], RAGGED], ids=["one", "packed"])
def test_phases_prep_then_walk_bitwise(lengths):
    """kda_chunk_fwd_phases: the prep on one stream, the walk on another after an
    event, gives o and final states bit-identical to the one-call kda_chunk_fwd;
    the prep alone writes neither o nor the final state (both stay NaN)."""
    spec = spec_of(lengths, H=3, h0=0.05, seed=len(lengths))
    inp = workloads.make_prefill(spec, DEV)
    ref = gpu_prefill(inp, spec)
    check_written(ref)
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    kw = dict(cu_seqlens=inp["cu_seqlens"], scale=spec.read_scale, initial_state=inp["h0"])
    T, H = spec.total_tokens, spec.heads
    ws = torch.full((kda.chunk_workspace_bytes(T, H, 128, 128, 64, torch.bfloat16,
                                               torch.float32),), 0xFF, dtype=torch.uint8,
                    device=DEV)
    o = torch.full((T, H, 128), float("nan"), device=DEV)
    hT = torch.full((len(lengths), H, 128, 128), float("nan"), device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        kda.chunk_fwd(*args, **kw, out=o, final_state=hT, workspace=ws, phases=kda.PHASE_PREP)
        done = torch.cuda.Event()
        done.record(side)
    torch.cuda.synchronize()
    assert bool(torch.isnan(o).all()) and bool(torch.isnan(hT).all())
    torch.cuda.current_stream().wait_event(done)
    kda.chunk_fwd(*args, **kw, out=o, final_state=hT, workspace=ws, phases=kda.PHASE_WALK)
    torch.cuda.synchronize()
    assert torch.equal(o, ref["o"]) and torch.equal(hT, ref["hT"])


def test_zero_tokens():
    spec = spec_of([0], H=2, h0=0.05, seed=7)
    inp = workloads.make_prefill(spec, DEV)
    got = gpu_prefill(inp, spec)
    check_written(got)
    assert got["o"].numel() == 0
    assert torch.equal(got["hT"], inp["h0"])


def test_repeat_calls_bitwise_identical():
    """Two calls on the same inputs give bit-identical o and final states: the kernels
    use no atomics and a fixed summation order.  The second call asks for 16-token
    chunks instead of 64: the kernels walk 16-token chunks for every requested size,
    so the request does not change the computation.  Both calls start from NaN-filled
    outputs and workspace, so a row one call left unwritten cannot pass."""
    spec = spec_of([333, 64, 1], H=3, h0=0.05, seed=8)
    inp = workloads.make_prefill(spec, DEV)
    a = gpu_prefill(inp, spec, chunk=64)
    check_written(a)
    b = gpu_prefill(inp, spec, chunk=16)
    check_written(b)
    assert torch.equal(a["o"], b["o"]) and torch.equal(a["hT"], b["hT"])


def test_final_state_in_place():
    """final_state may alias initial_state."""
    spec = spec_of([150], H=2, h0=0.05, seed=9)
    inp = workloads.make_prefill(spec, DEV)
    ref = gpu_prefill(inp, spec)
    check_written(ref)
    st = inp["h0"].clone()
    o, _ = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                         cu_seqlens=inp["cu_seqlens"], scale=spec.read_scale, initial_state=st,
                         final_state=st)
    torch.cuda.synchronize()
    assert torch.equal(st, ref["hT"]) and torch.equal(o, ref["o"])


# ------------------------------------------------------------------ fused bounded gate

def check_gated(spec, params=True, heads=None):
    inp = workloads.make_prefill(spec, DEV)
    gate = workloads.make_gate(spec, DEV)
    if not params:
        gate = dict(z=gate["z"], a_log=None, dt_bias=None)
    got = gpu_prefill(inp, spec, gate=gate)
    check_written(got)
    heads = list(range(spec.heads)) if heads is None else list(heads)
    ref = oracle_prefill(inp, spec, heads, gate=gate)
    tol = tol_for(spec.dtype)
    assert_parity("o (fused gate)", to64(got["o"][:, heads]), ref["o"], tol)
    assert_parity("final state (fused gate)", to64(got["hT"][:, heads]), ref["hT"], tol)
    return inp, gate, got


@pytest.mark.parametrize("params", [True, False], ids=["alog_dt", "z_only"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_gated_ragged_varlen(params, dtype):
    """g = lb sigmoid(e^{A_log} (z + dt_bias)) formed in the kernels, ragged packed batch, h0."""
    note("fused gate %s params=%s" % (dtype, params))
    check_gated(spec_of(RAGGED, H=2, dtype=dtype, h0=0.05, seed=31), params=params)


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 16)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_gated_head_dims(dk, dv, dtype):
    note("fused gate dims dk=%d dv=%d %s" % (dk, dv, dtype))
    check_gated(spec_of([200, 37], H=3, dk=dk, dv=dv, dtype=dtype, h0=0.1, seed=dk + 2 * dv))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_gated_strong_decay_and_prologue(dtype):
    """Gate floor -8 with a wide pre-activation, behind the conv + SiLU + L2 prologue."""
    check_gated(spec_of([300, 5, 129], H=2, dtype=dtype, conv=True, lb=-8.0, gate_std=2.0,
                        h0=0.05, seed=33))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_gated_wide_slices(dtype):
    """The fused gate in the 128-column workgroups (many units)."""
    check_gated(spec_of(WIDE_LENGTHS, H=2, dtype=dtype, h0=0.05, seed=76))


def test_gated_matches_plain_gate():
    """The fused path equals chunk_fwd fed with the same gate precomputed (fp32)."""
    spec = spec_of([150, 66], H=2, h0=0.05, seed=34)
    inp, gate, got = check_gated(spec)
    g = oracle.bounded_gate(to64(gate["z"]), to64(gate["a_log"]), to64(gate["dt_bias"]),
                            spec.gate_lb)
    inp["g"] = torch.from_numpy(g).float().to(DEV)
    plain = gpu_prefill(inp, spec)
    check_written(plain)
    assert_parity("o fused vs plain", to64(got["o"]), to64(plain["o"]), 1e-3)
    assert_parity("state fused vs plain", to64(got["hT"]), to64(plain["hT"]), 1e-3)


# ------------------------------------------------------------------ GDN: one decay per head

def check_gdn(spec):
    inp = workloads.make_prefill(spec, DEV)
    gh = workloads.make_head_gate(spec, DEV)
    T, H, DK = spec.total_tokens, spec.heads, spec.dk
    o, hT = kda.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], gh, inp["beta"],
                              cu_seqlens=inp["cu_seqlens"], scale=spec.read_scale,
                              gate_lower_bound=spec.gate_lb, chunk_size=spec.chunk,
                              initial_state=inp["h0"])
    torch.cuda.synchronize()
    # the oracle's recurrence with the head's decay on every key channel
    g = np.repeat(to64(gh)[:, :, None], DK, axis=2)
    h0 = None if inp["h0"] is None else to64(inp["h0"])
    ro, rh = oracle.recurrent(to64(inp["q"]), to64(inp["k"]), to64(inp["v"]), g,
                              to64(inp["beta"]), inp["cu_seqlens"].cpu().numpy(), spec.read_scale,
                              h0)
    tol = tol_for(spec.dtype)
    assert_parity("o (GDN)", to64(o), ro, tol)
    assert_parity("final state (GDN)", to64(hT), rh, tol)


@pytest.mark.parametrize("dk,dv", [(128, 128), (16, 16), (32, 64), (128, 16)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_gdn_chunk(dk, dv, dtype):
    note("GDN chunk dk=%d dv=%d %s" % (dk, dv, dtype))
    check_gdn(spec_of(RAGGED, H=2, dk=dk, dv=dv, dtype=dtype, h0=0.05, seed=41 + dk))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_gdn_strong_decay(dtype):
    check_gdn(spec_of([300, 41], H=3, dtype=dtype, lb=-8.0, gate_std=2.0, h0=0.05, seed=43))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_gdn_wide_slices(dtype):
    """One decay per (token, head) in the 128-column workgroups (many units)."""
    check_gdn(spec_of(WIDE_LENGTHS, H=2, dtype=dtype, h0=0.05, seed=77))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_gdn_decode(dtype):
    """GDN decode steps against the oracle's recurrence with the decay broadcast."""
    B, H, dk, dv, steps = 3, 2, 128, 64, 6
    spec = workloads.DecodeSpec("t", batch=B, heads=H, dk=dk, dv=dv, steps=steps, dtype=dtype,
                                seed=44)
    state = workloads.make_decode_state(spec, DEV)
    s0 = to64(state)
    ins, outs = [], []
    for t in range(steps):
        d = workloads.make_decode_step(spec, t, DEV)
        d["g"] = d["g"][:, :, 0].contiguous()       # one decay per (sequence, head)
        outs.append(kda.gdn_decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state))
        ins.append(d)
    torch.cuda.synchronize()

    def packed(key):
        x = torch.stack([i[key] for i in ins], dim=1)
        return to64(x.reshape(B * steps, *x.shape[2:]))

    g = np.repeat(packed("g")[:, :, None], dk, axis=2)
    cu = np.arange(B + 1) * steps
    o, hT = oracle.recurrent(packed("q"), packed("k"), packed("v"), g, packed("beta"), cu,
                             dk ** -0.5, s0)
    tol = tol_for(dtype)
    assert_parity("GDN decode o", to64(torch.stack(outs, dim=1).reshape(B * steps, H, dv)), o, tol)
    assert_parity("GDN decode state", to64(state), hT, tol)


# ------------------------------------------------------------------ decode with the conv

def decode_conv_case(B, H, dk, dv, steps, dtype, seed):
    """`steps` fused steps against the oracle's prefill of the same tokens: the B
    sequences packed, the initial conv caches as their conv history, the initial
    states as h0 (q, k, v not rounded in between on either side)."""
    spec = workloads.DecodeSpec("t", batch=B, heads=H, dk=dk, dv=dv, steps=steps, dtype=dtype,
                                seed=seed)
    state = workloads.make_decode_state(spec, DEV)
    cv = workloads.make_decode_conv(spec, DEV)
    s0 = state.clone()
    c0 = {n: cv["conv_" + n].clone() for n in "qkv"}
    ins, outs = [], []
    for t in range(steps):
        d = workloads.make_decode_conv_step(spec, t, DEV)
        outs.append(kda.decode_step_conv(d["q_raw"], d["k_raw"], d["v_raw"], cv["w_q"], cv["w_k"],
                                         cv["w_v"], cv["conv_q"], cv["conv_k"], cv["conv_v"],
                                         d["g"], d["beta"], state, scale=dk ** -0.5))
        ins.append(d)
    torch.cuda.synchronize()

    def packed(key):   # per-step [B, ...] -> sequence-major [B * steps, ...]
        x = torch.stack([i[key] for i in ins], dim=1)
        return to64(x.reshape(B * steps, *x.shape[2:]))

    cu = np.arange(B + 1) * steps
    q = oracle.prologue(packed("q_raw"), to64(cv["w_q"]), H, dk, cu, state_in=to64(c0["q"]),
                        normalize=True)
    k = oracle.prologue(packed("k_raw"), to64(cv["w_k"]), H, dk, cu, state_in=to64(c0["k"]),
                        normalize=True)
    v = oracle.prologue(packed("v_raw"), to64(cv["w_v"]), H, dv, cu, state_in=to64(c0["v"]))
    o, hT = oracle.recurrent(q, k, v, packed("g"), packed("beta"), cu, dk ** -0.5, to64(s0))
    tol = tol_for(dtype)
    assert_parity("decode+conv o", to64(torch.stack(outs, dim=1).reshape(B * steps, H, dv)), o,
                  tol)
    assert_parity("decode+conv state", to64(state), hT, tol)
    for n in "qkv":   # the caches end with the last three raw inputs, exactly
        hist = torch.cat([c0[n], torch.stack([i[n + "_raw"] for i in ins], dim=1)], dim=1)[:, -3:]
        assert torch.equal(cv["conv_" + n], hist), "conv cache " + n
    return cv, state


@pytest.mark.parametrize("dk,dv", [(128, 128), (16, 16), (32, 128), (128, 16), (64, 32)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_decode_conv(dk, dv, dtype):
    note("decode+conv dk=%d dv=%d %s" % (dk, dv, dtype))
    decode_conv_case(3, 2, dk, dv, 6, dtype, seed=dk + 3 * dv)


def test_decode_conv_caches_match_short_conv():
    """The fused step leaves exactly the conv caches kda_short_conv leaves for one token
    per sequence.  (o and the state are checked against the oracle elsewhere: the
    unfused pair rounds q, k, v to bf16 in between, which moves a single step's state
    by ~2^-9 of its update -- about 9% of the state's rms for these inputs.)"""
    B, H, dk, dv = 4, 3, 128, 64
    spec = workloads.DecodeSpec("t", batch=B, heads=H, dk=dk, dv=dv, steps=1, seed=71)
    cv = workloads.make_decode_conv(spec, DEV)
    d = workloads.make_decode_conv_step(spec, 0, DEV)
    st1 = workloads.make_decode_state(spec, DEV)
    st2 = st1.clone()
    caches = {n: cv["conv_" + n].clone() for n in "qkv"}
    o1 = kda.decode_step_conv(d["q_raw"], d["k_raw"], d["v_raw"], cv["w_q"], cv["w_k"], cv["w_v"],
                              cv["conv_q"], cv["conv_k"], cv["conv_v"], d["g"], d["beta"], st1)
    cu = torch.arange(B + 1, dtype=torch.int32, device=DEV)
    x = {}
    for n, D in (("q", dk), ("k", dk), ("v", dv)):
        x[n], caches[n] = kda.short_conv(d[n + "_raw"], cv["w_" + n], num_heads=H, head_dim=D,
                                         cu_seqlens=cu, conv_state=caches[n],
                                         output_final_state=True, l2_normalize=(n != "v"))
    o2 = kda.decode_step(x["q"], x["k"], x["v"], d["g"], d["beta"], st2)
    torch.cuda.synchronize()
    for n in "qkv":
        assert torch.equal(cv["conv_" + n], caches[n]), "conv cache " + n
    assert bool(torch.isfinite(o1).all()) and bool(torch.isfinite(o2).all())


# ------------------------------------------------------------------ output epilogue

def check_norm_gate(o, gate, w, eps):
    y = kda.output_norm_gate(o, gate, w, eps=eps)
    torch.cuda.synchronize()
    ref = oracle.output_norm_gate(to64(o), to64(gate), None if w is None else to64(w), eps)
    got = to64(y)
    if y.dtype == torch.bfloat16:
        # one rounding to bf16 (2^-9 relative) on top of fp32 arithmetic
        bound = 2.0 ** -8 * np.abs(ref) + 1e-6 * float(np.sqrt(np.mean(ref * ref)))
    else:
        bound = 1e-5 * np.abs(ref) + 1e-6 * float(np.sqrt(np.mean(ref * ref)))
    excess = np.abs(got - ref) - bound
    assert np.all(excess <= 0), "max excess %.3e" % float(np.max(excess))
    return y


@pytest.mark.parametrize("dv", [16, 32, 64, 128])
@pytest.mark.parametrize("odt,dt", [(torch.float32, torch.bfloat16), (torch.bfloat16, torch.bfloat16),
                                    (torch.float32, torch.float32)], ids=["f32o_bf16", "bf16", "fp32"])
def test_output_norm_gate(dv, odt, dt):
    """Per-head RMSNorm * sigmoid gate, element by element against the oracle; ragged
    row count, rows of very different scale, with and without the weight."""
    note("output_norm_gate dv=%d o=%s y=%s" % (dv, odt, dt))
    g = torch.Generator(device=DEV).manual_seed(50 + dv)
    T, H = 37, 3
    scale = torch.tensor([1e-3, 1.0, 30.0], device=DEV).view(1, H, 1)
    o = (torch.randn(T, H, dv, generator=g, device=DEV) * scale).to(odt)
    gate = (2.0 * torch.randn(T, H, dv, generator=g, device=DEV)).to(dt)
    w = 1.0 + 0.5 * torch.randn(dv, generator=g, device=DEV)
    check_norm_gate(o, gate, w, 1e-6)
    check_norm_gate(o, gate, None, 0.0)


def test_output_norm_gate_in_place_and_empty():
    g = torch.Generator(device=DEV).manual_seed(60)
    o = torch.randn(130, 96, 128, generator=g, device=DEV)
    gate = torch.randn(130, 96, 128, generator=g, device=DEV).bfloat16()
    w = torch.rand(128, generator=g, device=DEV) + 0.5
    ref = kda.output_norm_gate(o, gate, w)
    kda.output_norm_gate(o, gate, w, out=gate)          # y takes the gate's place
    torch.cuda.synchronize()
    assert torch.equal(gate, ref)
    e = torch.empty(0, 4, 64, device=DEV)
    assert kda.output_norm_gate(e, e.bfloat16()).numel() == 0


# ------------------------------------------------------------------ prologue alone

@pytest.mark.parametrize("width", [1, 2, 3, 4])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_short_conv_varlen_state(width, dtype):
    """conv with bias, history in/out, sequence resets, L2 on and off."""
    note("short_conv width=%d %s" % (width, dtype))
    g = torch.Generator(device=DEV).manual_seed(100 + width)
    lengths = [1, 2, 19, 40, 0, 7]
    cu = torch.tensor(np.cumsum([0] + lengths), dtype=torch.int32, device=DEV)
    T, H, D, N = sum(lengths), 3, 64, len(lengths)
    x = torch.randn(T, H * D, generator=g, device=DEV).to(dtype)
    w = (0.5 * torch.randn(H * D, width, generator=g, device=DEV)).to(dtype)
    b = (0.1 * torch.randn(H * D, generator=g, device=DEV)).to(dtype)
    st = torch.randn(N, width - 1, H * D, generator=g, device=DEV).to(dtype)
    eps = 2.0 ** -8 if dtype == torch.bfloat16 else 1e-5
    for l2 in (False, True):
        y, st_out = kda.short_conv(x, w, num_heads=H, head_dim=D, cu_seqlens=cu, bias=b,
                                   conv_state=st, output_final_state=True, l2_normalize=l2)
        torch.cuda.synchronize()
        ry, rst = oracle.short_conv(to64(x), to64(w), cu.cpu().numpy(), to64(st), to64(b),
                                    silu=True, return_state=True)
        if l2:
            ry = oracle.l2norm(ry, D, 1e-6)
        ry = ry.reshape(T, H, D)
        gy = to64(y)
        if dtype == torch.bfloat16:
            # bf16 outputs are the correctly rounded values: identical to the oracle's rounding
            rb = oracle.round_bf16(ry)
            assert np.array_equal(gy, rb), "%d values differ" % int(np.sum(gy != rb))
        else:
            bound = eps * np.abs(ry) + 1e-6
            assert np.all(np.abs(gy - ry) <= bound), \
                "max excess %.3e" % np.max(np.abs(gy - ry) - bound)
        assert np.array_equal(to64(st_out), rst), "conv history out"
    # in-place history update (state_out aliases conv_state)
    st2 = st.clone()
    kda.short_conv(x, w, num_heads=H, head_dim=D, cu_seqlens=cu, bias=b, conv_state=st2,
                   state_out=st2, l2_normalize=True)
    torch.cuda.synchronize()
    assert torch.equal(st2, st_out)


def test_short_conv_split_resume():
    """Two calls carrying the conv history equal one call (bf16, width 4, L2)."""
    g = torch.Generator(device=DEV).manual_seed(7)
    T, H, D = 50, 2, 128
    x = torch.randn(T, H * D, generator=g, device=DEV).bfloat16()
    w = (0.5 * torch.randn(H * D, 4, generator=g, device=DEV)).bfloat16()
    full, _ = kda.short_conv(x, w, num_heads=H, head_dim=D, l2_normalize=True)
    for cut in (1, 2, 3, 17):
        y1, st = kda.short_conv(x[:cut].contiguous(), w, num_heads=H, head_dim=D,
                                l2_normalize=True, output_final_state=True)
        y2, _ = kda.short_conv(x[cut:].contiguous(), w, num_heads=H, head_dim=D, l2_normalize=True,
                               conv_state=st)
        torch.cuda.synchronize()
        assert torch.equal(torch.cat([y1, y2]), full), "resume at %d" % cut


# ------------------------------------------------------------------ decode

def decode_case(B, H, dk, dv, steps, dtype, seed, pairs=None):
    spec = workloads.DecodeSpec("t", batch=B, heads=H, dk=dk, dv=dv, steps=steps, dtype=dtype,
                                seed=seed)
    state = workloads.make_decode_state(spec, DEV)
    s0 = state.clone()
    outs, ins = [], []
    for t in range(steps):
        inp = workloads.make_decode_step(spec, t, DEV)
        outs.append(kda.decode_step(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], state,
                                    scale=dk ** -0.5))
        ins.append(inp)
    torch.cuda.synchronize()
    pairs = [(b, h) for b in range(B) for h in range(H)] if pairs is None else pairs
    P = len(pairs)
    bi = torch.tensor([p[0] for p in pairs], device=DEV)
    hi = torch.tensor([p[1] for p in pairs], device=DEV)

    def seq(key):  # [steps, B, H, ...] -> packed [P*steps, 1, ...] (pair-major)
        x = torch.stack([i[key][bi, hi] for i in ins], dim=1)  # [P, steps, ...]
        return to64(x.reshape(P * steps, 1, *x.shape[2:]))

    cu = np.arange(P + 1) * steps
    o, hT = oracle.recurrent(seq("q"), seq("k"), seq("v"), seq("g"),
                             seq("beta").reshape(P * steps, 1), cu_seqlens=cu, scale=dk ** -0.5,
                             h0=to64(s0[bi, hi]).reshape(P, 1, dk, dv))
    got_o = torch.stack([x[bi, hi] for x in outs], dim=1).reshape(P * steps, 1, dv)
    tol = 2e-2 if dtype == torch.bfloat16 else 1e-4
    assert_parity("decode o", to64(got_o), o, tol)
    if dtype == torch.bfloat16:   # a bf16 o is the fp32 o rounded once
        st2 = s0.clone()
        for t in range(steps):
            d = ins[t]
            o16 = kda.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], st2,
                                  scale=dk ** -0.5, out_dtype=torch.bfloat16)
            assert torch.equal(o16, outs[t].to(torch.bfloat16))
        assert torch.equal(st2, state)
    assert_parity("decode state", to64(state[bi, hi]).reshape(P, 1, dk, dv), hT, tol)
    return state


@pytest.mark.parametrize("dk,dv", [(128, 128), (16, 16), (32, 128), (128, 16), (64, 64), (16, 32)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_decode_small(dk, dv, dtype):
    note("decode dk=%d dv=%d %s" % (dk, dv, dtype))
    decode_case(2, 4, dk, dv, 8, dtype, seed=dk * 3 + dv)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_decode_matches_chunk(dtype):
    """T decode steps equal one chunk_fwd call over the same T tokens."""
    spec = spec_of([77], H=2, dtype=dtype, h0=0.05, seed=12)
    inp = workloads.make_prefill(spec, DEV)
    got = gpu_prefill(inp, spec)
    check_written(got)
    state = inp["h0"].clone()
    os_ = []
    for t in range(77):
        os_.append(kda.decode_step(inp["q"][t:t + 1].contiguous(), inp["k"][t:t + 1].contiguous(),
                                   inp["v"][t:t + 1].contiguous(), inp["g"][t:t + 1].contiguous(),
                                   inp["beta"][t:t + 1].contiguous(), state,
                                   scale=spec.read_scale))
    torch.cuda.synchronize()
    tol = 2e-2 if dtype == torch.bfloat16 else 1e-4
    assert_parity("o decode vs chunk", to64(torch.cat(os_)), to64(got["o"]), tol)
    assert_parity("state decode vs chunk", to64(state), to64(got["hT"]), tol)
