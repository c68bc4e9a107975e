"""Pins of the fp64 oracle to what the pages and the mathematics fix.

Each ``pin_*`` takes an ``oracle.OracleLib`` and raises AssertionError when the
build disagrees with a worked example printed on the pages (fixtures under
tests/golden/, each citing its page and section), a closed form, an invariant,
a textbook/library special case, or brute-force agreement with the independently
derived chunkwise form.  test_oracle_pins.py runs them on the real oracle;
test_oracle_mutants.py runs them on deliberately broken builds and requires that
every plausible mistake trips at least one pin.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

from oracle import chunked

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _close(a, b, tol=1e-12, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * scale, "%s: max|diff| = %.3e (tol %.1e)" % (what, err, tol * scale)


def _unit(x, axis=-1):
    return x / np.linalg.norm(x, axis=axis, keepdims=True)


def _rand_inputs(rng, T, H, DK, DV, gate_lb=-5.0, unit=True):
    q = rng.standard_normal((T, H, DK))
    k = rng.standard_normal((T, H, DK))
    if unit:
        q, k = _unit(q), _unit(k)
    v = rng.standard_normal((T, H, DV))
    g = gate_lb / (1.0 + np.exp(-rng.standard_normal((T, H, DK))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    return q, k, v, g, beta


# ---------------------------------------------------------------- worked examples

def pin_unit_key_example(orc):
    """Walkthrough, 第四站: old read-out 10, target 14, beta 0.5 -> 12, 13, 13.5."""
    gd = golden("unit_key_correction.json")
    steps = len(gd["readouts_after_each_write"])
    DK, DV = 3, 2
    rng = np.random.default_rng(11)
    S0 = rng.standard_normal((1, 1, DK, DV))
    S0[0, 0, 1, 0] = gd["old_readout"]
    k = np.zeros((steps, 1, DK))
    k[:, 0, 1] = 1.0                                   # one fixed unit key e_1
    q = k.copy()                                       # read along the same direction
    v = np.zeros((steps, 1, DV))
    v[:, 0, 0] = gd["target_value"]
    v[:, 0, 1] = S0[0, 0, 1, 1]                        # second column already correct
    g = np.zeros((steps, 1, DK))                       # decay off
    beta = np.full((steps, 1), gd["beta"])
    o, hT = orc.recurrent(q, k, v, g, beta, h0=S0)
    _close(o[:, 0, 0], gd["readouts_after_each_write"], what="unit-key read-outs")
    _close(o[:, 0, 1], np.full(steps, S0[0, 0, 1, 1]), what="already-correct column")
    # rows of S that the key does not address are untouched
    _close(hT[0, 0, [0, 2]], S0[0, 0, [0, 2]], what="unaddressed rows")
    # closed form of repeated writes: 14 - 4 * 0.5^n
    n = np.arange(1, steps + 1)
    _close(o[:, 0, 0], 14.0 - 4.0 * 0.5 ** n, what="closed form")


def pin_one_dim_example(orc):
    """Workshop-16, 8.4: 0.7 towards 0.9 with beta 0.5 gives 0.8."""
    gd = golden("one_dim_correction.json")
    one = np.ones((1, 1, 1))
    o, hT = orc.recurrent(one, one, np.full((1, 1, 1), gd["target_value"]), np.zeros((1, 1, 1)),
                          np.full((1, 1), gd["beta"]), h0=np.full((1, 1, 1, 1), gd["old_readout"]))
    _close(o.ravel(), [gd["readout_after_write"]], what="1-D correction")
    _close(hT.ravel(), [gd["readout_after_write"]], what="1-D state")


def pin_two_address_example(orc):
    """Workshop-16, 5.1: one-hot keys address rows; a one-hot query reads its row back."""
    gd = golden("two_address.json")
    keys = np.array(gd["keys"])
    vals = np.array(gd["values"])
    T, DK, DV = keys.shape[0] + 1, keys.shape[1], vals.shape[1]
    k = np.zeros((T, 1, DK))
    v = np.zeros((T, 1, DV))
    k[:2, 0] = keys
    v[:2, 0] = vals
    q = np.zeros((T, 1, DK))
    q[2, 0] = gd["query"]
    g = np.zeros((T, 1, DK))
    beta = np.ones((T, 1))
    beta[2] = 0.0                                       # third step only reads
    for delta in (True, False):
        o, hT = orc.recurrent(q, k, v, g, beta, delta_rule=delta)
        _close(hT[0, 0], gd["expected_state_rows"], what="state rows (delta=%s)" % delta)
        _close(o[2, 0], gd["expected_readout"], what="read-out (delta=%s)" % delta)


# ---------------------------------------------------------------- closed forms

def pin_update_order(orc):
    """Walkthrough, 第三站/第四站: forget first, then predict from the decayed state.

    S0 = 10 along a unit key, alpha = 0.5, v = 14, beta = 0.5:
    decayed 5, prediction 5, error 9, new state 5 + 4.5 = 9.5.  (Predicting from
    the undecayed state would give 5 + 0.5 * (14 - 10) = 7.)
    """
    one = np.ones((1, 1, 1))
    o, hT = orc.recurrent(one, one, np.full((1, 1, 1), 14.0), np.full((1, 1, 1), math.log(0.5)),
                          np.full((1, 1), 0.5), h0=np.full((1, 1, 1, 1), 10.0))
    _close(hT.ravel(), [9.5], what="decay-then-correct state")
    _close(o.ravel(), [9.5], what="read-out after write")


def pin_identity(orc):
    """alpha = 1 and beta = 0 leave S unchanged; o_t = scale * S0^T q_t."""
    rng = np.random.default_rng(1)
    T, H, DK, DV = 9, 2, 5, 3
    q, k, v, _, _ = _rand_inputs(rng, T, H, DK, DV)
    S0 = rng.standard_normal((1, H, DK, DV))
    o, hT = orc.recurrent(q, k, v, np.zeros((T, H, DK)), np.zeros((T, H)), scale=0.7, h0=S0)
    _close(hT, S0, what="identity state")
    for h in range(H):
        _close(o[:, h], 0.7 * q[:, h] @ S0[0, h], what="identity read-out")


def pin_pure_decay(orc):
    """beta = 0: S_t = diag(exp(sum_{j<=t} g_j)) S0 (rows = key channels)."""
    rng = np.random.default_rng(2)
    T, H, DK, DV = 7, 2, 4, 4
    q, k, v, g, _ = _rand_inputs(rng, T, H, DK, DV)
    S0 = rng.standard_normal((1, H, DK, DV))
    o, hT = orc.recurrent(q, k, v, g, np.zeros((T, H)), h0=S0)
    G = np.cumsum(g, axis=0)
    for h in range(H):
        _close(hT[0, h], np.exp(G[-1, h])[:, None] * S0[0, h], what="decayed state")
        for t in range(T):
            _close(o[t, h], (np.exp(G[t, h])[:, None] * S0[0, h]).T @ q[t, h], what="decayed read")


def pin_overwrite(orc):
    """beta = 1, unit key, no decay: after the write the key reads back exactly v_t."""
    rng = np.random.default_rng(3)
    T, H, DK, DV = 12, 1, 6, 3
    _, k, v, _, _ = _rand_inputs(rng, T, H, DK, DV)
    S0 = rng.standard_normal((1, H, DK, DV))
    o, _ = orc.recurrent(k, k, v, np.zeros((T, H, DK)), np.ones((T, H)), h0=S0)
    _close(o, v, tol=1e-11, what="overwrite read-back")


def pin_linear_attention(orc):
    """Without the correction, alpha = 1, beta = 1, S0 = 0: O = scale * tril(Q K^T) V.

    Workshop-16, section 4: additive state S_t = S_{t-1} + k v^T read by q.
    """
    rng = np.random.default_rng(4)
    T, H, DK, DV = 11, 2, 4, 5
    q, k, v, _, _ = _rand_inputs(rng, T, H, DK, DV, unit=False)
    o, hT = orc.recurrent(q, k, v, np.zeros((T, H, DK)), np.ones((T, H)), scale=0.5,
                          delta_rule=False)
    for h in range(H):
        _close(o[:, h], 0.5 * np.tril(q[:, h] @ k[:, h].T) @ v[:, h], what="linear attention")
        _close(hT[0, h], k[:, h].T @ v[:, h], what="linear attention state")


def pin_gated_form(orc):
    """Without the correction: o_t = scale sum_{i<=t} beta_i ((q_t*exp(G_t-G_i)) . k_i) v_i.

    Workshop-16, section 7: S_t = A_t S_{t-1} + beta_t k_t v_t^T with a diagonal A_t.
    """
    rng = np.random.default_rng(5)
    T, H, DK, DV = 10, 1, 3, 2
    q, k, v, g, beta = _rand_inputs(rng, T, H, DK, DV)
    S0 = rng.standard_normal((1, H, DK, DV))
    o, hT = orc.recurrent(q, k, v, g, beta, scale=1.3, h0=S0, delta_rule=False)
    G = np.cumsum(g[:, 0], axis=0)
    for t in range(T):
        acc = (np.exp(G[t])[:, None] * S0[0, 0]).T @ q[t, 0]
        for i in range(t + 1):
            acc = acc + beta[i, 0] * np.dot(q[t, 0] * np.exp(G[t] - G[i]), k[i, 0]) * v[i, 0]
        _close(o[t, 0], 1.3 * acc, what="gated form t=%d" % t)
    S = np.exp(G[-1])[:, None] * S0[0, 0]
    for i in range(T):
        S = S + beta[i, 0] * np.outer(k[i, 0] * np.exp(G[-1] - G[i]), v[i, 0])
    _close(hT[0, 0], S, what="gated form state")


# ---------------------------------------------------------------- brute force

def pin_chunked_matches_recurrent(orc):
    """The independently derived chunkwise form equals the recurrence (fp64)."""
    rng = np.random.default_rng(6)
    lengths = [37, 5, 64, 1]
    T, H, DK, DV = sum(lengths), 2, 6, 4
    cu = np.cumsum([0] + lengths)
    q, k, v, g, beta = _rand_inputs(rng, T, H, DK, DV)
    h0 = rng.standard_normal((len(lengths), H, DK, DV)) * 0.3
    for use_h0 in (False, True):
        ro, rh = orc.recurrent(q, k, v, g, beta, cu_seqlens=cu, scale=0.6,
                               h0=h0 if use_h0 else None)
        for C in (1, 7, 16, 64):
            co, ch = chunked.chunked_forward(q, k, v, g, beta, cu, 0.6, h0 if use_h0 else None, C)
            _close(co, ro, tol=1e-11, what="chunked o (C=%d, h0=%s)" % (C, use_h0))
            _close(ch, rh, tol=1e-11, what="chunked state (C=%d, h0=%s)" % (C, use_h0))


def pin_causality(orc):
    """Changing token t' changes nothing before t' (conv and recurrence are causal)."""
    rng = np.random.default_rng(7)
    T, H, D = 20, 1, 4
    x = rng.standard_normal((T, H * D))
    w = rng.standard_normal((H * D, 4))
    q, k, v, g, beta = _rand_inputs(rng, T, H, D, D)
    tp = 9
    y0 = orc.short_conv(x, w)
    x2 = x.copy()
    x2[tp] += 1.0
    y1 = orc.short_conv(x2, w)
    assert np.array_equal(y0[:tp], y1[:tp]), "conv looks ahead"
    assert not np.allclose(y0[tp], y1[tp]), "conv ignores the current token"
    o0, _ = orc.recurrent(q, k, v, g, beta)
    k2, v2 = k.copy(), v.copy()
    k2[tp] = _unit(k2[tp] + 0.5)
    v2[tp] += 1.0
    o1, _ = orc.recurrent(q, k2, v2, g, beta)
    assert np.array_equal(o0[:tp], o1[:tp]), "recurrence looks ahead"
    assert not np.allclose(o0[tp], o1[tp]), "token does not affect its own read-out"


def pin_conv_library(orc):
    """The conv equals numpy's correlation on the zero- or history-padded input,
    an impulse reproduces the taps in time order (w[:, W-1] on the current token),
    SiLU equals y * scipy's expit(y), and the returned history is the last W-1 inputs."""
    from scipy.special import expit
    rng = np.random.default_rng(8)
    T, C, W = 13, 5, 4
    x = rng.standard_normal((T, C))
    w = rng.standard_normal((C, W))
    b = rng.standard_normal(C)
    hist = rng.standard_normal((1, W - 1, C))
    y, st = orc.short_conv(x, w, state_in=hist, bias=b, silu=False, return_state=True)
    ys = orc.short_conv(x, w, state_in=hist, bias=b, silu=True)
    for c in range(C):
        xe = np.concatenate([hist[0, :, c], x[:, c]])
        ref = np.correlate(xe, w[c], mode="valid") + b[c]
        _close(y[:, c], ref, what="conv vs np.correlate")
        _close(ys[:, c], ref * expit(ref), what="SiLU")
        _close(st[0, :, c], xe[-(W - 1):], what="returned history")
    imp = np.zeros((T, C))
    imp[4] = 1.0
    yi = orc.short_conv(imp, w, silu=False)
    for j in range(W):
        _close(yi[4 + j], w[:, W - 1 - j], what="impulse response lag %d" % j)
    _close(yi[:4], np.zeros((4, C)), what="impulse before onset")


def pin_l2norm(orc):
    """L2 normalisation (Walkthrough 第二站) equals x / sqrt(||x||^2 + eps)."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal((7, 3, 16)) * 3.0
    for eps in (0.0, 1e-6):
        y = orc.l2norm(x, 16, eps).reshape(x.shape)
        ref = x / np.sqrt(np.linalg.norm(x, axis=-1, keepdims=True) ** 2 + eps)
        _close(y, ref, what="l2norm eps=%g" % eps)
    y = orc.l2norm(x, 16, 0.0).reshape(x.shape)
    _close(np.linalg.norm(y, axis=-1), np.ones((7, 3)), what="unit length")


def pin_round_bf16(orc):
    """bf16 rounding: ties go to the even neighbour; other values match torch's
    float32 -> bfloat16 conversion (a library routine) on fp32-representable inputs."""
    import torch
    ties = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 3 * 2.0 ** -9 + 2.0 ** -1,
                     0.0, 2.0 ** 20 * (1 + 2.0 ** -8)])
    want = np.array([1.0, 1 + 2.0 ** -6, -1.0, 0.5 + 2.0 ** -7, 0.0, 2.0 ** 20])
    _close(orc.round_bf16(ties), want, tol=0.0, what="bf16 ties")
    rng = np.random.default_rng(13)
    x = (rng.standard_normal(5000) * np.exp(rng.uniform(-20, 20, 5000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    got = orc.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref), "bf16 rounding differs from torch on %d values" % int(
        np.sum(got != ref))


def pin_varlen_and_resume(orc):
    """Packed sequences equal separate runs; a split carrying (S, conv history)
    equals the unsplit run."""
    rng = np.random.default_rng(10)
    lengths = [6, 1, 15]
    T, H, D = sum(lengths), 2, 4
    cu = np.cumsum([0] + lengths)
    x = rng.standard_normal((T, H * D))
    w = rng.standard_normal((H * D, 4))
    q, k, v, g, beta = _rand_inputs(rng, T, H, D, D)
    h0 = rng.standard_normal((len(lengths), H, D, D))
    yp = orc.short_conv(x, w, cu_seqlens=cu)
    op, hp = orc.recurrent(q, k, v, g, beta, cu_seqlens=cu, h0=h0, scale=0.9)
    for n in range(len(lengths)):
        s, e = cu[n], cu[n + 1]
        _close(yp[s:e], orc.short_conv(x[s:e], w), what="packed conv seq %d" % n)
        on, hn = orc.recurrent(q[s:e], k[s:e], v[s:e], g[s:e], beta[s:e], h0=h0[n:n + 1],
                               scale=0.9)
        _close(op[s:e], on, what="packed o seq %d" % n)
        _close(hp[n], hn[0], what="packed state seq %d" % n)
    # split the last sequence at every point and resume
    s, e = cu[-2], cu[-1]
    for cut in (1, 2, 7, 14):
        m = s + cut
        y1, st = orc.short_conv(x[s:m], w, return_state=True)
        y2 = orc.short_conv(x[m:e], w, state_in=st)
        _close(np.concatenate([y1, y2]), yp[s:e], what="conv resume at %d" % cut)
        o1, s1 = orc.recurrent(q[s:m], k[s:m], v[s:m], g[s:m], beta[s:m], h0=h0[-1:], scale=0.9)
        o2, s2 = orc.recurrent(q[m:e], k[m:e], v[m:e], g[m:e], beta[m:e], h0=s1, scale=0.9)
        _close(np.concatenate([o1, o2]), op[s:e], what="recurrence resume at %d" % cut)
        _close(s2[0], hp[-1], what="state resume at %d" % cut)


def pin_value_columns_independent(orc):
    """Columns of v (and of S) evolve independently: a column slice reproduces them."""
    rng = np.random.default_rng(12)
    T, H, DK, DV = 14, 2, 5, 6
    q, k, v, g, beta = _rand_inputs(rng, T, H, DK, DV)
    h0 = rng.standard_normal((1, H, DK, DV))
    o, hT = orc.recurrent(q, k, v, g, beta, h0=h0)
    for sl in (slice(0, 2), slice(2, 6), slice(5, 6)):
        os_, hs = orc.recurrent(q, k, v[:, :, sl], g, beta, h0=h0[:, :, :, sl])
        _close(os_, o[:, :, sl], what="o column slice")
        _close(hs, hT[:, :, :, sl], what="state column slice")


def pin_k3_sizes(orc=None):
    """Walkthrough 回头看看 / 彩蛋: state size and the 16-token decay bound."""
    gd = golden("k3_sizes.json")
    n = gd["heads"] * gd["dk"] * gd["dv"]
    assert n == gd["state_elements_per_layer_per_sequence"]
    assert round(n * 4 / 2 ** 20) == gd["fp32_state_bytes_approx_MiB"]
    lo, hi = gd["subchunk_cumulative_log_decay_range"]
    assert gd["subchunk_tokens"] * gd["gate_lower_bound"] == lo and hi == 0.0


def pin_bounded_gate(orc):
    """Walkthrough 彩蛋: g = lb * sigmoid(e^{A_log[h]} (z + dt_bias[h, c])).

    sigmoid(0) = 1/2 and sigmoid(ln 3) = 3/4 give closed forms; A_log enters
    through its exponential (per head), dt_bias is added per (head, channel),
    and lb <= g <= 0 with g decreasing in z.
    """
    T, H, D = 3, 2, 4
    ln3 = np.log(3.0)
    for lb in (-5.0, -8.0):
        # no A_log, no bias: rows z = 0, ln 3, -ln 3
        z = np.zeros((T, H, D))
        z[1], z[2] = ln3, -ln3
        g = orc.bounded_gate(z, lower_bound=lb)
        for t, f in enumerate((0.5, 0.75, 0.25)):
            _close(g[t], np.full((H, D), f * lb), 1e-15, "gate closed form row %d" % t)
        # A_log = ln 2 doubles the argument of head 1 only
        z = np.full((T, H, D), ln3 / 2)
        g = orc.bounded_gate(z, a_log=np.array([0.0, np.log(2.0)]), lower_bound=lb)
        _close(g[:, 1], np.full((T, D), 0.75 * lb), 1e-15, "gate A_log head 1")
        _close(g[:, 0], np.full((T, D), lb / (1.0 + 3.0 ** -0.5)), 1e-15, "gate A_log head 0")
        # the per-channel bias shifts z: z = ln 3 - dt gives 3/4 everywhere
        dt = 0.1 * np.arange(1, H * D + 1).reshape(H, D)
        g = orc.bounded_gate(np.broadcast_to(ln3 - dt, (T, H, D)), dt_bias=dt, lower_bound=lb)
        _close(g, np.full((T, H, D), 0.75 * lb), 1e-14, "gate dt_bias")
    # bounds and monotonicity on random pre-activations
    rng = np.random.default_rng(21)
    z = np.sort(rng.normal(0.0, 4.0, (64, 1, 1)), axis=0)
    g = orc.bounded_gate(z, a_log=np.array([0.3]), dt_bias=np.array([[0.2]]), lower_bound=-5.0)
    assert np.all(g >= -5.0) and np.all(g <= 0.0), "gate outside [lb, 0]"
    assert np.all(np.diff(g[:, 0, 0]) <= 0.0), "gate not decreasing in z"


def pin_output_norm_gate(orc):
    """Walkthrough 第六站: per-head RMSNorm of the read-out, then the sigmoid output gate.

    A constant row c normalises to sign(c) (eps = 0); gate 0 halves and gate ln 3
    keeps three quarters; the norm is per (token, head) and invariant to the row's
    scale; the normalised row has unit root-mean-square.
    """
    ln3 = np.log(3.0)
    T, H, D = 2, 3, 8
    o = np.empty((T, H, D))
    for t in range(T):
        for h in range(H):
            o[t, h] = (-1.0) ** (t + h) * 10.0 ** (h - 1)       # constant rows, scales 0.1 .. 10
    gate = np.zeros((T, H, D))
    gate[1] = ln3
    w = 1.0 + 0.25 * np.arange(D)
    y = orc.output_norm_gate(o, gate, w, eps=0.0)
    for t, f in enumerate((0.5, 0.75)):
        for h in range(H):
            _close(y[t, h], np.sign(o[t, h]) * w * f, 1e-14, "constant row t=%d h=%d" % (t, h))
    rng = np.random.default_rng(23)
    o = rng.standard_normal((4, H, D)) * np.array([0.01, 1.0, 50.0])[None, :, None]
    gate = rng.standard_normal((4, H, D))
    y = orc.output_norm_gate(o, gate, None, eps=0.0)
    _close(orc.output_norm_gate(7.5 * o, gate, None, eps=0.0), y, 1e-13, "scale invariance")
    yn = y * (1.0 + np.exp(-gate))                      # undo the gate: unit-rms rows
    _close(np.sqrt(np.mean(yn * yn, axis=-1)), np.ones((4, H)), 1e-13, "unit rms per row")
    ref = o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + 1e-3) / (1.0 + np.exp(-gate))
    _close(orc.output_norm_gate(o, gate, None, eps=1e-3), ref, 1e-13, "eps inside the root")


ALL_PINS = [
    pin_unit_key_example, pin_one_dim_example, pin_two_address_example, pin_update_order,
    pin_identity, pin_pure_decay, pin_overwrite, pin_linear_attention, pin_gated_form,
    pin_chunked_matches_recurrent, pin_causality, pin_conv_library, pin_l2norm, pin_round_bf16,
    pin_varlen_and_resume, pin_value_columns_independent, pin_k3_sizes, pin_bounded_gate,
    pin_output_norm_gate,
]
