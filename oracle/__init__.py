"""fp64 CPU oracle for the Kimi Delta Attention (KDA) forward pass.

TEST INFRASTRUCTURE ONLY.  The oracle is the plain, slow, obviously-correct
definition of what the GPU path computes.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with ``channel_gated_delta_amd`` (neither package
imports the other) and the GPU path never falls back to it.

Sources are web pages, cited by title and section:

* [Walkthrough] "Kimi K3的线性注意力：从源码看懂KDA如何更新记忆" -- the source-code
  walkthrough of the KDA layer; sections 第二站 (short conv + SiLU, q/k L2 norm),
  第三站 (per-key-channel decay first), 第四站 (prediction, error, corrective
  write), 第五站 (read-out after the write), 彩蛋 (recurrent vs chunked execution).
* [K3-memory] "Kimi K3 记忆架构总览：KDA、MLA、AttnRes 各管什么" -- section
  "KDA 谱系速查" (read, difference, overwrite; the I - beta k k^T rewrite).
* [Replication-2] "KimiK3轻量化复刻实现KDA并行解析，Chunkwise并行与状态压缩机制详解"
  -- figure 1 (chunk-level composition of affine state transitions).
* [Workshop-16] "AI-Workshop 文献分享 #16 — KDA：给长文本建立可更新的记忆" --
  sections 4 (linear attention), 5.1 (two-address example), 7 (gated form),
  8.4 (one-dimensional correction example).

Contents:

* ``bounded_gate`` (O0) log-decay from the bounded gate's pre-activation -- C, fp64
* ``short_conv``  (O1a) causal depthwise conv + SiLU with conv cache  -- C, fp64
* ``l2norm``      (O1b) q/k L2 normalisation                          -- C, fp64
* ``round_bf16``  (O1c) rounding of an interface tensor to bf16         -- C, fp64
* ``prologue``    O1a + O1b (+ O1c) for one of q, k, v                 -- C, fp64
* ``recurrent``   (O2) token-by-token KDA recurrence                   -- C, fp64
* ``output_norm_gate`` (O3) per-head RMSNorm times the sigmoid output gate -- C, fp64
* ``oracle.chunked.chunked_forward``: an independently derived chunkwise
  form, used only as a brute-force pin of ``recurrent`` on tiny inputs.

Parity pins (tests/test_oracle_pins.py) tie every function here to the pages'
worked examples, closed forms and invariants; no function is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)


def compile_library(src: str, out: str) -> str:
    """gcc -O2 -fopenmp: build one shared object of the C oracle."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call(
        ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", src, "-o", tmp, "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile the C oracle in-tree."""
    if force or not os.path.exists(_LIB_PATH):
        compile_library(SOURCE, _LIB_PATH)
    return _LIB_PATH


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(_dp)


def _seqlens(cu_seqlens, total: int) -> np.ndarray:
    if cu_seqlens is None:
        return np.array([0, total], dtype=np.int32)
    return np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))


class OracleLib:
    """ctypes view of one build of kda_oracle.c."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        lib.kda_oracle_short_conv.argtypes = [
            _dp, ctypes.c_int64, ctypes.c_int64, _dp, ctypes.c_int, _dp, _ip, ctypes.c_int,
            _dp, _dp, ctypes.c_int, _dp]
        lib.kda_oracle_short_conv.restype = ctypes.c_int
        lib.kda_oracle_l2norm.argtypes = [_dp, ctypes.c_int64, ctypes.c_int64, ctypes.c_double]
        lib.kda_oracle_l2norm.restype = None
        lib.kda_oracle_recurrent.argtypes = [
            _dp, _dp, _dp, _dp, _dp, _ip, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_double, _dp, _dp, _dp, ctypes.c_int]
        lib.kda_oracle_recurrent.restype = ctypes.c_int
        lib.kda_oracle_round_bf16.argtypes = [_dp, ctypes.c_int64]
        lib.kda_oracle_round_bf16.restype = None
        lib.kda_oracle_bounded_gate.argtypes = [
            _dp, ctypes.c_int64, ctypes.c_int, ctypes.c_int, _dp, _dp, ctypes.c_double, _dp]
        lib.kda_oracle_bounded_gate.restype = None
        lib.kda_oracle_output_norm_gate.argtypes = [
            _dp, _dp, ctypes.c_int64, ctypes.c_int, ctypes.c_int, _dp, ctypes.c_double, _dp]
        lib.kda_oracle_output_norm_gate.restype = None
        lib.kda_oracle_num_threads.argtypes = []
        lib.kda_oracle_num_threads.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def num_threads(self) -> int:
        return int(self.lib.kda_oracle_num_threads())

    def bounded_gate(self, z, a_log=None, dt_bias=None, lower_bound: float = -5.0):
        """O0: g = lower_bound * sigmoid(exp(A_log[h]) * (z + dt_bias[h, c])).

        z: [T, H, D]; a_log: [H] or None (0); dt_bias: [H, D] or None (0).
        Returns g [T, H, D], the log-decay (lower_bound <= g <= 0).
        """
        z = _f64(z)
        T, H, D = z.shape
        al = None if a_log is None else _f64(a_log).reshape(H)
        dt = None if dt_bias is None else _f64(dt_bias).reshape(H, D)
        g = np.empty((T, H, D))
        self.lib.kda_oracle_bounded_gate(_ptr(z), T, H, D, _ptr(al), _ptr(dt),
                                         float(lower_bound), _ptr(g))
        return g

    def short_conv(self, x, w, cu_seqlens=None, state_in=None, bias=None, silu=True,
                   return_state=False):
        """O1a: causal depthwise conv over packed sequences.

        x: [T, C]; w: [C, W] (w[:, W-1] multiplies the current token);
        state_in: [N, W-1, C] history (oldest first) or None for zeros.
        Returns y [T, C] (and the new history [N, W-1, C] if return_state).
        """
        x = _f64(x)
        w = _f64(w)
        T, C = x.shape
        W = w.shape[1]
        cu = _seqlens(cu_seqlens, T)
        N = cu.shape[0] - 1
        sin = None if state_in is None else _f64(state_in).reshape(N, W - 1, C)
        sout = np.zeros((N, W - 1, C)) if return_state else None
        b = None if bias is None else _f64(bias)
        y = np.empty((T, C))
        rc = self.lib.kda_oracle_short_conv(
            _ptr(x), T, C, _ptr(w), W, _ptr(b), cu.ctypes.data_as(_ip), N,
            _ptr(sin), _ptr(sout), 1 if silu else 0, _ptr(y))
        if rc != 0:
            raise ValueError("kda_oracle_short_conv failed (%d)" % rc)
        return (y, sout) if return_state else y

    def l2norm(self, x, D: int, eps: float = 1e-6) -> np.ndarray:
        """O1b: scale each group of D consecutive values by 1/sqrt(sum x^2 + eps)."""
        y = _f64(x).copy()
        rows = y.size // D
        self.lib.kda_oracle_l2norm(_ptr(y), rows, D, float(eps))
        return y

    def round_bf16(self, x) -> np.ndarray:
        """O1c: round to the nearest bf16 value (ties to even)."""
        y = _f64(x).copy()
        self.lib.kda_oracle_round_bf16(_ptr(y), y.size)
        return y

    def prologue(self, x, w, H: int, D: int, cu_seqlens=None, state_in=None, bias=None,
                 normalize: bool = False, eps: float = 1e-6, return_state=False,
                 out_bf16: bool = False):
        """O1: conv + SiLU, then (q and k only) per-head L2 normalisation.

        x: [T, H*D] raw projection; returns [T, H, D] (and the conv history).
        out_bf16: the result is the pipeline's bf16 interface tensor (O1c).
        """
        out = self.short_conv(x, w, cu_seqlens, state_in, bias, silu=True,
                              return_state=return_state)
        y, st = out if return_state else (out, None)
        T = y.shape[0]
        if normalize:
            y = self.l2norm(y, D, eps)
        if out_bf16:
            y = self.round_bf16(y)
        y = y.reshape(T, H, D)
        return (y, st) if return_state else y

    def output_norm_gate(self, o, gate, w=None, eps: float = 1e-6):
        """O3: y = o / sqrt(mean(o^2) + eps) * w * sigmoid(gate), per (token, head) row.

        o, gate: [T, H, D]; w: [D] or None (1).  Returns y [T, H, D].
        """
        o, gate = _f64(o), _f64(gate)
        T, H, D = o.shape
        wa = None if w is None else _f64(w).reshape(D)
        y = np.empty((T, H, D))
        self.lib.kda_oracle_output_norm_gate(_ptr(o), _ptr(gate), T, H, D, _ptr(wa), float(eps),
                                             _ptr(y))
        return y

    def recurrent(self, q, k, v, g, beta, cu_seqlens=None, scale: float = 1.0, h0=None,
                  delta_rule: bool = True):
        """O2: the KDA recurrence, token by token, in fp64.

        q, k, g: [T, H, DK]; v: [T, H, DV]; beta: [T, H]; h0: [N, H, DK, DV] or None.
        Returns (o [T, H, DV], hT [N, H, DK, DV]).
        """
        q, k, v, g, beta = (_f64(a) for a in (q, k, v, g, beta))
        T, H, DK = q.shape
        DV = v.shape[2]
        cu = _seqlens(cu_seqlens, T)
        N = cu.shape[0] - 1
        h0a = None if h0 is None else _f64(h0).reshape(N, H, DK, DV)
        o = np.empty((T, H, DV))
        hT = np.empty((N, H, DK, DV))
        rc = self.lib.kda_oracle_recurrent(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), cu.ctypes.data_as(_ip), N, T, H,
            DK, DV, float(scale), _ptr(h0a), _ptr(o), _ptr(hT), 1 if delta_rule else 0)
        if rc != 0:
            raise ValueError("kda_oracle_recurrent failed (%d)" % rc)
        return o, hT


_default = None


def default() -> OracleLib:
    """The in-tree build of the oracle (rebuilt when the source is newer)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(SOURCE):
            build()
        _default = OracleLib(_LIB_PATH)
    return _default


def num_threads() -> int:
    return default().num_threads()


def bounded_gate(*a, **kw):
    return default().bounded_gate(*a, **kw)


def short_conv(*a, **kw):
    return default().short_conv(*a, **kw)


def l2norm(*a, **kw):
    return default().l2norm(*a, **kw)


def prologue(*a, **kw):
    return default().prologue(*a, **kw)


def round_bf16(*a, **kw):
    return default().round_bf16(*a, **kw)


def recurrent(*a, **kw):
    return default().recurrent(*a, **kw)


def output_norm_gate(*a, **kw):
    return default().output_norm_gate(*a, **kw)


def rel_err(got, ref) -> float:
    """max|got - ref| / rms(ref), in fp64 (the parity metric)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    if rms == 0.0:
        return float(np.max(np.abs(got - ref))) if got.size else 0.0
    return float(np.max(np.abs(got - ref)) / rms)
