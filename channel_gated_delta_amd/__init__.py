"""KDA (Kimi Delta Attention) forward pass on AMD MI355X -- Python binding of libkda.

Thin ctypes binding over the C ABI in include/kda.h.  It only checks and
marshals arguments: every step of the computation runs in the HIP kernels of
libkda.so.  PyTorch provides device memory and the current stream.  There is no
fallback: if libkda.so is missing the calls raise.

    short_conv(x, weight, ...)              -> (y, conv_state)   conv4 + SiLU (+ L2)
    chunk_fwd(q, k, v, g, beta, ...)        -> (o, final_state)  chunkwise prefill
    chunk_fwd_gated(q, k, v, z, beta, ...)  -> (o, final_state)  the same, bounded gate fused
    chunk_fwd_noalloc(q, k, v, g, beta, out, final_state, ...)   no workspace (static scratch)
    output_norm_gate(o, gate, weight, ...)  -> y                 per-head RMSNorm * sigmoid gate
    gdn_chunk_fwd / gdn_decode_step         one decay per (token, head): g [T, H] / [B, H]
    decode_step(q, k, v, g, beta, state)    -> o                 one recurrent step
    decode_step_conv(q_raw, ..., state)     -> o                 conv + SiLU + L2 + the step

Build the library with ``python -m channel_gated_delta_amd.build``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = ["KdaError", "library", "short_conv", "chunk_fwd", "chunk_fwd_gated", "decode_step",
           "output_norm_gate", "decode_step_conv", "gdn_chunk_fwd", "gdn_decode_step",
           "chunk_fwd_noalloc", "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")

KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_HIP, KDA_ERR_WORKSPACE = 0, 1, 2, 3, 4
PHASE_PREP, PHASE_WALK, PHASE_ALL = 1, 2, 3   # kda_chunk_fwd_phases
_DTYPES = {torch.float32: 0, torch.bfloat16: 1}

_lib = None
_vp = ctypes.c_void_p
_i32, _i64, _f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float


class KdaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("libkda status %d: %s" % (status, msg))
        self.status = status


def library() -> ctypes.CDLL:
    """Load libkda.so (raises when it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libkda.so is not built (%s); run `python -m "
                               "channel_gated_delta_amd.build`" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        lib.kda_short_conv.argtypes = [_vp, _vp, _vp, _vp, _i32, _i64, _i32, _i32, _i32, _vp, _vp,
                                       _i32, _i32, _f32, _i32, _vp, _vp]
        lib.kda_chunk_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i64, _i32, _i32, _i32,
                                      _i32, _f32, _f32, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                                      _i32, _i32, _vp]
        lib.kda_chunk_fwd_gated.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _f32, _vp, _vp, _i32,
                                            _i64, _i32, _i32, _i32, _i32, _f32, _vp, _vp, _vp,
                                            _vp, ctypes.c_size_t, _i32, _i32, _vp]
        lib.kda_decode_step_conv.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32,
                                             _vp, _vp, _vp, _i32, _i32, _i32, _i32, _f32, _vp,
                                             _i32, _i32, _vp]
        lib.kda_output_norm_gate.argtypes = [_vp, _vp, _vp, _f32, _i64, _i32, _i32, _i32, _vp,
                                             _vp]
        lib.kda_chunk_fwd_workspace_size.argtypes = [_i64, _i32, _i32, _i32, _i32, _i32, _i32,
                                                     ctypes.POINTER(ctypes.c_size_t)]
        lib.kda_decode_step.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _f32,
                                        _vp, _i32, _i32, _vp]
        lib.kda_gdn_chunk_fwd.argtypes = lib.kda_chunk_fwd.argtypes
        lib.kda_chunk_fwd_phases.argtypes = lib.kda_chunk_fwd.argtypes[:-1] + [_i32, _vp]
        lib.kda_chunk_fwd_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i64, _i32, _i32,
                                              _i32, _i32, _f32, _f32, _vp, _vp, _vp, _i32, _i32,
                                              _vp]
        lib.kda_gdn_decode_step.argtypes = lib.kda_decode_step.argtypes
        for fn in ("kda_short_conv", "kda_chunk_fwd", "kda_chunk_fwd_gated",
                   "kda_chunk_fwd_workspace_size", "kda_decode_step", "kda_output_norm_gate",
                   "kda_decode_step_conv", "kda_gdn_chunk_fwd", "kda_gdn_decode_step",
                   "kda_chunk_fwd_noalloc", "kda_chunk_fwd_phases"):
            getattr(lib, fn).restype = ctypes.c_int
        lib.kda_status_string.argtypes = [ctypes.c_int]
        lib.kda_status_string.restype = ctypes.c_char_p
        lib.kda_last_error.argtypes = []
        lib.kda_last_error.restype = ctypes.c_char_p
        lib.kda_version.argtypes = []
        lib.kda_version.restype = ctypes.c_int32
        _lib = lib
    return _lib


def _check(status: int) -> None:
    if status != KDA_OK:
        lib = library()
        detail = lib.kda_last_error().decode() or lib.kda_status_string(status).decode()
        raise KdaError(status, detail)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else _vp(t.data_ptr())


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    return t


def _stream(t: torch.Tensor):
    return _vp(torch.cuda.current_stream(t.device).cuda_stream)


def _seqs(cu_seqlens: Optional[torch.Tensor], total: int) -> int:
    if cu_seqlens is None:
        return 1
    _dev(cu_seqlens, "cu_seqlens", torch.int32)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be 1-D with num_seqs + 1 entries")
    return cu_seqlens.numel() - 1


def short_conv(x: torch.Tensor, weight: torch.Tensor, *, num_heads: int, head_dim: int,
               cu_seqlens: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
               conv_state: Optional[torch.Tensor] = None, output_final_state: bool = False,
               silu: bool = True, l2_normalize: bool = False, l2_eps: float = 1e-6,
               out: Optional[torch.Tensor] = None, state_out: Optional[torch.Tensor] = None
               ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Causal depthwise conv (+SiLU, +per-head L2) over packed sequences.

    x: [T, H*D]; weight: [H*D, W]; conv_state: [N, W-1, H*D] or None.
    Returns y [T, H, D] and the new conv state [N, W-1, H*D] (if output_final_state
    or ``state_out`` is given; ``state_out`` may be ``conv_state`` itself).
    """
    _dev(x, "x")
    dt = x.dtype
    if dt not in _DTYPES:
        raise ValueError("x must be bf16 or fp32")
    T = x.shape[0]
    C = num_heads * head_dim
    _dev(x, "x", dt, (T, C))
    W = weight.shape[1] if weight.dim() == 2 else -1
    _dev(weight, "weight", dt, (C, W))
    if bias is not None:
        _dev(bias, "bias", dt, (C,))
    N = _seqs(cu_seqlens, T)
    if conv_state is not None:
        _dev(conv_state, "conv_state", dt, (N, W - 1, C))
    y = out if out is not None else torch.empty((T, num_heads, head_dim), dtype=dt, device=x.device)
    _dev(y, "out", dt, (T, num_heads, head_dim))
    new_state = state_out
    if new_state is None and output_final_state:
        new_state = torch.empty((N, W - 1, C), dtype=dt, device=x.device)
    if new_state is not None:
        _dev(new_state, "state_out", dt, (N, W - 1, C))
    _check(library().kda_short_conv(
        _ptr(x), _ptr(weight), _ptr(bias), _ptr(cu_seqlens), N, T, num_heads, head_dim, W,
        _ptr(conv_state), _ptr(new_state), 1 if silu else 0, 1 if l2_normalize else 0,
        float(l2_eps), _DTYPES[dt], _ptr(y), _stream(x)))
    return y, new_state


def chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
              beta: torch.Tensor, *, cu_seqlens: Optional[torch.Tensor] = None,
              scale: Optional[float] = None, gate_lower_bound: float = -5.0, chunk_size: int = 64,
              initial_state: Optional[torch.Tensor] = None, output_final_state: bool = True,
              out: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
              out_dtype: torch.dtype = torch.float32, workspace: Optional[torch.Tensor] = None,
              phases: int = 3) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunkwise KDA prefill.  q, k, g: [T, H, dk]; v: [T, H, dv]; beta: [T, H].

    Returns o [T, H, dv] (``out_dtype``, fp32 by default) and the final states
    [N, H, dk, dv] (fp32) if requested.  ``workspace`` (a uint8 GPU tensor of at
    least ``chunk_workspace_bytes(...)`` bytes) is allocated when not given.
    ``phases`` (kda_chunk_fwd_phases): PHASE_PREP enqueues the prep only (into
    ``workspace``, which the caller then passes to the PHASE_WALK call with the
    same arguments), PHASE_WALK the walk only, PHASE_ALL both.
    """
    T, H, dk = q.shape
    _dev(g, "g", torch.float32, (T, H, dk))
    return _chunk(q, k, v, g, None, beta, cu_seqlens, scale, gate_lower_bound, chunk_size,
                  initial_state, output_final_state, out, final_state, out_dtype, workspace,
                  phases)


def chunk_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                      beta: torch.Tensor, out: torch.Tensor, final_state: Optional[torch.Tensor],
                      *, cu_seqlens: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                      gate_lower_bound: float = -5.0, chunk_size: int = 64,
                      initial_state: Optional[torch.Tensor] = None) -> None:
    """``chunk_fwd`` through kda_chunk_fwd_noalloc: no workspace, the library's static
    device scratch instead (at most 524288 token-heads per call; calls that overlap
    on one GPU race).  The caller passes the outputs ``out`` [T, H, dv] (fp32, or
    bf16 with bf16 inputs) and ``final_state`` [N, H, dk, dv] fp32 (or None); this
    wrapper allocates nothing either."""
    _dev(q, "q")
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError("q must be bf16 or fp32")
    T, H, dk = q.shape
    dv = v.shape[-1]
    _dev(k, "k", dt, (T, H, dk))
    _dev(v, "v", dt, (T, H, dv))
    _dev(g, "g", torch.float32, (T, H, dk))
    _dev(beta, "beta", torch.float32, (T, H))
    N = _seqs(cu_seqlens, T)
    if initial_state is not None:
        _dev(initial_state, "initial_state", torch.float32, (N, H, dk, dv))
    if final_state is not None:
        _dev(final_state, "final_state", torch.float32, (N, H, dk, dv))
    if out.dtype not in _DTYPES:
        raise ValueError("out must be bf16 or fp32")
    _dev(out, "out", out.dtype, (T, H, dv))
    sc = dk ** -0.5 if scale is None else float(scale)
    _check(library().kda_chunk_fwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), N, T, H, dk, dv,
        int(chunk_size), sc, float(gate_lower_bound), _ptr(initial_state), _ptr(final_state),
        _ptr(out), _DTYPES[dt], _DTYPES[out.dtype], _stream(q)))


def gdn_chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                  beta: torch.Tensor, *, cu_seqlens: Optional[torch.Tensor] = None,
                  scale: Optional[float] = None, gate_lower_bound: float = -5.0,
                  chunk_size: int = 64, initial_state: Optional[torch.Tensor] = None,
                  output_final_state: bool = True, out: Optional[torch.Tensor] = None,
                  final_state: Optional[torch.Tensor] = None,
                  out_dtype: torch.dtype = torch.float32,
                  workspace: Optional[torch.Tensor] = None
                  ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """``chunk_fwd`` with one decay per (token, head): g [T, H] fp32 (GDN's gate)."""
    T, H, dk = q.shape
    _dev(g, "g", torch.float32, (T, H))
    return _chunk(q, k, v, g, "head", beta, cu_seqlens, scale, gate_lower_bound, chunk_size,
                  initial_state, output_final_state, out, final_state, out_dtype, workspace)


def chunk_fwd_gated(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, z: torch.Tensor,
                    beta: torch.Tensor, *, a_log: Optional[torch.Tensor] = None,
                    dt_bias: Optional[torch.Tensor] = None, lower_bound: float = -5.0,
                    cu_seqlens: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                    chunk_size: int = 64, initial_state: Optional[torch.Tensor] = None,
                    output_final_state: bool = True, out: Optional[torch.Tensor] = None,
                    final_state: Optional[torch.Tensor] = None,
                    out_dtype: torch.dtype = torch.float32,
                    workspace: Optional[torch.Tensor] = None
                    ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunkwise KDA prefill with the bounded gate fused in: the kernels form
    g = lower_bound * sigmoid(exp(a_log[h]) * (z + dt_bias[h, c])) from z [T, H, dk]
    (q's dtype), a_log [H] and dt_bias [H, dk] (fp32, optional).  Otherwise as
    ``chunk_fwd``."""
    T, H, dk = q.shape
    _dev(z, "z", q.dtype, (T, H, dk))
    if a_log is not None:
        _dev(a_log, "a_log", torch.float32, (H,))
    if dt_bias is not None:
        _dev(dt_bias, "dt_bias", torch.float32, (H, dk))
    return _chunk(q, k, v, None, (z, a_log, dt_bias), beta, cu_seqlens, scale, lower_bound,
                  chunk_size, initial_state, output_final_state, out, final_state, out_dtype,
                  workspace)


def _chunk(q, k, v, g, gate, beta, cu_seqlens, scale, lower_bound, chunk_size, initial_state,
           output_final_state, out, final_state, out_dtype, workspace, phases=3):
    _dev(q, "q")
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError("q must be bf16 or fp32")
    T, H, dk = q.shape
    dv = v.shape[-1]
    _dev(k, "k", dt, (T, H, dk))
    _dev(v, "v", dt, (T, H, dv))
    _dev(beta, "beta", torch.float32, (T, H))
    N = _seqs(cu_seqlens, T)
    if initial_state is not None:
        _dev(initial_state, "initial_state", torch.float32, (N, H, dk, dv))
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    if final_state is not None:
        _dev(final_state, "final_state", torch.float32, (N, H, dk, dv))
    if out is not None:
        out_dtype = out.dtype
    if out_dtype not in _DTYPES:
        raise ValueError("out_dtype must be bf16 or fp32")
    o = out if out is not None else torch.empty((T, H, dv), dtype=out_dtype, device=q.device)
    _dev(o, "out", out_dtype, (T, H, dv))
    sc = dk ** -0.5 if scale is None else float(scale)
    need = chunk_workspace_bytes(T, H, dk, dv, chunk_size, dt, out_dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace", torch.uint8)
    if gate is None and phases != PHASE_ALL:
        _check(library().kda_chunk_fwd_phases(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), N, T, H, dk, dv,
            int(chunk_size), sc, float(lower_bound), _ptr(initial_state), _ptr(final_state),
            _ptr(o), _ptr(workspace), workspace.numel(), _DTYPES[dt], _DTYPES[out_dtype],
            int(phases), _stream(q)))
    elif gate is None or gate == "head":
        fn = library().kda_chunk_fwd if gate is None else library().kda_gdn_chunk_fwd
        _check(fn(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), N, T, H, dk, dv,
            int(chunk_size), sc, float(lower_bound), _ptr(initial_state), _ptr(final_state),
            _ptr(o), _ptr(workspace), workspace.numel(), _DTYPES[dt], _DTYPES[out_dtype],
            _stream(q)))
    else:
        z, a_log, dt_bias = gate
        _check(library().kda_chunk_fwd_gated(
            _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(a_log), _ptr(dt_bias), float(lower_bound),
            _ptr(beta), _ptr(cu_seqlens), N, T, H, dk, dv, int(chunk_size), sc,
            _ptr(initial_state), _ptr(final_state), _ptr(o), _ptr(workspace), workspace.numel(),
            _DTYPES[dt], _DTYPES[out_dtype], _stream(q)))
    return o, final_state


def output_norm_gate(o: torch.Tensor, gate: torch.Tensor, weight: Optional[torch.Tensor] = None,
                     *, eps: float = 1e-6, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = o / sqrt(mean(o^2) + eps) * weight * sigmoid(gate) per (token, head) row.

    o: [..., dv] (fp32 or bf16); gate: same shape in the activation dtype (bf16 or
    fp32), which y takes; weight: [dv] fp32 or None.  ``out`` may be ``gate``.
    """
    _dev(o, "o")
    _dev(gate, "gate", None, tuple(o.shape))
    if o.dtype not in _DTYPES or gate.dtype not in _DTYPES:
        raise ValueError("o and gate must be bf16 or fp32")
    dv = o.shape[-1]
    if weight is not None:
        _dev(weight, "weight", torch.float32, (dv,))
    y = out if out is not None else torch.empty_like(gate)
    _dev(y, "out", gate.dtype, tuple(o.shape))
    rows = o.numel() // dv if dv else 0
    _check(library().kda_output_norm_gate(_ptr(o), _ptr(gate), _ptr(weight), float(eps), rows,
                                          dv, _DTYPES[o.dtype], _DTYPES[gate.dtype], _ptr(y),
                                          _stream(o)))
    return y


def chunk_workspace_bytes(total_tokens: int, num_heads: int, dk: int, dv: int,
                          chunk_size: int = 64, dtype: torch.dtype = torch.bfloat16,
                          out_dtype: torch.dtype = torch.float32) -> int:
    """Device workspace bytes ``chunk_fwd`` needs for these sizes."""
    n = ctypes.c_size_t(0)
    _check(library().kda_chunk_fwd_workspace_size(int(total_tokens), int(num_heads), int(dk),
                                                  int(dv), int(chunk_size), _DTYPES[dtype],
                                                  _DTYPES[out_dtype], ctypes.byref(n)))
    return int(n.value)


def decode_step_conv(q_raw: torch.Tensor, k_raw: torch.Tensor, v_raw: torch.Tensor,
                     w_q: torch.Tensor, w_k: torch.Tensor, w_v: torch.Tensor,
                     conv_q: torch.Tensor, conv_k: torch.Tensor, conv_v: torch.Tensor,
                     g: torch.Tensor, beta: torch.Tensor, state: torch.Tensor, *,
                     scale: Optional[float] = None, l2_eps: float = 1e-6,
                     out: Optional[torch.Tensor] = None,
                     out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """One generation step from raw projections: width-4 conv over the conv caches
    (updated in place), SiLU, q/k L2, then the recurrent step (``state`` in place).

    q_raw, k_raw: [B, H*dk]; v_raw: [B, H*dv]; w_*: [H*d, 4]; conv_*: [B, 3, H*d]
    (all in the activation dtype); g: [B, H, dk]; beta: [B, H]; state fp32.
    """
    _dev(q_raw, "q_raw")
    dt = q_raw.dtype
    if dt not in _DTYPES:
        raise ValueError("q_raw must be bf16 or fp32")
    B, H, dk = g.shape
    dv = state.shape[-1]
    for t, name, d in ((q_raw, "q_raw", dk), (k_raw, "k_raw", dk), (v_raw, "v_raw", dv)):
        _dev(t, name, dt, (B, H * d))
    for t, name, d in ((w_q, "w_q", dk), (w_k, "w_k", dk), (w_v, "w_v", dv)):
        _dev(t, name, dt, (H * d, 4))
    for t, name, d in ((conv_q, "conv_q", dk), (conv_k, "conv_k", dk), (conv_v, "conv_v", dv)):
        _dev(t, name, dt, (B, 3, H * d))
    _dev(g, "g", torch.float32, (B, H, dk))
    _dev(beta, "beta", torch.float32, (B, H))
    _dev(state, "state", torch.float32, (B, H, dk, dv))
    if out is not None:
        out_dtype = out.dtype
    if out_dtype not in _DTYPES:
        raise ValueError("out_dtype must be bf16 or fp32")
    o = out if out is not None else torch.empty((B, H, dv), dtype=out_dtype, device=g.device)
    _dev(o, "out", out_dtype, (B, H, dv))
    sc = dk ** -0.5 if scale is None else float(scale)
    _check(library().kda_decode_step_conv(
        _ptr(q_raw), _ptr(k_raw), _ptr(v_raw), _ptr(w_q), _ptr(w_k), _ptr(w_v), _ptr(conv_q),
        _ptr(conv_k), _ptr(conv_v), float(l2_eps), _ptr(g), _ptr(beta), _ptr(state), B, H, dk,
        dv, sc, _ptr(o), _DTYPES[dt], _DTYPES[out_dtype], _stream(g)))
    return o


def gdn_decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                    beta: torch.Tensor, state: torch.Tensor, *, scale: Optional[float] = None,
                    out: Optional[torch.Tensor] = None,
                    out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """``decode_step`` with one decay per (sequence, head): g [B, H] fp32 (GDN's gate)."""
    return decode_step(q, k, v, g, beta, state, scale=scale, out=out, out_dtype=out_dtype,
                       _head_gate=True)


def decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                beta: torch.Tensor, state: torch.Tensor, *, scale: Optional[float] = None,
                out: Optional[torch.Tensor] = None,
                out_dtype: torch.dtype = torch.float32, _head_gate: bool = False) -> torch.Tensor:
    """One recurrent step; ``state`` [B, H, dk, dv] fp32 is updated in place.

    q, k, g: [B, H, dk]; v: [B, H, dv]; beta: [B, H].  Returns o [B, H, dv]
    (``out_dtype``, fp32 by default).
    """
    _dev(q, "q")
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError("q must be bf16 or fp32")
    B, H, dk = q.shape
    dv = v.shape[-1]
    _dev(k, "k", dt, (B, H, dk))
    _dev(v, "v", dt, (B, H, dv))
    _dev(g, "g", torch.float32, (B, H) if _head_gate else (B, H, dk))
    _dev(beta, "beta", torch.float32, (B, H))
    _dev(state, "state", torch.float32, (B, H, dk, dv))
    if out is not None:
        out_dtype = out.dtype
    if out_dtype not in _DTYPES:
        raise ValueError("out_dtype must be bf16 or fp32")
    o = out if out is not None else torch.empty((B, H, dv), dtype=out_dtype, device=q.device)
    _dev(o, "out", out_dtype, (B, H, dv))
    sc = dk ** -0.5 if scale is None else float(scale)
    fn = library().kda_gdn_decode_step if _head_gate else library().kda_decode_step
    _check(fn(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), B, H, dk, dv, sc, _ptr(o),
        _DTYPES[dt], _DTYPES[out_dtype], _stream(q)))
    return o
