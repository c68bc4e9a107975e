// kda_api.cpp -- the C ABI of libkda: host-side argument checks, then one or
// two kernel launches on the caller's stream.  No allocation, no host sync.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include "kda.h"
#include "kda_launch.h"

namespace {

thread_local char g_last_error[512] = "";

kda_status_t fail(kda_status_t st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

kda_status_t from_hip(hipError_t e, const char *what) {
    if (e == hipSuccess) return KDA_OK;
    if (e == hipErrorNotSupported) return fail(KDA_ERR_UNSUPPORTED, "%s: unsupported shape", what);
    return fail(KDA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool valid_dtype(kda_dtype_t d) { return d == KDA_DTYPE_F32 || d == KDA_DTYPE_BF16; }
bool head_dim_ok(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }
int vec_elems(kda_dtype_t) { return 4; }   // channels per lane of the conv kernel

}  // namespace

namespace {

// gate: 0 = g [T, H, dk], 1 = the fused bounded gate, 2 = g [T, H] (one decay per head)
kda::ChunkLauncher chunk_launcher(kda_dtype_t dtype, kda_dtype_t out_dtype, int gate = 0) {
    if (gate == 2)
        return dtype == KDA_DTYPE_F32       ? kda::launch_chunk_f32_gdn
               : out_dtype == KDA_DTYPE_F32 ? kda::launch_chunk_bf16_f32out_gdn
                                            : kda::launch_chunk_bf16_bf16out_gdn;
    if (gate == 1)
        return dtype == KDA_DTYPE_F32       ? kda::launch_chunk_f32_gz
               : out_dtype == KDA_DTYPE_F32 ? kda::launch_chunk_bf16_f32out_gz
                                            : kda::launch_chunk_bf16_bf16out_gz;
    return dtype == KDA_DTYPE_F32       ? kda::launch_chunk_f32
           : out_dtype == KDA_DTYPE_F32 ? kda::launch_chunk_bf16_f32out
                                        : kda::launch_chunk_bf16_bf16out;
}

// Shape checks shared by kda_chunk_fwd and its workspace query; returns the
// internal chunk size (> 0) or 0 after recording the failure.
int chunk_shape_check(const char *who, int64_t total_tokens, int32_t num_heads, int32_t dk,
                      int32_t dv, int32_t chunk_size, kda_dtype_t dtype, kda_dtype_t out_dtype,
                      kda_status_t *st) {
    *st = KDA_OK;
    if (total_tokens < 0 || num_heads < 1 || num_heads > 65535) {
        *st = fail(KDA_ERR_INVALID_ARG, "%s: bad sizes", who);
        return 0;
    }
    if (!valid_dtype(dtype) || !valid_dtype(out_dtype)) {
        *st = fail(KDA_ERR_INVALID_ARG, "%s: bad dtype", who);
        return 0;
    }
    if (dtype == KDA_DTYPE_F32 && out_dtype != KDA_DTYPE_F32) {
        *st = fail(KDA_ERR_UNSUPPORTED, "%s: fp32 inputs need an fp32 output", who);
        return 0;
    }
    if (!head_dim_ok(dk) || !head_dim_ok(dv)) {
        *st = fail(KDA_ERR_UNSUPPORTED, "%s: dk/dv not in {16,32,64,128}", who);
        return 0;
    }
    if (chunk_size != 16 && chunk_size != 32 && chunk_size != 64) {
        *st = fail(KDA_ERR_UNSUPPORTED, "%s: chunk_size not in {16,32,64}", who);
        return 0;
    }
    kda::ChunkArgs probe{};
    probe.heads = num_heads;
    probe.dk = dk;
    probe.dv = dv;
    probe.chunk = chunk_size;
    int c = 0;
    (void)chunk_launcher(dtype, out_dtype)(probe, nullptr, false, &c);
    if (c == 0) *st = fail(KDA_ERR_UNSUPPORTED, "%s: no kernel for dk=%d dv=%d", who, dk, dv);
    return c;
}

kda_status_t scratch_address(const char *who, float **out) {
    void *p = nullptr;
    const hipError_t e = kda::scratch_address(&p);
    if (e == hipErrorInvalidDevice)
        return fail(KDA_ERR_UNSUPPORTED, "%s: the current device is beyond the %d supported", who,
                    kda::kScratchMaxDevices);
    if (e != hipSuccess || !p)
        return fail(KDA_ERR_HIP, "%s: static scratch address: %s", who, hipGetErrorString(e));
    *out = static_cast<float *>(p);
    return KDA_OK;
}

// The checks and the launch shared by kda_chunk_fwd, kda_chunk_fwd_gated,
// kda_gdn_chunk_fwd and kda_chunk_fwd_noalloc; `gate` is g, the gate's
// pre-activation z, or the per-head g (mode 0, 1, 2 as for chunk_launcher).  With
// use_scratch the workspace is the static `scratch` of the current device.
kda_status_t chunk_checked_launch(const char *who, const kda::ChunkArgs &a, const void *gate,
                                  int mode, size_t workspace_bytes, kda_dtype_t dtype,
                                  kda_dtype_t out_dtype, void *stream, bool use_scratch = false) {
    const bool gated = mode == 1;
    if (a.total_tokens > 0 && (!a.q || !a.k || !a.v || !gate || !a.beta || !a.o))
        return fail(KDA_ERR_INVALID_ARG, "%s: NULL q/k/v/%s/beta/o", who, gated ? "z" : "g");
    if (a.num_seqs < 1) return fail(KDA_ERR_INVALID_ARG, "%s: bad sizes", who);
    if (!a.cu_seqlens && a.num_seqs != 1)
        return fail(KDA_ERR_INVALID_ARG, "%s: cu_seqlens NULL needs num_seqs == 1", who);
    if (!isfinite(a.scale)) return fail(KDA_ERR_INVALID_ARG, "%s: scale not finite", who);
    if (a.o && (a.o == a.q || a.o == a.k || a.o == a.v || a.o == gate ||
                a.o == (const void *)a.beta || a.o == (const void *)a.workspace ||
                (gated && a.o && (a.o == (const void *)a.a_log || a.o == (const void *)a.dt_bias))))
        return fail(KDA_ERR_INVALID_ARG, "%s: o aliases an input or the workspace", who);
    if (!(a.gate_lb <= 0.f)) return fail(KDA_ERR_INVALID_ARG, "%s: gate bound > 0 or NaN", who);
    if (a.gate_lb < -9.f) return fail(KDA_ERR_UNSUPPORTED, "%s: gate bound below -9", who);
    kda_status_t st;
    const int c = chunk_shape_check(who, a.total_tokens, a.heads, a.dk, a.dv, a.chunk, dtype,
                                    out_dtype, &st);
    if (c == 0) return st;
    if ((int64_t)a.num_seqs * a.heads * (a.dv / 16) > ((int64_t)1 << 28) ||
        a.total_tokens / c >= ((int64_t)1 << 31) - 1)   // tiles of the prep grid
        return fail(KDA_ERR_UNSUPPORTED, "%s: grid too large", who);
    const size_t need = kda::chunk_workspace_bytes(a.total_tokens, a.heads, c);
    kda::ChunkArgs run = a;
    if (use_scratch) {
        if (need > kda::kScratchBytes)
            return fail(KDA_ERR_UNSUPPORTED,
                        "%s: %lld tokens x %d heads need %zu bytes of scratch; the static "
                        "scratch holds %zu (at most %zu token-heads)",
                        who, (long long)a.total_tokens, a.heads, need, kda::kScratchBytes,
                        (kda::kScratchBytes - kda::kOrderBytes) / (2 * sizeof(float) * c));
        run.workspace = nullptr;
        if (a.total_tokens > 0) {
            const kda_status_t s2 = scratch_address(who, &run.workspace);
            if (s2 != KDA_OK) return s2;
        }
    } else if (a.total_tokens > 0 && (!a.workspace || workspace_bytes < need)) {
        return fail(KDA_ERR_WORKSPACE, "%s: workspace %s of %zu bytes, %zu needed", who,
                    a.workspace ? "" : "(NULL)", workspace_bytes, need);
    }
    int used = 0;
    return from_hip(chunk_launcher(dtype, out_dtype, mode)(run, (hipStream_t)stream, true, &used),
                    who);
}

kda_status_t decode_checked(const char *who, const void *q, const void *k, const void *v,
                            const float *g, const float *beta, float *state, int32_t batch,
                            int32_t num_heads, int32_t dk, int32_t dv, float scale, void *o,
                            kda_dtype_t dtype, kda_dtype_t out_dtype, bool head_gate,
                            void *stream) {
    if (batch > 0 && (!q || !k || !v || !g || !beta || !state || !o))
        return fail(KDA_ERR_INVALID_ARG, "%s: NULL pointer", who);
    if (batch < 0 || num_heads < 1) return fail(KDA_ERR_INVALID_ARG, "%s: bad sizes", who);
    if (!valid_dtype(dtype) || !valid_dtype(out_dtype))
        return fail(KDA_ERR_INVALID_ARG, "%s: bad dtype", who);
    if (dtype == KDA_DTYPE_F32 && out_dtype != KDA_DTYPE_F32)
        return fail(KDA_ERR_UNSUPPORTED, "%s: fp32 inputs need an fp32 output", who);
    if (!isfinite(scale)) return fail(KDA_ERR_INVALID_ARG, "%s: scale not finite", who);
    if (o && (o == q || o == k || o == v || o == (const void *)g || o == (const void *)beta ||
              o == (const void *)state))
        return fail(KDA_ERR_INVALID_ARG, "%s: o aliases an input", who);
    if (!head_dim_ok(dk) || !head_dim_ok(dv))
        return fail(KDA_ERR_UNSUPPORTED, "%s: dk/dv not in {16,32,64,128}", who);
    if ((int64_t)batch * num_heads > ((int64_t)1 << 31) - 1)
        return fail(KDA_ERR_UNSUPPORTED, "%s: grid too large", who);
    kda::DecodeArgs a{q, k, v, g, beta, state, batch, num_heads, dk, dv, scale, o,
                      out_dtype == KDA_DTYPE_F32, false, {}, head_gate};
    return from_hip(kda::launch_decode_step(a, dtype == KDA_DTYPE_BF16, (hipStream_t)stream), who);
}

}  // namespace

extern "C" {

KDA_API const char *kda_status_string(kda_status_t s) {
    switch (s) {
        case KDA_OK: return "ok";
        case KDA_ERR_INVALID_ARG: return "invalid argument";
        case KDA_ERR_UNSUPPORTED: return "unsupported shape, dtype or gate bound";
        case KDA_ERR_HIP: return "HIP runtime error";
        case KDA_ERR_WORKSPACE: return "workspace missing or too small";
    }
    return "unknown status";
}

KDA_API const char *kda_last_error(void) { return g_last_error; }

KDA_API int32_t kda_version(void) { return 10000; }

KDA_API kda_status_t kda_short_conv(const void *x, const void *weight, const void *bias,
                                    const int32_t *cu_seqlens, int32_t num_seqs,
                                    int64_t total_tokens, int32_t num_heads, int32_t head_dim,
                                    int32_t width, const void *conv_state_in, void *conv_state_out,
                                    int32_t apply_silu, int32_t l2_normalize, float l2_eps,
                                    kda_dtype_t dtype, void *y, void *stream) {
    g_last_error[0] = '\0';
    if (!weight || (total_tokens > 0 && (!x || !y)))
        return fail(KDA_ERR_INVALID_ARG, "kda_short_conv: NULL x/weight/y");
    if (num_seqs < 1 || total_tokens < 0 || num_heads < 1 || head_dim < 1)
        return fail(KDA_ERR_INVALID_ARG, "kda_short_conv: bad sizes");
    if (!cu_seqlens && num_seqs != 1)
        return fail(KDA_ERR_INVALID_ARG, "kda_short_conv: cu_seqlens NULL needs num_seqs == 1");
    if (!valid_dtype(dtype)) return fail(KDA_ERR_INVALID_ARG, "kda_short_conv: bad dtype");
    if (x && x == y) return fail(KDA_ERR_INVALID_ARG, "kda_short_conv: y aliases x");
    if (l2_normalize && !(l2_eps >= 0.f && isfinite(l2_eps)))
        return fail(KDA_ERR_INVALID_ARG, "kda_short_conv: l2_eps must be finite and >= 0");
    if (width < 1 || width > 4) return fail(KDA_ERR_UNSUPPORTED, "kda_short_conv: width not in 1..4");
    const int ve = vec_elems(dtype);
    if (head_dim % ve != 0)
        return fail(KDA_ERR_UNSUPPORTED, "kda_short_conv: head_dim not a multiple of %d", ve);
    if (l2_normalize) {
        const int lanes = head_dim / ve;
        if (lanes > 64 || (lanes & (lanes - 1)) != 0)
            return fail(KDA_ERR_UNSUPPORTED, "kda_short_conv: head_dim/%d must be a power of two <= 64", ve);
    }
    if ((int64_t)num_heads * head_dim > (int64_t)1 << 30 || total_tokens > ((int64_t)1 << 40))
        return fail(KDA_ERR_UNSUPPORTED, "kda_short_conv: size too large");
    kda::ConvArgs a{x, weight, bias, cu_seqlens, num_seqs, total_tokens, num_heads, head_dim,
                    width, conv_state_in, conv_state_out, apply_silu, l2_normalize, l2_eps, y};
    return from_hip(kda::launch_short_conv(a, dtype == KDA_DTYPE_BF16, (hipStream_t)stream),
                    "kda_short_conv");
}

KDA_API kda_status_t kda_chunk_fwd_workspace_size(int64_t total_tokens, int32_t num_heads,
                                                  int32_t dk, int32_t dv, int32_t chunk_size,
                                                  kda_dtype_t dtype, kda_dtype_t out_dtype,
                                                  size_t *bytes) {
    g_last_error[0] = '\0';
    if (!bytes) return fail(KDA_ERR_INVALID_ARG, "kda_chunk_fwd_workspace_size: NULL bytes");
    kda_status_t st;
    const int c = chunk_shape_check("kda_chunk_fwd_workspace_size", total_tokens, num_heads, dk,
                                    dv, chunk_size, dtype, out_dtype, &st);
    if (c == 0) return st;
    *bytes = kda::chunk_workspace_bytes(total_tokens, num_heads, c);
    return KDA_OK;
}

KDA_API kda_status_t kda_chunk_fwd(const void *q, const void *k, const void *v, const float *g,
                                   const float *beta, const int32_t *cu_seqlens, int32_t num_seqs,
                                   int64_t total_tokens, int32_t num_heads, int32_t dk, int32_t dv,
                                   int32_t chunk_size, float scale, float gate_lower_bound,
                                   const float *initial_state, float *final_state, void *o,
                                   void *workspace, size_t workspace_bytes, kda_dtype_t dtype,
                                   kda_dtype_t out_dtype, void *stream) {
    g_last_error[0] = '\0';
    const kda::ChunkArgs a{q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens, num_heads, dk,
                           dv, chunk_size, scale, gate_lower_bound, initial_state, final_state, o,
                           (float *)workspace, nullptr, nullptr, nullptr};
    return chunk_checked_launch("kda_chunk_fwd", a, g, 0, workspace_bytes, dtype, out_dtype,
                                stream);
}

KDA_API kda_status_t kda_chunk_fwd_phases(const void *q, const void *k, const void *v,
                                          const float *g, const float *beta,
                                          const int32_t *cu_seqlens, int32_t num_seqs,
                                          int64_t total_tokens, int32_t num_heads, int32_t dk,
                                          int32_t dv, int32_t chunk_size, float scale,
                                          float gate_lower_bound, const float *initial_state,
                                          float *final_state, void *o, void *workspace,
                                          size_t workspace_bytes, kda_dtype_t dtype,
                                          kda_dtype_t out_dtype, int32_t phases, void *stream) {
    g_last_error[0] = '\0';
    if (phases != KDA_PHASE_PREP && phases != KDA_PHASE_WALK && phases != KDA_PHASE_ALL)
        return fail(KDA_ERR_INVALID_ARG, "kda_chunk_fwd_phases: phases %d not 1, 2 or 3", phases);
    kda::ChunkArgs a{q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens, num_heads, dk,
                     dv, chunk_size, scale, gate_lower_bound, initial_state, final_state, o,
                     (float *)workspace, nullptr, nullptr, nullptr};
    a.phases = phases;
    return chunk_checked_launch("kda_chunk_fwd_phases", a, g, 0, workspace_bytes, dtype,
                                out_dtype, stream);
}

KDA_API kda_status_t kda_chunk_fwd_noalloc(const void *q, const void *k, const void *v,
                                           const float *g, const float *beta,
                                           const int32_t *cu_seqlens, int32_t num_seqs,
                                           int64_t total_tokens, int32_t num_heads, int32_t dk,
                                           int32_t dv, int32_t chunk_size, float scale,
                                           float gate_lower_bound, const float *initial_state,
                                           float *final_state, void *o, kda_dtype_t dtype,
                                           kda_dtype_t out_dtype, void *stream) {
    g_last_error[0] = '\0';
    const kda::ChunkArgs a{q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens, num_heads, dk,
                           dv, chunk_size, scale, gate_lower_bound, initial_state, final_state, o,
                           nullptr, nullptr, nullptr, nullptr};
    return chunk_checked_launch("kda_chunk_fwd_noalloc", a, g, 0, 0, dtype, out_dtype, stream,
                                true);
}

KDA_API kda_status_t kda_gdn_chunk_fwd(const void *q, const void *k, const void *v, const float *g,
                                       const float *beta, const int32_t *cu_seqlens,
                                       int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                                       int32_t dk, int32_t dv, int32_t chunk_size, float scale,
                                       float gate_lower_bound, const float *initial_state,
                                       float *final_state, void *o, void *workspace,
                                       size_t workspace_bytes, kda_dtype_t dtype,
                                       kda_dtype_t out_dtype, void *stream) {
    g_last_error[0] = '\0';
    const kda::ChunkArgs a{q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens, num_heads, dk,
                           dv, chunk_size, scale, gate_lower_bound, initial_state, final_state, o,
                           (float *)workspace, nullptr, nullptr, nullptr};
    return chunk_checked_launch("kda_gdn_chunk_fwd", a, g, 2, workspace_bytes, dtype, out_dtype,
                                stream);
}

KDA_API kda_status_t kda_chunk_fwd_gated(const void *q, const void *k, const void *v,
                                         const void *z, const float *a_log, const float *dt_bias,
                                         float lower_bound, const float *beta,
                                         const int32_t *cu_seqlens, int32_t num_seqs,
                                         int64_t total_tokens, int32_t num_heads, int32_t dk,
                                         int32_t dv, int32_t chunk_size, float scale,
                                         const float *initial_state, float *final_state, void *o,
                                         void *workspace, size_t workspace_bytes,
                                         kda_dtype_t dtype, kda_dtype_t out_dtype, void *stream) {
    g_last_error[0] = '\0';
    const kda::ChunkArgs a{q, k, v, nullptr, beta, cu_seqlens, num_seqs, total_tokens, num_heads,
                           dk, dv, chunk_size, scale, lower_bound, initial_state, final_state, o,
                           (float *)workspace, z, a_log, dt_bias};
    return chunk_checked_launch("kda_chunk_fwd_gated", a, z, 1, workspace_bytes, dtype,
                                out_dtype, stream);
}

KDA_API kda_status_t kda_output_norm_gate(const void *o, const void *gate, const float *weight,
                                          float eps, int64_t rows, int32_t dv,
                                          kda_dtype_t o_dtype, kda_dtype_t dtype, void *y,
                                          void *stream) {
    g_last_error[0] = '\0';
    if (rows > 0 && (!o || !gate || !y))
        return fail(KDA_ERR_INVALID_ARG, "kda_output_norm_gate: NULL o/gate/y");
    if (rows < 0) return fail(KDA_ERR_INVALID_ARG, "kda_output_norm_gate: bad sizes");
    if (!valid_dtype(o_dtype) || !valid_dtype(dtype))
        return fail(KDA_ERR_INVALID_ARG, "kda_output_norm_gate: bad dtype");
    if (!(eps >= 0.f && isfinite(eps)))
        return fail(KDA_ERR_INVALID_ARG, "kda_output_norm_gate: eps negative or not finite");
    if (o && o == y && o_dtype != dtype)
        return fail(KDA_ERR_INVALID_ARG, "kda_output_norm_gate: y aliases o of another dtype");
    if (y && (y == (const void *)weight))
        return fail(KDA_ERR_INVALID_ARG, "kda_output_norm_gate: y aliases the weight");
    if (!head_dim_ok(dv)) return fail(KDA_ERR_UNSUPPORTED, "kda_output_norm_gate: dv not in {16,32,64,128}");
    if (o_dtype == KDA_DTYPE_BF16 && dtype != KDA_DTYPE_BF16)
        return fail(KDA_ERR_UNSUPPORTED, "kda_output_norm_gate: bf16 o needs a bf16 gate and y");
    if (rows > ((int64_t)1 << 40) || (rows * (dv / 4) + 255) / 256 > ((int64_t)1 << 31) - 1)
        return fail(KDA_ERR_UNSUPPORTED, "kda_output_norm_gate: grid too large");
    const kda::NormGateArgs a{o, gate, weight, eps, rows, dv, y};
    return from_hip(kda::launch_norm_gate(a, o_dtype == KDA_DTYPE_BF16, dtype == KDA_DTYPE_BF16,
                                          (hipStream_t)stream),
                    "kda_output_norm_gate");
}

KDA_API kda_status_t kda_decode_step(const void *q, const void *k, const void *v, const float *g,
                                     const float *beta, float *state, int32_t batch,
                                     int32_t num_heads, int32_t dk, int32_t dv, float scale,
                                     void *o, kda_dtype_t dtype, kda_dtype_t out_dtype,
                                     void *stream) {
    g_last_error[0] = '\0';
    return decode_checked("kda_decode_step", q, k, v, g, beta, state, batch, num_heads, dk, dv,
                          scale, o, dtype, out_dtype, false, stream);
}

KDA_API kda_status_t kda_gdn_decode_step(const void *q, const void *k, const void *v,
                                         const float *g, const float *beta, float *state,
                                         int32_t batch, int32_t num_heads, int32_t dk, int32_t dv,
                                         float scale, void *o, kda_dtype_t dtype,
                                         kda_dtype_t out_dtype, void *stream) {
    g_last_error[0] = '\0';
    return decode_checked("kda_gdn_decode_step", q, k, v, g, beta, state, batch, num_heads, dk,
                          dv, scale, o, dtype, out_dtype, true, stream);
}

KDA_API kda_status_t kda_decode_step_conv(const void *q_raw, const void *k_raw, const void *v_raw,
                                          const void *w_q, const void *w_k, const void *w_v,
                                          void *conv_q, void *conv_k, void *conv_v, float l2_eps,
                                          const float *g, const float *beta, float *state,
                                          int32_t batch, int32_t num_heads, int32_t dk, int32_t dv,
                                          float scale, void *o, kda_dtype_t dtype,
                                          kda_dtype_t out_dtype, void *stream) {
    g_last_error[0] = '\0';
    const char *who = "kda_decode_step_conv";
    if (batch > 0 && (!q_raw || !k_raw || !v_raw || !w_q || !w_k || !w_v || !conv_q ||
                      !conv_k || !conv_v || !g || !beta || !state || !o))
        return fail(KDA_ERR_INVALID_ARG, "%s: NULL pointer", who);
    if (batch < 0 || num_heads < 1) return fail(KDA_ERR_INVALID_ARG, "%s: bad sizes", who);
    if (!valid_dtype(dtype) || !valid_dtype(out_dtype))
        return fail(KDA_ERR_INVALID_ARG, "%s: bad dtype", who);
    if (dtype == KDA_DTYPE_F32 && out_dtype != KDA_DTYPE_F32)
        return fail(KDA_ERR_UNSUPPORTED, "%s: fp32 inputs need an fp32 output", who);
    if (!isfinite(scale)) return fail(KDA_ERR_INVALID_ARG, "%s: scale not finite", who);
    if (!(l2_eps >= 0.f && isfinite(l2_eps)))
        return fail(KDA_ERR_INVALID_ARG, "%s: l2_eps negative or not finite", who);
    const void *ins[] = {q_raw, k_raw, v_raw, w_q, w_k, w_v, conv_q, conv_k, conv_v, g, beta,
                         state};
    for (const void *p : ins)
        if (o && o == p) return fail(KDA_ERR_INVALID_ARG, "%s: o aliases an input", who);
    if (batch > 0 && (conv_q == conv_k || conv_q == conv_v || conv_k == conv_v))
        return fail(KDA_ERR_INVALID_ARG, "%s: the three conv caches must be distinct", who);
    if (!head_dim_ok(dk) || !head_dim_ok(dv))
        return fail(KDA_ERR_UNSUPPORTED, "%s: dk/dv not in {16,32,64,128}", who);
    if ((int64_t)batch * num_heads > ((int64_t)1 << 31) - 1)
        return fail(KDA_ERR_UNSUPPORTED, "%s: grid too large", who);
    kda::DecodeArgs a{nullptr, nullptr, nullptr, g, beta, state, batch, num_heads, dk, dv, scale,
                      o, out_dtype == KDA_DTYPE_F32, true,
                      kda::DecodeConvIn{q_raw, k_raw, v_raw, w_q, w_k, w_v, conv_q, conv_k,
                                        conv_v, l2_eps, num_heads},
                      false};
    return from_hip(kda::launch_decode_step(a, dtype == KDA_DTYPE_BF16, (hipStream_t)stream), who);
}

}  // extern "C"
