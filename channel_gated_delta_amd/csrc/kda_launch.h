// kda_launch.h -- internal launchers behind the C ABI (host code; not exported).
#pragma once

#include <atomic>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct ConvArgs {
    const void *x, *weight, *bias;
    const int32_t *cu_seqlens;
    int32_t num_seqs;
    int64_t total_tokens;
    int32_t heads, head_dim, width;
    const void *state_in;
    void *state_out;
    int32_t silu, l2;
    float eps;
    void *y;
};

struct ChunkArgs {
    const void *q, *k, *v;
    const float *g, *beta;
    const int32_t *cu_seqlens;
    int32_t num_seqs;
    int64_t total_tokens;
    int32_t heads, dk, dv, chunk;
    float scale, gate_lb;
    const float *h0;
    float *hT;
    void *o;        // output dtype chosen by the launcher called
    float *workspace;   // 2 * total_tokens * heads * C floats (C = the internal chunk)
    // fused bounded gate (the *_gz launchers): pre-activation z [T, H, dk] in the
    // activation dtype, A_log [H] and dt_bias [H, dk] (NULL = 0); gate_lb is its bound
    const void *gz;
    const float *a_log, *dt_bias;
    // which launches to enqueue: 1 the prep (a packed batch's walking order, then
    // Tb / P into the workspace), 2 the walk over the chunks, 3 both
    int32_t phases = 3;
};

// Packed batches of up to kOrderMaxSeqs sequences run their longest sequences
// first: the state kernel's dispatch order, order[rank] = sequence, sits after
// the Tb and P rows in the workspace.
constexpr int kOrderMaxSeqs = 1024;
constexpr size_t kOrderBytes = (size_t)kOrderMaxSeqs * sizeof(int32_t);

// Workspace of the chunk prefill for internal chunk c: Tb and scale * P rows and
// the dispatch order (nothing without tokens).
inline size_t chunk_workspace_bytes(int64_t total_tokens, int32_t heads, int c) {
    if (total_tokens <= 0) return 0;
    return (size_t)2 * (size_t)total_tokens * (size_t)heads * (size_t)c * sizeof(float) +
           kOrderBytes;
}

// The library's static device scratch (kda_scratch.hip), the workspace of
// kda_chunk_fwd_noalloc: its size, and its address on the calling thread's
// current device (looked up once per device; hipErrorInvalidDevice for a device
// index at or beyond kScratchMaxDevices).
constexpr size_t kScratchBytes = ((size_t)64 << 20) + kOrderBytes;
constexpr int kScratchMaxDevices = 64;
hipError_t scratch_address(void **ptr);

// Compute units of the current device, looked up once per device (the layout
// choice of the chunk kernels depends on it; both layouts give the same results,
// so a failed lookup falls back to 256, the count of gfx950's MI355X).
inline int device_cus() {
    static std::atomic<int> cache[kScratchMaxDevices];   // 0: not looked up yet
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchMaxDevices) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

struct NormGateArgs {
    const void *o, *gate;
    const float *weight;   // [dv] or NULL
    float eps;
    int64_t rows;          // tokens * heads
    int32_t dv;
    void *y;
};

// Conv inputs of the fused decode step: this token's raw projections, the
// width-4 conv weights and the conv caches (the last three raw inputs of every
// sequence, oldest first; updated in place).
struct DecodeConvIn {
    const void *xq, *xk, *xv;   // [B, H*dk], [B, H*dk], [B, H*dv]
    const void *wq, *wk, *wv;   // [H*dk, 4], [H*dk, 4], [H*dv, 4]
    void *cq, *ck, *cv;         // [B, 3, H*dk], [B, 3, H*dk], [B, 3, H*dv]
    float eps;                  // of the q / k L2 normalisation
    int32_t heads;
};

struct DecodeArgs {
    const void *q, *k, *v;      // unused with the conv
    const float *g, *beta;
    float *state;
    int32_t batch, heads, dk, dv;
    float scale;
    void *o;
    bool out_f32;   // o in fp32 (else in the input dtype)
    bool with_conv;
    DecodeConvIn conv;
    bool head_gate;  // g is [B, H]: one decay per (sequence, head) (GDN's gate)
};

// Each launcher returns hipSuccess, hipErrorNotSupported for a shape it has no
// kernel for (checked before anything is enqueued), or the launch error.
hipError_t launch_short_conv(const ConvArgs &a, bool bf16, hipStream_t s);
// Chunk prefill per dtype: *chunk_used receives the internal chunk size (0 if the
// shape is not supported); with launch == false nothing is enqueued.
hipError_t launch_chunk_bf16_f32out(const ChunkArgs &a, hipStream_t s, bool launch, int *chunk_used);
hipError_t launch_chunk_bf16_bf16out(const ChunkArgs &a, hipStream_t s, bool launch, int *chunk_used);
hipError_t launch_chunk_f32(const ChunkArgs &a, hipStream_t s, bool launch, int *chunk_used);
// The same with the fused bounded gate (reads gz, a_log, dt_bias instead of g).
hipError_t launch_chunk_bf16_f32out_gz(const ChunkArgs &a, hipStream_t s, bool launch, int *chunk_used);
hipError_t launch_chunk_bf16_bf16out_gz(const ChunkArgs &a, hipStream_t s, bool launch, int *chunk_used);
hipError_t launch_chunk_f32_gz(const ChunkArgs &a, hipStream_t s, bool launch, int *chunk_used);
// The same with one decay per (token, head): ChunkArgs::g is [T, H] (GDN's gate).
hipError_t launch_chunk_bf16_f32out_gdn(const ChunkArgs &a, hipStream_t s, bool launch, int *chunk_used);
hipError_t launch_chunk_bf16_bf16out_gdn(const ChunkArgs &a, hipStream_t s, bool launch, int *chunk_used);
hipError_t launch_chunk_f32_gdn(const ChunkArgs &a, hipStream_t s, bool launch, int *chunk_used);
typedef hipError_t (*ChunkLauncher)(const ChunkArgs &, hipStream_t, bool, int *);
hipError_t launch_decode_step(const DecodeArgs &a, bool bf16, hipStream_t s);
// o_bf16: o is bf16 (needs bf16 gate / y); y_bf16: gate and y are bf16.
hipError_t launch_norm_gate(const NormGateArgs &a, bool o_bf16, bool y_bf16, hipStream_t s);

}  // namespace kda
