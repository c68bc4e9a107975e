// kda_chunk_dispatch.cuh -- host-side choice of the chunk kernel instantiations
// (value-slice width BV; the internal chunk is 16 tokens) for one operand dtype, and the two
// launches: the parallel prep kernel (Tb, scale * P for every chunk and head)
// followed by the sequential state kernel.
#pragma once

#include "kda_chunk_prep.cuh"
#include "kda_chunk_state.cuh"
#include "kda_launch.h"

namespace kda {
namespace chunk_detail {

template <class T, int DK, int BV, int C>
constexpr bool fits() {
    return PrepCfg<T, DK, C>::kFits && StateCfg<T, DK, BV, C>::kFits;
}

// Value-slice width.  Wave w of a state workgroup owns state columns [16w, 16w+16)
// of its slice; the chunk-operand work (the producers' loads and exponentials)
// is repeated once per slice.  A workgroup's step time is set by its chain of
// dependent chunk steps, so while the grid fits the GPU's CUs, narrower slices
// (64 columns, one consumer wave per SIMD) finish sooner.  Once there are more
// workgroups than CUs the work is throughput-bound: one workgroup per head with
// all 128 columns (two consumer waves per SIMD, producers shared) then does a
// head's work for one set of producer work.  Else 64 columns when dv allows,
// else 32, else 16.
inline int pick_bv(int dv, int dk, int64_t units) {
#ifdef KDA_CHUNK_BV
    if (dv % KDA_CHUNK_BV == 0) return KDA_CHUNK_BV;
#endif
    if (dv == 128 && dk == 128 && units * 2 > device_cus()) return 128;
    return dv % 64 == 0 ? 64 : (dv % 32 == 0 ? 32 : 16);
}

// Internal chunk: 16 tokens for every requested chunk size (0 when the working
// sets do not fit).  The result does not depend on the chunking beyond rounding.
template <class T, int DK>
int pick_chunk(int) {
    return fits<T, DK, 64, kChunk>() ? kChunk : 0;
}

template <class T, class TO, int DK, int BV, int C, int GM>
hipError_t run(const ChunkArgs &a, hipStream_t s) {
    if constexpr (!fits<T, DK, BV, C>()) {
        return hipErrorNotSupported;
    } else {
        float *tb = a.workspace;
        const GateSrc gs{a.g, a.gz, a.a_log, a.dt_bias, a.gate_lb};
        float *pm = tb ? tb + (size_t)a.total_tokens * a.heads * C : nullptr;
        int32_t *order = nullptr;
        if (a.total_tokens > 0 && a.cu_seqlens && a.num_seqs > 1 && a.num_seqs <= kOrderMaxSeqs)
            order = reinterpret_cast<int32_t *>(pm + (size_t)a.total_tokens * a.heads * C);
        if (order && (a.phases & 1)) {
            hipLaunchKernelGGL(seq_order_kernel<kOrderMaxSeqs>,
                               dim3((unsigned)((a.num_seqs + 255) / 256)),
                               dim3(256), 0, s, a.cu_seqlens, a.num_seqs, a.total_tokens, order);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        if (a.total_tokens > 0 && (a.phases & 1)) {
            const int64_t ntiles = (a.total_tokens + C - 1) / C;
            if constexpr (std::is_same<T, bf16>::value && DK % 32 == 0) {
                // one wave per (tile, head), four per workgroup
                const int64_t units = ntiles * a.heads;
                hipLaunchKernelGGL((chunk_prep16_kernel<DK, GM>), dim3((unsigned)((units + 3) / 4)),
                                   dim3(256), 0, s, (const bf16 *)a.q, (const bf16 *)a.k, gs,
                                   a.beta, a.cu_seqlens, a.num_seqs, a.total_tokens, a.heads,
                                   a.scale, units, tb, pm);
            } else {
                const dim3 g1((unsigned)ntiles, (unsigned)a.heads);
                hipLaunchKernelGGL((chunk_prep_kernel<T, DK, C, GM>), g1, dim3(256), 0, s,
                                   (const T *)a.q, (const T *)a.k, gs, a.beta, a.cu_seqlens,
                                   a.num_seqs, a.total_tokens, a.heads, a.scale, tb, pm);
            }
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        if (!(a.phases & 2)) return hipSuccess;
        // The state kernel also runs without tokens: it writes h0 (or zeros) to hT.
        const int units = a.num_seqs * a.heads;
        const int nslice = a.dv / BV;
        const unsigned g2 = (unsigned)(((units + 7) / 8) * 8 * nslice);
        hipLaunchKernelGGL((chunk_state_kernel<T, TO, DK, BV, C, GM>), dim3(g2),
                           dim3(StateCfg<T, DK, BV, C>::NT), 0, s,
                           (const T *)a.q, (const T *)a.k, (const T *)a.v, gs, tb, pm,
                           a.cu_seqlens, a.total_tokens, a.heads, a.dv, a.scale, a.h0, a.hT,
                           (TO *)a.o, units, nslice, order);
        return hipGetLastError();
    }
}

template <class T, class TO, int DK, int C, int GM>
hipError_t run_bv(const ChunkArgs &a, hipStream_t s) {
    switch (pick_bv(a.dv, DK, (int64_t)a.num_seqs * a.heads)) {
        case 128:
            if constexpr (DK == 128) return run<T, TO, DK, 128, C, GM>(a, s);
            return hipErrorNotSupported;
        case 64: return run<T, TO, DK, 64, C, GM>(a, s);
        case 32: return run<T, TO, DK, 32, C, GM>(a, s);
        default: return run<T, TO, DK, 16, C, GM>(a, s);
    }
}

template <class T, class TO, int DK, int GM>
hipError_t run_dk(const ChunkArgs &a, hipStream_t s, bool launch, int *chunk_used) {
    const int c = pick_chunk<T, DK>(a.chunk);
    *chunk_used = c;
    if (c == 0) return hipErrorNotSupported;
    if (!launch) return hipSuccess;
    return run_bv<T, TO, DK, kChunk, GM>(a, s);
}

// GM: the gate mode (kGatePlain, kGateFused: ChunkArgs::gz and friends, kGateHead: g [T, H]).
template <class T, class TO, int GM>
hipError_t dispatch(const ChunkArgs &a, hipStream_t s, bool launch, int *chunk_used) {
    *chunk_used = 0;
    if (a.dv != 16 && a.dv != 32 && a.dv != 64 && a.dv != 128) return hipErrorNotSupported;
    switch (a.dk) {
        case 16: return run_dk<T, TO, 16, GM>(a, s, launch, chunk_used);
        case 32: return run_dk<T, TO, 32, GM>(a, s, launch, chunk_used);
        case 64: return run_dk<T, TO, 64, GM>(a, s, launch, chunk_used);
        case 128: return run_dk<T, TO, 128, GM>(a, s, launch, chunk_used);
    }
    return hipErrorNotSupported;
}

}  // namespace chunk_detail
}  // namespace kda
