// kda_chunk_dispatch.cuh -- host-side choice of the chunk kernel instantiation
// (value-slice width BV, internal chunk) for one operand dtype.
#pragma once

#include "kda_chunk.cuh"
#include "kda_launch.h"

namespace kda {
namespace chunk_detail {

template <class T, class TO, int DK, int BV, int C>
hipError_t run(const ChunkArgs &a, hipStream_t s) {
    if constexpr (!ChunkCfg<T, DK, BV, C>::kFits) {
        return hipErrorNotSupported;
    } else {
        const int units = a.num_seqs * a.heads;
        const int nslice = a.dv / BV;
        if (units == 0) return hipSuccess;
        const unsigned grid = (unsigned)(((units + 7) / 8) * 8 * nslice);
        hipLaunchKernelGGL((chunk_kernel<T, TO, DK, BV, C>), dim3(grid), dim3(256), 0, s,
                           (const T *)a.q, (const T *)a.k, (const T *)a.v, a.g, a.beta,
                           a.cu_seqlens, a.total_tokens, a.heads, a.dv, a.scale, a.h0, a.hT,
                           (TO *)a.o, units, nslice);
        return hipGetLastError();
    }
}

// Value-slice width.  Wave w of a workgroup owns state columns [16w, 16w+16) of
// its slice, so a 64-column slice keeps all four waves busy in the state chain;
// the key-side work (decay factors, Gram matrices, inverse) is repeated once per
// slice.  LDS use does not depend on the slice width.  64 columns when dv allows,
// else 32, else 16.
template <class T, int DK, int C>
constexpr int pick_bv(int dv) {
#ifdef KDA_CHUNK_BV
    if (dv % KDA_CHUNK_BV == 0 && ChunkCfg<T, DK, KDA_CHUNK_BV, C>::kFits) return KDA_CHUNK_BV;
#endif
    if (!ChunkCfg<T, DK, 16, C>::kFits) return 0;
    if (dv % 64 == 0) return 64;
    if (dv % 32 == 0) return 32;
    return dv % 16 == 0 ? 16 : 0;
}

template <class T, class TO, int DK, int C>
hipError_t run_c(const ChunkArgs &a, hipStream_t s, bool launch, bool *ok) {
    const int bv = pick_bv<T, DK, C>(a.dv);
    *ok = bv != 0;
    if (!launch || !*ok) return *ok ? hipSuccess : hipErrorNotSupported;
    switch (bv) {
        case 64: return run<T, TO, DK, 64, C>(a, s);
        case 32: return run<T, TO, DK, 32, C>(a, s);
        default: return run<T, TO, DK, 16, C>(a, s);
    }
}

// Internal chunk: the largest of 64, 32, 16 that does not exceed the requested
// size, fits in LDS and is not above the preferred maximum (KDA_CHUNK_MAX).
#ifndef KDA_CHUNK_MAX
#define KDA_CHUNK_MAX 64
#endif
template <class T, class TO, int DK>
hipError_t run_dk(const ChunkArgs &a, hipStream_t s, bool launch, bool *ok) {
    *ok = false;
    hipError_t e = hipErrorNotSupported;
    if (a.chunk >= 64 && KDA_CHUNK_MAX >= 64) {
        e = run_c<T, TO, DK, 64>(a, s, launch, ok);
        if (*ok) return e;
    }
    if (a.chunk >= 32 && KDA_CHUNK_MAX >= 32) {
        e = run_c<T, TO, DK, 32>(a, s, launch, ok);
        if (*ok) return e;
    }
    if (a.chunk >= 16) {
        e = run_c<T, TO, DK, 16>(a, s, launch, ok);
        if (*ok) return e;
    }
    return hipErrorNotSupported;
}

template <class T, class TO>
hipError_t dispatch(const ChunkArgs &a, hipStream_t s, bool launch, bool *ok) {
    *ok = false;
    if (a.dv != 16 && a.dv != 32 && a.dv != 64 && a.dv != 128) return hipErrorNotSupported;
    switch (a.dk) {
        case 16: return run_dk<T, TO, 16>(a, s, launch, ok);
        case 32: return run_dk<T, TO, 32>(a, s, launch, ok);
        case 64: return run_dk<T, TO, 64>(a, s, launch, ok);
        case 128: return run_dk<T, TO, 128>(a, s, launch, ok);
    }
    return hipErrorNotSupported;
}

}  // namespace chunk_detail
}  // namespace kda
