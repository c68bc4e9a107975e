// kda_device.cuh -- device-side building blocks shared by the KDA kernels:
// element types, vector loads, wave reductions and 16x16 MFMA tile fragments
// for CDNA4 (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

// One 16-byte vector of T (8 bf16 or 4 fp32).
template <class T> struct Vec16;
template <> struct Vec16<bf16> { static constexpr int n = 8; typedef bf16x8 type; };
template <> struct Vec16<float> { static constexpr int n = 4; typedef f32x4 type; };

template <class T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// 2^x on the transcendental unit (v_exp_f32); the argument is clamped so the
// result stays finite (2^126 < FLT_MAX).
__device__ __forceinline__ float exp2_clamped(float x) {
    return __builtin_amdgcn_exp2f(fminf(x, 126.0f));
}

// 2^x for x <= 0 (the result is in [0, 1]; no clamp needed).
__device__ __forceinline__ float exp2_nonpos(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup barrier that orders LDS accesses only.  Global loads and stores in
// flight stay in flight: __syncthreads() would also wait for them, because one
// counter tracks both global loads and stores, which defeats loads issued ahead
// of their use.  Use only where no global-memory ordering between waves is needed.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------------------
// Cross-lane sums without the LDS: DPP moves inside a row of 16 lanes
// (quad_perm [1,0,3,2] and [2,3,0,1] pair lanes l^1 and l^2; row_half_mirror
// pairs quad 0 with quad 1 of each 8-lane half, row_mirror the two halves of a
// row) and the gfx950 permlane swaps across rows (16-lane rows swapped in pairs,
// 32-lane halves swapped).  Every lane of a group ends with the same sum.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) { return __uint_as_float(dpp_mov<CTRL>(__float_as_uint(v))); }
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
    const uint64_t u = __double_as_longlong(v);
    const uint64_t lo = dpp_mov<CTRL>((uint32_t)u), hi = dpp_mov<CTRL>((uint32_t)(u >> 32));
    return __longlong_as_double((long long)(lo | (hi << 32)));
}
// (row pair) swap: element 0 holds this lane's value for even rows / the even
// row's for odd rows, element 1 the odd row's; their sum is the pair's sum.
__device__ __forceinline__ float rowpair_sum(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float halves_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ double rowpair_sum(double v) {
    const uint64_t u = __double_as_longlong(v);
    const auto a = __builtin_amdgcn_permlane16_swap((uint32_t)u, (uint32_t)u, false, false);
    const auto b = __builtin_amdgcn_permlane16_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
    return __longlong_as_double((long long)(a[0] | ((uint64_t)b[0] << 32))) +
           __longlong_as_double((long long)(a[1] | ((uint64_t)b[1] << 32)));
}
__device__ __forceinline__ double halves_sum(double v) {
    const uint64_t u = __double_as_longlong(v);
    const auto a = __builtin_amdgcn_permlane32_swap((uint32_t)u, (uint32_t)u, false, false);
    const auto b = __builtin_amdgcn_permlane32_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
    return __longlong_as_double((long long)(a[0] | ((uint64_t)b[0] << 32))) +
           __longlong_as_double((long long)(a[1] | ((uint64_t)b[1] << 32)));
}

// Sum over aligned groups of `width` consecutive lanes (width a power of two <= 64).
template <int width>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (width >= 2) v += dpp_f<0xB1>(v);
    if constexpr (width >= 4) v += dpp_f<0x4E>(v);
    if constexpr (width >= 8) v += dpp_f<0x141>(v);
    if constexpr (width >= 16) v += dpp_f<0x140>(v);
    if constexpr (width >= 32) v = rowpair_sum(v);
    if constexpr (width >= 64) v = halves_sum(v);
    return v;
}
template <int width>
__device__ __forceinline__ double group_sum(double v) {
    if constexpr (width >= 2) v += dpp_d<0xB1>(v);
    if constexpr (width >= 4) v += dpp_d<0x4E>(v);
    if constexpr (width >= 8) v += dpp_d<0x141>(v);
    if constexpr (width >= 16) v += dpp_d<0x140>(v);
    if constexpr (width >= 32) v = rowpair_sum(v);
    if constexpr (width >= 64) v = halves_sum(v);
    return v;
}

// Inclusive prefix and total over the four 16-lane rows of a wave, lane by lane
// (row r of the result holds a_0 + .. + a_r of the same lane index).
__device__ __forceinline__ void rows4_prefix(float a, int row, float &incl, float &total) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false, false);
    const float p0 = __uint_as_float(p[0]), pair = p0 + __uint_as_float(p[1]);
    const float x = (row & 1) ? a + p0 : a;
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(pair), __float_as_uint(pair), false, false);
    const float q0 = __uint_as_float(q[0]);
    incl = row >= 2 ? x + q0 : x;
    total = q0 + __uint_as_float(q[1]);
}

// ---------------------------------------------------------------------------
// 16x16 MFMA tiles.
//
// A tile product D(16x16) += A(16xK) * B(Kx16) is issued in K-steps of
// 4*KPL: lane l supplies row (l & 15) of A and column (l & 15) of B, each with
// the KPL consecutive k indices starting at (l >> 4) * KPL.  Both operands are
// read from LDS matrices stored with k contiguous: A as [rows][K] and B as
// [cols][K] (i.e. B transposed).  The accumulator holds D[(l >> 4) * 4 + r][l & 15]
// in element r.
//
// KPL = 8 (bf16): v_mfma_f32_16x16x32_bf16;  KPL = 4 (bf16): ..._16x16x16_bf16;
// KPL = 1 (fp32): v_mfma_f32_16x16x4_f32.
// ---------------------------------------------------------------------------
template <class T, int KPL> struct Frag;
template <> struct Frag<bf16, 8> { typedef bf16x8 type; };
template <> struct Frag<bf16, 4> { typedef bf16x4 type; };
template <> struct Frag<float, 1> { typedef float type; };

template <class T, int KPL>
__device__ __forceinline__ typename Frag<T, KPL>::type load_frag(const T *base, int ld, int row0,
                                                                 int k0, int lane) {
    const T *p = base + (row0 + (lane & 15)) * ld + k0 + (lane >> 4) * KPL;
    return *reinterpret_cast<const typename Frag<T, KPL>::type *>(p);
}

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                     __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// D = A B + C with D in registers disjoint from C.  Left to itself the compiler
// may give a 16x16 product a destination that overlaps its accumulator input by
// half a tile (D starting two registers below or above C), and the matrix unit
// does not form the right sum for such a partial overlap; accumulating in place
// (D and C the same registers) is fine.  Keeping C live past the product rules
// the overlap out.  For accumulator chains whose in-place form the compiler
// keeps on its own, plain mma() is used.
template <class A, class B>
__device__ __forceinline__ f32x4 mma_sep(A a, B b, f32x4 c) {
    const f32x4 d = mma(a, b, c);
    asm volatile("" ::"v"(c));
    return d;
}

// k per lane for a product whose reduction length is K.
template <class T, int K> struct KplFor { static constexpr int value = 1; };
template <int K> struct KplFor<bf16, K> { static constexpr int value = (K % 32 == 0) ? 8 : 4; };

// D += A[arow0.., kbeg..kend) * B[brow0.., kbeg..kend)^T with A, B k-contiguous in LDS.
// kbeg/kend must be multiples of the K-step 4*KPL.
template <class T, int KPL>
__device__ __forceinline__ f32x4 tile_mma(f32x4 acc, const T *A, int lda, int arow0, const T *B,
                                          int ldb, int brow0, int kbeg, int kend, int lane) {
    for (int k0 = kbeg; k0 < kend; k0 += 4 * KPL) {
        auto a = load_frag<T, KPL>(A, lda, arow0, k0, lane);
        auto b = load_frag<T, KPL>(B, ldb, brow0, k0, lane);
        acc = mma(a, b, acc);
    }
    return acc;
}

__device__ __forceinline__ int acc_row(int lane, int r) { return (lane >> 4) * 4 + r; }
__device__ __forceinline__ int acc_col(int lane) { return lane & 15; }

}  // namespace kda
