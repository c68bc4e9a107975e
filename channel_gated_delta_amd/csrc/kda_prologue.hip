// kda_prologue.hip -- fused causal short conv + SiLU + per-head L2 norm.
//
// [Walkthrough] 第二站: each of q, k, v passes a width-4 causal depthwise conv
// (current position plus up to three earlier ones, history carried by a conv
// cache, packed sequences via cu_seqlens) with SiLU inside the conv module; the
// KDA operator then L2-normalises q and k.  [Replication-2]: one causal Conv1D
// per channel.
//
// The prologue is a pure stream (read x once, write y once), so the kernel is
// laid out for HBM: each lane owns one 16-byte vector of channels (8 bf16 or 4
// fp32) and walks a tile of TT consecutive tokens, keeping the conv window in
// registers; a wave covers 64 contiguous vectors of a token row, so every load
// and store is a full 1 KiB coalesced access.  The lanes of one head form an
// aligned power-of-two group inside the wave, so the L2 sum of squares is a
// few lane shuffles.  Sequence starts inside a tile switch the out-of-sequence
// taps to the caller's conv history (or zeros).
//
// Rounding.  With bf16 outputs every value is computed in fp64 and rounded
// once to bf16 (nearest, ties to even), so the result is the correctly rounded
// conv/SiLU/L2 value; an fp32 evaluation would round a value lying within its
// own error of a bf16 rounding midpoint to either side, and such 1-ulp flips of
// q and k move the recurrence's largest outputs by far more than one ulp.  With
// fp32 outputs the arithmetic is fp32.
#include <type_traits>

#include "kda_device.cuh"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kConvThreads = 256;
constexpr int kConvTile = 16;  // tokens per thread

// Offset i of the packed batch, clamped to [0, total]; cu == NULL is one sequence.
__device__ __forceinline__ int64_t seq_off(const int32_t *cu, int i, int64_t total) {
    if (!cu) return i == 0 ? 0 : total;
    return min((int64_t)max(cu[i], 0), total);
}

// Nearest bf16 (ties to even) of a double.  The float conversion rounds first;
// if that lands exactly on a bf16 midpoint that d itself is not on, the second
// rounding must go to d's side rather than to the even neighbour.
__device__ __forceinline__ bf16 bf16_from_f64(double d) {
    const float f = (float)d;
    uint32_t u = __float_as_uint(f);
    if ((u & 0xffffu) == 0x8000u && (double)f != d) {
        u = (u & 0xffff0000u) + (fabs(d) > fabs((double)f) ? 0x10000u : 0u);
        return __builtin_bit_cast(bf16, (uint16_t)(u >> 16));
    }
    return (bf16)f;
}

template <class T> struct ConvAcc { typedef float type; };
template <> struct ConvAcc<bf16> { typedef double type; };

__device__ __forceinline__ float silu_of(float a) { return a / (1.0f + __expf(-a)); }
__device__ __forceinline__ double silu_of(double a) { return a / (1.0 + exp(-a)); }
__device__ __forceinline__ float inv_norm(float ss, float eps) { return 1.0f / sqrtf(ss + eps); }
__device__ __forceinline__ double inv_norm(double ss, float eps) { return 1.0 / sqrt(ss + (double)eps); }
__device__ __forceinline__ float store_val(float x, float) { return x; }
__device__ __forceinline__ bf16 store_val(double x, bf16) { return bf16_from_f64(x); }

// Sequence containing token t: the largest n with cu[n] <= t.
__device__ __forceinline__ int find_seq(const int32_t *cu, int nseq, int64_t t) {
    if (!cu) return 0;
    int lo = 0, hi = nseq - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int64_t)cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

template <class T, int W, int LPG>  // LPG: lanes per L2 group (0 = no L2)
__global__ __launch_bounds__(kConvThreads)
void conv_kernel(const T *__restrict__ x, const T *__restrict__ w, const T *__restrict__ bias,
                 const int32_t *__restrict__ cu_seqlens, int nseq, int64_t total, int64_t C,
                 const T *__restrict__ hist, int silu, float eps, T *__restrict__ y) {
    constexpr int V = Vec16<T>::n;
    typedef typename Vec16<T>::type VT;
    typedef typename ConvAcc<T>::type A;
    const int64_t nvec = C / V;
    const int64_t cv = (int64_t)blockIdx.x * kConvThreads + threadIdx.x;  // channel vector
    const bool active = cv < nvec;
    const int64_t c0 = cv * V;
    const int64_t t0 = (int64_t)blockIdx.y * kConvTile;

    A wt[W][V], bs[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
        bs[e] = (active && bias) ? (A)to_f32(bias[c0 + e]) : (A)0;
#pragma unroll
        for (int i = 0; i < W; ++i) wt[i][e] = active ? (A)to_f32(w[(c0 + e) * W + i]) : (A)0;
    }

    // Raw rows t0-(W-1) .. t0+TT-1 (rows outside [0, total) are never used as data).
    VT raw[kConvTile + W - 1];
#pragma unroll
    for (int r = 0; r < kConvTile + W - 1; ++r) {
        const int64_t p = t0 - (W - 1) + r;
        if (active && p >= 0 && p < total)
            raw[r] = *reinterpret_cast<const VT *>(x + p * C + c0);
        else
            raw[r] = VT{};
    }

    int n = find_seq(cu_seqlens, nseq, t0 < total ? t0 : total - 1);
    int64_t bos = seq_off(cu_seqlens, n, total);
    int64_t eos = seq_off(cu_seqlens, n + 1, total);

#pragma unroll
    for (int tt = 0; tt < kConvTile; ++tt) {
        const int64_t t = t0 + tt;
        if (t >= total) break;                      // uniform across the block
        while (t >= eos && n + 1 < nseq) {           // next (possibly empty) sequence
            ++n;
            bos = seq_off(cu_seqlens, n, total);
            eos = seq_off(cu_seqlens, n + 1, total);
        }
        A acc[V];
#pragma unroll
        for (int e = 0; e < V; ++e) acc[e] = bs[e];
#pragma unroll
        for (int i = 0; i < W; ++i) {
            const int64_t p = t - (W - 1) + i;
            if (p >= bos) {
#pragma unroll
                for (int e = 0; e < V; ++e) acc[e] += wt[i][e] * (A)to_f32(raw[tt + i][e]);
            } else if (hist && active) {
                const T *h = hist + ((int64_t)n * (W - 1) + (p - bos + (W - 1))) * C + c0;
                const VT hv = *reinterpret_cast<const VT *>(h);
#pragma unroll
                for (int e = 0; e < V; ++e) acc[e] += wt[i][e] * (A)to_f32(hv[e]);
            }
        }
        if (silu) {
#pragma unroll
            for (int e = 0; e < V; ++e) acc[e] = silu_of(acc[e]);
        }
        if constexpr (LPG > 0) {
            A ss = 0;
#pragma unroll
            for (int e = 0; e < V; ++e) ss += acc[e] * acc[e];
            ss = group_sum<LPG>(ss);
            const A inv = inv_norm(ss, eps);
#pragma unroll
            for (int e = 0; e < V; ++e) acc[e] *= inv;
        }
        if (active) {
            VT out;
#pragma unroll
            for (int e = 0; e < V; ++e) out[e] = store_val(acc[e], T());
            *reinterpret_cast<VT *>(y + t * C + c0) = out;
        }
    }
}

// New conv history of every sequence: the last W-1 entries of [history, x_seq].
// One thread per (sequence, channel); it reads everything it needs before it
// writes, so the output may alias the input history.
template <class T, int W>
__global__ __launch_bounds__(256)
void conv_state_kernel(const T *__restrict__ x, const int32_t *__restrict__ cu_seqlens, int nseq,
                       int64_t total, int64_t C, const T *hist_in, T *hist_out) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)nseq * C) return;
    const int n = (int)(idx / C);
    const int64_t c = idx % C;
    const int64_t bos = seq_off(cu_seqlens, n, total);
    const int64_t eos = max(seq_off(cu_seqlens, n + 1, total), bos);
    T vals[W > 1 ? W - 1 : 1];
#pragma unroll
    for (int j = 0; j < W - 1; ++j) {
        const int64_t p = eos - (W - 1) + j;
        if (p >= bos)
            vals[j] = x[p * C + c];
        else
            vals[j] = hist_in ? hist_in[((int64_t)n * (W - 1) + (p - bos + (W - 1))) * C + c]
                              : from_f32<T>(0.f);
    }
#pragma unroll
    for (int j = 0; j < W - 1; ++j) hist_out[((int64_t)n * (W - 1) + j) * C + c] = vals[j];
}

template <class T, int W, int LPG>
hipError_t launch_conv(const ConvArgs &a, hipStream_t s) {
    const int64_t C = (int64_t)a.heads * a.head_dim;
    if (a.total_tokens > 0) {
        const int64_t nvec = C / Vec16<T>::n;
        dim3 grid((unsigned)((nvec + kConvThreads - 1) / kConvThreads),
                  (unsigned)((a.total_tokens + kConvTile - 1) / kConvTile));
        hipLaunchKernelGGL((conv_kernel<T, W, LPG>), grid, dim3(kConvThreads), 0, s,
                           (const T *)a.x, (const T *)a.weight, (const T *)a.bias, a.cu_seqlens,
                           a.num_seqs, a.total_tokens, C, (const T *)a.state_in, a.silu, a.eps,
                           (T *)a.y);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if (a.state_out && W > 1) {
        const int64_t n = (int64_t)a.num_seqs * C;
        hipLaunchKernelGGL((conv_state_kernel<T, W>), dim3((unsigned)((n + 255) / 256)), dim3(256),
                           0, s, (const T *)a.x, a.cu_seqlens, a.num_seqs, a.total_tokens, C,
                           (const T *)a.state_in, (T *)a.state_out);
        return hipGetLastError();
    }
    return hipSuccess;
}

template <class T, int W>
hipError_t dispatch_lpg(const ConvArgs &a, hipStream_t s) {
    if (!a.l2) return launch_conv<T, W, 0>(a, s);
    switch (a.head_dim / Vec16<T>::n) {
        case 1: return launch_conv<T, W, 1>(a, s);
        case 2: return launch_conv<T, W, 2>(a, s);
        case 4: return launch_conv<T, W, 4>(a, s);
        case 8: return launch_conv<T, W, 8>(a, s);
        case 16: return launch_conv<T, W, 16>(a, s);
        case 32: return launch_conv<T, W, 32>(a, s);
        case 64: return launch_conv<T, W, 64>(a, s);
    }
    return hipErrorNotSupported;
}

template <class T>
hipError_t dispatch_width(const ConvArgs &a, hipStream_t s) {
    switch (a.width) {
        case 1: return dispatch_lpg<T, 1>(a, s);
        case 2: return dispatch_lpg<T, 2>(a, s);
        case 3: return dispatch_lpg<T, 3>(a, s);
        case 4: return dispatch_lpg<T, 4>(a, s);
    }
    return hipErrorNotSupported;
}

}  // namespace

hipError_t launch_short_conv(const ConvArgs &a, bool bf16, hipStream_t s) {
    return bf16 ? dispatch_width<kda::bf16>(a, s) : dispatch_width<float>(a, s);
}

}  // namespace kda
