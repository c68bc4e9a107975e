// kda_prologue.hip -- fused causal short conv + SiLU + per-head L2 norm.
//
// [Walkthrough] 第二站: each of q, k, v passes a width-4 causal depthwise conv
// (current position plus up to three earlier ones, history carried by a conv
// cache, packed sequences via cu_seqlens) with SiLU inside the conv module; the
// KDA operator then L2-normalises q and k.  [Replication-2]: one causal Conv1D
// per channel.
//
// The prologue is a pure stream (read x once, write y once), so the kernel is
// laid out for HBM: each lane owns 4 consecutive channels (8 bytes of bf16, 16
// of fp32; 4 rather than 8 bf16 channels keeps the fp64 arithmetic below half
// the register file, for occupancy) and walks a tile of consecutive tokens,
// keeping the conv window in registers; a wave covers 256 contiguous channels
// of a token row, so every load and store is one coalesced access.  The lanes
// of one head form an aligned power-of-two group inside the wave, so the L2
// sum of squares is a few lane shuffles.  Sequence starts inside a tile switch
// the out-of-sequence taps to the caller's conv history (or zeros).
//
// Rounding.  With bf16 outputs every value is rounded once to bf16 (nearest,
// ties to even) from its exact conv/SiLU/L2 value, i.e. the result is correctly
// rounded: a plain fp32 evaluation would round a value lying within its own
// error of a bf16 rounding midpoint to either side, and such 1-ulp flips of q
// and k move the recurrence's largest outputs by far more than one ulp.  The
// conv is exact in fp64; the sigmoid and the norm take a fast route with a
// proven error bound, and the few tokens whose result the bound cannot place on
// one side of a midpoint are redone in full fp64.  With fp32 outputs the
// arithmetic is fp32.
#include <type_traits>

#include "kda_device.cuh"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kConvThreads = 256;
#ifndef KDA_CONV_TILE
#define KDA_CONV_TILE 16
#endif
constexpr int kConvTile = KDA_CONV_TILE;  // tokens per thread
// Workgroups per CU the register allocation must allow (4 = 4 waves per SIMD):
// the straight-line interior tile would otherwise trade occupancy for
// instruction-level parallelism far beyond what pays.
#ifndef KDA_CONV_MINB
#define KDA_CONV_MINB 4
#endif
#ifndef KDA_CONV_GROUP
#define KDA_CONV_GROUP 2
#endif
constexpr int kConvGroup = KDA_CONV_GROUP;
#ifndef KDA_CONV_AHEAD
#define KDA_CONV_AHEAD 4
#endif
constexpr int kConvAhead = KDA_CONV_AHEAD;  // rows loaded this many tokens ahead of use

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

// e^x in fp64 for the SiLU, from the mathematics: x = n ln2 + r with n the
// nearest integer to x / ln2 (Cody-Waite reduction: ln2 split into a 32-bit
// head, so n * head is exact for |n| < 2^20, and a tail holding the next 53
// bits), |r| <= ln2 / 2, then e^r by its Taylor polynomial to degree 12
// (truncation below 2.5e-16 relative) and the scaling by 2^n.  x is clamped to
// [-708, 708]; outside, the SiLU is already a or 0 to far below bf16 precision.
__device__ __forceinline__ double exp_f64(double x) {
    constexpr double kInvLn2 = 0x1.71547652b82fep+0;
    constexpr double kLn2Hi = 0x1.62e42fee00000p-1;    // ln 2 to 32 significant bits
    constexpr double kLn2Lo = 0x1.a39ef35793c76p-33;   // ln 2 - kLn2Hi
    x = fmin(fmax(x, -708.0), 708.0);
    const double n = __builtin_rint(x * kInvLn2);
    double r = fma(-n, kLn2Hi, x);
    r = fma(-n, kLn2Lo, r);
    double p = 1.0 / 479001600.0;                       // 1 / 12!
    p = fma(p, r, 1.0 / 39916800.0);
    p = fma(p, r, 1.0 / 3628800.0);
    p = fma(p, r, 1.0 / 362880.0);
    p = fma(p, r, 1.0 / 40320.0);
    p = fma(p, r, 1.0 / 5040.0);
    p = fma(p, r, 1.0 / 720.0);
    p = fma(p, r, 1.0 / 120.0);
    p = fma(p, r, 1.0 / 24.0);
    p = fma(p, r, 1.0 / 6.0);
    p = fma(p, r, 0.5);
    p = fma(p, r, 1.0);
    p = fma(p, r, 1.0);
    return __builtin_ldexp(p, (int)n);
}

// a * sigmoid(a) = a / (1 + e^{-a}) in fp64: the reciprocal from the hardware
// estimate refined by two Newton steps (each squares the relative error).
__device__ __forceinline__ double silu_of(double a) {
    const double d = 1.0 + exp_f64(-a);
    double r = __builtin_amdgcn_rcp(d);
    r = fma(r, fma(-d, r, 1.0), r);
    r = fma(r, fma(-d, r, 1.0), r);
    return a * r;
}
__device__ __forceinline__ float inv_norm(float ss, float eps) { return 1.0f / sqrtf(ss + eps); }
__device__ __forceinline__ double inv_norm(double ss, float eps) { return 1.0 / sqrt(ss + (double)eps); }

// Sigmoid 1 / (1 + e^-a) to within 1.8 u relative (u = 2^-24) for a >= -80, at a
// fraction of the fp64 cost: e^-a = 2^x with x = -a log2 e split in fp64 into an
// integer n and |f| <= 1/2 (f exact), 2^f from the hardware exp2 (below 0.77 fp32
// ulp on that range, i.e. 1.54 u relative) of f rounded to fp32 (0.17 u more),
// scaled by 2^n exactly; the reciprocal of 1 + e^-a from the hardware estimate
// refined by one Newton step in fp64 (error squared to below 2^-44).  An error
// eta in e^-a reaches the sigmoid as eta (1 - sigmoid) <= eta.  For a < -80 the
// fp32 estimates leave their range and the result means nothing.
__device__ __forceinline__ double sigmoid_fast(double a) {
    const double x = a * -0x1.71547652b82fep+0;
    const double n = __builtin_rint(x);
    const float f = (float)(x - n);
    const double e = __builtin_ldexp((double)__builtin_amdgcn_exp2f(f), (int)n);
    const double d = 1.0 + e;
    const double r = (double)__builtin_amdgcn_rcpf((float)d);
    return fma(r, fma(-d, r, 1.0), r);
}

// s^(-1/2) for 2^-100 <= s <= 2^100: the hardware estimate and one Newton step
// in fp64 (relative error below 2^-42).
__device__ __forceinline__ double rsqrt_fast(double s) {
    const double r = (double)__builtin_amdgcn_rsqf((float)s);
    return r * fma(-0.5 * s * r, r, 1.5);
}

// Whether an fp32 value known to lie within 5 of its ulps of the exact result
// rounds to the same bf16 as that result: its 16 bits below the bf16 precision
// must be more than 6 ulps away from the rounding midpoint 0x8000.  (Binade
// edges are 0x8000 ulps away from any midpoint, and both signs round alike.)
__device__ __forceinline__ bool bf16_rounding_sure(float v) {
    const uint32_t low = __float_as_uint(v) & 0xffffu;
    return low - (0x8000u - 6u) > 12u;
}

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

// Channels per lane: a 16-byte vector for fp32; for bf16 a tunable 8 (16 bytes)
// or 4 (8 bytes; fewer registers per lane for the fp64 arithmetic).
#ifndef KDA_CONV_VEC_BF16
#define KDA_CONV_VEC_BF16 4
#endif
template <class T> struct ConvVec { static constexpr int n = 4; typedef f32x4 type; };
template <> struct ConvVec<bf16> {
    static constexpr int n = KDA_CONV_VEC_BF16;
    typedef bf16 type __attribute__((ext_vector_type(KDA_CONV_VEC_BF16)));
};

typedef ConvVec<bf16>::type BfVec;
constexpr int kBfVec = ConvVec<bf16>::n;

// Fast finish of one bf16 token row: sigmoid_fast, an fp64 sum of squares over
// the head and rsqrt_fast.  Each y carries at most 1.8 u relative error from its
// sigmoid and the norm at most the largest of those over the head, so the fp32
// rounding of the result lies within 2 * 1.8 u * 2^24 + 1/2 < 4.2 fp32 ulps of
// the exact value and rounds to the correctly rounded bf16 whenever
// bf16_rounding_sure says so.  Returns whether this lane has a value it cannot
// vouch for (then the token must be redone by finish_exact).
template <int LPG>
__device__ __forceinline__ bool finish_fast(const double (&acc)[kBfVec], bool silu, float eps,
                                            BfVec &out) {
    double yv[kBfVec];
    bool unsure = false;
#pragma unroll
    for (int e = 0; e < kBfVec; ++e) {
        yv[e] = silu ? acc[e] * sigmoid_fast(acc[e]) : acc[e];
        unsure |= silu && acc[e] < -80.0;
    }
    if constexpr (LPG > 0) {
        double ss = 0;
#pragma unroll
        for (int e = 0; e < kBfVec; ++e) ss += yv[e] * yv[e];
        const double s = group_sum<LPG>(ss) + (double)eps;
        unsure |= !(s >= 0x1p-100 && s <= 0x1p100);
        const double inv = rsqrt_fast(s);
#pragma unroll
        for (int e = 0; e < kBfVec; ++e) yv[e] *= inv;
    }
#pragma unroll
    for (int e = 0; e < kBfVec; ++e) {
        const float yf = (float)yv[e];
        unsure |= !bf16_rounding_sure(yf);
        out[e] = (bf16)yf;
    }
    return unsure;
}

// The same token row entirely in fp64 (all lanes of each head group take part).
template <int LPG>
__device__ __forceinline__ void finish_exact(double (&acc)[kBfVec], bool silu, float eps,
                                             BfVec &out) {
    if (silu) {
#pragma unroll
        for (int e = 0; e < kBfVec; ++e) acc[e] = silu_of(acc[e]);
    }
    if constexpr (LPG > 0) {
        double ss = 0;
#pragma unroll
        for (int e = 0; e < kBfVec; ++e) ss += acc[e] * acc[e];
        ss = group_sum<LPG>(ss);
        const double inv = inv_norm(ss, eps);
#pragma unroll
        for (int e = 0; e < kBfVec; ++e) acc[e] *= inv;
    }
#pragma unroll
    for (int e = 0; e < kBfVec; ++e) out[e] = bf16_from_f64(acc[e]);
}

// A row of V channels at a 32-bit byte offset from a uniform base (the scalar
// base + vector offset addressing form).
template <class VT>
__device__ __forceinline__ VT ld_row(const void *base, uint32_t byte_off) {
    return *reinterpret_cast<const VT *>(reinterpret_cast<const char *>(base) + byte_off);
}
template <class VT>
__device__ __forceinline__ void st_row(void *base, uint32_t byte_off, VT v) {
    *reinterpret_cast<VT *>(reinterpret_cast<char *>(base) + byte_off) = v;
}

// Fp32 finish of one token row (fp32 outputs): SiLU and the head's L2 norm.
template <int LPG>
__device__ __forceinline__ void finish_plain(float (&acc)[4], bool silu, float eps, f32x4 &out) {
    if (silu) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = silu_of(acc[e]);
    }
    if constexpr (LPG > 0) {
        float ss = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) ss += acc[e] * acc[e];
        const float inv = inv_norm(group_sum<LPG>(ss), eps);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] *= inv;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = acc[e];
}

// LPG: lanes per L2 group (0 = no L2).  SILU: 0 or 1 fixes the activation at
// compile time; -1 takes the run-time flag.
template <class T, int W, int LPG, int SILU>
__global__ __launch_bounds__(kConvThreads, KDA_CONV_MINB)
void conv_kernel(const T *__restrict__ x, const T *__restrict__ w, const T *__restrict__ bias,
                 const int32_t *__restrict__ cu_seqlens, int nseq, int64_t total, int64_t C,
                 const T *__restrict__ hist, int silu_flag, float eps, T *__restrict__ y) {
    constexpr bool kBf16 = std::is_same<T, bf16>::value;
    const bool silu = SILU < 0 ? silu_flag != 0 : SILU != 0;
    constexpr int V = ConvVec<T>::n;
    typedef typename ConvVec<T>::type VT;
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

    int n = find_seq(cu_seqlens, nseq, t0 < total ? t0 : total - 1);
    int64_t bos = seq_off(cu_seqlens, n, total);
    int64_t eos = seq_off(cu_seqlens, n + 1, total);

    // Interior tile (the common case): every lane of the block is in range and
    // every tap of the tile's tokens lies inside one sequence, so the tile is
    // straight-line code.  Rows are read kConvAhead tokens ahead of use, converted
    // once, and slide through `win` (win[i] holds position t-(W-1)+i).  With bf16
    // outputs each token is finished on the fast route and stored; the tokens
    // where some lane could not vouch for its value are then redone in fp64 and
    // stored again (same lane, same address: the later store wins).
    if ((int64_t)(blockIdx.x + 1) * kConvThreads <= nvec && t0 - (W - 1) >= bos &&
        t0 + kConvTile <= eos && C * (kConvTile + W) * (int64_t)sizeof(T) < (1ll << 31)) {
        constexpr int R = kConvTile + W - 1;          // rows t0-(W-1) .. t0+TT-1
        const T *xb = x + (t0 - (W - 1)) * C;
        T *yb = y + t0 * C;
        const uint32_t lane_off = (uint32_t)c0 * (uint32_t)sizeof(T);
        const uint32_t row_bytes = (uint32_t)C * (uint32_t)sizeof(T);
        VT raw[R];
#pragma unroll
        for (int r = 0; r < W - 1 + kConvAhead && r < R; ++r)
            raw[r] = ld_row<VT>(xb, lane_off + r * row_bytes);
        A win[W][V];
#pragma unroll
        for (int i = 1; i < W; ++i)
#pragma unroll
            for (int e = 0; e < V; ++e) win[i][e] = (A)to_f32(raw[i - 1][e]);
        uint32_t flags = 0;
#pragma unroll
        for (int tt = 0; tt < kConvTile; ++tt) {
            constexpr int kNext = W - 1 + kConvAhead;
            if (tt + kNext < R) raw[tt + kNext] = ld_row<VT>(xb, lane_off + (tt + kNext) * row_bytes);
#pragma unroll
            for (int i = 0; i + 1 < W; ++i)
#pragma unroll
                for (int e = 0; e < V; ++e) win[i][e] = win[i + 1][e];
#pragma unroll
            for (int e = 0; e < V; ++e) win[W - 1][e] = (A)to_f32(raw[tt + W - 1][e]);
            A acc[V];
#pragma unroll
            for (int e = 0; e < V; ++e) {
                acc[e] = bs[e];
#pragma unroll
                for (int i = 0; i < W; ++i) acc[e] += wt[i][e] * win[i][e];
            }
            VT out;
            if constexpr (kBf16)
                flags |= (uint32_t)finish_fast<LPG>(acc, silu, eps, out) << tt;
            else
                finish_plain<LPG>(acc, silu, eps, out);
            st_row<VT>(yb, lane_off + tt * row_bytes, out);
            // Scheduling regions of kConvGroup tokens: interleaving neighbouring
            // tokens hides latency; hoisting work across the whole tile only
            // raises register pressure.
            if ((tt + 1) % kConvGroup == 0) __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (kBf16) {
#pragma unroll 1
            for (int tt = 0; tt < kConvTile; ++tt) {
                if (__builtin_amdgcn_ballot_w64((flags >> tt) & 1u) != 0) {
                    A acc[V];
#pragma unroll
                    for (int e = 0; e < V; ++e) acc[e] = bs[e];
#pragma unroll
                    for (int i = 0; i < W; ++i) {
                        const VT r = ld_row<VT>(xb, lane_off + (tt + i) * row_bytes);
#pragma unroll
                        for (int e = 0; e < V; ++e) acc[e] += wt[i][e] * (A)to_f32(r[e]);
                    }
                    VT out;
                    finish_exact<LPG>(acc, silu, eps, out);
                    st_row<VT>(yb, lane_off + tt * row_bytes, out);
                }
            }
        }
        return;
    }

    // General tile (a sequence start near or inside the tile, a ragged channel
    // block, the end of the batch): one token at a time, each tap read directly,
    // from the batch or, before the sequence start, from the caller's conv
    // history (zeros without one).
#pragma unroll 1
    for (int tt = 0; tt < kConvTile; ++tt) {
        const int64_t t = t0 + tt;
        if (t >= total) break;                       // uniform across the block
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
            VT r = VT{};
            if (active) {
                if (p >= bos)
                    r = *reinterpret_cast<const VT *>(x + p * C + c0);
                else if (hist)
                    r = *reinterpret_cast<const VT *>(
                        hist + ((int64_t)n * (W - 1) + (p - bos + (W - 1))) * C + c0);
            }
#pragma unroll
            for (int e = 0; e < V; ++e) acc[e] += wt[i][e] * (A)to_f32(r[e]);
        }
        VT out;
        if constexpr (kBf16) {
            if (__builtin_amdgcn_ballot_w64(finish_fast<LPG>(acc, silu, eps, out) && active) != 0)
                finish_exact<LPG>(acc, silu, eps, out);
        } else {
            finish_plain<LPG>(acc, silu, eps, out);
        }
        if (active) *reinterpret_cast<VT *>(y + t * C + c0) = out;
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
        const int64_t nvec = C / ConvVec<T>::n;
        dim3 grid((unsigned)((nvec + kConvThreads - 1) / kConvThreads),
                  (unsigned)((a.total_tokens + kConvTile - 1) / kConvTile));
        // bf16: the activation is a template switch (it sits inside the straight-line
        // interior tile); fp32 takes the run-time flag.
        decltype(&conv_kernel<T, W, LPG, -1>) kernel;
        if constexpr (std::is_same<T, bf16>::value)
            kernel = a.silu ? conv_kernel<T, W, LPG, 1> : conv_kernel<T, W, LPG, 0>;
        else
            kernel = conv_kernel<T, W, LPG, -1>;
        hipLaunchKernelGGL(kernel, grid, dim3(kConvThreads), 0, s,
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
    switch (a.head_dim / ConvVec<T>::n) {
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
