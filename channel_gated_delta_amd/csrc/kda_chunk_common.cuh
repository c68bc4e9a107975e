// kda_chunk_common.cuh -- pieces shared by the two chunk kernels of the KDA
// prefill (kda_chunk_prep.cuh, kda_chunk_state.cuh).
//
// Semantics: the token recurrence of [Walkthrough] 第三站-第五站 (decay the rows
// of S by exp(g_t), predict S^T k_t, write beta_t k_t (v_t - S^T k_t)^T, read
// scale * S^T q_t), executed chunk by chunk ([Walkthrough] 彩蛋: chunks pass the
// state, the work inside a chunk becomes matrix products; [Replication-2] 图1:
// transitions compose into one chunk-level transform).
//
// Chunk algebra (derived from the recurrence; state S0 entering a chunk of n
// tokens, G_t = sum_{j<=t} g_j per key channel, exponentials of differences only):
//   A_ti = sum_c k_tc k_ic e^{G_tc - G_ic}  (i < t),   P_ti = sum_c q_tc k_ic e^{G_tc - G_ic}  (i <= t)
//   Tb   = (I + diag(beta) A)^{-1} diag(beta)
//   U    = Tb (V - (K * e^{G}) S0)
//   O    = scale (Q * e^{G}) S0 + scale P U
//   S    = diag(e^{G_n}) S0 + (K * e^{G_n - G})^T U
// Tb and scale*P depend on q, k, g, beta of the chunk only, not on the state, so
// a first kernel computes them for every (chunk, head) at once (fully parallel)
// and a second kernel walks the chunks of each sequence with the state on chip.
//
// Precision.  The outputs are heavy-tailed (the largest |o| is 10-30x the rms),
// so one bf16 rounding of a product operand already costs ~2^-9 * 30 of the rms.
// With bf16 inputs every product therefore uses split operands x = hi + lo
// (both bf16, |lo| <= 2^-9 |x|) and the three-term product hi*hi + hi*lo + lo*hi
// (~2^-16 relative); the diagonal of P (the token's own term, scale q_t . k_t)
// is computed exactly in fp32.  With fp32 inputs the products run on fp32 MFMA.
#pragma once

#include <type_traits>

#include "kda_device.cuh"

namespace kda {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two adjacent elements of T.
template <class T> struct Pair;
template <> struct Pair<bf16> { typedef bf16x2 type; };
template <> struct Pair<float> { typedef f32x2 type; };

// Load / store at a uniform base plus a 32-bit byte offset (lets the compiler use
// the scalar-base + vector-offset addressing form instead of 64-bit address math).
template <class V>
__device__ __forceinline__ V ld_off(const void *base, uint32_t byte_off) {
    return *reinterpret_cast<const V *>(reinterpret_cast<const char *>(base) + byte_off);
}
template <class V>
__device__ __forceinline__ void st_off(void *base, uint32_t byte_off, V x) {
    *reinterpret_cast<V *>(reinterpret_cast<char *>(base) + byte_off) = x;
}

// Source of the log-decay g of every (token, head, key channel), chosen by the
// kernels' compile-time gate mode GM:
//  * kGatePlain: read from g [T, H, dk] (fp32);
//  * kGateFused: the bounded gate ([Walkthrough] 彩蛋: the gate function with a
//    lower bound) formed from its pre-activation z [T, H, dk] (activation dtype),
//    a per-head A_log and a per-channel bias as
//        g = lb * sigmoid(e^{A_log[h]} (z + dt_bias[h, c])),
//    so lb <= g <= 0 by construction;
//  * kGateHead: one decay per (token, head), g [T, H] (fp32), the same for every
//    key channel -- the head-wise forget gate of GDN, the coarser variant the
//    pages compare KDA with ([Replication-1]).
enum { kGatePlain = 0, kGateFused = 1, kGateHead = 2 };
struct GateSrc {
    const float *g;        // plain gate [T, H, dk], or the per-head gate [T, H]
    const void *z;         // fused gate: pre-activation
    const float *a_log;    // [H], NULL = 0
    const float *dt_bias;  // [H, dk], NULL = 0
    float lb;              // fused gate: the lower bound
};

// The fused gate in log2 units, x = g log2(e).  With the (head, channel)
// constants c1 = -log2(e) e^{A_log[h]} and c2 = c1 dt_bias[h, c], the sigmoid's
// argument y satisfies -y log2(e) = z c1 + c2, so x = lb log2(e) / (1 + 2^{z c1 + c2}).
// The hardware exp2 (+inf for large arguments: the sigmoid is then 0) and
// reciprocal estimate are each within about one ulp.
__device__ __forceinline__ float gate_c1(const GateSrc &gs, int h) {
    return -kLog2e * (gs.a_log ? expf(gs.a_log[h]) : 1.f);
}
__device__ __forceinline__ float gate_c2(const GateSrc &gs, float c1, int h, int dk, int c) {
    return gs.dt_bias ? c1 * gs.dt_bias[(size_t)h * dk + c] : 0.f;
}
__device__ __forceinline__ float gate_log2(float z, float c1, float c2, float lb_log2e) {
    return lb_log2e * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(fmaf(z, c1, c2)));
}

// Packed-sequence offset i clamped to [0, total]; cu == NULL is one sequence.
__device__ __forceinline__ int64_t chunk_seq_off(const int32_t *cu, int i, int64_t total) {
    if (!cu) return i == 0 ? 0 : total;
    return min((int64_t)max(cu[i], 0), total);
}

// Dispatch order of a packed batch for the state kernel: every sequence's rank
// by decreasing length (ties: lower index first), stored as order[rank] = n.
// With the longest sequences dispatched first, the state kernel's last
// workgroups are short ones (list scheduling, longest job first).  The ranks
// form a permutation of 0 .. nseq-1 for any offsets (the order is strict), so
// every entry of `order` is written exactly once.  MAXSEQ bounds nseq (the host
// launches it only for batches that fit).
template <int MAXSEQ>
__global__ __launch_bounds__(256) void seq_order_kernel(const int32_t *__restrict__ cu, int nseq,
                                                        int64_t total, int32_t *__restrict__ order) {
    __shared__ int64_t len[MAXSEQ];
    if (nseq > MAXSEQ) return;
    for (int i = threadIdx.x; i < nseq; i += 256) {
        const int64_t b = chunk_seq_off(cu, i, total);
        len[i] = max(chunk_seq_off(cu, i + 1, total), b) - b;
    }
    __syncthreads();
    const int n = blockIdx.x * 256 + threadIdx.x;
    if (n >= nseq) return;
    const int64_t ln = len[n];
    int rank = 0;
    for (int m = 0; m < nseq; ++m) rank += (len[m] > ln) | ((len[m] == ln) & (m < n));
    order[rank] = n;
}

__device__ __forceinline__ void split2(float x, bf16 &hh, bf16 &ll) {
    hh = (bf16)x;
    ll = (bf16)(x - (float)hh);
}

// Split two floats into packed bf16 pairs hi = (h0, h1), lo = (l0, l1) with
// x = h + l: one packed conversion for the high parts, their exact fp32 values
// by shifting the bits back, two subtractions, one packed conversion.
__device__ __forceinline__ void split_pair(float x0, float x1, bf16x2 &hi, bf16x2 &lo) {
    bf16x2 h;
    h[0] = (bf16)x0;
    h[1] = (bf16)x1;
    uint32_t hb = __builtin_bit_cast(uint32_t, h);
    // (opaque to the optimiser, which would otherwise convert x0 a second time
    // to rebuild h0 instead of shifting the packed pair)
    asm("" : "+v"(hb));
    const float h0 = __uint_as_float(hb << 16), h1 = __uint_as_float(hb & 0xffff0000u);
    bf16x2 l;
    l[0] = (bf16)(x0 - h0);
    l[1] = (bf16)(x1 - h1);
    hi = __builtin_bit_cast(bf16x2, hb);
    lo = l;
}

// Eight floats split into 16x16x32 operand tuples hi, lo (x = hi + lo), with the
// packed high parts kept as one register tuple (no copies into the operand).
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8 &hi, bf16x8 &lo) {
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    u4 hb, lb;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        bf16x2 h;
        h[0] = (bf16)x[2 * e];
        h[1] = (bf16)x[2 * e + 1];
        hb[e] = __builtin_bit_cast(uint32_t, h);
    }
    asm("" : "+v"(hb));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        bf16x2 l;
        l[0] = (bf16)(x[2 * e] - __uint_as_float(hb[e] << 16));
        l[1] = (bf16)(x[2 * e + 1] - __uint_as_float(hb[e] & 0xffff0000u));
        lb[e] = __builtin_bit_cast(uint32_t, l);
    }
    hi = __builtin_bit_cast(bf16x8, hb);
    lo = __builtin_bit_cast(bf16x8, lb);
}

// Store x0, x1 at H[i], H[i+1] (and the low parts at L[i], L[i+1] when T is bf16).
template <class T>
__device__ __forceinline__ void put2(T *H, T *L, int i, float x0, float x1) {
    typedef typename Pair<T>::type P2;
    if constexpr (std::is_same<T, bf16>::value) {
        P2 h, l;
        split_pair(x0, x1, h, l);
        *reinterpret_cast<P2 *>(H + i) = h;
        *reinterpret_cast<P2 *>(L + i) = l;
    } else {
        *reinterpret_cast<P2 *>(H + i) = P2{x0, x1};
    }
}
template <class T>
__device__ __forceinline__ void put1(T *H, T *L, int i, float x) {
    if constexpr (std::is_same<T, bf16>::value) {
        split2(x, H[i], L[i]);
    } else {
        H[i] = x;
    }
}

template <class F>
__device__ __forceinline__ void scale_frag(F &f, const float *s) {
    if constexpr (std::is_same<F, float>::value) {
        f *= s[0];
    } else {
        constexpr int n = sizeof(F) / sizeof(bf16);
#pragma unroll
        for (int e = 0; e < n; ++e) f[e] = (bf16)((float)f[e] * s[e]);
    }
}

// (hi + lo) * s re-split into a new (hi, lo) pair, in fp32.
template <class F>
__device__ __forceinline__ void rescale_split(F &hi, F &lo, const float *s) {
    constexpr int n = sizeof(F) / sizeof(bf16);
#pragma unroll
    for (int e = 0; e < n; ++e) {
        const float x = ((float)hi[e] + (float)lo[e]) * s[e];
        const bf16 hh = (bf16)x;
        hi[e] = hh;
        lo[e] = (bf16)(x - (float)hh);
    }
}

// ---------------------------------------------------------------------------
// Products whose B operand is an accumulator tile held in registers.
//
// An accumulator tile holds B[(l >> 4) * 4 + r][l & 15] in element r of lane l.
// For a 32-row k block made of two such tiles (a: rows 0-15, b: rows 16-31), the
// lane's 8 B values are rows {(l>>4)*4 + 0..3} of a and of b; the hardware pairs
// A and B entries by (lane group, element), so the A fragment is read with the
// same k order: A[row][k0 + (l>>4)*4 + 0..3] and A[row][k0 + 16 + (l>>4)*4 + 0..3].
// A 16-row block uses the 16x16x16 instruction with one tile.  fp32 uses four
// 16x16x4 steps per 16-row block, step s taking element s.
// ---------------------------------------------------------------------------
struct BReg8 { bf16x8 h, l; };
struct BReg4 { bf16x4 h, l; };

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t bits(bf16x2 x) { return __builtin_bit_cast(uint32_t, x); }

// Split accumulator tiles into (hi, lo) B operands, assembling the vectors from
// whole 32-bit pairs (no per-element insertion).
__device__ __forceinline__ BReg8 breg8(const f32x4 &a, const f32x4 &b) {
    bf16x2 h0, l0, h1, l1, h2, l2, h3, l3;
    split_pair(a[0], a[1], h0, l0);
    split_pair(a[2], a[3], h1, l1);
    split_pair(b[0], b[1], h2, l2);
    split_pair(b[2], b[3], h3, l3);
    BReg8 r;
    r.h = __builtin_bit_cast(bf16x8, u32x4{bits(h0), bits(h1), bits(h2), bits(h3)});
    r.l = __builtin_bit_cast(bf16x8, u32x4{bits(l0), bits(l1), bits(l2), bits(l3)});
    return r;
}
__device__ __forceinline__ BReg4 breg4(const f32x4 &a) {
    bf16x2 h0, l0, h1, l1;
    split_pair(a[0], a[1], h0, l0);
    split_pair(a[2], a[3], h1, l1);
    BReg4 r;
    r.h = __builtin_bit_cast(bf16x4, u32x2{bits(h0), bits(h1)});
    r.l = __builtin_bit_cast(bf16x4, u32x2{bits(l0), bits(l1)});
    return r;
}

// A fragments (hi, lo) from bf16 LDS matrices [rows][ld], permuted k order.
__device__ __forceinline__ void afrag8(const bf16 *Mh, const bf16 *Ml, int ld, int row0, int k0,
                                       int lane, bf16x8 &hh, bf16x8 &ll) {
    const int off = (row0 + (lane & 15)) * ld + k0 + (lane >> 4) * 4;
    const u32x2 h0 = *reinterpret_cast<const u32x2 *>(Mh + off);
    const u32x2 h1 = *reinterpret_cast<const u32x2 *>(Mh + off + 16);
    const u32x2 l0 = *reinterpret_cast<const u32x2 *>(Ml + off);
    const u32x2 l1 = *reinterpret_cast<const u32x2 *>(Ml + off + 16);
    hh = __builtin_bit_cast(bf16x8, u32x4{h0[0], h0[1], h1[0], h1[1]});
    ll = __builtin_bit_cast(bf16x8, u32x4{l0[0], l0[1], l1[0], l1[1]});
}
__device__ __forceinline__ void afrag4(const bf16 *Mh, const bf16 *Ml, int ld, int row0, int k0,
                                       int lane, bf16x4 &hh, bf16x4 &ll) {
    const int off = (row0 + (lane & 15)) * ld + k0 + (lane >> 4) * 4;
    hh = *reinterpret_cast<const bf16x4 *>(Mh + off);
    ll = *reinterpret_cast<const bf16x4 *>(Ml + off);
}

__device__ __forceinline__ f32x4 mma3(const bf16x8 &ah, const bf16x8 &al, const BReg8 &bb,
                                      f32x4 c) {
    c = mma_sep(ah, bb.h, c);
    c = mma_sep(ah, bb.l, c);
    return mma_sep(al, bb.h, c);
}
__device__ __forceinline__ f32x4 mma3(const bf16x4 &ah, const bf16x4 &al, const BReg4 &bb,
                                      f32x4 c) {
    c = mma_sep(ah, bb.h, c);
    c = mma_sep(ah, bb.l, c);
    return mma_sep(al, bb.h, c);
}

// D += A[row0.., 0..16*nb) * B, with B given as NBLK 16-row accumulator tiles
// (prepared once, used for several products) and A from (hi, lo) matrices of T
// in LDS (bf16: three-term split products; fp32: Ml unused, fp32 MFMA).
template <class T, int NBLK>
struct RegB {
    BReg8 b8[NBLK / 2 > 0 ? NBLK / 2 : 1];
    BReg4 b4;
    const f32x4 *tiles;
    __device__ __forceinline__ void prepare(const f32x4 *t) {
        tiles = t;
        if constexpr (std::is_same<T, bf16>::value) {
#pragma unroll
            for (int j = 0; j < NBLK / 2; ++j) b8[j] = breg8(t[2 * j], t[2 * j + 1]);
            if constexpr (NBLK % 2) b4 = breg4(t[NBLK - 1]);
        }
    }
    __device__ __forceinline__ f32x4 mul(f32x4 acc, const T *Mh, const T *Ml, int ld, int row0,
                                         int nb, int lane) const {
        if constexpr (std::is_same<T, bf16>::value) {
#pragma unroll
            for (int j = 0; j < NBLK / 2; ++j) {
                if (2 * j < nb) {
                    if (2 * j + 1 < nb) {
                        bf16x8 ah, al;
                        afrag8(Mh, Ml, ld, row0, 32 * j, lane, ah, al);
                        acc = mma3(ah, al, b8[j], acc);
                    } else {   // only the first tile of this pair is inside the range
                        bf16x4 ah, al;
                        afrag4(Mh, Ml, ld, row0, 32 * j, lane, ah, al);
                        BReg4 bb;
#pragma unroll
                        for (int e = 0; e < 4; ++e) { bb.h[e] = b8[j].h[e]; bb.l[e] = b8[j].l[e]; }
                        acc = mma3(ah, al, bb, acc);
                    }
                }
            }
            if constexpr (NBLK % 2) {
                if (NBLK - 1 < nb) {
                    bf16x4 ah, al;
                    afrag4(Mh, Ml, ld, row0, 16 * (NBLK - 1), lane, ah, al);
                    acc = mma3(ah, al, b4, acc);
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < NBLK; ++j) {
                if (j < nb) {
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const int col = 16 * j + (lane >> 4) * 4 + s;
                        acc = mma(Mh[(row0 + (lane & 15)) * ld + col], tiles[j][s], acc);
                    }
                }
            }
        }
        return acc;
    }
};

}  // namespace kda
