// kda_chunk_prep.cuh -- first kernel of the chunkwise KDA prefill: for every
// (chunk, head) at once, Tb = (I + diag(beta) A)^{-1} diag(beta) and scale * P
// (chunk algebra in kda_chunk_common.cuh).  These depend on q, k, g, beta of the
// chunk only, so the whole batch is one parallel grid; the sequential kernel
// (kda_chunk_state.cuh) reads them back.
//
// Output (workspace, fp32): row t of a chunk starting at token cs is stored at
// tb[(t * H + h) * C + i] (i = 0..C-1, column i is token cs + i; zero for i > t)
// and likewise scale * P (its diagonal scale * q_t . k_t exact in fp32).
//
// Decay numerics ([Walkthrough] 彩蛋: products of retention factors and their
// reciprocals must stay inside the floating-point range).  A and P factor
// e^{G_t - G_i} through the chunk's middle row m: rows e^{G_t - G_m}, columns
// e^{G_m - G_i}, both within e^{+-8|lb|}; a column factor can only underflow
// (< e^-87) where the lost term is below e^{-87 + 8|lb|}, negligible for
// lb >= -9.  Exponents are in log2 units.
//
// Chunks are 16 tokens: the Gram matrices are single 16 x 16 MFMA tiles and the
// inverse is one forward substitution.  Two forms:
//  * chunk_prep_kernel (fp32 operands, or dk = 16): one workgroup (4 waves) per
//    (16-token tile of the packed batch, head); it handles the chunk (if any) of
//    every sequence whose chunk start lies in its tile.  Thread (cp, part) owns
//    key channels 2cp, 2cp+1 of the rows [part*RP, part*RP + RP) for the decay
//    phase; the Gram operands go through LDS; wave 0 runs the two products and
//    the substitution (one lane per column).
//  * chunk_prep16_kernel (bf16, dk a multiple of 32): one wave per (tile, head),
//    operands in registers (below).
#pragma once

#include "kda_chunk_common.cuh"

namespace kda {

// Internal chunk of the prefill kernels.
constexpr int kChunk = 16;

template <class T, int DK_, int C_>
struct PrepCfg {
    static constexpr int DK = DK_, C = C_;
    static_assert(C == kChunk, "chunks are 16 tokens");
    static constexpr bool kSplit = std::is_same<T, bf16>::value;
    static constexpr int NSPLIT = kSplit ? 2 : 1;
    static constexpr int NW = 4, NT = NW * kWave;
    static constexpr int PAD = 16 / (int)sizeof(T);
    static constexpr int LDK = DK + PAD;                        // [C][DK] operand rows
    static constexpr int LDA = C + 4;                           // fp32 [C][C] rows
    static constexpr int KPL_DK = KplFor<T, DK>::value;
    static constexpr int NPC = DK / 2;                          // channel pairs
    static constexpr int NPART = (NT / NPC) < C ? (NT / NPC) : C;
    static constexpr int RP = C / NPART;                        // rows per part
    static_assert(NPART * RP == C && NPC <= kWave, "shape");

    static constexpr size_t al(size_t x) { return (x + 15) & ~(size_t)15; }
    static constexpr size_t szCK = al((size_t)C * LDK * sizeof(T));
    static constexpr size_t szCC = al((size_t)C * LDA * 4);
    static constexpr size_t szSmall = al((size_t)(2 * C + DK + NPART * DK) * 4);
    static constexpr size_t oGram = 0;                              // q*Dr, k*Dr, k*Dc (hi, lo)
    static constexpr size_t oA = oGram + 3 * NSPLIT * szCK;         // A -> Tb (fp32)
    static constexpr size_t oP = oA + szCC;                         // scale * P (fp32)
    static constexpr size_t oSmall = oP + szCC;
    static constexpr size_t kLds = oSmall + szSmall;
    static constexpr bool kFits = kLds <= 160 * 1024;
    static constexpr int kMinWg = kLds <= 53 * 1024 ? 3 : (kLds <= 80 * 1024 ? 2 : 1);
};

template <class T, int DK, int C, int GM>
__global__ __launch_bounds__(256, (PrepCfg<T, DK, C>::kMinWg))
void chunk_prep_kernel(const T *__restrict__ q, const T *__restrict__ k, GateSrc gs,
                       const float *__restrict__ beta,
                       const int32_t *__restrict__ cu_seqlens, int nseq, int64_t total, int H,
                       float scale, float *__restrict__ tb_out, float *__restrict__ p_out) {
    using Cfg = PrepCfg<T, DK, C>;
    constexpr bool SPLIT = Cfg::kSplit;
    constexpr int NT = Cfg::NT;
    constexpr int LDK = Cfg::LDK, LDA = Cfg::LDA, KPL_DK = Cfg::KPL_DK;
    constexpr int NPC = Cfg::NPC, NPART = Cfg::NPART, RP = Cfg::RP;
    typedef typename Pair<T>::type T2;

    __shared__ __attribute__((aligned(16))) char smem[Cfg::kLds];
    constexpr size_t CKE = Cfg::szCK / sizeof(T);
    T *sQDh = reinterpret_cast<T *>(smem + Cfg::oGram);
    T *sKDh = sQDh + Cfg::NSPLIT * CKE;
    T *sKCh = sKDh + Cfg::NSPLIT * CKE;
    T *sQDl = sQDh + (SPLIT ? CKE : 0);
    T *sKDl = sKDh + (SPLIT ? CKE : 0);
    T *sKCl = sKCh + (SPLIT ? CKE : 0);
    float *sA = reinterpret_cast<float *>(smem + Cfg::oA);
    float *sPf = reinterpret_cast<float *>(smem + Cfg::oP);
    float *sBeta = reinterpret_cast<float *>(smem + Cfg::oSmall);
    float *sPd = sBeta + C;                                            // scale q_t . k_t
    float *sGm = sPd + C;                                              // G at the middle row
    float *sTot = sGm + DK;                                            // part sums of g

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int h = blockIdx.y;
    const int64_t t0 = (int64_t)blockIdx.x * C, t1 = min(t0 + C, total);
    const size_t rowQK = (size_t)H * DK;
    const int cp = tid % NPC, part = tid / NPC;
    const bool fthread = part < NPART;
    // fused gate: this thread's constants for channels 2cp, 2cp+1
    float gc1 = 0.f, gc2a = 0.f, gc2b = 0.f, glb = 0.f;
    if constexpr (GM == kGateFused) {
        gc1 = gate_c1(gs, h);
        gc2a = gate_c2(gs, gc1, h, DK, 2 * cp);
        gc2b = gate_c2(gs, gc1, h, DK, 2 * cp + 1);
        glb = gs.lb * kLog2e;
    }

    // The sequences overlapping [t0, t1): the first is the last n with cu[n] <= t0.
    int n = 0;
    if (cu_seqlens) {
        int lo = 0, hi = nseq - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (chunk_seq_off(cu_seqlens, mid, total) <= t0) lo = mid; else hi = mid - 1;
        }
        n = lo;
    }
    bool first = true;
    for (; n < nseq; ++n) {
        const int64_t bos = chunk_seq_off(cu_seqlens, n, total);
        if (bos >= t1) break;
        const int64_t eos = max(chunk_seq_off(cu_seqlens, n + 1, total), bos);
        // this sequence's chunk start inside [t0, t1), if any
        const int64_t cs = bos >= t0 ? bos : bos + ((t0 - bos + C - 1) / C) * C;
        if (cs >= t1 || cs >= eos) continue;
        const int nt = (int)min((int64_t)C, eos - cs);
        if (!first) __syncthreads();   // the previous chunk's LDS reads are done
        first = false;

        // ---- loads and the in-chunk cumulative log2-decay (rows >= nt are zero)
        float qv[RP][2], kv[RP][2], gam[RP][2];
        if (fthread) {
            T2 qr[RP], kr[RP];
            f32x2 gr[RP];   // log2-decay of the two channels
#pragma unroll
            for (int j = 0; j < RP; ++j) {
                const int r = min(part * RP + j, nt - 1);
                const size_t off = (size_t)(cs + r) * rowQK + (size_t)h * DK + 2 * cp;
                qr[j] = *reinterpret_cast<const T2 *>(q + off);
                kr[j] = *reinterpret_cast<const T2 *>(k + off);
                if constexpr (GM == kGateFused) {
                    const T2 zr = *reinterpret_cast<const T2 *>(static_cast<const T *>(gs.z) + off);
                    gr[j][0] = gate_log2(to_f32(zr[0]), gc1, gc2a, glb);
                    gr[j][1] = gate_log2(to_f32(zr[1]), gc1, gc2b, glb);
                } else if constexpr (GM == kGateHead) {
                    gr[j][0] = gr[j][1] = gs.g[(size_t)(cs + r) * H + h] * kLog2e;
                } else {
                    const f32x2 gv = *reinterpret_cast<const f32x2 *>(gs.g + off);
                    gr[j][0] = gv[0] * kLog2e;
                    gr[j][1] = gv[1] * kLog2e;
                }
            }
            float a0 = 0.f, a1 = 0.f;
#pragma unroll
            for (int j = 0; j < RP; ++j) {
                const bool in = part * RP + j < nt;
                qv[j][0] = in ? to_f32(qr[j][0]) : 0.f;
                qv[j][1] = in ? to_f32(qr[j][1]) : 0.f;
                kv[j][0] = in ? to_f32(kr[j][0]) : 0.f;
                kv[j][1] = in ? to_f32(kr[j][1]) : 0.f;
                a0 += in ? gr[j][0] : 0.f;
                a1 += in ? gr[j][1] : 0.f;
                gam[j][0] = a0;
                gam[j][1] = a1;
                // exact diagonal of P: scale * q_r . k_r over the NPC lanes of this part
                const float dot = group_sum<NPC>(qv[j][0] * kv[j][0] + qv[j][1] * kv[j][1]);
                if (cp == 0) sPd[part * RP + j] = scale * dot;
            }
            sTot[part * DK + 2 * cp] = a0;
            sTot[part * DK + 2 * cp + 1] = a1;
        }
        if (tid < C) sBeta[tid] = tid < nt ? beta[(size_t)(cs + tid) * H + h] : 0.f;
        __syncthreads();
        if (fthread) {
            float o0 = 0.f, o1 = 0.f;
            for (int p = 0; p < part; ++p) {
                o0 += sTot[p * DK + 2 * cp];
                o1 += sTot[p * DK + 2 * cp + 1];
            }
#pragma unroll
            for (int j = 0; j < RP; ++j) {
                gam[j][0] += o0;
                gam[j][1] += o1;
                if (part * RP + j == C / 2) {
                    sGm[2 * cp] = gam[j][0];
                    sGm[2 * cp + 1] = gam[j][1];
                }
            }
        }
        __syncthreads();

        // ---- Gram operands (hi, lo): q e^{G_t-G_m}, k e^{G_t-G_m}, k e^{G_m-G_t}
        if (fthread) {
#pragma unroll
            for (int j = 0; j < RP; ++j) {
                const int r = part * RP + j;
                float dr[2], dc[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const float d = gam[j][e] - sGm[2 * cp + e];
                    dr[e] = exp2_clamped(d);
                    dc[e] = exp2_clamped(-d);
                }
                const int i = r * LDK + 2 * cp;
                put2(sQDh, sQDl, i, qv[j][0] * dr[0], qv[j][1] * dr[1]);
                put2(sKDh, sKDl, i, kv[j][0] * dr[0], kv[j][1] * dr[1]);
                put2(sKCh, sKCl, i, kv[j][0] * dc[0], kv[j][1] * dc[1]);
            }
        }
        __syncthreads();

        if (wave == 0) {
            // ---- A (strict lower) and scale * P (lower, exact diagonal): one tile each
            f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
            for (int k0 = 0; k0 < DK; k0 += 4 * KPL_DK) {
                auto kh = load_frag<T, KPL_DK>(sKDh, LDK, 0, k0, lane);
                auto qh = load_frag<T, KPL_DK>(sQDh, LDK, 0, k0, lane);
                auto ch = load_frag<T, KPL_DK>(sKCh, LDK, 0, k0, lane);
                if constexpr (SPLIT) {
                    auto kl = load_frag<T, KPL_DK>(sKDl, LDK, 0, k0, lane);
                    auto ql = load_frag<T, KPL_DK>(sQDl, LDK, 0, k0, lane);
                    auto cl = load_frag<T, KPL_DK>(sKCl, LDK, 0, k0, lane);
                    accA = mma_sep(kh, cl, accA);
                    accA = mma_sep(kl, ch, accA);
                    accP = mma_sep(qh, cl, accP);
                    accP = mma_sep(ql, ch, accP);
                }
                accA = mma_sep(kh, ch, accA);
                accP = mma_sep(qh, ch, accP);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = acc_row(lane, r), col = acc_col(lane);
                sA[row * LDA + col] = row > col ? accA[r] : 0.f;
                sPf[row * LDA + col] = row > col ? scale * accP[r] : (row == col ? sPd[row] : 0.f);
            }
            // wave-private from here to the barrier: its LDS ops complete in order
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");

            // ---- (I + diag(beta) A)^{-1}: lane i builds column i by forward substitution
            const int i = lane;
            float x[C];
#pragma unroll
            for (int r = 0; r < C; ++r) {
                const float br = sBeta[r];
                float s = 0.f;
#pragma unroll
                for (int m2 = 0; m2 < r; ++m2) s += sA[r * LDA + m2] * x[m2];
                x[r] = (r == i) ? 1.f : (r < i ? 0.f : -br * s);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
            if (i < C) {
#pragma unroll
                for (int r = 0; r < C; ++r) sA[r * LDA + i] = x[r];
            }
        }
        __syncthreads();

        // ---- write Tb = X diag(beta) and scale * P, rows < nt, 4 columns per item
        for (int idx = tid; idx < C * C / 4; idx += NT) {
            const int r = (idx * 4) / C, c0 = (idx * 4) % C;
            if (r < nt) {
                f32x4 tv, pv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    tv[e] = sA[r * LDA + c0 + e] * sBeta[c0 + e];
                    pv[e] = sPf[r * LDA + c0 + e];
                }
                const size_t o = ((size_t)(cs + r) * H + h) * C + c0;
                *reinterpret_cast<f32x4 *>(tb_out + o) = tv;
                *reinterpret_cast<f32x4 *>(p_out + o) = pv;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// One wave per (16-token tile, head): the bf16, 16-token form of the prep kernel.
//
// Lane l holds row t = l & 15 of the chunk and, for key block j, channels
// 32j + 8(l >> 4) .. +7 -- exactly the A / B fragment layout of the 16x16x32
// product -- so the Gram operands are built and split in registers and go
// straight into the MFMA (M = X Y^T when both operands are row fragments).  The
// in-chunk log2-decay prefix runs over the 16 rows of a DPP row (row_shr steps),
// the middle-row reference comes from lane 8 of the row, and the exact diagonal
// of P is a 4-lane sum.  Only the 16 x 16 forward substitution goes through a
// small wave-private LDS tile; there is no workgroup barrier.
// ---------------------------------------------------------------------------
#ifndef KDA_PREP16_MINB
#define KDA_PREP16_MINB 3
#endif
template <int S>
__device__ __forceinline__ float row_shr_zero(float v) {   // lane l%16 >= S: lane l-S, else 0
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x110 + S, 0xf, 0xf, false));
}

template <int DK, int GM>
__global__ __launch_bounds__(256, KDA_PREP16_MINB)
void chunk_prep16_kernel(const bf16 *__restrict__ q, const bf16 *__restrict__ k, GateSrc gs,
                         const float *__restrict__ beta,
                         const int32_t *__restrict__ cu_seqlens, int nseq, int64_t total, int H,
                         float scale, int64_t units, float *__restrict__ tb_out,
                         float *__restrict__ p_out) {
    constexpr int C = 16, NKB = DK / 32, LDA = C + 4;   // 16-byte aligned tile rows
    static_assert(DK % 32 == 0, "shape");
    __shared__ __attribute__((aligned(16))) float smem[4][2 * C * LDA + C];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int64_t unit = (int64_t)blockIdx.x * 4 + wave;
    if (unit >= units) return;                 // the whole wave: no workgroup barriers below
    float *sA = smem[wave], *sP = sA + C * LDA, *sB = sP + C * LDA;
    const int h = (int)(unit % H);             // heads fastest: a workgroup shares its rows
    const int64_t t0 = (unit / H) * C, t1 = min(t0 + C, total);
    const size_t rowQK = (size_t)H * DK;
    const int t = lane & 15, kb = lane >> 4;
    float gc1 = 0.f, glb = 0.f;   // fused gate: this head's constants
    if constexpr (GM == kGateFused) {
        gc1 = gate_c1(gs, h);
        glb = gs.lb * kLog2e;
    }

    int n = 0;
    if (cu_seqlens) {
        int lo = 0, hi = nseq - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (chunk_seq_off(cu_seqlens, mid, total) <= t0) lo = mid; else hi = mid - 1;
        }
        n = lo;
    }
    for (; n < nseq; ++n) {
        const int64_t bos = chunk_seq_off(cu_seqlens, n, total);
        if (bos >= t1) break;
        const int64_t eos = max(chunk_seq_off(cu_seqlens, n + 1, total), bos);
        const int64_t cs = bos >= t0 ? bos : bos + ((t0 - bos + C - 1) / C) * C;
        if (cs >= t1 || cs >= eos) continue;
        const int nt = __builtin_amdgcn_readfirstlane((int)min((int64_t)C, eos - cs));
        // Rows >= nt read copies of the last row and are left unmasked: no row < nt
        // depends on them (the prefix runs forward, the substitution reads A[r][m]
        // with m < r, P is lower triangular) and they are never written; the middle-
        // row reference stays within 8 rows of decay of every row either way.
        const size_t off = (size_t)(cs + min(t, nt - 1)) * rowQK + (size_t)h * DK + 8 * kb;
        f32x4 A3[3], P3[3];
#pragma unroll
        for (int i = 0; i < 3; ++i) A3[i] = P3[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        float dg = 0.f;                        // this lane's part of q_t . k_t
#pragma unroll
        for (int j = 0; j < NKB; ++j) {
            const bf16x8 qr = *reinterpret_cast<const bf16x8 *>(q + off + 32 * j);
            const bf16x8 kr = *reinterpret_cast<const bf16x8 *>(k + off + 32 * j);
            float x[8], qd[8], kd[8], kc[8];
            if constexpr (GM == kGateHead) {
                // one decay per (token, head): the same for the lane's 8 channels
                const float xh = gs.g[(size_t)(cs + min(t, nt - 1)) * H + h] * kLog2e;
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = xh;
            } else if constexpr (GM == kGateFused) {
                const bf16x8 zr = *reinterpret_cast<const bf16x8 *>(
                    static_cast<const bf16 *>(gs.z) + off + 32 * j);
                const int c0 = 32 * j + 8 * kb;
                f32x4 d0 = f32x4{0.f, 0.f, 0.f, 0.f}, d1 = d0;
                if (gs.dt_bias) {
                    d0 = *reinterpret_cast<const f32x4 *>(gs.dt_bias + (size_t)h * DK + c0);
                    d1 = *reinterpret_cast<const f32x4 *>(gs.dt_bias + (size_t)h * DK + c0 + 4);
                }
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    x[e] = gate_log2((float)zr[e], gc1, gc1 * (e < 4 ? d0[e] : d1[e - 4]), glb);
            } else {
                const f32x4 g0 = *reinterpret_cast<const f32x4 *>(gs.g + off + 32 * j);
                const f32x4 g1 = *reinterpret_cast<const f32x4 *>(gs.g + off + 32 * j + 4);
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = (e < 4 ? g0[e] : g1[e - 4]) * kLog2e;
            }
            // inclusive prefix over the rows (G_t, log2 units)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                x[e] += row_shr_zero<1>(x[e]);
                x[e] += row_shr_zero<2>(x[e]);
                x[e] += row_shr_zero<4>(x[e]);
                x[e] += row_shr_zero<8>(x[e]);
            }
            // the middle row's G (lane 8 of each row), all eight requests in flight
            float gm[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) gm[e] = __shfl(x[e], (lane & ~15) | 8, kWave);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // referenced at the middle row: |d| <= 8 |lb| log2 e <= 104 for gates
                // down to -9, so both factors are finite normal numbers
                const float d = x[e] - gm[e];
                const float dr = __builtin_amdgcn_exp2f(d), dc = __builtin_amdgcn_exp2f(-d);
                const float qv = (float)qr[e], kv = (float)kr[e];
                dg += qv * kv;
                qd[e] = qv * dr;
                kd[e] = kv * dr;
                kc[e] = kv * dc;
            }
            bf16x8 QH, QL, KH, KL, CH, CL;
            split8(qd, QH, QL);
            split8(kd, KH, KL);
            split8(kc, CH, CL);
            // A = Kd Kc^T, P = Qd Kc^T (hi*hi + hi*lo + lo*hi, one accumulator per term)
            A3[0] = mma(KH, CH, A3[0]);
            P3[0] = mma(QH, CH, P3[0]);
            A3[1] = mma(KH, CL, A3[1]);
            P3[1] = mma(QH, CL, P3[1]);
            A3[2] = mma(KL, CH, A3[2]);
            P3[2] = mma(QL, CH, P3[2]);
        }
        // q_t . k_t over the four lanes of row t (one per 16-lane row of the wave)
        dg = halves_sum(rowpair_sum(dg));

        // A (strictly lower) and scale * P (lower, exact diagonal) into the wave's tiles
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = acc_row(lane, r), col = acc_col(lane);
            const float a = A3[0][r] + (A3[1][r] + A3[2][r]);
            const float p = P3[0][r] + (P3[1][r] + P3[2][r]);
            sA[row * LDA + col] = row > col ? a : 0.f;
            // the exact diagonal: lane col holds row col's dot product
            sP[row * LDA + col] = row > col ? scale * p : (row == col ? scale * dg : 0.f);
        }
        if (lane < C) sB[lane] = lane < nt ? beta[(size_t)(cs + lane) * H + h] : 0.f;
        // wave-private tiles: the LDS ops of one wave complete in order
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");

        // Tb = (I + diag(beta) A)^{-1} diag(beta): lane i builds column i by forward
        // substitution (rows above i come out zero by themselves: every term of their
        // sums is), scales it by beta_i and writes it over the A tile, which no lane
        // reads any more once the substitution is done.
        if (lane < C) {
            const int i = lane;
            float xs[C];
#pragma unroll
            for (int r = 0; r < C; ++r) {
                float sum = 0.f;
#pragma unroll
                for (int m = 0; m < r; ++m) sum = fmaf(sA[r * LDA + m], xs[m], sum);
                const float v = -sB[r] * sum;
                xs[r] = r == i ? 1.f : v;
            }
            const float bi = sB[i];
#pragma unroll
            for (int r = 0; r < C; ++r) sA[r * LDA + i] = xs[r] * bi;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
        // rows of Tb and P: lane l writes columns 4 (l & 3) .. +3 of row l >> 2
        {
            const int rr = lane >> 2, cc = 4 * (lane & 3);
            if (rr < nt) {
                const size_t o = ((size_t)(cs + rr) * H + h) * C + cc;
                *reinterpret_cast<f32x4 *>(tb_out + o) = *reinterpret_cast<const f32x4 *>(sA + rr * LDA + cc);
                *reinterpret_cast<f32x4 *>(p_out + o) = *reinterpret_cast<const f32x4 *>(sP + rr * LDA + cc);
            }
        }
        // the next chunk of this tile reuses the tile only after every lane's reads
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    }
}

}  // namespace kda
