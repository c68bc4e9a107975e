// kda_chunk.cuh -- chunkwise-parallel KDA prefill kernel (included by the
// per-dtype translation units kda_chunk_bf16.hip / kda_chunk_f32.hip).
//
// Semantics: the token recurrence of [Walkthrough] 第三站-第五站 (decay the rows
// of S by exp(g_t), predict S^T k_t, write beta_t k_t (v_t - S^T k_t)^T, read
// scale * S^T q_t), executed chunk by chunk ([Walkthrough] 彩蛋: chunks pass the
// state, the work inside a chunk becomes matrix products; [Replication-2] 图1:
// transitions compose into one chunk-level transform).
//
// Chunk algebra (derived from the recurrence; state S0 entering a chunk of n
// tokens, G_t = sum_{j<=t} g_j per key channel, all exponentials of differences):
//   A_ti = sum_c k_tc k_ic e^{G_tc - G_ic}  (i < t),   P_ti = sum_c q_tc k_ic e^{G_tc - G_ic}  (i <= t)
//   T    = (I + diag(beta) A)^{-1},  Tb = T diag(beta)
//   W    = Tb (K * e^{G}),  U~ = Tb V,  U = U~ - W S0
//   O    = scale (Q * e^{G}) S0 + scale P U
//   S    = diag(e^{G_n}) S0 + (K * e^{G_n - G})^T U
//
// Work decomposition.  One workgroup (4 waves) owns one (sequence, head, value
// slice of BV columns) and walks the chunks of its sequence; value columns of S
// evolve independently, so slicing multiplies the parallelism of a head.  The
// fp32 state slice lives in MFMA accumulator registers for the whole sequence
// and is mirrored into LDS in the operand dtype once per chunk.  All products
// run on 16x16 MFMA tiles (bf16 in, fp32 accumulate; fp32 MFMA for the fp32
// dtype); the 64x64 unit-lower-triangular inverse is done in fp32 (16x16
// forward substitution per diagonal block, then blockwise fp32 MFMA merges).
//
// Decay numerics ([Walkthrough] 彩蛋: products of retention factors and their
// reciprocals must stay inside the floating-point range).  The intra-chunk Gram
// matrices factor e^{G_t - G_i} through 16-token sub-tiles referenced at the
// tile's middle row m: rows use e^{G_t - G_m}, columns e^{G_m - G_i}, which are
// bounded by e^{8|lb|} (finite for lb >= -10); off-diagonal tile pairs (R, I)
// multiply the column operand by the per-channel boundary factor
// e^{G_{m_R} - G_{m_I}} <= 1.  Every other factor (e^{G_t}, e^{G_n - G_t},
// e^{G_n}) is <= 1 and is exponentiated directly.  Exponents are kept in log2
// units and evaluated with v_exp_f32.
#pragma once

#include "kda_device.cuh"

namespace kda {

template <class T, int DK_, int BV_, int C_>
struct ChunkCfg {
    static constexpr int DK = DK_, BV = BV_, C = C_;
    static constexpr int NW = 4, NT = NW * kWave;
    static constexpr int NTC = C / 16, NTK = DK / 16, NTV = BV / 16;
    static constexpr int VEC = 16 / (int)sizeof(T);             // elements per 16-byte vector
    static constexpr int PAD = 16 / (int)sizeof(T);             // LDS row padding (elements)
    static constexpr int LDK = DK + PAD;                        // [*][DK] operand rows
    static constexpr int LDC = C + PAD;                         // [*][C] operand rows
    static constexpr int LDA = C + 1;                           // fp32 A / T matrix rows
    static constexpr int KPL_DK = KplFor<T, DK>::value;
    static constexpr int KPL_C = KplFor<T, C>::value;
    static constexpr int NPAIR = NTC * (NTC - 1) / 2;
    static constexpr int NS_TILES = NTK * NTV, NSW = (NS_TILES + NW - 1) / NW;
    static constexpr int NU_TILES = NTC * NTV, NUW = (NU_TILES + NW - 1) / NW;

    static constexpr size_t al(size_t x) { return (x + 15) & ~(size_t)15; }
    static constexpr size_t mx(size_t a, size_t b) { return a > b ? a : b; }
    static constexpr size_t szQ = al((size_t)C * LDK * sizeof(T));
    static constexpr size_t szK = al(mx((size_t)C * LDK, (size_t)DK * LDC) * sizeof(T));
    static constexpr size_t szX = al((size_t)C * LDK * sizeof(T));
    static constexpr size_t szKdT = al((size_t)DK * LDC * sizeof(T));
    static constexpr size_t szTb = al((size_t)C * LDC * sizeof(T));
    static constexpr size_t szG = al(mx((size_t)C * DK * 4, szKdT + szTb));
    static constexpr size_t szV = al((size_t)BV * LDC * sizeof(T));
    static constexpr size_t szA = al((size_t)C * LDA * 4);
    static constexpr size_t szP = al((size_t)C * LDC * sizeof(T));
    static constexpr size_t szU = al((size_t)BV * LDC * sizeof(T));
    static constexpr size_t szS = al((size_t)BV * LDK * sizeof(T));
    static constexpr size_t szY = al((size_t)(NTC > 1 ? NTC - 1 : 1) * 256 * 4);
    static constexpr size_t szSmall =
        al((size_t)(C + (NPAIR > 0 ? NPAIR : 1) * DK + DK) * 4);
    static constexpr size_t oQ = 0, oK = oQ + szQ, oX = oK + szK, oG = oX + szX, oV = oG + szG,
                            oA = oV + szV, oP = oA + szA, oU = oP + szP, oS = oU + szU,
                            oY = oS + szS, oSmall = oY + szY;
    static constexpr size_t kLds = oSmall + szSmall;
    static constexpr bool kFits = kLds <= 160 * 1024;
};

// Per-channel block offset for a packed batch; cu == NULL is one sequence.
__device__ __forceinline__ int64_t chunk_seq_off(const int32_t *cu, int i, int64_t total) {
    if (!cu) return i == 0 ? 0 : total;
    return min((int64_t)max(cu[i], 0), total);
}

__device__ __forceinline__ void scale_frag(float &f, const float *s) { f *= s[0]; }
__device__ __forceinline__ void scale_frag(bf16x4 &f, const float *s) {
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = (bf16)((float)f[e] * s[e]);
}
__device__ __forceinline__ void scale_frag(bf16x8 &f, const float *s) {
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (bf16)((float)f[e] * s[e]);
}

template <class T, int DK, int BV, int C>
__global__ __launch_bounds__(256, 1)
void chunk_kernel(const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
                  const float *__restrict__ g, const float *__restrict__ beta,
                  const int32_t *__restrict__ cu_seqlens, int64_t total, int H, int DV,
                  float scale, const float *__restrict__ h0, float *__restrict__ hT,
                  T *__restrict__ o, int units, int nslice) {
    using Cfg = ChunkCfg<T, DK, BV, C>;
    constexpr int NW = Cfg::NW, NT = Cfg::NT, NTC = Cfg::NTC, NTK = Cfg::NTK, NTV = Cfg::NTV;
    constexpr int VEC = Cfg::VEC, LDK = Cfg::LDK, LDC = Cfg::LDC, LDA = Cfg::LDA;
    constexpr int KPL_DK = Cfg::KPL_DK, KPL_C = Cfg::KPL_C;
    constexpr int KSTEP_C = 4 * KPL_C;
    typedef typename Vec16<T>::type VT;       // 16-byte vector of T

    __shared__ __attribute__((aligned(16))) char smem[Cfg::kLds];
    T *sQ = reinterpret_cast<T *>(smem + Cfg::oQ);     // raw q -> q*Dr -> scale*q*e^G
    T *sK = reinterpret_cast<T *>(smem + Cfg::oK);     // raw k -> k*Dr -> (k*e^{Gn-G})^T
    T *sX = reinterpret_cast<T *>(smem + Cfg::oX);     // k*Dc -> -W   (Dr, Dc: sub-tile factors)
    float *sGam = reinterpret_cast<float *>(smem + Cfg::oG);  // G (log2 units)
    T *sKdT = reinterpret_cast<T *>(smem + Cfg::oG);          // (k*e^G)^T   (reuses G)
    T *sTb = reinterpret_cast<T *>(smem + Cfg::oG + Cfg::szKdT);  // T diag(beta)
    T *sVT = reinterpret_cast<T *>(smem + Cfg::oV);    // V^T slice
    float *sA = reinterpret_cast<float *>(smem + Cfg::oA);  // A -> T (fp32)
    T *sP = reinterpret_cast<T *>(smem + Cfg::oP);     // scale * masked P
    T *sUT = reinterpret_cast<T *>(smem + Cfg::oU);    // U^T
    T *sST = reinterpret_cast<T *>(smem + Cfg::oS);    // S^T (operand copy of the state)
    float *sY = reinterpret_cast<float *>(smem + Cfg::oY);  // inverse scratch
    float *sBeta = reinterpret_cast<float *>(smem + Cfg::oSmall);
    float *sBnd = sBeta + C;                            // e^{G_mR - G_mI}, I < R
    float *sEGn = sBnd + (Cfg::NPAIR > 0 ? Cfg::NPAIR : 1) * DK;  // e^{G_last}

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;

    // Block -> (unit, slice): the slices of one unit share an XCD (blocks are
    // dispatched to the 8 XCDs round-robin), so their common q/k/g reads meet
    // in that XCD's L2.
    const int b = blockIdx.x, xcd = b & 7, slot = b >> 3;
    const int slice = slot % nslice;
    const int unit = (slot / nslice) * 8 + xcd;
    if (unit >= units) return;
    const int n = unit / H, h = unit % H;
    const int64_t bos = chunk_seq_off(cu_seqlens, n, total);
    const int64_t eos = max(chunk_seq_off(cu_seqlens, n + 1, total), bos);
    const int v0 = slice * BV;
    const size_t rowQK = (size_t)H * DK, rowV = (size_t)H * DV;

    // ---- state slice: accumulator tiles (rt, ct), tile id = rt*NTV + ct, wave = id % NW
    f32x4 Sacc[Cfg::NSW];
#pragma unroll
    for (int i = 0; i < Cfg::NSW; ++i) {
        const int id = wave + i * NW;
        Sacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (id < Cfg::NS_TILES && h0) {
            const int rt = id / NTV, ct = id % NTV;
            const float *src = h0 + ((size_t)unit * DK) * DV + v0;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Sacc[i][r] = src[(size_t)(rt * 16 + acc_row(lane, r)) * DV + ct * 16 + acc_col(lane)];
        }
    }
    auto store_state_operand = [&]() {
#pragma unroll
        for (int i = 0; i < Cfg::NSW; ++i) {
            const int id = wave + i * NW;
            if (id < Cfg::NS_TILES) {
                const int rt = id / NTV, ct = id % NTV;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sST[(ct * 16 + acc_col(lane)) * LDK + rt * 16 + acc_row(lane, r)] =
                        from_f32<T>(Sacc[i][r]);
            }
        }
    };
    store_state_operand();

    for (int64_t c0 = bos; c0 < eos; c0 += C) {
        const int nt = (int)min((int64_t)C, eos - c0);

        // ================= L: load the chunk (rows >= nt are zero) =================
        for (int idx = tid; idx < C * (DK / VEC); idx += NT) {
            const int r = idx / (DK / VEC), cv = idx % (DK / VEC);
            VT qv = VT{}, kv = VT{};
            if (r < nt) {
                const size_t off = (size_t)(c0 + r) * rowQK + (size_t)h * DK + cv * VEC;
                qv = *reinterpret_cast<const VT *>(q + off);
                kv = *reinterpret_cast<const VT *>(k + off);
            }
            *reinterpret_cast<VT *>(sQ + r * LDK + cv * VEC) = qv;
            *reinterpret_cast<VT *>(sK + r * LDK + cv * VEC) = kv;
        }
        for (int idx = tid; idx < C * (BV / VEC); idx += NT) {
            const int r = idx / (BV / VEC), cv = idx % (BV / VEC);
            VT vv = VT{};
            if (r < nt)
                vv = *reinterpret_cast<const VT *>(v + (size_t)(c0 + r) * rowV + (size_t)h * DV +
                                                   v0 + cv * VEC);
#pragma unroll
            for (int e = 0; e < VEC; ++e) sVT[(cv * VEC + e) * LDC + r] = vv[e];
        }
        if (tid < C) sBeta[tid] = tid < nt ? beta[(size_t)(c0 + tid) * H + h] : 0.f;
        {
            // cumulative log2-decay per key channel: NP parts of RP rows, then a prefix fix-up
            constexpr int NP = NT / DK, RP = C / NP;
            static_assert(NP * DK == NT && NP * RP == C, "cumsum split");
            const int c = tid % DK, part = tid / DK;
            float gv[RP];
#pragma unroll
            for (int j = 0; j < RP; ++j) {
                const int r = part * RP + j;
                gv[j] = r < nt ? g[(size_t)(c0 + r) * rowQK + (size_t)h * DK + c] : 0.f;
            }
            float acc = 0.f;
#pragma unroll
            for (int j = 0; j < RP; ++j) {
                acc += gv[j] * kLog2e;
                sGam[(part * RP + j) * DK + c] = acc;
            }
            if constexpr (NP > 1) {
                __syncthreads();
                float off = 0.f;
                for (int p = 0; p < part; ++p) off += sGam[((p + 1) * RP - 1) * DK + c];
                __syncthreads();
#pragma unroll
                for (int j = 0; j < RP; ++j) sGam[(part * RP + j) * DK + c] += off;
            }
        }
        __syncthreads();

        // ================= F: decay factors =================
        // Gram operands to LDS: q e^{G_t-G_m}, k e^{G_t-G_m}, k e^{G_m-G_t} (m = middle
        // row of t's 16-token tile).  Chunk-level operands kept in registers until
        // the Gram products are done: scale q e^{G_t}, k e^{G_t}, k e^{G_n-G_t}.
        constexpr int PER = (C * (DK / VEC) + NT - 1) / NT;
        VT rQd[PER], rKd[PER], rKr[PER];
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int idx = tid + j * NT;
            if (idx < C * (DK / VEC)) {
                const int r = idx / (DK / VEC), cv = idx % (DK / VEC);
                const int m = (r / 16) * 16 + 8;
                const VT qv = *reinterpret_cast<const VT *>(sQ + r * LDK + cv * VEC);
                const VT kv = *reinterpret_cast<const VT *>(sK + r * LDK + cv * VEC);
                VT qd, kd, kc;
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const int c = cv * VEC + e;
                    const float gt = sGam[r * DK + c];
                    const float d = gt - sGam[m * DK + c];
                    const float dr = exp2_clamped(d), dc = exp2_clamped(-d);
                    const float eg = exp2_clamped(gt);
                    const float egr = exp2_clamped(sGam[(C - 1) * DK + c] - gt);
                    const float qf = to_f32(qv[e]), kf = to_f32(kv[e]);
                    qd[e] = from_f32<T>(qf * dr);
                    kd[e] = from_f32<T>(kf * dr);
                    kc[e] = from_f32<T>(kf * dc);
                    rQd[j][e] = from_f32<T>(qf * eg * scale);
                    rKd[j][e] = from_f32<T>(kf * eg);
                    rKr[j][e] = from_f32<T>(kf * egr);
                }
                *reinterpret_cast<VT *>(sQ + r * LDK + cv * VEC) = qd;
                *reinterpret_cast<VT *>(sK + r * LDK + cv * VEC) = kd;
                *reinterpret_cast<VT *>(sX + r * LDK + cv * VEC) = kc;
            }
        }
        for (int c = tid; c < DK; c += NT) {
            sEGn[c] = exp2_clamped(sGam[(C - 1) * DK + c]);
#pragma unroll
            for (int R = 1; R < NTC; ++R)
#pragma unroll
                for (int I = 0; I < R; ++I)
                    sBnd[(R * (R - 1) / 2 + I) * DK + c] =
                        exp2_clamped(sGam[(R * 16 + 8) * DK + c] - sGam[(I * 16 + 8) * DK + c]);
        }
        __syncthreads();

        // ================= G: Gram tiles A (strict lower) and P (lower) =================
        for (int p = wave; p < NTC * NTC; p += NW) {
            const int R = p / NTC, I = p % NTC;
            f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
            if (I <= R) {
                const float *bnd = sBnd + (I < R ? (R * (R - 1) / 2 + I) * DK : 0);
                for (int k0 = 0; k0 < DK; k0 += 4 * KPL_DK) {
                    auto ak = load_frag<T, KPL_DK>(sK, LDK, R * 16, k0, lane);
                    auto aq = load_frag<T, KPL_DK>(sQ, LDK, R * 16, k0, lane);
                    auto bc = load_frag<T, KPL_DK>(sX, LDK, I * 16, k0, lane);
                    if (I < R) scale_frag(bc, bnd + k0 + (lane >> 4) * KPL_DK);
                    accA = mma(ak, bc, accA);
                    accP = mma(aq, bc, accP);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = R * 16 + acc_row(lane, r), col = I * 16 + acc_col(lane);
                sA[row * LDA + col] = row > col ? accA[r] : 0.f;
                sP[row * LDC + col] = from_f32<T>(row >= col ? scale * accP[r] : 0.f);
            }
        }
        __syncthreads();

        // ================= X: chunk-level operands; inverse diagonal blocks =================
        // The Gram operands and G are dead: Qd over q*Dr, (k e^G)^T over G, (k e^{Gn-G})^T over k*Dr.
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int idx = tid + j * NT;
            if (idx < C * (DK / VEC)) {
                const int r = idx / (DK / VEC), cv = idx % (DK / VEC);
                *reinterpret_cast<VT *>(sQ + r * LDK + cv * VEC) = rQd[j];
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    sKdT[(cv * VEC + e) * LDC + r] = rKd[j][e];
                    sK[(cv * VEC + e) * LDC + r] = rKr[j][e];
                }
            }
        }
        // diagonal 16x16 blocks of (I + diag(beta) A)^{-1}: lane i builds column i
        for (int R = wave; R < NTC; R += NW) {
            const int i = lane;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float br = sBeta[R * 16 + r];
                float s = 0.f;
#pragma unroll
                for (int m2 = 0; m2 < r; ++m2) s += br * sA[(R * 16 + r) * LDA + R * 16 + m2] * x[m2];
                x[r] = (r == i) ? 1.f : (r < i ? 0.f : -s);
            }
            if (i < 16) {
#pragma unroll
                for (int r = 0; r < 16; ++r) sA[(R * 16 + r) * LDA + R * 16 + i] = x[r];
            }
        }
        __syncthreads();

        // off-diagonal blocks, one block row at a time (fp32 MFMA)
        for (int R = 1; R < NTC; ++R) {
            // Y_I = sum_{M=I}^{R-1} diag(beta_R) A_RM X_MI
            for (int I = wave; I < R; I += NW) {
                f32x4 y = {0.f, 0.f, 0.f, 0.f};
                const float br = sBeta[R * 16 + (lane & 15)];
                for (int k0 = I * 16; k0 < R * 16; k0 += 4) {
                    const float a = br * sA[(R * 16 + (lane & 15)) * LDA + k0 + (lane >> 4)];
                    const float bb = sA[(k0 + (lane >> 4)) * LDA + I * 16 + (lane & 15)];
                    y = mma(a, bb, y);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) sY[I * 256 + acc_row(lane, r) * 16 + acc_col(lane)] = y[r];
            }
            __syncthreads();
            // X_RI = -X_RR Y_I
            for (int I = wave; I < R; I += NW) {
                f32x4 xx = {0.f, 0.f, 0.f, 0.f};
                for (int k0 = 0; k0 < 16; k0 += 4) {
                    const float a = sA[(R * 16 + (lane & 15)) * LDA + R * 16 + k0 + (lane >> 4)];
                    const float bb = sY[I * 256 + (k0 + (lane >> 4)) * 16 + (lane & 15)];
                    xx = mma(a, bb, xx);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sA[(R * 16 + acc_row(lane, r)) * LDA + I * 16 + acc_col(lane)] = -xx[r];
            }
            __syncthreads();
        }

        // Tb = T diag(beta) in the operand dtype
        for (int idx = tid; idx < C * C; idx += NT) {
            const int r = idx / C, i = idx % C;
            sTb[r * LDC + i] = from_f32<T>(sA[r * LDA + i] * sBeta[i]);
        }
        __syncthreads();

        // ================= W = -Tb (K e^G) -> sX ;  U~ = Tb V -> registers =================
        for (int id = wave; id < NTC * NTK; id += NW) {
            const int R = id / NTK, ck = id % NTK;
            const int kend = ((R + 1) * 16 + KSTEP_C - 1) / KSTEP_C * KSTEP_C;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = tile_mma<T, KPL_C>(acc, sTb, LDC, R * 16, sKdT, LDC, ck * 16, 0,
                                     kend < C ? kend : C, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sX[(R * 16 + acc_row(lane, r)) * LDK + ck * 16 + acc_col(lane)] = from_f32<T>(-acc[r]);
        }
        f32x4 Uacc[Cfg::NUW], Oacc[Cfg::NUW];
#pragma unroll
        for (int i = 0; i < Cfg::NUW; ++i) {
            const int id = wave + i * NW;
            Uacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (id < Cfg::NU_TILES) {
                const int R = id / NTV, cv = id % NTV;
                const int kend = ((R + 1) * 16 + KSTEP_C - 1) / KSTEP_C * KSTEP_C;
                Uacc[i] = tile_mma<T, KPL_C>(Uacc[i], sTb, LDC, R * 16, sVT, LDC, cv * 16, 0,
                                             kend < C ? kend : C, lane);
            }
        }
        __syncthreads();

        // ================= U = U~ - W S ;  O = Qd S =================
#pragma unroll
        for (int i = 0; i < Cfg::NUW; ++i) {
            const int id = wave + i * NW;
            Oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (id < Cfg::NU_TILES) {
                const int R = id / NTV, cv = id % NTV;
                Uacc[i] = tile_mma<T, KPL_DK>(Uacc[i], sX, LDK, R * 16, sST, LDK, cv * 16, 0, DK, lane);
                Oacc[i] = tile_mma<T, KPL_DK>(Oacc[i], sQ, LDK, R * 16, sST, LDK, cv * 16, 0, DK, lane);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sUT[(cv * 16 + acc_col(lane)) * LDC + R * 16 + acc_row(lane, r)] =
                        from_f32<T>(Uacc[i][r]);
            }
        }
        __syncthreads();

        // ================= O += P U -> global ;  S = e^{Gn} S + (K e^{Gn-G})^T U =================
#pragma unroll
        for (int i = 0; i < Cfg::NUW; ++i) {
            const int id = wave + i * NW;
            if (id < Cfg::NU_TILES) {
                const int R = id / NTV, cv = id % NTV;
                const int kend = ((R + 1) * 16 + KSTEP_C - 1) / KSTEP_C * KSTEP_C;
                Oacc[i] = tile_mma<T, KPL_C>(Oacc[i], sP, LDC, R * 16, sUT, LDC, cv * 16, 0,
                                             kend < C ? kend : C, lane);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = R * 16 + acc_row(lane, r);
                    if (row < nt)
                        o[(size_t)(c0 + row) * rowV + (size_t)h * DV + v0 + cv * 16 + acc_col(lane)] =
                            from_f32<T>(Oacc[i][r]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < Cfg::NSW; ++i) {
            const int id = wave + i * NW;
            if (id < Cfg::NS_TILES) {
                const int rt = id / NTV, ct = id % NTV;
#pragma unroll
                for (int r = 0; r < 4; ++r) Sacc[i][r] *= sEGn[rt * 16 + acc_row(lane, r)];
                Sacc[i] = tile_mma<T, KPL_C>(Sacc[i], sK, LDC, rt * 16, sUT, LDC, ct * 16, 0, C, lane);
            }
        }
        store_state_operand();
        __syncthreads();
    }

    if (hT) {
#pragma unroll
        for (int i = 0; i < Cfg::NSW; ++i) {
            const int id = wave + i * NW;
            if (id < Cfg::NS_TILES) {
                const int rt = id / NTV, ct = id % NTV;
                float *dst = hT + ((size_t)unit * DK) * DV + v0;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dst[(size_t)(rt * 16 + acc_row(lane, r)) * DV + ct * 16 + acc_col(lane)] = Sacc[i][r];
            }
        }
    }
}

}  // namespace kda
