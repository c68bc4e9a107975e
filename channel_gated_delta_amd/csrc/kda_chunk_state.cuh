// kda_chunk_state.cuh -- second kernel of the chunkwise KDA prefill: walks the
// chunks of each sequence with the state on chip (chunk algebra in
// kda_chunk_common.cuh; Tb and scale * P come from the prep kernel).
//
// Work decomposition.  One workgroup of 8 waves owns one (sequence, head, value
// slice of BV columns) and runs two pipelines that meet at one barrier per step:
//  * consumer waves 0 .. BV/16-1: wave w owns the 16 state columns [16w, 16w+16)
//    of the slice.  Its part of the fp32 state lives in MFMA accumulator
//    registers for the whole sequence, and the state-dependent chain of a chunk
//    (E = V - Kd S, U = Tb E, O = Qd S + P U, the state update) runs inside that
//    wave from registers -- an accumulator tile doubles as the B operand of the
//    next product when the A fragment is read with the matching k order.
//  * producer waves 4..7 build the next chunk's operands in the other half of a
//    double-buffered LDS stage: scale q e^{G}, k e^{G} and (k e^{G_n - G})^T
//    (all factors <= 1, exponentiated directly), the split Tb and P rows, V and
//    e^{G_n}.  A producer lane owns two key channels of a group of rows; the
//    in-chunk prefix of the log-decay over row groups is a few lane shuffles,
//    so the producers need no barrier of their own.
// At step s the producers fill stage s & 1 with chunk s while the consumers run
// chunk s-1 from stage (s-1) & 1; the barrier at the end of the step hands the
// stage over.  Producers load chunk s+1 into registers during step s.
#pragma once

#include "kda_chunk_common.cuh"

namespace kda {

template <class T, int DK_, int BV_, int C_>
struct StateCfg {
    static constexpr int DK = DK_, BV = BV_, C = C_;
    static constexpr bool kSplit = std::is_same<T, bf16>::value;
    static constexpr int NSPLIT = kSplit ? 2 : 1;
    static constexpr int NT = 512, NPW = 4;                     // threads, producer waves
    static constexpr int NTC = C / 16, NTK = DK / 16, NCW = BV / 16;
    static constexpr int PAD = 16 / (int)sizeof(T);
    static constexpr int LDK = DK + PAD;                        // [C][DK] operand rows
    static constexpr int LDC = C + PAD;                         // [*][C] operand rows
    static constexpr int LDV = BV + 4;                          // fp32 [C][BV] rows
    // producer lane mapping: CPW channel pairs x RG row groups of RP rows per wave
    static constexpr int CPW = DK / 2 / NPW;
    static constexpr int RG = (kWave / CPW) < C ? (kWave / CPW) : C;
    static constexpr int RP = C / RG;
    static constexpr int NPT = NPW * kWave;                     // producer threads
    static constexpr int NTB = C * C / NPT;                     // Tb / P elements per thread
    static constexpr int NVE = C * BV / NPT;                    // V elements per thread
    static_assert(CPW >= 1 && RG * RP == C && NCW <= 4 && BV % 16 == 0, "shape");
    static_assert(NTB >= 1 && (NTB == 1 || NTB % 4 == 0) && NVE >= 1, "shape");

    static constexpr size_t al(size_t x) { return (x + 15) & ~(size_t)15; }
    static constexpr size_t szCK = al((size_t)C * LDK * sizeof(T));      // [C][DK]
    static constexpr size_t szKC = al((size_t)DK * LDC * sizeof(T));     // [DK][C]
    static constexpr size_t szCC = al((size_t)C * LDC * sizeof(T));      // [C][C]
    static constexpr size_t oQd = 0;                                // scale q e^G (hi, lo)
    static constexpr size_t oKd = oQd + NSPLIT * szCK;              // k e^G (hi, lo)
    static constexpr size_t oKrT = oKd + NSPLIT * szCK;             // (k e^{Gn-G})^T (hi, lo)
    static constexpr size_t oTb = oKrT + NSPLIT * szKC;             // Tb (hi, lo)
    static constexpr size_t oP = oTb + NSPLIT * szCC;               // scale * P (hi, lo)
    static constexpr size_t oV = oP + NSPLIT * szCC;                // V (fp32)
    static constexpr size_t oEGn = oV + al((size_t)C * LDV * 4);    // e^{G_n}
    static constexpr size_t kStage = oEGn + al((size_t)DK * 4);
    static constexpr size_t kLds = 2 * kStage;
    static constexpr bool kFits = kLds <= 160 * 1024;
};

template <class T, class TO, int DK, int BV, int C>
__global__ __launch_bounds__(512, 1)
void chunk_state_kernel(const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
                        const float *__restrict__ g, const float *__restrict__ tb,
                        const float *__restrict__ pm, const int32_t *__restrict__ cu_seqlens,
                        int64_t total, int H, int DV, float scale, const float *__restrict__ h0,
                        float *__restrict__ hT, TO *__restrict__ o, int units, int nslice) {
    using Cfg = StateCfg<T, DK, BV, C>;
    constexpr bool SPLIT = Cfg::kSplit;
    constexpr int NTC = Cfg::NTC, NTK = Cfg::NTK, NCW = Cfg::NCW;
    constexpr int LDK = Cfg::LDK, LDC = Cfg::LDC, LDV = Cfg::LDV;
    constexpr int CPW = Cfg::CPW, RG = Cfg::RG, RP = Cfg::RP, NTB = Cfg::NTB, NVE = Cfg::NVE;
    constexpr size_t CKE = Cfg::szCK / sizeof(T), KCE = Cfg::szKC / sizeof(T);
    constexpr size_t CCE = Cfg::szCC / sizeof(T);
    typedef typename Pair<T>::type T2;
    typedef T TV __attribute__((ext_vector_type(NVE)));

    __shared__ __attribute__((aligned(16))) char smem[Cfg::kLds];

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
    const int nchunks = (int)((eos - bos + C - 1) / C);
    const int v0 = slice * BV;
    const size_t rowQK = (size_t)H * DK, rowV = (size_t)H * DV;

    if (wave >= 4) {
        // =============================== producers ===============================
        const int pt = tid - 4 * kWave;                       // 0 .. 255
        const int pw = wave - 4;
        const int cpair = pw * CPW + (lane % CPW);            // channels 2cpair, 2cpair+1
        const int rg = lane / CPW;                            // row group: rows rg*RP + j
        const bool act = rg < RG;
        const int tr = (pt * NTB) / C, tc = (pt * NTB) % C;   // Tb / P: row tr, cols tc..
        const int vr = (pt * NVE) / BV, vcol = (pt * NVE) % BV;  // V: row vr, cols vcol..

        T2 pq[RP], pk[RP];
        f32x2 pg[RP];
        float ptb[NTB], ppm[NTB];
        TV pvv;
        auto issue_loads = [&](int64_t cs) {
            const int last = (int)min((int64_t)C, eos - cs) - 1;
            if (act) {
#pragma unroll
                for (int j = 0; j < RP; ++j) {
                    const size_t off = (size_t)(cs + min(rg * RP + j, last)) * rowQK +
                                       (size_t)h * DK + 2 * cpair;
                    pq[j] = *reinterpret_cast<const T2 *>(q + off);
                    pk[j] = *reinterpret_cast<const T2 *>(k + off);
                    pg[j] = *reinterpret_cast<const f32x2 *>(g + off);
                }
            }
            const size_t wo = ((size_t)(cs + min(tr, last)) * H + h) * C + tc;
            if constexpr (NTB == 1) {
                ptb[0] = tb[wo];
                ppm[0] = pm[wo];
            } else {
#pragma unroll
                for (int j = 0; j < NTB / 4; ++j) {
                    const f32x4 a = *reinterpret_cast<const f32x4 *>(tb + wo + 4 * j);
                    const f32x4 c = *reinterpret_cast<const f32x4 *>(pm + wo + 4 * j);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        ptb[4 * j + e] = a[e];
                        ppm[4 * j + e] = c[e];
                    }
                }
            }
            pvv = *reinterpret_cast<const TV *>(v + (size_t)(cs + min(vr, last)) * rowV +
                                                (size_t)h * DV + v0 + vcol);
        };
        if (nchunks > 0) issue_loads(bos);

        for (int s = 0; s <= nchunks; ++s) {
            if (s < nchunks) {
                const int64_t cs = bos + (int64_t)s * C;
                const int nt = (int)min((int64_t)C, eos - cs);
                char *st = smem + (s & 1) * Cfg::kStage;
                T *sQdh = reinterpret_cast<T *>(st + Cfg::oQd), *sQdl = sQdh + (SPLIT ? CKE : 0);
                T *sKdh = reinterpret_cast<T *>(st + Cfg::oKd), *sKdl = sKdh + (SPLIT ? CKE : 0);
                T *sKrTh = reinterpret_cast<T *>(st + Cfg::oKrT), *sKrTl = sKrTh + (SPLIT ? KCE : 0);
                T *sTbh = reinterpret_cast<T *>(st + Cfg::oTb), *sTbl = sTbh + (SPLIT ? CCE : 0);
                T *sPh = reinterpret_cast<T *>(st + Cfg::oP), *sPl = sPh + (SPLIT ? CCE : 0);
                float *sV = reinterpret_cast<float *>(st + Cfg::oV);
                float *sEGn = reinterpret_cast<float *>(st + Cfg::oEGn);

                // consume the registers (rows >= nt are zero)
                float qv[RP][2], kv[RP][2], gam[RP][2];
                float a0 = 0.f, a1 = 0.f;
#pragma unroll
                for (int j = 0; j < RP; ++j) {
                    const bool in = act && rg * RP + j < nt;
                    qv[j][0] = in ? to_f32(pq[j][0]) : 0.f;
                    qv[j][1] = in ? to_f32(pq[j][1]) : 0.f;
                    kv[j][0] = in ? to_f32(pk[j][0]) : 0.f;
                    kv[j][1] = in ? to_f32(pk[j][1]) : 0.f;
                    a0 += (in ? pg[j][0] : 0.f) * kLog2e;
                    a1 += (in ? pg[j][1] : 0.f) * kLog2e;
                    gam[j][0] = a0;
                    gam[j][1] = a1;
                }
                float tbv[NTB], pmv[NTB];
#pragma unroll
                for (int e = 0; e < NTB; ++e) {
                    tbv[e] = tr < nt ? ptb[e] : 0.f;
                    pmv[e] = tr < nt ? ppm[e] : 0.f;
                }
                float vv[NVE];
#pragma unroll
                for (int e = 0; e < NVE; ++e) vv[e] = vr < nt ? to_f32(pvv[e]) : 0.f;
                if (s + 1 < nchunks) issue_loads(cs + C);

                // prefix of the row-group sums (lanes rg*CPW + i share a channel pair)
                float inc0 = a0, inc1 = a1;
#pragma unroll
                for (int d = 1; d < RG; d <<= 1) {
                    const float u0 = __shfl_up(inc0, d * CPW, kWave);
                    const float u1 = __shfl_up(inc1, d * CPW, kWave);
                    if (rg >= d) {
                        inc0 += u0;
                        inc1 += u1;
                    }
                }
                const int lastl = (RG - 1) * CPW + (lane % CPW);
                const float tot0 = __shfl(inc0, lastl, kWave), tot1 = __shfl(inc1, lastl, kWave);
                const float off0 = inc0 - a0, off1 = inc1 - a1;

                if (act) {
                    float krt[2][RP];
#pragma unroll
                    for (int j = 0; j < RP; ++j) {
                        const float g0 = gam[j][0] + off0, g1 = gam[j][1] + off1;
                        const float e0 = exp2_clamped(g0), e1 = exp2_clamped(g1);
                        krt[0][j] = kv[j][0] * exp2_clamped(tot0 - g0);
                        krt[1][j] = kv[j][1] * exp2_clamped(tot1 - g1);
                        const int i = (rg * RP + j) * LDK + 2 * cpair;
                        put2(sQdh, sQdl, i, qv[j][0] * e0 * scale, qv[j][1] * e1 * scale);
                        put2(sKdh, sKdl, i, kv[j][0] * e0, kv[j][1] * e1);
                    }
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int base = (2 * cpair + e) * LDC + rg * RP;
                        if constexpr (RP % 2 == 0) {
#pragma unroll
                            for (int j = 0; j < RP; j += 2)
                                put2(sKrTh, sKrTl, base + j, krt[e][j], krt[e][j + 1]);
                        } else {
#pragma unroll
                            for (int j = 0; j < RP; ++j) put1(sKrTh, sKrTl, base + j, krt[e][j]);
                        }
                    }
                    if (rg == 0) {
                        sEGn[2 * cpair] = exp2_clamped(tot0);
                        sEGn[2 * cpair + 1] = exp2_clamped(tot1);
                    }
                }
                {
                    const int i = tr * LDC + tc;
                    if constexpr (NTB == 1) {
                        put1(sTbh, sTbl, i, tbv[0]);
                        put1(sPh, sPl, i, pmv[0]);
                    } else {
#pragma unroll
                        for (int e = 0; e < NTB; e += 2) {
                            put2(sTbh, sTbl, i + e, tbv[e], tbv[e + 1]);
                            put2(sPh, sPl, i + e, pmv[e], pmv[e + 1]);
                        }
                    }
#pragma unroll
                    for (int e = 0; e < NVE; ++e) sV[vr * LDV + vcol + e] = vv[e];
                }
            }
            __syncthreads();
        }
    } else {
        // =============================== consumers ===============================
        const bool owner = wave < NCW;
        const int vc = v0 + (owner ? wave : 0) * 16 + (lane & 15);  // this lane's value column
        f32x4 Sacc[NTK];
#pragma unroll
        for (int rt = 0; rt < NTK; ++rt) {
            Sacc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (owner && h0) {
                const float *src = h0 + ((size_t)unit * DK) * DV;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Sacc[rt][r] = src[(size_t)(rt * 16 + acc_row(lane, r)) * DV + vc];
            }
        }
        for (int s = 0; s <= nchunks; ++s) {
            if (s >= 1 && owner) {
                const int64_t c0 = bos + (int64_t)(s - 1) * C;
                const int nt = (int)min((int64_t)C, eos - c0);
                const char *st = smem + ((s - 1) & 1) * Cfg::kStage;
                const T *sQdh = reinterpret_cast<const T *>(st + Cfg::oQd);
                const T *sQdl = sQdh + (SPLIT ? CKE : 0);
                const T *sKdh = reinterpret_cast<const T *>(st + Cfg::oKd);
                const T *sKdl = sKdh + (SPLIT ? CKE : 0);
                const T *sKrTh = reinterpret_cast<const T *>(st + Cfg::oKrT);
                const T *sKrTl = sKrTh + (SPLIT ? KCE : 0);
                const T *sTbh = reinterpret_cast<const T *>(st + Cfg::oTb);
                const T *sTbl = sTbh + (SPLIT ? CCE : 0);
                const T *sPh = reinterpret_cast<const T *>(st + Cfg::oP);
                const T *sPl = sPh + (SPLIT ? CCE : 0);
                const float *sV = reinterpret_cast<const float *>(st + Cfg::oV);
                const float *sEGn = reinterpret_cast<const float *>(st + Cfg::oEGn);

                RegB<T, NTK> Sb;
                Sb.prepare(Sacc);
                f32x4 Et[NTC], Ot[NTC], Ut[NTC];
                // E = V - Kd S and O = Qd S
#pragma unroll
                for (int R = 0; R < NTC; ++R) {
                    Et[R] = Sb.mul(f32x4{0.f, 0.f, 0.f, 0.f}, sKdh, sKdl, LDK, R * 16, NTK, lane);
                    Ot[R] = Sb.mul(f32x4{0.f, 0.f, 0.f, 0.f}, sQdh, sQdl, LDK, R * 16, NTK, lane);
                }
#pragma unroll
                for (int R = 0; R < NTC; ++R)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        Et[R][r] = sV[(R * 16 + acc_row(lane, r)) * LDV + wave * 16 + (lane & 15)] -
                                   Et[R][r];
                // U = Tb E
                RegB<T, NTC> Eb;
                Eb.prepare(Et);
#pragma unroll
                for (int R = 0; R < NTC; ++R)
                    Ut[R] = Eb.mul(f32x4{0.f, 0.f, 0.f, 0.f}, sTbh, sTbl, LDC, R * 16, R + 1, lane);
                // O += P U
                RegB<T, NTC> Ub;
                Ub.prepare(Ut);
#pragma unroll
                for (int R = 0; R < NTC; ++R) {
                    Ot[R] = Ub.mul(Ot[R], sPh, sPl, LDC, R * 16, R + 1, lane);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = R * 16 + acc_row(lane, r);
                        if (row < nt)
                            o[(size_t)(c0 + row) * rowV + (size_t)h * DV + vc] =
                                from_f32<TO>(Ot[R][r]);
                    }
                }
                // S = diag(e^{G_n}) S + Kr^T U
#pragma unroll
                for (int rt = 0; rt < NTK; ++rt) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) Sacc[rt][r] *= sEGn[rt * 16 + acc_row(lane, r)];
                    Sacc[rt] = Ub.mul(Sacc[rt], sKrTh, sKrTl, LDC, rt * 16, NTC, lane);
                }
            }
            __syncthreads();
        }
        if (hT && owner) {
            float *dst = hT + ((size_t)unit * DK) * DV;
#pragma unroll
            for (int rt = 0; rt < NTK; ++rt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dst[(size_t)(rt * 16 + acc_row(lane, r)) * DV + vc] = Sacc[rt][r];
        }
    }
}

}  // namespace kda
