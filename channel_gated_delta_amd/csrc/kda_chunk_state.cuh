// kda_chunk_state.cuh -- second kernel of the chunkwise KDA prefill: walks the
// chunks of each sequence with the state on chip (chunk algebra in
// kda_chunk_common.cuh; Tb and scale * P come from the prep kernel).
//
// Work decomposition.  One workgroup (4 waves) owns one (sequence, head, value
// slice of BV columns).  Wave w < BV/16 owns the 16 state columns [16w, 16w+16)
// of the slice: its part of the fp32 state lives in MFMA accumulator registers
// for the whole sequence, and the whole state-dependent chain of a chunk
// (E = V - Kd S, U = Tb E, O = Qd S + P U, the state update) runs inside that
// wave from registers -- an accumulator tile doubles as the B operand of the next
// product when the A fragment is read with the matching k order -- so the chain
// needs no LDS traffic of its own and no barrier.  The chunk operands
// scale q e^{G}, k e^{G}, (k e^{G_n - G})^T (all factors <= 1, exponentiated
// directly) and the split Tb, P are shared by the four waves through LDS; two
// barriers per chunk.
//
// Latency.  The inputs of chunk i+1 (q, k channel pairs, g, V in accumulator
// layout, Tb and P rows) are loaded into registers while chunk i is computed,
// with row indices clamped into the sequence so every load is unconditional;
// rows past the end are zeroed when the registers are consumed.
#pragma once

#include "kda_chunk_common.cuh"

namespace kda {

template <class T, int DK_, int BV_, int C_>
struct StateCfg {
    static constexpr int DK = DK_, BV = BV_, C = C_;
    static constexpr bool kSplit = std::is_same<T, bf16>::value;
    static constexpr int NSPLIT = kSplit ? 2 : 1;
    static constexpr int NW = 4, NT = NW * kWave;
    static constexpr int NTC = C / 16, NTK = DK / 16, NCW = BV / 16;
    static constexpr int PAD = 16 / (int)sizeof(T);
    static constexpr int LDK = DK + PAD;                        // [C][DK] operand rows
    static constexpr int LDC = C + PAD;                         // [*][C] operand rows
    static constexpr int NPC = DK / 2;                          // channel pairs
    static constexpr int NPART = (NT / NPC) < C ? (NT / NPC) : C;
    static constexpr int RP = C / NPART;                        // rows per part
    static constexpr int NTB = C * C / NT;                      // Tb / P elements per thread
    static_assert(NPART * RP == C && NCW <= NW && BV % 16 == 0 && NTB >= 1, "shape");
    static_assert(NTB == 1 || NTB % 4 == 0, "Tb rows are read in 16-byte pieces");

    static constexpr size_t al(size_t x) { return (x + 15) & ~(size_t)15; }
    static constexpr size_t szCK = al((size_t)C * LDK * sizeof(T));      // [C][DK]
    static constexpr size_t szKC = al((size_t)DK * LDC * sizeof(T));     // [DK][C]
    static constexpr size_t szCC = al((size_t)C * LDC * sizeof(T));      // [C][C]
    static constexpr size_t oQd = 0;                                // scale q e^G (hi, lo)
    static constexpr size_t oKd = oQd + NSPLIT * szCK;              // k e^G (hi, lo)
    static constexpr size_t oKrT = oKd + NSPLIT * szCK;             // (k e^{Gn-G})^T (hi, lo)
    static constexpr size_t oTb = oKrT + NSPLIT * szKC;             // Tb (hi, lo)
    static constexpr size_t oP = oTb + NSPLIT * szCC;               // scale * P (hi, lo)
    static constexpr size_t oSmall = oP + NSPLIT * szCC;
    static constexpr size_t kLds = oSmall + al((size_t)(NPART + 1) * DK * 4);
    static constexpr bool kFits = kLds <= 160 * 1024;
    // One workgroup per CU: a launch has (sequences x heads x slices) workgroups,
    // typically fewer than or about the 256 CUs, and the chain wants the registers.
    static constexpr int kMinWg = 1;
};

template <class T, class TO, int DK, int BV, int C>
__global__ __launch_bounds__(256, (StateCfg<T, DK, BV, C>::kMinWg))
void chunk_state_kernel(const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
                        const float *__restrict__ g, const float *__restrict__ tb,
                        const float *__restrict__ pm, const int32_t *__restrict__ cu_seqlens,
                        int64_t total, int H, int DV, float scale, const float *__restrict__ h0,
                        float *__restrict__ hT, TO *__restrict__ o, int units, int nslice) {
    using Cfg = StateCfg<T, DK, BV, C>;
    constexpr bool SPLIT = Cfg::kSplit;
    constexpr int NTC = Cfg::NTC, NTK = Cfg::NTK, NCW = Cfg::NCW;
    constexpr int LDK = Cfg::LDK, LDC = Cfg::LDC;
    constexpr int NPC = Cfg::NPC, NPART = Cfg::NPART, RP = Cfg::RP, NTB = Cfg::NTB;
    typedef typename Pair<T>::type T2;

    __shared__ __attribute__((aligned(16))) char smem[Cfg::kLds];
    constexpr size_t CKE = Cfg::szCK / sizeof(T), KCE = Cfg::szKC / sizeof(T);
    constexpr size_t CCE = Cfg::szCC / sizeof(T);
    T *sQdh = reinterpret_cast<T *>(smem + Cfg::oQd);
    T *sQdl = sQdh + (SPLIT ? CKE : 0);
    T *sKdh = reinterpret_cast<T *>(smem + Cfg::oKd);
    T *sKdl = sKdh + (SPLIT ? CKE : 0);
    T *sKrTh = reinterpret_cast<T *>(smem + Cfg::oKrT);
    T *sKrTl = sKrTh + (SPLIT ? KCE : 0);
    T *sTbh = reinterpret_cast<T *>(smem + Cfg::oTb);
    T *sTbl = sTbh + (SPLIT ? CCE : 0);
    T *sPh = reinterpret_cast<T *>(smem + Cfg::oP);
    T *sPl = sPh + (SPLIT ? CCE : 0);
    float *sTot = reinterpret_cast<float *>(smem + Cfg::oSmall);      // part sums of g
    float *sEGn = sTot + NPART * DK;                                   // e^{G_n}

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
    const bool owner = wave < NCW;                           // this wave owns state columns
    const int vc = v0 + (owner ? wave : 0) * 16 + (lane & 15);  // its value column

    // ---- state: tiles rt = 0..NTK-1 of rows [16 rt, 16 rt + 16), columns of this wave
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

    // channel-pair mapping of the decay phase: channels 2cp, 2cp+1, rows [part*RP, +RP)
    const int cp = tid % NPC, part = tid / NPC;
    const bool fthread = part < NPART;
    // Tb / P elements of this thread: row tr, columns [tc, tc + NTB)
    const int tr = (tid * NTB) / C, tc = (tid * NTB) % C;

    // ---- registers holding the next chunk's inputs (rows clamped into the sequence)
    T2 pq[RP], pk[RP];
    f32x2 pg[RP];
    T pv[NTC][4];            // kept in T: a conversion here would wait for the load
    float ptb[NTB], ppm[NTB];
    auto issue_loads = [&](int64_t cs) {
        const int last = (int)min((int64_t)C, eos - cs) - 1;
        if (fthread) {
#pragma unroll
            for (int j = 0; j < RP; ++j) {
                const size_t off =
                    (size_t)(cs + min(part * RP + j, last)) * rowQK + (size_t)h * DK + 2 * cp;
                pq[j] = *reinterpret_cast<const T2 *>(q + off);
                pk[j] = *reinterpret_cast<const T2 *>(k + off);
                pg[j] = *reinterpret_cast<const f32x2 *>(g + off);
            }
        }
        if (owner) {
#pragma unroll
            for (int R = 0; R < NTC; ++R)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = min(R * 16 + acc_row(lane, r), last);
                    pv[R][r] = v[(size_t)(cs + t) * rowV + (size_t)h * DV + vc];
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
    };
    if (bos < eos) issue_loads(bos);

    for (int64_t c0 = bos; c0 < eos; c0 += C) {
        const int nt = (int)min((int64_t)C, eos - c0);

        // ================= L: consume the prefetched registers (rows >= nt are zero) ====
        float qv[RP][2], kv[RP][2], gam[RP][2];
        if (fthread) {
            float a0 = 0.f, a1 = 0.f;
#pragma unroll
            for (int j = 0; j < RP; ++j) {
                const bool in = part * RP + j < nt;
                qv[j][0] = in ? to_f32(pq[j][0]) : 0.f;
                qv[j][1] = in ? to_f32(pq[j][1]) : 0.f;
                kv[j][0] = in ? to_f32(pk[j][0]) : 0.f;
                kv[j][1] = in ? to_f32(pk[j][1]) : 0.f;
                a0 += (in ? pg[j][0] : 0.f) * kLog2e;
                a1 += (in ? pg[j][1] : 0.f) * kLog2e;
                gam[j][0] = a0;
                gam[j][1] = a1;
            }
            sTot[part * DK + 2 * cp] = a0;
            sTot[part * DK + 2 * cp + 1] = a1;
        }
        float vin[NTC][4];
#pragma unroll
        for (int R = 0; R < NTC; ++R)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                vin[R][r] = (R * 16 + acc_row(lane, r) < nt) ? to_f32(pv[R][r]) : 0.f;
        float tbv[NTB], pmv[NTB];
#pragma unroll
        for (int e = 0; e < NTB; ++e) {
            tbv[e] = tr < nt ? ptb[e] : 0.f;
            pmv[e] = tr < nt ? ppm[e] : 0.f;
        }
        // the next chunk's loads fly while this chunk is computed
        if (c0 + C < eos) issue_loads(c0 + C);
        __syncthreads();

        // ================= F: chunk operands (hi, lo) and the split Tb, P ==============
        if (fthread) {
            float off[2] = {0.f, 0.f}, tot[2] = {0.f, 0.f};
            for (int p = 0; p < NPART; ++p) {
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const float s = sTot[p * DK + 2 * cp + e];
                    if (p < part) off[e] += s;
                    tot[e] += s;
                }
            }
            float krt[2][RP];
#pragma unroll
            for (int j = 0; j < RP; ++j) {
                const int r = part * RP + j;
                float eg[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const float gt = gam[j][e] + off[e];
                    eg[e] = exp2_clamped(gt);
                    krt[e][j] = kv[j][e] * exp2_clamped(tot[e] - gt);
                }
                const int i = r * LDK + 2 * cp;
                put2(sQdh, sQdl, i, qv[j][0] * eg[0] * scale, qv[j][1] * eg[1] * scale);
                put2(sKdh, sKdl, i, kv[j][0] * eg[0], kv[j][1] * eg[1]);
            }
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int base = (2 * cp + e) * LDC + part * RP;
                if constexpr (RP % 2 == 0) {
#pragma unroll
                    for (int j = 0; j < RP; j += 2) put2(sKrTh, sKrTl, base + j, krt[e][j], krt[e][j + 1]);
                } else {
#pragma unroll
                    for (int j = 0; j < RP; ++j) put1(sKrTh, sKrTl, base + j, krt[e][j]);
                }
            }
            if (part == 0) {
                sEGn[2 * cp] = exp2_clamped(tot[0]);
                sEGn[2 * cp + 1] = exp2_clamped(tot[1]);
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
        }
        __syncthreads();

        // ============ chain (state-column owners, registers only, no barriers) ============
        if (owner) {
            RegB<T, NTK> Sb;
            Sb.prepare(Sacc);
            f32x4 Et[NTC], Ot[NTC], Ut[NTC];
#pragma unroll
            for (int R = 0; R < NTC; ++R) {
                // E = V - Kd S
                const f32x4 ks = Sb.mul(f32x4{0.f, 0.f, 0.f, 0.f}, sKdh, sKdl, LDK, R * 16, NTK, lane);
#pragma unroll
                for (int r = 0; r < 4; ++r) Et[R][r] = vin[R][r] - ks[r];
                // O = Qd S
                Ot[R] = Sb.mul(f32x4{0.f, 0.f, 0.f, 0.f}, sQdh, sQdl, LDK, R * 16, NTK, lane);
            }
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
                        o[(size_t)(c0 + row) * rowV + (size_t)h * DV + vc] = from_f32<TO>(Ot[R][r]);
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
        // No barrier here: the next chunk's first barrier orders every read above
        // before the LDS writes that follow it.
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

}  // namespace kda
