// kda_chunk_state.cuh -- second kernel of the chunkwise KDA prefill: walks the
// chunks of each sequence with the state on chip (chunk algebra in
// kda_chunk_common.cuh; Tb and scale * P come from the prep kernel).
//
// Work decomposition.  One workgroup owns one (sequence, head, value slice of BV
// columns: 64, or all 128 when there are more workgroups than CUs) and runs two
// pipelines that meet at one barrier per step:
//  * consumer waves 0 .. BV/16-1: wave w owns the 16 state columns [16w, 16w+16)
//    of the slice.  Its part of the fp32 state lives in MFMA accumulator
//    registers for the whole sequence, and the state-dependent chain of a chunk
//    (E = V - Kd S, U = Tb E, O = Qd S + P U, the state update) runs inside that
//    wave from registers -- an accumulator tile doubles as the B operand of the
//    next product when the A fragment is read with the matching k order.
//  * the producer waves after them (4 of them) build the next chunk's operands
//    in the other half of a
//    double-buffered LDS stage: q e^{G}, k e^{G} and (k e^{G_n - G})^T
//    (all factors <= 1, exponentiated directly), the split Tb and P rows, V and
//    e^{G_n}.  A producer lane owns two key channels of a group of rows; the
//    in-chunk prefix of the log-decay over row groups is a few lane shuffles,
//    so the producers need no barrier of their own.
// At step s the producers fill stage s & 1 with chunk s while the consumers run
// chunk s-1 from stage (s-1) & 1; the barrier at the end of the step hands the
// stage over.  Producers load chunk s+1 into registers during step s.
#pragma once

#include "kda_chunk_common.cuh"

#ifndef KDA_STATE_NPW
#define KDA_STATE_NPW 4
#endif

namespace kda {

template <class T, int DK_, int BV_, int C_>
struct StateCfg {
    static constexpr int DK = DK_, BV = BV_, C = C_;
    static constexpr bool kSplit = std::is_same<T, bf16>::value;
    static constexpr int NSPLIT = kSplit ? 2 : 1;
    // producer waves (KDA_STATE_NPW for dk >= 64 and 16-token chunks); threads: NCS
    // consumer wave slots, then the producers
    static_assert(C == 16, "chunks are 16 tokens");
    static constexpr int NPW = DK >= 64 ? KDA_STATE_NPW : 4;
    static constexpr int NTC = C / 16, NTK = DK / 16, NCW = BV / 16;
    // consumer wave slots (waves 0 .. NCS-1; slices narrower than 64 columns leave
    // some idle), then the producers
    static constexpr int NCS = NCW > 4 ? NCW : 4;
    static constexpr int NT = (NCS + NPW) * kWave;
    // Row pitch padding (elements).  For bf16 the pitches come out at 2 (mod 32)
    // dwords, so the 16 rows one LDS cycle serves fall in 16 different bank pairs
    // (an 8-element pad would map rows r and r + 8 to the same banks); fragments are
    // 8-byte loads, so 8-byte row alignment suffices.
    static constexpr int PAD = 4;
    static constexpr int LDK = DK + PAD;                        // [C][DK] operand rows
    static constexpr int LDC = C + PAD;                         // [*][C] operand rows
    static constexpr int LDV = BV + 4;                          // fp32 [C][BV] rows
    // producer lane mapping: CPW channel pairs x RG row groups of RP rows per wave
    static constexpr int CPW = DK / 2 / NPW;
    static constexpr int RG = (kWave / CPW) < C ? (kWave / CPW) : C;
    static constexpr int RP = C / RG;
    static constexpr int NPT = NPW * kWave;                     // producer threads
    // Tb / P and V elements per thread; with more producer threads than elements
    // only the first C*C (C*BV) / NTB (NVE) threads take part
    static constexpr int NTB = C * C / NPT > 0 ? C * C / NPT : 1;
    static constexpr int NVE = C * BV / NPT > 0 ? C * BV / NPT : 1;
    static_assert(CPW >= 1 && RG * RP == C && NCW <= 8 && BV % 16 == 0, "shape");
    static_assert(NTB >= 1 && (NTB == 1 || NTB % 4 == 0) && NVE >= 1, "shape");

    // bf16 with dk a multiple of 32 (the register-B chain below): the 16-deep
    // operands (Kr^T, Tb, P) hold hi and lo interleaved by
    // 4-token group -- group g of a row is hi[4g..4g+3] then lo[4g..4g+3] -- so one
    // 16-byte read is the [hi | lo] operand of a 16x16x32 product.  The pitch, 2C + 8
    // elements (20 dwords), puts 8 consecutive rows on distinct banks.
    static constexpr int LDG = 2 * C + 8;
    static constexpr bool kIL = kSplit && DK % 32 == 0;   // the register-B chain's layout

    static constexpr size_t al(size_t x) { return (x + 15) & ~(size_t)15; }
    static constexpr size_t szCK = al((size_t)C * LDK * sizeof(T));      // [C][DK]
    static constexpr size_t szKC = al((size_t)DK * LDC * sizeof(T));     // [DK][C]
    static constexpr size_t szCC = al((size_t)C * LDC * sizeof(T));      // [C][C]
    static constexpr size_t szKrT = kIL ? al((size_t)DK * LDG * sizeof(T)) : NSPLIT * szKC;
    static constexpr size_t szTbP = kIL ? al((size_t)C * LDG * sizeof(T)) : NSPLIT * szCC;
    static constexpr size_t oQd = 0;                                // q e^G (hi, lo)
    static constexpr size_t oKd = oQd + NSPLIT * szCK;              // k e^G (hi, lo)
    static constexpr size_t oKrT = oKd + NSPLIT * szCK;             // (k e^{Gn-G})^T
    static constexpr size_t oTb = oKrT + szKrT;                     // Tb
    static constexpr size_t oP = oTb + szTbP;                       // scale * P
    static constexpr size_t oV = oP + szTbP;                        // V (fp32)
    static constexpr size_t oEGn = oV + al((size_t)C * LDV * 4);    // e^{G_n}
    static constexpr size_t kStage = oEGn + al((size_t)DK * 4);
    static constexpr size_t kLds = 2 * kStage;
    static constexpr bool kFits = kLds <= 160 * 1024;
};

// A fragments (hi, lo) in the permuted k order of the register-B products.
struct AF8 { bf16x8 h, l; };

__device__ __forceinline__ AF8 lda8(const bf16 *Mh, const bf16 *Ml, int ld, int row0, int k0,
                                    int lane) {
    AF8 f;
    afrag8(Mh, Ml, ld, row0, k0, lane, f.h, f.l);
    return f;
}

// The state chain of one 16-token chunk for one consumer wave, bf16 operands and
// dk a multiple of 32.  Written as explicit stages whose LDS fragment loads are
// issued one stage ahead of the products that use them (scheduling barriers keep
// the compiler from sinking the loads next to their first use, which would
// expose the LDS latency at every product).
//
// The read-out is formed transposed, O^T = S^T (q e^G)^T + U^T (scale P)^T: the
// MFMA operand layouts of A and B mirror each other, so the same registers serve
// with the operands swapped, and the accumulator then holds 4 consecutive value
// columns of one token per lane -- one 16-byte store instead of four scattered
// ones.  Ot[r] is O[token lane & 15][wcol + 4 (lane >> 4) + r].
// The 16-deep products (U = Tb E, P U, the state update) take their three split
// terms in two instructions: one operand as [hi | lo] read in one piece, the
// other's hi duplicated into both halves, so one 16x16x32 product sums two terms
// over a lane's 8 k slots (16x16x32 costs what 16x16x16 costs on this GPU), and a
// 16x16x16 product adds the third.
__device__ __forceinline__ bf16x4 lo_half(const bf16x8 &x) {
    return __builtin_shufflevector(x, x, 0, 1, 2, 3);
}
__device__ __forceinline__ bf16x8 twice(const bf16x4 &x) {
    return __builtin_shufflevector(x, x, 0, 1, 2, 3, 0, 1, 2, 3);
}
// Row `row0 + (lane & 15)`, group lane >> 4 of an interleaved [rows][LDG] operand.
template <int LDG>
__device__ __forceinline__ bf16x8 ldg8(const bf16 *M, int row0, int lane) {
    return *reinterpret_cast<const bf16x8 *>(M + (row0 + (lane & 15)) * LDG + (lane >> 4) * 8);
}

template <int DK, int LDK, int LDG, int LDV>
__device__ __forceinline__ void state_chain_bf16(
    f32x4 (&Sacc)[DK / 16], BReg8 (&sb)[DK / 32], f32x4 &Ot, const bf16 *sQdh, const bf16 *sQdl,
    const bf16 *sKdh, const bf16 *sKdl, const bf16 *sKrT, const bf16 *sTb, const bf16 *sP,
    const float *sV, const float *sEGn, float scale, int wcol, int lane) {
    constexpr int NTK = DK / 16, NKB = DK / 32;
    static_assert(DK % 32 == 0, "shape");
    // small operands first: Tb / P fragments and V
    const bf16x8 tb8 = ldg8<LDG>(sTb, 0, lane), p8 = ldg8<LDG>(sP, 0, lane);
    float vin[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) vin[r] = sV[acc_row(lane, r) * LDV + wcol + (lane & 15)];
    AF8 fk[2], fq[2];
    fk[0] = lda8(sKdh, sKdl, LDK, 0, 0, lane);
    fq[0] = lda8(sQdh, sQdl, LDK, 0, 0, lane);

    // E = Kd S, O = Qd S: k-block j's products while block j+1 loads.  The three
    // split terms accumulate in place (an MFMA that depends on the one before it
    // issues at the same rate), E and O products alternating.
    f32x4 Et = f32x4{0.f, 0.f, 0.f, 0.f};
    Ot = f32x4{0.f, 0.f, 0.f, 0.f};
    // The state is split into (hi, lo) B operands here, block by block: block j+1's
    // split runs beside block j's products instead of after the previous update.
    sb[0] = breg8(Sacc[0], Sacc[1]);
#pragma unroll
    for (int j = 0; j < NKB; ++j) {
        const int cur = j & 1, nxt = cur ^ 1;
        if (j + 1 < NKB) {
            fk[nxt] = lda8(sKdh, sKdl, LDK, 0, 32 * (j + 1), lane);
            fq[nxt] = lda8(sQdh, sQdl, LDK, 0, 32 * (j + 1), lane);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (j + 1 < NKB) sb[j + 1] = breg8(Sacc[2 * j + 2], Sacc[2 * j + 3]);
        Et = mma(fk[cur].h, sb[j].h, Et);
        Ot = mma(sb[j].h, fq[cur].h, Ot);
        Et = mma(fk[cur].h, sb[j].l, Et);
        Ot = mma(sb[j].l, fq[cur].h, Ot);
        Et = mma(fk[cur].l, sb[j].h, Et);
        Ot = mma(sb[j].h, fq[cur].l, Ot);
        __builtin_amdgcn_sched_barrier(0);
    }
    // first half of the state-update fragments load during the U and P U products
    constexpr int NK1 = NTK / 2;
    bf16x8 fr8[NTK];
#pragma unroll
    for (int rt = 0; rt < NK1; ++rt) fr8[rt] = ldg8<LDG>(sKrT, rt * 16, lane);
    __builtin_amdgcn_sched_barrier(0);
    // E = V - Kd S;  U = Tb E;  O = scale Qd S (the stage holds q e^G unscaled)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        Et[r] = vin[r] - Et[r];
        Ot[r] *= scale;
    }
    const BReg4 eb = breg4(Et);
    f32x4 Ut = mma(tb8, twice(eb.h), f32x4{0.f, 0.f, 0.f, 0.f});
    Ut = mma(lo_half(tb8), eb.l, Ut);
    const BReg4 ub4 = breg4(Ut);
    const bf16x8 uhh = twice(ub4.h);
    // O^T += [U_h | U_h] [P_h | P_l]^T + U_l P_h^T, each product into fresh
    // registers (a zero accumulator cannot overlap the running one) and added
    const f32x4 pu1 = mma(uhh, p8, f32x4{0.f, 0.f, 0.f, 0.f});
    const f32x4 pu2 = mma(ub4.l, lo_half(p8), f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int r = 0; r < 4; ++r) Ot[r] += pu1[r] + pu2[r];
    __builtin_amdgcn_sched_barrier(0);
    // second half of the fragments load during the first half's products
#pragma unroll
    for (int rt = NK1; rt < NTK; ++rt) fr8[rt] = ldg8<LDG>(sKrT, rt * 16, lane);
    f32x4 eg[NTK];
#pragma unroll
    for (int rt = 0; rt < NTK; ++rt)
        eg[rt] = *reinterpret_cast<const f32x4 *>(sEGn + rt * 16 + (lane >> 4) * 4);
    __builtin_amdgcn_sched_barrier(0);
    // S = diag(e^{G_n}) S + Kr^T U (term-major over the NTK accumulators)
#pragma unroll
    for (int rt = 0; rt < NTK; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) Sacc[rt][r] *= eg[rt][r];
#pragma unroll
    for (int rt = 0; rt < NTK; ++rt) Sacc[rt] = mma(fr8[rt], uhh, Sacc[rt]);
#pragma unroll
    for (int rt = 0; rt < NTK; ++rt) Sacc[rt] = mma(lo_half(fr8[rt]), ub4.l, Sacc[rt]);
}

template <class T, class TO, int DK, int BV, int C, int GM>
__global__ __launch_bounds__((StateCfg<T, DK, BV, C>::NT), 1)
void chunk_state_kernel(const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
                        GateSrc gs, const float *__restrict__ tb,
                        const float *__restrict__ pm, const int32_t *__restrict__ cu_seqlens,
                        int64_t total, int H, int DV, float scale, const float *__restrict__ h0,
                        float *__restrict__ hT, TO *__restrict__ o, int units, int nslice,
                        const int32_t *__restrict__ order) {
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
    const int pos = (slot / nslice) * 8 + xcd;    // position in the dispatch order
    if (pos >= units) return;
    // Packed batches (given `order`) take their sequences longest first.
    const int n = order ? order[pos / H] : pos / H, h = pos % H;
    const int unit = n * H + h;
    const int64_t bos = chunk_seq_off(cu_seqlens, n, total);
    const int64_t eos = max(chunk_seq_off(cu_seqlens, n + 1, total), bos);
    const int nchunks = (int)((eos - bos + C - 1) / C);
    const int nsteps = (nchunks + 2) & ~1;   // steps 1..nchunks consume chunks 0..nchunks-1
    const int v0 = slice * BV;
    const size_t rowQK = (size_t)H * DK, rowV = (size_t)H * DV;

    if (wave >= Cfg::NCS) {
        // =============================== producers ===============================
        const int pt = tid - Cfg::NCS * kWave;                // 0 .. 255
        const int pw = wave - Cfg::NCS;
        const int cpair = pw * CPW + (lane % CPW);            // channels 2cpair, 2cpair+1
        float gc1 = 0.f, gc2a = 0.f, gc2b = 0.f, glb = 0.f;   // fused gate constants
        if constexpr (GM == kGateFused) {
            gc1 = gate_c1(gs, h);
            gc2a = gate_c2(gs, gc1, h, DK, 2 * cpair);
            gc2b = gate_c2(gs, gc1, h, DK, 2 * cpair + 1);
            glb = gs.lb * kLog2e;
        }
        const int rg = lane / CPW;                            // row group: rows rg*RP + j
        const bool act = rg < RG;
        const int tr = (pt * NTB) / C, tc = (pt * NTB) % C;   // Tb / P: row tr, cols tc..
        const int vr = (pt * NVE) / BV, vcol = (pt * NVE) % BV;  // V: row vr, cols vcol..
        const bool tb_act = tr < C, v_act = vr < C;           // (rows >= C: no part)

        // Two register sets for the prefetched inputs, used alternately: the loads
        // for chunk s+1 never target registers still holding chunk s, so no copy
        // (and no wait for the loads) is needed between steps.
        constexpr int NTB4 = NTB >= 4 ? NTB / 4 : 1;
        struct Regs {
            T2 q[RP], k[RP];
            // g (two channels), the gate's z, or the per-head decay of the row
            typename std::conditional<GM == kGateFused, T2,
                typename std::conditional<GM == kGateHead, float, f32x2>::type>::type g[RP];
            f32x4 tb[NTB4], pm[NTB4];   // NTB == 1 uses element 0 of the first vector
            TV v;
        };
        // Chunk bases are uniform 64-bit pointers; per-lane offsets inside a chunk
        // fit 32 bits (rows < C), which keeps the address arithmetic scalar.
        auto load_small = [&](Regs &R, int64_t cs) {
            const int last = (int)min((int64_t)C, eos - cs) - 1;
            const float *tbb = tb + ((size_t)cs * H + h) * C;
            const float *pmb = pm + ((size_t)cs * H + h) * C;
            const uint32_t wo = ((uint32_t)min(tr, last) * (uint32_t)(H * C) + (uint32_t)tc) * 4u;
            if constexpr (NTB == 1) {
                R.tb[0][0] = ld_off<float>(tbb, wo);
                R.pm[0][0] = ld_off<float>(pmb, wo);
            } else {
#pragma unroll
                for (int j = 0; j < NTB4; ++j) {
                    R.tb[j] = ld_off<f32x4>(tbb, wo + 16u * j);
                    R.pm[j] = ld_off<f32x4>(pmb, wo + 16u * j);
                }
            }
            const T *vb = v + (size_t)cs * rowV + (size_t)h * DV + v0;
            R.v = ld_off<TV>(vb, ((uint32_t)min(vr, last) * (uint32_t)rowV + (uint32_t)vcol) *
                                     (uint32_t)sizeof(T));
        };
        auto load_row = [&](Regs &R, int64_t cs, int j) {
            if (!act) return;
            const int last = (int)min((int64_t)C, eos - cs) - 1;
            const size_t bq = (size_t)cs * rowQK + (size_t)h * DK;
            const uint32_t row = (uint32_t)min(rg * RP + j, last);
            const uint32_t off = row * (uint32_t)rowQK + (uint32_t)(2 * cpair);
            R.q[j] = ld_off<T2>(q + bq, off * (uint32_t)sizeof(T));
            R.k[j] = ld_off<T2>(k + bq, off * (uint32_t)sizeof(T));
            if constexpr (GM == kGateFused)
                R.g[j] = ld_off<T2>(static_cast<const T *>(gs.z) + bq, off * (uint32_t)sizeof(T));
            else if constexpr (GM == kGateHead)
                R.g[j] = ld_off<float>(gs.g + (size_t)cs * H + h, row * (uint32_t)H * 4u);
            else
                R.g[j] = ld_off<f32x2>(gs.g + bq, off * 4u);
        };
        auto load_all = [&](Regs &R, int64_t cs) {
            load_small(R, cs);
#pragma unroll
            for (int j = 0; j < RP; ++j) load_row(R, cs, j);
        };

        // Element (row, token t) of an interleaved split operand (bf16 only).
        auto put_il = [&](T *M, int row, int t, float x) {
            if constexpr (Cfg::kIL) {
                T *p = M + row * Cfg::LDG + (t >> 2) * 8 + (t & 3);
                split2(x, p[0], p[4]);
            }
        };

        // Step s: build stage s & 1 from chunk s (if s < nchunks) out of `cur`, and
        // load chunk s+1 (clamped to the last chunk) into `nxt`.
        auto step = [&](Regs &cur, Regs &nxt, int s) {
            const bool work = s < nchunks;
            const int64_t cs = bos + (int64_t)s * C;
            const int nt = work ? (int)min((int64_t)C, eos - cs) : 0;
            // Rows past the end of the sequence (nt <= row < C) hold a copy of the last
            // row.  Only g (so the decay stops there) and the Tb, P rows are zeroed:
            // zero rows of Tb make U zero there, which removes every other
            // contribution of those rows (V, k e^G, k e^{Gn-G}); their rows of
            // q e^G only produce outputs that are never stored.
            float qv[RP][2], kv[RP][2], gam[RP][2];
            float a0 = 0.f, a1 = 0.f;
#pragma unroll
            for (int j = 0; j < RP; ++j) {
                const bool in = rg * RP + j < nt;
                qv[j][0] = to_f32(cur.q[j][0]);
                qv[j][1] = to_f32(cur.q[j][1]);
                kv[j][0] = to_f32(cur.k[j][0]);
                kv[j][1] = to_f32(cur.k[j][1]);
                if constexpr (GM == kGateFused) {
                    a0 += in ? gate_log2(to_f32(cur.g[j][0]), gc1, gc2a, glb) : 0.f;
                    a1 += in ? gate_log2(to_f32(cur.g[j][1]), gc1, gc2b, glb) : 0.f;
                } else if constexpr (GM == kGateHead) {
                    const float xh = (in ? cur.g[j] : 0.f) * kLog2e;
                    a0 += xh;
                    a1 += xh;
                } else {
                    a0 += (in ? cur.g[j][0] : 0.f) * kLog2e;
                    a1 += (in ? cur.g[j][1] : 0.f) * kLog2e;
                }
                gam[j][0] = a0;
                gam[j][1] = a1;
            }
            float tbv[NTB], pmv[NTB];
#pragma unroll
            for (int e = 0; e < NTB; ++e) {
                tbv[e] = tr < nt ? cur.tb[e / 4][e % 4] : 0.f;
                pmv[e] = tr < nt ? cur.pm[e / 4][e % 4] : 0.f;
            }
            float vv[NVE];
#pragma unroll
            for (int e = 0; e < NVE; ++e) vv[e] = to_f32(cur.v[e]);
            // `cur` was loaded a step ago: wait for it explicitly before the next loads
            // are issued (vmcnt(0) here costs nothing).  Global loads and stores share
            // one in-order counter, so a wait placed after the new loads -- where the
            // compiler would put it, at the first use of `cur` -- also waits for them.
            // The next chunk's loads are all issued here, a whole step ahead of their
            // use (issued later, their latency shows at the next step's start).  A
            // step without a chunk is followed only by steps without one, so it
            // loads nothing.
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0), expcnt and lgkmcnt untouched
            if (!work) return;
            load_all(nxt, bos + (int64_t)min(s + 1, nchunks - 1) * C);
            // Pin the loads here: the step barriers order LDS only, so without a
            // compiler memory barrier the loads would be sunk to their use in the
            // next step and their latency exposed there.
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);

            char *st = smem + (s & 1) * Cfg::kStage;
            T *sQdh = reinterpret_cast<T *>(st + Cfg::oQd), *sQdl = sQdh + (SPLIT ? CKE : 0);
            T *sKdh = reinterpret_cast<T *>(st + Cfg::oKd), *sKdl = sKdh + (SPLIT ? CKE : 0);
            T *sKrTh = reinterpret_cast<T *>(st + Cfg::oKrT), *sKrTl = sKrTh + (SPLIT ? KCE : 0);
            T *sTbh = reinterpret_cast<T *>(st + Cfg::oTb), *sTbl = sTbh + (SPLIT ? CCE : 0);
            T *sPh = reinterpret_cast<T *>(st + Cfg::oP), *sPl = sPh + (SPLIT ? CCE : 0);
            float *sV = reinterpret_cast<float *>(st + Cfg::oV);
            float *sEGn = reinterpret_cast<float *>(st + Cfg::oEGn);
            if (tb_act) {
                if constexpr (Cfg::kIL) {
#pragma unroll
                    for (int e = 0; e < NTB; ++e) {
                        put_il(sTbh, tr, tc + e, tbv[e]);
                        put_il(sPh, tr, tc + e, pmv[e]);
                    }
                } else {
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
            }
            if (v_act) {
#pragma unroll
                for (int e = 0; e < NVE; ++e) sV[vr * LDV + vcol + e] = vv[e];
            }

            // prefix of the row-group sums (lanes rg*CPW + i share a channel pair)
            float inc0 = a0, inc1 = a1, tot0, tot1;
            if constexpr (CPW == 16 && RG == 4) {   // row groups are the 16-lane rows
                rows4_prefix(a0, rg, inc0, tot0);
                rows4_prefix(a1, rg, inc1, tot1);
            } else {
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
                tot0 = __shfl(inc0, lastl, kWave);
                tot1 = __shfl(inc1, lastl, kWave);
            }
            const float off0 = inc0 - a0, off1 = inc1 - a1;

            if (act) {
                float krt[2][RP];
#pragma unroll
                for (int j = 0; j < RP; ++j) {
                    const float g0 = gam[j][0] + off0, g1 = gam[j][1] + off1;
                    // all exponents are <= 0 for g <= 0 (the gate's contract)
                    const float e0 = exp2_nonpos(g0), e1 = exp2_nonpos(g1);
                    krt[0][j] = kv[j][0] * exp2_nonpos(tot0 - g0);
                    krt[1][j] = kv[j][1] * exp2_nonpos(tot1 - g1);
                    const int i = (rg * RP + j) * LDK + 2 * cpair;
                    put2(sQdh, sQdl, i, qv[j][0] * e0, qv[j][1] * e1);
                    put2(sKdh, sKdl, i, kv[j][0] * e0, kv[j][1] * e1);
                }
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int ch = 2 * cpair + e;
                    if constexpr (Cfg::kIL && RP == 4) {
                        // the lane's 4 rows are token group rg: one 16-byte write
                        bf16x2 h01, l01, h23, l23;
                        split_pair(krt[e][0], krt[e][1], h01, l01);
                        split_pair(krt[e][2], krt[e][3], h23, l23);
                        *reinterpret_cast<u32x4 *>(sKrTh + ch * Cfg::LDG + rg * 8) =
                            u32x4{bits(h01), bits(h23), bits(l01), bits(l23)};
                    } else if constexpr (Cfg::kIL) {
#pragma unroll
                        for (int j = 0; j < RP; ++j) put_il(sKrTh, ch, rg * RP + j, krt[e][j]);
                    } else {
                        const int base = ch * LDC + rg * RP;
                        if constexpr (RP % 2 == 0) {
#pragma unroll
                            for (int j = 0; j < RP; j += 2)
                                put2(sKrTh, sKrTl, base + j, krt[e][j], krt[e][j + 1]);
                        } else {
#pragma unroll
                            for (int j = 0; j < RP; ++j) put1(sKrTh, sKrTl, base + j, krt[e][j]);
                        }
                    }
                }
                if (rg == 0) {
                    sEGn[2 * cpair] = exp2_nonpos(tot0);
                    sEGn[2 * cpair + 1] = exp2_nonpos(tot1);
                }
            }
        };

        Regs A, B;
        if (nchunks > 0) load_all(A, bos);
        // nsteps = nchunks + 1 rounded up to even; one barrier per step
        for (int s = 0; s < nsteps; s += 2) {
            step(A, B, s);
            lds_barrier();
            step(B, A, s + 1);
            lds_barrier();
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
        // Wait for the h0 loads here, once.  The memory counter also counts this
        // wave's output stores, and a load still pending into the state registers
        // at the loop entry would make the compiler wait for the counter inside the
        // loop -- for the previous step's stores to complete, at every step.
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0), expcnt and lgkmcnt untouched
        // (hi, lo) B operands of the state, built block by block inside each chain
        constexpr int NKB = DK / 32 > 0 ? DK / 32 : 1;
        BReg8 sbs[NKB];
        // Step s consumes chunk s-1 from stage (s-1) & 1; the loop runs steps in pairs so
        // that the stage (and every LDS address below) is a constant of the code.
        auto cstep = [&](int s, const int stage) {
            if (s >= 1 && s <= nchunks && owner) {
                const int64_t c0 = bos + (int64_t)(s - 1) * C;
                const int nt = (int)min((int64_t)C, eos - c0);
                const char *st = smem + stage * Cfg::kStage;
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

                if constexpr (SPLIT && DK % 32 == 0) {
                    f32x4 Ot;
                    state_chain_bf16<DK, LDK, Cfg::LDG, LDV>(Sacc, sbs, Ot, sQdh, sQdl, sKdh,
                                                             sKdl, sKrTh, sTbh, sPh, sV, sEGn,
                                                             scale, wave * 16, lane);
                    // Ot holds token lane & 15, value columns oc .. oc + 3
                    TO *ob = o + (size_t)c0 * rowV + (size_t)h * DV;
                    const int tok = lane & 15;
                    const int oc = v0 + wave * 16 + (lane >> 4) * 4;
                    if (tok < nt) {
                        typedef TO TO4 __attribute__((ext_vector_type(4)));
                        TO4 ov;
#pragma unroll
                        for (int r = 0; r < 4; ++r) ov[r] = from_f32<TO>(Ot[r]);
                        st_off<TO4>(ob, ((uint32_t)tok * (uint32_t)rowV + (uint32_t)oc) *
                                            (uint32_t)sizeof(TO), ov);
                    }
                } else {
                RegB<T, NTK> Sb;
                Sb.prepare(Sacc);
                f32x4 Et[NTC], Ot[NTC], Ut[NTC];
                // E = V - Kd S and O = scale Qd S
#pragma unroll
                for (int R = 0; R < NTC; ++R) {
                    Et[R] = Sb.mul(f32x4{0.f, 0.f, 0.f, 0.f}, sKdh, sKdl, LDK, R * 16, NTK, lane);
                    Ot[R] = Sb.mul(f32x4{0.f, 0.f, 0.f, 0.f}, sQdh, sQdl, LDK, R * 16, NTK, lane);
#pragma unroll
                    for (int r = 0; r < 4; ++r) Ot[R][r] *= scale;
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
            }
        };
        for (int s = 0; s < nsteps; s += 2) {   // nsteps is even
            cstep(s, 1);
            lds_barrier();
            cstep(s + 1, 0);
            lds_barrier();
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
