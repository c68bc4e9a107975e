// kda_epilogue.hip -- the read-out's exit path before the output projection
// ([Walkthrough] 第六站): a per-head RMSNorm of o followed by the output gate,
// channel by channel:
//     y[c] = o[c] / sqrt(mean_c' o[c']^2 + eps) * w[c] * sigmoid(gate[c])
// for every (token, head) row of dv channels.
//
// A pure stream (read o and the gate once, write y once), laid out for HBM: a
// lane owns 4 consecutive channels of a row (16 bytes of fp32 o, 8 of a bf16
// gate), the dv / 4 lanes of a row form an aligned power-of-two group inside
// the wave, so the sum of squares is a few DPP / permlane steps and a wave
// covers 64 * 4 / dv rows with fully coalesced accesses.  A workgroup handles
// kSlabs slabs of 256 consecutive vectors and every lane issues all its
// (non-temporal) loads before any arithmetic, to keep more bytes in flight.  Each lane reads all its
// inputs before it writes, so y may take the place of o or of the gate.
#include "kda_device.cuh"
#include "kda_launch.h"

namespace kda {
namespace {

template <class T> struct Vec4;
template <> struct Vec4<float> { typedef f32x4 type; };
template <> struct Vec4<bf16> { typedef bf16x4 type; };

// Two slabs with non-temporal loads and stores (o and the gate are read once, y
// is not read back here): 62.5 us for the 4096 x 96 x 128 read-out, 81% of HBM;
// one slab 75 us, four 67 us, and 73 us with cached accesses.
#ifndef KDA_EPI_SLABS
#define KDA_EPI_SLABS 2
#endif
constexpr int kSlabs = KDA_EPI_SLABS;

template <class TO_, class T, int LPR>   // o dtype, gate / y dtype, lanes per row
__global__ __launch_bounds__(256)
void norm_gate_kernel(const TO_ *__restrict__ o, const T *gate, const float *__restrict__ w,
                      float eps, float inv_dv, int64_t nvec, T *y) {
    typedef typename Vec4<TO_>::type VO;
    typedef typename Vec4<T>::type VG;
    // 4-channel vector index of slab k: i0 + 256 k.  Rows are whole lane groups,
    // slabs start at multiples of 256 and nvec is a multiple of the row length,
    // so a group is either entirely in range or entirely out: the reduction below
    // only ever mixes lanes of one row, all of them active.
    const int64_t i0 = (int64_t)blockIdx.x * (256 * kSlabs) + threadIdx.x;
    VO ov[kSlabs];
    VG gv[kSlabs];
#pragma unroll
    for (int k = 0; k < kSlabs; ++k) {
        if (i0 + 256 * k < nvec) {
            ov[k] = __builtin_nontemporal_load(reinterpret_cast<const VO *>(o) + i0 + 256 * k);
            gv[k] = __builtin_nontemporal_load(reinterpret_cast<const VG *>(gate) + i0 + 256 * k);
        }
    }
    const int c0 = (int)(threadIdx.x % LPR) * 4;   // 256 k is a multiple of LPR
    float wv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) wv[e] = w ? w[c0 + e] : 1.0f;
#pragma unroll
    for (int k = 0; k < kSlabs; ++k) {
        if (i0 + 256 * k < nvec) {
            float x[4], ss = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[e] = to_f32(ov[k][e]);
                ss += x[e] * x[e];
            }
            ss = group_sum<LPR>(ss);
            const float inv = 1.0f / sqrtf(ss * inv_dv + eps);
            VG out;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float sg = 1.0f / (1.0f + __expf(-to_f32(gv[k][e])));
                out[e] = from_f32<T>(x[e] * inv * wv[e] * sg);
            }
            __builtin_nontemporal_store(out, reinterpret_cast<VG *>(y) + i0 + 256 * k);
        }
    }
}

template <class TO_, class T>
hipError_t launch_typed(const NormGateArgs &a, hipStream_t s) {
    const int64_t nvec = a.rows * (a.dv / 4);
    if (nvec == 0) return hipSuccess;
    const dim3 grid((unsigned)((nvec + 256 * kSlabs - 1) / (256 * kSlabs)));
    const float inv_dv = 1.0f / (float)a.dv;
    switch (a.dv) {
        case 16:
            hipLaunchKernelGGL((norm_gate_kernel<TO_, T, 4>), grid, dim3(256), 0, s,
                               (const TO_ *)a.o, (const T *)a.gate, a.weight, a.eps, inv_dv, nvec,
                               (T *)a.y);
            break;
        case 32:
            hipLaunchKernelGGL((norm_gate_kernel<TO_, T, 8>), grid, dim3(256), 0, s,
                               (const TO_ *)a.o, (const T *)a.gate, a.weight, a.eps, inv_dv, nvec,
                               (T *)a.y);
            break;
        case 64:
            hipLaunchKernelGGL((norm_gate_kernel<TO_, T, 16>), grid, dim3(256), 0, s,
                               (const TO_ *)a.o, (const T *)a.gate, a.weight, a.eps, inv_dv, nvec,
                               (T *)a.y);
            break;
        case 128:
            hipLaunchKernelGGL((norm_gate_kernel<TO_, T, 32>), grid, dim3(256), 0, s,
                               (const TO_ *)a.o, (const T *)a.gate, a.weight, a.eps, inv_dv, nvec,
                               (T *)a.y);
            break;
        default:
            return hipErrorNotSupported;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_norm_gate(const NormGateArgs &a, bool o_bf16, bool y_bf16, hipStream_t s) {
    if (a.dv != 16 && a.dv != 32 && a.dv != 64 && a.dv != 128) return hipErrorNotSupported;
    if (y_bf16) return o_bf16 ? launch_typed<bf16, bf16>(a, s) : launch_typed<float, bf16>(a, s);
    return o_bf16 ? hipErrorNotSupported : launch_typed<float, float>(a, s);
}

}  // namespace kda
