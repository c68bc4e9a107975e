// kda_decode.hip -- fused, memory-bound KDA decode step (one token per sequence).
//
// Per (sequence b, head h) the step is ([Walkthrough] 第三站-第五站, update order
// decay -> predict -> correct -> read out):
//     S <- diag(a) S,  a = exp(g);  e = v - S^T k;  S <- S + beta k e^T;  o = scale S^T q.
// Expanding the read-out of the updated state gives one pass over the old S:
//     pred_j = sum_c (a_c k_c) S[c][j]
//     r_j    = sum_c (a_c q_c) S[c][j]
//     e_j    = v_j - pred_j
//     o_j    = scale * (r_j + beta e_j (k . q))
//     S'[c][j] = a_c S[c][j] + k_c (beta e_j)
// so every state element is read once and written once: the 128x128 fp32 state
// of a head (64 KiB) is loaded into registers with 16-byte coalesced loads, the
// two column reductions go through LDS, and the new state is stored in place.
// A workgroup of 1024 threads (16 waves, four rows of the state per thread) per
// head keeps more of the state in flight per CU than 256 threads with sixteen
// rows each: 74.8% against 72.0% of HBM bandwidth at 64 sequences x 96 heads.
// A barrier-free layout with one wave per 32-column slice was slower (67%):
// each of its loads touches eight rows 512 bytes apart.
// The step is bound by HBM bandwidth (2 * dk * dv * 4 bytes per head).
#include "kda_device.cuh"
#include "kda_launch.h"

namespace kda {
namespace {

template <class T, int DK, int DV>
struct DecodeCfg {
    static constexpr int kF4 = DK * DV / 4;                    // float4s per state
    static constexpr int kThreads = kF4 < 1024 ? kF4 : 1024;
    static constexpr int kColThreads = DV / 4;                 // threads across one row
    static constexpr int kRowThreads = kThreads / kColThreads; // thread rows
    static constexpr int kRowsPerThread = DK / kRowThreads;
    static_assert(kRowThreads * kRowsPerThread == DK, "row split");
};

template <class T, class TO, int DK, int DV>
__global__ __launch_bounds__(1024)
void decode_kernel(const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
                   const float *__restrict__ g, const float *__restrict__ beta,
                   float *__restrict__ state, float scale, TO *__restrict__ o) {
    using Cfg = DecodeCfg<T, DK, DV>;
    constexpr int NT = Cfg::kThreads, RT = Cfg::kRowThreads, RPT = Cfg::kRowsPerThread;
    __shared__ float s_ka[DK];        // a_c * k_c
    __shared__ float s_qa[DK];        // a_c * q_c
    __shared__ float s_a[DK];         // a_c
    __shared__ float s_k[DK];
    __shared__ float s_qk[NT / kWave + 1];
    __shared__ float s_red[2][RT][DV];
    __shared__ float s_be[DV];        // beta * e_j

    const int bh = blockIdx.x;        // (sequence, head) pair
    const int tid = threadIdx.x;
    const int cg = tid % Cfg::kColThreads;
    const int rg = tid / Cfg::kColThreads;
    float *S = state + (size_t)bh * DK * DV;

    // Issue the state loads first: RPT float4 per thread, rows rg + i*RT.
    f32x4 st[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        st[i] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4 *>(S + (size_t)(rg + i * RT) * DV) + cg);

    float qk_part = 0.f;
    for (int c = tid; c < DK; c += NT) {
        const float a = __expf(g[(size_t)bh * DK + c]);
        const float kc = to_f32(k[(size_t)bh * DK + c]);
        const float qc = to_f32(q[(size_t)bh * DK + c]);
        s_a[c] = a;
        s_k[c] = kc;
        s_ka[c] = a * kc;
        s_qa[c] = a * qc;
        qk_part += kc * qc;
    }
    qk_part = group_sum<kWave>(qk_part);
    if ((tid & (kWave - 1)) == 0) s_qk[tid / kWave] = qk_part;
    __syncthreads();

    float pred[4] = {0.f, 0.f, 0.f, 0.f}, rd[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int c = rg + i * RT;
        const float ka = s_ka[c], qa = s_qa[c];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pred[j] += ka * st[i][j];
            rd[j] += qa * st[i][j];
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        s_red[0][rg][cg * 4 + j] = pred[j];
        s_red[1][rg][cg * 4 + j] = rd[j];
    }
    __syncthreads();

    if (tid < DV) {
        float p = 0.f, r = 0.f;
#pragma unroll
        for (int i = 0; i < RT; ++i) { p += s_red[0][i][tid]; r += s_red[1][i][tid]; }
        float qk = 0.f;
#pragma unroll
        for (int i = 0; i < (NT + kWave - 1) / kWave; ++i) qk += s_qk[i];
        const float b = beta[bh];
        const float e = to_f32(v[(size_t)bh * DV + tid]) - p;
        s_be[tid] = b * e;
        o[(size_t)bh * DV + tid] = from_f32<TO>(scale * (r + b * e * qk));
    }
    __syncthreads();

    float be[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) be[j] = s_be[cg * 4 + j];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int c = rg + i * RT;
        const float a = s_a[c], kc = s_k[c];
        f32x4 n;
#pragma unroll
        for (int j = 0; j < 4; ++j) n[j] = a * st[i][j] + kc * be[j];
        __builtin_nontemporal_store(n, reinterpret_cast<f32x4 *>(S + (size_t)c * DV) + cg);
    }
}

template <class T, int DK, int DV>
hipError_t launch_typed(const DecodeArgs &a, hipStream_t s) {
    const int blocks = a.batch * a.heads;
    if (blocks == 0) return hipSuccess;
    if (a.out_f32)
        hipLaunchKernelGGL((decode_kernel<T, float, DK, DV>), dim3(blocks),
                           dim3(DecodeCfg<T, DK, DV>::kThreads), 0, s,
                           (const T *)a.q, (const T *)a.k, (const T *)a.v, a.g, a.beta, a.state,
                           a.scale, (float *)a.o);
    else
        hipLaunchKernelGGL((decode_kernel<T, T, DK, DV>), dim3(blocks),
                           dim3(DecodeCfg<T, DK, DV>::kThreads), 0, s,
                           (const T *)a.q, (const T *)a.k, (const T *)a.v, a.g, a.beta, a.state,
                           a.scale, (T *)a.o);
    return hipGetLastError();
}

template <class T, int DK>
hipError_t dispatch_dv(const DecodeArgs &a, hipStream_t s) {
    switch (a.dv) {
        case 16: return launch_typed<T, DK, 16>(a, s);
        case 32: return launch_typed<T, DK, 32>(a, s);
        case 64: return launch_typed<T, DK, 64>(a, s);
        case 128: return launch_typed<T, DK, 128>(a, s);
    }
    return hipErrorNotSupported;
}

template <class T>
hipError_t dispatch_dk(const DecodeArgs &a, hipStream_t s) {
    switch (a.dk) {
        case 16: return dispatch_dv<T, 16>(a, s);
        case 32: return dispatch_dv<T, 32>(a, s);
        case 64: return dispatch_dv<T, 64>(a, s);
        case 128: return dispatch_dv<T, 128>(a, s);
    }
    return hipErrorNotSupported;
}

}  // namespace

hipError_t launch_decode_step(const DecodeArgs &a, bool bf16, hipStream_t s) {
    return bf16 ? dispatch_dk<kda::bf16>(a, s) : dispatch_dk<float>(a, s);
}

}  // namespace kda
