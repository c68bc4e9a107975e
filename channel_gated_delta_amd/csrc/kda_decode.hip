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
//
// The conv variant (kda_decode_step_conv) runs the token's prologue in the same
// workgroup first ([Walkthrough] 第二站: width-4 causal conv over the conv
// cache, SiLU, then q and k scaled to unit length): one thread per channel of
// q | k | v of the head computes its conv from the three cached inputs and this
// token's raw projection, shifts the cache by one, and the L2 sums of squares
// are reduced over the workgroup.  q, k and v stay in fp32 on chip.
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

// Width-4 conv of one channel for the fused step.  conv_load reads the history
// h0..h2 (oldest first), the current raw input and the weights (w[3] multiplies
// the current input); conv_finish returns SiLU of the conv and shifts the cache
// by one in place (this thread owns the channel).  The loads are issued before
// the state loads, so the conv waits only for its own inputs.
template <class T>
struct ConvTap {
    T x[4], w[4];   // h0, h1, h2, x_t and the channel's weights
    T *cache;
    size_t row;
};
template <class T>
__device__ __forceinline__ void conv_load(ConvTap<T> &c, const T *__restrict__ x,
                                          const T *__restrict__ w, T *cache, size_t row,
                                          size_t ch) {
    c.x[0] = cache[ch];
    c.x[1] = cache[row + ch];
    c.x[2] = cache[2 * row + ch];
    c.x[3] = x[ch];
#pragma unroll
    for (int i = 0; i < 4; ++i) c.w[i] = w[ch * 4 + i];
    c.cache = cache + ch;
    c.row = row;
}
template <class T>
__device__ __forceinline__ float conv_value(const ConvTap<T> &c) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc += to_f32(c.w[i]) * to_f32(c.x[i]);
    return acc / (1.0f + expf(-acc));
}
template <class T>
__device__ __forceinline__ void conv_shift(const ConvTap<T> &c) {
    c.cache[0] = c.x[1];
    c.cache[c.row] = c.x[2];
    c.cache[2 * c.row] = c.x[3];
}

template <class T, class TO, int DK, int DV, bool CONV, bool HG>   // HG: g is [B, H]
__global__ __launch_bounds__(1024)
void decode_kernel(const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
                   const float *__restrict__ g, const float *__restrict__ beta,
                   float *__restrict__ state, float scale, TO *__restrict__ o, DecodeConvIn cv) {
    using Cfg = DecodeCfg<T, DK, DV>;
    constexpr int NT = Cfg::kThreads, RT = Cfg::kRowThreads, RPT = Cfg::kRowsPerThread;
    static_assert(!CONV || 2 * DK + DV <= NT, "one thread per conv channel");
    __shared__ float s_ka[DK];        // a_c * k_c
    __shared__ float s_qa[DK];        // a_c * q_c
    __shared__ float s_a[DK];         // a_c
    __shared__ float s_k[DK];
    __shared__ float s_qk[NT / kWave + 1];
    __shared__ float s_red[2][RT][DV];
    __shared__ float s_be[DV];        // beta * e_j
    __shared__ float s_x[CONV ? 2 * DK + DV : 1];       // conv + SiLU of q | k | v
    __shared__ float s_ss[2][CONV ? NT / kWave + 1 : 1];  // sums of squares of q, k

    const int bh = blockIdx.x;        // (sequence, head) pair
    const int tid = threadIdx.x;
    const int cg = tid % Cfg::kColThreads;
    const int rg = tid / Cfg::kColThreads;
    float *S = state + (size_t)bh * DK * DV;

    // The per-head inputs: a thread owns key channel tid (threads DK and up load
    // channel DK-1 again and use nothing), so the loads need no branch.
    static_assert(NT >= DK, "one thread per key channel");
    const size_t kc_off = (size_t)bh * DK + min(tid, DK - 1);
    const float g_in = HG ? g[bh] : g[kc_off];
    T q_in{}, k_in{};
    if constexpr (!CONV) {
        q_in = q[kc_off];
        k_in = k[kc_off];
    }

    // Fused conv: this thread's channel of q | k | v.  Threads 2 DK + DV and up own
    // none; they load the last v channel again and store nothing.  These loads are
    // issued before the state's and need no branch, so the conv arithmetic waits
    // only for them (the memory counter is in order) and overlaps the state's
    // arrival; a branch would make the compiler wait for them at its end.
    ConvTap<T> tap{};
    const bool has_ch = CONV && tid < 2 * DK + DV;
    const int which = tid >= 2 * DK ? 2 : tid / DK;   // 0: q, 1: k, 2: v
    if constexpr (CONV) {
        const int b = bh / cv.heads, h = bh % cv.heads;
        const int D = which == 2 ? DV : DK;
        const int c = which == 2 ? min(tid - 2 * DK, DV - 1) : tid % DK;
        const size_t row = (size_t)cv.heads * D, ch = (size_t)h * D + c;
        const T *x = static_cast<const T *>(which == 0 ? cv.xq : which == 1 ? cv.xk : cv.xv);
        const T *w = static_cast<const T *>(which == 0 ? cv.wq : which == 1 ? cv.wk : cv.wv);
        T *cache = static_cast<T *>(which == 0 ? cv.cq : which == 1 ? cv.ck : cv.cv);
        conv_load(tap, x + (size_t)b * row, w, cache + (size_t)b * 3 * row, row, ch);
    }

    // Issue the state loads next: RPT float4 per thread, rows rg + i*RT.  Compiler
    // barriers keep the conv loads above these and the conv arithmetic below.
    asm volatile("" ::: "memory");
    f32x4 st[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        st[i] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4 *>(S + (size_t)(rg + i * RT) * DV) + cg);
    __builtin_amdgcn_sched_barrier(0);

    float inv_q = 1.f, inv_k = 1.f;
    if constexpr (CONV) {
        // every lane computes (lanes without a channel on a copy): the loads are then
        // consumed on one straight path, and only the stores depend on the channel
        const float y = conv_value(tap);
        const float sq = has_ch && which == 0 ? y * y : 0.f;
        const float sk = has_ch && which == 1 ? y * y : 0.f;
        if (has_ch) {
            s_x[tid] = y;
            conv_shift(tap);
        }
        const float wsq = group_sum<kWave>(sq), wsk = group_sum<kWave>(sk);
        if ((tid & (kWave - 1)) == 0) {
            s_ss[0][tid / kWave] = wsq;
            s_ss[1][tid / kWave] = wsk;
        }
        __syncthreads();
        float nq = 0.f, nk = 0.f;
#pragma unroll
        for (int i = 0; i < (NT + kWave - 1) / kWave; ++i) {
            nq += s_ss[0][i];
            nk += s_ss[1][i];
        }
        inv_q = 1.0f / sqrtf(nq + cv.eps);
        inv_k = 1.0f / sqrtf(nk + cv.eps);
    }

    float qk_part = 0.f;
    if (tid < DK) {
        const int c = tid;
        const float a = __expf(g_in);
        const float kc = CONV ? s_x[DK + c] * inv_k : to_f32(k_in);
        const float qc = CONV ? s_x[c] * inv_q : to_f32(q_in);
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
        const float e = (CONV ? s_x[2 * DK + tid] : to_f32(v[(size_t)bh * DV + tid])) - p;
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

template <class T, int DK, int DV, bool CONV, bool HG>
hipError_t launch_conv_or_not(const DecodeArgs &a, hipStream_t s) {
    const int blocks = a.batch * a.heads;
    if (a.out_f32)
        hipLaunchKernelGGL((decode_kernel<T, float, DK, DV, CONV, HG>), dim3(blocks),
                           dim3(DecodeCfg<T, DK, DV>::kThreads), 0, s,
                           (const T *)a.q, (const T *)a.k, (const T *)a.v, a.g, a.beta, a.state,
                           a.scale, (float *)a.o, a.conv);
    else
        hipLaunchKernelGGL((decode_kernel<T, T, DK, DV, CONV, HG>), dim3(blocks),
                           dim3(DecodeCfg<T, DK, DV>::kThreads), 0, s,
                           (const T *)a.q, (const T *)a.k, (const T *)a.v, a.g, a.beta, a.state,
                           a.scale, (T *)a.o, a.conv);
    return hipGetLastError();
}

template <class T, int DK, int DV>
hipError_t launch_typed(const DecodeArgs &a, hipStream_t s) {
    if (a.batch * a.heads == 0) return hipSuccess;
    if (a.head_gate) return launch_conv_or_not<T, DK, DV, false, true>(a, s);
    return a.with_conv ? launch_conv_or_not<T, DK, DV, true, false>(a, s)
                       : launch_conv_or_not<T, DK, DV, false, false>(a, s);
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
