/*
 * kda_oracle.c -- fp64 CPU oracle for the Kimi Delta Attention (KDA) forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously-correct
 * definition that the HIP kernels are checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It shares
 * no code, header, table or helper with the GPU library, and it must never be
 * used as a fallback for it.
 *
 * Sources (web pages; cited by title and section, see oracle/__init__.py):
 *   [Walkthrough]  "Kimi K3的线性注意力：从源码看懂KDA如何更新记忆"
 *   [Replication-2] "KimiK3轻量化复刻实现KDA并行解析，Chunkwise并行与状态压缩机制详解"
 *   [Workshop-16]  "AI-Workshop 文献分享 #16 — KDA：给长文本建立可更新的记忆"
 *
 * Everything is double precision.  Tensors are dense, row-major, contiguous:
 *   activations  [total_tokens, H, D]   (packed variable-length sequences)
 *   conv input   [total_tokens, C]      (C = H*D channels)
 *   state        [N, H, DK, DV]         (key index first, value index second)
 * cu_seqlens[N+1] holds the packed sequence offsets (cu_seqlens[0] = 0).
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC kda_oracle.c -o libkda_oracle.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_ENOMEM (-2)

static int check_seqlens(const int32_t *cu, int n, int64_t total) {
    if (!cu || n <= 0) return 0;
    if (cu[0] != 0 || cu[n] != total) return 0;
    for (int i = 0; i < n; ++i)
        if (cu[i + 1] < cu[i]) return 0;
    return 1;
}

/*
 * O1a. Causal depthwise short convolution with optional SiLU
 *      ([Walkthrough] 第二站: width-4 causal conv mixing the current position with
 *      up to three earlier ones, SiLU configured inside the conv module, a conv
 *      cache carried between calls, packed sequences via cu_seqlens;
 *      [Replication-2] per-channel causal Conv1D of width 4 over q/k/v).
 *
 * For sequence n and channel c, with history h_0..h_{W-2} (oldest first) taken
 * from state_in[n, :, c] or zeros, the extended input is
 *     xe = [h_0, ..., h_{W-2}, x_{bos}, ..., x_{eos-1}]
 * and for the j-th token of the sequence (j = 0..L-1)
 *     y = bias[c] + sum_{i=0}^{W-1} w[c, i] * xe[j + i]
 * so w[c, W-1] multiplies the current token.  With silu != 0, y <- y / (1 + e^-y).
 * The new history (state_out[n, :, c]) is the last W-1 entries of xe.
 *
 * x, y: [total_tokens, C]; w: [C, W]; bias: [C] or NULL;
 * state_in/state_out: [N, W-1, C] or NULL.  state_out may alias state_in.
 */
int kda_oracle_short_conv(const double *x, int64_t total_tokens, int64_t C,
                          const double *w, int W, const double *bias,
                          const int32_t *cu_seqlens, int N,
                          const double *state_in, double *state_out,
                          int silu, double *y) {
    if (!x || !w || !y || W < 1 || C <= 0) return ORACLE_EINVAL;
    if (!check_seqlens(cu_seqlens, N, total_tokens)) return ORACLE_EINVAL;
    const int H = W - 1;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t nc = 0; nc < (int64_t)N * C; ++nc) {
        const int n = (int)(nc / C);
        const int64_t c = nc % C;
        const int64_t bos = cu_seqlens[n], L = cu_seqlens[n + 1] - bos;
        double *xe = (double *)malloc(sizeof(double) * (size_t)(L + H + 1));
        if (!xe) { err = 1; continue; }
        for (int i = 0; i < H; ++i)
            xe[i] = state_in ? state_in[((int64_t)n * H + i) * C + c] : 0.0;
        for (int64_t j = 0; j < L; ++j) xe[H + j] = x[(bos + j) * C + c];
        for (int64_t j = 0; j < L; ++j) {
            double acc = bias ? bias[c] : 0.0;
            for (int i = 0; i < W; ++i) acc += w[c * W + i] * xe[j + i];
            if (silu) acc = acc / (1.0 + exp(-acc));
            y[(bos + j) * C + c] = acc;
        }
        if (state_out)
            for (int i = 0; i < H; ++i)
                state_out[((int64_t)n * H + i) * C + c] = xe[L + i];
        free(xe);
    }
    return err ? ORACLE_ENOMEM : ORACLE_OK;
}

/*
 * O0. Bounded forget gate ([Walkthrough] 彩蛋: the gate function with a lower
 *     bound).  From the gate's pre-activation z, a learnable per-head parameter
 *     A_log[h] and a per-channel bias dt_bias[h, c], the log-decay is
 *         g = lower_bound * sigmoid(exp(A_log[h]) * (z + dt_bias[h, c])),
 *     sigmoid(y) = 1 / (1 + e^-y), so lower_bound <= g <= 0 and the retention
 *     alpha = e^g lies in [e^lower_bound, 1] (lower_bound = -5 in K3).
 * z, g: [T, H, D]; a_log: [H] or NULL (0); dt_bias: [H, D] or NULL (0).
 */
void kda_oracle_bounded_gate(const double *z, int64_t T, int H, int D, const double *a_log,
                             const double *dt_bias, double lower_bound, double *g) {
    for (int64_t t = 0; t < T; ++t)
        for (int h = 0; h < H; ++h) {
            const double a = exp(a_log ? a_log[h] : 0.0);
            for (int c = 0; c < D; ++c) {
                const int64_t i = (t * H + h) * D + c;
                const double y = a * (z[i] + (dt_bias ? dt_bias[(int64_t)h * D + c] : 0.0));
                g[i] = lower_bound / (1.0 + exp(-y));
            }
        }
}

/*
 * O3. Output epilogue ([Walkthrough] 第六站: the read-out passes a per-head
 *     RMSNorm, then the output gate scales it channel by channel, before the
 *     output projection).  Per (token t, head h) row of D channels:
 *         y[c] = o[c] / sqrt(mean_c' o[c']^2 + eps) * w[c] * sigmoid(gate[c]),
 *     the gate being the output gate's pre-activation (its projection of the
 *     layer input is outside the path) and w the norm's per-channel weight.
 * o, gate, y: [T, H, D]; w: [D] or NULL (1).
 */
void kda_oracle_output_norm_gate(const double *o, const double *gate, int64_t T, int H, int D,
                                 const double *w, double eps, double *y) {
    for (int64_t r = 0; r < T * H; ++r) {
        const double *orow = o + r * D, *grow = gate + r * D;
        double ss = 0.0;
        for (int c = 0; c < D; ++c) ss += orow[c] * orow[c];
        const double inv = 1.0 / sqrt(ss / D + eps);
        for (int c = 0; c < D; ++c)
            y[r * D + c] = orow[c] * inv * (w ? w[c] : 1.0) / (1.0 + exp(-grow[c]));
    }
}

/*
 * O1b. L2 normalisation of q and k ([Walkthrough] 第二站: after conv+SiLU the
 *      query and key are scaled to (close to) unit length; the operator does it).
 * x: [rows, D], each row scaled in place by 1 / sqrt(sum_c x_c^2 + eps).
 */
void kda_oracle_l2norm(double *x, int64_t rows, int64_t D, double eps) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double ss = 0.0;
        for (int64_t c = 0; c < D; ++c) ss += x[r * D + c] * x[r * D + c];
        const double inv = 1.0 / sqrt(ss + eps);
        for (int64_t c = 0; c < D; ++c) x[r * D + c] *= inv;
    }
}

/*
 * O1c. Rounding to bf16 (8 significant bits, round half to even), in place.
 *      The pipeline hands q, k, v from the prologue to the recurrence as
 *      tensors of the activation dtype; with bf16 activations the oracle rounds
 *      its fp64 prologue result the same way before the recurrence.  Values in
 *      the bf16 normal range are assumed (|x| >= 2^-126 or 0).
 */
void kda_oracle_round_bf16(double *x, int64_t n) {
    for (int64_t i = 0; i < n; ++i) {
        if (x[i] == 0.0 || !isfinite(x[i])) continue;
        int e;
        const double m = frexp(x[i], &e);          /* x = m * 2^e, 0.5 <= |m| < 1 */
        x[i] = ldexp(nearbyint(ldexp(m, 8)), e - 8);
    }
}

/*
 * O2. The KDA recurrence, one token at a time, in the order the source-code
 *     walkthrough fixes ([Walkthrough] 第三站 forget first because the order
 *     matters; 第四站 read the prediction along k, form the error, write it
 *     back along k scaled by beta; 第五站 read out with q from the updated state).
 *
 * For each (sequence n, head h), S <- h0[n,h] (or zeros), then for every token t:
 *     S[c][:]  *= exp(g[t,h,c])                 per-key-channel decay (rows of S)
 *     pred[j]   = sum_c S[c][j] * k[t,h,c]       prediction S^T k
 *     e[j]      = v[t,h,j] - pred[j]             error (delta_rule == 0: e = v)
 *     S[c][j]  += beta[t,h] * k[t,h,c] * e[j]    rank-one corrective write
 *     o[t,h,j]  = scale * sum_c S[c][j] * q[t,h,c]
 * and hT[n,h] = S after the last token.  delta_rule == 0 drops the correction,
 * which reduces KDA to gated linear attention ([Workshop-16] 第7节); it exists only
 * so the tests can pin the oracle to those textbook forms.
 *
 * q,k: [T,H,DK]; v,o: [T,H,DV]; g: [T,H,DK] (log-decay); beta: [T,H];
 * h0, hT: [N,H,DK,DV] or NULL (h0 NULL = zeros; hT NULL = not written).
 */
int kda_oracle_recurrent(const double *q, const double *k, const double *v,
                         const double *g, const double *beta,
                         const int32_t *cu_seqlens, int N, int64_t total_tokens,
                         int H, int DK, int DV, double scale,
                         const double *h0, double *o, double *hT, int delta_rule) {
    if (!q || !k || !v || !g || !beta || !o || H <= 0 || DK <= 0 || DV <= 0)
        return ORACLE_EINVAL;
    if (!check_seqlens(cu_seqlens, N, total_tokens)) return ORACLE_EINVAL;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t nh = 0; nh < (int64_t)N * H; ++nh) {
        const int n = (int)(nh / H), h = (int)(nh % H);
        double *S = (double *)malloc(sizeof(double) * (size_t)DK * DV);
        double *e = (double *)malloc(sizeof(double) * (size_t)DV);
        if (!S || !e) { free(S); free(e); err = 1; continue; }
        const int64_t sbase = nh * (int64_t)DK * DV;
        for (int64_t i = 0; i < (int64_t)DK * DV; ++i) S[i] = h0 ? h0[sbase + i] : 0.0;

        for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t) {
            const double *qt = q + (t * H + h) * DK;
            const double *kt = k + (t * H + h) * DK;
            const double *gt = g + (t * H + h) * DK;
            const double *vt = v + (t * H + h) * DV;
            const double bt = beta[t * H + h];
            double *ot = o + (t * H + h) * DV;

            for (int c = 0; c < DK; ++c) {           /* decay */
                const double a = exp(gt[c]);
                for (int j = 0; j < DV; ++j) S[c * DV + j] *= a;
            }
            for (int j = 0; j < DV; ++j) {           /* predict, error */
                double pred = 0.0;
                for (int c = 0; c < DK; ++c) pred += S[c * DV + j] * kt[c];
                e[j] = delta_rule ? vt[j] - pred : vt[j];
            }
            for (int c = 0; c < DK; ++c)             /* correct */
                for (int j = 0; j < DV; ++j) S[c * DV + j] += bt * kt[c] * e[j];
            for (int j = 0; j < DV; ++j) {           /* read out */
                double acc = 0.0;
                for (int c = 0; c < DK; ++c) acc += S[c * DV + j] * qt[c];
                ot[j] = scale * acc;
            }
        }
        if (hT)
            for (int64_t i = 0; i < (int64_t)DK * DV; ++i) hT[sbase + i] = S[i];
        free(S);
        free(e);
    }
    return err ? ORACLE_ENOMEM : ORACLE_OK;
}

/* Number of OpenMP threads the oracle runs with (reported beside its timings). */
int kda_oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
