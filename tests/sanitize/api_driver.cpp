// api_driver.cpp -- the host half of libkda (kda_api.cpp: argument checks, status
// codes, error strings, launcher choice, the scratch lookup's error path) linked
// against stub launchers, for a host build under AddressSanitizer and
// UndefinedBehaviorSanitizer.  No GPU and no HIP runtime: the stubs record what
// the ABI would have launched.  Every entry point is called with valid arguments
// (one launch, with exactly the arguments given) and with each class of invalid
// argument (no launch, the documented status, a bounded message), including
// sizes at the edges of the checks.  Exits 0 and prints "ok" on success.
#include <stdio.h>
#include <string.h>

#include <limits>

#include "kda.h"
#include "kda_launch.h"

namespace {
int g_launches = 0;
kda::ChunkArgs g_chunk{};
kda::ConvArgs g_conv{};
kda::DecodeArgs g_decode{};
kda::NormGateArgs g_norm{};
void *const kScratch = reinterpret_cast<void *>(0x7f0000000000ull);
bool g_scratch_fails = false;
int failures = 0;

void expect(bool cond, const char *what, int line) {
    if (!cond) {
        fprintf(stderr, "FAILED (line %d): %s\n", line, what);
        ++failures;
    }
}
#define EXPECT(c) expect((c), #c, __LINE__)

hipError_t chunk_stub(const kda::ChunkArgs &a, bool launch, int *used) {
    *used = 16;
    if (launch) {
        ++g_launches;
        g_chunk = a;
    }
    return hipSuccess;
}
}  // namespace

// Stand-ins for the launchers of the HIP translation units and the one HIP
// runtime function kda_api.cpp calls.
namespace kda {
hipError_t launch_short_conv(const ConvArgs &a, bool, hipStream_t) {
    ++g_launches;
    g_conv = a;
    return hipSuccess;
}
#define STUB(name) \
    hipError_t name(const ChunkArgs &a, hipStream_t, bool l, int *u) { return chunk_stub(a, l, u); }
STUB(launch_chunk_bf16_f32out)
STUB(launch_chunk_bf16_bf16out)
STUB(launch_chunk_f32)
STUB(launch_chunk_bf16_f32out_gz)
STUB(launch_chunk_bf16_bf16out_gz)
STUB(launch_chunk_f32_gz)
STUB(launch_chunk_bf16_f32out_gdn)
STUB(launch_chunk_bf16_bf16out_gdn)
STUB(launch_chunk_f32_gdn)
#undef STUB
hipError_t launch_decode_step(const DecodeArgs &a, bool, hipStream_t) {
    ++g_launches;
    g_decode = a;
    return hipSuccess;
}
hipError_t launch_norm_gate(const NormGateArgs &a, bool, bool, hipStream_t) {
    ++g_launches;
    g_norm = a;
    return hipSuccess;
}
hipError_t scratch_address(void **p) {
    if (g_scratch_fails) return hipErrorNoDevice;
    *p = kScratch;
    return hipSuccess;
}
}  // namespace kda

const char *hipGetErrorString(hipError_t) { return "stub HIP error"; }

namespace {
char *P(uintptr_t x) { return reinterpret_cast<char *>(x << 12); }   // distinct fake pointers

// One chunk call; returns its status and whether it launched.
struct ChunkCall {
    const void *q = P(1), *k = P(2), *v = P(3);
    const float *g = (const float *)P(4), *beta = (const float *)P(5);
    const int32_t *cu = nullptr;
    int32_t N = 1;
    int64_t T = 64;
    int32_t H = 2, dk = 128, dv = 128, chunk = 64;
    float scale = 0.125f, lb = -5.f;
    const float *h0 = nullptr;
    float *hT = (float *)P(6);
    void *o = P(7), *ws = P(8);
    size_t wsb = (size_t)1 << 30;
    kda_dtype_t dt = KDA_DTYPE_BF16, odt = KDA_DTYPE_F32;
    int mode = 0;   // 0 plain, 1 gated, 2 GDN, 3 no-alloc

    kda_status_t run(bool *launched) const {
        const int before = g_launches;
        kda_status_t st;
        switch (mode) {
            case 1:
                st = kda_chunk_fwd_gated(q, k, v, g, (const float *)P(9), (const float *)P(10), lb,
                                         beta, cu, N, T, H, dk, dv, chunk, scale, h0, hT, o, ws,
                                         wsb, dt, odt, nullptr);
                break;
            case 2:
                st = kda_gdn_chunk_fwd(q, k, v, g, beta, cu, N, T, H, dk, dv, chunk, scale, lb,
                                       h0, hT, o, ws, wsb, dt, odt, nullptr);
                break;
            case 3:
                st = kda_chunk_fwd_noalloc(q, k, v, g, beta, cu, N, T, H, dk, dv, chunk, scale, lb,
                                           h0, hT, o, dt, odt, nullptr);
                break;
            default:
                st = kda_chunk_fwd(q, k, v, g, beta, cu, N, T, H, dk, dv, chunk, scale, lb, h0, hT,
                                   o, ws, wsb, dt, odt, nullptr);
        }
        *launched = g_launches != before;
        const char *msg = kda_last_error();
        EXPECT(msg && strlen(msg) < 512);
        EXPECT((st == KDA_OK) == (msg[0] == '\0'));
        return st;
    }
};

void chunk_cases() {
    for (int mode = 0; mode < 4; ++mode) {
        bool launched = false;
        ChunkCall c;
        c.mode = mode;
        EXPECT(c.run(&launched) == KDA_OK && launched);
        EXPECT(g_chunk.q == c.q && g_chunk.o == c.o && g_chunk.heads == 2 && g_chunk.scale == c.scale);
        EXPECT(g_chunk.workspace == (float *)(mode == 3 ? kScratch : c.ws));
        struct Bad {
            void (*set)(ChunkCall &);
            kda_status_t st;
        };
        const Bad bad[] = {
            {[](ChunkCall &x) { x.q = nullptr; }, KDA_ERR_INVALID_ARG},
            {[](ChunkCall &x) { x.o = nullptr; }, KDA_ERR_INVALID_ARG},
            {[](ChunkCall &x) { x.N = 0; }, KDA_ERR_INVALID_ARG},
            {[](ChunkCall &x) { x.N = 2; }, KDA_ERR_INVALID_ARG},
            {[](ChunkCall &x) { x.T = -1; }, KDA_ERR_INVALID_ARG},
            {[](ChunkCall &x) { x.H = 0; }, KDA_ERR_INVALID_ARG},
            {[](ChunkCall &x) { x.H = std::numeric_limits<int32_t>::max(); }, KDA_ERR_INVALID_ARG},
            {[](ChunkCall &x) { x.dt = (kda_dtype_t)7; }, KDA_ERR_INVALID_ARG},
            {[](ChunkCall &x) { x.scale = std::numeric_limits<float>::infinity(); },
             KDA_ERR_INVALID_ARG},
            {[](ChunkCall &x) { x.o = const_cast<void *>(x.q); }, KDA_ERR_INVALID_ARG},
            {[](ChunkCall &x) { x.lb = 0.5f; }, KDA_ERR_INVALID_ARG},
            {[](ChunkCall &x) { x.lb = std::numeric_limits<float>::quiet_NaN(); },
             KDA_ERR_INVALID_ARG},
            {[](ChunkCall &x) { x.lb = -9.5f; }, KDA_ERR_UNSUPPORTED},
            {[](ChunkCall &x) { x.dk = 48; }, KDA_ERR_UNSUPPORTED},
            {[](ChunkCall &x) { x.dv = 256; }, KDA_ERR_UNSUPPORTED},
            {[](ChunkCall &x) { x.chunk = 8; }, KDA_ERR_UNSUPPORTED},
            {[](ChunkCall &x) { x.dt = KDA_DTYPE_F32; x.odt = KDA_DTYPE_BF16; }, KDA_ERR_UNSUPPORTED},
            {[](ChunkCall &x) { x.T = std::numeric_limits<int64_t>::max(); }, KDA_ERR_UNSUPPORTED},
        };
        for (const Bad &b : bad) {
            ChunkCall x;
            x.mode = mode;
            b.set(x);
            if (mode == 2 && x.chunk == 8) continue;
            const kda_status_t st = x.run(&launched);
            EXPECT(st == b.st && !launched);
        }
        if (mode != 3) {   // the caller's workspace: missing or one byte short
            ChunkCall x;
            x.mode = mode;
            x.ws = nullptr;
            EXPECT(x.run(&launched) == KDA_ERR_WORKSPACE && !launched);
            size_t need = 0;
            EXPECT(kda_chunk_fwd_workspace_size(x.T, x.H, x.dk, x.dv, x.chunk, x.dt, x.odt,
                                                &need) == KDA_OK);
            x.ws = P(8);
            x.wsb = need - 1;
            EXPECT(x.run(&launched) == KDA_ERR_WORKSPACE && !launched);
            x.wsb = need;
            EXPECT(x.run(&launched) == KDA_OK && launched);
        } else {           // the static scratch: its size limit and a failed lookup
            ChunkCall x;
            x.mode = mode;
            x.T = 5462;
            x.H = 96;
            EXPECT(x.run(&launched) == KDA_ERR_UNSUPPORTED && !launched);
            EXPECT(strstr(kda_last_error(), "scratch") != nullptr);
            x.T = 5461;
            EXPECT(x.run(&launched) == KDA_OK && launched);
            g_scratch_fails = true;
            EXPECT(x.run(&launched) == KDA_ERR_HIP && !launched);
            g_scratch_fails = false;
            x.T = 0;   // no tokens: no scratch needed, the state copy still launches
            EXPECT(x.run(&launched) == KDA_OK && launched);
        }
    }
}

void other_cases() {
    const int before = g_launches;
    EXPECT(kda_short_conv(P(1), P(2), nullptr, nullptr, 1, 10, 2, 64, 4, nullptr, nullptr, 1, 1,
                          1e-6f, KDA_DTYPE_BF16, P(3), nullptr) == KDA_OK);
    EXPECT(g_launches == before + 1 && g_conv.x == P(1) && g_conv.y == P(3) && g_conv.width == 4);
    EXPECT(kda_short_conv(P(1), P(2), nullptr, nullptr, 1, 10, 2, 64, 5, nullptr, nullptr, 1, 1,
                          1e-6f, KDA_DTYPE_BF16, P(3), nullptr) == KDA_ERR_UNSUPPORTED);
    EXPECT(kda_short_conv(P(1), P(2), nullptr, nullptr, 1, 10, 2, 64, 4, nullptr, nullptr, 1, 1,
                          1e-6f, KDA_DTYPE_BF16, P(1), nullptr) == KDA_ERR_INVALID_ARG);
    EXPECT(kda_short_conv(P(1), P(2), nullptr, nullptr, 1, 10, 2, 6, 4, nullptr, nullptr, 1, 0,
                          1e-6f, KDA_DTYPE_BF16, P(3), nullptr) == KDA_ERR_UNSUPPORTED);
    EXPECT(kda_short_conv(P(1), P(2), nullptr, nullptr, 1, 10, 2, 512, 4, nullptr, nullptr, 1, 1,
                          1e-6f, KDA_DTYPE_BF16, P(3), nullptr) == KDA_ERR_UNSUPPORTED);
    EXPECT(kda_short_conv(P(1), P(2), nullptr, nullptr, 1, std::numeric_limits<int64_t>::max(), 2,
                          64, 4, nullptr, nullptr, 1, 1, 1e-6f, KDA_DTYPE_BF16, P(3),
                          nullptr) == KDA_ERR_UNSUPPORTED);
    EXPECT(g_launches == before + 1);

    EXPECT(kda_decode_step(P(1), P(2), P(3), (const float *)P(4), (const float *)P(5),
                           (float *)P(6), 64, 96, 128, 128, 0.1f, P(7), KDA_DTYPE_BF16,
                           KDA_DTYPE_F32, nullptr) == KDA_OK);
    EXPECT(g_decode.batch == 64 && g_decode.state == (float *)P(6) && !g_decode.head_gate);
    EXPECT(kda_gdn_decode_step(P(1), P(2), P(3), (const float *)P(4), (const float *)P(5),
                               (float *)P(6), 64, 96, 128, 128, 0.1f, P(7), KDA_DTYPE_BF16,
                               KDA_DTYPE_F32, nullptr) == KDA_OK && g_decode.head_gate);
    EXPECT(kda_decode_step(P(1), P(2), P(3), (const float *)P(4), (const float *)P(5),
                           (float *)P(6), 64, 96, 128, 128, 0.1f, P(6), KDA_DTYPE_BF16,
                           KDA_DTYPE_F32, nullptr) == KDA_ERR_INVALID_ARG);
    EXPECT(kda_decode_step(P(1), P(2), P(3), (const float *)P(4), (const float *)P(5),
                           (float *)P(6), std::numeric_limits<int32_t>::max(),
                           std::numeric_limits<int32_t>::max(), 128, 128, 0.1f, P(7),
                           KDA_DTYPE_BF16, KDA_DTYPE_F32, nullptr) == KDA_ERR_UNSUPPORTED);
    EXPECT(kda_decode_step_conv(P(1), P(2), P(3), P(4), P(5), P(6), P(7), P(8), P(9), 1e-6f,
                                (const float *)P(10), (const float *)P(11), (float *)P(12), 4, 2,
                                64, 32, 0.1f, P(13), KDA_DTYPE_BF16, KDA_DTYPE_F32,
                                nullptr) == KDA_OK);
    EXPECT(g_decode.with_conv && g_decode.conv.cq == P(7));
    EXPECT(kda_decode_step_conv(P(1), P(2), P(3), P(4), P(5), P(6), P(7), P(7), P(9), 1e-6f,
                                (const float *)P(10), (const float *)P(11), (float *)P(12), 4, 2,
                                64, 32, 0.1f, P(13), KDA_DTYPE_BF16, KDA_DTYPE_F32,
                                nullptr) == KDA_ERR_INVALID_ARG);
    EXPECT(kda_output_norm_gate(P(1), P(2), nullptr, 1e-6f, 4096 * 96, 128, KDA_DTYPE_F32,
                                KDA_DTYPE_BF16, P(3), nullptr) == KDA_OK);
    EXPECT(g_norm.rows == 4096 * 96 && g_norm.dv == 128);
    EXPECT(kda_output_norm_gate(P(1), P(2), nullptr, -1.f, 10, 128, KDA_DTYPE_F32,
                                KDA_DTYPE_BF16, P(3), nullptr) == KDA_ERR_INVALID_ARG);
    EXPECT(kda_output_norm_gate(P(1), P(2), nullptr, 1e-6f, std::numeric_limits<int64_t>::max() / 4,
                                128, KDA_DTYPE_F32, KDA_DTYPE_BF16, P(3),
                                nullptr) == KDA_ERR_UNSUPPORTED);
    for (int s = -3; s < 8; ++s) EXPECT(kda_status_string((kda_status_t)s) != nullptr);
    EXPECT(kda_version() >= 10000);
}
}  // namespace

int main() {
    chunk_cases();
    other_cases();
    if (failures) return 1;
    printf("ok\n");
    return 0;
}
