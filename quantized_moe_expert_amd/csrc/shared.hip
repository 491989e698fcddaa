// Shared expert launches (few tokens): the gate/up GEMV + SwiGLU into h,
// then the down GEMV into y, each over a resident grid of (token tile, row
// chunk) items (the item bodies are in shared_dev.h).  Also the int8
// dequantisation test hook.
#include "shared_dev.h"

namespace moeq4 {

template <int LPR>
__global__ __launch_bounds__(DEC_WAVES * 64) void shared_gateup_kernel(const uint16_t *__restrict__ x, int T,
                                                                       SharedPtrs S, float *__restrict__ h) {
    constexpr int BR = DEC_WAVES * (WAVE / LPR);
    const int ntt = (T + DECODE_TT - 1) / DECODE_TT;
    const Items it = decode_items(ntt, S.I, S.I / BR);
    __shared__ float s_out[DECODE_TT][DEC_RB_MAX];
    for (int w = it.first; w < it.end; w += it.stride) {
        const int j = w % ntt, chunk = w / ntt;  // chunk-major: a chunk's token tiles share an XCD
        const int tok0 = j * DECODE_TT, nt = T - tok0 < DECODE_TT ? T - tok0 : DECODE_TT;
        const ItemRows<BR> ir = item_rows<BR>(chunk, it, S.I);
        if (ir.steps <= 0) continue;
        shared_gateup_item<LPR>(x, S, tok0, nt, ir, h, s_out);
    }
}

template <int LPR>
__global__ __launch_bounds__(DEC_WAVES * 64) void shared_down_kernel(int T, SharedPtrs S,
                                                                     const float *__restrict__ h,
                                                                     float *__restrict__ y, int accumulate) {
    constexpr int BR = DEC_WAVES * (WAVE / LPR);
    const int ntt = (T + DECODE_TT - 1) / DECODE_TT;
    const Items it = decode_items(ntt, S.H, S.H / BR);
    __shared__ float s_out[DECODE_TT][DEC_RB_MAX];
    for (int w = it.first; w < it.end; w += it.stride) {
        const int j = w % ntt, chunk = w / ntt;  // chunk-major: a chunk's token tiles share an XCD
        const int tok0 = j * DECODE_TT, nt = T - tok0 < DECODE_TT ? T - tok0 : DECODE_TT;
        const ItemRows<BR> ir = item_rows<BR>(chunk, it, S.H);
        if (ir.steps <= 0) continue;
        shared_down_item<LPR, false>(S, tok0, nt, ir, h, y, accumulate != 0, s_out);
    }
}

hipError_t launch_shared(const uint16_t *x, int64_t T, const SharedPtrs &S, float *h, float *y, bool accumulate,
                         hipStream_t s, hipEvent_t e0, hipEvent_t e1, hipEvent_t e2, hipEvent_t e3) {
    const dim3 block(DEC_WAVES * 64);
    switch (S.H / 32) {
#define CASE(LP)                                                                                              \
    case LP: {                                                                                                \
        constexpr auto kern = shared_gateup_kernel<LP>;                                                       \
        launch_k(kern, dim3(resident_grid<kern>()), block, s, e0, e1, x, (int)T, S, h);                       \
    } break;
        CASE(4) CASE(8) CASE(16) CASE(32) CASE(64)
#undef CASE
        default: return hipErrorInvalidValue;
    }
    switch (S.I / 32) {
#define CASE(LP)                                                                                              \
    case LP: {                                                                                                \
        constexpr auto kern = shared_down_kernel<LP>;                                                         \
        launch_k(kern, dim3(resident_grid<kern>()), block, s, e2, e3, (int)T, S,                              \
                 (const float *)h, y, accumulate ? 1 : 0);                                                    \
    } break;
        CASE(4) CASE(8) CASE(16) CASE(32) CASE(64)
#undef CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// out[n][k] = float(q) * scale of one int8 projection, q decoded as the down
// GEMV decodes it (top bit flipped, inserted into the f16 pair (1024, 1024),
// 1152 subtracted); the product is exact in fp32.
__global__ __launch_bounds__(256) void dequant_int8_kernel(const int8_t *__restrict__ q,
                                                           const uint16_t *__restrict__ sc, int N, int K,
                                                           float *__restrict__ out) {
    const int64_t words = (int64_t)N * K / 4;
    const int64_t wi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (wi >= words) return;
    const int64_t n = wi / (K / 4);
    const int k0 = (int)(wi % (K / 4)) * 4;
    const uint32_t w = reinterpret_cast<const uint32_t *>(q)[wi] ^ SX_FLIP;
    const float s = f16_to_f32(sc[(size_t)n * (K / SX_GROUP) + k0 / SX_GROUP]);
    const uint32_t kf = MAGIC_F16;
    const uint32_t pa = sx_codes_f16(insert_codes<0x00ff00ffu>(w, kf));       // codes 0, 2
    const uint32_t pb = sx_codes_f16(insert_codes<0x00ff00ffu>(w >> 8, kf));  // codes 1, 3
    float *dst = out + (size_t)n * K + k0;
    dst[0] = f16_to_f32((uint16_t)(pa & 0xffffu)) * s;
    dst[1] = f16_to_f32((uint16_t)(pb & 0xffffu)) * s;
    dst[2] = f16_to_f32((uint16_t)(pa >> 16)) * s;
    dst[3] = f16_to_f32((uint16_t)(pb >> 16)) * s;
}

hipError_t launch_dequant_int8(const SharedPtrs &S, int proj, float *out, hipStream_t s) {
    const int N = proj == 2 ? S.H : S.I, K = proj == 2 ? S.I : S.H;
    const int8_t *q = proj == 0 ? S.gq : (proj == 1 ? S.uq : S.dq);
    const uint16_t *sc = proj == 0 ? S.gs : (proj == 1 ? S.us : S.ds);
    const int64_t words = (int64_t)N * K / 4;
    hipLaunchKernelGGL(dequant_int8_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, s, q, sc, N, K, out);
    return hipGetLastError();
}

}  // namespace moeq4
