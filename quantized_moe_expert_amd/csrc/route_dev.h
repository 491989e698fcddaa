// Device-side routing helpers shared by the routing kernels and the fused
// decode routing kernel (see route.hip for the method).
#pragma once

#include "moe_internal.h"

namespace moeq4 {

// Dot product of bf16 row x and bf16 row w (H elements) by one wave, summed
// in double (every bf16 x bf16 product is exact in double); the result is
// valid in lane 63.  With yres != null the activation is the residual step
// bf16(float(x) + yres) of a layer chain.
__device__ inline double router_dot_wave(const uint16_t *__restrict__ x, const float *__restrict__ yres,
                                         const uint16_t *__restrict__ w, int H) {
    const int lane = threadIdx.x & 63;
    double acc = 0.0;
    for (int h = lane * 8; h < H; h += WAVE * 8) {
        const uint4 xv = *reinterpret_cast<const uint4 *>(x + h);
        const uint4 wv = *reinterpret_cast<const uint4 *>(w + h);
        uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w};
        const uint32_t ws[4] = {wv.x, wv.y, wv.z, wv.w};
        if (yres) {
            const float4 ya = *reinterpret_cast<const float4 *>(yres + h);
            const float4 yb = *reinterpret_cast<const float4 *>(yres + h + 4);
            const float yv[8] = {ya.x, ya.y, ya.z, ya.w, yb.x, yb.y, yb.z, yb.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t lo = f32_to_bf16_rne(bf16_to_f32(xs[j] & 0xffffu) + yv[2 * j]);
                const uint32_t hi = f32_to_bf16_rne(bf16_to_f32(xs[j] >> 16) + yv[2 * j + 1]);
                xs[j] = lo | (hi << 16);
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc = fma((double)bf16_to_f32(xs[j] & 0xffffu), (double)bf16_to_f32(ws[j] & 0xffffu), acc);
            acc = fma((double)bf16_to_f32(xs[j] >> 16), (double)bf16_to_f32(ws[j] >> 16), acc);
        }
    }
    return wave_sum_f64_dpp(acc);
}

// Top-k of one token by one wave.  Each lane holds up to NPL logits (experts
// lane, lane+64, ...) as 32-bit keys (order(value) << 16 | (0xffff - e)),
// sorted in the lane, largest first; k rounds of a wave-wide max over the
// lanes' first keys pick the largest value and, among equal values, the
// lowest e (keys are unique), and the winning lane moves to its next key.
// Lane i keeps the i-th key, from which expert and logit are read back.
// Gates in double: exp(l_i - l_0) / sum_j exp(l_j - l_0).
template <int NPL>
__device__ inline void topk_token_wave(const uint16_t *__restrict__ l, int E, int k, int32_t *__restrict__ idx_out,
                                       float *__restrict__ gate_out, int32_t *idx_copy = nullptr) {
    const int lane = threadIdx.x & 63;
    // every load issued before the first use (clamped index, masked after),
    // so the NPL reads share one wait
    uint16_t lv[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
        const int e = j * WAVE + lane;
        lv[j] = l[e < E ? e : E - 1];
    }
    uint32_t key[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
        const int e = j * WAVE + lane;
        key[j] = e < E ? (bf16_order(lv[j]) << 16) | (0xffffu - (uint32_t)e) : 0u;
    }
    // sorting network, largest first
    auto cswap = [&](int a, int b) {
        const uint32_t hi = key[a] > key[b] ? key[a] : key[b], lo = key[a] > key[b] ? key[b] : key[a];
        key[a] = hi;
        key[b] = lo;
    };
    if constexpr (NPL == 2) {
        cswap(0, 1);
    } else if constexpr (NPL == 4) {
        cswap(0, 1), cswap(2, 3), cswap(0, 2), cswap(1, 3), cswap(1, 2);
    } else {
#pragma unroll
        for (int i = 0; i < NPL; ++i)
#pragma unroll
            for (int j = 0; j + 1 < NPL - i; ++j) cswap(j, j + 1);
    }
    uint32_t mine = 0;  // lane i < k: the i-th largest key
    for (int i = 0; i < k; ++i) {
        const uint32_t m = wave_max_u32(key[0]);
        if (lane == i) mine = m;
        if (key[0] == m) {  // the one lane holding it moves on
#pragma unroll
            for (int j = 0; j + 1 < NPL; ++j) key[j] = key[j + 1];
            key[NPL - 1] = 0u;
        }
    }
    const uint32_t m0 = (uint32_t)__builtin_amdgcn_readlane((int)mine, 0);
    const double l0 = (double)bf16_to_f32(bf16_from_order(m0 >> 16));
    double ex = 0.0;
    if (lane < k) ex = exp((double)bf16_to_f32(bf16_from_order(mine >> 16)) - l0);
    const double den = wave_allsum_f64_dpp(ex);
    if (lane < k) {
        const int my_e = (int)(0xffffu - (mine & 0xffffu));
        idx_out[lane] = my_e;
        gate_out[lane] = (float)(ex / den);
        if (idx_copy) idx_copy[lane] = my_e;
    }
}

}  // namespace moeq4
