// Router GEMV and top-k selection.
//
// Router weights are bf16 (drama-q4 card, "What's quantized"; MLX card,
// "Quantization and provenance").  The logit of (token t, expert e) is the
// dot product of bf16 x[t] and bf16 Wr[e] summed in double (every bf16 x bf16
// product is exact in double, so the sum does not depend on its order for
// inputs of ordinary magnitude), plus an optional bias, rounded to float and
// then to bf16.  Top-k and gates: the k largest logits, ties to the lower
// expert index, gates = softmax over the selected logits.
#include "route_dev.h"

namespace moeq4 {

// One wave per expert row; lanes cover H in 8-element (16-byte) chunks.  A
// block holds 4 experts and walks a range of tokens, keeping the expert row
// chunks in registers.
template <int CH>  // 16-byte chunks per lane = H / 512 (rounded up)
__global__ __launch_bounds__(256) void router_logits_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr, const float *__restrict__ bias,
    int64_t T, int H, int E, int tokens_per_block, uint16_t *__restrict__ logits) {
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (e >= E) return;
    const int64_t t0 = (int64_t)blockIdx.y * tokens_per_block;
    const int64_t t1 = t0 + tokens_per_block < T ? t0 + tokens_per_block : T;

    uint4 w[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int h = (c * WAVE + lane) * 8;
        w[c] = h < H ? *reinterpret_cast<const uint4 *>(wr + (size_t)e * H + h) : make_uint4(0, 0, 0, 0);
    }
    const double b = bias ? (double)bias[e] : 0.0;
    for (int64_t t = t0; t < t1; ++t) {
        double acc = 0.0;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int h = (c * WAVE + lane) * 8;
            if (h < H) {
                const uint4 xv = *reinterpret_cast<const uint4 *>(x + t * H + h);
                const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w};
                const uint32_t ws[4] = {w[c].x, w[c].y, w[c].z, w[c].w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc = fma((double)bf16_to_f32(xs[j] & 0xffffu), (double)bf16_to_f32(ws[j] & 0xffffu), acc);
                    acc = fma((double)bf16_to_f32(xs[j] >> 16), (double)bf16_to_f32(ws[j] >> 16), acc);
                }
            }
        }
        acc = wave_sum_f64(acc);
        if (lane == 0) logits[t * E + e] = f32_to_bf16_rne((float)(acc + b));
    }
}

template <int NPL>
__global__ __launch_bounds__(256) void topk_kernel(const uint16_t *__restrict__ logits, int64_t T, int E,
                                                   int k, int32_t *__restrict__ idx, float *__restrict__ gate) {
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    topk_token_wave<NPL>(logits + t * E, E, k, idx + t * k, gate + t * k);
}

hipError_t launch_router_logits(const uint16_t *x, const uint16_t *wr, const float *bias, int64_t T, int H,
                                int E, uint16_t *logits, hipStream_t s) {
    const int tpb = T >= 64 ? 16 : 4;
    dim3 grid((E + 3) / 4, (unsigned)((T + tpb - 1) / tpb));
    const int ch = (H + 511) / 512;
    switch (ch) {
#define CASE(C) \
    case C: hipLaunchKernelGGL(router_logits_kernel<C>, grid, dim3(256), 0, s, x, wr, bias, T, H, E, tpb, logits); break;
        CASE(1) CASE(2) CASE(3) CASE(4)
#undef CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_topk(const uint16_t *logits, int64_t T, int E, int k, int32_t *idx, float *gate, hipStream_t s) {
    dim3 grid((unsigned)((T + 3) / 4));
    const int npl = (E + 63) / 64;
    if (npl <= 4) hipLaunchKernelGGL(topk_kernel<4>, grid, dim3(256), 0, s, logits, T, E, k, idx, gate);
    else if (npl <= 8) hipLaunchKernelGGL(topk_kernel<8>, grid, dim3(256), 0, s, logits, T, E, k, idx, gate);
    else hipLaunchKernelGGL(topk_kernel<16>, grid, dim3(256), 0, s, logits, T, E, k, idx, gate);
    return hipGetLastError();
}

}  // namespace moeq4
