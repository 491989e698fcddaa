// Small kernels: the dequantisation test hooks (int4, fp8, NVFP4), the residual
// step of a chain of layers, and a float fill.
#include "moe_internal.h"

namespace moeq4 {

// out[n][k] of one projection, through the same nibble unpacking as the
// expert kernels: the code comes out of unpack_pair as the exact bf16 value
// 128 + q, then w = fma(q, scale, min) (asym) or (q - 8) * scale (sym), one
// rounding, as the format defines (drama-q4 card "What's quantized";
// drama-3-w4a16 card "How it was made").
template <int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t *__restrict__ q, const uint16_t *__restrict__ sm,
                                                      int N, int K, float *__restrict__ out) {
    const int G = FMT == 0 ? 64 : 128;
    const int64_t words = (int64_t)N * K / 8;
    const int64_t wi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (wi >= words) return;
    const int64_t n = wi / (K / 8);
    const int k0 = (int)(wi % (K / 8)) * 8;
    const uint32_t w = reinterpret_cast<const uint32_t *>(q)[wi];
    const size_t gi = (size_t)n * (K / G) + k0 / G;
    float s, m;
    if (FMT == 0) {
        s = f16_to_f32(sm[2 * gi]);
        m = f16_to_f32(sm[2 * gi + 1]);
    } else {
        s = f16_to_f32(sm[gi]);
        m = 0.f;
    }
    float *dst = out + (size_t)n * K + k0;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t pr = unpack_pair<MAGIC_BF16>(w, p);  // codes p and p + 4
        const float qa = bf16_to_f32(pr & 0xffffu) - OFFSET_BF16;
        const float qb = bf16_to_f32(pr >> 16) - OFFSET_BF16;
        if (FMT == 0) {
            dst[p] = fmaf(qa, s, m);
            dst[p + 4] = fmaf(qb, s, m);
        } else {
            dst[p] = (qa - 8.0f) * s;
            dst[p + 4] = (qb - 8.0f) * s;
        }
    }
}

// out[n][k] of one fp8 projection: the code converted as the expert kernels
// convert it (an exact bf16), times the float32 block scale, one rounding.
__global__ __launch_bounds__(256) void dequant_fp8_kernel(const uint8_t *__restrict__ q, const float *__restrict__ sc,
                                                          int N, int K, float *__restrict__ out) {
    const int64_t words = (int64_t)N * K / 4;
    const int64_t wi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (wi >= words) return;
    const int64_t n = wi / (K / 4);
    const int k0 = (int)(wi % (K / 4)) * 4;
    const uint32_t w = reinterpret_cast<const uint32_t *>(q)[wi];
    const float s = sc[(size_t)(n / 128) * (K / 128) + k0 / 128];
    const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
    const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
    float *dst = out + (size_t)n * K + k0;
    dst[0] = bf16_to_f32(lo & 0xffffu) * s;
    dst[1] = bf16_to_f32(lo >> 16) * s;
    dst[2] = bf16_to_f32(hi & 0xffffu) * s;
    dst[3] = bf16_to_f32(hi >> 16) * s;
}

// out[n][k] of one NVFP4 projection: codes converted as the expert kernels
// convert them (exact bf16), times the E4M3 block scale (exact product in
// fp32), times the global scale, one rounding.
__global__ __launch_bounds__(256) void dequant_nvfp4_kernel(const uint8_t *__restrict__ q,
                                                            const uint8_t *__restrict__ sb,
                                                            const float *__restrict__ gp, int N, int K,
                                                            float *__restrict__ out) {
    const int64_t words = (int64_t)N * K / 8;
    const int64_t wi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (wi >= words) return;
    const float glob = *gp;
    const int64_t n = wi / (K / 8);
    const int k0 = (int)(wi % (K / 8)) * 8;
    const uint32_t w = reinterpret_cast<const uint32_t *>(q)[wi];
    const float s = __builtin_amdgcn_cvt_f32_fp8((int)sb[(size_t)n * (K / 16) + k0 / 16], 0);
    const uint32_t p[4] = {
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3))};
    float *dst = out + (size_t)n * K + k0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        dst[2 * j] = (bf16_to_f32(p[j] & 0xffffu) * s) * glob;
        dst[2 * j + 1] = (bf16_to_f32(p[j] >> 16) * s) * glob;
    }
}

__global__ __launch_bounds__(256) void residual_kernel(const uint16_t *__restrict__ x, const float *__restrict__ y,
                                                       int64_t n, uint16_t *__restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = f32_to_bf16_rne(bf16_to_f32(x[i]) + y[i]);
}

hipError_t launch_dequant(const LayerPtrs &L, int expert, int proj, float *out, hipStream_t s) {
    const int G = L.fmt == 0 ? 64 : 128;
    const int N = proj == 2 ? L.H : L.I, K = proj == 2 ? L.I : L.H;
    const uint8_t *q = proj == 0 ? L.gq : (proj == 1 ? L.uq : L.dq);
    const uint16_t *sm = proj == 0 ? L.gsm : (proj == 1 ? L.usm : L.dsm);
    if (L.fmt == 3) {
        q += (size_t)expert * N * (K / 2);
        const uint8_t *sb = reinterpret_cast<const uint8_t *>(sm) + (size_t)expert * N * (K / 16);
        const int64_t words = (int64_t)N * K / 8;
        hipLaunchKernelGGL(dequant_nvfp4_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, s, q, sb,
                           L.glob + 2 * expert + (proj == 2 ? 1 : 0), N, K, out);
        return hipGetLastError();
    }
    if (L.fmt == 2) {
        q += (size_t)expert * N * K;
        const float *sc = reinterpret_cast<const float *>(sm) + (size_t)expert * (N / 128) * (K / 128);
        const int64_t words = (int64_t)N * K / 4;
        hipLaunchKernelGGL(dequant_fp8_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, s, q, sc, N, K,
                           out);
        return hipGetLastError();
    }
    q += (size_t)expert * N * (K / 2);
    sm += (size_t)expert * N * (K / G) * (L.fmt == 0 ? 2 : 1);
    const int64_t words = (int64_t)N * K / 8;
    dim3 grid((unsigned)((words + 255) / 256));
    if (L.fmt == 0) hipLaunchKernelGGL(dequant_kernel<0>, grid, dim3(256), 0, s, q, sm, N, K, out);
    else hipLaunchKernelGGL(dequant_kernel<1>, grid, dim3(256), 0, s, q, sm, N, K, out);
    return hipGetLastError();
}

hipError_t launch_residual(const uint16_t *x, const float *y, int64_t n, uint16_t *out, hipStream_t s) {
    hipLaunchKernelGGL(residual_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, y, n, out);
    return hipGetLastError();
}

}  // namespace moeq4
