// Prefill path: grouped expert GEMMs on the gfx950 matrix cores.
//
// Prefill runs the experts over rows grouped by routed expert (drama-rs page,
// "Apple Silicon (MLX)": prefill groups rows by routed expert; "Layout":
// prefill is a grouped MoE).  For expert e with M_e routed rows this is
//   GEMM1  [M_e x H] x [H x 2I]  (gate and up) -> SwiGLU -> h [M_e x I]
//   GEMM2  [M_e x I] x [I x H]   (down)        -> gate-weighted add into y.
//
// Exact integer tiles.  A 4-bit code unpacks to the exact 16-bit float
// OFF + q (bf16 OFF = 128 for GEMM1, whose other operand is bf16 x; f16
// OFF = 1024 for GEMM2, whose other operand is h rounded to f16).  With the
// row sums xs_g = sum_{k in group g} a_k of the activation operand,
//   sum_{k in g} a_k w_k = s_g * ( sum_{k in g} a_k (OFF + q_k) + c_g xs_g ),
//   c_g = m_g / s_g - OFF (asym, w = s q + m)  or  -8 - OFF (sym, w = s (q - 8)).
// The accumulator of a column is kept divided by the current group's scale:
// before group g it is rescaled by s_{g-1} / s_g and c_g xs_g is added; the
// matrix cores then add sum a (OFF + q) for the group; after the last group it
// is multiplied by s_last.  One fused multiply-add per output and group.  A
// zero scale is replaced by 2^-40 (its group then contributes m * xs, or 0,
// up to a relative 2^-40).
//
// Tiles: 128 rows (one tile-list entry, <= 128 rows of one expert) x 128
// columns per workgroup of 4 waves.  Wave w owns columns [32w, 32w+32) of
// both N-subtiles (GEMM1: the gate rows and the up rows of the same 32 h
// columns, so SwiGLU pairs in registers; GEMM2: two groups of 32 output
// columns, 64 per wave, 256 per workgroup) for all 4 M-subtiles of 32 rows.
// M-subtiles past the tile's rows are skipped.  The activation tile is staged
// in LDS (double-buffered, codes order PERM8 within 8-element groups); each
// lane streams the packed codes of its own column straight into registers
// one group ahead.
#include "moe_internal.h"

namespace moeq4 {

constexpr int PF_BLOCK = 256;
constexpr int BM = PREFILL_BM;  // 128
constexpr float ZERO_SCALE_SUB = 9.094947017729282e-13f;  // 2^-40

// xsum[t][g] = sum_{k in group g} x[t][k] (float), G = 64 or 128.
__global__ __launch_bounds__(256) void xsum_kernel(const uint16_t *__restrict__ x, int64_t T, int H, int G,
                                                   float *__restrict__ xsum) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int ng = H / G;
    if (i >= T * ng) return;
    const int64_t t = i / ng;
    const int g = (int)(i % ng);
    const uint4 *src = reinterpret_cast<const uint4 *>(x + t * H + (size_t)g * G);
    float s = 0.f;
    for (int j = 0; j < G / 8; ++j) {
        const uint4 v = src[j];
        s += bf16_pair_sum(v.x) + bf16_pair_sum(v.y) + bf16_pair_sum(v.z) + bf16_pair_sum(v.w);
    }
    xsum[i] = s;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float *__restrict__ p, int64_t n) {
    const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i + 3 < n) {
        *reinterpret_cast<float4 *>(p + i) = make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
        for (int64_t j = i; j < n; ++j) p[j] = 0.f;
    }
}

template <int FMT>
__device__ __forceinline__ void group_scale(const uint16_t *__restrict__ sm_row, int g, float &s, float &c,
                                            float off) {
    float m;
    if (FMT == 0) {
        const uint32_t p = *reinterpret_cast<const uint32_t *>(sm_row + 2 * g);
        s = f16_to_f32((uint16_t)(p & 0xffffu));
        m = f16_to_f32((uint16_t)(p >> 16));
    } else {
        s = f16_to_f32(sm_row[g]);
        m = 0.f;
    }
    if (s == 0.f) s = ZERO_SCALE_SUB;
    c = FMT == 0 ? __fdividef(m, s) - off : -8.0f - off;
}

// STAGE 1: A = x rows gathered through perm (bf16), B = gate | up codes,
//          epilogue SwiGLU -> h (f16) and hsum per h group.
// STAGE 2: A = h rows (f16, contiguous sorted rows), B = down codes,
//          epilogue gate-weighted float atomic add into y.
template <int FMT, int STAGE>
__global__ __launch_bounds__(PF_BLOCK) void grouped_gemm_kernel(
    const uint16_t *__restrict__ act,      // STAGE 1: x [T][H]; STAGE 2: h [P][I]
    const float *__restrict__ act_sum,     // STAGE 1: xsum [T][H/G]; STAGE 2: hsum [P][I/G]
    int H, int I, int k, LayerPtrs L, const Tile *__restrict__ tiles, const int32_t *__restrict__ ntiles,
    const int32_t *__restrict__ perm, const float *__restrict__ topk_gate,
    uint16_t *__restrict__ h_out, float *__restrict__ hsum_out, float *__restrict__ y) {
    constexpr int G = FMT == 0 ? 64 : 128;
    constexpr int KSUB = G / 16;            // MFMA k-steps per group
    constexpr int PITCH = G + 8;            // LDS row pitch in 16-bit elements
    constexpr int CHUNKS = G / 8;           // 16-byte chunks per staged row
    constexpr int ALOADS = BM * CHUNKS / PF_BLOCK;  // staged chunks per thread
    constexpr int BDW = G / 16;             // code dwords per lane per N-subtile per group
    constexpr float OFF = STAGE == 1 ? OFFSET_BF16 : OFFSET_F16;
    constexpr uint32_t MAGIC = STAGE == 1 ? MAGIC_BF16 : MAGIC_F16;

    const int j = blockIdx.y;
    if (j >= *ntiles) return;
    const Tile tile = tiles[j];
    const int e = tile.expert, rows = tile.rows, row0 = tile.row0;
    const int K = STAGE == 1 ? H : I;         // contraction length
    const int NG = K / G;                     // groups along K
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;

    __shared__ __attribute__((aligned(16))) uint16_t s_a[2][BM * PITCH];
    __shared__ __attribute__((aligned(16))) float s_xs[(2048 / G) * BM];   // [group][row], NG <= 2048 / G
    __shared__ int s_tok[BM];
    __shared__ float s_gate[BM];

    // ---- rows of this tile: token (stage 1) or (token, gate) (stage 2)
    if (tid < BM) {
        int t = 0;
        float gt = 0.f;
        if (tid < rows) {
            const int p = perm[row0 + tid];
            t = p / k;
            gt = STAGE == 2 ? topk_gate[p] : 0.f;
        }
        s_tok[tid] = t;
        s_gate[tid] = gt;
    }
    __syncthreads();
    // activation row sums for all groups: s_xs[g][r]
    for (int i = tid; i < NG * BM; i += PF_BLOCK) {
        const int g = i / BM, r = i % BM;
        float v = 0.f;
        if (r < rows) v = STAGE == 1 ? act_sum[(size_t)s_tok[r] * NG + g] : act_sum[(size_t)(row0 + r) * NG + g];
        s_xs[i] = v;
    }

    // ---- columns of this lane
    // STAGE 1: n-subtile 0 = gate row, 1 = up row, both h column hc.
    // STAGE 2: n-subtile ns = down row d = base + 64 w + 32 ns + l32.
    const int col_base = STAGE == 1 ? blockIdx.x * 128 + wave * 32 : blockIdx.x * 256 + wave * 64;
    const uint8_t *bq[2];
    const uint16_t *bsm[2];
    {
        const size_t row_bytes = (size_t)K / 2;
        const size_t sm_row = (size_t)NG * (FMT == 0 ? 2 : 1);
        if (STAGE == 1) {
            const size_t r = (size_t)e * I + col_base + l32;
            bq[0] = L.gq + r * row_bytes;
            bq[1] = L.uq + r * row_bytes;
            bsm[0] = L.gsm + r * sm_row;
            bsm[1] = L.usm + r * sm_row;
        } else {
#pragma unroll
            for (int ns = 0; ns < 2; ++ns) {
                const size_t r = (size_t)e * H + col_base + 32 * ns + l32;
                bq[ns] = L.dq + r * row_bytes;
                bsm[ns] = L.dsm + r * sm_row;
            }
        }
    }

    // ---- staging of activation chunks: chunk i of this thread = row r, 8-col chunk cc
    auto load_a = [&](int g, uint4 (&areg)[ALOADS]) {
#pragma unroll
        for (int i = 0; i < ALOADS; ++i) {
            const int flat = tid + i * PF_BLOCK;
            const int r = flat / CHUNKS, cc = flat % CHUNKS;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (r < rows) {
                const uint16_t *src = STAGE == 1 ? act + (size_t)s_tok[r] * H : act + (size_t)(row0 + r) * I;
                v = *reinterpret_cast<const uint4 *>(src + (size_t)g * G + cc * 8);
            }
            areg[i] = v;
        }
    };
    auto store_a = [&](int buf, const uint4 (&areg)[ALOADS]) {
#pragma unroll
        for (int i = 0; i < ALOADS; ++i) {
            const int flat = tid + i * PF_BLOCK;
            const int r = flat / CHUNKS, cc = flat % CHUNKS;
            uint4 o;
            perm8(areg[i].x, areg[i].y, areg[i].z, areg[i].w, o.x, o.y, o.z, o.w);
            *reinterpret_cast<uint4 *>(&s_a[buf][r * PITCH + cc * 8]) = o;
        }
    };
    auto load_b = [&](int g, uint32_t (&bd)[2][BDW], float (&s)[2], float (&c)[2]) {
#pragma unroll
        for (int ns = 0; ns < 2; ++ns) {
            const uint8_t *src = bq[ns] + (size_t)g * (G / 2) + hf * (G / 4);
#pragma unroll
            for (int q = 0; q < BDW; q += 4) {
                const uint4 v = *reinterpret_cast<const uint4 *>(src + 4 * q);
                bd[ns][q] = v.x;
                bd[ns][q + 1] = v.y;
                bd[ns][q + 2] = v.z;
                bd[ns][q + 3] = v.w;
            }
            group_scale<FMT>(bsm[ns], g, s[ns], c[ns], OFF);
        }
    };

    f32x16_t acc[4][2];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ns = 0; ns < 2; ++ns)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][ns][r] = 0.f;

    uint4 areg[ALOADS];
    uint32_t bcur[2][BDW], bnext[2][BDW];
    float scur[2], ccur[2], snext[2], cnext[2], sprev[2] = {1.f, 1.f};
    load_a(0, areg);
    load_b(0, bcur, scur, ccur);
    store_a(0, areg);
    __syncthreads();

    const int msub = (rows + 31) / 32;  // active M-subtiles
    for (int g = 0; g < NG; ++g) {
        const int buf = g & 1;
        if (g + 1 < NG) {
            load_a(g + 1, areg);
            load_b(g + 1, bnext, snext, cnext);
        }
        // rescale to this group's scale and add c_g * xs_g (rows of this lane)
#pragma unroll
        for (int ns = 0; ns < 2; ++ns) {
            const float ratio = g == 0 ? 0.f : __fdividef(sprev[ns], scur[ns]);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                if (mi < msub) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float4 xv = *reinterpret_cast<const float4 *>(
                            &s_xs[g * BM + 32 * mi + 8 * q + 4 * hf]);
                        acc[mi][ns][4 * q + 0] = fmaf(acc[mi][ns][4 * q + 0], ratio, ccur[ns] * xv.x);
                        acc[mi][ns][4 * q + 1] = fmaf(acc[mi][ns][4 * q + 1], ratio, ccur[ns] * xv.y);
                        acc[mi][ns][4 * q + 2] = fmaf(acc[mi][ns][4 * q + 2], ratio, ccur[ns] * xv.z);
                        acc[mi][ns][4 * q + 3] = fmaf(acc[mi][ns][4 * q + 3], ratio, ccur[ns] * xv.w);
                    }
                }
            }
        }
        // matrix cores: acc += A (OFF + q)
#pragma unroll
        for (int s = 0; s < KSUB; ++s) {
            uint32_t bw[2][4];
#pragma unroll
            for (int ns = 0; ns < 2; ++ns)
#pragma unroll
                for (int p = 0; p < 4; ++p) bw[ns][p] = unpack_pair<MAGIC>(bcur[ns][s], p);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                if (mi < msub) {
                    const uint4 av = *reinterpret_cast<const uint4 *>(
                        &s_a[buf][(32 * mi + l32) * PITCH + hf * (G / 2) + 8 * s]);
#pragma unroll
                    for (int ns = 0; ns < 2; ++ns) {
                        const u32x4_t bv = {bw[ns][0], bw[ns][1], bw[ns][2], bw[ns][3]};
                        const u32x4_t aw = {av.x, av.y, av.z, av.w};
                        if (STAGE == 1)
                            acc[mi][ns] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                __builtin_bit_cast(bf16x8_t, aw), __builtin_bit_cast(bf16x8_t, bv), acc[mi][ns], 0, 0, 0);
                        else
                            acc[mi][ns] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                                __builtin_bit_cast(f16x8_t, aw), __builtin_bit_cast(f16x8_t, bv), acc[mi][ns], 0, 0, 0);
                    }
                }
            }
        }
        if (g + 1 < NG) store_a(buf ^ 1, areg);
        __syncthreads();
        if (g + 1 < NG) {
#pragma unroll
            for (int ns = 0; ns < 2; ++ns) {
                sprev[ns] = scur[ns];
                scur[ns] = snext[ns];
                ccur[ns] = cnext[ns];
#pragma unroll
                for (int q = 0; q < BDW; ++q) bcur[ns][q] = bnext[ns][q];
            }
        }
    }

    // ---- epilogue.  Accumulator element r of lane (l32, hf) in M-subtile mi
    // is row 32 mi + 8 (r / 4) + 4 hf + (r % 4), column l32 of the subtile.
    if (STAGE == 1) {
        // h tile [BM][128] f16 in LDS (reusing the staging buffers), then
        // coalesced stores and per-group sums of the rounded values.
        uint16_t *s_h = &s_a[0][0];
        constexpr int HP = 128 + 8;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = 32 * mi + 8 * (r / 4) + 4 * hf + (r % 4);
                const float gv = acc[mi][0][r] * scur[0];
                const float uv = acc[mi][1][r] * scur[1];
                const _Float16 hv = (_Float16)(silu(gv) * uv);
                s_h[row * HP + wave * 32 + l32] = __builtin_bit_cast(uint16_t, hv);
            }
        }
        __syncthreads();
        // stores: 128 rows x 256 bytes
        for (int i = tid; i < BM * 16; i += PF_BLOCK) {
            const int row = i / 16, cc = i % 16;
            if (row < rows)
                *reinterpret_cast<uint4 *>(h_out + (size_t)(row0 + row) * I + blockIdx.x * 128 + cc * 8) =
                    *reinterpret_cast<const uint4 *>(&s_h[row * HP + cc * 8]);
        }
        // group sums of h for the second product: 128 / G groups per row
        constexpr int GPR = 128 / G;
        for (int i = tid; i < BM * GPR; i += PF_BLOCK) {
            const int row = i / GPR, gg = i % GPR;
            if (row < rows) {
                float sum = 0.f;
                for (int c = 0; c < G; ++c) sum += (float)__builtin_bit_cast(_Float16, s_h[row * HP + gg * G + c]);
                hsum_out[(size_t)(row0 + row) * (I / G) + blockIdx.x * GPR + gg] = sum;
            }
        }
    } else {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            if (mi < msub) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 32 * mi + 8 * (r / 4) + 4 * hf + (r % 4);
                    if (row < rows) {
                        const float gt = s_gate[row];
                        float *dst = y + (size_t)s_tok[row] * H + col_base + l32;
                        unsafeAtomicAdd(dst, gt * (acc[mi][0][r] * scur[0]));
                        unsafeAtomicAdd(dst + 32, gt * (acc[mi][1][r] * scur[1]));
                    }
                }
            }
        }
    }
}

template <int FMT>
static hipError_t launch_prefill_fmt(const uint16_t *x, const float *gate, int64_t T, int k, const LayerPtrs &L,
                                     const GroupOut &g, float *xsum, uint16_t *h, float *hsum, float *y,
                                     hipStream_t s, hipEvent_t const *ev) {
    constexpr int G = FMT == 0 ? 64 : 128;
    const int H = L.H, I = L.I;
    const int64_t tiles = max_tiles(T * k, L.E, BM);
    {
        const int64_t n = T * (H / G);
        hipLaunchKernelGGL(xsum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, T, H, G, xsum);
    }
    {
        const int64_t n = T * (int64_t)H;
        hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n / 4 + 256) / 256)), dim3(256), 0, s, y, n);
    }
    launch_k(grouped_gemm_kernel<FMT, 1>, dim3(I / 128, (unsigned)tiles), dim3(PF_BLOCK), s, ev ? ev[0] : nullptr,
             ev ? ev[1] : nullptr, x, (const float *)xsum, H, I, k, L, (const Tile *)g.tiles,
             (const int32_t *)g.ntiles, (const int32_t *)g.perm, gate, h, hsum, y);
    launch_k(grouped_gemm_kernel<FMT, 2>, dim3(H / 256, (unsigned)tiles), dim3(PF_BLOCK), s, ev ? ev[2] : nullptr,
             ev ? ev[3] : nullptr, (const uint16_t *)h, (const float *)hsum, H, I, k, L, (const Tile *)g.tiles,
             (const int32_t *)g.ntiles, (const int32_t *)g.perm, gate, h, hsum, y);
    return hipGetLastError();
}

hipError_t launch_fill_zero(float *p, int64_t n, hipStream_t s) {
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n / 4 + 256) / 256)), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

hipError_t launch_fill_zero_u32(uint32_t *p, int64_t n, hipStream_t s) {
    return launch_fill_zero(reinterpret_cast<float *>(p), n, s);  // all-zero bits either way
}

hipError_t launch_prefill_experts(const uint16_t *x, const float *gate, int64_t T, int k, const LayerPtrs &L,
                                  const GroupOut &g, float *xsum, uint16_t *h, float *hsum, float *y,
                                  hipStream_t s, hipEvent_t const *ev) {
    return L.fmt == 0 ? launch_prefill_fmt<0>(x, gate, T, k, L, g, xsum, h, hsum, y, s, ev)
                      : launch_prefill_fmt<1>(x, gate, T, k, L, g, xsum, h, hsum, y, s, ev);
}

}  // namespace moeq4
