// Decode path: fused-dequant GEMVs over the active experts' packed nibbles.
//
// Decode is bound by the bytes of expert weights read from HBM (drama-rs
// page, "Experts: where they run": decode reads about 1 GB of FP8 experts per
// frame and is memory-bandwidth-bound).  Each code is read once, coalesced (a
// lane takes 16 bytes = 32 codes, consecutive lanes consecutive bytes), and
// applied to every token routed to its expert.
//
// One kernel per layer does all expert work.  Workgroup (tile j, chunk c)
// takes the <= 4 tokens of tile j (one expert e) and the 64 rows
// [64c, 64c+64) of h:
//   1. gate/up GEMV over those 64 rows (lanes along the input dimension, a
//      segmented wave reduction per row), SwiGLU in registers, h chunk -> LDS;
//   2. the matching split-K slice of the down GEMV: every output row d, the 64
//      inputs of the chunk (two lanes per row), multiplied by the token's gate
//      and added into y with float atomics (y is cleared beforehand).
// So the down codes of an expert are read once in total, split over its
// chunk workgroups; chunk workgroups of one tile are numbered to land on the
// same XCD so that they share the L2 lines of the down rows.
//
// Group arithmetic.  For a group of codes q_k with scale s and min m,
//   sum_k a_k (s q_k + m) = s * sum_k a_k (OFF + q_k) + (m - OFF s) * sum_k a_k
// where OFF + q_k is the exact bf16 value a nibble unpacks to (OFF = 128);
// symmetric groups use m = -8 s.  sum a (OFF + q) runs on the packed bf16
// dot-product instruction with fp32 accumulation.  h stays fp32 between the
// two products: for the down slice it is split into bf16 hi + lo parts
// (|h - hi - lo| <= 2^-17 |h|).
#include "group_dev.h"
#include "route_dev.h"

namespace moeq4 {

constexpr int DX_BLOCK = 256;
constexpr int DX_CH = 64;  // h rows per workgroup = down K-chunk

// Activation chunk [32c, 32c+32) of a bf16 row in PERM8 order, and its sum.
__device__ __forceinline__ void load_x_chunk(const uint16_t *__restrict__ xrow, int c, uint32_t xp[16],
                                             float &xs) {
    const uint4 *src = reinterpret_cast<const uint4 *>(xrow + 32 * c);
    xs = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint4 v = src[j];
        perm8(v.x, v.y, v.z, v.w, xp[4 * j + 0], xp[4 * j + 1], xp[4 * j + 2], xp[4 * j + 3]);
        xs += bf16_pair_sum(v.x) + bf16_pair_sum(v.y) + bf16_pair_sum(v.z) + bf16_pair_sum(v.w);
    }
}

// Scale and min of group g of a row (sym: min = -8 scale).
template <int FMT>
__device__ __forceinline__ void load_group(const uint16_t *__restrict__ sm_row, int g, float &s, float &m) {
    if (FMT == 0) {
        const uint32_t p = *reinterpret_cast<const uint32_t *>(sm_row + 2 * g);
        s = f16_to_f32((uint16_t)(p & 0xffffu));
        m = f16_to_f32((uint16_t)(p >> 16));
    } else {
        s = f16_to_f32(sm_row[g]);
        m = -8.0f * s;
    }
}

// sum over the 32 codes of a dword quad (PERM8 order) against activations a.
__device__ __forceinline__ float dot32(const uint4 w, const uint32_t a[16], float acc) {
    const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int p = 0; p < 4; ++p) acc = dot2_bf16(unpack_pair<MAGIC_BF16>(d[q], p), a[4 * q + p], acc);
    return acc;
}

// Tile fields made safe to index with (a workspace that was never filled
// gives garbage numbers, not out-of-bounds accesses).
__device__ __forceinline__ Tile sane_tile(Tile t, int E, int P) {
    t.expert = clamp_expert(t.expert, E);
    t.rows = t.rows < 0 ? 0 : (t.rows > DECODE_TT ? DECODE_TT : t.rows);
    t.rows = t.rows > P ? P : t.rows;
    t.row0 = t.row0 < 0 ? 0 : (t.row0 > P - t.rows ? P - t.rows : t.row0);
    return t;
}

// grid.x = ntg * (I / 64) workgroups: tile j = bid % ntg, chunk c = bid / ntg
// (ntg a multiple of 8, so that all chunks of a tile share bid mod 8).
// LPR = H / 32 lanes per gate/up row.
template <int LPR, int FMT>
__global__ __launch_bounds__(DX_BLOCK) void decode_experts_kernel(
    const uint16_t *__restrict__ x, int H, int I, int k, int P, LayerPtrs L, const Tile *__restrict__ tiles,
    const int32_t *__restrict__ ntiles, const int32_t *__restrict__ perm, const float *__restrict__ topk_gate,
    int ntg, float *__restrict__ y) {
    constexpr int RPW = WAVE / LPR;           // gate/up rows per wave per load
    constexpr int ITERS = DX_CH / 4 / RPW > 0 ? DX_CH / 4 / RPW : 1;  // loads per wave for 64 rows
    constexpr int NB = ITERS < 4 ? ITERS : 4;                        // rows in flight per wave
    constexpr int G = FMT == 0 ? 64 : 128;
    __shared__ float s_h[DECODE_TT][DX_CH];
    __shared__ int s_tok[DECODE_TT];
    __shared__ float s_gate[DECODE_TT];

    const int j = blockIdx.x % ntg, chunk = blockIdx.x / ntg;
    if (j >= *ntiles) return;
    const Tile tile = sane_tile(tiles[j], L.E, P);
    const int e = tile.expert, nt = tile.rows;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = chunk * DX_CH;

    if (tid < DECODE_TT) {
        int t = 0;
        float gt = 0.f;
        if (tid < nt) {
            int p = perm[tile.row0 + tid];
            p = p < 0 ? 0 : (p >= P ? P - 1 : p);
            t = p / k;
            gt = topk_gate[p];
        }
        s_tok[tid] = t;
        s_gate[tid] = gt;
    }
    __syncthreads();

    // ---- 1. gate/up rows [n0, n0 + 64) + SwiGLU -> s_h
    {
        const int c = lane % LPR, sub = lane / LPR;
        uint32_t xp[DECODE_TT][16];
        float xs[DECODE_TT];
#pragma unroll
        for (int u = 0; u < DECODE_TT; ++u) {
            if (u < nt) {
                load_x_chunk(x + (size_t)s_tok[u] * H, c, xp[u], xs[u]);
            } else {
#pragma unroll
                for (int q = 0; q < 16; ++q) xp[u][q] = 0u;
                xs[u] = 0.f;
            }
        }
        const size_t row_bytes = (size_t)H / 2;
        const size_t smr = (size_t)(H / G) * (FMT == 0 ? 2 : 1);
        const int gi = (32 * c) / G;
        for (int it0 = 0; it0 < ITERS; it0 += NB) {
            uint4 gv[NB], uv[NB];
            float sg[NB], mg[NB], su[NB], mu[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) {  // NB rows of gate and of up in flight
                const int nl = ((it0 + b) * 4 + wave) * RPW + sub;
                const size_t row = (size_t)e * I + n0 + (nl < DX_CH ? nl : 0);
                gv[b] = *reinterpret_cast<const uint4 *>(L.gq + row * row_bytes + 16 * c);
                uv[b] = *reinterpret_cast<const uint4 *>(L.uq + row * row_bytes + 16 * c);
                load_group<FMT>(L.gsm + row * smr, gi, sg[b], mg[b]);
                load_group<FMT>(L.usm + row * smr, gi, su[b], mu[b]);
            }
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int nl = ((it0 + b) * 4 + wave) * RPW + sub;  // >= 64 only when H < 512
                const float cg = mg[b] - OFFSET_BF16 * sg[b], cu = mu[b] - OFFSET_BF16 * su[b];
#pragma unroll
                for (int u = 0; u < DECODE_TT; ++u) {
                    const float pg = seg_sum<LPR>(fmaf(sg[b], dot32(gv[b], xp[u], 0.f), cg * xs[u]));
                    const float pu = seg_sum<LPR>(fmaf(su[b], dot32(uv[b], xp[u], 0.f), cu * xs[u]));
                    if (c == 0 && nl < DX_CH) s_h[u][nl] = silu(pg) * pu;
                }
            }
        }
    }
    __syncthreads();

    // ---- 2. down rows d, inputs [n0, n0 + 64): two lanes per row, 32 rows per wave
    {
        const int half = lane & 1, rr = lane >> 1;
        uint32_t hh[DECODE_TT][16], hl[DECODE_TT][16];
        float hs[DECODE_TT];
#pragma unroll
        for (int u = 0; u < DECODE_TT; ++u) {
            hs[u] = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t hi[4], lo[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const float v0 = s_h[u][32 * half + 8 * q + 2 * p], v1 = s_h[u][32 * half + 8 * q + 2 * p + 1];
                    const uint32_t h0 = f32_to_bf16_rne(v0), h1 = f32_to_bf16_rne(v1);
                    const uint32_t l0 = f32_to_bf16_rne(v0 - bf16_to_f32(h0));
                    const uint32_t l1 = f32_to_bf16_rne(v1 - bf16_to_f32(h1));
                    hi[p] = h0 | (h1 << 16);
                    lo[p] = l0 | (l1 << 16);
                    hs[u] += (bf16_to_f32(h0) + bf16_to_f32(l0)) + (bf16_to_f32(h1) + bf16_to_f32(l1));
                }
                perm8(hi[0], hi[1], hi[2], hi[3], hh[u][4 * q], hh[u][4 * q + 1], hh[u][4 * q + 2], hh[u][4 * q + 3]);
                perm8(lo[0], lo[1], lo[2], lo[3], hl[u][4 * q], hl[u][4 * q + 1], hl[u][4 * q + 2], hl[u][4 * q + 3]);
            }
        }
        const size_t row_bytes = (size_t)I / 2;
        const size_t smr = (size_t)(I / G) * (FMT == 0 ? 2 : 1);
        const int gi = n0 / G;
        constexpr int BATCH = 4;
        for (int d0 = wave * 32; d0 < H; d0 += 128 * BATCH) {
            uint4 dv[BATCH];
            float sd[BATCH], md[BATCH];
#pragma unroll
            for (int b = 0; b < BATCH; ++b) {
                const int d = d0 + b * 128 + rr;
                dv[b] = make_uint4(0, 0, 0, 0);
                sd[b] = md[b] = 0.f;
                if (d < H) {
                    const size_t row = (size_t)e * H + d;
                    dv[b] = *reinterpret_cast<const uint4 *>(L.dq + row * row_bytes + n0 / 2 + 16 * half);
                    load_group<FMT>(L.dsm + row * smr, gi, sd[b], md[b]);
                }
            }
#pragma unroll
            for (int b = 0; b < BATCH; ++b) {
                const int d = d0 + b * 128 + rr;
                const float cd = md[b] - OFFSET_BF16 * sd[b];
#pragma unroll
                for (int u = 0; u < DECODE_TT; ++u) {
                    float a = dot32(dv[b], hh[u], 0.f);
                    a = dot32(dv[b], hl[u], a);
                    float part = fmaf(sd[b], a, cd * hs[u]);
                    part += __shfl_xor(part, 1, WAVE);
                    if (half == 0 && u < nt && d < H)
                        unsafeAtomicAdd(y + (size_t)s_tok[u] * H + d, s_gate[u] * part);
                }
            }
        }
    }
}

// Routing of a few tokens in one launch.  Workgroups of 16 waves compute the
// router logits (one expert per wave, when router weights are given); the
// workgroup that arrives last (a counter in the workspace, zero between
// calls) takes the top-k of every token and groups the pairs by expert.  With
// yres the layer input is the residual step bf16(x + yres), computed on the
// fly and written to xout.  Every workgroup also clears its share of y for the
// expert kernel's atomics.
template <int NPL>
__global__ __launch_bounds__(1024) void decode_route_group_kernel(
    const uint16_t *__restrict__ x, const float *__restrict__ yres, uint16_t *__restrict__ xout,
    const uint16_t *__restrict__ wr, const float *__restrict__ bias, int T, int H, int E, int k,
    uint16_t *__restrict__ logits, int32_t *__restrict__ idx, float *__restrict__ gate, GroupOut g,
    float *__restrict__ yclear, unsigned int *__restrict__ counter) {
    __shared__ int s_last;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nb = gridDim.x;
    const int64_t n = (int64_t)T * H;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + tid; i < n; i += (int64_t)nb * blockDim.x) {
        yclear[i] = 0.f;
        if (yres) xout[i] = f32_to_bf16_rne(bf16_to_f32(x[i]) + yres[i]);
    }
    if (wr) {
        const int e = blockIdx.x * 16 + wave;
        if (e < E) {
            const double b = bias ? (double)bias[e] : 0.0;
            for (int t = 0; t < T; ++t) {
                const double acc = router_dot_wave(x + (size_t)t * H, yres ? yres + (size_t)t * H : nullptr,
                                                   wr + (size_t)e * H, H);
                if (lane == 0) logits[(size_t)t * E + e] = f32_to_bf16_rne((float)(acc + b));
            }
        }
    }
    if (nb > 1) {
        __threadfence();
        __syncthreads();
        if (tid == 0) s_last = atomicAdd(counter, 1u) == (unsigned)(nb - 1);
        __syncthreads();
        if (!s_last) return;
        __threadfence();
    }
    for (int t = wave; t < T; t += 16) topk_token_wave<NPL>(logits + (size_t)t * E, E, k, idx + t * k, gate + t * k);
    __syncthreads();
    group_block_single(idx, T * k, E, g);
    if (tid == 0 && nb > 1) *counter = 0u;
}

template <int FMT>
static hipError_t launch_experts_fmt(const uint16_t *x, const float *gate, int64_t T, int k, const LayerPtrs &L,
                                     const GroupOut &g, float *y, hipStream_t s) {
    const int H = L.H, I = L.I;
    const int P = (int)(T * k);
    const int ntg = (int)((max_tiles(P, L.E, DECODE_TT) + 7) / 8 * 8);
    dim3 grid((unsigned)(ntg * (I / DX_CH)));
    switch (H / 32) {
#define CASE(LP) \
    case LP: hipLaunchKernelGGL((decode_experts_kernel<LP, FMT>), grid, dim3(DX_BLOCK), 0, s, x, H, I, k, P, L, g.tiles, g.ntiles, g.perm, gate, ntg, y); break;
        CASE(2) CASE(4) CASE(8) CASE(16) CASE(32) CASE(64)
#undef CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_decode_experts(const uint16_t *x, const float *gate, int64_t T, int k, const LayerPtrs &L,
                                 const GroupOut &g, float *y, hipStream_t s) {
    return L.fmt == 0 ? launch_experts_fmt<0>(x, gate, T, k, L, g, y, s)
                      : launch_experts_fmt<1>(x, gate, T, k, L, g, y, s);
}

hipError_t launch_decode_route_group(const uint16_t *x, const float *yres, uint16_t *xout, const uint16_t *wr,
                                     const float *bias, int T, int H, int E, int k, uint16_t *logits, int32_t *idx,
                                     float *gate, const GroupOut &g, float *yclear, unsigned int *counter,
                                     hipStream_t s) {
    const int nb = wr ? (E + 15) / 16 : 1;
    const int npl = (E + 63) / 64;
#define LAUNCH(N) \
    hipLaunchKernelGGL(decode_route_group_kernel<N>, dim3(nb), dim3(1024), 0, s, x, yres, xout, wr, bias, T, H, E, k, logits, idx, gate, g, yclear, counter)
    if (npl <= 4) LAUNCH(4);
    else if (npl <= 8) LAUNCH(8);
    else LAUNCH(16);
#undef LAUNCH
    return hipGetLastError();
}

}  // namespace moeq4
