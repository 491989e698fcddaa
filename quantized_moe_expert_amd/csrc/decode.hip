// Decode path: fused-dequant GEMVs over the active experts' packed nibbles.
//
// Decode is bound by the bytes of expert weights read from HBM (drama-rs
// page, "Experts: where they run": decode reads about 1 GB of FP8 experts per
// frame and is memory-bandwidth-bound).  Each row of packed codes is read
// once, coalesced (a lane takes 16 bytes = 32 codes, consecutive lanes take
// consecutive bytes), and applied to every token routed to that expert.
//
// Group arithmetic.  For a group of codes q_k with scale s and min m,
//   sum_k x_k (s q_k + m) = s * sum_k x_k (OFF + q_k) + (m - OFF s) * sum_k x_k
// where OFF + q_k is the exact bf16 value the nibble unpacks to (OFF = 128);
// symmetric groups use m = -8 s.  The sums over x_k*(OFF+q_k) run on the
// packed bf16 dot-product instruction with fp32 accumulation; scale and min are
// applied once per 32 codes per lane, then a segmented wave reduction finishes
// each row.  h stays fp32: for the down projection it is split exactly-enough
// into bf16 hi + lo parts (h - hi - lo is below 2^-17 |h|).
#include "moe_internal.h"

namespace moeq4 {

constexpr int DEC_BLOCK = 256;

// Tokens of a tile -> per-lane activation chunks in PERM8 order.
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

// Scale and (asym) min of the group holding codes [32c, 32c+32) of a row.
template <int FMT>
__device__ __forceinline__ void load_group_params(const uint16_t *__restrict__ sm_row, int c, float &s, float &m) {
    if (FMT == 0) {
        const uint32_t p = *reinterpret_cast<const uint32_t *>(sm_row + 2 * (c >> 1));
        s = f16_to_f32((uint16_t)(p & 0xffffu));
        m = f16_to_f32((uint16_t)(p >> 16));
    } else {
        s = f16_to_f32(sm_row[c >> 2]);
        m = -8.0f * s;
    }
}

// gate/up + SwiGLU.  grid = (I / rows_per_block, max tiles); LPR = H / 32.
template <int LPR, int FMT>
__global__ __launch_bounds__(DEC_BLOCK) void decode_gateup_kernel(
    const uint16_t *__restrict__ x, int H, int I, int k, LayerPtrs L, const Tile *__restrict__ tiles,
    const int32_t *__restrict__ ntiles, const int32_t *__restrict__ perm, int rows_per_block,
    float *__restrict__ h) {
    constexpr int RPW = WAVE / LPR;  // rows per wave per step
    const int j = blockIdx.y;
    if (j >= *ntiles) return;
    const Tile tile = tiles[j];
    const int e = tile.expert, nt = tile.rows;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = lane % LPR, sub = lane / LPR;

    uint32_t xp[DECODE_TT][16];
    float xs[DECODE_TT];
#pragma unroll
    for (int u = 0; u < DECODE_TT; ++u) {
        if (u < nt) {
            const int t = perm[tile.row0 + u] / k;
            load_x_chunk(x + (size_t)t * H, c, xp[u], xs[u]);
        } else {
#pragma unroll
            for (int q = 0; q < 16; ++q) xp[u][q] = 0u;
            xs[u] = 0.f;
        }
    }
    const int G = FMT == 0 ? 64 : 128;
    const size_t row_bytes = (size_t)H / 2;
    const size_t sm_per_row = (size_t)(H / G) * (FMT == 0 ? 2 : 1);
    const int n_begin = blockIdx.x * rows_per_block;
    for (int r = wave * RPW; r < rows_per_block; r += 4 * RPW) {
        const bool valid = r + sub < rows_per_block;  // false only when I is smaller than one block step
        const int n = n_begin + (valid ? r + sub : 0);
        const size_t row = (size_t)e * I + n;
        uint4 gv = make_uint4(0, 0, 0, 0), uv = gv;
        float sg = 0.f, mg = 0.f, su = 0.f, mu = 0.f;
        if (valid) {
            gv = *reinterpret_cast<const uint4 *>(L.gq + row * row_bytes + 16 * c);
            uv = *reinterpret_cast<const uint4 *>(L.uq + row * row_bytes + 16 * c);
            load_group_params<FMT>(L.gsm + row * sm_per_row, c, sg, mg);
            load_group_params<FMT>(L.usm + row * sm_per_row, c, su, mu);
        }
        uint32_t gw[16], uw[16];
        const uint32_t gd[4] = {gv.x, gv.y, gv.z, gv.w}, ud[4] = {uv.x, uv.y, uv.z, uv.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                gw[4 * q + p] = unpack_pair<MAGIC_BF16>(gd[q], p);
                uw[4 * q + p] = unpack_pair<MAGIC_BF16>(ud[q], p);
            }
        const float cg = mg - OFFSET_BF16 * sg, cu = mu - OFFSET_BF16 * su;
        float pg[DECODE_TT], pu[DECODE_TT];
#pragma unroll
        for (int u = 0; u < DECODE_TT; ++u) {
            float ag = 0.f, au = 0.f;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                ag = dot2_bf16(gw[q], xp[u][q], ag);
                au = dot2_bf16(uw[q], xp[u][q], au);
            }
            pg[u] = seg_sum<LPR>(fmaf(sg, ag, cg * xs[u]));
            pu[u] = seg_sum<LPR>(fmaf(su, au, cu * xs[u]));
        }
        if (c == 0 && valid) {
#pragma unroll
            for (int u = 0; u < DECODE_TT; ++u)
                if (u < nt) h[(size_t)(tile.row0 + u) * I + n] = silu(pg[u]) * pu[u];
        }
    }
}

// down.  grid = (H / rows_per_block, max tiles); LPR = I / 32.
template <int LPR, int FMT>
__global__ __launch_bounds__(DEC_BLOCK) void decode_down_kernel(int H, int I, LayerPtrs L,
                                                                const Tile *__restrict__ tiles,
                                                                const int32_t *__restrict__ ntiles,
                                                                const float *__restrict__ h, int rows_per_block,
                                                                float *__restrict__ o) {
    constexpr int RPW = WAVE / LPR;
    const int j = blockIdx.y;
    if (j >= *ntiles) return;
    const Tile tile = tiles[j];
    const int e = tile.expert, nt = tile.rows;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = lane % LPR, sub = lane / LPR;

    uint32_t hh[DECODE_TT][16], hl[DECODE_TT][16];
    float hs[DECODE_TT];
#pragma unroll
    for (int u = 0; u < DECODE_TT; ++u) {
        hs[u] = 0.f;
        if (u < nt) {
            const float4 *src = reinterpret_cast<const float4 *>(h + (size_t)(tile.row0 + u) * I + 32 * c);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 a = src[2 * q], b = src[2 * q + 1];
                const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
                uint32_t hi[4], lo[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const uint32_t h0 = f32_to_bf16_rne(v[2 * p]), h1 = f32_to_bf16_rne(v[2 * p + 1]);
                    const uint32_t l0 = f32_to_bf16_rne(v[2 * p] - bf16_to_f32(h0));
                    const uint32_t l1 = f32_to_bf16_rne(v[2 * p + 1] - bf16_to_f32(h1));
                    hi[p] = h0 | (h1 << 16);
                    lo[p] = l0 | (l1 << 16);
                    hs[u] += (bf16_to_f32(h0) + bf16_to_f32(l0)) + (bf16_to_f32(h1) + bf16_to_f32(l1));
                }
                perm8(hi[0], hi[1], hi[2], hi[3], hh[u][4 * q], hh[u][4 * q + 1], hh[u][4 * q + 2], hh[u][4 * q + 3]);
                perm8(lo[0], lo[1], lo[2], lo[3], hl[u][4 * q], hl[u][4 * q + 1], hl[u][4 * q + 2], hl[u][4 * q + 3]);
            }
        } else {
#pragma unroll
            for (int q = 0; q < 16; ++q) hh[u][q] = hl[u][q] = 0u;
        }
    }
    const int G = FMT == 0 ? 64 : 128;
    const size_t row_bytes = (size_t)I / 2;
    const size_t sm_per_row = (size_t)(I / G) * (FMT == 0 ? 2 : 1);
    const int d_begin = blockIdx.x * rows_per_block;
    for (int r = wave * RPW; r < rows_per_block; r += 4 * RPW) {
        const bool valid = r + sub < rows_per_block;  // false only when H is smaller than one block step
        const int d = d_begin + (valid ? r + sub : 0);
        const size_t row = (size_t)e * H + d;
        uint4 dv = make_uint4(0, 0, 0, 0);
        float sd = 0.f, md = 0.f;
        if (valid) {
            dv = *reinterpret_cast<const uint4 *>(L.dq + row * row_bytes + 16 * c);
            load_group_params<FMT>(L.dsm + row * sm_per_row, c, sd, md);
        }
        uint32_t dw[16];
        const uint32_t dd[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int p = 0; p < 4; ++p) dw[4 * q + p] = unpack_pair<MAGIC_BF16>(dd[q], p);
        const float cd = md - OFFSET_BF16 * sd;
        float po[DECODE_TT];
#pragma unroll
        for (int u = 0; u < DECODE_TT; ++u) {
            float a = 0.f;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                a = dot2_bf16(dw[q], hh[u][q], a);
                a = dot2_bf16(dw[q], hl[u][q], a);
            }
            po[u] = seg_sum<LPR>(fmaf(sd, a, cd * hs[u]));
        }
        if (c == 0 && valid) {
#pragma unroll
            for (int u = 0; u < DECODE_TT; ++u)
                if (u < nt) o[(size_t)(tile.row0 + u) * H + d] = po[u];
        }
    }
}

// y[t][d] = sum_i gate[t][i] * o[inv[t*k+i]][d], slot order.
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ o, const float *__restrict__ gate,
                                                      const int32_t *__restrict__ inv, int H, int k,
                                                      float *__restrict__ y) {
    const int64_t t = blockIdx.y;
    const int d = blockIdx.x * 256 + threadIdx.x;
    if (d >= H) return;
    float acc = 0.f;
    for (int i = 0; i < k; ++i) acc = fmaf(gate[t * k + i], o[(size_t)inv[t * k + i] * H + d], acc);
    y[t * H + d] = acc;
}

template <int FMT>
static hipError_t launch_decode_fmt(const uint16_t *x, const float *gate, int64_t T, int k, const LayerPtrs &L,
                                    const GroupOut &g, float *h, float *o, float *y, hipStream_t s,
                                    hipEvent_t const *ev) {
    const int H = L.H, I = L.I;
    const int64_t tiles = max_tiles(T * k, L.E, DECODE_TT);
    stage_mark(ev, 0, s);
    // gate/up: 16 rows per block unless I is smaller
    {
        const int lpr = H / 32, rpw = 64 / lpr;
        int rpb = 4 * rpw < I ? 4 * rpw : I;
        while (rpb < 16 && rpb * 2 <= I) rpb *= 2;
        dim3 grid(I / rpb, (unsigned)tiles);
        switch (lpr) {
#define CASE(LP) \
    case LP: hipLaunchKernelGGL((decode_gateup_kernel<LP, FMT>), grid, dim3(DEC_BLOCK), 0, s, x, H, I, k, L, g.tiles, g.ntiles, g.perm, rpb, h); break;
            CASE(2) CASE(4) CASE(8) CASE(16) CASE(32) CASE(64)
#undef CASE
            default: return hipErrorInvalidValue;
        }
    }
    stage_mark(ev, 1, s);
    {
        const int lpr = I / 32, rpw = 64 / lpr;
        int rpb = 4 * rpw < H ? 4 * rpw : H;
        while (rpb < 32 && rpb * 2 <= H) rpb *= 2;
        dim3 grid(H / rpb, (unsigned)tiles);
        switch (lpr) {
#define CASE(LP) \
    case LP: hipLaunchKernelGGL((decode_down_kernel<LP, FMT>), grid, dim3(DEC_BLOCK), 0, s, H, I, L, g.tiles, g.ntiles, h, rpb, o); break;
            CASE(2) CASE(4) CASE(8) CASE(16) CASE(32) CASE(64)
#undef CASE
            default: return hipErrorInvalidValue;
        }
    }
    stage_mark(ev, 2, s);
    hipLaunchKernelGGL(combine_kernel, dim3((H + 255) / 256, (unsigned)T), dim3(256), 0, s, o, gate, g.inv, H, k, y);
    stage_mark(ev, 3, s);
    return hipGetLastError();
}

hipError_t launch_decode_experts(const uint16_t *x, const float *gate, int64_t T, int k, const LayerPtrs &L,
                                 const GroupOut &g, float *h, float *o, float *y, hipStream_t s,
                                 hipEvent_t const *ev) {
    return L.fmt == 0 ? launch_decode_fmt<0>(x, gate, T, k, L, g, h, o, y, s, ev)
                      : launch_decode_fmt<1>(x, gate, T, k, L, g, h, o, y, s, ev);
}

}  // namespace moeq4
