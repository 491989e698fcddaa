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

constexpr int DX_WAVES = 8;  // waves per expert workgroup

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

// 16 bf16 pairs (32 codes in PERM8 order) of a dword quad.
__device__ __forceinline__ void unpack32(const uint4 w, uint32_t out[16]) {
    const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int p = 0; p < 4; ++p) out[4 * q + p] = unpack_pair<MAGIC_BF16>(d[q], p);
}

__device__ __forceinline__ float dot16(const uint32_t w[16], const uint32_t a[16], float acc) {
#pragma unroll
    for (int i = 0; i < 16; ++i) acc = dot2_bf16(w[i], a[i], acc);
    return acc;
}

// Scale and min of a packed {scale, min} f16 pair (asym) or a scale (sym).
template <int FMT>
__device__ __forceinline__ uint32_t load_group_word(const uint16_t *__restrict__ sm_row, int g) {
    if (FMT == 0) return *reinterpret_cast<const uint32_t *>(sm_row + 2 * g);
    return (uint32_t)sm_row[g];
}
template <int FMT>
__device__ __forceinline__ void group_params(uint32_t word, float &s, float &m) {
    s = f16_to_f32((uint16_t)(word & 0xffffu));
    m = FMT == 0 ? f16_to_f32((uint16_t)(word >> 16)) : -8.0f * s;
}

// grid.x = ntg * (I / CH) workgroups of DX_WAVES waves (ntg = tile slots, a
// multiple of 8).  LPR = H / 32 lanes per gate/up row.  Every
// weight load of both phases is issued before any arithmetic, so a workgroup
// has all of its ~100 KB in flight at once.
template <int LPR, int FMT, int CH>
__global__ __launch_bounds__(DX_WAVES * 64) void decode_experts_kernel(
    const uint16_t *__restrict__ x, int H, int I, int k, int P, LayerPtrs L, const Tile *__restrict__ tiles,
    const int32_t *__restrict__ ntiles, const int32_t *__restrict__ perm, const float *__restrict__ topk_gate,
    int ntg, float *__restrict__ y) {
    constexpr int RPW = WAVE / LPR;                                          // gate/up rows per wave-load
    constexpr int GU = CH / DX_WAVES / RPW > 0 ? CH / DX_WAVES / RPW : 1;    // gate/up loads per lane
    constexpr int G = FMT == 0 ? 64 : 128;
    constexpr int DL = CH / 32;                                              // lanes per down row (1 or 2)
    constexpr int DRW = WAVE / DL;                                           // down rows per wave-load
    constexpr int DN = 2048 / (DX_WAVES * DRW);                              // down loads per lane (H <= 2048)
    __shared__ float s_h[DECODE_TT][CH];
    __shared__ int s_tok[DECODE_TT];
    __shared__ float s_gate[DECODE_TT];

    // Workgroups are dispatched round-robin over the 8 XCDs (bid mod 8).  The
    // I / CH chunks of tile j get bids (j / 8) * 8 * nch + c * 8 + j % 8: one
    // XCD, dispatched together, so they share that L2's lines of the down rows
    // (each chunk reads only a CH/2-byte slice of every row).
    const int nch = I / CH;
    const int j = (blockIdx.x % 8) + 8 * (blockIdx.x / (8 * nch)), chunk = (blockIdx.x / 8) % nch;
    if (j >= *ntiles) return;
    const Tile tile = sane_tile(tiles[j], L.E, P);
    const int e = tile.expert, nt = tile.rows;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = chunk * CH;

    // ---- issue every weight load: gate/up rows of this chunk, down slices
    const int c = lane % LPR, sub = lane / LPR;
    const int half = DL == 2 ? (lane & 1) : 0, rr = lane / DL;
    uint4 gv[GU], uv[GU], dv[DN];
    uint32_t gs[GU], us[GU], ds[DN];
    {
        const size_t row_bytes = (size_t)H / 2;
        const size_t smr = (size_t)(H / G) * (FMT == 0 ? 2 : 1);
        const int gi = (32 * c) / G;
#pragma unroll
        for (int b = 0; b < GU; ++b) {
            const int nl = (b * DX_WAVES + wave) * RPW + sub;
            const size_t row = (size_t)e * I + n0 + (nl < CH ? nl : 0);
            gv[b] = *reinterpret_cast<const uint4 *>(L.gq + row * row_bytes + 16 * c);
            uv[b] = *reinterpret_cast<const uint4 *>(L.uq + row * row_bytes + 16 * c);
            gs[b] = load_group_word<FMT>(L.gsm + row * smr, gi);
            us[b] = load_group_word<FMT>(L.usm + row * smr, gi);
        }
    }
    {
        const size_t row_bytes = (size_t)I / 2;
        const size_t smr = (size_t)(I / G) * (FMT == 0 ? 2 : 1);
        const int gi = n0 / G;
#pragma unroll
        for (int b = 0; b < DN; ++b) {
            const int d = (b * DX_WAVES + wave) * DRW + rr;
            const size_t row = (size_t)e * H + (d < H ? d : 0);
            dv[b] = *reinterpret_cast<const uint4 *>(L.dq + row * row_bytes + n0 / 2 + 16 * half);
            ds[b] = load_group_word<FMT>(L.dsm + row * smr, gi);
        }
    }
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

    // ---- 1. gate/up rows [n0, n0 + CH) + SwiGLU -> s_h
    {
        uint32_t xp[DECODE_TT][16];
        float xs[DECODE_TT];
#pragma unroll
        for (int u = 0; u < DECODE_TT; ++u) {
            xs[u] = 0.f;
            if (u < nt) load_x_chunk(x + (size_t)s_tok[u] * H, c, xp[u], xs[u]);
        }
#pragma unroll
        for (int b = 0; b < GU; ++b) {
            const int nl = (b * DX_WAVES + wave) * RPW + sub;  // >= CH only when H is small
            float sg, mg, su, mu;
            group_params<FMT>(gs[b], sg, mg);
            group_params<FMT>(us[b], su, mu);
            const float cg = mg - OFFSET_BF16 * sg, cu = mu - OFFSET_BF16 * su;
            uint32_t gw[16], uw[16];
            unpack32(gv[b], gw);
            unpack32(uv[b], uw);
#pragma unroll
            for (int u = 0; u < DECODE_TT; ++u) {
                if (u < nt) {
                    const float pg = seg_sum_dpp<LPR>(fmaf(sg, dot16(gw, xp[u], 0.f), cg * xs[u]));
                    const float pu = seg_sum_dpp<LPR>(fmaf(su, dot16(uw, xp[u], 0.f), cu * xs[u]));
                    if (c == LPR - 1 && nl < CH) s_h[u][nl] = silu(pg) * pu;
                }
            }
        }
    }
    __syncthreads();

    // ---- 2. down rows d, inputs [n0, n0 + CH): DL lanes per row
    {
        uint32_t hh[DECODE_TT][16], hl[DECODE_TT][16];
        float hs[DECODE_TT];
#pragma unroll
        for (int u = 0; u < DECODE_TT; ++u) {
            hs[u] = 0.f;
            if (u < nt) {
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
        }
#pragma unroll
        for (int b = 0; b < DN; ++b) {
            const int d = (b * DX_WAVES + wave) * DRW + rr;
            float sd, md;
            group_params<FMT>(ds[b], sd, md);
            const float cd = md - OFFSET_BF16 * sd;
            uint32_t dw[16];
            unpack32(dv[b], dw);
#pragma unroll
            for (int u = 0; u < DECODE_TT; ++u) {
                if (u < nt) {
                    float a = dot16(dw, hh[u], 0.f);
                    a = dot16(dw, hl[u], a);
                    float part = fmaf(sd, a, cd * hs[u]);
                    if (DL == 2) part = seg_sum_dpp<2>(part);
                    if (half == 0 && d < H) unsafeAtomicAdd(y + (size_t)s_tok[u] * H + d, s_gate[u] * part);
                }
            }
        }
    }
}

// Routing of a few tokens in one launch.  Workgroup e (16 waves) computes
// the router logits of expert e, wave w taking tokens w, w + 16, ...  The
// logits travel to the workgroup that arrives last through agent-scope
// relaxed atomic stores and loads (coherent across the XCDs' L2 caches) and a
// counter in the workspace (zero between calls): each workgroup waits for its
// stores to complete, then counts itself in.  This avoids whole-L2 write-back
// and invalidate fences, which cost far more than the routing itself when
// hundreds of workgroups issue them.  The last workgroup stages the logits in
// LDS, takes the top-k of every token and groups the pairs by expert.
// Without router weights one workgroup does top-k and grouping on the given
// logits.  With yres the layer input is the residual step bf16(x + yres),
// computed on the fly and written to xout.  The workgroups also clear y for
// the expert kernel's atomics.
template <int NPL>
__global__ __launch_bounds__(1024) void decode_route_group_kernel(
    const uint16_t *__restrict__ x, const float *__restrict__ yres, uint16_t *__restrict__ xout,
    const uint16_t *__restrict__ wr, const float *__restrict__ bias, int T, int H, int E, int k,
    uint16_t *__restrict__ logits, int32_t *__restrict__ idx, float *__restrict__ gate, GroupOut g,
    float *__restrict__ yclear, unsigned int *__restrict__ counter, unsigned int *__restrict__ handoff) {
    __shared__ int s_last;
    __shared__ uint16_t s_lg[ROUTE_LDS_LOGITS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nb = gridDim.x;
    const int64_t n = (int64_t)T * H;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + tid; i < n; i += (int64_t)nb * blockDim.x) {
        yclear[i] = 0.f;
        if (yres) xout[i] = f32_to_bf16_rne(bf16_to_f32(x[i]) + yres[i]);
    }
    const uint16_t *lsrc = logits;
    if (wr) {
        const int e = blockIdx.x;
        const double b = bias ? (double)bias[e] : 0.0;
        for (int t = wave; t < T; t += 16) {
            const double acc = router_dot_wave(x + (size_t)t * H, yres ? yres + (size_t)t * H : nullptr,
                                               wr + (size_t)e * H, H);
            if (lane == 63) {
                const uint16_t v = f32_to_bf16_rne((float)(acc + b));
                logits[(size_t)t * E + e] = v;
                __hip_atomic_store(handoff + (size_t)t * E + e, (unsigned int)v, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have completed
        __syncthreads();
        if (tid == 0)
            s_last = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                     (unsigned)(nb - 1);
        __syncthreads();
        if (!s_last) return;
        for (int i = tid; i < T * E; i += blockDim.x)
            s_lg[i] = (uint16_t)__hip_atomic_load(handoff + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        lsrc = s_lg;
    }
    for (int t = wave; t < T; t += 16) topk_token_wave<NPL>(lsrc + (size_t)t * E, E, k, idx + t * k, gate + t * k);
    __syncthreads();
    group_block_single(idx, T * k, E, g);
    if (tid == 0 && wr) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int FMT>
static hipError_t launch_experts_fmt(const uint16_t *x, const float *gate, int64_t T, int k, const LayerPtrs &L,
                                     const GroupOut &g, float *y, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    const int H = L.H, I = L.I;
    const int P = (int)(T * k);
    const int64_t mt = max_tiles(P, L.E, DECODE_TT);
    const int ntg = (int)((mt + 7) / 8 * 8);
    // few tiles: 32-row chunks so that more workgroups stream the weights
    const bool small = mt <= 48;
    const int ch = small ? 32 : 64;
    dim3 grid((unsigned)(ntg * (I / ch)));
    switch ((H / 32) * (small ? 1 : -1)) {
#define CASE(LP) \
    case LP: launch_k(decode_experts_kernel<LP, FMT, 32>, grid, dim3(DX_WAVES * 64), s, e0, e1, x, H, I, k, P, L, g.tiles, g.ntiles, g.perm, gate, ntg, y); break; \
    case -LP: launch_k(decode_experts_kernel<LP, FMT, 64>, grid, dim3(DX_WAVES * 64), s, e0, e1, x, H, I, k, P, L, g.tiles, g.ntiles, g.perm, gate, ntg, y); break;
        CASE(2) CASE(4) CASE(8) CASE(16) CASE(32) CASE(64)
#undef CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_decode_experts(const uint16_t *x, const float *gate, int64_t T, int k, const LayerPtrs &L,
                                 const GroupOut &g, float *y, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    return L.fmt == 0 ? launch_experts_fmt<0>(x, gate, T, k, L, g, y, s, e0, e1)
                      : launch_experts_fmt<1>(x, gate, T, k, L, g, y, s, e0, e1);
}

hipError_t launch_decode_route_group(const uint16_t *x, const float *yres, uint16_t *xout, const uint16_t *wr,
                                     const float *bias, int T, int H, int E, int k, uint16_t *logits, int32_t *idx,
                                     float *gate, const GroupOut &g, float *yclear, unsigned int *counter,
                                     unsigned int *handoff, hipStream_t s) {
    if (wr && T * E > ROUTE_LDS_LOGITS) return hipErrorInvalidValue;
    const int nb = wr ? E : 1;
    const int npl = (E + 63) / 64;
#define LAUNCH(N) \
    hipLaunchKernelGGL(decode_route_group_kernel<N>, dim3(nb), dim3(1024), 0, s, x, yres, xout, wr, bias, T, H, E, k, logits, idx, gate, g, yclear, counter, handoff)
    if (npl <= 4) LAUNCH(4);
    else if (npl <= 8) LAUNCH(8);
    else LAUNCH(16);
#undef LAUNCH
    return hipGetLastError();
}

}  // namespace moeq4
