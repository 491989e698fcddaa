// Decode path: fused-dequant GEMVs over the active experts' packed nibbles.
//
// Decode is bound by the bytes of expert weights read from HBM (drama-rs
// page, "Experts: where they run": decode reads about 1 GB of FP8 experts per
// frame and is memory-bandwidth-bound).  Each code is read once, coalesced (a
// lane takes 16 bytes = 32 codes, consecutive lanes consecutive bytes), and
// applied to every token routed to its expert.
//
// Two kernels per layer do the expert work:
//   1. gate/up GEMV + SwiGLU: every active expert's gate and up rows, applied
//      to the tokens routed to it, h in fp32 (workspace);
//   2. down GEMV over full rows of h, multiplied by each token's gate and
//      added into y with float atomics (y is cleared by the routing kernel).
// Both launch as many workgroups as the chip holds at once and cut the work
// on the device, from the actual tile count, into that many items (tile,
// row chunk), so a layer's expert work runs in one round.  Items are spread
// XCD-locally (workgroup b runs on XCD b mod 8 and takes a contiguous range
// of items), so the chunks of one tile and the tiles of one expert share an
// L2.  Each item issues its first weight loads before it fetches token
// indices and activations.
//
// Group arithmetic.  For a group of codes q_k with scale s and min m,
//   sum_k a_k (s q_k + m) = s * sum_k a_k (OFF + q_k) + (m - OFF s) * sum_k a_k
// where OFF + q_k is the exact 16-bit float value a nibble unpacks to;
// symmetric groups use m = -8 s.  sum a (OFF + q) runs on the packed
// dot-product instructions with fp32 accumulation: bf16 (OFF = 128) against
// x in the gate/up GEMV, f16 (OFF = 1024) against h in the down GEMV, each
// row of h scaled by a power of two and rounded to f16 (decode_dev.h).
#include "decode_dev.h"
#include "fp8_dev.h"
#include "nvfp4_dev.h"
#include "group_dev.h"
#include "shared_dev.h"
#include "route_dev.h"

namespace moeq4 {


// Tile fields made safe to index with (a workspace that was never filled
// gives garbage numbers, not out-of-bounds accesses).
__device__ __forceinline__ Tile sane_tile(Tile t, int E, int P) {
    t.expert = clamp_expert(t.expert, E);
    t.rows = t.rows < 0 ? 0 : (t.rows > DECODE_TT ? DECODE_TT : t.rows);
    t.rows = t.rows > P ? P : t.rows;
    t.row0 = t.row0 < 0 ? 0 : (t.row0 > P - t.rows ? P - t.rows : t.row0);
#pragma unroll
    for (int u = 0; u < DECODE_TT; ++u) t.pair[u] = t.pair[u] < 0 ? 0 : (t.pair[u] >= P ? P - 1 : t.pair[u]);
    return t;
}

// 16 bf16 pairs (32 codes in PERM8 order) of a dword quad.
// 32 codes as bf16 pairs 128 + q in PERM8 order (kb = opaque MAGIC_BF16).
__device__ __forceinline__ void unpack32(const uint4 w, uint32_t out[16], uint32_t kb) {
    const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int p = 0; p < 4; ++p) out[4 * q + p] = insert_codes<0x000f000fu>(d[q] >> (4 * p), kb);
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

// Routing inside an expert workgroup (few tokens): top-k per token and the
// one-block grouping from the logits lg (written by the previous launch),
// into LDS.  Every workgroup does it; workgroup 0 also publishes the
// indices, gates and grouping arrays (idx_out, gate_out, gout) for the
// caller.  Returns the tile count; *tiles_lds and *gates_lds point at the
// LDS copies.
__device__ __forceinline__ int route_in_block(const uint16_t *__restrict__ lg, int T, int E, int k, int P,
                                              int32_t *__restrict__ idx_out, float *__restrict__ gate_out,
                                              const GroupOut &gout, const Tile **tiles_lds,
                                              const float **gates_lds) {
    __shared__ int32_t r_idx[DEC_ROUTE_PMAX];
    __shared__ float r_gate[DEC_ROUTE_PMAX];
    __shared__ int32_t r_cnt[DEC_ROUTE_EMAX], r_off[DEC_ROUTE_EMAX + 1], r_perm[DEC_ROUTE_PMAX],
        r_inv[DEC_ROUTE_PMAX];
    __shared__ Tile r_tiles[DEC_ROUTE_TMAX];
    __shared__ int32_t r_nt;
    __shared__ __attribute__((aligned(16))) uint16_t r_lg[DEC_ROUTE_LOGITS];
    const int tid = threadIdx.x, wave = tid >> 6;
    const bool b0 = blockIdx.x == 0;
    // all logits in one coalesced pass (the top-k rounds then read LDS only)
    {
        const int n = T * E;
        for (int i = tid * 8; i < n; i += blockDim.x * 8) {
            if (i + 8 <= n && ((reinterpret_cast<uintptr_t>(lg) & 15) == 0))
                *reinterpret_cast<uint4 *>(&r_lg[i]) = *reinterpret_cast<const uint4 *>(lg + i);
            else
                for (int q = i; q < n && q < i + 8; ++q) r_lg[q] = lg[q];
        }
    }
    __syncthreads();
    for (int t = wave; t < T; t += blockDim.x / 64)
        topk_token_wave<DEC_ROUTE_NPL>(r_lg + (size_t)t * E, E, k, r_idx + t * k, r_gate + t * k);
    __syncthreads();
    GroupOut gl;
    gl.cnt = r_cnt;
    gl.off = r_off;
    gl.perm = r_perm;
    gl.inv = r_inv;
    gl.tiles = r_tiles;
    gl.ntiles = &r_nt;
    gl.rows_per_tile = DECODE_TT;
    gl.chunk_cnt = gl.chunk_base = nullptr;
    gl.order = nullptr;
    group_block_single(r_idx, P, E, gl);
    __syncthreads();
    const int nt_all = r_nt;
    if (b0) {
        for (int i = tid; i < P; i += blockDim.x) {
            idx_out[i] = r_idx[i];
            gate_out[i] = r_gate[i];
            gout.perm[i] = r_perm[i];
            gout.inv[i] = r_inv[i];
        }
        for (int i = tid; i < E; i += blockDim.x) gout.cnt[i] = r_cnt[i];
        for (int i = tid; i <= E; i += blockDim.x) gout.off[i] = r_off[i];
        for (int i = tid; i < nt_all; i += blockDim.x) gout.tiles[i] = r_tiles[i];
        if (tid == 0) *gout.ntiles = nt_all;
    }
    *tiles_lds = r_tiles;
    *gates_lds = r_gate;
    return nt_all;
}

constexpr int DEC_GU_STAGES = 2;  // register stages of the gate/up GEMV

// gate/up GEMV + SwiGLU for one item (tile: one expert, up to DECODE_TT
// tokens; rows ir of I) into h.  Lanes run along the input dimension: LPR =
// H / 64 lanes per row, each lane 32 bytes = 64 codes, so a wave-load covers
// RPW = 64 / LPR rows of gate and of up (2 rows of 1 KB each when H = 2048).
// Lane c takes bytes [16c, 16c + 16) of the row's first half and of its
// second half, so each 16-byte load instruction reads whole cache lines
// (32 B per lane in one piece left every line half read by each of two
// instructions: frame 2.29 against 2.31 ms, decode step 17.75 against
// 18.1 us); each half lies in one scale group.  The next wave-load is in
// flight while the current one is reduced.  h is written in fp32, natural
// order.
// SHORT: items of a single wave-load are common (few tokens), and take a
// straight path instead of issuing unused stages.
template <int LPR, int FMT, bool SHORT>
__device__ __forceinline__ void gateup_item(const uint16_t *__restrict__ x, int H, int I, int k, const LayerPtrs &L,
                                            const Tile &tile, const ItemRows<DEC_WAVES * WAVE / LPR> &ir,
                                            float *__restrict__ h, float (*s_out)[DEC_RB_MAX]) {
    constexpr int RPW = WAVE / LPR;  // rows per wave-load
    constexpr int G = FMT == 0 ? 64 : 128;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane % LPR, sub = lane / LPR;
    const size_t row_bytes = (size_t)H / 2;
    const size_t smr = (size_t)(H / G) * (FMT == 0 ? 2 : 1);
    // lane c: codes [32c, 32c + 32) and [H/2 + 32c, H/2 + 32c + 32)
    const int gi0 = (32 * c) / G, gi1 = (H / 2 + 32 * c) / G;
    const uint32_t kb = opaque_magic(MAGIC_BF16);
    struct Stage {
        uint4 g[2], u[2];
        uint32_t gs[2], us[2];
    };
    const int e = tile.expert, nt = tile.rows;
    const int steps = ir.steps;         // wave-loads per wave
    const int lrow = wave * RPW + sub;  // the lane's row within a step
    auto row_of = [&](int s) { return s * (DEC_WAVES * RPW) + lrow; };
    auto issue = [&](Stage &st, int s) {
        const size_t row = (size_t)e * I + (ir.valid_step(s, lrow) ? ir.grow_step(s, lrow) : ir.grow(0));
        const uint4 *gp = reinterpret_cast<const uint4 *>(L.gq + row * row_bytes + 16 * c);
        const uint4 *up = reinterpret_cast<const uint4 *>(L.uq + row * row_bytes + 16 * c);
        st.g[0] = gp[0];
        st.g[1] = gp[LPR];
        st.u[0] = up[0];
        st.u[1] = up[LPR];
        st.gs[0] = load_group_word<FMT>(L.gsm + row * smr, gi0);
        st.gs[1] = load_group_word<FMT>(L.gsm + row * smr, gi1);
        st.us[0] = load_group_word<FMT>(L.usm + row * smr, gi0);
        st.us[1] = load_group_word<FMT>(L.usm + row * smr, gi1);
    };
    // Activations: fetched before the first weight stages (they depend on
    // the tile only), reordered after them, so that waiting for them leaves
    // the stages in flight.
    uint32_t xp[DECODE_TT][32];
    float xs[DECODE_TT][2];
    auto fetch_x = [&]() {
#pragma unroll
        for (int u = 0; u < DECODE_TT; ++u) {
            if (u < nt) {
                const uint16_t *xrow = x + (size_t)(tile.pair[u] / k) * H;
                fetch_x_chunk(xrow, c, xp[u]);
                fetch_x_chunk(xrow, LPR + c, xp[u] + 16);
            }
        }
    };
    auto prep_x = [&]() {
#pragma unroll
        for (int u = 0; u < DECODE_TT; ++u) {
            xs[u][0] = xs[u][1] = 0.f;
            if (u < nt) {
                xs[u][0] = perm_x_chunk(xp[u]);
                xs[u][1] = perm_x_chunk(xp[u] + 16);
            }
        }
    };
    Stage st[DEC_GU_STAGES];
    auto consume = [&](const Stage &st, int s) {
        const int nl = row_of(s);
        float sg[2], mg[2], su[2], mu[2], cg[2], cu[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            group_params<FMT>(st.gs[hh], sg[hh], mg[hh]);
            group_params<FMT>(st.us[hh], su[hh], mu[hh]);
            cg[hh] = mg[hh] - OFFSET_BF16 * sg[hh];
            cu[hh] = mu[hh] - OFFSET_BF16 * su[hh];
        }
        // one code quad unpacked at a time, applied to every token of the tile
        float dg[DECODE_TT][2], du[DECODE_TT][2];
#pragma unroll
        for (int u = 0; u < DECODE_TT; ++u) dg[u][0] = dg[u][1] = du[u][0] = du[u][1] = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t wq[16];
            unpack32(q == 0 ? st.g[0] : q == 1 ? st.g[1] : q == 2 ? st.u[0] : st.u[1], wq, kb);
#pragma unroll
            for (int u = 0; u < DECODE_TT; ++u) {
                if (u < nt) {
                    if (q < 2) dg[u][q & 1] = dot16(wq, xp[u] + 16 * (q & 1), 0.f);
                    else du[u][q & 1] = dot16(wq, xp[u] + 16 * (q & 1), 0.f);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < DECODE_TT; ++u) {
            if (u < nt) {
                const float pg = seg_sum_dpp<LPR>(fmaf(sg[0], dg[u][0], cg[0] * xs[u][0]) +
                                                  fmaf(sg[1], dg[u][1], cg[1] * xs[u][1]));
                const float pu = seg_sum_dpp<LPR>(fmaf(su[0], du[u][0], cu[0] * xs[u][0]) +
                                                  fmaf(su[1], du[u][1], cu[1] * xs[u][1]));
                if (c == LPR - 1 && ir.valid_step(s, lrow)) s_out[u][nl] = silu(pg) * pu;
            }
        }
    };
    // DEC_GU_STAGES register stages, the next ones in flight while the
    // current one is reduced.  The first rows depend only on the tile, so
    // they are issued before the tokens are known.  The loop issues every
    // stage (rows past the item re-read its first row) and outputs go to LDS,
    // so it holds only loads and the compiler's memory-counter waits stay
    // exact.
    if (SHORT && steps == 1) {
        fetch_x();
        issue(st[0], 0);
        prep_x();
        consume(st[0], 0);
    } else {
        fetch_x();
#pragma unroll
        for (int u = 0; u < DEC_GU_STAGES; ++u) issue(st[u], u);
        prep_x();
        for (int s = 0; s < steps; s += DEC_GU_STAGES) {
#pragma unroll
            for (int u = 0; u < DEC_GU_STAGES; ++u) {
                if (u == 0 || s + u < steps) consume(st[u], s + u);
                issue(st[u], s + u + DEC_GU_STAGES);
            }
        }
    }
    __syncthreads();
    {
        for (int i = tid; i < nt * ir.nloc; i += blockDim.x) {
            const int u = i / ir.nloc, nl = i % ir.nloc;
            if (!ir.valid(nl)) continue;
            h[(size_t)(tile.row0 + u) * I + ir.grow(nl)] = s_out[u][nl];
        }
    }
    __syncthreads();
}

// down GEMV for one item (tile; output rows ir of H) over the full inner
// dimension (LPR = I / 32 lanes per row, a contiguous 256-byte row when I =
// 512), multiplied by each token's gate and added into y (float atomics;
// each output receives one add per routed (token, slot)).
template <int LPR, int FMT>
__device__ __forceinline__ void down_item(int H, int I, int k, const LayerPtrs &L, const Tile &tile,
                                          const ItemRows<DEC_WAVES * WAVE / LPR> &ir,
                                          const float *__restrict__ topk_gate, const float *__restrict__ h,
                                          float *__restrict__ y, float *__restrict__ zrows,
                                          float (*s_out)[DEC_RB_MAX]) {
    constexpr int RPW = WAVE / LPR;
    constexpr int G = FMT == 0 ? 64 : 128;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane % LPR, sub = lane / LPR;
    const size_t row_bytes = (size_t)I / 2;
    const size_t smr = (size_t)(I / G) * (FMT == 0 ? 2 : 1);
    const int gi = (32 * c) / G;
    const uint32_t kf = opaque_magic(MAGIC_F16);
    struct Stage {
        uint4 v[DEC_NB];
        uint32_t s[DEC_NB];
    };
    const int e = tile.expert, nt = tile.rows;
    const int steps = ir.steps;
    const int lrow = wave * RPW + sub;  // the lane's row within a step
    auto row_of = [&](int s) { return s * (DEC_WAVES * RPW) + lrow; };
    auto issue = [&](Stage &st, int s0) {
#pragma unroll
        for (int b = 0; b < DEC_NB; ++b) {
            const int sb_ = s0 + b;
            const size_t row = (size_t)e * H + (ir.valid_step(sb_, lrow) ? ir.grow_step(sb_, lrow) : ir.grow(0));
            st.v[b] = *reinterpret_cast<const uint4 *>(L.dq + row * row_bytes + 16 * c);
            st.s[b] = load_group_word<FMT>(L.dsm + row * smr, gi);
        }
    };
    Stage sa, sb;
    int tok[DECODE_TT];
    float gt[DECODE_TT];
    uint32_t hp[DECODE_TT][16];
    HFetch hf;
    __shared__ __attribute__((aligned(16))) uint16_t s_h[DECODE_TT * DEC_HMAX];
    // The lane's h elements in f16 (the row scaled by a power of two), odd
    // ones divided by 16 (they meet codes 1024 + 16 q); ha = sum of the
    // offsets those products carry (1024 per even element, 64 per odd one,
    // times h), hb = sum of h.
    float ha[DECODE_TT], hb[DECODE_TT];
    // h and the gates: fetched before the first weight stages (they depend on
    // the tile only), staged through LDS in f16 and summed after them.
    auto fetch_h = [&]() {
#pragma unroll
        for (int u = 0; u < DECODE_TT; ++u) {
            tok[u] = 0;
            gt[u] = 0.f;
            if (u < nt) {
                const int p = tile.pair[u];
                tok[u] = p / k;
                gt[u] = topk_gate[p];
            }
        }
        h_fetch(h, tile.row0, nt, I, hf);
    };
    auto sum_h = [&]() {
        float inv[DECODE_TT];
        h_to_lds<true>(hf, nt, I, s_h, inv);
#pragma unroll
        for (int u = 0; u < DECODE_TT; ++u) {
            ha[u] = hb[u] = 0.f;
            if (u < nt) {
                gt[u] *= inv[u];
                h_from_lds(s_h + u * DEC_HMAX, c, hp[u]);
                float se = 0.f, so = 0.f;  // sums of the even elements and of the odd ones (/16)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    se = dot2_f16(hp[u][4 * q + 0], ONES_F16X2, dot2_f16(hp[u][4 * q + 2], ONES_F16X2, se));
                    so = dot2_f16(hp[u][4 * q + 1], ONES_F16X2, dot2_f16(hp[u][4 * q + 3], ONES_F16X2, so));
                }
                ha[u] = OFFSET_F16 * (se + so);
                hb[u] = fmaf(16.f, so, se);
            }
        }
    };
    auto consume = [&](const Stage &st, int s0) {
#pragma unroll
        for (int b = 0; b < DEC_NB; ++b) {
            const int dl = row_of(s0 + b);
            float sd, md;
            group_params<FMT>(st.s[b], sd, md);
            // even codes enter as 1024 + q, odd codes in place as
            // 1024 + 16 q against h / 16: the dot is sum h q + ha
            const uint32_t d4[4] = {st.v[b].x, st.v[b].y, st.v[b].z, st.v[b].w};
            uint32_t dw[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t w8 = d4[q] >> 8;
                dw[4 * q + 0] = insert_codes<0x000f000fu>(d4[q], kf);  // codes 0, 4
                dw[4 * q + 1] = insert_codes<0x00f000f0u>(d4[q], kf);  // codes 1, 5 (x16)
                dw[4 * q + 2] = insert_codes<0x000f000fu>(w8, kf);     // codes 2, 6
                dw[4 * q + 3] = insert_codes<0x00f000f0u>(w8, kf);     // codes 3, 7 (x16)
            }
#pragma unroll
            for (int u = 0; u < DECODE_TT; ++u) {
                if (u < nt) {
                    float a = 0.f;
#pragma unroll
                    for (int i = 0; i < 16; ++i) a = dot2_f16(dw[i], hp[u][i], a);
                    const float o = seg_sum_dpp<LPR>(fmaf(sd, a - ha[u], md * hb[u]));
                    if (c == LPR - 1 && ir.valid_step(s0 + b, lrow)) s_out[u][dl] = gt[u] * o;
                }
            }
        }
    };
    // stages of DEC_NB row loads, pipelined as in the gate/up GEMV
    const int nst = (steps + DEC_NB - 1) / DEC_NB;
    if (nst == 1) {
        fetch_h();
        issue(sa, 0);
        sum_h();
        consume(sa, 0);
    } else {
        fetch_h();
        issue(sa, 0);
        issue(sb, DEC_NB);
        sum_h();
        for (int q = 0; q < nst; q += 2) {
            consume(sa, q * DEC_NB);
            issue(sa, (q + 2) * DEC_NB);
            if (q + 1 < nst) consume(sb, (q + 1) * DEC_NB);
            issue(sb, (q + 3) * DEC_NB);
        }
    }
    __syncthreads();
    // one float atomic (or one store) per output and routed (token, slot)
    emit_down_rows(y, zrows, tile, tok, nt, H, ir, s_out);
    __syncthreads();
}

// gate/up GEMV + SwiGLU over all items (tiles x row chunks of I), h to the
// workspace for the down launch.  With ROUTE, every workgroup first routes
// the tokens itself (route_in_block), which replaces a serial
// last-workgroup step of the routing launch.  With SHARED the layer's shared
// expert runs in the same launch: its (token tile, row chunk) items form a
// second list, dealt over the grid like the first, its SwiGLU output going
// to hs.
template <int LPR, int FMT, bool ROUTE, bool SHARED>
__global__ __launch_bounds__(DEC_WAVES * 64) void decode_gateup_kernel(
    const uint16_t *__restrict__ x, int H, int I, int k, int P, LayerPtrs L, const Tile *__restrict__ tiles,
    const int32_t *__restrict__ ntiles, int max_nt, float *__restrict__ h, const uint16_t *__restrict__ lg,
    int T, int32_t *__restrict__ idx_out, float *__restrict__ gate_out, GroupOut gout, SharedPtrs S,
    float *__restrict__ hs) {
    // lanes per gate/up row: H / 64 for int4 (64 codes a lane), H / 32 for
    // fp8 (32 codes a lane)
    constexpr int LPG = FMT == 2 ? 2 * LPR : LPR;
    constexpr int BR = DEC_WAVES * (WAVE / LPG);
    __shared__ float s_out[DECODE_TT][DEC_RB_MAX];
    if constexpr (SHARED && LPR >= 2) {  // shared expert: H / 32 lanes per row
        constexpr int LPS = 2 * LPR, BRS = DEC_WAVES * (WAVE / LPS);
        const int ntt = (T + DECODE_TT - 1) / DECODE_TT;
        const Items is = decode_items(ntt, S.I, S.I / BRS);
        for (int w = is.first; w < is.end; w += is.stride) {
            const int j = w % ntt, chunk = w / ntt;  // chunk-major: a chunk's token tiles share an XCD
            const int tok0 = j * DECODE_TT, nt = T - tok0 < DECODE_TT ? T - tok0 : DECODE_TT;
            const ItemRows<BRS> ir = item_rows<BRS>(chunk, is, S.I);
            if (ir.steps <= 0) continue;
            shared_gateup_item<LPS>(x, S, tok0, nt, ir, hs, s_out);
        }
    }
    int nt_all;
    if constexpr (ROUTE) {
        const Tile *tiles_lds;
        const float *gates_lds;
        nt_all = route_in_block(lg, T, L.E, k, P, idx_out, gate_out, gout, &tiles_lds, &gates_lds);
        tiles = tiles_lds;
    } else {
        nt_all = *ntiles;
    }
    nt_all = nt_all < 0 ? 0 : (nt_all > max_nt ? max_nt : nt_all);
    const Items it = decode_items(nt_all, I, I / BR);
    for (int w = it.first; w < it.end; w += it.stride) {
        const int j = w / it.nch, chunk = w % it.nch;
        const Tile tile = sane_tile(tiles[j], L.E, P);
        const ItemRows<BR> ir = item_rows<BR>(chunk, it, I);
        if (ir.steps <= 0) continue;
        if constexpr (FMT == 2) fp8_gateup_item<LPG, ROUTE>(x, H, I, k, L, tile, ir, h, s_out);
        else if constexpr (FMT == 3) nvfp4_gateup_item<LPR, ROUTE>(x, H, I, k, L, tile, ir, h, s_out);
        else gateup_item<LPR, FMT, ROUTE>(x, H, I, k, L, tile, ir, h, s_out);
    }
}

// down GEMV over all items (tiles x row chunks of H), h from the gate/up
// launch (fp32; each row scaled and rounded to f16).  With SHARED the shared expert's down
// items (its inner size equal to the routed experts') follow, added into y
// with float atomics as well.
template <int LPR, int FMT, bool SHARED>
__global__ __launch_bounds__(DEC_WAVES * 64) void decode_down_kernel(
    int H, int I, int k, int P, LayerPtrs L, const Tile *__restrict__ tiles, const int32_t *__restrict__ ntiles,
    int max_nt, const float *__restrict__ topk_gate, const float *__restrict__ h, float *__restrict__ y, int T,
    SharedPtrs S, const float *__restrict__ hs, float *__restrict__ zrows) {
    constexpr int BR = DEC_WAVES * (WAVE / LPR);
    int nt_all = *ntiles;
    nt_all = nt_all < 0 ? 0 : (nt_all > max_nt ? max_nt : nt_all);
    const Items it = decode_items(nt_all, H, H / BR);
    __shared__ float s_out[DECODE_TT][DEC_RB_MAX];
    for (int w = it.first; w < it.end; w += it.stride) {
        const int j = w / it.nch, chunk = w % it.nch;
        const Tile tile = sane_tile(tiles[j], L.E, P);
        const ItemRows<BR> ir = item_rows<BR>(chunk, it, H);
        if (ir.steps <= 0) continue;
        if constexpr (FMT == 2) fp8_down_item<LPR>(H, I, k, L, tile, ir, topk_gate, h, y, zrows, s_out);
        else if constexpr (FMT == 3) nvfp4_down_item<LPR>(H, I, k, L, tile, ir, topk_gate, h, y, zrows, s_out);
        else down_item<LPR, FMT>(H, I, k, L, tile, ir, topk_gate, h, y, zrows, s_out);
    }
    if constexpr (SHARED && LPR >= 4) {
        const int ntt = (T + DECODE_TT - 1) / DECODE_TT;
        const Items is = decode_items(ntt, H, H / BR);
        for (int w = is.first; w < is.end; w += is.stride) {
            const int j = w % ntt, chunk = w / ntt;  // chunk-major: a chunk's token tiles share an XCD
            const int tok0 = j * DECODE_TT, nt = T - tok0 < DECODE_TT ? T - tok0 : DECODE_TT;
            const ItemRows<BR> ir = item_rows<BR>(chunk, is, H);
            if (ir.steps <= 0) continue;
            shared_down_item<LPR, true>(S, tok0, nt, ir, hs, y, true, s_out);
        }
    }
}

// Router logits only (the expert launch takes top-k and grouping itself):
// workgroup e computes expert e's logit for every token, wave w taking
// tokens w, w + 4, ...; a lane reads its 8-element slices of the router row,
// of x and of yres straight from memory (no staging), forms the residual
// input bf16(x + yres) and sums x w in double (exact products).  The grid
// also clears y and writes the residual input to xout.
__global__ __launch_bounds__(256) void decode_router_kernel(
    const uint16_t *__restrict__ x, const float *__restrict__ yres, uint16_t *__restrict__ xout,
    const uint16_t *__restrict__ wr, const float *__restrict__ bias, int T, int H, int E,
    uint16_t *__restrict__ logits, float *__restrict__ yclear) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nb = gridDim.x;
    const int64_t n = (int64_t)T * H;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + tid; i < n; i += (int64_t)nb * blockDim.x) {
        yclear[i] = 0.f;
        if (yres) xout[i] = f32_to_bf16_rne(bf16_to_f32(x[i]) + yres[i]);
    }
    if (!wr) return;
    const int e = blockIdx.x;  // grid = E
    uint4 wv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int hh = (q * WAVE + lane) * 8;
        wv[q] = make_uint4(0, 0, 0, 0);
        if (hh < H) wv[q] = *reinterpret_cast<const uint4 *>(wr + (size_t)e * H + hh);
    }
    const double b = bias ? (double)bias[e] : 0.0;
    for (int t = wave; t < T; t += 4) {
        uint4 xv[4];
        float4 ya[4], yb[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int hh = (q * WAVE + lane) * 8;
            xv[q] = make_uint4(0, 0, 0, 0);
            if (hh < H) {
                const size_t gi = (size_t)t * H + hh;
                xv[q] = *reinterpret_cast<const uint4 *>(x + gi);
                if (yres) {
                    ya[q] = *reinterpret_cast<const float4 *>(yres + gi);
                    yb[q] = *reinterpret_cast<const float4 *>(yres + gi + 4);
                }
            }
        }
        double acc = 0.0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if ((q * WAVE + lane) * 8 < H) {
                uint32_t xs4[4] = {xv[q].x, xv[q].y, xv[q].z, xv[q].w};
                if (yres) {
                    const float yv[8] = {ya[q].x, ya[q].y, ya[q].z, ya[q].w, yb[q].x, yb[q].y, yb[q].z, yb[q].w};
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const uint32_t lo = f32_to_bf16_rne(bf16_to_f32(xs4[jj] & 0xffffu) + yv[2 * jj]);
                        const uint32_t hi = f32_to_bf16_rne(bf16_to_f32(xs4[jj] >> 16) + yv[2 * jj + 1]);
                        xs4[jj] = lo | (hi << 16);
                    }
                }
                const uint32_t ws4[4] = {wv[q].x, wv[q].y, wv[q].z, wv[q].w};
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    acc = fma((double)bf16_to_f32(xs4[jj] & 0xffffu), (double)bf16_to_f32(ws4[jj] & 0xffffu), acc);
                    acc = fma((double)bf16_to_f32(xs4[jj] >> 16), (double)bf16_to_f32(ws4[jj] >> 16), acc);
                }
            }
        }
        acc = wave_sum_f64_dpp(acc);
        if (lane == 63) logits[(size_t)t * E + e] = f32_to_bf16_rne((float)(acc + b));
    }
}

// Routing of a few tokens in one launch.  A workgroup (16 waves) computes
// the router logits of ROUTE_EG experts for ROUTE_TG tokens, one (expert,
// token) dot per wave; the tokens' input rows are staged in LDS once per
// workgroup (so every input row is formed E / ROUTE_EG times, not E).  The
// logits travel to the workgroup that arrives last through agent-scope
// relaxed atomic stores and loads (coherent across the XCDs' L2 caches) and
// a counter in the workspace (zero between calls): each workgroup waits for
// its stores to complete, then counts itself in.  Why this is ordered
// without release / acquire: (1) every shared value is itself an
// agent-scope atomic, so all of them live at the device's coherence point
// and no cache needs writing back or invalidating; (2) s_waitcnt vmcnt(0)
// returns only once each store is acknowledged there, and the workgroup's
// barrier puts every wave's wait before thread 0's count-in; (3) the last
// workgroup issues its loads only after the count-in's returned value,
// through a barrier, so no load can be served before that value existed.
// A fence would add what (1) makes unnecessary: whole-L2 write-back and
// invalidate, which cost far more than the routing itself when hundreds of
// workgroups issue them.  A launch that never completes would leave the
// counter non-zero (the next call's output is then wrong, not hung);
// moe_q4_workspace_init clears it.  The last
// workgroup stages the logits in LDS, takes the top-k of every token and
// groups the pairs by expert (from LDS copies of the indices).  Without
// router weights one workgroup does top-k and grouping on the given logits.
// With yres the layer input is the residual step bf16(x + yres), computed on
// the fly and written to xout.  The workgroups also clear y for the expert
// kernels' atomics.
template <int NPL>
__global__ __launch_bounds__(1024) void decode_route_group_kernel(
    const uint16_t *__restrict__ x, const float *__restrict__ yres, uint16_t *__restrict__ xout,
    const uint16_t *__restrict__ wr, const float *__restrict__ bias, int T, int H, int E, int k,
    uint16_t *__restrict__ logits, int32_t *__restrict__ idx, float *__restrict__ gate, GroupOut g,
    float *__restrict__ yclear, unsigned int *__restrict__ counter, unsigned int *__restrict__ handoff,
    bool tail) {
    __shared__ int s_last;
    __shared__ uint16_t s_lg[ROUTE_LDS_LOGITS];
    __shared__ int32_t s_idx[GROUP_SINGLE_MAX];
    __shared__ __attribute__((aligned(16))) uint16_t s_x[ROUTE_TG * 2048];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nb = gridDim.x;
    const int64_t n = (int64_t)T * H;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + tid; i < n; i += (int64_t)nb * blockDim.x) {
        yclear[i] = 0.f;
        if (yres) xout[i] = f32_to_bf16_rne(bf16_to_f32(x[i]) + yres[i]);
    }
    if (wr) {
        // workgroup = (group of ROUTE_EG experts, group of ROUTE_TG tokens);
        // wave w takes expert w / ROUTE_TG and token w % ROUTE_TG of them
        const int neg = (E + ROUTE_EG - 1) / ROUTE_EG;
        const int eg = blockIdx.x % neg, tg = blockIdx.x / neg;
        const int e = eg * ROUTE_EG + wave / ROUTE_TG, tl = wave % ROUTE_TG;
        const int t0 = tg * ROUTE_TG;
        const int tc = T - t0 < ROUTE_TG ? T - t0 : ROUTE_TG;
        // the expert's router row, 8 bf16 per lane and quarter (H <= 2048)
        uint4 wv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int hh = (q * WAVE + lane) * 8;
            wv[q] = make_uint4(0, 0, 0, 0);
            if (e < E && hh < H) wv[q] = *reinterpret_cast<const uint4 *>(wr + (size_t)e * H + hh);
        }
        const double b = bias && e < E ? (double)bias[e] : 0.0;
        // the group's input rows (with the residual) in LDS, 16 bytes per piece
        for (int i = tid; i < tc * (H / 8); i += blockDim.x) {
            const size_t gi = (size_t)(t0 + i / (H / 8)) * H + (i % (H / 8)) * 8;
            uint4 o = *reinterpret_cast<const uint4 *>(x + gi);
            if (yres) {
                const float4 ya = *reinterpret_cast<const float4 *>(yres + gi);
                const float4 yb = *reinterpret_cast<const float4 *>(yres + gi + 4);
                const float yv[8] = {ya.x, ya.y, ya.z, ya.w, yb.x, yb.y, yb.z, yb.w};
                uint32_t w4[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const uint32_t lo = f32_to_bf16_rne(bf16_to_f32(w4[jj] & 0xffffu) + yv[2 * jj]);
                    const uint32_t hi = f32_to_bf16_rne(bf16_to_f32(w4[jj] >> 16) + yv[2 * jj + 1]);
                    w4[jj] = lo | (hi << 16);
                }
                o = make_uint4(w4[0], w4[1], w4[2], w4[3]);
            }
            *reinterpret_cast<uint4 *>(&s_x[(i / (H / 8)) * H + (i % (H / 8)) * 8]) = o;
        }
        __syncthreads();
        if (e < E && tl < tc) {
            double acc = 0.0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int hh = (q * WAVE + lane) * 8;
                if (hh < H) {
                    const uint4 xv = *reinterpret_cast<const uint4 *>(&s_x[tl * H + hh]);
                    const uint32_t xs4[4] = {xv.x, xv.y, xv.z, xv.w};
                    const uint32_t ws4[4] = {wv[q].x, wv[q].y, wv[q].z, wv[q].w};
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        acc = fma((double)bf16_to_f32(xs4[jj] & 0xffffu), (double)bf16_to_f32(ws4[jj] & 0xffffu),
                                  acc);
                        acc = fma((double)bf16_to_f32(xs4[jj] >> 16), (double)bf16_to_f32(ws4[jj] >> 16), acc);
                    }
                }
            }
            acc = wave_sum_f64_dpp(acc);
            if (lane == 63) {
                const int t = t0 + tl;
                const uint16_t v = f32_to_bf16_rne((float)(acc + b));
                logits[(size_t)t * E + e] = v;
                if (tail)
                    __hip_atomic_store(handoff + (size_t)t * E + e, (unsigned int)v, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        if (!tail) return;  // top-k and grouping run in the next launch
        __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have completed
        __syncthreads();
        if (tid == 0) {
            // two-level count (one counter per group of workgroups b mod 8, then
            // one global count of finished groups): same-address atomics
            // serialise, so no counter sees more than ~E/8 arrivals
            const int grp = blockIdx.x % 8, ngrp = nb < 8 ? nb : 8;
            const unsigned in_grp = (unsigned)((nb - grp + 7) / 8);
            bool last = false;
            if (__hip_atomic_fetch_add(counter + ROUTE_COUNTER_STRIDE * (grp + 1), 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT) == in_grp - 1)
                last = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                       (unsigned)(ngrp - 1);
            s_last = last;
        }
        __syncthreads();
        if (!s_last) return;
        // every hand-off load of the thread in flight before the first is
        // used (one memory round trip, not one per load); the launch has
        // 1024 threads and T * E <= ROUTE_LDS_LOGITS
        static_assert(ROUTE_LDS_LOGITS % 1024 == 0, "hand-off loads per thread");
        constexpr int HO = ROUTE_LDS_LOGITS / 1024;
        const int n_lg = T * E;
        uint32_t hv[HO];
#pragma unroll
        for (int j = 0; j < HO; ++j) {
            const int i = tid + j * 1024;
            if (j * 1024 < n_lg) hv[j] = __hip_atomic_load(handoff + (i < n_lg ? i : n_lg - 1), __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int j = 0; j < HO; ++j) {
            const int i = tid + j * 1024;
            if (i < n_lg) s_lg[i] = (uint16_t)hv[j];
        }
        __syncthreads();
        // top-k from the LDS copy (LDS reads, not generic ones)
        for (int t = wave; t < T; t += 16)
            topk_token_wave<NPL>(s_lg + (size_t)t * E, E, k, idx + t * k, gate + t * k, s_idx + t * k);
    } else {
        if (!tail) return;
        for (int t = wave; t < T; t += 16)
            topk_token_wave<NPL>(logits + (size_t)t * E, E, k, idx + t * k, gate + t * k, s_idx + t * k);
    }
    __syncthreads();
    group_block_single(s_idx, T * k, E, g);
    if (wr && tid < 9)  // every workgroup has counted in: reset for the next call
        __hip_atomic_store(counter + ROUTE_COUNTER_STRIDE * tid, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// y[t] = z[t k] + z[t k + 1] + ... + z[t k + k - 1] (rows of H floats), the
// routed rows of a token added in slot order, so that every run gives the
// same bits; one float4 of y per thread.
__global__ __launch_bounds__(256) void decode_combine_kernel(const float *__restrict__ z, int T, int k, int H,
                                                             float *__restrict__ y) {
    const int h4 = H / 4;
    const int64_t n4 = (int64_t)T * h4;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = i / h4, c = i % h4;
        const float4 *zr = reinterpret_cast<const float4 *>(z) + t * k * h4 + c;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int s0 = 0; s0 < k; s0 += 8) {
            float4 v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (s0 + j < k) v[j] = zr[(int64_t)(s0 + j) * h4];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (s0 + j < k) {
                    acc.x += v[j].x;
                    acc.y += v[j].y;
                    acc.z += v[j].z;
                    acc.w += v[j].w;
                }
        }
        reinterpret_cast<float4 *>(y)[i] = acc;
    }
}

hipError_t launch_decode_combine(const float *z, int64_t T, int k, int H, float *y, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    if (H % 4 || k < 1) return hipErrorInvalidValue;
    const int64_t n4 = T * (H / 4);
    const int grid = (int)((n4 + 255) / 256 < 1024 ? (n4 + 255) / 256 : 1024);
    launch_k(decode_combine_kernel, dim3(grid), dim3(256), s, nullptr, nullptr, z, (int)T, k, H, y);
    return hipGetLastError();
}

template <int FMT, bool ROUTE, bool SHARED>
static hipError_t launch_experts_fmt(const uint16_t *x, const float *gate, int64_t T, int k, const LayerPtrs &L,
                                     const GroupOut &g, float *h, float *y, hipStream_t s, hipEvent_t e0,
                                     hipEvent_t e1, const uint16_t *lg, int32_t *idx_out, float *gate_out,
                                     const SharedPtrs &S, float *hs, float *zrows, int grid_div) {
    const int H = L.H, I = L.I;
    const int P = (int)(T * k);
    // 1/grid_div of the resident grid, a multiple of 8 (at least 8)
    auto grid = [&](int resident) {
        const int v = resident / grid_div / 8 * 8;
        return dim3(v < 8 ? 8 : v);
    };
    const int mt = (int)max_tiles(P, L.E, DECODE_TT);
    const dim3 block(DEC_WAVES * 64);
    switch (H / 64) {
#define CASE(LP)                                                                                                 \
    case LP: {                                                                                                   \
        constexpr auto kern = decode_gateup_kernel<LP, FMT, ROUTE, SHARED>;                                      \
        launch_k(kern, grid(resident_grid<kern>()), block, s, e0, e1, x, H, I, k, P, L, (const Tile *)g.tiles,    \
                 (const int32_t *)g.ntiles, mt, h, lg, (int)T, idx_out, gate_out, g, S, hs);                     \
    } break;
        CASE(1) CASE(2) CASE(4) CASE(8) CASE(16) CASE(32)
#undef CASE
        default: return hipErrorInvalidValue;
    }
    switch (I / 32) {
#define CASE(LP)                                                                                                 \
    case LP: {                                                                                                   \
        constexpr auto kern = decode_down_kernel<LP, FMT, SHARED>;                                               \
        launch_k(kern, grid(resident_grid<kern>()), block, s, nullptr, nullptr, H, I, k, P, L,                    \
                 (const Tile *)g.tiles, (const int32_t *)g.ntiles, mt, gate, (const float *)h, y, (int)T, S,  \
                 (const float *)hs, zrows);                                                                   \
    } break;
        CASE(2) CASE(4) CASE(8) CASE(16) CASE(32) CASE(64)
#undef CASE
        default: return hipErrorInvalidValue;
    }
    if (zrows) return launch_decode_combine(zrows, T, k, H, y, s);
    return hipGetLastError();
}

// The shared expert rides in the routed launches when its sizes fit them
// (same hidden size, same inner size, H >= 128); otherwise the caller runs it
// on its own.
bool decode_fuses_shared(const LayerPtrs &L, const SharedPtrs *S) {
    return S && S->H == L.H && S->I == L.I && L.H >= 128 && L.I >= 128;
}

template <bool ROUTE>
static hipError_t launch_experts_any(const uint16_t *x, const float *gate, int64_t T, int k, const LayerPtrs &L,
                                     const GroupOut &g, float *h, float *y, hipStream_t s, hipEvent_t e0,
                                     hipEvent_t e1, const uint16_t *lg, int32_t *idx_out, float *gate_out,
                                     const SharedPtrs *S, float *hs, float *zrows, int grid_div) {
    if (S && (zrows || !decode_fuses_shared(L, S))) return hipErrorInvalidValue;
    if (grid_div < 1) return hipErrorInvalidValue;
    const SharedPtrs none{};
#define FMT_CASE(F)                                                                                            \
    case F:                                                                                                    \
        return S ? launch_experts_fmt<F, ROUTE, true>(x, gate, T, k, L, g, h, y, s, e0, e1, lg, idx_out, gate_out, \
                                                      *S, hs, nullptr, grid_div)                               \
                 : launch_experts_fmt<F, ROUTE, false>(x, gate, T, k, L, g, h, y, s, e0, e1, lg, idx_out,      \
                                                       gate_out, none, nullptr, zrows, grid_div);
    switch (L.fmt) {
        FMT_CASE(0) FMT_CASE(1) FMT_CASE(2) FMT_CASE(3)
        default: return hipErrorInvalidValue;
    }
#undef FMT_CASE
}

hipError_t launch_decode_experts(const uint16_t *x, const float *gate, int64_t T, int k, const LayerPtrs &L,
                                 const GroupOut &g, float *h, float *y, hipStream_t s, hipEvent_t e0,
                                 hipEvent_t e1, const SharedPtrs *S, float *hs, float *zrows, int grid_div) {
    return launch_experts_any<false>(x, gate, T, k, L, g, h, y, s, e0, e1, nullptr, nullptr, nullptr, S, hs, zrows,
                                     grid_div);
}

// Every expert workgroup repeats this routing before its first weight load,
// so it pays off only while it is short: a few tokens (measured on MI355X:
// 1 token saves ~3 us per layer, 16 tokens lose ~2 us against the one-launch
// routing's last-workgroup step).
bool decode_routes_in_block(int64_t T, int k, int E) {
    return E <= DEC_ROUTE_EMAX && T * k <= DEC_ROUTE_PMAX_FAST && T * E <= DEC_ROUTE_LOGITS;
}

hipError_t launch_decode_experts_routed(const uint16_t *x, const uint16_t *logits, int64_t T, int k,
                                        const LayerPtrs &L, const GroupOut &g, int32_t *idx, float *gate, float *h,
                                        float *y, hipStream_t s, hipEvent_t e0, hipEvent_t e1, const SharedPtrs *S,
                                        float *hs, float *zrows, int grid_div) {
    if (!decode_routes_in_block(T, k, L.E)) return hipErrorInvalidValue;
    return launch_experts_any<true>(x, gate, T, k, L, g, h, y, s, e0, e1, logits, idx, gate, S, hs, zrows,
                                    grid_div);
}

hipError_t launch_decode_route_group(const uint16_t *x, const float *yres, uint16_t *xout, const uint16_t *wr,
                                     const float *bias, int T, int H, int E, int k, uint16_t *logits, int32_t *idx,
                                     float *gate, const GroupOut &g, float *yclear, unsigned int *counter,
                                     unsigned int *handoff, hipStream_t s, bool tail, hipEvent_t e0,
                                     hipEvent_t e1) {
    if (!tail) {  // logits only: the lean launch
        if (H > 2048) return hipErrorInvalidValue;
        launch_k(decode_router_kernel, dim3(wr ? E : 64), dim3(256), s, e0, e1, x, yres, xout, wr, bias, T, H, E,
                 logits, yclear);
        return hipGetLastError();
    }
    if (wr && T * E > ROUTE_LDS_LOGITS) return hipErrorInvalidValue;
    if (T * k > GROUP_SINGLE_MAX) return hipErrorInvalidValue;
    const int nb = wr ? (E + ROUTE_EG - 1) / ROUTE_EG * ((T + ROUTE_TG - 1) / ROUTE_TG) : 1;
    const int npl = (E + 63) / 64;
#define LAUNCH(N) \
    launch_k(decode_route_group_kernel<N>, dim3(nb), dim3(1024), s, e0, e1, x, yres, xout, wr, bias, T, H, E, k, \
             logits, idx, gate, g, yclear, counter, handoff, tail)
    if (npl <= 4) LAUNCH(4);
    else if (npl <= 8) LAUNCH(8);
    else LAUNCH(16);
#undef LAUNCH
    return hipGetLastError();
}

}  // namespace moeq4
