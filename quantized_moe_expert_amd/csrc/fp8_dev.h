// Block-FP8 routed experts on the decode GEMVs: E4M3 codes, one byte per
// weight, with one float32 scale per block of 128 rows x 128 inputs (the
// released experts' format: drama-3-w4a16 card, "At a glance" table, each
// matrix dequantised with its block scales, "How it was made").
//
// A lane takes 32 codes of a row as two 16-byte loads, [16c, 16c + 16) of
// the row's first half and of its second half (so each load instruction
// reads whole cache lines); each half lies in one 128-input block, whose
// scale multiplies the half's partial sum before the lanes of a row are
// added.  Codes are converted two at a time
// by the gfx950 conversion instructions, exactly (every E4M3 value, the
// subnormals included, is a bf16 and an f16 value):
//   gate/up: codes -> bf16 pairs in natural order, packed dot against the bf16
//     activations (exact products, fp32 sums);
//   down: codes -> f16 pairs in natural order, packed dot against h (each
//     row scaled by a power of two, rounded to f16; exact products, fp32
//     sums).
// h is kept in natural order for this format.
#pragma once

#include "decode_dev.h"

namespace moeq4 {

// Codes 2 hi .. 2 hi + 1 of a dword as an exact bf16 / f16 pair.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pair_bf16(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pair_f16(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
}

// Block scale of weight row n, inputs [k0, k0 + 32) of expert e's [N][K] matrix.
__device__ __forceinline__ float fp8_block_scale(const uint16_t *sm, int e, int N, int K, int n, int k0) {
    const float *s = reinterpret_cast<const float *>(sm);
    return s[((size_t)e * (N / 128) + n / 128) * (K / 128) + k0 / 128];
}

// gate/up GEMV + SwiGLU for one item (tile: one expert, up to DECODE_TT
// tokens; rows ir of I) into h (fp32, natural order).  LPR = H / 32 lanes per
// row; a wave-load covers 64 / LPR rows of gate and of up.  Pipelined in two
// register stages as the int4 gate/up GEMV.
template <int LPR, bool SHORT>
__device__ __forceinline__ void fp8_gateup_item(const uint16_t *__restrict__ x, int H, int I, int k,
                                                const LayerPtrs &L, const Tile &tile,
                                                const ItemRows<DEC_WAVES * WAVE / LPR> &ir,
                                                float *__restrict__ h, float (*s_out)[DEC_RB_MAX]) {
    constexpr int RPW = WAVE / LPR;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane % LPR, sub = lane / LPR;
    struct Stage {
        uint4 g[2], u[2];
        float gs[2], us[2];
    };
    const int e = tile.expert, nt = tile.rows;
    const int steps = ir.steps;
    const int lrow = wave * RPW + sub;
    auto issue = [&](Stage &st, int s) {
        const int n = ir.valid_step(s, lrow) ? ir.grow_step(s, lrow) : ir.grow(0);
        const size_t row = (size_t)e * I + n;
        const uint4 *gp = reinterpret_cast<const uint4 *>(L.gq + row * H + 16 * c);
        const uint4 *up = reinterpret_cast<const uint4 *>(L.uq + row * H + 16 * c);
        st.g[0] = gp[0];
        st.g[1] = gp[LPR];
        st.u[0] = up[0];
        st.u[1] = up[LPR];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            st.gs[hh] = fp8_block_scale(L.gsm, e, I, H, n, hh * (H / 2) + 16 * c);
            st.us[hh] = fp8_block_scale(L.usm, e, I, H, n, hh * (H / 2) + 16 * c);
        }
    };
    uint32_t xp[DECODE_TT][16];  // the lane's 32 activations of each token, bf16 pairs
    auto fetch_x = [&]() {
#pragma unroll
        for (int u = 0; u < DECODE_TT; ++u)
            if (u < nt) fetch_x_halves(x + (size_t)(tile.pair[u] / k) * H, c, H / 2, xp[u]);
    };
    auto consume = [&](const Stage &st, int s) {
        const int nl = s * (DEC_WAVES * RPW) + lrow;
        float dg[DECODE_TT][2], du[DECODE_TT][2];
#pragma unroll
        for (int u = 0; u < DECODE_TT; ++u) dg[u][0] = dg[u][1] = du[u][0] = du[u][1] = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 v = q == 0 ? st.g[0] : q == 1 ? st.g[1] : q == 2 ? st.u[0] : st.u[1];
            const uint32_t d4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t lo = e4m3_pair_bf16<false>(d4[j]), hi = e4m3_pair_bf16<true>(d4[j]);
                const int xi = 8 * (q & 1) + 2 * j;  // x words of codes 4j .. 4j + 3 of half q & 1
#pragma unroll
                for (int u = 0; u < DECODE_TT; ++u) {
                    if (u < nt) {
                        float &a = q < 2 ? dg[u][q & 1] : du[u][q & 1];
                        a = dot2_bf16(hi, xp[u][xi + 1], dot2_bf16(lo, xp[u][xi], a));
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < DECODE_TT; ++u) {
            if (u < nt) {
                const float pg = seg_sum_dpp<LPR>(fmaf(st.gs[0], dg[u][0], st.gs[1] * dg[u][1]));
                const float pu = seg_sum_dpp<LPR>(fmaf(st.us[0], du[u][0], st.us[1] * du[u][1]));
                if (c == LPR - 1 && ir.valid_step(s, lrow)) s_out[u][nl] = silu(pg) * pu;
            }
        }
    };
    Stage sa, sb;
    if (SHORT && steps == 1) {
        fetch_x();
        issue(sa, 0);
        consume(sa, 0);
    } else {
        fetch_x();
        issue(sa, 0);
        issue(sb, 1);
        for (int s = 0; s < steps; s += 2) {
            consume(sa, s);
            issue(sa, s + 2);
            if (s + 1 < steps) consume(sb, s + 1);
            issue(sb, s + 3);
        }
    }
    __syncthreads();
    for (int i = tid; i < nt * ir.nloc; i += blockDim.x) {
        const int u = i / ir.nloc, nl = i % ir.nloc;
        if (!ir.valid(nl)) continue;
        h[(size_t)(tile.row0 + u) * I + ir.grow(nl)] = s_out[u][nl];
    }
    __syncthreads();
}

// down GEMV for one item (tile; output rows ir of H) over the full inner
// dimension (LPR = I / 32 lanes per row, 32 codes each), multiplied by each
// token's gate and added into y (float atomics).
template <int LPR>
__device__ __forceinline__ void fp8_down_item(int H, int I, int k, const LayerPtrs &L, const Tile &tile,
                                              const ItemRows<DEC_WAVES * WAVE / LPR> &ir,
                                              const float *__restrict__ topk_gate, const float *__restrict__ h,
                                              float *__restrict__ y, float *__restrict__ zrows,
                                              float (*s_out)[DEC_RB_MAX]) {
    constexpr int RPW = WAVE / LPR;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane % LPR, sub = lane / LPR;
    struct Stage {
        uint4 v[DEC_NB][2];
        float s[DEC_NB][2];
    };
    const int e = tile.expert, nt = tile.rows;
    const int steps = ir.steps;
    const int lrow = wave * RPW + sub;
    auto issue = [&](Stage &st, int s0) {
#pragma unroll
        for (int b = 0; b < DEC_NB; ++b) {
            const int sb_ = s0 + b;
            const int d = ir.valid_step(sb_, lrow) ? ir.grow_step(sb_, lrow) : ir.grow(0);
            const uint4 *src = reinterpret_cast<const uint4 *>(L.dq + ((size_t)e * H + d) * I + 16 * c);
            st.v[b][0] = src[0];
            st.v[b][1] = src[LPR];
            st.s[b][0] = fp8_block_scale(L.dsm, e, H, I, d, 16 * c);
            st.s[b][1] = fp8_block_scale(L.dsm, e, H, I, d, I / 2 + 16 * c);
        }
    };
    int tok[DECODE_TT];
    float gt[DECODE_TT];
    uint32_t hp[DECODE_TT][16];
    HFetch hf;
    __shared__ __attribute__((aligned(16))) uint16_t s_h[DECODE_TT * DEC_HMAX];
    // h (fp32) and the gates, fetched before the first weight stages; the
    // rows are staged through LDS in f16 (each scaled by a power of two) after
    // them, the inverse power going with the gate
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
    auto conv_h = [&]() {
        float inv[DECODE_TT];
        h_to_lds<false>(hf, nt, I, s_h, inv);
#pragma unroll
        for (int u = 0; u < DECODE_TT; ++u) {
            if (u < nt) {
                gt[u] *= inv[u];
                h_from_lds_halves(s_h + u * DEC_HMAX, c, I / 2, hp[u]);
            }
        }
    };
    auto consume = [&](const Stage &st, int s0) {
#pragma unroll
        for (int b = 0; b < DEC_NB; ++b) {
            const int dl = (s0 + b) * (DEC_WAVES * RPW) + lrow;
            const uint32_t d8[8] = {st.v[b][0].x, st.v[b][0].y, st.v[b][0].z, st.v[b][0].w,
                                    st.v[b][1].x, st.v[b][1].y, st.v[b][1].z, st.v[b][1].w};
            float a[DECODE_TT][2];
#pragma unroll
            for (int u = 0; u < DECODE_TT; ++u) a[u][0] = a[u][1] = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t lo = e4m3_pair_f16<false>(d8[j]), hi = e4m3_pair_f16<true>(d8[j]);
#pragma unroll
                for (int u = 0; u < DECODE_TT; ++u)
                    if (u < nt)
                        a[u][j / 4] = dot2_f16(hi, hp[u][2 * j + 1], dot2_f16(lo, hp[u][2 * j], a[u][j / 4]));
            }
#pragma unroll
            for (int u = 0; u < DECODE_TT; ++u) {
                if (u < nt) {
                    const float o = seg_sum_dpp<LPR>(fmaf(st.s[b][0], a[u][0], st.s[b][1] * a[u][1]));
                    if (c == LPR - 1 && ir.valid_step(s0 + b, lrow)) s_out[u][dl] = gt[u] * o;
                }
            }
        }
    };
    Stage sa, sb;
    const int nst = (steps + DEC_NB - 1) / DEC_NB;
    if (nst == 1) {
        fetch_h();
        issue(sa, 0);
        conv_h();
        consume(sa, 0);
    } else {
        fetch_h();
        issue(sa, 0);
        issue(sb, DEC_NB);
        conv_h();
        for (int q = 0; q < nst; q += 2) {
            consume(sa, q * DEC_NB);
            issue(sa, (q + 2) * DEC_NB);
            if (q + 1 < nst) consume(sb, (q + 1) * DEC_NB);
            issue(sb, (q + 3) * DEC_NB);
        }
    }
    __syncthreads();
    emit_down_rows(y, zrows, tile, tok, nt, H, ir, s_out);
    __syncthreads();
}

}  // namespace moeq4
