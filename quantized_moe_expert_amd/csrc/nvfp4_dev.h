// NVFP4 routed experts on the decode GEMVs: packed E2M1 codes (two per byte,
// as the int4 formats), one E4M3 scale per 16 input weights and a float32
// global scale per matrix, the gate and up projections of an expert sharing
// theirs (drama-3-nvfp4 card, "Quantization"):
//   w[n][k] = e2m1(q[n][k]) * e4m3(scale[n][k/16]) * global.
//
// Lanes take the int4 formats' shares (gate/up: 64 codes, down: 32 codes).
// The gfx950 conversion instructions turn a byte's two codes into an exact
// bf16 (gate/up) or f16 (down) pair in natural order, one instruction per
// byte; a 16-code block's dot product is multiplied by its E4M3 scale
// (converted exactly to fp32), and the global scale multiplies the row.
// h is kept in natural order for this format.
#pragma once

#include "decode_dev.h"

namespace moeq4 {

template <int BYTE>
__device__ __forceinline__ uint32_t e2m1_pair_bf16(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, BYTE));
}
template <int BYTE>
__device__ __forceinline__ uint32_t e2m1_pair_f16(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, BYTE));
}
// E4M3 byte b of a dword as fp32 (exact).
template <int B>
__device__ __forceinline__ float e4m3_byte(uint32_t w) {
    return __builtin_amdgcn_cvt_f32_fp8((int)w, B);
}

// dot of the 8 codes of dword w with 4 bf16 pairs of x (natural order)
__device__ __forceinline__ float nv_dot8_bf16(uint32_t w, const uint32_t *x, float acc) {
    acc = dot2_bf16(e2m1_pair_bf16<0>(w), x[0], acc);
    acc = dot2_bf16(e2m1_pair_bf16<1>(w), x[1], acc);
    acc = dot2_bf16(e2m1_pair_bf16<2>(w), x[2], acc);
    return dot2_bf16(e2m1_pair_bf16<3>(w), x[3], acc);
}

// gate/up GEMV + SwiGLU for one item into h (fp32, natural order).  LPR =
// H / 64 lanes per row; a lane's 64 codes are 4 blocks of 16, whose scales
// are one dword of the row's scale bytes.
template <int LPR, bool SHORT>
__device__ __forceinline__ void nvfp4_gateup_item(const uint16_t *__restrict__ x, int H, int I, int k,
                                                  const LayerPtrs &L, const Tile &tile,
                                                  const ItemRows<DEC_WAVES * WAVE / LPR> &ir,
                                                  float *__restrict__ h, float (*s_out)[DEC_RB_MAX]) {
    constexpr int RPW = WAVE / LPR;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane % LPR, sub = lane / LPR;
    struct Stage {
        uint4 g[2], u[2];
        uint32_t gs, us;
    };
    const int e = tile.expert, nt = tile.rows;
    const int steps = ir.steps;
    const int lrow = wave * RPW + sub;
    const uint8_t *gsb = reinterpret_cast<const uint8_t *>(L.gsm), *usb = reinterpret_cast<const uint8_t *>(L.usm);
    const float glob = L.glob[2 * e];
    auto issue = [&](Stage &st, int s) {
        const int n = ir.valid_step(s, lrow) ? ir.grow_step(s, lrow) : ir.grow(0);
        const size_t row = (size_t)e * I + n;
        const uint4 *gp = reinterpret_cast<const uint4 *>(L.gq + row * (H / 2) + 32 * c);
        const uint4 *up = reinterpret_cast<const uint4 *>(L.uq + row * (H / 2) + 32 * c);
        st.g[0] = gp[0];
        st.g[1] = gp[1];
        st.u[0] = up[0];
        st.u[1] = up[1];
        st.gs = *reinterpret_cast<const uint32_t *>(gsb + row * (H / 16) + 4 * c);
        st.us = *reinterpret_cast<const uint32_t *>(usb + row * (H / 16) + 4 * c);
    };
    uint32_t xp[DECODE_TT][32];  // the lane's 64 activations of each token, bf16 pairs
    auto fetch_x = [&]() {
#pragma unroll
        for (int u = 0; u < DECODE_TT; ++u) {
            if (u < nt) {
                const uint16_t *xrow = x + (size_t)(tile.pair[u] / k) * H;
                fetch_x_chunk(xrow, 2 * c, xp[u]);
                fetch_x_chunk(xrow, 2 * c + 1, xp[u] + 16);
            }
        }
    };
    auto consume = [&](const Stage &st, int s) {
        const int nl = s * (DEC_WAVES * RPW) + lrow;
        float dg[DECODE_TT], du[DECODE_TT];
#pragma unroll
        for (int u = 0; u < DECODE_TT; ++u) dg[u] = du[u] = 0.f;
#pragma unroll
        for (int m = 0; m < 2; ++m) {  // gate, up
            const uint32_t d[8] = {m ? st.u[0].x : st.g[0].x, m ? st.u[0].y : st.g[0].y,
                                   m ? st.u[0].z : st.g[0].z, m ? st.u[0].w : st.g[0].w,
                                   m ? st.u[1].x : st.g[1].x, m ? st.u[1].y : st.g[1].y,
                                   m ? st.u[1].z : st.g[1].z, m ? st.u[1].w : st.g[1].w};
            const uint32_t sw = m ? st.us : st.gs;
            const float sc[4] = {e4m3_byte<0>(sw), e4m3_byte<1>(sw), e4m3_byte<2>(sw), e4m3_byte<3>(sw)};
#pragma unroll
            for (int b = 0; b < 4; ++b) {  // block of 16 codes: dwords 2b, 2b + 1
#pragma unroll
                for (int u = 0; u < DECODE_TT; ++u) {
                    if (u < nt) {
                        const float pb = nv_dot8_bf16(d[2 * b + 1], xp[u] + 8 * b + 4,
                                                      nv_dot8_bf16(d[2 * b], xp[u] + 8 * b, 0.f));
                        if (m == 0) dg[u] = fmaf(sc[b], pb, dg[u]);
                        else du[u] = fmaf(sc[b], pb, du[u]);
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < DECODE_TT; ++u) {
            if (u < nt) {
                const float pg = glob * seg_sum_dpp<LPR>(dg[u]);
                const float pu = glob * seg_sum_dpp<LPR>(du[u]);
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

// down GEMV for one item over the full inner dimension (LPR = I / 32 lanes
// per row, 32 codes = two 16-code blocks each), multiplied by each token's
// gate and added into y (float atomics).
template <int LPR>
__device__ __forceinline__ void nvfp4_down_item(int H, int I, int k, const LayerPtrs &L, const Tile &tile,
                                                const ItemRows<DEC_WAVES * WAVE / LPR> &ir,
                                                const float *__restrict__ topk_gate, const float *__restrict__ h,
                                                float *__restrict__ y, float *__restrict__ zrows,
                                                float (*s_out)[DEC_RB_MAX]) {
    constexpr int RPW = WAVE / LPR;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane % LPR, sub = lane / LPR;
    struct Stage {
        uint4 v[DEC_NB];
        uint32_t s[DEC_NB];
    };
    const int e = tile.expert, nt = tile.rows;
    const int steps = ir.steps;
    const int lrow = wave * RPW + sub;
    const uint8_t *dsb = reinterpret_cast<const uint8_t *>(L.dsm);
    const float glob = L.glob[2 * e + 1];
    auto issue = [&](Stage &st, int s0) {
#pragma unroll
        for (int b = 0; b < DEC_NB; ++b) {
            const int sb_ = s0 + b;
            const int d = ir.valid_step(sb_, lrow) ? ir.grow_step(sb_, lrow) : ir.grow(0);
            const size_t row = (size_t)e * H + d;
            st.v[b] = *reinterpret_cast<const uint4 *>(L.dq + row * (I / 2) + 16 * c);
            st.s[b] = *reinterpret_cast<const uint16_t *>(dsb + row * (I / 16) + 2 * c);
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
                h_from_lds(s_h + u * DEC_HMAX, c, hp[u]);
            }
        }
    };
    auto consume = [&](const Stage &st, int s0) {
#pragma unroll
        for (int b = 0; b < DEC_NB; ++b) {
            const int dl = (s0 + b) * (DEC_WAVES * RPW) + lrow;
            const uint32_t d4[4] = {st.v[b].x, st.v[b].y, st.v[b].z, st.v[b].w};
            const float sc[2] = {e4m3_byte<0>(st.s[b]), e4m3_byte<1>(st.s[b])};
            float a[DECODE_TT];
#pragma unroll
            for (int u = 0; u < DECODE_TT; ++u) a[u] = 0.f;
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
                for (int u = 0; u < DECODE_TT; ++u) {
                    if (u < nt) {
                        float pb = 0.f;
#pragma unroll
                        for (int q = 0; q < 2; ++q) {
                            const uint32_t w = d4[2 * blk + q];
                            const uint32_t *hh = hp[u] + 8 * blk + 4 * q;
                            pb = dot2_f16(e2m1_pair_f16<0>(w), hh[0], pb);
                            pb = dot2_f16(e2m1_pair_f16<1>(w), hh[1], pb);
                            pb = dot2_f16(e2m1_pair_f16<2>(w), hh[2], pb);
                            pb = dot2_f16(e2m1_pair_f16<3>(w), hh[3], pb);
                        }
                        a[u] = fmaf(sc[blk], pb, a[u]);
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < DECODE_TT; ++u) {
                if (u < nt) {
                    const float o = glob * seg_sum_dpp<LPR>(a[u]);
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
