// Shared expert GEMV item bodies: a SwiGLU MLP every token passes through,
// its linears int8 symmetric with one f16 scale per 128 input weights,
// w = scale * q (drama-q4 card, "What's quantized": the shared expert's
// linears are int8, symmetric, group 128).  Used by the shared expert's own
// launches and, beside the routed experts' items, by the decode launches of
// the layer.
//
// Work items are (token tile of up to DECODE_TT tokens, row chunk), cut as
// the routed decode items (decode_items, item_rows) but numbered chunk-major,
// so that the token tiles of one row chunk fall in one XCD's contiguous range
// and read the chunk's codes through one L2.
//
// Code arithmetic.  A signed byte q becomes u = q + 128 by flipping its top
// bit (one XOR per four codes):
//   gate/up: u goes to fp32 by the byte conversion instruction, u * x is exact
//     in fp32 (8-bit u, bf16 x), and sum_k q x = sum_k u x - 128 sum_k x with
//     the lane's sum of x taken once per token;
//   down: u is inserted into the mantissa of the f16 pair (1024, 1024) and
//     1152 is subtracted, which leaves q exactly as f16; q * h is exact in
//     fp32 against h scaled per token row by a power of two and rounded to
//     f16.
// A lane's codes are two 16-byte pieces, one in each half of the row, each
// inside one group; the group scale multiplies each piece's partial sum
// before the lanes of a row are added.
#pragma once

#include "decode_dev.h"

namespace moeq4 {

// Shared expert pointers as the kernels take them.
struct SharedPtrs {
    int H, I;
    const int8_t *gq, *uq, *dq;
    const uint16_t *gs, *us, *ds;
};

constexpr int SX_GROUP = 128;
constexpr uint32_t SX_FLIP = 0x80808080u;  // signed byte q -> u = q + 128

// f16 pair (1024 + u_a, 1024 + u_b) -> (q_a, q_b), exact.
__device__ __forceinline__ uint32_t sx_codes_f16(uint32_t pair) {
    const half2v_t off = {(_Float16)1152.0f, (_Float16)1152.0f};
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v_t, pair) - off);
}

// gate/up GEMV + SwiGLU of tokens tok0 .. tok0 + nt - 1 over rows ir of I,
// h (fp32, [T][I]) out.  LPR = H / 32 lanes per row, each
// lane 32 codes: [16c, 16c + 16) of the row's first half and of its second
// half (two 16-byte loads, each instruction reading whole cache lines; each
// half in one 128-group); a wave-load covers RPW = 64 / LPR rows of gate and
// of up.  Pipelined in two register stages as the routed gate/up GEMV.
template <int LPR>
__device__ __forceinline__ void shared_gateup_item(const uint16_t *__restrict__ x, const SharedPtrs &S, int tok0,
                                                   int nt, const ItemRows<DEC_WAVES * WAVE / LPR> &ir,
                                                   float *__restrict__ h, float (*s_out)[DEC_RB_MAX]) {
    constexpr int RPW = WAVE / LPR;
    const int H = S.H, I = S.I;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane % LPR, sub = lane / LPR;
    const int gi0 = (16 * c) / SX_GROUP, gi1 = (H / 2 + 16 * c) / SX_GROUP;
    const size_t smr = (size_t)(H / SX_GROUP);
    struct Stage {
        uint4 g[2], u[2];
        uint32_t gs[2], us[2];
    };
    const int steps = ir.steps;
    const int lrow = wave * RPW + sub;
    auto issue = [&](Stage &st, int s) {
        const size_t row = (size_t)(ir.valid_step(s, lrow) ? ir.grow_step(s, lrow) : ir.grow(0));
        const uint4 *gp = reinterpret_cast<const uint4 *>(S.gq + row * H + 16 * c);
        const uint4 *up = reinterpret_cast<const uint4 *>(S.uq + row * H + 16 * c);
        st.g[0] = gp[0];
        st.g[1] = gp[LPR];
        st.u[0] = up[0];
        st.u[1] = up[LPR];
        st.gs[0] = S.gs[row * smr + gi0];
        st.gs[1] = S.gs[row * smr + gi1];
        st.us[0] = S.us[row * smr + gi0];
        st.us[1] = S.us[row * smr + gi1];
    };
    uint32_t xp[DECODE_TT][16];
    float xf[DECODE_TT][32], xs[DECODE_TT][2];
    auto fetch_x = [&]() {
#pragma unroll
        for (int u = 0; u < DECODE_TT; ++u)
            if (u < nt) fetch_x_halves(x + (size_t)(tok0 + u) * H, c, H / 2, xp[u]);
    };
    auto prep_x = [&]() {
#pragma unroll
        for (int u = 0; u < DECODE_TT; ++u) {
            xs[u][0] = xs[u][1] = 0.f;
            if (u < nt) {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    xf[u][2 * j] = bf16_to_f32(xp[u][j] & 0xffffu);
                    xf[u][2 * j + 1] = bf16_to_f32(xp[u][j] >> 16);
                    xs[u][j / 8] += xf[u][2 * j] + xf[u][2 * j + 1];
                }
            }
        }
    };
    auto consume = [&](const Stage &st, int s) {
        const int nl = s * (DEC_WAVES * RPW) + lrow;
        const float sg[2] = {f16_to_f32((uint16_t)st.gs[0]), f16_to_f32((uint16_t)st.gs[1])};
        const float su[2] = {f16_to_f32((uint16_t)st.us[0]), f16_to_f32((uint16_t)st.us[1])};
        float dg[DECODE_TT][2], du[DECODE_TT][2];
#pragma unroll
        for (int u = 0; u < DECODE_TT; ++u) dg[u][0] = dg[u][1] = du[u][0] = du[u][1] = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 v = q == 0 ? st.g[0] : q == 1 ? st.g[1] : q == 2 ? st.u[0] : st.u[1];
            const uint32_t d4[4] = {v.x ^ SX_FLIP, v.y ^ SX_FLIP, v.z ^ SX_FLIP, v.w ^ SX_FLIP};
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const float f = (float)((d4[j] >> (8 * b)) & 0xffu);  // u, exact
                    const int e = 16 * (q & 1) + 4 * j + b;  // half q & 1
#pragma unroll
                    for (int u = 0; u < DECODE_TT; ++u) {
                        if (u < nt) {
                            if (q < 2) dg[u][q & 1] = fmaf(f, xf[u][e], dg[u][q & 1]);
                            else du[u][q & 1] = fmaf(f, xf[u][e], du[u][q & 1]);
                        }
                    }
                }
        }
#pragma unroll
        for (int u = 0; u < DECODE_TT; ++u) {
            if (u < nt) {
                const float pg = seg_sum_dpp<LPR>(fmaf(sg[0], fmaf(-128.f, xs[u][0], dg[u][0]),
                                                       sg[1] * fmaf(-128.f, xs[u][1], dg[u][1])));
                const float pu = seg_sum_dpp<LPR>(fmaf(su[0], fmaf(-128.f, xs[u][0], du[u][0]),
                                                       su[1] * fmaf(-128.f, xs[u][1], du[u][1])));
                if (c == LPR - 1 && ir.valid_step(s, lrow)) s_out[u][nl] = silu(pg) * pu;
            }
        }
    };
    Stage sa, sb;
    if (steps == 1) {
        fetch_x();
        issue(sa, 0);
        prep_x();
        consume(sa, 0);
    } else {
        fetch_x();
        issue(sa, 0);
        issue(sb, 1);
        prep_x();
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
        h[(size_t)(tok0 + u) * I + ir.grow(nl)] = s_out[u][nl];
    }
    __syncthreads();
}

// down GEMV of tokens tok0 .. tok0 + nt - 1 over output rows ir of H, full
// rows of h (LPR = I / 32 lanes per row, 32 codes each, split across the
// row's halves as in the gate/up GEMV; each token's fp32 h
// row staged once per item in LDS, scaled by the power of two that puts its
// largest magnitude in [2^14, 2^15) and rounded to f16, the outputs scaled
// back; h_to_lds), added into y:
// ATOMIC with float atomics (y shared with the routed experts' adds),
// otherwise y = (accumulate ? y : 0) + o by the one thread that owns the
// output.
template <int LPR, bool ATOMIC>
__device__ __forceinline__ void shared_down_item(const SharedPtrs &S, int tok0, int nt,
                                                 const ItemRows<DEC_WAVES * WAVE / LPR> &ir,
                                                 const float *__restrict__ h, float *__restrict__ y,
                                                 bool accumulate, float (*s_out)[DEC_RB_MAX]) {
    constexpr int RPW = WAVE / LPR;
    const int H = S.H, I = S.I;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane % LPR, sub = lane / LPR;
    const int gi0 = (16 * c) / SX_GROUP, gi1 = (I / 2 + 16 * c) / SX_GROUP;
    const size_t smr = (size_t)(I / SX_GROUP);
    const uint32_t kf = opaque_magic(MAGIC_F16);
    struct Stage {
        uint4 v[DEC_NB][2];
        uint32_t s[DEC_NB][2];
    };
    const int steps = ir.steps;
    const int lrow = wave * RPW + sub;
    auto issue = [&](Stage &st, int s0) {
#pragma unroll
        for (int b = 0; b < DEC_NB; ++b) {
            const int sb_ = s0 + b;
            const size_t row = (size_t)(ir.valid_step(sb_, lrow) ? ir.grow_step(sb_, lrow) : ir.grow(0));
            const uint4 *src = reinterpret_cast<const uint4 *>(S.dq + row * I + 16 * c);
            st.v[b][0] = src[0];
            st.v[b][1] = src[LPR];
            st.s[b][0] = S.ds[row * smr + gi0];
            st.s[b][1] = S.ds[row * smr + gi1];
        }
    };
    // the tokens' h rows: fetched before the first weight stages, staged in
    // LDS after them; then the lane's 32 values of each (f16 pairs (n0, n2),
    // (n1, n3) of each 4-block)
    HFetch hfe;
    __shared__ __attribute__((aligned(16))) uint16_t s_hs[DECODE_TT * DEC_HMAX];
    uint32_t hp[DECODE_TT][16];
    float hinv[DECODE_TT];
    auto fetch_h = [&]() { h_fetch(h, tok0, nt, I, hfe); };
    auto conv_h = [&]() {
        h_to_lds<false, true>(hfe, nt, I, s_hs, hinv);
#pragma unroll
        for (int u = 0; u < DECODE_TT; ++u) {
            if (u < nt) h_from_lds_halves(s_hs + u * DEC_HMAX, c, I / 2, hp[u]);
        }
    };
    auto consume = [&](const Stage &st, int s0) {
#pragma unroll
        for (int b = 0; b < DEC_NB; ++b) {
            const int dl = (s0 + b) * (DEC_WAVES * RPW) + lrow;
            const float sd0 = f16_to_f32((uint16_t)st.s[b][0]), sd1 = f16_to_f32((uint16_t)st.s[b][1]);
            const uint32_t d8[8] = {st.v[b][0].x, st.v[b][0].y, st.v[b][0].z, st.v[b][0].w,
                                    st.v[b][1].x, st.v[b][1].y, st.v[b][1].z, st.v[b][1].w};
            float a[DECODE_TT][2];
#pragma unroll
            for (int u = 0; u < DECODE_TT; ++u) a[u][0] = a[u][1] = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t w = d8[j] ^ SX_FLIP;
                const uint32_t qa = sx_codes_f16(insert_codes<0x00ff00ffu>(w, kf));       // codes 0, 2
                const uint32_t qb = sx_codes_f16(insert_codes<0x00ff00ffu>(w >> 8, kf));  // codes 1, 3
#pragma unroll
                for (int u = 0; u < DECODE_TT; ++u)
                    if (u < nt)
                        a[u][j / 4] = dot2_f16(qb, hp[u][2 * j + 1], dot2_f16(qa, hp[u][2 * j], a[u][j / 4]));
            }
#pragma unroll
            for (int u = 0; u < DECODE_TT; ++u) {
                if (u < nt) {
                    const float o = seg_sum_dpp<LPR>(fmaf(sd0, a[u][0], sd1 * a[u][1])) * hinv[u];
                    if (c == LPR - 1 && ir.valid_step(s0 + b, lrow)) s_out[u][dl] = o;
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
    for (int i = tid; i < nt * ir.nloc; i += blockDim.x) {
        const int u = i / ir.nloc, d = i % ir.nloc;
        if (!ir.valid(d)) continue;
        float *dst = y + (size_t)(tok0 + u) * H + ir.grow(d);
        if (ATOMIC) unsafeAtomicAdd(dst, s_out[u][d]);
        else *dst = accumulate ? *dst + s_out[u][d] : s_out[u][d];
    }
    __syncthreads();
}

}  // namespace moeq4
