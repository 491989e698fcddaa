// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_ext.h>

#include "moe_common.h"

namespace moeq4 {

constexpr int DECODE_TT = 2;  // tokens per decode work item

// Work item of the expert kernels: `rows` consecutive sorted rows of one
// expert starting at sorted position `row0`; pair[u] is the flat (token,
// slot) index t * k + i of row row0 + u for u < min(rows, DECODE_TT) (-1
// otherwise), so that the decode kernels need no permutation lookup.
struct Tile {
    int expert;
    int row0;
    int rows;
    int pad;
    int pair[DECODE_TT];
    int pad2[4 - DECODE_TT];
};
static_assert(sizeof(Tile) == 32, "Tile is two 16-byte words");

struct SharedPtrs;

// Layer pointers as the kernels take them.
struct LayerPtrs {
    int E, H, I, fmt;
    const uint8_t *gq, *uq, *dq;
    const uint16_t *gsm, *usm, *dsm;
    const float *glob;  // NVFP4 global scales [E][2] = {gate and up, down}
    const uint8_t *pack;  // prefill copy (tiles of 256 weight rows per K-step) or null
};

// Byte offsets of the prefill copy's regions: gate|up codes, gate|up scale
// words, down codes, down scale words, the int4 formats' per-row lifts
// (gate|up, down), and its size.  Block FP8 (format 2) has one byte per
// code and no scale regions (its block scales are read from the canonical
// array); NVFP4 (format 3) has no lifts.
struct PackLayout {
    size_t gu_q, gu_s, d_q, d_s, gu_l, d_l, total;
};
__host__ __device__ inline PackLayout pack_layout(int E, int H, int I, int fmt) {
    const size_t eih = (size_t)E * I * H;
    if (fmt == 2) return PackLayout{0, 2 * eih, 2 * eih, 3 * eih, 3 * eih, 3 * eih, 3 * eih};
    const size_t end = eih + eih / 8 + eih / 2 + eih / 16;
    if (fmt == 3) return PackLayout{0, eih, eih + eih / 8, eih + eih / 8 + eih / 2, end, end, end};
    return PackLayout{0, eih, eih + eih / 8, eih + eih / 8 + eih / 2, end, end + 2 * (size_t)E * I,
                      end + 2 * (size_t)E * I + (size_t)E * H};
}

// Power-of-two lift L of an int4 weight row (formats 0 and 1) in the prefill
// GEMMs: with A the largest magnitude of the row's f16 scales and mins
// (every |w| <= 16 A), the row's scale and min are taken times 2^L, L = 10 -
// floor(log2 A), so the row's weights dequantise to f16 below 2^15 and its
// small groups keep scale / 16 a normal f16; the output column is
// multiplied by 2^-L.  a_bits: A's f16 bit pattern (0: L = 0).
__host__ __device__ inline int row_lift_from_max(uint32_t a_bits) {
    a_bits &= 0x7fffu;
    if (a_bits == 0u) return 0;
    const int e = (int)(a_bits >> 10);
    int lg;  // floor(log2 A)
    if (e > 0) {
        lg = e - 15;
    } else {  // subnormal: A = m 2^-24
        int m = (int)a_bits, b = -1;
        while (m) {
            m >>= 1;
            ++b;
        }
        lg = b - 24;
    }
    return 10 - lg;
}

constexpr int GROUP_CHUNK = 64;          // (token, slot) pairs per grouping chunk
constexpr int GROUP_SINGLE_MAX = 1024;   // pairs handled by the one-block grouping
constexpr int GROUP_RANK_MAX = 64;       // pairs up to which it ranks them directly (no scans)
constexpr int PREFILL_BM = 128;          // rows per prefill tile
constexpr int ROUTE_LDS_LOGITS = 16384;  // T * E limit of the one-launch decode routing
constexpr int ROUTE_TG = 4;              // tokens per workgroup of the one-launch routing
constexpr int ROUTE_EG = 4;              // experts per workgroup of it (ROUTE_TG * ROUTE_EG = 16 waves)
constexpr int DEC_ROUTE_EMAX = 256;      // experts of the per-workgroup decode routing
constexpr int DEC_ROUTE_PMAX = 256;      // (token, slot) pairs of the per-workgroup decode routing
constexpr int DEC_ROUTE_PMAX_FAST = 64;  // pairs up to which the forward call uses it
constexpr int DEC_ROUTE_NPL = 4;         // logits per lane in its top-k (E <= 256)
constexpr int DEC_ROUTE_LOGITS = 8192;   // T * E logits it stages in LDS
constexpr int DEC_ROUTE_TMAX = DEC_ROUTE_PMAX / DECODE_TT + DEC_ROUTE_PMAX + 1;  // tiles it can form
constexpr int ROUTE_COUNTER_STRIDE = 32; // uint32 spacing (128 B) of the one-launch routing's 9 counters
constexpr size_t ROUTE_CONTROL_BYTES = 2048;  // control block holding them (cleared once)

inline int64_t max_tiles(int64_t pairs, int E, int rows_per_tile) {
    return pairs / rows_per_tile + (pairs < E ? pairs : E) + 1;
}

// Grouping outputs plus the derived tile list (tiles of at most rows_per_tile
// rows per expert, in expert order) and its length.
struct GroupOut {
    int32_t *cnt, *off, *perm, *inv;
    Tile *tiles;
    int32_t *ntiles;
    int rows_per_tile;
    int32_t *chunk_cnt;   // [nchunks][E] scratch (multi-block path)
    int32_t *chunk_base;  // [nchunks][E] scratch (multi-block path)
    int32_t *order = nullptr;  // or null: the tiles as the grouped GEMMs take them (see emit_offsets_and_tiles)
    int32_t *order2 = nullptr;  // or null: the down GEMM's own schedule (else it takes order)
};

hipError_t launch_router_logits(const uint16_t *x, const uint16_t *wr, const float *bias, int64_t T, int H,
                                int E, uint16_t *logits, hipStream_t s);
hipError_t launch_topk(const uint16_t *logits, int64_t T, int E, int k, int32_t *idx, float *gate, hipStream_t s);

// Grouping; on the one-block path (T*k <= GROUP_SINGLE_MAX) it can also clear
// yclear[0..yclear_n).
hipError_t launch_group(const int32_t *idx, int64_t T, int k, int E, const GroupOut &g, hipStream_t s,
                        float *yclear = nullptr, int64_t yclear_n = 0, hipEvent_t e0 = nullptr,
                        hipEvent_t e1 = nullptr);
// The multi-block grouping after its count step (T*k > GROUP_SINGLE_MAX,
// g.chunk_cnt filled, e.g. by launch_prefill_prep).
hipError_t launch_group_after_count(const int32_t *idx, int64_t T, int k, int E, const GroupOut &g, hipStream_t s,
                                    hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);

// Decode expert kernels: gate/up + SwiGLU -> h (fp32 [T*k][I]), then down
// (each row of h scaled by a power of two and rounded to f16) with the
// gate-weighted add into y (y must be cleared first).  e0 / e1 time the
// gate/up kernel.  With S the shared expert's items run in the same two
// launches (hs: its fp32 [T][I] SwiGLU output); S needs
// decode_fuses_shared.  With zrows ([T*k][H] floats) the down kernel stores
// each routed row there instead of adding into y, and a third launch sums
// each token's rows into y in slot order (run-to-run identical y); zrows
// excludes S.  grid_div > 1 launches each expert kernel over 1/grid_div of
// its resident grid (a multiple of 8, so the XCD dealing is unchanged), for
// token lanes that run side by side on their own streams.
bool decode_fuses_shared(const LayerPtrs &L, const SharedPtrs *S);
hipError_t launch_decode_experts(const uint16_t *x, const float *gate, int64_t T, int k, const LayerPtrs &L,
                                 const GroupOut &g, float *h, float *y, hipStream_t s, hipEvent_t e0 = nullptr,
                                 hipEvent_t e1 = nullptr, const SharedPtrs *S = nullptr, float *hs = nullptr,
                                 float *zrows = nullptr, int grid_div = 1);
hipError_t launch_decode_combine(const float *z, int64_t T, int k, int H, float *y, hipStream_t s);

// Router logits (when wr != null), top-k and one-block grouping of T <= 64
// tokens in one launch; clears y (T*H floats); with yres writes the residual
// input bf16(x + yres) to xout.  counter: zero on entry, zero on exit.  With
// tail == false the launch stops after the logits (and y, xout): top-k and
// grouping are left to launch_decode_experts_routed.
hipError_t launch_decode_route_group(const uint16_t *x, const float *yres, uint16_t *xout, const uint16_t *wr,
                                     const float *bias, int T, int H, int E, int k, uint16_t *logits, int32_t *idx,
                                     float *gate, const GroupOut &g, float *yclear, unsigned int *counter,
                                     unsigned int *handoff, hipStream_t s, bool tail = true,
                                     hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);

// Decode experts that route in every workgroup from the logits (written by
// an earlier launch): top-k into idx / gate and grouping into g are computed
// per workgroup in LDS and published by workgroup 0.  Used for E <= 256,
// T * k <= 64, T * E <= 8192 (decode_routes_in_block; the kernel itself
// holds up to 256 pairs).  y must be cleared first.
bool decode_routes_in_block(int64_t T, int k, int E);
hipError_t launch_decode_experts_routed(const uint16_t *x, const uint16_t *logits, int64_t T, int k,
                                        const LayerPtrs &L, const GroupOut &g, int32_t *idx, float *gate, float *h,
                                        float *y, hipStream_t s, hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr,
                                        const SharedPtrs *S = nullptr, float *hs = nullptr,
                                        float *zrows = nullptr, int grid_div = 1);

hipError_t launch_fill_zero(float *p, int64_t n, hipStream_t s);
hipError_t launch_fill_zero_u32(uint32_t *p, int64_t n, hipStream_t s);

// Grouped GEMMs of the prefill path; h: f16 [T*k][I] and its exponents hx
// int8 [T*k][I/128]; z: f16 [T*k][H] (the combine's input) and its
// exponents zx int8 [T*k][H/64].  y is written whole (no clearing needed).
hipError_t launch_prefill_experts(const uint16_t *x, const float *gate, int64_t T, int k, const LayerPtrs &L,
                                  const GroupOut &g, uint16_t *x16, int32_t *xexp, uint16_t *h, uint16_t *z,
                                  int8_t *hx, int8_t *zx, float *y, hipStream_t s, hipEvent_t const *ev = nullptr,
                                  bool x16_ready = false);
// Top-k of the given logits, the grouping's count step and the f16 rows of
// x (format fmt's order; none for block FP8) in one launch, for
// T*k > GROUP_SINGLE_MAX (then launch_group_after_count, and the experts
// with x16_ready).
hipError_t launch_prefill_prep(const uint16_t *logits, int64_t T, int E, int k, int32_t *idx, float *gate,
                               const GroupOut &g, const uint16_t *x, int H, uint16_t *x16, int32_t *xexp, int fmt,
                               hipStream_t s);

// Launch on s; when e0 is given the runtime records e0 / e1 at the kernel's
// own start and end (AMD extended launch), which times exactly that kernel.
template <typename F, typename... Args>
inline void launch_k(F kernel, dim3 grid, dim3 block, hipStream_t s, hipEvent_t e0, hipEvent_t e1, Args... args) {
    if (e0)
        hipExtLaunchKernelGGL(kernel, grid, block, 0, s, e0, e1, 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
}

hipError_t launch_dequant(const LayerPtrs &L, int expert, int proj, float *out, hipStream_t s);
// Writes the prefill copy of L's codes and scales (int4 formats, NVFP4) to dst.
hipError_t launch_prefill_pack(const LayerPtrs &L, uint8_t *dst, hipStream_t s);

// Shared expert (int8 symmetric group 128) for few tokens: gate/up + SwiGLU
// -> h (fp32 [T][I] workspace), then down (each h row scaled by a power of
// two and rounded to f16) -> y = (accumulate ? y : 0) + o.
// e0 / e1 time the gate/up kernel, e2 / e3 the down kernel.
hipError_t launch_shared(const uint16_t *x, int64_t T, const SharedPtrs &S, float *h, float *y, bool accumulate,
                         hipStream_t s, hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr, hipEvent_t e2 = nullptr,
                         hipEvent_t e3 = nullptr);
hipError_t launch_dequant_int8(const SharedPtrs &S, int proj, float *out, hipStream_t s);
// Shared expert for many tokens: dense f16 matrix-core GEMMs (x16, xexp: the
// [T][H] f16 activations and per-token exponents, h: [T][I] f16 and hx: its
// exponents [T][I / 128], all workspace).  Needs H % 256 == 0, I <= 2048.
constexpr int SHARED_GEMM_MIN_T = 65;  // token count from which the GEMMs run
hipError_t launch_shared_gemm(const uint16_t *x, int64_t T, const SharedPtrs &S, uint16_t *x16, int32_t *xexp,
                              uint16_t *h, int8_t *hx, float *y, bool accumulate, hipStream_t s, hipEvent_t e0 = nullptr,
                              hipEvent_t e1 = nullptr, hipEvent_t e2 = nullptr, hipEvent_t e3 = nullptr);
hipError_t launch_residual(const uint16_t *x, const float *y, int64_t n, uint16_t *out, hipStream_t s);

}  // namespace moeq4
