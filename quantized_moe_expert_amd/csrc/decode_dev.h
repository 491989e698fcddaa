// Building blocks of the weight-streaming GEMV kernels (routed decode
// experts and the shared expert): activation fetch, the (tile, row chunk)
// work decomposition over a resident grid, and packed dot products.
#pragma once

#include <atomic>

#include "moe_internal.h"

namespace moeq4 {

// Activation chunk [32c, 32c+32) of a bf16 row, as loaded (natural order).
__device__ __forceinline__ void fetch_x_chunk(const uint16_t *__restrict__ xrow, int c, uint32_t xp[16]) {
    const uint4 *src = reinterpret_cast<const uint4 *>(xrow + 32 * c);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint4 v = src[j];
        xp[4 * j + 0] = v.x;
        xp[4 * j + 1] = v.y;
        xp[4 * j + 2] = v.z;
        xp[4 * j + 3] = v.w;
    }
}
// Activations [16c, 16c + 16) and [n2 + 16c, n2 + 16c + 16) of a bf16 row
// (the two 16-code halves a lane takes when its loads are split across the
// row's halves, n2 = half the row), natural order, 4 pairs each.
__device__ __forceinline__ void fetch_x_halves(const uint16_t *__restrict__ xrow, int c, int n2, uint32_t xp[16]) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const uint4 *src = reinterpret_cast<const uint4 *>(xrow + hh * n2 + 16 * c);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint4 v = src[j];
            xp[8 * hh + 4 * j + 0] = v.x;
            xp[8 * hh + 4 * j + 1] = v.y;
            xp[8 * hh + 4 * j + 2] = v.z;
            xp[8 * hh + 4 * j + 3] = v.w;
        }
    }
}
// The fetched chunk put in PERM8 order in place; returns its sum.
__device__ __forceinline__ float perm_x_chunk(uint32_t xp[16]) {
    float xs = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t v0 = xp[4 * j], v1 = xp[4 * j + 1], v2 = xp[4 * j + 2], v3 = xp[4 * j + 3];
        xs += bf16_pair_sum(v0) + bf16_pair_sum(v1) + bf16_pair_sum(v2) + bf16_pair_sum(v3);
        perm8(v0, v1, v2, v3, xp[4 * j + 0], xp[4 * j + 1], xp[4 * j + 2], xp[4 * j + 3]);
    }
    return xs;
}

constexpr uint32_t ONES_F16X2 = 0x3c003c00u;  // f16 pair (1, 1)


// Work decomposition shared by the two GEMV kernels: nt tiles, each cut into
// nch chunks of `rows` consecutive rows out of N (nch as large as the grid
// allows, at most maxch, and enough that rows <= DEC_RB_MAX; every chunk
// starts inside the N rows, the last one may be shorter), items (tile, chunk)
// numbered tile-major and dealt to the XCDs in contiguous ranges.  The grid
// is a multiple of 8.
constexpr int DEC_RB_MAX = 256;  // rows per item (outputs staged in LDS)
struct Items {
    int nch, rows, items, first, stride, end;
};
__device__ __forceinline__ Items decode_items(int nt, int N, int maxch) {
    Items it;
    const int grid = gridDim.x;
    maxch = maxch < 1 ? 1 : maxch;
    int nch = nt > 0 ? grid / nt : 1;
    nch = nch < 1 ? 1 : (nch > maxch ? maxch : nch);
    const int minch = (N + DEC_RB_MAX - 1) / DEC_RB_MAX;  // at most DEC_RB_MAX rows per item
    nch = nch < minch ? minch : nch;
    it.rows = (N + nch - 1) / nch;
    it.nch = (N + it.rows - 1) / it.rows;  // <= nch; chunk c starts at c * rows < N
    it.items = nt * it.nch;
    const int per = (it.items + 7) / 8;
    const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
    it.first = xcd * per + slot;
    it.stride = grid / 8;
    const int e = (xcd + 1) * per;
    it.end = e < it.items ? e : it.items;
    return it;
}

// Rows of one item.  With DEC_INTERLEAVE, chunk `chunk` of nch takes the
// row blocks chunk, chunk + nch, chunk + 2 nch, ... of BR rows (BR: the rows
// one step of the workgroup covers), so that at any time the workgroups of a
// tile read neighbouring blocks of the expert's matrix; otherwise it takes
// `rows` consecutive rows.  Local row nl (0 <= nl < nloc = steps * BR, or the
// chunk's row count) is global row grow(nl); valid() excludes rows past N.
// nloc <= DEC_RB_MAX: decode_items makes nch >= N / DEC_RB_MAX, and BR is a
// power of two dividing DEC_RB_MAX.
constexpr bool DEC_INTERLEAVE = true;
template <int BR>
struct ItemRows {
    int chunk, nch, rows, steps, nloc, N;
    __device__ __forceinline__ int grow(int nl) const {
        return DEC_INTERLEAVE ? ((nl / BR) * nch + chunk) * BR + nl % BR : chunk * rows + nl;
    }
    __device__ __forceinline__ bool valid(int nl) const { return nl < nloc && grow(nl) < N; }
    // the same for local row s * BR + lrow (step s, 0 <= lrow < BR)
    __device__ __forceinline__ int grow_step(int s, int lrow) const {
        return DEC_INTERLEAVE ? (s * nch + chunk) * BR + lrow : chunk * rows + s * BR + lrow;
    }
    __device__ __forceinline__ bool valid_step(int s, int lrow) const {
        return s < steps && grow_step(s, lrow) < N && (DEC_INTERLEAVE || s * BR + lrow < nloc);
    }
};
template <int BR>
__device__ __forceinline__ ItemRows<BR> item_rows(int chunk, const Items &it, int N) {
    static_assert(BR > 0 && (BR & (BR - 1)) == 0 && DEC_RB_MAX % BR == 0, "row blocks tile DEC_RB_MAX");
    ItemRows<BR> r;
    r.chunk = chunk;
    r.nch = it.nch;
    r.rows = it.rows;
    r.N = N;
    if (DEC_INTERLEAVE) {
        const int nblk = (N + BR - 1) / BR;
        r.steps = chunk < nblk ? (nblk - chunk + it.nch - 1) / it.nch : 0;
        r.nloc = r.steps * BR;
    } else {
        const int n0 = chunk * it.rows;
        r.nloc = N - n0 < it.rows ? N - n0 : it.rows;
        r.nloc = r.nloc < 0 ? 0 : r.nloc;
        r.steps = (r.nloc + BR - 1) / BR;
    }
    return r;
}

// A down item's outputs (s_out[u][d]: pair u of the tile, local row d,
// gate applied): added into y[token] with one float atomic each, or, with
// zrows, stored as row d of the routed pair's own [H] row of zrows (a
// [T * k][H] array that a slot-ordered sum turns into y).
template <int BR>
__device__ __forceinline__ void emit_down_rows(float *__restrict__ y, float *__restrict__ zrows, const Tile &tile,
                                               const int (&tok)[DECODE_TT], int nt, int H, const ItemRows<BR> &ir,
                                               float (*s_out)[DEC_RB_MAX]) {
    for (int i = threadIdx.x; i < nt * ir.nloc; i += blockDim.x) {
        const int u = i / ir.nloc, d = i % ir.nloc;
        if (!ir.valid(d)) continue;
        // pair / token of slot u by selects (a dynamic index would move the
        // per-thread arrays to memory)
        int p = tile.pair[0], t = tok[0];
#pragma unroll
        for (int q = 1; q < DECODE_TT; ++q)
            if (u == q) p = tile.pair[q], t = tok[q];
        if (zrows) zrows[(size_t)p * H + ir.grow(d)] = s_out[u][d];
        else unsafeAtomicAdd(y + (size_t)t * H + ir.grow(d), s_out[u][d]);
    }
}

constexpr int DEC_WAVES = 4;  // waves per decode workgroup
constexpr int DEC_NB = 2;     // row loads per lane per pipeline stage

// Packed f16 dot product with fp32 accumulation.
typedef _Float16 half2v_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v_t, a), __builtin_bit_cast(half2v_t, b), c, false);
}

// h between the two decode GEMVs is fp32 [T*k][I] in natural order, the
// gate/up GEMV's SwiGLU output as computed.  A down-GEMV item stages the h
// rows of its tile's tokens once: the workgroup loads them (coalesced, one
// 16-byte load per thread and 512 values), finds each row's largest
// magnitude, scales the row by the power of two that puts it in
// [2^14, 2^15) (exact) and rounds it to f16 into LDS, so that f16's range
// never limits h (only its 11-bit precision does).  The row's outputs are
// multiplied back by the inverse power of two (exact) with the gate.
constexpr int DEC_HMAX = 2048;  // largest inner size of the decode GEMVs
// Thread tid takes the float4s i = tid + 256 j of the nt rows taken as one
// array.  The first (all of them up to 2 x 512 values) is loaded early, in
// flight with the weight stages; the others, for larger inner sizes, when
// the rows are staged.
struct HFetch {
    const float4 *src;
    float4 v0;
};
__device__ __forceinline__ void h_fetch(const float *__restrict__ h, int row0, int nt, int I, HFetch &f) {
    const int tid = threadIdx.x, tot = nt * (I / 4);
    f.src = reinterpret_cast<const float4 *>(h + (size_t)row0 * I);
    f.v0 = tid < tot ? f.src[tid] : make_float4(0.f, 0.f, 0.f, 0.f);
}
// The fetched rows scaled and rounded to f16 into s_h (row u at
// s_h + u * DEC_HMAX), in natural order, or with PERM8 in the int4 down
// GEMV's operand order (0,4 | 1,5 | 2,6 | 3,7 in each 8-block, the odd
// elements also divided by 16: odd codes enter in place as 1024 + 16 q),
// or with PAIR02 in the int8 down GEMV's order (n0, n2, n1, n3 in each
// 4-block: the pairs it forms from a code word); inv[u] = the inverse of
// row u's scale.  Every thread of the workgroup calls it (two barriers);
// s_h is complete on return.
template <bool PERM8, bool PAIR02 = false>
__device__ __forceinline__ void h_to_lds(const HFetch &f, int nt, int I, uint16_t *__restrict__ s_h,
                                         float inv[DECODE_TT]) {
    __shared__ uint32_t s_red[DECODE_TT][DEC_WAVES];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n4 = I / 4, tot = nt * n4;
    // pass 1: the largest magnitude of each row (the float4s past the first
    // are loaded here, one at a time: inner sizes above 512 only)
    uint32_t m[DECODE_TT];
#pragma unroll
    for (int u = 0; u < DECODE_TT; ++u) m[u] = 0u;
    auto row_max = [&](int i, const float4 &v) {
        // non-negative floats order as their bits
        const uint32_t mx = __float_as_uint(fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
#pragma unroll
        for (int u = 0; u < DECODE_TT; ++u)
            if (i / n4 == u) m[u] = m[u] > mx ? m[u] : mx;
    };
    if (tid < tot) row_max(tid, f.v0);
#pragma unroll 1
    for (int i = tid + DEC_WAVES * WAVE; i < tot; i += DEC_WAVES * WAVE) row_max(i, f.src[i]);
#pragma unroll
    for (int u = 0; u < DECODE_TT; ++u) {
        const uint32_t w = wave_max_u32(m[u]);
        if (lane == 0) s_red[u][wave] = w;
    }
    __syncthreads();
    float sc[DECODE_TT];
#pragma unroll
    for (int u = 0; u < DECODE_TT; ++u) {
        uint32_t r = 0u;
#pragma unroll
        for (int w = 0; w < DEC_WAVES; ++w) r = r > s_red[u][w] ? r : s_red[u][w];
        const RowScale rs = row_scale(__uint_as_float(r));
        sc[u] = rs.sc;
        inv[u] = exp2i(-rs.s);
    }
    // pass 2: scale, round to f16, store
    auto store = [&](int i, const float4 &v) {
        const int u = i / n4, n = 4 * (i - u * n4);
        float s = sc[0];
#pragma unroll
        for (int uu = 1; uu < DECODE_TT; ++uu) s = u == uu ? sc[uu] : s;
        uint16_t *row = s_h + u * DEC_HMAX;
        if (PERM8) {
            // n is 0 or 4 mod 8: elements n .. n + 3 go to slots
            // (n % 8 == 4 ? 1 : 0) + {0, 2, 4, 6} of the 8-block
            const float so = s * 0.0625f;
            const int b = (n & ~7) + ((n >> 2) & 1);
            row[b + 0] = __builtin_bit_cast(uint16_t, (_Float16)(v.x * s));
            row[b + 2] = __builtin_bit_cast(uint16_t, (_Float16)(v.y * so));
            row[b + 4] = __builtin_bit_cast(uint16_t, (_Float16)(v.z * s));
            row[b + 6] = __builtin_bit_cast(uint16_t, (_Float16)(v.w * so));
        } else if (PAIR02) {
            *reinterpret_cast<uint2 *>(row + n) = make_uint2(pack_f16x2(v.x * s, v.z * s), pack_f16x2(v.y * s, v.w * s));
        } else {
            const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(v.x * s)) |
                                ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(v.y * s)) << 16);
            const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(v.z * s)) |
                                ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(v.w * s)) << 16);
            *reinterpret_cast<uint2 *>(row + n) = make_uint2(lo, hi);
        }
    };
    if (tid < tot) store(tid, f.v0);
#pragma unroll 1
    for (int i = tid + DEC_WAVES * WAVE; i < tot; i += DEC_WAVES * WAVE) store(i, f.src[i]);
    __syncthreads();
}
// The lane's 32 staged values [16 c, 16 c + 16) and [n2 + 16 c, n2 + 16 c +
// 16) of a row (n2 = half the row) as 16 f16 pairs.
__device__ __forceinline__ void h_from_lds_halves(const uint16_t *__restrict__ s_row, int c, int n2,
                                                  uint32_t hp[16]) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const uint4 *src = reinterpret_cast<const uint4 *>(s_row + hh * n2 + 16 * c);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const uint4 v = src[q];
            hp[8 * hh + 4 * q + 0] = v.x;
            hp[8 * hh + 4 * q + 1] = v.y;
            hp[8 * hh + 4 * q + 2] = v.z;
            hp[8 * hh + 4 * q + 3] = v.w;
        }
    }
}
// The lane's 32 staged values [32 c, 32 c + 32) of row u as 16 f16 pairs.
__device__ __forceinline__ void h_from_lds(const uint16_t *__restrict__ s_row, int c, uint32_t hp[16]) {
    const uint4 *src = reinterpret_cast<const uint4 *>(s_row + 32 * c);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint4 v = src[q];
        hp[4 * q + 0] = v.x;
        hp[4 * q + 1] = v.y;
        hp[4 * q + 2] = v.z;
        hp[4 * q + 3] = v.w;
    }
}

// Workgroups of kernel K (256 threads) the device holds at once, a multiple
// of 8 (queried once per kernel and device).
template <auto K>
static int resident_grid() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, K, DEC_WAVES * 64, 0) != hipSuccess || per_cu < 1)
        per_cu = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    v = per_cu * cus;
    v = v < 8 ? 8 : v / 8 * 8;
    cache[dev].store(v, std::memory_order_relaxed);
    return v;
}

}  // namespace moeq4
