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

constexpr int DEC_WAVES = 4;  // waves per decode workgroup
constexpr int DEC_NB = 2;     // row loads per lane per pipeline stage

// Packed f16 dot product with fp32 accumulation.
typedef _Float16 half2v_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v_t, a), __builtin_bit_cast(half2v_t, b), c, false);
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
