// Grouping of (token, slot) pairs by routed expert: histogram, exclusive
// scan and a stable permutation (drama-rs page, "Apple Silicon (MLX)": prefill
// groups rows by routed expert; "Layout": grouped MoE prefill).
//
// Pairs are processed in chunks of 64 consecutive flat indices p = t*k + i.
// Inside a chunk, a 64-bit mask per expert marks the pairs routed to it, and
// the stable rank of a pair among its expert's pairs in the chunk is the
// population count of the mask bits below it.  Adding the number of that
// expert's pairs in earlier chunks and the expert's offset gives the sorted
// position.  The same pass emits the tile list used by the expert kernels:
// each expert's rows cut into tiles of at most rows_per_tile.
#include "moe_internal.h"

namespace moeq4 {

// Exclusive scan over the block (blockDim.x a multiple of 64, at most 1024).
// Returns the exclusive prefix of v; *total receives the block sum.
__device__ int block_exclusive_scan(int v, int *lds16, int *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    int inc = v;
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) {
        const int n = __shfl_up(inc, o, WAVE);
        if (lane >= o) inc += n;
    }
    if (lane == 63) lds16[wave] = inc;
    __syncthreads();
    if (wave == 0) {
        int w = lane < nw ? lds16[lane] : 0;
        int winc = w;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
            const int n = __shfl_up(winc, o, WAVE);
            if (lane >= o) winc += n;
        }
        if (lane < nw) lds16[lane] = winc - w;   // exclusive wave offsets
        if (lane == nw - 1) lds16[16] = winc;    // block total
    }
    __syncthreads();
    const int r = lds16[wave] + inc - v;
    *total = lds16[16];
    __syncthreads();
    return r;
}

// Offsets + tile list from per-expert counts held by thread e (< E).
__device__ void emit_offsets_and_tiles(int v, int E, int P, const GroupOut &g, int *lds16, int *excl_out) {
    const int e = threadIdx.x;
    int total;
    const int excl = block_exclusive_scan(v, lds16, &total);
    if (e < E) {
        g.cnt[e] = v;
        g.off[e] = excl;
    }
    if (e == 0) g.off[E] = P;
    const int S = g.rows_per_tile;
    const int nt = e < E ? (v + S - 1) / S : 0;
    int ntot;
    const int toff = block_exclusive_scan(nt, lds16, &ntot);
    for (int j = 0; j < nt; ++j) {
        Tile t;
        t.expert = e;
        t.row0 = excl + j * S;
        t.rows = v - j * S < S ? v - j * S : S;
        t.pad = 0;
        g.tiles[toff + j] = t;
    }
    if (e == 0) *g.ntiles = ntot;
    *excl_out = excl;
}

// Whole grouping in one block of 1024 threads (pairs P <= GROUP_SINGLE_MAX).
__global__ __launch_bounds__(1024) void group_single_kernel(const int32_t *__restrict__ idx, int P, int E,
                                                            GroupOut g) {
    __shared__ int s_cnt[1024];
    __shared__ int s_base[1024];
    __shared__ unsigned long long s_mask[1024];
    __shared__ int s_scan[17];
    const int tid = threadIdx.x;
    if (tid < E) s_cnt[tid] = 0;
    __syncthreads();
    for (int p = tid; p < P; p += blockDim.x) atomicAdd(&s_cnt[clamp_expert(idx[p], E)], 1);
    __syncthreads();
    int excl;
    emit_offsets_and_tiles(tid < E ? s_cnt[tid] : 0, E, P, g, s_scan, &excl);
    if (tid < E) s_base[tid] = excl;
    for (int c0 = 0; c0 < P; c0 += GROUP_CHUNK) {
        if (tid < E) s_mask[tid] = 0ull;
        __syncthreads();
        int e = 0;
        const bool mine = tid < GROUP_CHUNK && c0 + tid < P;
        if (mine) {
            e = clamp_expert(idx[c0 + tid], E);
            atomicOr(&s_mask[e], 1ull << tid);
        }
        __syncthreads();
        if (mine) {
            const int pos = s_base[e] + __popcll(s_mask[e] & ((1ull << tid) - 1ull));
            g.perm[pos] = c0 + tid;
            g.inv[c0 + tid] = pos;
        }
        __syncthreads();
        if (tid < E) s_base[tid] += __popcll(s_mask[tid]);
        __syncthreads();
    }
}

// Multi-block path, step 1: per-chunk expert counts.
__global__ __launch_bounds__(256) void group_count_kernel(const int32_t *__restrict__ idx, int P, int E,
                                                          int32_t *__restrict__ chunk_cnt) {
    __shared__ unsigned long long s_mask[1024];
    const int c = blockIdx.x, tid = threadIdx.x;
    for (int e = tid; e < E; e += blockDim.x) s_mask[e] = 0ull;
    __syncthreads();
    const int p = c * GROUP_CHUNK + tid;
    if (tid < GROUP_CHUNK && p < P) atomicOr(&s_mask[clamp_expert(idx[p], E)], 1ull << tid);
    __syncthreads();
    for (int e = tid; e < E; e += blockDim.x) chunk_cnt[(size_t)c * E + e] = __popcll(s_mask[e]);
}

// Step 2 (one block of 1024): per-expert running counts over chunks, offsets,
// tiles, and each chunk's starting position for each expert.
__global__ __launch_bounds__(1024) void group_scan_kernel(int nchunks, int P, int E, GroupOut g) {
    __shared__ int s_scan[17];
    const int e = threadIdx.x;
    int run = 0;
    if (e < E)
        for (int c = 0; c < nchunks; ++c) {
            const int v = g.chunk_cnt[(size_t)c * E + e];
            g.chunk_base[(size_t)c * E + e] = run;
            run += v;
        }
    int excl;
    emit_offsets_and_tiles(e < E ? run : 0, E, P, g, s_scan, &excl);
    if (e < E)
        for (int c = 0; c < nchunks; ++c) g.chunk_base[(size_t)c * E + e] += excl;
}

// Step 3: stable placement inside each chunk.
__global__ __launch_bounds__(256) void group_scatter_kernel(const int32_t *__restrict__ idx, int P, int E,
                                                            GroupOut g) {
    __shared__ unsigned long long s_mask[1024];
    const int c = blockIdx.x, tid = threadIdx.x;
    for (int e = tid; e < E; e += blockDim.x) s_mask[e] = 0ull;
    __syncthreads();
    const int p = c * GROUP_CHUNK + tid;
    const bool mine = tid < GROUP_CHUNK && p < P;
    int e = 0;
    if (mine) {
        e = clamp_expert(idx[p], E);
        atomicOr(&s_mask[e], 1ull << tid);
    }
    __syncthreads();
    if (mine) {
        const int pos = g.chunk_base[(size_t)c * E + e] + __popcll(s_mask[e] & ((1ull << tid) - 1ull));
        g.perm[pos] = p;
        g.inv[p] = pos;
    }
}

hipError_t launch_group(const int32_t *idx, int64_t T, int k, int E, const GroupOut &g, hipStream_t s) {
    const int P = (int)(T * k);
    if (P <= GROUP_SINGLE_MAX) {
        hipLaunchKernelGGL(group_single_kernel, dim3(1), dim3(1024), 0, s, idx, P, E, g);
        return hipGetLastError();
    }
    const int nch = (P + GROUP_CHUNK - 1) / GROUP_CHUNK;
    hipLaunchKernelGGL(group_count_kernel, dim3(nch), dim3(256), 0, s, idx, P, E, g.chunk_cnt);
    hipLaunchKernelGGL(group_scan_kernel, dim3(1), dim3(1024), 0, s, nch, P, E, g);
    hipLaunchKernelGGL(group_scatter_kernel, dim3(nch), dim3(256), 0, s, idx, P, E, g);
    return hipGetLastError();
}

}  // namespace moeq4
