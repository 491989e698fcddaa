// Device-side grouping helpers shared by the grouping kernels and the fused
// decode routing kernel (see group.hip for the method).
#pragma once

#include "moe_internal.h"

namespace moeq4 {

// Exclusive scan over the block (blockDim.x a multiple of 64, at most 1024).
// Returns the exclusive prefix of v; *total receives the block sum.
__device__ inline int block_exclusive_scan(int v, int *lds16, int *total) {
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

// Offsets + tile list from per-expert counts held by thread e (< E).  Only
// the tiles' first four fields are written here: pair[u] of every row u <
// min(rows, DECODE_TT) is written by record_tile_pair once the sorted
// positions are known (possibly by other blocks, hence no write of the pair
// fields here).  *tadj_out = toff * S - excl of expert e (toff: index of its
// first tile, S: rows per tile).
__device__ inline void emit_offsets_and_tiles(int v, int E, int P, const GroupOut &g, int *lds16, int *excl_out,
                                              int *tadj_out) {
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
        Tile &t = g.tiles[toff + j];
        t.expert = e;
        t.row0 = excl + j * S;
        t.rows = v - j * S < S ? v - j * S : S;
        t.pad = 0;
    }
    if (e == 0) *g.ntiles = ntot;
    *excl_out = excl;
    *tadj_out = toff * S - excl;
}

// Tile field of the pair at sorted position pos of an expert with tile
// adjustment tadj (see emit_offsets_and_tiles): the pair is row u of tile t.
__device__ inline void record_tile_pair(const GroupOut &g, int pos, int tadj, int p) {
    const int S = g.rows_per_tile;
    const int r = pos + tadj;  // toff * S + rank within the expert
    const int u = r % S;
    if (u < DECODE_TT) g.tiles[r / S].pair[u] = p;
}

// Whole grouping by one block of 1024 threads (pairs P <= GROUP_SINGLE_MAX).
// idx may have been written earlier by this same block (visible after a
// __syncthreads()).
__device__ inline void group_block_single(const int32_t *idx, int P, int E, const GroupOut &g) {
    __shared__ int s_cnt[1024];
    __shared__ int s_base[1024];
    __shared__ unsigned long long s_mask[1024];
    __shared__ int s_tadj[1024];
    __shared__ int s_scan[17];
    const int tid = threadIdx.x;
    if (tid < E) s_cnt[tid] = 0;
    __syncthreads();
    for (int p = tid; p < P; p += blockDim.x) atomicAdd(&s_cnt[clamp_expert(idx[p], E)], 1);
    __syncthreads();
    int excl, tadj;
    emit_offsets_and_tiles(tid < E ? s_cnt[tid] : 0, E, P, g, s_scan, &excl, &tadj);
    if (tid < E) {
        s_base[tid] = excl;
        s_tadj[tid] = tadj;
    }
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
            record_tile_pair(g, pos, s_tadj[e], c0 + tid);
        }
        __syncthreads();
        if (tid < E) s_base[tid] += __popcll(s_mask[tid]);
        __syncthreads();
    }
}

}  // namespace moeq4
