// Device-side grouping helpers shared by the grouping kernels and the fused
// decode routing kernel (see group.hip for the method).
#pragma once

#include "moe_internal.h"

namespace moeq4 {

// Exclusive scan over the block (blockDim.x a multiple of 64, at most 1024).
// Returns the exclusive prefix of v; *total receives the block sum.
__device__ inline int block_exclusive_scan(int v, int *lds16, int *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int inc = wave_inclusive_scan_i32(v);
    if (lane == 63) lds16[wave] = inc;
    __syncthreads();
    int pre = 0, tot = 0;  // totals of the waves before this one, of all waves
    for (int w = 0; w < nw; ++w) {
        const int t = lds16[w];
        pre += w < wave ? t : 0;
        tot += t;
    }
    __syncthreads();  // lds16 free for the next scan
    *total = tot;
    return pre + inc - v;
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
    const int S = g.rows_per_tile;
    const int nt = e < E ? (v + S - 1) / S : 0;
    int excl, toff, ntot;
    if (P < 32768) {
        // counts and tile counts in one scan, 16 bits each: every prefix of
        // either is at most P (an expert's tiles are at most its rows)
        int tot;
        const int pk = block_exclusive_scan((e < E ? v : 0) | (nt << 16), lds16, &tot);
        excl = pk & 0xffff;
        toff = pk >> 16;
        ntot = tot >> 16;
    } else {
        int total;
        excl = block_exclusive_scan(v, lds16, &total);
        toff = block_exclusive_scan(nt, lds16, &ntot);
    }
    if (e < E) {
        g.cnt[e] = v;
        g.off[e] = excl;
    }
    if (e == 0) g.off[E] = P;
    for (int j = 0; j < nt; ++j) {
        Tile &t = g.tiles[toff + j];
        t.expert = e;
        t.row0 = excl + j * S;
        t.rows = v - j * S < S ? v - j * S : S;
        t.pad = 0;
    }
    if (e == 0) *g.ntiles = ntot;
    if (g.order) {
        // Schedule for the grouped GEMMs: the tiles ranked by their count of
        // S/4-row subtiles, most first (full tiles, then partial tiles of 4,
        // 3, 2 and 1 subtiles), each expert's in tile order within a rank.
        const int nf = e < E ? v / S : 0, rem = e < E ? v - nf * S : 0;
        const int qp = rem > 0 ? (rem + S / 4 - 1) / (S / 4) : 0;  // subtiles of the partial tile
        int base = 0;
        for (int q = 4; q >= 1; --q) {
            const int cq = (q == 4 ? nf : 0) + (qp == q ? 1 : 0);
            int tq;
            const int oq = block_exclusive_scan(cq, lds16, &tq);
            if (q == 4)
                for (int j = 0; j < nf; ++j) g.order[base + oq + j] = toff + j;
            if (qp == q) g.order[base + oq + (q == 4 ? nf : 0)] = toff + nf;
            base += tq;
        }
    }
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

// Grouping of few pairs (P <= GROUP_RANK_MAX, at most one pair per thread)
// without scans: pair i's sorted position is the number of pairs (e_j, j)
// ordered before (e_i, i); its row within its expert, its expert's count and
// offset, and the tiles of the experts before it are counts over the same P
// pairs (an expert's tiles counted at its first pair).  Same outputs as the
// scan path below; no tile schedule.
__device__ inline void group_block_rank(const int32_t *idx, int P, int E, const GroupOut &g) {
    __shared__ int s_e[GROUP_RANK_MAX];
    __shared__ int s_nt[GROUP_RANK_MAX];  // tiles of the pair's expert at its first pair, else 0
    const int tid = threadIdx.x;
    const int S = g.rows_per_tile;
    int e = 0, pos = 0, rin = 0, cnt = 0;
    if (tid < P) s_e[tid] = e = clamp_expert(idx[tid], E);
    __syncthreads();
    if (tid < P) {
#pragma unroll 8
        for (int j = 0; j < P; ++j) {
            const int ej = s_e[j];
            pos += ej < e || (ej == e && j < tid);
            rin += ej == e && j < tid;
            cnt += ej == e;
        }
        s_nt[tid] = rin == 0 ? (cnt + S - 1) / S : 0;
    }
    __syncthreads();
    for (int x = tid; x < E; x += blockDim.x) {
        int c = 0, o = 0;
#pragma unroll 8
        for (int j = 0; j < P; ++j) {
            const int ej = s_e[j];
            c += ej == x;
            o += ej < x;
        }
        g.cnt[x] = c;
        g.off[x] = o;
    }
    if (tid == 0) g.off[E] = P;
    if (tid < P) {
        int toff = 0, ntot = 0;
#pragma unroll 8
        for (int j = 0; j < P; ++j) {
            const int ntj = s_nt[j];
            ntot += ntj;
            toff += s_e[j] < e ? ntj : 0;
        }
        const int t = toff + rin / S, u = rin % S;
        g.perm[pos] = tid;
        g.inv[tid] = pos;
        if (u == 0) {
            Tile &tl = g.tiles[t];
            tl.expert = e;
            tl.row0 = pos;
            tl.rows = cnt - rin < S ? cnt - rin : S;
            tl.pad = 0;
        }
        if (u < DECODE_TT) g.tiles[t].pair[u] = tid;
        if (tid == 0) *g.ntiles = ntot;
    }
}

// Whole grouping by one block of 1024 threads (pairs P <= GROUP_SINGLE_MAX).
// idx may have been written earlier by this same block (visible after a
// __syncthreads()).
__device__ inline void group_block_single(const int32_t *idx, int P, int E, const GroupOut &g) {
    if (P <= GROUP_RANK_MAX && P <= (int)blockDim.x && !g.order) {
        group_block_rank(idx, P, E, g);
        return;
    }
    __shared__ int s_cnt[1024];
    __shared__ int s_base[1024];
    __shared__ unsigned long long s_mask[1024];
    __shared__ int s_tadj[1024];
    __shared__ int s_scan[17];
    const int tid = threadIdx.x;
    const int nch = (P + GROUP_CHUNK - 1) / GROUP_CHUNK;
    if (nch * E <= 1024) {
        // One pass over all chunks: s_mask[c * E + e] marks the pairs of
        // chunk c routed to expert e; counts and stable ranks are population
        // counts of these words.
        for (int i = tid; i < nch * E; i += blockDim.x) s_mask[i] = 0ull;
        __syncthreads();
        for (int p = tid; p < P; p += blockDim.x)
            atomicOr(&s_mask[(p / GROUP_CHUNK) * E + clamp_expert(idx[p], E)], 1ull << (p % GROUP_CHUNK));
        __syncthreads();
        int v = 0;
        if (tid < E)
            for (int c = 0; c < nch; ++c) v += __popcll(s_mask[c * E + tid]);
        int excl, tadj;
        emit_offsets_and_tiles(v, E, P, g, s_scan, &excl, &tadj);
        if (tid < E) {
            s_base[tid] = excl;
            s_tadj[tid] = tadj;
        }
        __syncthreads();
        for (int p = tid; p < P; p += blockDim.x) {
            const int e = clamp_expert(idx[p], E), c = p / GROUP_CHUNK;
            int r = __popcll(s_mask[c * E + e] & ((1ull << (p % GROUP_CHUNK)) - 1ull));
            for (int cc = 0; cc < c; ++cc) r += __popcll(s_mask[cc * E + e]);
            const int pos = s_base[e] + r;
            g.perm[pos] = p;
            g.inv[p] = pos;
            record_tile_pair(g, pos, s_tadj[e], p);
        }
        return;
    }
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
