// Device-side grouping helpers shared by the grouping kernels and the fused
// decode routing kernel (see group.hip for the method).
#pragma once

#include "moe_internal.h"

namespace moeq4 {

// N exclusive scans over the block at once (blockDim.x a multiple of 64, at
// most 1024), sharing the two barriers.  lds: GROUP_SCAN_LDS ints.  Each
// wave publishes its totals; lane w of every wave then reads wave w's, and
// one wave scan over those lanes gives the wave's prefix (lane wave - 1) and
// the block total (lane 15): one LDS read per value, few registers.
constexpr int GROUP_SCAN_N = 5;
constexpr int GROUP_SCAN_LDS = 16 * GROUP_SCAN_N;
template <int N>
__device__ inline void block_exclusive_scan_n(const int (&v)[N], int *lds, int (&excl)[N], int (&total)[N]) {
    static_assert(N >= 1 && N <= GROUP_SCAN_N, "scan count");
    const int lane = threadIdx.x & 63, nw = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    int inc[N];
#pragma unroll
    for (int j = 0; j < N; ++j) {
        inc[j] = wave_inclusive_scan_i32(v[j]);
        if (lane == 63) lds[16 * j + wave] = inc[j];
    }
    __syncthreads();
    int t[N];
#pragma unroll
    for (int j = 0; j < N; ++j) t[j] = lane < nw ? lds[16 * j + lane] : 0;
#pragma unroll
    for (int j = 0; j < N; ++j) {
        const int p = wave_inclusive_scan_i32(t[j]);  // lane w: totals of waves 0..w
        const int pre = wave > 0 ? __builtin_amdgcn_readlane(p, wave - 1) : 0;
        total[j] = __builtin_amdgcn_readlane(p, 15);  // lanes nw..15 add 0
        excl[j] = pre + inc[j] - v[j];
    }
    __syncthreads();  // lds free for the next scan
}

// One exclusive scan over the block; *total receives the block sum.
__device__ inline int block_exclusive_scan(int v, int *lds, int *total) {
    const int in[1] = {v};
    int ex[1], tt[1];
    block_exclusive_scan_n<1>(in, lds, ex, tt);
    *total = tt[0];
    return ex[0];
}

// Offsets + tile list from per-expert counts held by thread e (< E).  Only
// the tiles' first four fields are written here: pair[u] of every row u <
// min(rows, DECODE_TT) is written by record_tile_pair once the sorted
// positions are known (possibly by other blocks, hence no write of the pair
// fields here).  *tadj_out = toff * S - excl of expert e (toff: index of its
// first tile, S: rows per tile).  lds: GROUP_SCAN_LDS ints.
//
// With g.order, also the schedules of the grouped GEMMs, which run tile rank
// t on XCD t mod 8, consecutive ranks of one XCD one after another.
//   order (gate/up GEMM): tiles by their count of S/4-row subtiles, most
//     first (full tiles, then partial tiles of 4, 3, 2 and 1 subtiles), each
//     expert's in tile order within a count;
//   order2 (down GEMM, when set):
//     A. full tiles, expert order (a paired expert's last one excepted);
//     B. pairs in blocks of 16 ranks: 8 experts' last full tiles, then their
//        partial tiles in the same order, so each partial tile runs on its
//        full tile's XCD right after it and reads the same weights while they
//        are in that XCD's L2 (the experts with full tiles and a partial one,
//        in expert order, as many as fill whole blocks of 8);
//     C. the other partial tiles by subtile count, most first.
// Largest work first, so each XCD ends with its smallest tiles (order2 gives
// up some of that for the shared weight reads).
__device__ inline void emit_offsets_and_tiles(int v, int E, int P, const GroupOut &g, int *lds, int *excl_out,
                                              int *tadj_out) {
    const int e = threadIdx.x;
    const int S = g.rows_per_tile;
    const int vv = e < E ? v : 0;
    const int nt = (vv + S - 1) / S;
    const int nf = vv / S, rem = vv - nf * S;
    const int qp = rem > 0 ? (rem + S / 4 - 1) / (S / 4) : 0;  // subtiles of the partial tile
    const int flag = g.order2 && nf > 0 && rem > 0;          // pairing candidate
    int excl, toff, ntot, pi = 0, npair = 0;
    if (P < 65536 && P / S + (P < E ? P : E) < 32768) {
        // counts and tile counts in one value, 16 bits each (every prefix of
        // the counts is at most P, of the tile counts below 2^15)
        const int pk = vv | (nt << 16);
        int tot;
        if (g.order2) {
            const int in[2] = {pk, flag};
            int ex[2], tt[2];
            block_exclusive_scan_n<2>(in, lds, ex, tt);
            excl = ex[0] & 0xffff;
            toff = ex[0] >> 16;
            tot = tt[0];
            pi = ex[1];
            npair = tt[1];
        } else {
            const int ex = block_exclusive_scan(pk, lds, &tot);
            excl = ex & 0xffff;
            toff = ex >> 16;
        }
        ntot = tot >> 16;
    } else {
        const int in[3] = {vv, nt, flag};
        int ex[3], tt[3];
        block_exclusive_scan_n<3>(in, lds, ex, tt);
        excl = ex[0];
        toff = ex[1];
        ntot = tt[1];
        pi = ex[2];
        npair = tt[2];
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
        t.rows = vv - j * S < S ? vv - j * S : S;
        t.pad = 0;
    }
    if (e == 0) *g.ntiles = ntot;
    if (g.order) {
        const int in[4] = {nf + (qp == 4), qp == 3, qp == 2, qp == 1};
        int ex[4], tt[4];
        block_exclusive_scan_n<4>(in, lds, ex, tt);
        for (int j = 0; j < nf; ++j) g.order[ex[0] + j] = toff + j;
        if (qp > 0) {
            int base = 0;
            for (int q = 4; q > qp; --q) base += tt[4 - q];
            g.order[base + ex[4 - qp] + (qp == 4 ? nf : 0)] = toff + nf;
        }
    }
    if (g.order2) {
        const int nblk = npair / 8;
        const bool paired = flag && pi < 8 * nblk;
        // counts per section: A, then C by subtile count 4, 3, 2, 1
        const int in[5] = {nf - (paired ? 1 : 0), !paired && qp == 4, !paired && qp == 3, !paired && qp == 2,
                           !paired && qp == 1};
        int ex[5], tt[5];
        block_exclusive_scan_n<5>(in, lds, ex, tt);
        for (int j = 0; j < in[0]; ++j) g.order2[ex[0] + j] = toff + j;
        const int base_b = tt[0];
        if (paired) {
            const int r = base_b + 16 * (pi / 8) + pi % 8;
            g.order2[r] = toff + nf - 1;
            g.order2[r + 8] = toff + nf;
        } else if (qp > 0) {
            int base = base_b + 16 * nblk;
            for (int q = 4; q > qp; --q) base += tt[5 - q];
            g.order2[base + ex[5 - qp]] = toff + nf;
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
    __shared__ int s_scan[GROUP_SCAN_LDS];
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
