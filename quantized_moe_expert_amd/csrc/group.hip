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
#include "group_dev.h"

namespace moeq4 {

// Whole grouping in one block of 1024 threads (pairs P <= GROUP_SINGLE_MAX);
// optionally clears y (n floats) for the atomic accumulation that follows.
__global__ __launch_bounds__(1024) void group_single_kernel(const int32_t *__restrict__ idx, int P, int E,
                                                            GroupOut g, float *__restrict__ yclear, int64_t n) {
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) yclear[i] = 0.f;
    group_block_single(idx, P, E, g);
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

// Step 2: one block per expert; exclusive scan of the expert's counts over
// the chunks (chunk order = pair order), written as each chunk's starting rank
// inside the expert; the total goes to cnt[e].
__global__ __launch_bounds__(1024) void group_colscan_kernel(int nchunks, int E, GroupOut g) {
    __shared__ int s_scan[GROUP_SCAN_LDS];
    const int e = blockIdx.x;
    int carry = 0;
    for (int c0 = 0; c0 < nchunks; c0 += blockDim.x) {
        const int c = c0 + threadIdx.x;
        const int v = c < nchunks ? g.chunk_cnt[(size_t)c * E + e] : 0;
        int total;
        const int excl = block_exclusive_scan(v, s_scan, &total);
        if (c < nchunks) g.chunk_base[(size_t)c * E + e] = carry + excl;
        carry += total;
    }
    if (threadIdx.x == 0) g.cnt[e] = carry;
}

// Step 3: stable placement inside each chunk.  Every block rebuilds the
// expert offsets (exclusive scan of cnt, at most 1024 experts); block 0 also
// publishes off[] and the tile list.
__global__ __launch_bounds__(1024) void group_scatter_kernel(const int32_t *__restrict__ idx, int P, int E,
                                                             GroupOut g) {
    __shared__ unsigned long long s_mask[1024];
    __shared__ int s_off[1024];
    __shared__ int s_tadj[1024];
    __shared__ int s_scan[GROUP_SCAN_LDS];
    const int c = blockIdx.x, tid = threadIdx.x;
    const int v = tid < E ? g.cnt[tid] : 0;
    if (tid < E) s_mask[tid] = 0ull;
    int excl, tadj;
    if (c == 0) {
        emit_offsets_and_tiles(v, E, P, g, s_scan, &excl, &tadj);
    } else {
        const int S = g.rows_per_tile;
        const int in[2] = {v, tid < E ? (v + S - 1) / S : 0};
        int ex[2], tt[2];
        block_exclusive_scan_n<2>(in, s_scan, ex, tt);
        excl = ex[0];
        tadj = ex[1] * S - excl;
    }
    if (tid < E) {
        s_off[tid] = excl;
        s_tadj[tid] = tadj;
    }
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
        const int pos = s_off[e] + g.chunk_base[(size_t)c * E + e] + __popcll(s_mask[e] & ((1ull << tid) - 1ull));
        g.perm[pos] = p;
        g.inv[p] = pos;
        record_tile_pair(g, pos, s_tadj[e], p);
    }
}

hipError_t launch_group(const int32_t *idx, int64_t T, int k, int E, const GroupOut &g, hipStream_t s,
                        float *yclear, int64_t yclear_n, hipEvent_t e0, hipEvent_t e1) {
    const int P = (int)(T * k);
    if (P <= GROUP_SINGLE_MAX) {
        launch_k(group_single_kernel, dim3(1), dim3(1024), s, e0, e1, idx, P, E, g, yclear, yclear_n);
        return hipGetLastError();
    }
    if (yclear) return hipErrorInvalidValue;  // clearing is only offered on the one-block path
    const int nch = (P + GROUP_CHUNK - 1) / GROUP_CHUNK;
    hipLaunchKernelGGL(group_count_kernel, dim3(nch), dim3(256), 0, s, idx, P, E, g.chunk_cnt);
    return launch_group_after_count(idx, T, k, E, g, s, e0, e1);
}

hipError_t launch_group_after_count(const int32_t *idx, int64_t T, int k, int E, const GroupOut &g, hipStream_t s,
                                    hipEvent_t e0, hipEvent_t e1) {
    const int P = (int)(T * k);
    if (P <= GROUP_SINGLE_MAX) return hipErrorInvalidValue;
    const int nch = (P + GROUP_CHUNK - 1) / GROUP_CHUNK;
    hipLaunchKernelGGL(group_colscan_kernel, dim3(E), dim3(nch >= 1024 ? 1024 : ((nch + 63) / 64) * 64), 0, s,
                       nch, E, g);
    launch_k(group_scatter_kernel, dim3(nch), dim3(E > 64 ? ((E + 63) / 64) * 64 : 64), s, e0, e1, idx, P, E, g);
    return hipGetLastError();
}

}  // namespace moeq4
