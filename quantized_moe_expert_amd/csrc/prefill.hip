// Prefill path: grouped expert GEMMs on the gfx950 matrix cores.
//
// Prefill runs the experts over rows grouped by routed expert (drama-rs page,
// "Apple Silicon (MLX)": prefill groups rows by routed expert; "Layout":
// prefill is a grouped MoE).  For expert e with M_e routed rows this is
//   GEMM1  [M_e x H] x [H x 2I]  (gate and up) -> SwiGLU -> h [M_e x I]
//   GEMM2  [M_e x I] x [I x H]   (down)        -> gate-weighted add into y.
//
// Arithmetic.  Both products run as f16 x f16 -> fp32 on the matrix cores.
//  * Activations: x (bf16) is converted once to f16 after scaling its row by
//    a power of two 2^-e that puts the row's largest magnitude in
//    [2^14, 2^15).  The conversion is exact for every element within 2^31 of
//    that maximum (f16 keeps bf16's 8-bit significand down to 2^-24), and the
//    GEMM1 outputs are multiplied back by 2^e.  h is rounded to f16 by GEMM1,
//    so |h| must stay below 65504.
//  * Weights: a code unpacks to the exact f16 1024 + q; subtracting 1024
//    (asym) or 1032 (sym) gives q or q - 8 exactly, and one packed f16 fma
//    (s q + m) or multiply (s (q - 8)) dequantises two weights with a single
//    rounding to f16 (relative error <= 2^-11 per weight; the GEMM sums
//    these errors with random signs, about 2^-12 relative on an output).
//    Per-group scales therefore never touch the fp32 accumulators.
//
// Tiles: 128 rows (one tile-list entry, <= 128 rows of one expert) x 256
// weight rows per workgroup of 4 waves.  Wave w owns 32 columns in each of
// two N-subtiles (GEMM1: the gate rows and the up rows of the same 32 h
// columns, so SwiGLU pairs in registers; GEMM2: two groups of 32 output
// columns) for every M-subtile of 32 rows the tile uses; the main loop is
// instantiated per M-subtile count, so ragged tiles issue neither the loads
// nor the matrix-core work of their empty subtiles.  Both operands travel
// global -> LDS by direct-to-LDS loads (global_load_lds_dwordx4) through a
// 4-stage ring of 64-element K-steps; the block's scale words are staged in
// LDS once.
#include "moe_internal.h"

namespace moeq4 {

constexpr int PF_BLOCK = 256;
constexpr int BM = PREFILL_BM;  // 128

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------ x -> f16
//
// One wave per row: e = floor(log2 max|x|) - 14 (0 for a zero row or one
// holding inf / NaN), x16 = f16(x * 2^-e), xexp[t] = e.
__global__ __launch_bounds__(256) void x_to_f16_kernel(const uint16_t *__restrict__ x, int64_t T, int H,
                                                       uint16_t *__restrict__ x16, int32_t *__restrict__ xexp) {
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (t >= T) return;
    const uint4 *src = reinterpret_cast<const uint4 *>(x + t * H);
    uint32_t mx = 0;
    for (int i = lane; i < H / 8; i += 64) {
        const uint4 v = src[i];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t a = w[q] & 0x7fffu, b = (w[q] >> 16) & 0x7fffu;
            mx = a > mx ? a : mx;
            mx = b > mx ? b : mx;
        }
    }
    mx = wave_max_u32(mx);
    int e = 0;
    if (mx != 0 && mx < 0x7f80u) {
        const int be = (int)(mx >> 7);                  // biased exponent (0: subnormal)
        e = (be == 0 ? -126 : be - 127) - 14;
    }
    uint4 *dst = reinterpret_cast<uint4 *>(x16 + t * H);
    for (int i = lane; i < H / 8; i += 64) {
        const uint4 v = src[i];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const _Float16 lo = (_Float16)ldexpf(bf16_to_f32(w[q] & 0xffffu), -e);
            const _Float16 hi = (_Float16)ldexpf(bf16_to_f32(w[q] >> 16), -e);
            o[q] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
        dst[i] = make_uint4(o[0], o[1], o[2], o[3]);
    }
    if (lane == 0) xexp[t] = e;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float *__restrict__ p, int64_t n) {
    const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i + 3 < n) {
        *reinterpret_cast<float4 *>(p + i) = make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
        for (int64_t j = i; j < n; ++j) p[j] = 0.f;
    }
}

// ------------------------------------------------------------ weights
//
// Natural-order unpack: the 8 codes of a dword become four f16 pairs
// (k0,k1) (k2,k3) (k4,k5) (k6,k7), each half exactly 1024 + q.
__device__ __forceinline__ void unpack_natural_f16(uint32_t w, uint32_t out[4]) {
    const uint32_t lo = w & 0x0f0f0f0fu;          // bytes: k0 k2 k4 k6
    const uint32_t hi = (w >> 4) & 0x0f0f0f0fu;   // bytes: k1 k3 k5 k7
    const uint32_t c = 0x64646464u;               // high byte of f16 1024
    // v_perm_b32: selector bytes 0-3 pick the second operand, 4-7 the first
    const uint32_t t0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);  // k0 k1 k2 k3
    const uint32_t t1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);  // k4 k5 k6 k7
    out[0] = __builtin_amdgcn_perm(c, t0, 0x04010400u);
    out[1] = __builtin_amdgcn_perm(c, t0, 0x04030402u);
    out[2] = __builtin_amdgcn_perm(c, t1, 0x04010400u);
    out[3] = __builtin_amdgcn_perm(c, t1, 0x04030402u);
}

// Two weights from a pair of 1024 + q halves: s q + m (asym) or s (q - 8)
// (sym), each rounded once to f16.
template <int FMT>
__device__ __forceinline__ uint32_t dequant_pair(uint32_t v, half2_t s2, half2_t m2) {
    const half2_t off = {(_Float16)(FMT == 0 ? 1024.0f : 1032.0f), (_Float16)(FMT == 0 ? 1024.0f : 1032.0f)};
    const half2_t q = __builtin_bit_cast(half2_t, v) - off;
    const half2_t r = FMT == 0 ? __builtin_elementwise_fma(s2, q, m2) : s2 * q;
    return __builtin_bit_cast(uint32_t, r);
}

// ------------------------------------------------------------ grouped GEMM

// s_waitcnt on the vector-memory counter (n <= 63) and on LDS (0): this
// wave's direct-to-LDS loads older than the n youngest have landed and its
// LDS reads are done.
#define MOEQ4_WAIT_VM_LDS(n) __builtin_amdgcn_s_waitcnt(((n) & 0xf) | (((n) >> 4) << 14) | (0x7 << 4))

constexpr int KS = 64;       // contraction elements per pipeline stage
constexpr int NST = 4;       // LDS ring stages
constexpr int BROWS = 256;   // weight rows per workgroup (gate 128 + up 128, or 256 down rows)
constexpr int A_BYTES = BM * KS * 2;            // 16 KB: 128 rows x 64 f16
constexpr int B_BYTES = BROWS * KS / 2;         // 8 KB: 256 rows x 64 codes
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;  // 24 KB
constexpr int B_LOADS = B_BYTES / 16 / PF_BLOCK;  // 2 sixteen-byte loads per thread and stage
constexpr int SM_PITCH = BROWS + 1;             // LDS pitch of the per-group scale rows

// Per-block operand sources and LDS addresses used by the main loop.
struct GemmCtx {
    const uint8_t *a_src[4];   // this thread's A chunk source, one per 32-row subtile
    const uint8_t *b_src[B_LOADS];
    uint8_t *ring;
    const uint32_t *sm;        // [group][SM_PITCH] scale words
    int brow[2];               // this lane's weight rows (block-local) of the two N-subtiles
    int nk;                    // K-steps
};

// Barrier between the waves of the block that orders their LDS traffic
// without waiting for outstanding direct-to-LDS loads (the waits above do
// that, counted).
__device__ __forceinline__ void lds_barrier() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// One thread's share of K-step `ks` into ring slot `slot`: MS A loads (one per
// 32-row subtile in use) and B_LOADS B loads, 16 bytes each, lane-ordered.
template <int MS>
__device__ __forceinline__ void issue_stage(const GemmCtx &c, int ks, int slot, int wave) {
    uint8_t *sa = c.ring + slot * STAGE_BYTES;
    uint8_t *sb = sa + A_BYTES;
#pragma unroll
    for (int i = 0; i < MS; ++i)
        __builtin_amdgcn_global_load_lds((const void *)(c.a_src[i] + (size_t)ks * (KS * 2)),
                                         (__attribute__((address_space(3))) void *)(sa + (i * 4 + wave) * 1024),
                                         16, 0, 0);
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i)
        __builtin_amdgcn_global_load_lds((const void *)(c.b_src[i] + (size_t)ks * (KS / 2)),
                                         (__attribute__((address_space(3))) void *)(sb + (i * 4 + wave) * 1024),
                                         16, 0, 0);
}

// Main loop over K for a tile of MS x 32 rows.
template <int FMT, int MS>
__device__ __forceinline__ void gemm_main(const GemmCtx &c, f32x16_t (&acc)[4][2], int wave, int lane) {
    constexpr int G = FMT == 0 ? 64 : 128;
    constexpr int KPG = G / KS;
    constexpr int LPS = MS + B_LOADS;  // loads per thread and stage
    const int l32 = lane & 31, hf = lane >> 5;
    const int NK = c.nk;

#pragma unroll
    for (int u = 0; u < NST - 1; ++u)
        if (u < NK) issue_stage<MS>(c, u, u, wave);

    half2_t s2[2], m2[2];
    for (int kk = 0; kk < NK; kk += NST) {
#pragma unroll
        for (int u = 0; u < NST; ++u) {
            const int ks = kk + u;
            if (ks < NK) {
                // K-step ks has landed once at most `later` younger stages are in flight
                const int later = NK - 1 - ks < NST - 2 ? NK - 1 - ks : NST - 2;
                if (later >= 2) MOEQ4_WAIT_VM_LDS(2 * LPS);
                else if (later == 1) MOEQ4_WAIT_VM_LDS(LPS);
                else MOEQ4_WAIT_VM_LDS(0);
                lds_barrier();  // every wave's share of ks is in LDS; slot (u - 1) % NST is free
                if (ks + NST - 1 < NK) issue_stage<MS>(c, ks + NST - 1, (u + NST - 1) % NST, wave);
                const uint8_t *sa = c.ring + u * STAGE_BYTES;
                const uint8_t *sb = sa + A_BYTES;
                if (ks % KPG == 0) {
                    const int g = ks / KPG;
#pragma unroll
                    for (int ns = 0; ns < 2; ++ns) {
                        const uint32_t pw = c.sm[g * SM_PITCH + c.brow[ns]];
                        s2[ns] = __builtin_bit_cast(half2_t, (pw & 0xffffu) * 0x10001u);
                        m2[ns] = __builtin_bit_cast(half2_t, (pw >> 16) * 0x10001u);
                    }
                }
                // B: 16 bytes (32 codes) of each of this lane's two weight rows
                uint4 bw[2];
#pragma unroll
                for (int ns = 0; ns < 2; ++ns) {
                    const int rb = c.brow[ns];
                    bw[ns] = *reinterpret_cast<const uint4 *>(sb + rb * 32 + 16 * (hf ^ ((rb >> 3) & 1)));
                }
#pragma unroll
                for (int s = 0; s < 4; ++s) {  // matrix-core K-steps of 16: elements [32 hf + 8 s, +8) per lane
                    u32x4_t bv[2];
#pragma unroll
                    for (int ns = 0; ns < 2; ++ns) {
                        const uint32_t word = s == 0 ? bw[ns].x : s == 1 ? bw[ns].y : s == 2 ? bw[ns].z : bw[ns].w;
                        uint32_t p[4];
                        unpack_natural_f16(word, p);
                        bv[ns] = u32x4_t{dequant_pair<FMT>(p[0], s2[ns], m2[ns]), dequant_pair<FMT>(p[1], s2[ns], m2[ns]),
                                         dequant_pair<FMT>(p[2], s2[ns], m2[ns]), dequant_pair<FMT>(p[3], s2[ns], m2[ns])};
                    }
                    const int ch = 4 * hf + s;  // logical 16-byte chunk of the A row
#pragma unroll
                    for (int mi = 0; mi < MS; ++mi) {
                        const int r = 32 * mi + l32;
                        const uint4 av = *reinterpret_cast<const uint4 *>(sa + r * 128 + 16 * (ch ^ ((r >> 1) & 7)));
                        const f16x8_t a8 = __builtin_bit_cast(f16x8_t, u32x4_t{av.x, av.y, av.z, av.w});
                        acc[mi][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a8, __builtin_bit_cast(f16x8_t, bv[0]),
                                                                            acc[mi][0], 0, 0, 0);
                        acc[mi][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a8, __builtin_bit_cast(f16x8_t, bv[1]),
                                                                            acc[mi][1], 0, 0, 0);
                    }
                }
            }
        }
    }
}

// STAGE 1: A = x16 rows gathered through perm, B = gate | up codes,
//          epilogue * 2^e(token), SwiGLU -> h (f16).
// STAGE 2: A = h rows (contiguous sorted rows), B = down codes,
//          epilogue gate-weighted float atomic add into y.
// Work item w = (tile j, column block cb) with cb fastest.  Workgroups are
// spread over the 8 XCDs round-robin (XCD = block index mod 8); each XCD
// takes a contiguous range of work items, so the column blocks of one tile
// (same A rows) and the tiles of one expert (same weights) meet in one L2.
// In the ring, A row r (128 bytes per stage) holds its 16-byte chunk c at
// c ^ ((r >> 1) & 7) and B row rb (32 bytes) at c ^ ((rb >> 3) & 1), so that
// the fragment reads of 16 lanes hit distinct LDS banks.
template <int FMT, int STAGE>
__global__ __launch_bounds__(PF_BLOCK) void grouped_gemm_kernel(
    const uint16_t *__restrict__ act,      // STAGE 1: x16 [T][H]; STAGE 2: h [P][I]
    const int32_t *__restrict__ xexp,      // STAGE 1: per-token exponent e
    int H, int I, int k, LayerPtrs L, const Tile *__restrict__ tiles, const int32_t *__restrict__ ntiles,
    const int32_t *__restrict__ perm, const float *__restrict__ topk_gate,
    uint16_t *__restrict__ h_out, float *__restrict__ y) {
    constexpr int G = FMT == 0 ? 64 : 128;
    constexpr int NGMAX = 2048 / G;

    const int ncb = STAGE == 1 ? I / 128 : H / BROWS;
    const int nwork = *ntiles * ncb;
    const int per = (nwork + 7) / 8;
    const int bx = blockIdx.x;
    if (bx / 8 >= per) return;
    const int w = (bx % 8) * per + bx / 8;
    if (w >= nwork) return;
    const int j = w / ncb, cb = w % ncb;
    const Tile tile = tiles[j];
    const int e = tile.expert, rows = tile.rows, row0 = tile.row0;
    const int K = STAGE == 1 ? H : I;
    const int NG = K / G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;
    const int col_base = cb * (STAGE == 1 ? 128 : BROWS);

    __shared__ __attribute__((aligned(16))) uint8_t s_ring[NST * STAGE_BYTES];
    __shared__ uint32_t s_sm[NGMAX * SM_PITCH];
    __shared__ int s_tok[BM];
    __shared__ float s_rs[BM];  // STAGE 1: 2^e of the row's token; STAGE 2: the row's gate

    if (tid < BM) {
        int t = 0;
        float v = 0.f;
        if (tid < rows) {
            const int p = perm[row0 + tid];
            t = p / k;
            v = STAGE == 2 ? topk_gate[p] : ldexpf(1.0f, xexp[t]);
        }
        s_tok[tid] = t;
        s_rs[tid] = v;
    }
    // scale words [g][weight row] into LDS
    for (int i = tid; i < BROWS * NG; i += PF_BLOCK) {
        const int rb = i / NG, g = i % NG;
        size_t wrow;
        const uint16_t *smb;
        if (STAGE == 1) {
            smb = rb < 128 ? L.gsm : L.usm;
            wrow = (size_t)e * I + col_base + (rb & 127);
        } else {
            smb = L.dsm;
            wrow = (size_t)e * H + col_base + rb;
        }
        uint32_t v;
        if (FMT == 0) v = reinterpret_cast<const uint32_t *>(smb)[wrow * NG + g];
        else v = smb[wrow * NG + g];
        s_sm[g * SM_PITCH + rb] = v;
    }
    __syncthreads();

    GemmCtx c;
    c.ring = s_ring;
    c.sm = s_sm;
    c.nk = K / KS;
    // A slot S = (i * 4 + wave) * 64 + lane (16 bytes): row S / 8 = 32 i + 8 wave + lane / 8,
    // stored chunk S % 8 holding logical chunk (S % 8) ^ ((row >> 1) & 7).
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 32 * i + 8 * wave + (lane >> 3);
        const int ch = (lane & 7) ^ ((r >> 1) & 7);
        const int rr = r < rows ? r : 0;  // padding rows read row 0; their outputs are dropped
        const uint16_t *rowp = STAGE == 1 ? act + (size_t)s_tok[rr] * H : act + (size_t)(row0 + rr) * I;
        c.a_src[i] = reinterpret_cast<const uint8_t *>(rowp + 8 * ch);
    }
    // B slot S: weight row S / 2, stored chunk S % 2 holding logical chunk (S % 2) ^ ((row >> 3) & 1)
    {
        const size_t row_bytes = (size_t)K / 2;
#pragma unroll
        for (int i = 0; i < B_LOADS; ++i) {
            const int S = (i * 4 + wave) * 64 + lane;
            const int rb = S / 2, ch = (S % 2) ^ ((rb >> 3) & 1);
            const uint8_t *base;
            if (STAGE == 1) base = rb < 128 ? L.gq + ((size_t)e * I + col_base + rb) * row_bytes
                                            : L.uq + ((size_t)e * I + col_base + rb - 128) * row_bytes;
            else base = L.dq + ((size_t)e * H + col_base + rb) * row_bytes;
            c.b_src[i] = base + 16 * ch;
        }
    }
#pragma unroll
    for (int ns = 0; ns < 2; ++ns) c.brow[ns] = STAGE == 1 ? ns * 128 + wave * 32 + l32 : wave * 64 + ns * 32 + l32;

    f32x16_t acc[4][2];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ns = 0; ns < 2; ++ns)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][ns][r] = 0.f;
    const int msub = (rows + 31) / 32;
    switch (msub) {
        case 1: gemm_main<FMT, 1>(c, acc, wave, lane); break;
        case 2: gemm_main<FMT, 2>(c, acc, wave, lane); break;
        case 3: gemm_main<FMT, 3>(c, acc, wave, lane); break;
        default: gemm_main<FMT, 4>(c, acc, wave, lane); break;
    }
    __syncthreads();  // ring no longer read: the epilogue may reuse it

    // ---- epilogue.  Accumulator element r of lane (l32, hf) in M-subtile mi
    // is row 32 mi + 8 (r / 4) + 4 hf + (r % 4), column l32 of the subtile.
    if (STAGE == 1) {
        // h tile [BM][128] f16 in LDS, then coalesced 16-byte stores.
        uint16_t *s_h = reinterpret_cast<uint16_t *>(s_ring);
        constexpr int HP = 128 + 8;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            if (mi < msub) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 32 * mi + 8 * (r / 4) + 4 * hf + (r % 4);
                    const float sc = s_rs[row];
                    const float gv = acc[mi][0][r] * sc;
                    const float uv = acc[mi][1][r] * sc;
                    const _Float16 hv = (_Float16)(silu(gv) * uv);
                    s_h[row * HP + wave * 32 + l32] = __builtin_bit_cast(uint16_t, hv);
                }
            }
        }
        __syncthreads();
        for (int i = tid; i < BM * 16; i += PF_BLOCK) {
            const int row = i / 16, cc = i % 16;
            if (row < rows)
                *reinterpret_cast<uint4 *>(h_out + (size_t)(row0 + row) * I + cb * 128 + cc * 8) =
                    *reinterpret_cast<const uint4 *>(&s_h[row * HP + cc * 8]);
        }
    } else {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            if (mi < msub) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 32 * mi + 8 * (r / 4) + 4 * hf + (r % 4);
                    if (row < rows) {
                        const float gt = s_rs[row];
                        float *dst = y + (size_t)s_tok[row] * H + col_base + wave * 64 + l32;
                        unsafeAtomicAdd(dst, gt * acc[mi][0][r]);
                        unsafeAtomicAdd(dst + 32, gt * acc[mi][1][r]);
                    }
                }
            }
        }
    }
}

template <int FMT>
static hipError_t launch_prefill_fmt(const uint16_t *x, const float *gate, int64_t T, int k, const LayerPtrs &L,
                                     const GroupOut &g, uint16_t *x16, int32_t *xexp, uint16_t *h, float *y,
                                     hipStream_t s, hipEvent_t const *ev) {
    const int H = L.H, I = L.I;
    const int64_t tiles = max_tiles(T * k, L.E, BM);
    hipLaunchKernelGGL(x_to_f16_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, x, T, H, x16, xexp);
    {
        const int64_t n = T * (int64_t)H;
        hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n / 4 + 256) / 256)), dim3(256), 0, s, y, n);
    }
    const unsigned nb1 = (unsigned)(((I / 128) * tiles + 7) / 8 * 8);
    const unsigned nb2 = (unsigned)(((H / BROWS) * tiles + 7) / 8 * 8);
    launch_k(grouped_gemm_kernel<FMT, 1>, dim3(nb1), dim3(PF_BLOCK), s, ev ? ev[0] : nullptr, ev ? ev[1] : nullptr,
             (const uint16_t *)x16, (const int32_t *)xexp, H, I, k, L, (const Tile *)g.tiles,
             (const int32_t *)g.ntiles, (const int32_t *)g.perm, gate, h, y);
    launch_k(grouped_gemm_kernel<FMT, 2>, dim3(nb2), dim3(PF_BLOCK), s, ev ? ev[2] : nullptr, ev ? ev[3] : nullptr,
             (const uint16_t *)h, (const int32_t *)nullptr, H, I, k, L, (const Tile *)g.tiles,
             (const int32_t *)g.ntiles, (const int32_t *)g.perm, gate, h, y);
    return hipGetLastError();
}

hipError_t launch_fill_zero(float *p, int64_t n, hipStream_t s) {
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n / 4 + 256) / 256)), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

hipError_t launch_fill_zero_u32(uint32_t *p, int64_t n, hipStream_t s) {
    return launch_fill_zero(reinterpret_cast<float *>(p), n, s);  // all-zero bits either way
}

hipError_t launch_prefill_experts(const uint16_t *x, const float *gate, int64_t T, int k, const LayerPtrs &L,
                                  const GroupOut &g, uint16_t *x16, int32_t *xexp, uint16_t *h, float *y,
                                  hipStream_t s, hipEvent_t const *ev) {
    return L.fmt == 0 ? launch_prefill_fmt<0>(x, gate, T, k, L, g, x16, xexp, h, y, s, ev)
                      : launch_prefill_fmt<1>(x, gate, T, k, L, g, x16, xexp, h, y, s, ev);
}

}  // namespace moeq4
