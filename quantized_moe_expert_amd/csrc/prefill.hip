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
//    GEMM1 outputs are multiplied back by 2^e.
//  * h: GEMM1 rounds h to f16 after scaling it by powers of two: each row by
//    2^-2e (h grows as the square of its token's activations, so this puts
//    every token in the same range), then the workgroup's 128 columns of
//    its rows by the 2^s that puts their largest magnitude in [2^14, 2^15);
//    s is stored beside h (int8, per row and 128-column block).  GEMM2 takes
//    the smallest s of its rows' blocks, s_min, as its unit and folds
//    2^(s_min - s_b) into the dequantised weights of block b (a power of
//    two: exact), and multiplies its outputs by 2^-s_min.  So f16's range
//    never limits h, only its 11-bit precision does.
//  * Weights: a code unpacks to the exact f16 1024 + q; subtracting 1024
//    (asym) or 1032 (sym) gives q or q - 8 exactly, and one packed f16 fma
//    (s q + m) or multiply (s (q - 8)) dequantises two weights with a single
//    rounding to f16 (relative error <= 2^-11 per weight; the GEMM sums
//    these errors with random signs, about 2^-12 relative on an output).
//    Per-group scales therefore never touch the fp32 accumulators.  Each
//    int4 weight row's scales and mins enter lifted by a power of two 2^L
//    (row_lift_from_max: the row's weights below 2^15, its small groups'
//    scale / 16 a normal f16), and the output column is multiplied by 2^-L.
//
// Layout of the f16 activations (x16, h): inside every group of 8 elements
// the order is 0,4,1,5,2,6,3,7 (PERM8), the order in which a packed code
// dword unpacks most cheaply, so a 16-byte fragment of either operand holds
// the same 8 contraction indices.
//
// Combine.  GEMM2 writes each routed row's gate-weighted output once, as f16
// (z, [T*k][H] in sorted row order), scaled by 2^-2e per row and by the
// power of two s_z that puts the largest magnitude of each 32-row x
// 64-column piece in [2^14, 2^15) (stored per row and 64 columns), with
// coalesced stores;
// a last kernel sums each token's k rows times 2^(2e - s_z) in fp32 into y.
// Scattering the rows into y with float atomics (k adds per output, done at
// the memory side so that the XCDs' L2s agree) took longer than GEMM2's
// matrix work.
//
// Tiles: 128 rows (one tile-list entry, <= 128 rows of one expert) x 256
// weight rows per workgroup of 4 waves, two workgroups per CU.  Wave w owns 32 columns in each of
// two N-subtiles (GEMM1: the gate rows and the up rows of the same 32 h
// columns, so SwiGLU pairs in registers; GEMM2: two groups of 32 output
// columns) for every M-subtile of 32 rows the tile uses; the main loop is
// instantiated per M-subtile count, so ragged tiles issue neither the loads
// nor the matrix-core work of their empty subtiles.  The A rows travel
// global -> LDS by direct-to-LDS loads (global_load_lds_dwordx4) through a
// ring of 64-element K-steps, one LDS array per slot, 4 to 5 stages deep; a
// lane's codes and scale words of each stage go straight to registers (from
// the prefill copy when the layer has one: contiguous per wave and step).
// The tiles are taken largest first (the grouping's schedule), dealt to the
// XCDs round-robin.
#include "moe_internal.h"
#include "route_dev.h"
#include "shared_dev.h"

namespace moeq4 {

constexpr int PF_BLOCK = 256;
constexpr int BM = PREFILL_BM;  // 128

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------ x -> f16
//
// One wave per row: e = floor(log2 max|x|) - 14 (0 for a zero row or one
// holding inf / NaN), x16 = f16(x * 2^-e), xexp[t] = e.  ORDER of the
// elements inside each group of 8: 0 natural, 1 PERM8 (0,4,1,5,2,6,3,7),
// 2 PERM4 (0,2,1,3,4,6,5,7); 3: xexp only (no x16; the block-FP8 GEMMs read
// x as given and use e only to scale h and z).
template <int ORDER>
__device__ __forceinline__ void x_row_to_f16(const uint16_t *__restrict__ x, int64_t t, int H,
                                             uint16_t *__restrict__ x16, int32_t *__restrict__ xexp) {
    const int lane = threadIdx.x & 63;
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
    uint4 *dst = ORDER == 3 ? nullptr : reinterpret_cast<uint4 *>(x16 + t * H);
    for (int i = lane; ORDER != 3 && i < H / 8; i += 64) {
        const uint4 v = src[i];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const _Float16 lo = (_Float16)ldexpf(bf16_to_f32(w[q] & 0xffffu), -e);
            const _Float16 hi = (_Float16)ldexpf(bf16_to_f32(w[q] >> 16), -e);
            o[q] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
        uint32_t p[4] = {o[0], o[1], o[2], o[3]};
        if (ORDER == 1) perm8(o[0], o[1], o[2], o[3], p[0], p[1], p[2], p[3]);
        if (ORDER == 2) {
#pragma unroll
            for (int j = 0; j < 4; j += 2) {
                p[j] = (o[j] & 0xffffu) | (o[j + 1] << 16);
                p[j + 1] = (o[j] >> 16) | (o[j + 1] & 0xffff0000u);
            }
        }
        dst[i] = make_uint4(p[0], p[1], p[2], p[3]);
    }
    if (lane == 0) xexp[t] = e;
}

template <int ORDER>
__global__ __launch_bounds__(256) void x_to_f16_kernel(const uint16_t *__restrict__ x, int64_t T, int H,
                                                       uint16_t *__restrict__ x16, int32_t *__restrict__ xexp) {
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t < T) x_row_to_f16<ORDER>(x, t, H, x16, xexp);
}

// Preparation of the prefill path for more than GROUP_SINGLE_MAX pairs, in
// one launch.  Workgroup c < nch takes grouping chunk c (pairs 64 c ..
// 64 c + 63): it takes the top-k of every token with a pair in the chunk and
// keeps the chunk's pairs (a token across two chunks is ranked by both, each
// keeping its own pairs) and counts them per expert as the grouping's count
// step does.  The workgroups after them convert the x rows, one per wave
// (ORDER as x_to_f16_kernel; none when CONVERT is false).
constexpr int PREP_WAVES = 8;  // one token of a top-8 chunk per wave

template <int NPL, int ORDER, bool CONVERT>
__global__ __launch_bounds__(PREP_WAVES * 64) void prefill_prep_kernel(const uint16_t *__restrict__ logits, int64_t T, int E,
                                                           int k, int32_t *__restrict__ idx,
                                                           float *__restrict__ gate, int32_t *__restrict__ chunk_cnt,
                                                           const uint16_t *__restrict__ x, int H,
                                                           uint16_t *__restrict__ x16, int32_t *__restrict__ xexp) {
    __shared__ unsigned long long s_mask[1024];
    __shared__ int32_t s_ti[PREP_WAVES][32];
    __shared__ float s_tg[PREP_WAVES][32];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t P = T * k;
    const int nch = (int)((P + GROUP_CHUNK - 1) / GROUP_CHUNK);
    if ((int)blockIdx.x >= nch) {
        const int64_t t = (int64_t)(blockIdx.x - nch) * PREP_WAVES + wave;
        if (CONVERT && t < T) x_row_to_f16<ORDER>(x, t, H, x16, xexp);
        return;
    }
    const int c = blockIdx.x;
    const int64_t p0 = (int64_t)c * GROUP_CHUNK;
    const int64_t p1 = p0 + GROUP_CHUNK < P ? p0 + GROUP_CHUNK : P;
    for (int e = tid; e < E; e += blockDim.x) s_mask[e] = 0ull;
    __syncthreads();
    for (int64_t t = p0 / k + wave; t <= (p1 - 1) / k; t += PREP_WAVES) {
        topk_token_wave<NPL>(logits + t * E, E, k, s_ti[wave], s_tg[wave]);
        if (lane < k) {
            const int64_t p = t * k + lane;
            if (p >= p0 && p < p1) {
                const int32_t e = s_ti[wave][lane];
                idx[p] = e;
                gate[p] = s_tg[wave][lane];
                atomicOr(&s_mask[clamp_expert(e, E)], 1ull << (p - p0));
            }
        }
    }
    __syncthreads();
    for (int e = tid; e < E; e += blockDim.x) chunk_cnt[(size_t)c * E + e] = __popcll(s_mask[e]);
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
// Two weights from a pair of unpacked halves v = 1024 + q (codes 0 and 4, 2
// and 6 of a dword) or v = 1024 + 16 q (codes 1 and 5, 3 and 7, taken in
// place: see insert_codes): (v - off) is exact and equals q, q - 8, 16 q or
// 16 q - 128; times s2 (the group scale, or scale / 16 for the 16 q pairs,
// exact while scale / 16 is a normal f16: the row lift keeps it so) plus m2
// (asym min) it is s q + m or s (q - 8), rounded once to f16.
template <int FMT>
__device__ __forceinline__ uint32_t dequant_pair(uint32_t v, half2_t off, half2_t s2, half2_t m2) {
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
constexpr int BROWS = 256;   // weight rows per workgroup (gate 128 + up 128, or 256 down rows)
constexpr int A_BYTES = BM * KS * 2;            // 16 KB: 128 rows x 64 f16
constexpr int B_BYTES = BROWS * KS / 2;         // 8 KB: 256 rows x 64 codes
constexpr int S_BYTES = BROWS * 4;              // 1 KB: one scale word per weight row

// The LDS ring holds the A rows of each stage (4 KB per 32-row subtile in
// use); a lane's codes and scale words of a stage go to registers (10 VGPRs
// per stage beside 32 accumulators per subtile).  Single-subtile tiles keep
// five K-steps in flight, the others four.
template <int MS>
constexpr int stage_bytes() { return MS * (A_BYTES / 4); }
template <int MS>
constexpr int ring_depth() { return MS == 1 ? 5 : 4; }
// Each ring slot is an LDS array of its own.  The compiler orders a read of
// LDS after every direct-to-LDS load that may write the same bytes; with one
// array for the whole ring it could not tell the slots apart and made each
// step wait for the loads just issued for later steps.  Slots 0-2 also hold
// 32 rows of the epilogue's output tile.
constexpr int RSLOT_BIG = 32 * (BROWS + 8) * 2;  // 16,896 B
constexpr int RSLOT3 = RSLOT_BIG;
constexpr int RSLOT4 = stage_bytes<1>();
static_assert(stage_bytes<4>() <= RSLOT_BIG && ring_depth<4>() == 4 && ring_depth<1>() == 5, "ring slots fit");

// Wait until at most n stages of LPS loads each are in flight (n <= 4; the
// count must be an immediate).
template <int LPS>
__device__ __forceinline__ void wait_stages(int n) {
    switch (n) {
        case 0: MOEQ4_WAIT_VM_LDS(0); break;
        case 1: MOEQ4_WAIT_VM_LDS(LPS); break;
        case 2: MOEQ4_WAIT_VM_LDS(2 * LPS); break;
        case 3: MOEQ4_WAIT_VM_LDS(3 * LPS); break;
        default: MOEQ4_WAIT_VM_LDS(4 * LPS); break;
    }
}

// Per-block operand sources used by the main loop.  Sources are a base that
// is uniform over the wave plus a 32-bit per-thread byte offset.
struct GemmCtx {
    const uint8_t *a_base;
    uint32_t a_off[4];               // A chunk of each 32-row subtile
    const uint8_t *b_base[2];        // per N-subtile: codes of the lane's weight row
    uint32_t b_off[2];               //   the lane's 16 bytes of K-step 0
    uint32_t b_kstep;                // bytes between K-steps of a weight row chunk
    const uint8_t *s_base[2];        // per N-subtile: the row's scale words
    uint32_t s_off[2];               //   its entry of group 0 (before 4-byte alignment)
    uint32_t s_step;                 // bytes between groups: 4 (scale+min) or 2 (scale); 0 in the copy
    uint32_t s_kstep;                // bytes between K-steps: 0, or 1 KB in the copy
    uint8_t *ring[5];                // the ring slots
    int brow[2];                     // this lane's weight rows (block-local) of the two N-subtiles
    uint32_t spar[2];                // sym: parity of the scale entry of group 0 of brow[ns]
    int nk;                          // K-steps
    int lexp[2];                     // int4: the rows' lifts L, applied to the scale words when
    bool lift_rt;                    //   lift_rt (the canonical arrays; the copy holds them lifted)
    const float *fb;                 // GEMM2: LDS [16], 2^(s_min - s_b) per 128-input block b (null in GEMM1)
};

// Barrier between the waves of the block that orders their LDS traffic
// without waiting for outstanding direct-to-LDS loads (those waits are
// counted explicitly).
__device__ __forceinline__ void lds_barrier() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// One thread's share of K-step `ks` (group g): MS A loads of 16 bytes (one
// per 32-row subtile in use) into ring slot `slot`, lane-ordered; and into
// registers, the lane's 16 bytes of codes of each of its two weight rows and
// the word holding each row's scale entry of group g: MS + 4 loads.
template <int MS>
__device__ __forceinline__ void issue_stage(const GemmCtx &c, int ks, int g, int slot, int wave, uint4 (&bq)[2],
                                            uint32_t (&sw)[2]) {
    uint8_t *sa = c.ring[slot];
    const uint8_t *ab = c.a_base + (size_t)ks * (KS * 2);  // uniform part of the addresses
#pragma unroll
    for (int i = 0; i < MS; ++i)
        __builtin_amdgcn_global_load_lds((const void *)(ab + c.a_off[i]),
                                         (__attribute__((address_space(3))) void *)(sa + (i * 4 + wave) * 1024),
                                         16, 0, 0);
#pragma unroll
    for (int ns = 0; ns < 2; ++ns)
        bq[ns] = *reinterpret_cast<const uint4 *>(c.b_base[ns] + (size_t)ks * c.b_kstep + c.b_off[ns]);
#pragma unroll
    for (int ns = 0; ns < 2; ++ns)
        sw[ns] = *reinterpret_cast<const uint32_t *>(
            c.s_base[ns] + ((c.s_off[ns] + (uint32_t)ks * c.s_kstep + (uint32_t)g * c.s_step) & ~3u));
}

// Main loop over K for a tile of MS x 32 rows.
template <int FMT, int MS>
__device__ __forceinline__ void gemm_main(const GemmCtx &c, f32x16_t (&acc)[4][2], int wave, int lane) {
    // K elements per scale word of the ring (NVFP4: one word of four E4M3
    // block scales per weight row and K-step)
    constexpr int G = FMT == 0 || FMT == 3 ? 64 : 128;
    constexpr int KPG = G / KS;
    constexpr int LPS = MS + 4;          // loads per thread and stage
    constexpr int D = ring_depth<MS>();  // stages in flight for this tile height
    static_assert(D >= 3 && (D - 2) * LPS <= 63, "wait counts fit vmcnt");
    const int l32 = lane & 31, hf = lane >> 5;
    const int NK = c.nk;
    uint4 bq[D][2];      // per stage: the lane's codes of its two weight rows
    uint32_t sw[D][2];   // per stage: their scale words

    // Every step issues one stage, the steps past the end the last K-step
    // again (never consumed), so that D - 1 stages are always in flight: one
    // wait count for all steps, and no loads on conditional paths in the loop.
#pragma unroll
    for (int u = 0; u < D - 1; ++u) {
        const int kn = u < NK ? u : NK - 1;
        issue_stage<MS>(c, kn, kn / KPG, u, wave, bq[u], sw[u]);
    }

    // per N-subtile: scale and min of the current group, for the 1024 + q
    // pairs (index 0) and the 1024 + 16 q pairs (index 1)
    half2_t s2[2][2], m2[2];
    uint32_t nvs[2][2];  // NVFP4: the lane's two block scales of the K-step, as f16 pairs (s, s)
    const uint32_t kf = opaque_magic(MAGIC_F16);
    const half2_t off0 = {(_Float16)(FMT == 0 ? 1024.0f : 1032.0f), (_Float16)(FMT == 0 ? 1024.0f : 1032.0f)};
    const half2_t off1 = {(_Float16)(FMT == 0 ? 1024.0f : 1152.0f), (_Float16)(FMT == 0 ? 1024.0f : 1152.0f)};
    const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    // K-step ks from ring slot u (a constant once the callers' loops unroll)
    auto step = [&](int ks, int u) __attribute__((always_inline)) {
        wait_stages<LPS>(D - 2);  // K-step ks has landed: only the D - 2 stages issued after it are in flight
        lds_barrier();            // every wave's share of ks is in LDS; slot (u + D - 1) % D is free
        const int kn = ks + D - 1 < NK ? ks + D - 1 : NK - 1;
        issue_stage<MS>(c, kn, kn / KPG, (u + D - 1) % D, wave, bq[(u + D - 1) % D], sw[(u + D - 1) % D]);
        const uint8_t *sa = c.ring[u];
        // GEMM2: this 128-input block's factor 2^(s_min - s_b), folded into the weights
        const float fbk = c.fb ? c.fb[ks >> 1] : 1.0f;
        if (FMT == 3) {
#pragma unroll
            for (int ns = 0; ns < 2; ++ns) {
                // blocks 2 hf and 2 hf + 1 of the K-step: k in [32 hf, 32 hf + 32)
                const uint32_t pw = sw[u][ns] >> (16 * hf);
                const uint32_t sp =
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(pw, fbk, false));
                nvs[ns][0] = (sp & 0xffffu) * 0x10001u;
                nvs[ns][1] = (sp >> 16) * 0x10001u;
            }
        } else if (ks % KPG == 0) {
#pragma unroll
            for (int ns = 0; ns < 2; ++ns) {
                const uint32_t pw = sw[u][ns];
                if (FMT == 0) {
                    uint32_t sb = pw & 0xffffu, mb = pw >> 16;
                    if (c.lift_rt) {
                        sb = __builtin_bit_cast(uint16_t, __builtin_ldexpf16(__builtin_bit_cast(_Float16, (uint16_t)sb),
                                                                             c.lexp[ns]));
                        mb = __builtin_bit_cast(uint16_t, __builtin_ldexpf16(__builtin_bit_cast(_Float16, (uint16_t)mb),
                                                                             c.lexp[ns]));
                    }
                    s2[ns][0] = __builtin_bit_cast(half2_t, sb * 0x10001u);
                    m2[ns] = __builtin_bit_cast(half2_t, mb * 0x10001u);
                } else {
                    uint32_t h = ((c.spar[ns] + (uint32_t)(ks / KPG)) & 1u) ? pw >> 16 : pw & 0xffffu;
                    if (c.lift_rt)
                        h = __builtin_bit_cast(uint16_t, __builtin_ldexpf16(__builtin_bit_cast(_Float16, (uint16_t)h),
                                                                            c.lexp[ns]));
                    s2[ns][0] = __builtin_bit_cast(half2_t, h * 0x10001u);
                    m2[ns] = s2[ns][0];
                }
                if (c.fb) {
                    const half2_t f2 = {(_Float16)fbk, (_Float16)fbk};
                    s2[ns][0] = s2[ns][0] * f2;
                    m2[ns] = m2[ns] * f2;
                }
                s2[ns][1] = s2[ns][0] * sixteenth;
            }
        }
        // B: 16 bytes (32 codes) of each of this lane's two weight rows
        const uint4 *bw = bq[u];
#pragma unroll
        for (int s = 0; s < 4; ++s) {  // matrix-core K-steps of 16: elements [32 hf + 8 s, +8) per lane
            u32x4_t bv[2];
#pragma unroll
            for (int ns = 0; ns < 2; ++ns) {
                const uint32_t word = s == 0 ? bw[ns].x : s == 1 ? bw[ns].y : s == 2 ? bw[ns].z : bw[ns].w;
                if constexpr (FMT == 3) {
                    // E2M1 pairs in natural order times the block scale: exact in f16
                    const half2_t sc = __builtin_bit_cast(half2_t, nvs[ns][s >> 1]);
                    auto nv = [&](uint32_t p) {
                        return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, p) * sc);
                    };
                    bv[ns] = u32x4_t{
                        nv(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 0))),
                        nv(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 1))),
                        nv(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 2))),
                        nv(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 3)))};
                } else {
                    const uint32_t w8 = word >> 8;
                    bv[ns] = u32x4_t{
                        dequant_pair<FMT>(insert_codes<0x000f000fu>(word, kf), off0, s2[ns][0], m2[ns]),
                        dequant_pair<FMT>(insert_codes<0x00f000f0u>(word, kf), off1, s2[ns][1], m2[ns]),
                        dequant_pair<FMT>(insert_codes<0x000f000fu>(w8, kf), off0, s2[ns][0], m2[ns]),
                        dequant_pair<FMT>(insert_codes<0x00f000f0u>(w8, kf), off1, s2[ns][1], m2[ns])};
                }
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
    };
    int kk = 0;
    for (; kk + D <= NK; kk += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) step(kk + u, u);
    }
#pragma unroll
    for (int u = 0; u < D - 1; ++u)
        if (kk + u < NK) step(kk + u, u);
    MOEQ4_WAIT_VM_LDS(0);  // the stages issued past the end have landed before the ring is reused
}

// The largest of the workgroup's non-negative values v (one per thread), in
// every thread (a barrier; s_red: 4 words of LDS).
__device__ __forceinline__ float block_max_nonneg(float v, uint32_t *s_red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t w = wave_max_u32(__float_as_uint(v));  // non-negative floats order as their bits
    if (lane == 0) s_red[wave] = w;
    __syncthreads();
    uint32_t m = s_red[0];
#pragma unroll
    for (int i = 1; i < PF_BLOCK / 64; ++i) m = m > s_red[i] ? m : s_red[i];
    return __uint_as_float(m);
}

// The largest f16 magnitude (as bits) among an int4 weight row's scales and
// mins in the canonical scale array: asym [NG] words {scale, min}, sym [NG]
// scales.
template <int FMT>
__device__ __forceinline__ uint32_t canonical_row_max(const uint16_t *__restrict__ sm, size_t row, int NG) {
    uint32_t a = 0u;
    if (FMT == 0) {
        const uint32_t *w = reinterpret_cast<const uint32_t *>(sm) + row * NG;
        for (int i = 0; i < NG; ++i) {
            const uint32_t v = w[i], lo = v & 0x7fffu, hi = (v >> 16) & 0x7fffu;
            a = lo > a ? lo : a;
            a = hi > a ? hi : a;
        }
    } else {
        const uint16_t *h = sm + row * NG;
        for (int i = 0; i < NG; ++i) {
            const uint32_t v = h[i] & 0x7fffu;
            a = v > a ? v : a;
        }
    }
    return a;
}

// STAGE 1: A = x16 rows gathered through perm, B = gate | up codes,
//          epilogue SwiGLU of the accumulators times 2^e(token) -> h (f16,
//          scaled per row and per block as described at the epilogue).
// STAGE 2: A = h rows (contiguous sorted rows), B = down codes,
//          epilogue gate-weighted rows of z (f16, scaled the same way) for
//          the combine kernel.
// Work items are (tile, column block).  Workgroups are spread over the 8 XCDs
// round-robin (XCD = block index mod 8).  Tile rank t of the schedule `order`
// (largest tiles first; null: the tile list's own order) goes to XCD t % 8,
// where its column blocks run one after another (same A rows in one L2).
// Each XCD so starts with its largest tiles and gets an even share of them,
// and the small tiles fill the end of the launch.
// In the ring, A row r (128 bytes per stage) holds its 16-byte chunk c at
// c ^ ((r >> 1) & 7) and B row rb (32 bytes) at c ^ ((rb >> 3) & 1), so that
// the fragment reads of 16 lanes hit distinct LDS banks.
// ONE: each workgroup takes one 32-row subtile of a tile (the subtiles of a
// tile on one XCD, one after another), in a build for single subtiles only:
// a third of the LDS and the registers of one subtile, three workgroups per
// CU for GEMM1 and four for GEMM2 (128 VGPRs, no spills; four for GEMM1 as
// well made the NVFP4 GEMM1 slower).  The host takes it when tiles are
// mostly single subtiles.
template <int FMT, int STAGE, bool ONE>
__global__ __launch_bounds__(PF_BLOCK) __attribute__((amdgpu_waves_per_eu(ONE ? (STAGE == 2 ? 4 : 3) : 2,
                                                                          ONE ? (STAGE == 2 ? 4 : 3) : 2))) void grouped_gemm_kernel(
    const uint16_t *__restrict__ act,      // STAGE 1: x16 [T][H]; STAGE 2: h [P][I]
    const int32_t *__restrict__ xexp,      // STAGE 1: per-token exponent e
    int H, int I, int k, LayerPtrs L, const Tile *__restrict__ tiles, const int32_t *__restrict__ ntiles,
    const int32_t *__restrict__ perm, const float *__restrict__ topk_gate,
    uint16_t *__restrict__ h_out, uint16_t *__restrict__ z, const int32_t *__restrict__ order,
    int8_t *__restrict__ hx,   // h's exponent per row and 128-column block: STAGE 1 writes, STAGE 2 reads
    int8_t *__restrict__ zx) { // STAGE 2: z's exponent per row and 64 columns
    constexpr int G = FMT == 0 || FMT == 3 ? 64 : 128;  // K elements per scale word (see gemm_main)

    const int ncb = STAGE == 1 ? I / 128 : H / BROWS;
    constexpr int MSPLIT = ONE ? BM / 32 : 1;  // workgroups per tile and column block
    const int bx = blockIdx.x, local = bx / 8;
    const int t = (local / (ncb * MSPLIT)) * 8 + bx % 8;  // rank in the schedule
    if (t >= *ntiles) return;
    const int cb = local % ncb;
    const int j = order ? order[t] : t;
    const Tile tile = tiles[j];
    const int e = tile.expert;
    int rows = tile.rows, row0 = tile.row0;
    if constexpr (ONE) {
        const int m = (local / ncb) % MSPLIT;  // the subtile
        if (32 * m >= rows) return;
        row0 += 32 * m;
        rows = rows - 32 * m < 32 ? rows - 32 * m : 32;
    }
    const int K = STAGE == 1 ? H : I;
    const int NG = K / G;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS slot addresses stay scalar
    const int l32 = lane & 31, hf = lane >> 5;
    const int col_base = cb * (STAGE == 1 ? 128 : BROWS);

    __shared__ __attribute__((aligned(16))) uint8_t s_ring0[RSLOT_BIG];
    __shared__ __attribute__((aligned(16))) uint8_t s_ring1[ONE ? RSLOT4 : RSLOT_BIG];
    __shared__ __attribute__((aligned(16))) uint8_t s_ring2[ONE ? RSLOT4 : RSLOT_BIG];
    __shared__ __attribute__((aligned(16))) uint8_t s_ring3[ONE ? RSLOT4 : RSLOT3];
    __shared__ __attribute__((aligned(16))) uint8_t s_ring4[RSLOT4];
    __shared__ int s_tok[BM];
    __shared__ float s_rs[BM];  // STAGE 1: 2^e of the row's token; STAGE 2: the row's gate times 2^-s_min
    __shared__ float s_ri[BM];  // STAGE 1: 2^-e
    __shared__ float s_fb[16];  // STAGE 2: 2^(s_min - s_b) per 128-input block b of h
    __shared__ uint32_t s_red[PF_BLOCK / 64];
    const int nbh = I / 128;    // h blocks of 128 (<= 16)

    // STAGE 2: the exponents of h's blocks are the same for all the rows of
    // this workgroup (they were scaled by one GEMM1 workgroup per block)
    int smin = 64;
    if (STAGE == 2 && tid < BM)
        for (int b = 0; b < nbh; ++b) {
            const int sb = hx[(size_t)row0 * nbh + b];
            smin = sb < smin ? sb : smin;
        }
    if (STAGE == 2 && tid < nbh) s_fb[tid] = exp2i(smin - (int)hx[(size_t)row0 * nbh + tid]);
    if (tid < BM) {
        int t = 0;
        float v = 0.f, vi = 0.f;
        if (tid < rows) {
            const int p = perm[row0 + tid];
            t = p / k;
            v = STAGE == 2 ? topk_gate[p] * exp2i(-smin) : ldexpf(1.0f, xexp[t]);
            vi = STAGE == 2 ? 0.f : ldexpf(1.0f, -xexp[t]);
            if (FMT == 3) {  // NVFP4 global scale (gate and up share theirs)
                const float gs = L.glob[2 * e + (STAGE == 2 ? 1 : 0)];
                v *= gs;
                vi *= gs;
            }
        }
        s_tok[tid] = t;
        s_rs[tid] = v;
        s_ri[tid] = vi;
    }
    __syncthreads();

    GemmCtx c;
    c.ring[0] = s_ring0;
    c.ring[1] = s_ring1;
    c.ring[2] = s_ring2;
    c.ring[3] = s_ring3;
    c.ring[4] = s_ring4;
    c.nk = K / KS;
    c.a_base = reinterpret_cast<const uint8_t *>(act);
    // A slot S = (i * 4 + wave) * 64 + lane (16 bytes): row S / 8 = 32 i + 8 wave + lane / 8,
    // stored chunk S % 8 holding logical chunk (S % 8) ^ ((row >> 1) & 7).
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 32 * i + 8 * wave + (lane >> 3);
        const int ch = (lane & 7) ^ ((r >> 1) & 7);
        const int rr = r < rows ? r : 0;  // padding rows read row 0; their outputs are dropped
        const uint32_t arow = STAGE == 1 ? (uint32_t)s_tok[rr] * (uint32_t)H : (uint32_t)(row0 + rr) * (uint32_t)I;
        c.a_off[i] = (arow + 8u * ch) * 2u;
    }
    // B: lane (l32, hf) takes, of N-subtile ns, weight row brow[ns] (block
    // rows 0-127 gate, 128-255 up in GEMM1) and per K-step the half hf of its
    // 32 code bytes, with the row's scale word.
    const uint32_t row_bytes = (uint32_t)K / 2;
    const uint32_t esz = FMT == 0 || FMT == 3 ? 4u : 2u;
    const PackLayout pl = pack_layout(L.E, H, I, FMT);
    const size_t tix = (size_t)e * ncb + cb;  // the tile's index in the copy
    float lf[2] = {1.f, 1.f};                 // the output columns' 2^-L
    c.lift_rt = (FMT == 0 || FMT == 1) && !L.pack;
#pragma unroll
    for (int ns = 0; ns < 2; ++ns) {
        const int rb = STAGE == 1 ? ns * 128 + wave * 32 + l32 : wave * 64 + ns * 32 + l32;
        c.brow[ns] = rb;
        const uint32_t wrow = STAGE == 1 ? (uint32_t)e * I + col_base + (rb & 127) : (uint32_t)e * H + col_base + rb;
        c.spar[ns] = (wrow * (uint32_t)NG) & 1u;
        c.lexp[ns] = 0;
        if (FMT == 0 || FMT == 1) {
            int lift;
            if (L.pack) {
                lift = (int)(int8_t)L.pack[(STAGE == 1 ? pl.gu_l : pl.d_l) + tix * BROWS + rb];
            } else {
                const uint16_t *sm = STAGE == 1 ? (ns == 0 ? L.gsm : L.usm) : L.dsm;
                lift = row_lift_from_max(canonical_row_max<FMT == 0 ? 0 : 1>(sm, wrow, NG));
            }
            c.lexp[ns] = lift;
            lf[ns] = exp2i(-lift);
        }
        if (L.pack) {
            // prefill copy: per K-step, tile (e, cb) holds its 256 rows' 32-byte
            // chunks in row order (halves swapped when bit 3 of the row is set),
            // then their scale words in row order
            c.b_base[ns] = L.pack + (STAGE == 1 ? pl.gu_q : pl.d_q) + tix * (size_t)c.nk * B_BYTES;
            c.b_off[ns] = (uint32_t)rb * 32u + 16u * (uint32_t)(hf ^ ((rb >> 3) & 1));
            c.s_base[ns] = L.pack + (STAGE == 1 ? pl.gu_s : pl.d_s) + tix * (size_t)c.nk * S_BYTES;
            c.s_off[ns] = 4u * (uint32_t)rb;
        } else {
            c.b_base[ns] = STAGE == 1 ? (ns == 0 ? L.gq : L.uq) : L.dq;
            c.b_off[ns] = wrow * row_bytes + 16u * (uint32_t)hf;
            c.s_base[ns] = reinterpret_cast<const uint8_t *>(STAGE == 1 ? (ns == 0 ? L.gsm : L.usm) : L.dsm);
            c.s_off[ns] = wrow * (uint32_t)NG * esz;
        }
    }
    c.b_kstep = L.pack ? B_BYTES : KS / 2;
    c.s_step = L.pack ? 0u : esz;
    c.s_kstep = L.pack ? S_BYTES : 0u;
    c.fb = STAGE == 2 ? s_fb : nullptr;

    f32x16_t acc[4][2];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ns = 0; ns < 2; ++ns)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][ns][r] = 0.f;
    const int msub = ONE ? 1 : (rows + 31) / 32;
    switch (msub) {
        case 1: gemm_main<FMT, 1>(c, acc, wave, lane); break;
        case 2: gemm_main<FMT, 2>(c, acc, wave, lane); break;
        case 3: gemm_main<FMT, 3>(c, acc, wave, lane); break;
        default: gemm_main<FMT, 4>(c, acc, wave, lane); break;
    }
    __syncthreads();  // ring no longer read: the epilogue may reuse it

    // ---- epilogue: values in the unit that their f16 rounding uses (h:
    // per row h 2^-2e; z: per row z 2^-2e = g 2^-s_min acc), times the power
    // of two 2^s that puts their largest magnitude in [2^14, 2^15)
    // (row_scale), one 32-row subtile at a time through ring slots 0-2 in
    // turn (a slot is written again only after two more barriers): f16 in
    // LDS, then coalesced 16-byte stores.  h takes one s for the
    // workgroup's 128 columns of all its rows (GEMM2 folds it into its
    // weights, so it must be uniform over a GEMM2 workgroup's rows); z one s
    // per subtile and wave (64 columns), stored per row for the combine.
    // Accumulator element r of lane (l32, hf) in M-subtile mi is row
    // 32 mi + 8 (r / 4) + 4 hf + (r % 4), column l32 of the subtile.
    __shared__ int s_zs[4][PF_BLOCK / 64];
    RowScale rs{1.0f, 0};
    if (STAGE == 1) {
        float mloc = 0.f;
#pragma unroll
        for (int mi = 0; mi < (ONE ? 1 : 4); ++mi) {
            if (mi >= msub) break;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lr = 32 * mi + 8 * (r / 4) + 4 * hf + (r % 4);
                // h 2^-2e = silu(a) (b 2^-2e) with a = acc 2^e and b 2^-2e = acc 2^-e
                const float hn = silu(acc[mi][0][r] * s_rs[lr] * lf[0]) * (acc[mi][1][r] * s_ri[lr] * lf[1]);
                acc[mi][0][r] = hn;
                mloc = fmaxf(mloc, fabsf(hn));
            }
        }
        rs = row_scale(block_max_nonneg(mloc, s_red));
    }
#pragma unroll
    for (int mi = 0; mi < (ONE ? 1 : 4); ++mi) {
        if (mi >= msub) break;
        uint16_t *s_t = reinterpret_cast<uint16_t *>(mi % 3 == 0 ? s_ring0 : mi % 3 == 1 ? s_ring1 : s_ring2);
        if (STAGE == 1) {
            // h rows [32][128] f16 in LDS, then coalesced 16-byte stores in PERM8 order
            constexpr int HP = 128 + 8;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lr = 8 * (r / 4) + 4 * hf + (r % 4);
                s_t[lr * HP + wave * 32 + l32] = __builtin_bit_cast(uint16_t, (_Float16)(acc[mi][0][r] * rs.sc));
            }
            __syncthreads();
            for (int i = tid; i < 32 * 16; i += PF_BLOCK) {
                const int lr = i / 16, cc = i % 16, row = 32 * mi + lr;
                if (row < rows) {
                    const uint4 v = *reinterpret_cast<const uint4 *>(&s_t[lr * HP + cc * 8]);
                    uint4 o = v;
                    if (FMT != 3) perm8(v.x, v.y, v.z, v.w, o.x, o.y, o.z, o.w);
                    *reinterpret_cast<uint4 *>(h_out + (size_t)(row0 + row) * I + cb * 128 + cc * 8) = o;
                    if (cc == 0) hx[(size_t)(row0 + row) * nbh + cb] = (int8_t)rs.s;
                }
            }
        } else {
            // z rows [32][256] f16 in LDS (this wave's 64 columns with their own s), then coalesced 16-byte stores
            constexpr int ZP = BROWS + 8;
            float mloc = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lr = 32 * mi + 8 * (r / 4) + 4 * hf + (r % 4);
#pragma unroll
                for (int ns = 0; ns < 2; ++ns) {
                    const float zn = acc[mi][ns][r] * s_rs[lr] * lf[ns];
                    acc[mi][ns][r] = zn;
                    mloc = fmaxf(mloc, fabsf(zn));
                }
            }
            const RowScale zs = row_scale(__uint_as_float(wave_max_u32(__float_as_uint(mloc))));
            if (lane == 0) s_zs[mi][wave] = zs.s;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lr = 8 * (r / 4) + 4 * hf + (r % 4);
                s_t[lr * ZP + wave * 64 + l32] = __builtin_bit_cast(uint16_t, (_Float16)(acc[mi][0][r] * zs.sc));
                s_t[lr * ZP + wave * 64 + 32 + l32] = __builtin_bit_cast(uint16_t, (_Float16)(acc[mi][1][r] * zs.sc));
            }
            __syncthreads();
            for (int i = tid; i < 32 * (BROWS / 8); i += PF_BLOCK) {
                const int lr = i / (BROWS / 8), cc = i % (BROWS / 8), row = 32 * mi + lr;
                if (row < rows) {
                    *reinterpret_cast<uint4 *>(z + (size_t)(row0 + row) * H + col_base + cc * 8) =
                        *reinterpret_cast<const uint4 *>(&s_t[lr * ZP + cc * 8]);
                    if ((cc & 7) == 0) zx[(size_t)(row0 + row) * (H / 64) + (col_base + cc * 8) / 64] = (int8_t)s_zs[mi][cc >> 3];
                }
            }
        }
    }
}

// ------------------------------------------------------- block-FP8 GEMMs
//
// The same grouped GEMMs for block-FP8 experts (E4M3 codes, one float32
// scale per 128 weight rows x 128 inputs; the released experts' format,
// drama-3-w4a16 card "At a glance", each matrix dequantised with its block
// scales, "How it was made").  Codes are converted to 16-bit floats exactly
// (two per gfx950 conversion instruction; every E4M3 value is a bf16 and an
// f16), so both operands of the matrix cores are exact:
//   GEMM1: A = the token's bf16 x row itself (no f16 pass), B = codes as
//          bf16, bf16 MFMA;
//   GEMM2: A = h (f16), B = codes as f16, f16 MFMA.
// Block scales.  A wave's 32 output columns of an N-subtile lie in one
// 128-row block, so its scale is uniform over the subtile for each 128-input
// block of K.  The accumulator carries sum_b s_b P_b / sigma, sigma the last
// nonzero block scale met: at each K-block with scale s != 0 it is multiplied
// by sigma / s (rounded once) before the block's products, and by sigma at
// the end.  An all-zero block (scale 0, codes 0) adds nothing.
// Tiles and work order are as above.  Both the A rows and the codes (64
// bytes per weight row and K-step, from the prefill copy when there is one)
// go through a two-stage LDS ring, one array per slot (two workgroups per
// CU); each wave's block scales along K sit in a small LDS array of their own.

constexpr int NST8 = 2;
constexpr int B8_BYTES = BROWS * KS;             // 16 KB: 256 rows x 64 codes
constexpr int STAGE8_BYTES = A_BYTES + B8_BYTES;
constexpr int B8_LOADS = B8_BYTES / 16 / PF_BLOCK;  // 4 sixteen-byte loads per thread and stage
constexpr int ZP8 = BROWS + 8;
static_assert(32 * ZP8 * 2 <= STAGE8_BYTES, "32 epilogue rows fit a ring slot");

typedef __bf16 bf16x8v_t __attribute__((ext_vector_type(8)));

struct Gemm8Ctx {
    const uint8_t *a_base;
    uint32_t a_off[4];
    const uint8_t *b_base[B8_LOADS];
    uint32_t b_off[B8_LOADS];
    uint32_t b_kstep;    // bytes between K-steps of a weight row chunk
    const float *sc;     // LDS: block scales of this wave's two N-subtiles, [2][16] (one per 128 inputs)
    uint8_t *ring[NST8]; // the ring slots, one LDS array each (see ring_depth)
    int brow[2];
    int nk;
};

template <int MS>
__device__ __forceinline__ void issue_stage8(const Gemm8Ctx &c, int ks, int slot, int wave) {
    uint8_t *sa = c.ring[slot];
    uint8_t *sb = sa + A_BYTES;
    const uint8_t *ab = c.a_base + (size_t)ks * (KS * 2);
#pragma unroll
    for (int i = 0; i < MS; ++i)
        __builtin_amdgcn_global_load_lds((const void *)(ab + c.a_off[i]),
                                         (__attribute__((address_space(3))) void *)(sa + (i * 4 + wave) * 1024),
                                         16, 0, 0);
#pragma unroll
    for (int i = 0; i < B8_LOADS; ++i)
        __builtin_amdgcn_global_load_lds((const void *)((c.b_base[i] + (size_t)ks * c.b_kstep) + c.b_off[i]),
                                         (__attribute__((address_space(3))) void *)(sb + (i * 4 + wave) * 1024),
                                         16, 0, 0);
}

// Four codes of a dword as four exact 16-bit floats (bf16 for GEMM1, f16 for
// GEMM2), in order.
template <int STAGE>
__device__ __forceinline__ uint2 e4m3x4(uint32_t w) {
    if (STAGE == 1)
        return make_uint2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)));
    return make_uint2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true)));
}

template <int STAGE, int MS>
__device__ __forceinline__ void gemm8_main(const Gemm8Ctx &c, f32x16_t (&acc)[4][2], int wave, int lane) {
    constexpr int LPS = MS + B8_LOADS;  // loads per thread and stage
    const int l32 = lane & 31, hf = lane >> 5;
    const int NK = c.nk;
#pragma unroll
    for (int u = 0; u < NST8 - 1; ++u)
        if (u < NK) issue_stage8<MS>(c, u, u, wave);
    float sig[2] = {1.f, 1.f};
    float snext[2] = {c.sc[0], c.sc[16]};
    for (int kk = 0; kk < NK; kk += NST8) {
#pragma unroll
        for (int u = 0; u < NST8; ++u) {
            const int ks = kk + u;
            if (ks < NK) {
                // stage ks has landed once only the stages issued after it are in flight
                if (NST8 > 2 && ks + 1 < NK) MOEQ4_WAIT_VM_LDS(LPS);
                else MOEQ4_WAIT_VM_LDS(0);
                lds_barrier();
                if (ks + NST8 - 1 < NK) issue_stage8<MS>(c, ks + NST8 - 1, (u + NST8 - 1) % NST8, wave);
                if ((ks & 1) == 0) {  // a new 128-input block
                    const int kb = ks >> 1;
#pragma unroll
                    for (int ns = 0; ns < 2; ++ns) {
                        const float sb = snext[ns];
                        if (sb != 0.f) {
                            if (kb > 0) {
                                const float r = sig[ns] / sb;
#pragma unroll
                                for (int mi = 0; mi < MS; ++mi)
#pragma unroll
                                    for (int q = 0; q < 16; ++q) acc[mi][ns][q] *= r;
                            }
                            sig[ns] = sb;
                        }
                        if (2 * (kb + 1) < NK) snext[ns] = c.sc[16 * ns + kb + 1];
                    }
                }
                const uint8_t *sa = c.ring[u];
                const uint8_t *sbp = sa + A_BYTES;
                // B: the lane's 32 codes (k in [32 hf, 32 hf + 32)) of each of its two weight rows
                uint4 bw[2][2];
#pragma unroll
                for (int ns = 0; ns < 2; ++ns) {
                    const int rb = c.brow[ns];
#pragma unroll
                    for (int t = 0; t < 2; ++t)
                        bw[ns][t] = *reinterpret_cast<const uint4 *>(sbp + rb * 64 + 16 * ((2 * hf + t) ^ ((rb >> 2) & 3)));
                }
#pragma unroll
                for (int s = 0; s < 4; ++s) {  // matrix-core K-steps of 16: elements [32 hf + 8 s, +8) per lane
                    u32x4_t bv[2];
#pragma unroll
                    for (int ns = 0; ns < 2; ++ns) {
                        const uint4 v = bw[ns][s >> 1];
                        const uint32_t d0 = (s & 1) ? v.z : v.x, d1 = (s & 1) ? v.w : v.y;
                        const uint2 p0 = e4m3x4<STAGE>(d0), p1 = e4m3x4<STAGE>(d1);
                        bv[ns] = u32x4_t{p0.x, p0.y, p1.x, p1.y};
                    }
                    const int ch = 4 * hf + s;
#pragma unroll
                    for (int mi = 0; mi < MS; ++mi) {
                        const int r = 32 * mi + l32;
                        const uint4 av = *reinterpret_cast<const uint4 *>(sa + r * 128 + 16 * (ch ^ ((r >> 1) & 7)));
                        const u32x4_t a4 = u32x4_t{av.x, av.y, av.z, av.w};
#pragma unroll
                        for (int ns = 0; ns < 2; ++ns) {
                            if (STAGE == 1)
                                acc[mi][ns] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                    __builtin_bit_cast(bf16x8v_t, a4), __builtin_bit_cast(bf16x8v_t, bv[ns]),
                                    acc[mi][ns], 0, 0, 0);
                            else
                                acc[mi][ns] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                                    __builtin_bit_cast(f16x8_t, a4), __builtin_bit_cast(f16x8_t, bv[ns]),
                                    acc[mi][ns], 0, 0, 0);
                        }
                    }
                }
            }
        }
    }
#pragma unroll
    for (int mi = 0; mi < MS; ++mi)
#pragma unroll
        for (int ns = 0; ns < 2; ++ns)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[mi][ns][q] *= sig[ns];
}

// STAGE 1: A = x rows (bf16) gathered through perm, B = gate | up codes,
//          epilogue SwiGLU -> h (f16, natural order).
// STAGE 2: A = h rows, B = down codes, epilogue gate-weighted rows of z (f16).
template <int STAGE>
__global__ __launch_bounds__(PF_BLOCK) __attribute__((amdgpu_waves_per_eu(2, 2))) void grouped_gemm_fp8_kernel(
    const uint16_t *__restrict__ act, int H, int I, int k, LayerPtrs L, const Tile *__restrict__ tiles,
    const int32_t *__restrict__ ntiles, const int32_t *__restrict__ perm, const float *__restrict__ topk_gate,
    uint16_t *__restrict__ h_out, uint16_t *__restrict__ z, const int32_t *__restrict__ order,
    int8_t *__restrict__ hx, int8_t *__restrict__ zx,  // exponents of h and z, as grouped_gemm_kernel
    const int32_t *__restrict__ xexp) {                 // STAGE 1: the per-token exponent e
    const int ncb = STAGE == 1 ? I / 128 : H / BROWS;
    const int bx = blockIdx.x, local = bx / 8;
    const int t = (local / ncb) * 8 + bx % 8;  // rank in the schedule (as grouped_gemm_kernel)
    if (t >= *ntiles) return;
    const int cb = local % ncb;
    const int j = order ? order[t] : t;
    const Tile tile = tiles[j];
    const int e = tile.expert, rows = tile.rows, row0 = tile.row0;
    const int K = STAGE == 1 ? H : I;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hf = lane >> 5;
    const int col_base = cb * (STAGE == 1 ? 128 : BROWS);

    __shared__ __attribute__((aligned(16))) uint8_t s_ring0[STAGE8_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t s_ring1[STAGE8_BYTES];
    __shared__ float s_sc8[4][2][16];  // per wave and N-subtile: the block scales along K (K <= 2048)
    __shared__ int s_tok[BM];
    __shared__ float s_gt[BM];  // STAGE 1: 2^-e of the row's token (0 for padding rows); STAGE 2: gate 2^-s_min
    __shared__ float s_fb[16];  // STAGE 2: 2^(s_min - s_b) per 128-input block b of h
    __shared__ uint32_t s_red[PF_BLOCK / 64];
    const int nbh = I / 128;
    int smin = 64;  // as grouped_gemm_kernel
    if (STAGE == 2 && tid < BM)
        for (int b = 0; b < nbh; ++b) {
            const int sb = hx[(size_t)row0 * nbh + b];
            smin = sb < smin ? sb : smin;
        }
    if (STAGE == 2 && tid < nbh) s_fb[tid] = exp2i(smin - (int)hx[(size_t)row0 * nbh + tid]);
    if (tid < BM) {
        int t = 0;
        float v = 0.f;
        if (tid < rows) {
            const int p = perm[row0 + tid];
            t = p / k;
            v = STAGE == 2 ? topk_gate[p] * exp2i(-smin) : exp2i(-xexp[t]);
        }
        s_tok[tid] = t;
        s_gt[tid] = v;
    }
    __syncthreads();

    Gemm8Ctx c;
    c.ring[0] = s_ring0;
    c.ring[1] = s_ring1;
    c.nk = K / KS;
    c.a_base = reinterpret_cast<const uint8_t *>(act);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 32 * i + 8 * wave + (lane >> 3);
        const int ch = (lane & 7) ^ ((r >> 1) & 7);
        const int rr = r < rows ? r : 0;  // padding rows read row 0; their outputs are dropped
        const uint32_t arow = STAGE == 1 ? (uint32_t)s_tok[rr] * (uint32_t)H : (uint32_t)(row0 + rr) * (uint32_t)I;
        c.a_off[i] = (arow + 8u * ch) * 2u;
    }
    // B slot S: weight row rb = S / 4 (rows 0-127 gate, 128-255 up in GEMM1),
    // stored chunk S % 4 holding logical chunk (S % 4) ^ ((rb >> 2) & 3).
#pragma unroll
    for (int i = 0; i < B8_LOADS; ++i) {
        const int S = (i * 4 + wave) * 64 + lane;
        const int rb = S / 4, ch = (S % 4) ^ ((rb >> 2) & 3);
        uint32_t wrow;
        if (STAGE == 1) {
            c.b_base[i] = i < 2 ? L.gq : L.uq;  // slots of loads 0-1 are rows 0-127, of loads 2-3 rows 128-255
            wrow = (uint32_t)e * I + col_base + (rb & 127);
        } else {
            c.b_base[i] = L.dq;
            wrow = (uint32_t)e * H + col_base + rb;
        }
        c.b_off[i] = wrow * (uint32_t)K + 16u * ch;
    }
    c.b_kstep = KS;
    if (L.pack) {
        // prefill copy: per K-step, tile (e, cb) holds its 256 rows' 64-byte chunks in slot order
        const PackLayout pl = pack_layout(L.E, H, I, 2);
        const uint8_t *q =
            L.pack + (STAGE == 1 ? pl.gu_q : pl.d_q) + ((size_t)e * ncb + cb) * (size_t)c.nk * B8_BYTES;
#pragma unroll
        for (int i = 0; i < B8_LOADS; ++i) {
            c.b_base[i] = q;
            c.b_off[i] = 16u * (uint32_t)((i * 4 + wave) * 64 + lane);
        }
        c.b_kstep = B8_BYTES;
    }
    const int nkb = K / 128;
#pragma unroll
    for (int ns = 0; ns < 2; ++ns) {
        c.brow[ns] = STAGE == 1 ? ns * 128 + wave * 32 + l32 : wave * 64 + ns * 32 + l32;
        // the subtile's 128-row block (GEMM1: ns 0 the gate rows, ns 1 the up rows)
        const int nrow = STAGE == 1 ? col_base : col_base + wave * 64 + ns * 32;
        const float *sbase = reinterpret_cast<const float *>(STAGE == 1 ? (ns == 0 ? L.gsm : L.usm) : L.dsm);
        const int N = STAGE == 1 ? I : H;
        // the wave's own copy in LDS: read in the loop without joining the
        // vector-memory count that orders the ring
        // GEMM2: each block's scale times the factor 2^(s_min - s_b) of h's block
        const int kb = lane & 15;
        if ((lane >> 4) == ns && kb < nkb)
            s_sc8[wave][ns][kb] =
                sbase[((size_t)e * (N / 128) + nrow / 128) * nkb + kb] * (STAGE == 2 ? s_fb[kb] : 1.0f);
    }
    c.sc = &s_sc8[wave][0][0];

    f32x16_t acc[4][2];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ns = 0; ns < 2; ++ns)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][ns][r] = 0.f;
    const int msub = (rows + 31) / 32;
    switch (msub) {
        case 1: gemm8_main<STAGE, 1>(c, acc, wave, lane); break;
        case 2: gemm8_main<STAGE, 2>(c, acc, wave, lane); break;
        case 3: gemm8_main<STAGE, 3>(c, acc, wave, lane); break;
        default: gemm8_main<STAGE, 4>(c, acc, wave, lane); break;
    }
    __syncthreads();  // ring no longer read: the epilogue may reuse it

    // epilogue as grouped_gemm_kernel's, one 32-row subtile at a time through
    // the two ring slots in turn.  x enters unscaled, so GEMM1 forms
    // h 2^-2e = (silu(acc) 2^-e) (acc_u 2^-e) here; GEMM2's z then carries
    // 2^-2e as well, which the combine takes off.
    __shared__ int s_zs[4][PF_BLOCK / 64];
    RowScale rs{1.0f, 0};
    if (STAGE == 1) {
        float mloc = 0.f;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            if (mi >= msub) break;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lr = 32 * mi + 8 * (r / 4) + 4 * hf + (r % 4);
                const float hv = (silu(acc[mi][0][r]) * s_gt[lr]) * (acc[mi][1][r] * s_gt[lr]);
                acc[mi][0][r] = hv;
                mloc = fmaxf(mloc, fabsf(hv));
            }
        }
        rs = row_scale(block_max_nonneg(mloc, s_red));
    }
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        if (mi >= msub) break;
        uint16_t *s_t = reinterpret_cast<uint16_t *>(mi % 2 == 0 ? s_ring0 : s_ring1);
        if (STAGE == 1) {
            constexpr int HP = 128 + 8;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lr = 8 * (r / 4) + 4 * hf + (r % 4);
                s_t[lr * HP + wave * 32 + l32] = __builtin_bit_cast(uint16_t, (_Float16)(acc[mi][0][r] * rs.sc));
            }
            __syncthreads();
            for (int i = tid; i < 32 * 16; i += PF_BLOCK) {
                const int lr = i / 16, cc = i % 16, row = 32 * mi + lr;
                if (row < rows) {
                    *reinterpret_cast<uint4 *>(h_out + (size_t)(row0 + row) * I + cb * 128 + cc * 8) =
                        *reinterpret_cast<const uint4 *>(&s_t[lr * HP + cc * 8]);
                    if (cc == 0) hx[(size_t)(row0 + row) * nbh + cb] = (int8_t)rs.s;
                }
            }
        } else {
            float mloc = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lr = 32 * mi + 8 * (r / 4) + 4 * hf + (r % 4);
#pragma unroll
                for (int ns = 0; ns < 2; ++ns) {
                    const float zn = acc[mi][ns][r] * s_gt[lr];
                    acc[mi][ns][r] = zn;
                    mloc = fmaxf(mloc, fabsf(zn));
                }
            }
            const RowScale zs = row_scale(__uint_as_float(wave_max_u32(__float_as_uint(mloc))));
            if (lane == 0) s_zs[mi][wave] = zs.s;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lr = 8 * (r / 4) + 4 * hf + (r % 4);
                s_t[lr * ZP8 + wave * 64 + l32] = __builtin_bit_cast(uint16_t, (_Float16)(acc[mi][0][r] * zs.sc));
                s_t[lr * ZP8 + wave * 64 + 32 + l32] = __builtin_bit_cast(uint16_t, (_Float16)(acc[mi][1][r] * zs.sc));
            }
            __syncthreads();
            for (int i = tid; i < 32 * (BROWS / 8); i += PF_BLOCK) {
                const int lr = i / (BROWS / 8), cc = i % (BROWS / 8), row = 32 * mi + lr;
                if (row < rows) {
                    *reinterpret_cast<uint4 *>(z + (size_t)(row0 + row) * H + col_base + cc * 8) =
                        *reinterpret_cast<const uint4 *>(&s_t[lr * ZP8 + cc * 8]);
                    if ((cc & 7) == 0) zx[(size_t)(row0 + row) * (H / 64) + (col_base + cc * 8) / 64] = (int8_t)s_zs[mi][cc >> 3];
                }
            }
        }
    }
}

// ------------------------------------------------- shared expert GEMMs
//
// The layer's shared expert (int8 symmetric, one f16 scale per 128 input
// weights; drama-q4 card, "What's quantized") for many tokens: the same two
// products as the routed experts over every token, as dense GEMMs on the f16
// matrix cores.  Tiles are 128 consecutive tokens x 256 weight rows (GEMM1:
// the gate and up rows of 128 h columns; GEMM2: 256 output columns), 4
// waves, the tile operand and the codes staged through a two-stage LDS ring
// (64 code bytes per weight row and K-step, as the FP8 GEMMs).
// Codes: the signed byte's top bit is flipped (u = q + 128) and two bytes
// are inserted into the f16 pair (1024, 1024); subtracting 1152 leaves q
// exactly, and one packed multiply by the row's group scale rounds s q once
// to f16 (as the int4 path rounds its weights).  A code dword gives the pairs
// (q0, q2) and (q1, q3), so x16 and h are kept in PERM4 order (0,2,1,3 in each
// group of 4).  x16 is x scaled per token by a power of two 2^-e
// (x_to_f16).  h is scaled as in the routed GEMM1: each row by 2^-2e, then
// the workgroup's 128 columns of its rows by the 2^s that puts their largest
// magnitude in [2^14, 2^15) (s stored per row and 128-column block in hx);
// GEMM2 runs on the same row tiles, folds 2^(s_min - s_b) into its scales of
// input block b (a group of 128 is one h block) and writes y (or adds into
// it) from the accumulators times 2^(2e - s_min), each output owned by one
// lane.  So f16's range limits neither x nor h.

constexpr int SG_NST = 2;
constexpr int SG_B_BYTES = BROWS * KS;            // 16 KB: 256 rows x 64 int8 codes
constexpr int SG_STAGE = A_BYTES + SG_B_BYTES;    // 32 KB
constexpr int SG_B_LOADS = SG_B_BYTES / 16 / PF_BLOCK;  // 4
constexpr int SG_HP = 128 + 8;
static_assert(32 * SG_HP * 2 <= SG_STAGE, "32 epilogue rows fit a ring slot");

struct SGemmCtx {
    const uint8_t *a_base;
    uint32_t a_off[4];
    const uint8_t *b_base[SG_B_LOADS];
    uint32_t b_off[SG_B_LOADS];
    const uint16_t *srow[2];  // this lane's two weight rows' group scales
    const uint32_t *fb;       // GEMM2: LDS [16], 2^(s_min - s_b) per group (h block) b as an f16 pair
    uint8_t *ring[SG_NST];  // the ring slots, one LDS array each (see ring_depth)
    int brow[2];
    int nk;
};

template <int MS>
__device__ __forceinline__ void sg_issue(const SGemmCtx &c, int ks, int slot, int wave) {
    uint8_t *sa = c.ring[slot];
    uint8_t *sb = sa + A_BYTES;
    const uint8_t *ab = c.a_base + (size_t)ks * (KS * 2);
#pragma unroll
    for (int i = 0; i < MS; ++i)
        __builtin_amdgcn_global_load_lds((const void *)(ab + c.a_off[i]),
                                         (__attribute__((address_space(3))) void *)(sa + (i * 4 + wave) * 1024),
                                         16, 0, 0);
#pragma unroll
    for (int i = 0; i < SG_B_LOADS; ++i)
        __builtin_amdgcn_global_load_lds((const void *)((c.b_base[i] + (size_t)ks * KS) + c.b_off[i]),
                                         (__attribute__((address_space(3))) void *)(sb + (i * 4 + wave) * 1024),
                                         16, 0, 0);
}

// four int8 codes of a dword (top bits flipped) as f16 pairs (q0, q2), (q1, q3)
// times the scale pair
__device__ __forceinline__ uint2 sg_codes(uint32_t w, uint32_t kf, half2_t sc) {
    const half2_t off = {(_Float16)1152.0f, (_Float16)1152.0f};
    const uint32_t u = w ^ 0x80808080u;
    const half2_t a = __builtin_bit_cast(half2_t, insert_codes<0x00ff00ffu>(u, kf)) - off;
    const half2_t b = __builtin_bit_cast(half2_t, insert_codes<0x00ff00ffu>(u >> 8, kf)) - off;
    return make_uint2(__builtin_bit_cast(uint32_t, a * sc), __builtin_bit_cast(uint32_t, b * sc));
}

template <int MS, bool FB>
__device__ __forceinline__ void sg_main(const SGemmCtx &c, f32x16_t (&acc)[4][2], int wave, int lane) {
    const int l32 = lane & 31, hf = lane >> 5;
    const int NK = c.nk;
    const uint32_t kf = opaque_magic(MAGIC_F16);
    sg_issue<MS>(c, 0, 0, wave);
    half2_t sc[2];
    uint32_t snext[2] = {(uint32_t)c.srow[0][0], (uint32_t)c.srow[1][0]};
    uint32_t fnext = 0x3c003c00u;  // GEMM2: the next group's factor (1.0 until read)
    for (int kk = 0; kk < NK; kk += SG_NST) {
#pragma unroll
        for (int u = 0; u < SG_NST; ++u) {
            const int ks = kk + u;
            if (ks < NK) {
                MOEQ4_WAIT_VM_LDS(0);  // stage ks has landed (only it was in flight)
                lds_barrier();
                if (ks + 1 < NK) sg_issue<MS>(c, ks + 1, (u + 1) % SG_NST, wave);
                if ((ks & 1) == 0) {  // a new group of 128 inputs
                    const int kg = ks >> 1;
                    if (FB && kg == 0) fnext = c.fb[0];  // after the first barrier
                    const half2_t f2 = __builtin_bit_cast(half2_t, fnext);
#pragma unroll
                    for (int ns = 0; ns < 2; ++ns) {
                        sc[ns] = __builtin_bit_cast(half2_t, snext[ns] * 0x10001u);
                        if (FB) sc[ns] = sc[ns] * f2;
                        if (2 * (kg + 1) < NK) snext[ns] = (uint32_t)c.srow[ns][kg + 1];
                    }
                    if (FB && 2 * (kg + 1) < NK) fnext = c.fb[kg + 1];
                }
                const uint8_t *sa = c.ring[u];
                const uint8_t *sbp = sa + A_BYTES;
                uint4 bw[2][2];
#pragma unroll
                for (int ns = 0; ns < 2; ++ns) {
                    const int rb = c.brow[ns];
#pragma unroll
                    for (int t = 0; t < 2; ++t)
                        bw[ns][t] = *reinterpret_cast<const uint4 *>(sbp + rb * 64 + 16 * ((2 * hf + t) ^ ((rb >> 2) & 3)));
                }
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    u32x4_t bv[2];
#pragma unroll
                    for (int ns = 0; ns < 2; ++ns) {
                        const uint4 v = bw[ns][s >> 1];
                        const uint32_t d0 = (s & 1) ? v.z : v.x, d1 = (s & 1) ? v.w : v.y;
                        const uint2 p0 = sg_codes(d0, kf, sc[ns]), p1 = sg_codes(d1, kf, sc[ns]);
                        bv[ns] = u32x4_t{p0.x, p0.y, p1.x, p1.y};
                    }
                    const int ch = 4 * hf + s;
#pragma unroll
                    for (int mi = 0; mi < MS; ++mi) {
                        const int r = 32 * mi + l32;
                        const uint4 av = *reinterpret_cast<const uint4 *>(sa + r * 128 + 16 * (ch ^ ((r >> 1) & 7)));
                        const f16x8_t a8 = __builtin_bit_cast(f16x8_t, u32x4_t{av.x, av.y, av.z, av.w});
#pragma unroll
                        for (int ns = 0; ns < 2; ++ns)
                            acc[mi][ns] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                                a8, __builtin_bit_cast(f16x8_t, bv[ns]), acc[mi][ns], 0, 0, 0);
                    }
                }
            }
        }
    }
}

// STAGE 1: A = x16 rows (PERM4), B = gate | up codes, epilogue SwiGLU of the
//          accumulators times 2^e, scaled as above -> h (f16, PERM4), hx.
// STAGE 2: A = h rows, B = down codes (scales times 2^(s_min - s_b)),
//          epilogue y = (accumulate ? y : 0) + acc 2^(2e - s_min).
// Both launches take the same tile_rows, so a GEMM2 tile's rows share their
// h exponents.
template <int STAGE>
__global__ __launch_bounds__(PF_BLOCK) __attribute__((amdgpu_waves_per_eu(2, 2))) void shared_gemm_kernel(
    const uint16_t *__restrict__ act, const int32_t *__restrict__ xexp, int T, int H, int I, SharedPtrs S,
    uint16_t *__restrict__ h_out, int8_t *__restrict__ hx, float *__restrict__ y, int accumulate, int tile_rows) {
    const int ncb = STAGE == 1 ? I / 128 : H / BROWS;
    const int ntiles = (T + tile_rows - 1) / tile_rows;
    const int nwork = ntiles * ncb;
    const int per = (nwork + 7) / 8;
    const int bx = blockIdx.x;
    if (bx / 8 >= per) return;
    const int w = (bx % 8) * per + bx / 8;
    if (w >= nwork) return;
    const int j = w / ncb, cb = w % ncb;
    const int row0 = j * tile_rows, rows = T - row0 < tile_rows ? T - row0 : tile_rows;
    const int K = STAGE == 1 ? H : I;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hf = lane >> 5;
    const int col_base = cb * (STAGE == 1 ? 128 : BROWS);

    __shared__ __attribute__((aligned(16))) uint8_t s_ring0[SG_STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t s_ring1[SG_STAGE];
    __shared__ uint32_t s_red[PF_BLOCK / 64];
    __shared__ uint32_t s_fb[16];  // STAGE 2: 2^(s_min - s_b) per h block b (I <= 2048), f16 pair
    __shared__ __attribute__((aligned(16))) int32_t s_xe[BM];  // the tile rows' exponents e
    const int nbh = I / 128;
    // STAGE 2: the tile's h exponents (one per 128-column block, the same
    // for all its rows) and their smallest
    int smin = 64;
    if (STAGE == 2) {
        int sb[16];  // all loads issued before the first use
#pragma unroll
        for (int b = 0; b < 16; ++b) sb[b] = b < nbh ? (int)hx[(size_t)row0 * nbh + b] : 64;
#pragma unroll
        for (int b = 0; b < 16; ++b) smin = sb[b] < smin ? sb[b] : smin;
        if (tid < 16) {
            int mine = 64;
#pragma unroll
            for (int b = 0; b < 16; ++b) mine = tid == b ? sb[b] : mine;
            const _Float16 f = (_Float16)exp2i(smin - mine);
            s_fb[tid] = __builtin_bit_cast(uint16_t, f) * 0x10001u;
        }
    }
    if (tid < rows) s_xe[tid] = xexp[row0 + tid];  // read after the main loop's barriers
    SGemmCtx c;
    c.fb = s_fb;
    c.ring[0] = s_ring0;
    c.ring[1] = s_ring1;
    c.nk = K / KS;
    c.a_base = reinterpret_cast<const uint8_t *>(act);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 32 * i + 8 * wave + (lane >> 3);
        const int ch = (lane & 7) ^ ((r >> 1) & 7);
        const int rr = r < rows ? r : 0;  // padding rows read row 0; their outputs are dropped
        c.a_off[i] = ((uint32_t)(row0 + rr) * (uint32_t)K + 8u * ch) * 2u;
    }
#pragma unroll
    for (int i = 0; i < SG_B_LOADS; ++i) {
        const int S_ = (i * 4 + wave) * 64 + lane;
        const int rb = S_ / 4, ch = (S_ % 4) ^ ((rb >> 2) & 3);
        uint32_t wrow;
        if (STAGE == 1) {
            c.b_base[i] = reinterpret_cast<const uint8_t *>(i < 2 ? S.gq : S.uq);
            wrow = (uint32_t)col_base + (rb & 127);
        } else {
            c.b_base[i] = reinterpret_cast<const uint8_t *>(S.dq);
            wrow = (uint32_t)col_base + rb;
        }
        c.b_off[i] = wrow * (uint32_t)K + 16u * ch;
    }
#pragma unroll
    for (int ns = 0; ns < 2; ++ns) {
        c.brow[ns] = STAGE == 1 ? ns * 128 + wave * 32 + l32 : wave * 64 + ns * 32 + l32;
        const int wrow = STAGE == 1 ? col_base + wave * 32 + l32 : col_base + c.brow[ns];
        const uint16_t *sb = STAGE == 1 ? (ns == 0 ? S.gs : S.us) : S.ds;
        c.srow[ns] = sb + (size_t)wrow * (K / 128);
    }

    f32x16_t acc[4][2];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ns = 0; ns < 2; ++ns)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][ns][r] = 0.f;
    const int msub = (rows + 31) / 32;
    switch (msub) {
        case 1: sg_main<1, STAGE == 2>(c, acc, wave, lane); break;
        case 2: sg_main<2, STAGE == 2>(c, acc, wave, lane); break;
        case 3: sg_main<3, STAGE == 2>(c, acc, wave, lane); break;
        default: sg_main<4, STAGE == 2>(c, acc, wave, lane); break;
    }
    __syncthreads();  // ring no longer read

    if (STAGE == 1) {
        // h 2^-2e = silu(acc 2^e) (acc_u 2^-e) per row, then one power of two
        // for the workgroup's block
        float mloc = 0.f;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            if (mi >= msub) break;
            const int4 *xe4 = reinterpret_cast<const int4 *>(s_xe + 32 * mi + 4 * hf);  // rows r % 4 of group r / 4
            const int4 ev[4] = {xe4[0], xe4[2], xe4[4], xe4[6]};
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = 32 * mi + 8 * (r / 4) + 4 * hf + (r % 4);
                float hn = 0.f;
                if (row < rows) {
                    const int4 q = ev[r / 4];
                    const int e = r % 4 == 0 ? q.x : (r % 4 == 1 ? q.y : (r % 4 == 2 ? q.z : q.w));
                    hn = silu(acc[mi][0][r] * exp2i(e)) * (acc[mi][1][r] * exp2i(-e));
                }
                acc[mi][0][r] = hn;
                mloc = fmaxf(mloc, fabsf(hn));
            }
        }
        const RowScale rs = row_scale(block_max_nonneg(mloc, s_red));
        // one 32-row subtile at a time through the two ring slots in turn
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            if (mi >= msub) break;
            uint16_t *s_h = reinterpret_cast<uint16_t *>(mi % 2 == 0 ? s_ring0 : s_ring1);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lr = 8 * (r / 4) + 4 * hf + (r % 4);
                s_h[lr * SG_HP + wave * 32 + l32] = __builtin_bit_cast(uint16_t, (_Float16)(acc[mi][0][r] * rs.sc));
            }
            __syncthreads();
            for (int i = tid; i < 32 * 16; i += PF_BLOCK) {
                const int lr = i / 16, cc = i % 16, row = 32 * mi + lr;
                if (row < rows) {
                    const uint4 v = *reinterpret_cast<const uint4 *>(&s_h[lr * SG_HP + cc * 8]);
                    const uint4 o = make_uint4((v.x & 0xffffu) | (v.y << 16), (v.x >> 16) | (v.y & 0xffff0000u),
                                               (v.z & 0xffffu) | (v.w << 16), (v.z >> 16) | (v.w & 0xffff0000u));
                    *reinterpret_cast<uint4 *>(h_out + (size_t)(row0 + row) * I + cb * 128 + cc * 8) = o;
                    if (cc == 0) hx[(size_t)(row0 + row) * nbh + cb] = (int8_t)rs.s;
                }
            }
        }
    } else {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            if (mi < msub) {
                const int4 *xe4 = reinterpret_cast<const int4 *>(s_xe + 32 * mi + 4 * hf);
                const int4 ev[4] = {xe4[0], xe4[2], xe4[4], xe4[6]};
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 32 * mi + 8 * (r / 4) + 4 * hf + (r % 4);
                    if (row < rows) {
                        const int4 q = ev[r / 4];
                        const int e = r % 4 == 0 ? q.x : (r % 4 == 1 ? q.y : (r % 4 == 2 ? q.z : q.w));
                        const float f = exp2i(2 * e - smin);
#pragma unroll
                        for (int ns = 0; ns < 2; ++ns) {
                            float *dst = y + (size_t)(row0 + row) * H + col_base + wave * 64 + ns * 32 + l32;
                            *dst = accumulate ? *dst + acc[mi][ns][r] * f : acc[mi][ns][r] * f;
                        }
                    }
                }
            }
        }
    }
}

// Token rows per tile: the largest of 128, 64, 32 that still gives
// SG_MIN_WORK work items (more, shorter tiles fill the chip when the
// products are small; the codes they re-read come from L2).
constexpr int SG_MIN_WORK = 512;
static int sg_tile_rows(int64_t T, int ncb) {
    for (int tr = BM; tr > 32; tr /= 2)
        if ((T + tr - 1) / tr * ncb >= SG_MIN_WORK) return tr;
    return 32;
}

hipError_t launch_shared_gemm(const uint16_t *x, int64_t T, const SharedPtrs &S, uint16_t *x16, int32_t *xexp,
                              uint16_t *h, int8_t *hx, float *y, bool accumulate, hipStream_t s, hipEvent_t e0,
                              hipEvent_t e1, hipEvent_t e2, hipEvent_t e3) {
    const int H = S.H, I = S.I;
    if (I > 2048) return hipErrorInvalidValue;  // s_fb holds 16 blocks
    hipLaunchKernelGGL(x_to_f16_kernel<2>, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, x, T, H, x16, xexp);
    // one tiling for both launches, so that a GEMM2 tile's rows share their
    // h exponents: the larger tile of the two choices (measured faster than
    // the smaller one for both GEMMs at 4096 tokens, H = 2048, I = 512)
    const int tr_a = sg_tile_rows(T, I / 128), tr_b = sg_tile_rows(T, H / BROWS);
    const int tr1 = tr_a < tr_b ? tr_b : tr_a, tr2 = tr1;
    const unsigned nb1 = (unsigned)(((I / 128) * ((T + tr1 - 1) / tr1) + 7) / 8 * 8);
    const unsigned nb2 = (unsigned)(((H / BROWS) * ((T + tr2 - 1) / tr2) + 7) / 8 * 8);
    launch_k(shared_gemm_kernel<1>, dim3(nb1), dim3(PF_BLOCK), s, e0, e1, (const uint16_t *)x16,
             (const int32_t *)xexp, (int)T, H, I, S, h, hx, y, accumulate ? 1 : 0, tr1);
    launch_k(shared_gemm_kernel<2>, dim3(nb2), dim3(PF_BLOCK), s, e2, e3, (const uint16_t *)h, (const int32_t *)xexp,
             (int)T, H, I, S, h, hx, y, accumulate ? 1 : 0, tr2);
    return hipGetLastError();
}

// y[t] = sum over the token's k routed rows of z (fp32).  One workgroup of
// 256 threads per token, 8 columns per thread and pass.
// Row r of z is z 2^(s - 2e): 2^-2e per token (xexp: e per token, or null
// for 0) and 2^s per row and 64 columns (zx[r * H / 64 + c / 64], for
// column c), both taken off here.
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t *__restrict__ z, const int8_t *__restrict__ zx,
                                                      const int32_t *__restrict__ xexp,
                                                      const int32_t *__restrict__ inv, int64_t T, int k, int H,
                                                      int64_t P, float *__restrict__ y) {
    const int64_t t = blockIdx.x;
    if (t >= T) return;
    const int e2 = xexp ? 2 * xexp[t] : 0;
    for (int c = threadIdx.x * 8; c < H; c += blockDim.x * 8) {
        float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int i = 0; i < k; ++i) {
            int64_t row = inv[t * k + i];
            row = row < 0 ? 0 : (row >= P ? P - 1 : row);
            const uint4 v = *reinterpret_cast<const uint4 *>(z + row * H + c);
            const float f = exp2i(e2 - (int)zx[row * (H / 64) + (c / 64)]);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                s[2 * q] = fmaf((float)__builtin_bit_cast(_Float16, (uint16_t)(w[q] & 0xffffu)), f, s[2 * q]);
                s[2 * q + 1] = fmaf((float)__builtin_bit_cast(_Float16, (uint16_t)(w[q] >> 16)), f, s[2 * q + 1]);
            }
        }
        float4 *dst = reinterpret_cast<float4 *>(y + t * H + c);
        dst[0] = make_float4(s[0], s[1], s[2], s[3]);
        dst[1] = make_float4(s[4], s[5], s[6], s[7]);
    }
}

// ------------------------------------------------------- prefill copy
//
// Gather of the canonical codes and scale words into the GEMMs' tile order
// (the layout is stated with moe_q4_prefill_pack in the public header).
// Codes: one thread per 16-byte chunk of the copy, in the order in which the
// GEMM's direct-to-LDS loads place them: with RB bytes of a row per K-step
// (32: 4-bit codes, 64: FP8), slot S of a K-step holds chunk
// (S % 2) ^ ((row >> 3) & 1) of row S / 2, or (S % 4) ^ ((row >> 2) & 3) of
// row S / 4.
template <int STAGE, int RB>
__global__ __launch_bounds__(256) void pack_codes_kernel(LayerPtrs L, uint8_t *__restrict__ dst) {
    const int H = L.H, I = L.I;
    const int ncb = STAGE == 1 ? I / 128 : H / BROWS;
    const int K = STAGE == 1 ? H : I, nk = K / KS;
    constexpr int SLOTS = BROWS * RB / 16;
    const int64_t n = (int64_t)L.E * ncb * nk * SLOTS;
    const int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (o >= n) return;
    const int S = (int)(o % SLOTS);
    const int64_t t = o / SLOTS;
    const int ks = (int)(t % nk);
    const int64_t tile = t / nk;
    const int cb = (int)(tile % ncb), e = (int)(tile / ncb);
    constexpr int CPR = RB / 16;  // chunks per row and K-step
    const int rb = S / CPR, ch = CPR == 2 ? (S % 2) ^ ((rb >> 3) & 1) : (S % 4) ^ ((rb >> 2) & 3);
    const uint8_t *src;
    size_t row;
    if (STAGE == 1) {
        src = rb < 128 ? L.gq : L.uq;
        row = (size_t)e * I + cb * 128 + (rb & 127);
    } else {
        src = L.dq;
        row = (size_t)e * H + cb * BROWS + rb;
    }
    const size_t row_bytes = (size_t)K * RB / KS;
    const uint4 v = *reinterpret_cast<const uint4 *>(src + row * row_bytes + (size_t)ks * RB + 16 * ch);
    const PackLayout pl = pack_layout(L.E, H, I, L.fmt);
    *reinterpret_cast<uint4 *>(dst + (STAGE == 1 ? pl.gu_q : pl.d_q) + (size_t)o * 16) = v;
}

// Lifts (int4 formats): one thread per weight row slot r of a tile: the
// row's power-of-two lift L (row_lift_from_max over its canonical scales and
// mins), one signed byte.
template <int STAGE>
__global__ __launch_bounds__(256) void pack_lift_kernel(LayerPtrs L, uint8_t *__restrict__ dst) {
    const int H = L.H, I = L.I;
    const int ncb = STAGE == 1 ? I / 128 : H / BROWS;
    const int K = STAGE == 1 ? H : I;
    const int64_t n = (int64_t)L.E * ncb * BROWS;
    const int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (o >= n) return;
    const int r = (int)(o % BROWS);
    const int64_t tile = o / BROWS;
    const int cb = (int)(tile % ncb), e = (int)(tile / ncb);
    const uint16_t *src;
    size_t row;
    if (STAGE == 1) {
        src = r < 128 ? L.gsm : L.usm;
        row = (size_t)e * I + cb * 128 + (r & 127);
    } else {
        src = L.dsm;
        row = (size_t)e * H + cb * BROWS + r;
    }
    const int lift = L.fmt == 0 ? row_lift_from_max(canonical_row_max<0>(src, row, K / 64))
                                : row_lift_from_max(canonical_row_max<1>(src, row, K / 128));
    const PackLayout pl = pack_layout(L.E, H, I, L.fmt);
    dst[(STAGE == 1 ? pl.gu_l : pl.d_l) + o] = (uint8_t)(int8_t)lift;
}

// Scale words: one thread per word; K-step j of slot r gets the aligned word
// of the row's canonical scale array holding its group 64 j / G entry, its
// f16 halves times 2^L (the row's lift: ldexp, one rounding) for the int4
// formats.
template <int STAGE>
__global__ __launch_bounds__(256) void pack_scales_kernel(LayerPtrs L, uint8_t *__restrict__ dst) {
    const int H = L.H, I = L.I;
    const int ncb = STAGE == 1 ? I / 128 : H / BROWS;
    const int K = STAGE == 1 ? H : I, nk = K / KS;
    const int64_t n = (int64_t)L.E * ncb * nk * BROWS;
    const int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (o >= n) return;
    const int r = (int)(o % BROWS);
    const int64_t t = o / BROWS;
    const int ks = (int)(t % nk);
    const int64_t tile = t / nk;
    const int cb = (int)(tile % ncb), e = (int)(tile / ncb);
    const int G = L.fmt == 1 ? 128 : 64;  // NVFP4: four 16-input scales per word, as one 64-input entry
    const int esz = L.fmt == 1 ? 2 : 4;
    const uint16_t *src;
    size_t row;
    if (STAGE == 1) {
        src = r < 128 ? L.gsm : L.usm;
        row = (size_t)e * I + cb * 128 + (r & 127);
    } else {
        src = L.dsm;
        row = (size_t)e * H + cb * BROWS + r;
    }
    const size_t byte = ((row * (size_t)(K / G) + (size_t)(ks * KS / G)) * esz) & ~(size_t)3;
    uint32_t wv = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint8_t *>(src) + byte);
    const PackLayout pl = pack_layout(L.E, H, I, L.fmt);
    if (L.fmt == 0 || L.fmt == 1) {
        const int lift = (int)(int8_t)dst[(STAGE == 1 ? pl.gu_l : pl.d_l) + tile * BROWS + r];
        const uint32_t lo = __builtin_bit_cast(uint16_t, __builtin_ldexpf16(__builtin_bit_cast(_Float16, (uint16_t)(wv & 0xffffu)), lift));
        const uint32_t hi = __builtin_bit_cast(uint16_t, __builtin_ldexpf16(__builtin_bit_cast(_Float16, (uint16_t)(wv >> 16)), lift));
        wv = lo | (hi << 16);
    }
    reinterpret_cast<uint32_t *>(dst + (STAGE == 1 ? pl.gu_s : pl.d_s))[o] = wv;
}

hipError_t launch_prefill_pack(const LayerPtrs &L, uint8_t *dst, hipStream_t s) {
    const int64_t E = L.E, H = L.H, I = L.I;
    const int64_t t1 = E * (I / 128) * (H / KS), t2 = E * (H / BROWS) * (I / KS);  // (tile, K-step) blocks
    if (L.fmt == 2) {  // block FP8: 64 bytes per row and K-step, no scale regions
        const int64_t n1 = t1 * (BROWS * 64 / 16), n2 = t2 * (BROWS * 64 / 16);
        hipLaunchKernelGGL((pack_codes_kernel<1, 64>), dim3((unsigned)((n1 + 255) / 256)), dim3(256), 0, s, L, dst);
        hipLaunchKernelGGL((pack_codes_kernel<2, 64>), dim3((unsigned)((n2 + 255) / 256)), dim3(256), 0, s, L, dst);
        return hipGetLastError();
    }
    const int64_t n1 = t1 * (BROWS * 32 / 16), n2 = t2 * (BROWS * 32 / 16);
    const int64_t s1 = t1 * BROWS, s2 = t2 * BROWS;
    hipLaunchKernelGGL((pack_codes_kernel<1, 32>), dim3((unsigned)((n1 + 255) / 256)), dim3(256), 0, s, L, dst);
    hipLaunchKernelGGL((pack_codes_kernel<2, 32>), dim3((unsigned)((n2 + 255) / 256)), dim3(256), 0, s, L, dst);
    if (L.fmt == 0 || L.fmt == 1) {  // the lifts first: the scale words are taken times 2^L
        const int64_t l1 = E * (I / 128) * BROWS, l2 = E * (H / BROWS) * BROWS;
        hipLaunchKernelGGL(pack_lift_kernel<1>, dim3((unsigned)((l1 + 255) / 256)), dim3(256), 0, s, L, dst);
        hipLaunchKernelGGL(pack_lift_kernel<2>, dim3((unsigned)((l2 + 255) / 256)), dim3(256), 0, s, L, dst);
    }
    hipLaunchKernelGGL(pack_scales_kernel<1>, dim3((unsigned)((s1 + 255) / 256)), dim3(256), 0, s, L, dst);
    hipLaunchKernelGGL(pack_scales_kernel<2>, dim3((unsigned)((s2 + 255) / 256)), dim3(256), 0, s, L, dst);
    return hipGetLastError();
}

template <int FMT>
static hipError_t launch_prefill_fmt(const uint16_t *x, const float *gate, int64_t T, int k, const LayerPtrs &L,
                                     const GroupOut &g, uint16_t *x16, int32_t *xexp, uint16_t *h, uint16_t *z,
                                     int8_t *hx, int8_t *zx, float *y, hipStream_t s, hipEvent_t const *ev,
                                     bool x16_ready) {
    const int H = L.H, I = L.I;
    const int64_t tiles = max_tiles(T * k, L.E, BM);
    if (!x16_ready)
        hipLaunchKernelGGL(x_to_f16_kernel<FMT == 3 ? 0 : 1>, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, x, T,
                           H, x16, xexp);
    // mean rows per expert within one 32-row subtile: the single-subtile build
    const bool one = T * k <= 32 * (int64_t)L.E;
    const unsigned split = one ? BM / 32 : 1;
    const unsigned nb1 = (unsigned)(8 * ((tiles + 7) / 8) * (I / 128)) * split;  // 8 XCDs x ranks x column blocks
    const unsigned nb2 = (unsigned)(8 * ((tiles + 7) / 8) * (H / BROWS)) * split;
    auto k1 = one ? grouped_gemm_kernel<FMT, 1, true> : grouped_gemm_kernel<FMT, 1, false>;
    auto k2 = one ? grouped_gemm_kernel<FMT, 2, true> : grouped_gemm_kernel<FMT, 2, false>;
    launch_k(k1, dim3(nb1), dim3(PF_BLOCK), s, ev ? ev[0] : nullptr, ev ? ev[1] : nullptr,
             (const uint16_t *)x16, (const int32_t *)xexp, H, I, k, L, (const Tile *)g.tiles,
             (const int32_t *)g.ntiles, (const int32_t *)g.perm, gate, h, z, (const int32_t *)g.order, hx, zx);
    launch_k(k2, dim3(nb2), dim3(PF_BLOCK), s, ev ? ev[2] : nullptr, ev ? ev[3] : nullptr,
             (const uint16_t *)h, (const int32_t *)nullptr, H, I, k, L, (const Tile *)g.tiles,
             (const int32_t *)g.ntiles, (const int32_t *)g.perm, gate, h, z,
             (const int32_t *)(g.order2 ? g.order2 : g.order), hx, zx);
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)T), dim3(256), 0, s, (const uint16_t *)z, (const int8_t *)zx,
                       (const int32_t *)xexp, (const int32_t *)g.inv, T, k, H, T * (int64_t)k, y);
    return hipGetLastError();
}

hipError_t launch_fill_zero(float *p, int64_t n, hipStream_t s) {
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n / 4 + 256) / 256)), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

hipError_t launch_fill_zero_u32(uint32_t *p, int64_t n, hipStream_t s) {
    return launch_fill_zero(reinterpret_cast<float *>(p), n, s);  // all-zero bits either way
}

static hipError_t launch_prefill_fp8(const uint16_t *x, const float *gate, int64_t T, int k, const LayerPtrs &L,
                                     const GroupOut &g, int32_t *xexp, uint16_t *h, uint16_t *z, int8_t *hx,
                                     int8_t *zx, float *y, hipStream_t s, hipEvent_t const *ev, bool xexp_ready) {
    const int H = L.H, I = L.I;
    const int64_t tiles = max_tiles(T * k, L.E, BM);
    if (!xexp_ready)  // the per-token exponents only
        hipLaunchKernelGGL(x_to_f16_kernel<3>, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, x, T, H,
                           (uint16_t *)nullptr, xexp);
    const unsigned nb1 = (unsigned)(8 * ((tiles + 7) / 8) * (I / 128));  // as launch_prefill_fmt
    const unsigned nb2 = (unsigned)(8 * ((tiles + 7) / 8) * (H / BROWS));
    launch_k(grouped_gemm_fp8_kernel<1>, dim3(nb1), dim3(PF_BLOCK), s, ev ? ev[0] : nullptr, ev ? ev[1] : nullptr, x,
             H, I, k, L, (const Tile *)g.tiles, (const int32_t *)g.ntiles, (const int32_t *)g.perm, gate, h, z,
             (const int32_t *)g.order, hx, zx, (const int32_t *)xexp);
    launch_k(grouped_gemm_fp8_kernel<2>, dim3(nb2), dim3(PF_BLOCK), s, ev ? ev[2] : nullptr, ev ? ev[3] : nullptr,
             (const uint16_t *)h, H, I, k, L, (const Tile *)g.tiles, (const int32_t *)g.ntiles,
             (const int32_t *)g.perm, gate, h, z, (const int32_t *)(g.order2 ? g.order2 : g.order), hx, zx,
             (const int32_t *)nullptr);
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)T), dim3(256), 0, s, (const uint16_t *)z, (const int8_t *)zx,
                       (const int32_t *)xexp, (const int32_t *)g.inv, T, k, H, T * (int64_t)k, y);
    return hipGetLastError();
}

hipError_t launch_prefill_experts(const uint16_t *x, const float *gate, int64_t T, int k, const LayerPtrs &L,
                                  const GroupOut &g, uint16_t *x16, int32_t *xexp, uint16_t *h, uint16_t *z,
                                  int8_t *hx, int8_t *zx, float *y, hipStream_t s, hipEvent_t const *ev,
                                  bool x16_ready) {
    switch (L.fmt) {
        case 0: return launch_prefill_fmt<0>(x, gate, T, k, L, g, x16, xexp, h, z, hx, zx, y, s, ev, x16_ready);
        case 1: return launch_prefill_fmt<1>(x, gate, T, k, L, g, x16, xexp, h, z, hx, zx, y, s, ev, x16_ready);
        case 2: return launch_prefill_fp8(x, gate, T, k, L, g, xexp, h, z, hx, zx, y, s, ev, x16_ready);
        case 3: return launch_prefill_fmt<3>(x, gate, T, k, L, g, x16, xexp, h, z, hx, zx, y, s, ev, x16_ready);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_prefill_prep(const uint16_t *logits, int64_t T, int E, int k, int32_t *idx, float *gate,
                               const GroupOut &g, const uint16_t *x, int H, uint16_t *x16, int32_t *xexp, int fmt,
                               hipStream_t s) {
    const int64_t P = T * k;
    if (P <= GROUP_SINGLE_MAX || E > 1024 || k > 32) return hipErrorInvalidValue;
    const int64_t nch = (P + GROUP_CHUNK - 1) / GROUP_CHUNK;
    const int64_t nconv = (T + PREP_WAVES - 1) / PREP_WAVES;  // row-conversion workgroups
    const dim3 grid((unsigned)(nch + nconv)), block(PREP_WAVES * 64);
    const int npl = (E + 63) / 64;
#define PREP(N, O, C) \
    hipLaunchKernelGGL((prefill_prep_kernel<N, O, C>), grid, block, 0, s, logits, T, E, k, idx, gate, g.chunk_cnt, x, H, x16, xexp)
#define PREP_N(O, C) \
    if (npl <= 4) PREP(4, O, C); else if (npl <= 8) PREP(8, O, C); else PREP(16, O, C)
    if (fmt == 2) PREP_N(3, true);        // block FP8: the GEMMs read x as given; the exponents only
    else if (fmt == 3) PREP_N(0, true);   // NVFP4: x16 in natural order
    else PREP_N(1, true);                 // int4: x16 in PERM8 order
#undef PREP_N
#undef PREP
    return hipGetLastError();
}

}  // namespace moeq4
