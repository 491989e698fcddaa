/*
 * moe_oracle.c -- plain CPU oracle of the routed int4 MoE expert layer.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the package's smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or helper with the HIP library: every conversion and every step is
 * written out here from its definition, in double precision, one result at a
 * time, with no blocking and no fused or reordered arithmetic.  Build:
 *   gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC moe_oracle.c -o liboracle.so -lm
 * (-ffp-contract=off: no multiply-add contraction, so each double operation
 * rounds once, as written.)
 *
 * What is computed and where it comes from (web pages on the Fish Audio
 * Drama 3 4-bit builds):
 *   - routed experts with gate, up and down projections: NVFP4 routed experts
 *     card, "Quantization" (three projections per expert);
 *   - int4 asymmetric group-64 experts with an f16 scale and f16 min:
 *     drama-q4 card, "What's quantized"; the values map losslessly onto an
 *     affine scale*q + bias format: drama-rs page, "Apple Silicon (MLX)";
 *     so w = scale * q + min with q in 0..15;
 *   - int4 symmetric group 128 with one f16 scale per 128 input weights:
 *     drama-3-w4a16 card, "At a glance" and "How it was made";
 *   - groups run along the input dimension ("per 128 input weights");
 *   - router weights are bf16: drama-q4 "What's quantized", MLX card
 *     "Quantization and provenance";
 *   - rows grouped by routed expert: drama-rs page, "Apple Silicon (MLX)"
 *     and "Layout" (grouped MoE prefill);
 *   - the shared expert's linears are int8 symmetric group 128: drama-q4
 *     card, "What's quantized" (see oracle_shared);
 *   - block-FP8 experts with one scale per 128 x 128 block, each matrix
 *     dequantised with its block scales: drama-3-w4a16 card, "At a glance"
 *     table and "How it was made" (the released experts' format);
 *   - NVFP4 experts: packed E2M1 values, one E4M3 scale per 16 input
 *     weights and a float32 global scale per matrix, gate and up sharing
 *     theirs within an expert: drama-3-nvfp4 card, "Quantization".
 * The pages do not state the routing function, the activation or the combine.
 * This library takes: bf16 router logits, the 8 (k) largest selected with
 * ties to the lower expert index, gates = softmax over the selected logits
 * (the same as a softmax over all experts renormalised over the selected),
 * a SwiGLU expert MLP silu(gate x) * (up x) followed by down, and an output
 * y[t] = sum_i gate[t,i] * expert_out[t,i] in slot order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_FMT_ASYM_G64 0
#define ORACLE_FMT_SYM_G128 1
#define ORACLE_FMT_FP8_B128 2
#define ORACLE_FMT_NVFP4 3

/* ---------------------------------------------------------------- numbers */

/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_f16_value(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                  /* subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f | 0x400), e - 25);     /* (1.f) * 2^(e-15)     */
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE-754 binary32. */
double oracle_bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* binary32 -> bfloat16, round to nearest, ties to even.  The 16 bits that
 * are dropped are compared with one half of the kept last place: above it
 * rounds up, below it rounds down, exactly half rounds to the even one. */
uint16_t oracle_bf16_round(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u)            /* NaN stays NaN (quiet) */
        return (uint16_t)((u >> 16) | 0x40);
    uint32_t kept = u >> 16;
    uint32_t dropped = u & 0xffffu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))
        kept += 1;                                  /* carries into the exponent
                                                       (or to infinity) as IEEE does */
    return (uint16_t)kept;
}

/*
 * OCP 8-bit float E4M3 ("fn": no infinities): sign bit 7, exponent bits 6..3
 * with bias 7, mantissa bits 2..0.  Exponent 0 is subnormal, m/8 * 2^-6; the
 * pattern S.1111.111 is NaN; the largest finite value is 1.75 * 2^8 = 448.
 */
double oracle_e4m3_value(uint8_t b)
{
    int sgn = b >> 7, e = (b >> 3) & 0xf, m = b & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp((double)(8 + m), e - 10);
    return sgn ? -v : v;
}

/*
 * OCP 4-bit float E2M1 (the element type of the MX and NVFP4 formats): sign
 * bit 3, exponent bits 2..1 with bias 1, mantissa bit 0; exponent 0 is
 * subnormal, m * 2^-1.  The magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6.
 */
double oracle_e2m1_value(uint8_t c)
{
    int sgn = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
    double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return (sgn ? -1.0 : 1.0) * v;
}

/* --------------------------------------------------------------- dequant */

static int group_of(int fmt)
{
    return fmt == ORACLE_FMT_ASYM_G64 ? 64 : fmt == ORACLE_FMT_NVFP4 ? 16 : 128;
}
static int known_fmt(int fmt)
{
    return fmt == ORACLE_FMT_ASYM_G64 || fmt == ORACLE_FMT_SYM_G128 || fmt == ORACLE_FMT_FP8_B128 ||
           fmt == ORACLE_FMT_NVFP4;
}

/* 4-bit code of input index k in a packed row: byte k/2, low nibble for even k. */
static int nibble(const uint8_t *row, int k)
{
    return (row[k / 2] >> (4 * (k & 1))) & 0xf;
}

/* Exact value of weight (n, k) of one [N][K] matrix.
 *   asym g64:  w = scale * q + min,  scale/min f16 at sm[(n*(K/64) + k/64)*2 + {0,1}]
 *   sym g128:  w = scale * (q - 8),  scale f16 at sm[n*(K/128) + k/128]
 *   fp8 b128:  w = e4m3(q[n][k]) * scale, scale float32 at
 *              ((const float *)sm)[(n/128)*(K/128) + k/128] (one per block of
 *              128 rows x 128 inputs), codes one byte per weight
 *   nvfp4:     w = e2m1(q) * e4m3(((const uint8_t *)sm)[n*(K/16) + k/16]),
 *              nibbles packed as the int4 formats; the matrix's global scale
 *              is applied by the caller
 * All are exact in double (at most 15 + 40, or 4 + 24, significant bits). */
static double weight(int fmt, const uint8_t *q, const uint16_t *sm, int K, int n, int k)
{
    if (fmt == ORACLE_FMT_NVFP4) {
        const uint8_t *sb = (const uint8_t *)sm;
        return oracle_e2m1_value((uint8_t)nibble(q + (size_t)n * (K / 2), k)) *
               oracle_e4m3_value(sb[(size_t)n * (K / 16) + k / 16]);
    }
    if (fmt == ORACLE_FMT_FP8_B128) {
        const float *bs = (const float *)sm;
        return oracle_e4m3_value(q[(size_t)n * K + k]) * (double)bs[(size_t)(n / 128) * (K / 128) + k / 128];
    }
    int g = group_of(fmt);
    int code = nibble(q + (size_t)n * (K / 2), k);
    size_t gi = (size_t)n * (K / g) + (size_t)(k / g);
    if (fmt == ORACLE_FMT_ASYM_G64)
        return (double)code * oracle_f16_value(sm[2 * gi]) + oracle_f16_value(sm[2 * gi + 1]);
    return (double)(code - 8) * oracle_f16_value(sm[gi]);
}

/* Dequantise one [N][K] matrix to float32 (the exact value times the
 * matrix's global scale, rounded once; the global scale is used by NVFP4
 * only, the other formats have none). */
int oracle_dequant_global(int fmt, const uint8_t *q, const uint16_t *sm, float global, int N, int K, float *out)
{
    if (!known_fmt(fmt) || K % group_of(fmt) || (fmt == ORACLE_FMT_FP8_B128 && N % 128))
        return -1;
    double g = fmt == ORACLE_FMT_NVFP4 ? (double)global : 1.0;
    for (int n = 0; n < N; n++)
        for (int k = 0; k < K; k++)
            out[(size_t)n * K + k] = (float)(weight(fmt, q, sm, K, n, k) * g);
    return 0;
}

int oracle_dequant(int fmt, const uint8_t *q, const uint16_t *sm, int N, int K, float *out)
{
    return oracle_dequant_global(fmt, q, sm, 1.0f, N, K, out);
}

/* ---------------------------------------------------------------- router */

/* logits[t][e] = bf16( float( sum_h x[t][h] * Wr[e][h] + bias[e] ) ).
 * The products of two bf16 numbers are exact in double and the sum is taken
 * in double, so the value before the two final roundings does not depend on
 * the order of summation for inputs of ordinary magnitude. */
void oracle_router(const uint16_t *x, const uint16_t *wr, const float *bias,
                   int64_t T, int H, int E, uint16_t *logits)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; t++)
        for (int e = 0; e < E; e++) {
            double acc = 0.0;
            for (int h = 0; h < H; h++)
                acc += oracle_bf16_value(x[t * H + h]) * oracle_bf16_value(wr[(size_t)e * H + h]);
            if (bias)
                acc += (double)bias[e];
            logits[t * E + e] = oracle_bf16_round((float)acc);
        }
}

/* ----------------------------------------------------------------- top-k */

static double logit_value(uint16_t b)
{
    double v = oracle_bf16_value(b);
    return isnan(v) ? -INFINITY : v;  /* a NaN logit ranks as -inf (ties with it by index) */
}

/* k rounds of "largest remaining logit, lowest expert index among equals";
 * gates = exp(l_i - l_0) / sum_j exp(l_j - l_0) over the k selected. */
void oracle_topk(const uint16_t *logits, int64_t T, int E, int k, int32_t *idx, float *gate)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; t++) {
        const uint16_t *l = logits + t * E;
        char *taken = calloc((size_t)E, 1);
        for (int i = 0; i < k; i++) {
            int best = -1;
            double bv = 0.0;
            for (int e = 0; e < E; e++) {
                if (taken[e])
                    continue;
                double v = logit_value(l[e]);
                if (best < 0 || v > bv) {            /* strict: equal keeps lower e */
                    best = e;
                    bv = v;
                }
            }
            taken[best] = 1;
            idx[t * k + i] = best;
        }
        free(taken);
        double l0 = logit_value(l[idx[t * k]]);
        double den = 0.0;
        for (int j = 0; j < k; j++)
            den += exp(logit_value(l[idx[t * k + j]]) - l0);
        for (int i = 0; i < k; i++)
            gate[t * k + i] = (float)(exp(logit_value(l[idx[t * k + i]]) - l0) / den);
    }
}

/* ---------------------------------------------------------------- group */

/* Stable counting sort of the T*k (token, slot) pairs by routed expert.
 *   cnt[e]      number of pairs routed to e
 *   off[e]      exclusive prefix sum of cnt, off[E] = T*k
 *   perm[r]     the pair (t*k + i) at sorted position r; pairs of one expert
 *               appear in (t, i) order
 *   inv[t*k+i]  sorted position of pair (t, i)  */
int oracle_group(const int32_t *idx, int64_t T, int k, int E,
                 int32_t *cnt, int32_t *off, int32_t *perm, int32_t *inv)
{
    int64_t P = T * k;
    for (int e = 0; e < E; e++)
        cnt[e] = 0;
    for (int64_t p = 0; p < P; p++) {
        if (idx[p] < 0 || idx[p] >= E)
            return -1;
        cnt[idx[p]]++;
    }
    off[0] = 0;
    for (int e = 0; e < E; e++)
        off[e + 1] = off[e] + cnt[e];
    int32_t *next = malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    for (int e = 0; e < E; e++)
        next[e] = off[e];
    for (int64_t p = 0; p < P; p++) {
        int e = idx[p];
        perm[next[e]] = (int32_t)p;
        inv[p] = next[e];
        next[e]++;
    }
    free(next);
    return 0;
}

/* --------------------------------------------------------------- experts */

static double silu(double a) { return a / (1.0 + exp(-a)); }

/*
 * y[j][:] for the tokens listed in tok[0..ntok) (tok == NULL: all T tokens,
 * tok[j] = j), given the routing idx[T][k] and gates gate[T][k]:
 *   a = Wg[e] x_t,  b = Wu[e] x_t,  h = silu(a) * b,  o = Wd[e] h   (per pair)
 *   y[t] = float( sum_{i = 0..k-1} gate[t][i] * o(t, i) )        (slot order)
 * Each expert that a listed token uses is dequantised (exactly, in double)
 * once, then applied to every listed (token, slot) routed to it.
 * Layout of the code tensors: [E][N][K/2] bytes (int4, NVFP4) or [E][N][K]
 * (fp8); scales as in weight(), one matrix after another; NVFP4 global
 * scales glob[E][2] = {gate and up, down} (NULL for the other formats).
 */
int oracle_experts(int fmt, int E, int H, int I,
                   const uint8_t *gate_q, const uint8_t *up_q, const uint8_t *down_q,
                   const uint16_t *gate_sm, const uint16_t *up_sm, const uint16_t *down_sm,
                   const uint16_t *x, const int32_t *idx, const float *gate,
                   int64_t T, int k, const int64_t *tok, int64_t ntok, float *y, const float *glob)
{
    int g = group_of(fmt);
    if (!known_fmt(fmt) || H % g || I % g || (fmt == ORACLE_FMT_NVFP4 && !glob))
        return -1;
    if (!tok)
        ntok = T;
    for (int64_t j = 0; j < ntok; j++) {
        int64_t t = tok ? tok[j] : j;
        if (t < 0 || t >= T)
            return -1;
        for (int i = 0; i < k; i++)
            if (idx[t * k + i] < 0 || idx[t * k + i] >= E)
                return -1;
    }
    size_t gu_bytes = (size_t)I * (H / 2), d_bytes = (size_t)H * (I / 2);
    size_t gu_sm = (size_t)I * (H / g) * (fmt == ORACLE_FMT_ASYM_G64 ? 2 : 1);
    size_t d_sm = (size_t)H * (I / g) * (fmt == ORACLE_FMT_ASYM_G64 ? 2 : 1);
    if (fmt == ORACLE_FMT_FP8_B128) {  /* bytes per code; float scales counted in 16-bit units */
        gu_bytes = (size_t)I * H;
        d_bytes = (size_t)H * I;
        gu_sm = (size_t)(I / 128) * (H / 128) * 2;
        d_sm = (size_t)(H / 128) * (I / 128) * 2;
    }
    if (fmt == ORACLE_FMT_NVFP4) {  /* one byte per 16 weights, counted in 16-bit units */
        gu_sm = (size_t)I * (H / 16) / 2;
        d_sm = (size_t)H * (I / 16) / 2;
    }
    /* o[j][i][d] for every listed (token, slot) */
    double *o = calloc((size_t)ntok * k * H, sizeof(double));
    if (!o)
        return -2;
    int failed = 0;
#pragma omp parallel
    {
        double *wg = malloc(sizeof(double) * (size_t)I * H);
        double *wu = malloc(sizeof(double) * (size_t)I * H);
        double *wd = malloc(sizeof(double) * (size_t)H * I);
        double *xt = malloc(sizeof(double) * (size_t)H);
        double *h = malloc(sizeof(double) * (size_t)I);
        if (!wg || !wu || !wd || !xt || !h) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int e = 0; e < E; e++) {
            if (failed)
                continue;
            int used = 0;
            for (int64_t j = 0; j < ntok && !used; j++) {
                int64_t t = tok ? tok[j] : j;
                for (int i = 0; i < k; i++)
                    used |= idx[t * k + i] == e;
            }
            if (!used)
                continue;
            const uint8_t *gq = gate_q + e * gu_bytes, *uq = up_q + e * gu_bytes, *dq = down_q + e * d_bytes;
            const uint16_t *gs = gate_sm + e * gu_sm, *us = up_sm + e * gu_sm, *ds = down_sm + e * d_sm;
            double ggu = fmt == ORACLE_FMT_NVFP4 ? (double)glob[2 * e] : 1.0;
            double gd = fmt == ORACLE_FMT_NVFP4 ? (double)glob[2 * e + 1] : 1.0;
            for (int n = 0; n < I; n++)
                for (int kk = 0; kk < H; kk++) {
                    wg[(size_t)n * H + kk] = weight(fmt, gq, gs, H, n, kk) * ggu;
                    wu[(size_t)n * H + kk] = weight(fmt, uq, us, H, n, kk) * ggu;
                }
            for (int d = 0; d < H; d++)
                for (int n = 0; n < I; n++)
                    wd[(size_t)d * I + n] = weight(fmt, dq, ds, I, d, n) * gd;
            for (int64_t j = 0; j < ntok; j++) {
                int64_t t = tok ? tok[j] : j;
                for (int i = 0; i < k; i++) {
                    if (idx[t * k + i] != e)
                        continue;
                    for (int kk = 0; kk < H; kk++)
                        xt[kk] = oracle_bf16_value(x[t * H + kk]);
                    for (int n = 0; n < I; n++) {
                        double a = 0.0, b = 0.0;
                        for (int kk = 0; kk < H; kk++) {
                            a += wg[(size_t)n * H + kk] * xt[kk];
                            b += wu[(size_t)n * H + kk] * xt[kk];
                        }
                        h[n] = silu(a) * b;
                    }
                    double *od = o + ((size_t)j * k + i) * H;
                    for (int d = 0; d < H; d++) {
                        double acc = 0.0;
                        for (int n = 0; n < I; n++)
                            acc += wd[(size_t)d * I + n] * h[n];
                        od[d] = acc;
                    }
                }
            }
        }
        free(wg);
        free(wu);
        free(wd);
        free(xt);
        free(h);
    }
    if (failed) {
        free(o);
        return -2;
    }
    for (int64_t j = 0; j < ntok; j++) {
        int64_t t = tok ? tok[j] : j;
        for (int d = 0; d < H; d++) {
            double acc = 0.0;
            for (int i = 0; i < k; i++)
                acc += (double)gate[t * k + i] * o[((size_t)j * k + i) * H + d];
            y[(size_t)j * H + d] = (float)acc;
        }
    }
    free(o);
    return 0;
}

/* --------------------------------------------------------- shared expert */

/*
 * The shared expert's linears are int8, symmetric, group 128 (drama-q4 card,
 * "What's quantized": attention / DeltaNet / shared expert / codebook decoder
 * linears): one f16 scale per 128 input weights and w = scale * q with q a
 * signed byte.  Layout: q [N][K] int8 with k contiguous, scales [N][K/128]
 * f16.  scale * q is exact in binary32 (11 + 8 significant bits).
 */
static double weight_int8(const int8_t *q, const uint16_t *s, int K, int n, int k)
{
    return oracle_f16_value(s[(size_t)n * (K / 128) + k / 128]) * (double)q[(size_t)n * K + k];
}

int oracle_dequant_int8(const int8_t *q, const uint16_t *s, int N, int K, float *out)
{
    if (N < 1 || K < 128 || K % 128)
        return -1;
    for (int n = 0; n < N; n++)
        for (int k = 0; k < K; k++)
            out[(size_t)n * K + k] = (float)weight_int8(q, s, K, n, k);
    return 0;
}

/*
 * The shared expert of a layer, which every token passes through (the pages
 * name no gate for it, so its output is added as is):
 *   a = Wg x_t,  b = Wu x_t,  h = silu(a) * b,  o = Wd h,
 *   y[j] = float( y_in[j] + o )   (y_in == NULL: 0)
 * for the tokens tok[0..ntok) (tok == NULL: all T), Wg / Wu [I][H] and
 * Wd [H][I] in int8 symmetric group 128.
 */
int oracle_shared(int H, int I, const int8_t *gate_q, const int8_t *up_q, const int8_t *down_q,
                  const uint16_t *gate_s, const uint16_t *up_s, const uint16_t *down_s,
                  const uint16_t *x, int64_t T, const int64_t *tok, int64_t ntok,
                  const float *y_in, float *y)
{
    if (H < 128 || I < 128 || H % 128 || I % 128)
        return -1;
    if (!tok)
        ntok = T;
    for (int64_t j = 0; j < ntok; j++)
        if (tok && (tok[j] < 0 || tok[j] >= T))
            return -1;
    double *wg = malloc(sizeof(double) * (size_t)I * H);
    double *wu = malloc(sizeof(double) * (size_t)I * H);
    double *wd = malloc(sizeof(double) * (size_t)H * I);
    if (!wg || !wu || !wd) {
        free(wg);
        free(wu);
        free(wd);
        return -2;
    }
    for (int n = 0; n < I; n++)
        for (int k = 0; k < H; k++) {
            wg[(size_t)n * H + k] = weight_int8(gate_q, gate_s, H, n, k);
            wu[(size_t)n * H + k] = weight_int8(up_q, up_s, H, n, k);
        }
    for (int d = 0; d < H; d++)
        for (int n = 0; n < I; n++)
            wd[(size_t)d * I + n] = weight_int8(down_q, down_s, I, d, n);
    int failed = 0;
#pragma omp parallel
    {
        double *xt = malloc(sizeof(double) * (size_t)H);
        double *h = malloc(sizeof(double) * (size_t)I);
        if (!xt || !h) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t j = 0; j < ntok; j++) {
            if (failed)
                continue;
            int64_t t = tok ? tok[j] : j;
            for (int k = 0; k < H; k++)
                xt[k] = oracle_bf16_value(x[t * H + k]);
            for (int n = 0; n < I; n++) {
                double a = 0.0, b = 0.0;
                for (int k = 0; k < H; k++) {
                    a += wg[(size_t)n * H + k] * xt[k];
                    b += wu[(size_t)n * H + k] * xt[k];
                }
                h[n] = b * silu(a);
            }
            for (int d = 0; d < H; d++) {
                double acc = y_in ? (double)y_in[(size_t)j * H + d] : 0.0;
                for (int n = 0; n < I; n++)
                    acc += h[n] * wd[(size_t)d * I + n];
                y[(size_t)j * H + d] = (float)acc;
            }
        }
        free(xt);
        free(h);
    }
    free(wg);
    free(wu);
    free(wd);
    return failed ? -2 : 0;
}

/* ------------------------------------------------------------- residual */

/* Next layer's input in a chain of layers: x' = bf16( float(x) + y ), the
 * sum taken in binary32 (one rounding), then rounded to bf16. */
void oracle_residual(const uint16_t *x, const float *y, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; i++) {
        float s = (float)oracle_bf16_value(x[i]) + y[i];
        out[i] = oracle_bf16_round(s);
    }
}
