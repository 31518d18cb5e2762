/*
 * CPU oracle for the block-scaled fp8 GEMM path.  TEST INFRASTRUCTURE ONLY:
 * the tests, the smoke check and the CPU-baseline leg of the benchmark are the
 * only callers.  The GPU library never links, loads or calls this file, and
 * this file includes nothing from the GPU library.
 *
 * Plain, slow and written from the definitions.  Every floating-point result
 * is either exact or computed in fp64 and rounded once, except where the
 * method itself fixes an fp32 step (the quantisation scale and the quotient
 * a/s, which the method defines as fp32 arithmetic).
 *
 * Sources (the r9700-stack release pages):
 *   - "v0.3.1: decode step 16.4 -> 15.0 ms ...", section "What changed for
 *     someone running it": the dense fp8 block GEMM whose per-token-group-128
 *     activation quant runs inside the GEMM's A-load (r9k_gemm_fp8_block_qa),
 *     with bit-identical operands to the split (separate quant) form.
 *   - "v0.3.2: KV cache +14% ...", section "What changed for someone running
 *     it": weights quantised to fp8 once at load, bf16 copies freed; the fp8
 *     kernels used to 255 rows, the tiled fp8 GEMMs above.
 *   - "v0.3.3: the October 12 vLLM nightly pin ...", section "What changed for
 *     someone running it": the MoE decode path with silu(gate)*up in the
 *     gate_up GEMM's epilogue and the fp8 row quant inside the down GEMM's
 *     A-load, bit-identical to the three-launch path.
 * The pages name the operations but not the number format; the readings taken
 * (OCP e4m3fn, 128x128 weight blocks, scale = max(amax, 1e-10f)/448 in fp32,
 * quotient rounded to fp32 then to e4m3 with ties to even and saturation at
 * +-448, bf16 outputs rounded to nearest even) are the workload's stated rules.
 *
 * Build: gcc -O2 -std=c11 -fno-fast-math -ffp-contract=off -fPIC -shared -pthread
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* small helpers                                                             */
/* ------------------------------------------------------------------------ */

static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* Run fn(lo, hi, ctx) over [0, n) split in contiguous chunks on nthreads
 * threads.  Results never depend on the split: every output element is
 * computed by exactly one call and in a fixed order inside it. */
typedef void (*range_fn)(int64_t lo, int64_t hi, void *ctx);
struct range_job { range_fn fn; void *ctx; int64_t lo, hi; };
static void *range_trampoline(void *p) {
    struct range_job *j = (struct range_job *)p;
    j->fn(j->lo, j->hi, j->ctx);
    return NULL;
}
static void parallel_for(int64_t n, int nthreads, range_fn fn, void *ctx) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (n < nthreads) nthreads = n > 0 ? (int)n : 1;
    if (nthreads == 1) { fn(0, n, ctx); return; }
    pthread_t th[256];
    struct range_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t].fn = fn;
        jobs[t].ctx = ctx;
        jobs[t].lo = n * t / nthreads;
        jobs[t].hi = n * (t + 1) / nthreads;
        pthread_create(&th[t], NULL, range_trampoline, &jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------------------ */
/* O1: fp8 e4m3fn (OCP 8-bit floating point, E4M3 with no infinities)        */
/* ------------------------------------------------------------------------ */

/* Value of an e4m3fn code: sign bit, 4 exponent bits (bias 7), 3 mantissa
 * bits.  Exponent field 0 encodes subnormals m/8 * 2^-6; S.1111.111 is NaN;
 * everything else is normal (1 + m/8) * 2^(e-7).  Largest finite 0x7E = 448. */
double ora_e4m3_value(uint8_t code) {
    int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* Encode an fp32 value: round to the nearest e4m3fn value with ties to the
 * even mantissa, saturating at +-448 (so +-inf also give +-448) and keeping
 * the sign of zero; NaN gives 0x7F.
 * Below 2^-6 the grid spacing is 2^-9 (subnormals); in [2^E, 2^(E+1)) with
 * E >= -6 it is 2^(E-3).  Rounding |x| / spacing to an integer with ties to
 * even picks the even mantissa because the integer is 8 + mantissa (normal) or
 * the mantissa itself (subnormal). */
uint8_t ora_e4m3_encode(float x) {
    if (isnan(x)) return 0x7F;
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    double ax = fabs((double)x);
    if (ax >= 448.0) return sign | 0x7E;
    int e2;
    (void)frexp(ax, &e2);          /* ax in [2^(e2-1), 2^e2) */
    int E = e2 - 1;
    if (ax == 0.0 || E < -6) E = -6;
    double spacing = ldexp(1.0, E - 3);
    double n = rint(ax / spacing);  /* exact quotient; rint rounds ties to even */
    double v = n * spacing;         /* the rounded magnitude, on the e4m3 grid */
    if (v == 0.0) return sign;
    if (v < ldexp(1.0, -6)) return sign | (uint8_t)n;  /* subnormal code = n */
    (void)frexp(v, &e2);
    int Ev = e2 - 1;
    int mant = (int)(ldexp(v, -Ev) * 8.0) - 8;       /* exact: v = (1+mant/8) 2^Ev */
    return sign | (uint8_t)(((Ev + 7) << 3) | mant);
}

struct enc_ctx { const float *x; uint8_t *out; };
static void enc_range(int64_t lo, int64_t hi, void *p) {
    struct enc_ctx *c = (struct enc_ctx *)p;
    for (int64_t i = lo; i < hi; ++i) c->out[i] = ora_e4m3_encode(c->x[i]);
}
void ora_e4m3_encode_array(const float *x, int64_t n, uint8_t *out, int nthreads) {
    struct enc_ctx c = {x, out};
    parallel_for(n, nthreads, enc_range, &c);
}

/* ------------------------------------------------------------------------ */
/* O2: bf16 (the upper 16 bits of an IEEE binary32)                           */
/* ------------------------------------------------------------------------ */

float ora_bf16_value(uint16_t b) { return f32_from_bits((uint32_t)b << 16); }

/* Round a binary64 value to bf16 with ties to even, in one step from the
 * source precision.  bf16 has 8 significant bits and binary32's exponent
 * range: spacing 2^(E-7) in [2^E, 2^(E+1)) for E >= -126, and 2^-133 below
 * 2^-126 (subnormals).  A result of 2^128 or more overflows to infinity. */
uint16_t ora_bf16_round(double x) {
    if (isnan(x)) return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0x0000;
    double ax = fabs(x);
    if (isinf(ax)) return sign | 0x7F80;
    if (ax == 0.0) return sign;
    int e2;
    (void)frexp(ax, &e2);
    int E = e2 - 1;
    if (E < -126) E = -126;
    double spacing = ldexp(1.0, E - 7);
    double v = rint(ax / spacing) * spacing;
    if (v >= ldexp(1.0, 128)) return sign | 0x7F80;
    return sign | (uint16_t)(bits_from_f32((float)v) >> 16); /* v is a bf16 value */
}

struct bfr_ctx { const double *x; uint16_t *out; };
static void bfr_range(int64_t lo, int64_t hi, void *p) {
    struct bfr_ctx *c = (struct bfr_ctx *)p;
    for (int64_t i = lo; i < hi; ++i) c->out[i] = ora_bf16_round(c->x[i]);
}
void ora_bf16_round_array(const double *x, int64_t n, uint16_t *out, int nthreads) {
    struct bfr_ctx c = {x, out};
    parallel_for(n, nthreads, bfr_range, &c);
}

/* ------------------------------------------------------------------------ */
/* O3 / O4: group quantisation                                               */
/* ------------------------------------------------------------------------ */

/* One quantisation group: the values v[0..n) (bf16, read through `stride`)
 * share one fp32 scale s = max(amax, 1e-10f) / 448 (an fp32 division), and
 * each value becomes enc(a / s) with the quotient an fp32 division.  amax is
 * exact: the largest |v| of the group. */
static float quant_group(const uint16_t *v, int64_t n, int64_t stride, uint8_t *q, int64_t qstride) {
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(ora_bf16_value(v[i * stride]));
        if (a > amax) amax = a;
    }
    const float eps = 1e-10f;
    float s = (amax > eps ? amax : eps) / 448.0f;
    for (int64_t i = 0; i < n; ++i) {
        float a = ora_bf16_value(v[i * stride]);
        float quot = a / s;
        q[i * qstride] = ora_e4m3_encode(quot);
    }
    return s;
}

/* Activation quant: row m, group g = columns [128g, 128g+128) of that row.
 * a, q: [M][K] row-major; s: [M][K/128] row-major.  K must be a multiple of
 * 128 (the caller checks). */
struct qa_ctx { const uint16_t *a; int64_t K; uint8_t *q; float *s; };
static void qa_range(int64_t lo, int64_t hi, void *p) {
    struct qa_ctx *c = (struct qa_ctx *)p;
    int64_t G = c->K / 128;
    for (int64_t r = lo; r < hi; ++r)
        for (int64_t g = 0; g < G; ++g)
            c->s[r * G + g] = quant_group(c->a + r * c->K + 128 * g, 128, 1, c->q + r * c->K + 128 * g, 1);
}
void ora_quant_act(const uint16_t *a, int64_t M, int64_t K, uint8_t *q, float *s, int nthreads) {
    struct qa_ctx c = {a, K, q, s};
    parallel_for(M, nthreads, qa_range, &c);
}

/* Weight quant: one group per 128x128 block of W [N][K]; the group's scale
 * goes to s[N/128][K/128].  Same scale and encode rule as the activations. */
struct qw_ctx { const uint16_t *w; int64_t K; uint8_t *q; float *s; };
static void qw_range(int64_t lo, int64_t hi, void *p) {
    struct qw_ctx *c = (struct qw_ctx *)p;
    int64_t GK = c->K / 128;
    for (int64_t bn = lo; bn < hi; ++bn) {
        for (int64_t bk = 0; bk < GK; ++bk) {
            const uint16_t *blk = c->w + bn * 128 * c->K + bk * 128;
            float amax = 0.0f;
            for (int r = 0; r < 128; ++r)
                for (int k = 0; k < 128; ++k) {
                    float a = fabsf(ora_bf16_value(blk[r * c->K + k]));
                    if (a > amax) amax = a;
                }
            const float eps = 1e-10f;
            float s = (amax > eps ? amax : eps) / 448.0f;
            c->s[bn * GK + bk] = s;
            for (int r = 0; r < 128; ++r)
                for (int k = 0; k < 128; ++k) {
                    float a = ora_bf16_value(blk[r * c->K + k]);
                    c->q[(bn * 128 + r) * c->K + bk * 128 + k] = ora_e4m3_encode(a / s);
                }
        }
    }
}
void ora_quant_weight(const uint16_t *w, int64_t N, int64_t K, uint8_t *q, float *s, int nthreads) {
    struct qw_ctx c = {w, K, q, s};
    parallel_for(N / 128, nthreads, qw_range, &c);
}

/* ------------------------------------------------------------------------ */
/* O5: the block-scaled GEMM                                                 */
/* ------------------------------------------------------------------------ */

static double g_e4m3_table[256];
static pthread_once_t g_table_once = PTHREAD_ONCE_INIT;
static void build_table(void) {
    for (int c = 0; c < 256; ++c) g_e4m3_table[c] = ora_e4m3_value((uint8_t)c);
}
static const double *e4m3_table(void) {
    pthread_once(&g_table_once, build_table);
    return g_e4m3_table;
}

/* C[m][n] before rounding: sum over K-groups g (ascending) of
 *   P(m,n,g) * as[m][g] * ws[n/128][g],  P = sum_{k in g} dec(aq[m,k]) dec(wq[n,k]).
 * Each fp8 product is exact in binary64 and the 128-term sum is a multiple of
 * 2^-18 below 2^25, so P is exact whatever the order; the cross-group sum is
 * binary64, rounded to bf16 once by the caller. */
static double gemm_elem(const double *T, const uint8_t *arow, const float *asrow, const uint8_t *wrow,
                        const float *wsrow, int64_t K) {
    int64_t G = K / 128;
    double acc = 0.0;
    for (int64_t g = 0; g < G; ++g) {
        double P = 0.0;
        for (int k = 0; k < 128; ++k) P += T[arow[128 * g + k]] * T[wrow[128 * g + k]];
        acc += P * (double)asrow[g] * (double)wsrow[g];
    }
    return acc;
}

struct gemm_ctx {
    const uint8_t *aq; const float *as; int64_t M, K;
    const uint8_t *wq; const float *ws; int64_t N;
    uint16_t *c; double *c64;
    const int64_t *ms, *ns;
};
static void gemm_range(int64_t lo, int64_t hi, void *p) {
    struct gemm_ctx *c = (struct gemm_ctx *)p;
    const double *T = e4m3_table();
    int64_t G = c->K / 128;
    for (int64_t idx = lo; idx < hi; ++idx) {
        int64_t m = idx / c->N, n = idx % c->N;
        double v = gemm_elem(T, c->aq + m * c->K, c->as + m * G, c->wq + n * c->K, c->ws + (n / 128) * G, c->K);
        if (c->c64) c->c64[idx] = v;
        if (c->c) c->c[idx] = ora_bf16_round(v);
    }
}
/* aq [M][K], as [M][K/128], wq [N][K], ws [N/128][K/128] -> c [M][N] bf16 and
 * (if c64 is not NULL) the unrounded binary64 values. */
void ora_gemm_block(const uint8_t *aq, const float *as, int64_t M, int64_t K, const uint8_t *wq,
                    const float *ws, int64_t N, uint16_t *c, double *c64, int nthreads) {
    struct gemm_ctx ctx = {aq, as, M, K, wq, ws, N, c, c64, NULL, NULL};
    parallel_for(M * N, nthreads, gemm_range, &ctx);
}

static void gemm_at_range(int64_t lo, int64_t hi, void *p) {
    struct gemm_ctx *c = (struct gemm_ctx *)p;
    const double *T = e4m3_table();
    int64_t G = c->K / 128;
    for (int64_t i = lo; i < hi; ++i) {
        int64_t m = c->ms[i], n = c->ns[i];
        double v = gemm_elem(T, c->aq + m * c->K, c->as + m * G, c->wq + n * c->K, c->ws + (n / 128) * G, c->K);
        if (c->c64) c->c64[i] = v;
        if (c->c) c->c[i] = ora_bf16_round(v);
    }
}
/* The same definition evaluated at cnt sampled positions (ms[i], ns[i]). */
void ora_gemm_block_at(const uint8_t *aq, const float *as, int64_t M, int64_t K, const uint8_t *wq,
                       const float *ws, int64_t N, const int64_t *ms, const int64_t *ns, int64_t cnt,
                       uint16_t *c, double *c64, int nthreads) {
    (void)M;
    struct gemm_ctx ctx = {aq, as, M, K, wq, ws, N, c, c64, ms, ns};
    parallel_for(cnt, nthreads, gemm_at_range, &ctx);
}

/* ------------------------------------------------------------------------ */
/* O6: MoE decode                                                            */
/* ------------------------------------------------------------------------ */

/* Token t, slot j goes to expert e = ids[t][j] with weight w[t][j].
 *   x [T][H] bf16 -> xq, xs (activation quant over H)
 *   gu = bf16(GEMM row of xq[t] against w13[e] [2I][H])   (rows [0,I) gate, [I,2I) up)
 *   h[i] = bf16(silu(gu[i]) * gu[I+i]),  silu(z) = z / (1 + exp(-z)) in binary64
 *   hq, hs = activation quant of h over I
 *   y = GEMM row of hq against w2[e] [H][I], binary64, not rounded
 *   out[t] = bf16(sum_j w[t][j] * y(t, j)), j ascending, binary64.
 * A slot whose id lies outside [0, E) names no expert: it is skipped in the
 * sum, and its intermediates are written as zeros (the reading that such a
 * slot contributes nothing).
 * Intermediates are written per pair p = t*topk + j when the pointers are not
 * NULL: gu [P][2I] bf16, h [P][I] bf16, hq [P][I], hs [P][I/128], y [P][H]. */
/* h[i] = bf16(silu(gate[i]) * up[i]) for one pair, gate = gu[0..I), up =
 * gu[I..2I), silu(z) = z / (1 + exp(-z)), all in binary64, rounded once. */
static void silu_mul_row(const uint16_t *gu, int64_t I, uint16_t *h) {
    for (int64_t i = 0; i < I; ++i) {
        double g = (double)ora_bf16_value(gu[i]);
        double u = (double)ora_bf16_value(gu[I + i]);
        double silu = g / (1.0 + exp(-g));
        h[i] = ora_bf16_round(silu * u);
    }
}

/* The silu(gate) * up step alone, for P pairs: gu [P][2I] -> h [P][I]. */
void ora_moe_silu_mul(const uint16_t *gu, int64_t P, int64_t I, uint16_t *h) {
    for (int64_t p = 0; p < P; ++p) silu_mul_row(gu + p * 2 * I, I, h + p * I);
}

struct moe_ctx {
    const uint16_t *x; int64_t T, H;
    const int32_t *ids; const float *w; int64_t topk;
    const uint8_t *w13q; const float *w13s; const uint8_t *w2q; const float *w2s; int64_t E, I;
    const uint8_t *xq; const float *xs;
    uint16_t *gu_out, *h_out; uint8_t *hq_out; float *hs_out; double *y;
    const uint16_t *h_in;  /* when not NULL, the down stage reads these h rows */
};
static void moe_pair_range(int64_t lo, int64_t hi, void *p) {
    struct moe_ctx *c = (struct moe_ctx *)p;
    const double *T = e4m3_table();
    int64_t H = c->H, I = c->I, GH = H / 128, GI = I / 128;
    uint16_t *gu = (uint16_t *)malloc(sizeof(uint16_t) * 2 * I);
    uint16_t *h = (uint16_t *)malloc(sizeof(uint16_t) * I);
    uint8_t *hq = (uint8_t *)malloc(I);
    float *hs = (float *)malloc(sizeof(float) * GI);
    for (int64_t pr = lo; pr < hi; ++pr) {
        int64_t t = pr / c->topk;
        int64_t e = c->ids[pr];
        if (e < 0 || e >= c->E) {  /* no expert: zero intermediates, nothing read */
            for (int64_t n = 0; n < H; ++n) c->y[pr * H + n] = 0.0;
            if (c->gu_out && !c->h_in) memset(c->gu_out + pr * 2 * I, 0, sizeof(uint16_t) * 2 * I);
            if (c->h_out) memset(c->h_out + pr * I, 0, sizeof(uint16_t) * I);
            if (c->hq_out) memset(c->hq_out + pr * I, 0, I);
            if (c->hs_out) memset(c->hs_out + pr * GI, 0, sizeof(float) * GI);
            continue;
        }
        const uint8_t *w13 = c->w13q + e * 2 * I * H;
        const float *w13s = c->w13s + e * (2 * I / 128) * GH;
        const uint8_t *w2 = c->w2q + e * H * I;
        const float *w2s = c->w2s + e * (H / 128) * GI;
        if (c->h_in) {
            memcpy(h, c->h_in + pr * I, sizeof(uint16_t) * I);
        } else {
            for (int64_t n = 0; n < 2 * I; ++n)
                gu[n] = ora_bf16_round(gemm_elem(T, c->xq + t * H, c->xs + t * GH, w13 + n * H,
                                                 w13s + (n / 128) * GH, H));
            silu_mul_row(gu, I, h);
        }
        for (int64_t g = 0; g < GI; ++g) hs[g] = quant_group(h + 128 * g, 128, 1, hq + 128 * g, 1);
        for (int64_t n = 0; n < H; ++n)
            c->y[pr * H + n] = gemm_elem(T, hq, hs, w2 + n * I, w2s + (n / 128) * GI, I);
        if (c->gu_out && !c->h_in) memcpy(c->gu_out + pr * 2 * I, gu, sizeof(uint16_t) * 2 * I);
        if (c->h_out) memcpy(c->h_out + pr * I, h, sizeof(uint16_t) * I);
        if (c->hq_out) memcpy(c->hq_out + pr * I, hq, I);
        if (c->hs_out) memcpy(c->hs_out + pr * GI, hs, sizeof(float) * GI);
    }
    free(gu); free(h); free(hq); free(hs);
}

static void moe_run(struct moe_ctx *c, uint16_t *out, int nthreads) {
    int64_t T = c->T, H = c->H, P = T * c->topk;
    uint8_t *xq = (uint8_t *)malloc(T * H);
    float *xs = (float *)malloc(sizeof(float) * T * (H / 128));
    ora_quant_act(c->x, T, H, xq, xs, 1);
    c->xq = xq; c->xs = xs;
    int own_y = c->y == NULL;
    if (own_y) c->y = (double *)malloc(sizeof(double) * P * H);
    parallel_for(P, nthreads, moe_pair_range, c);
    for (int64_t t = 0; t < T; ++t)
        for (int64_t n = 0; n < H; ++n) {
            double acc = 0.0;
            for (int64_t j = 0; j < c->topk; ++j) {
                const int32_t e = c->ids[t * c->topk + j];
                if (e < 0 || e >= c->E) continue;
                acc += (double)c->w[t * c->topk + j] * c->y[(t * c->topk + j) * H + n];
            }
            out[t * H + n] = ora_bf16_round(acc);
        }
    if (own_y) { free(c->y); c->y = NULL; }
    free(xq); free(xs);
}

void ora_moe_decode(const uint16_t *x, int64_t T, int64_t H, const int32_t *ids, const float *w, int64_t topk,
                    const uint8_t *w13q, const float *w13s, const uint8_t *w2q, const float *w2s, int64_t E,
                    int64_t I, uint16_t *out, uint16_t *gu, uint16_t *h, uint8_t *hq, float *hs, double *y,
                    int nthreads) {
    struct moe_ctx c;
    memset(&c, 0, sizeof(c));
    c.x = x; c.T = T; c.H = H; c.ids = ids; c.w = w; c.topk = topk;
    c.w13q = w13q; c.w13s = w13s; c.w2q = w2q; c.w2s = w2s; c.E = E; c.I = I;
    c.gu_out = gu; c.h_out = h; c.hq_out = hq; c.hs_out = hs; c.y = y;
    moe_run(&c, out, nthreads);
}

/* The down stage and the combine alone, from given h rows [T*topk][I] (for
 * checking a GPU's down stage against its own h). */
void ora_moe_down_from_h(const uint16_t *h_in, int64_t T, int64_t H, const int32_t *ids, const float *w,
                         int64_t topk, const uint8_t *w2q, const float *w2s, int64_t E, int64_t I,
                         uint16_t *out, uint8_t *hq, float *hs, double *y, int nthreads) {
    struct moe_ctx c;
    memset(&c, 0, sizeof(c));
    uint16_t *dummy_x = (uint16_t *)calloc((size_t)(T * H), sizeof(uint16_t));
    c.x = dummy_x; c.T = T; c.H = H; c.ids = ids; c.w = w; c.topk = topk;
    c.w2q = w2q; c.w2s = w2s; c.E = E; c.I = I;
    c.hq_out = hq; c.hs_out = hs; c.y = y; c.h_in = h_in;
    moe_run(&c, out, nthreads);
    free(dummy_x);
}

/* ------------------------------------------------------------------------ */
/* MoE routing and the routed sum with the shared expert                     */
/* ------------------------------------------------------------------------ */

/* Routing of T tokens over E experts (release v0.3.0, "What changed for
 * someone running it": one-launch MoE routing).  Token t's experts are its
 * topk largest logits, a larger logit first and equal logits in ascending
 * expert id; the softmax is increasing in the logit, so these are the experts
 * of the topk largest probabilities.  Their weights are those probabilities
 * renormalised over the chosen experts, in which the softmax's denominator
 * cancels:
 *   w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0),  i, j over the chosen slots,
 * l_0 the largest logit, in binary64, rounded once to fp32.
 * Logits must be finite.  ids and w are [T][topk]. */
void ora_moe_route(const float *logits, int64_t T, int64_t E, int64_t topk, int32_t *ids, float *w) {
    char *taken = (char *)malloc((size_t)E);
    double *ex = (double *)malloc(sizeof(double) * (size_t)topk);
    for (int64_t t = 0; t < T; ++t) {
        const float *row = logits + t * E;
        int32_t *id = ids + t * topk;
        memset(taken, 0, (size_t)E);
        for (int64_t j = 0; j < topk; ++j) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; ++e)  /* strict >: the lower id wins a tie */
                if (!taken[e] && (best < 0 || row[e] > row[best])) best = e;
            taken[best] = 1;
            id[j] = (int32_t)best;
        }
        const double l0 = (double)row[id[0]];
        double sum = 0.0;
        for (int64_t j = 0; j < topk; ++j) {
            ex[j] = exp((double)row[id[j]] - l0);
            sum += ex[j];
        }
        for (int64_t j = 0; j < topk; ++j) w[t * topk + j] = (float)(ex[j] / sum);
    }
    free(taken);
    free(ex);
}

/* The routed sum with the shared expert added (release v0.3.0, same section:
 * the fused top-k sum with the shared expert):
 *   out[t][n] = bf16( sum_j w[t][j] * y[t*topk + j][n]  +  g[t] * s[t][n] )
 * with j ascending over the slots whose id lies in [0, E), binary64, rounded
 * once; g[t] = shared_w[t], or 1 when shared_w is NULL; the shared term is
 * absent when s is NULL.  y is [T*topk][H] binary64, s [T][H] bf16. */
void ora_moe_fold(const double *y, const int32_t *ids, const float *w, int64_t T, int64_t topk, int64_t H,
                  int64_t E, const uint16_t *s, const float *shared_w, uint16_t *out) {
    for (int64_t t = 0; t < T; ++t)
        for (int64_t n = 0; n < H; ++n) {
            double acc = 0.0;
            for (int64_t j = 0; j < topk; ++j) {
                const int32_t e = ids[t * topk + j];
                if (e < 0 || e >= E) continue;
                acc += (double)w[t * topk + j] * y[(t * topk + j) * H + n];
            }
            if (s) acc += (shared_w ? (double)shared_w[t] : 1.0) * (double)ora_bf16_value(s[t * H + n]);
            out[t * H + n] = ora_bf16_round(acc);
        }
}

/* ------------------------------------------------------------------------ */
/* The bf16-activation variant: fp8 block weights against unquantised bf16    */
/* activations                                                                */
/* ------------------------------------------------------------------------ */

/* Release v0.3.1, "What changed for someone running it": the decode GEMMs of
 * fp8 weights run against the unquantised bf16 activations.  With the weight
 * block scales applied per 128-K group, as in the block GEMM:
 *   C[m][n] = bf16( sum_g ws[n/128][g] * sum_{k in g} a[m][k] * dec(wq[n][k]) )
 * in binary64 (k and g ascending), rounded once.  A bf16 x e4m3 product is
 * exact in binary64; the sums are not exact in general (bf16 exponents span
 * more than binary64's precision), their error is of binary64's rounding. */
struct gemm_bf16a_ctx {
    const uint16_t *a; int64_t M, K;
    const uint8_t *wq; const float *ws; int64_t N;
    uint16_t *c; double *c64;
};
static void gemm_bf16a_range(int64_t lo, int64_t hi, void *p) {
    struct gemm_bf16a_ctx *c = (struct gemm_bf16a_ctx *)p;
    const double *T = e4m3_table();
    const int64_t K = c->K, G = K / 128;
    for (int64_t idx = lo; idx < hi; ++idx) {
        const int64_t m = idx / c->N, n = idx % c->N;
        const uint16_t *arow = c->a + m * K;
        const uint8_t *wrow = c->wq + n * K;
        const float *wsrow = c->ws + (n / 128) * G;
        double acc = 0.0;
        for (int64_t g = 0; g < G; ++g) {
            double P = 0.0;
            for (int k = 0; k < 128; ++k) P += (double)ora_bf16_value(arow[128 * g + k]) * T[wrow[128 * g + k]];
            acc += P * (double)wsrow[g];
        }
        if (c->c64) c->c64[idx] = acc;
        if (c->c) c->c[idx] = ora_bf16_round(acc);
    }
}
/* a [M][K] bf16, wq [N][K], ws [N/128][K/128] -> c [M][N] bf16 and (if c64 is
 * not NULL) the unrounded binary64 values. */
void ora_gemm_block_bf16a(const uint16_t *a, int64_t M, int64_t K, const uint8_t *wq, const float *ws, int64_t N,
                          uint16_t *c, double *c64, int nthreads) {
    struct gemm_bf16a_ctx ctx = {a, M, K, wq, ws, N, c, c64};
    parallel_for(M * N, nthreads, gemm_bf16a_range, &ctx);
}
