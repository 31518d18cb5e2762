/*
 * Independent re-derivations used to pin the oracle's codecs (tests only).
 *
 * Nothing here shares code with the oracle or with the GPU library.  Each
 * function reaches the same definition by a different route than the oracle
 * does (the oracle scales by a power of two and rounds with rint):
 *   - e4m3 by integer manipulation of the binary32 bit pattern,
 *   - e4m3 by searching all finite e4m3 values for the nearest one,
 *   - bf16 by the integer round-half-even of the low 16 bits.
 *   - the fused multiply-add division correction that a GPU kernel may use
 *     for RN(a/s), checked against the hardware division over every (a, amax)
 *     pair of bf16 values.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

static uint32_t ubits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float fbits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* e4m3 from the binary32 bits.  Normal e4m3 (|x| >= 2^-6): drop 20 mantissa
 * bits with round-half-even on the integer, then rebias the exponent from 127
 * to 7.  Subnormal e4m3: the value is n * 2^-9, n = RNE(|x| * 2^9), computed
 * by shifting the 24-bit significand. */
uint8_t pin_e4m3_encode_bits(float x) {
    uint32_t u = ubits(x);
    uint8_t sign = (uint8_t)((u >> 24) & 0x80);
    u &= 0x7FFFFFFFu;
    if (u > 0x7F800000u) return 0x7F;
    if (u >= 0x43E00000u) return sign | 0x7E; /* |x| >= 448 (incl. inf) */
    if (u >= 0x3C800000u) {                   /* |x| >= 2^-6 */
        uint32_t r = (u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20; /* (exp << 3) | mant, rounded */
        uint32_t code = r - (120u << 3);
        if (code > 0x7E) code = 0x7E; /* cannot happen below 448; kept for safety */
        return sign | (uint8_t)code;
    }
    /* |x| < 2^-6: n = RNE(|x| * 2^9) in 0..8 */
    uint32_t e = u >> 23;
    if (e == 0) return sign; /* binary32 subnormal: far below 2^-10 */
    uint32_t sig = (u & 0x7FFFFFu) | 0x800000u; /* |x| = sig * 2^(e - 150) */
    /* |x| * 2^9 = sig * 2^(e - 141); shift = 141 - e (>= 21 since e <= 120) */
    uint32_t shift = 141u - e;
    if (shift >= 32) return sign;
    uint32_t n = sig >> shift;
    uint32_t rem = sig & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (n & 1u))) n += 1;
    return sign | (uint8_t)n; /* n == 8 is the code of 2^-6 */
}

static double e4m3_mag(int c) { /* value of the non-negative code c (0..0x7E) */
    int e = (c >> 3) & 15, m = c & 7;
    return e == 0 ? m * 0x1p-9 : (8 + m) * ldexp(1.0, e - 10);
}

/* Nearest finite e4m3 value by exhaustive search; equidistant -> even code. */
uint8_t pin_e4m3_encode_search(float x) {
    if (isnan(x)) return 0x7F;
    uint8_t sign = signbit(x) ? 0x80 : 0;
    double ax = fabs((double)x);
    int best = 0;
    double bestd = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        double d = fabs(e4m3_mag(c) - ax);
        if (d < bestd || (d == bestd && (c & 1) == 0)) { bestd = d; best = c; }
    }
    return sign | (uint8_t)best;
}

/* bf16 from binary32 by integer round-half-even of the dropped 16 bits. */
uint16_t pin_bf16_round_bits(float x) {
    uint32_t u = ubits(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

/* ------------------------------------------------------------------------ */

typedef void (*range_fn)(int64_t lo, int64_t hi, void *ctx, int64_t *count);
struct job { range_fn fn; void *ctx; int64_t lo, hi, count; };
static void *tramp(void *p) { struct job *j = p; j->fn(j->lo, j->hi, j->ctx, &j->count); return NULL; }
static int64_t par(int64_t n, int nt, range_fn fn, void *ctx) {
    if (nt < 1) nt = 1;
    if (nt > 128) nt = 128;
    pthread_t th[128];
    struct job jb[128];
    for (int t = 0; t < nt; ++t) {
        jb[t] = (struct job){fn, ctx, n * t / nt, n * (t + 1) / nt, 0};
        pthread_create(&th[t], NULL, tramp, &jb[t]);
    }
    int64_t total = 0;
    for (int t = 0; t < nt; ++t) { pthread_join(th[t], NULL); total += jb[t].count; }
    return total;
}

struct arr { const float *x; void *out; };
static void enc_bits_rng(int64_t lo, int64_t hi, void *p, int64_t *cnt) {
    struct arr *a = p; uint8_t *o = a->out; (void)cnt;
    for (int64_t i = lo; i < hi; ++i) o[i] = pin_e4m3_encode_bits(a->x[i]);
}
static void enc_search_rng(int64_t lo, int64_t hi, void *p, int64_t *cnt) {
    struct arr *a = p; uint8_t *o = a->out; (void)cnt;
    for (int64_t i = lo; i < hi; ++i) o[i] = pin_e4m3_encode_search(a->x[i]);
}
static void bf16_bits_rng(int64_t lo, int64_t hi, void *p, int64_t *cnt) {
    struct arr *a = p; uint16_t *o = a->out; (void)cnt;
    for (int64_t i = lo; i < hi; ++i) o[i] = pin_bf16_round_bits(a->x[i]);
}
void pin_e4m3_encode_bits_array(const float *x, int64_t n, uint8_t *out, int nt) {
    struct arr a = {x, out}; par(n, nt, enc_bits_rng, &a);
}
void pin_e4m3_encode_search_array(const float *x, int64_t n, uint8_t *out, int nt) {
    struct arr a = {x, out}; par(n, nt, enc_search_rng, &a);
}
void pin_bf16_round_bits_array(const float *x, int64_t n, uint16_t *out, int nt) {
    struct arr a = {x, out}; par(n, nt, bf16_bits_rng, &a);
}

/* ------------------------------------------------------------------------ */
/* Division by a group scale with one reciprocal per group, as the GPU       */
/* kernels do it:                                                            */
/*   r = RN(1/s), q0 = RN(a*r), d = fma(q0, s, -a), q = fma(-d, r, q0)        */
/* (Markstein's correction; Muller et al., Handbook of Floating-Point        */
/* Arithmetic, division chapter).  Counted: pairs where the e4m3 code of q     */
/* differs from the e4m3 code of the correctly rounded a/s, over every        */
/* positive bf16 amax (and the eps floor) and every bf16 a with |a| <= amax,  */
/* both signs of a (so -0 too).  The e4m3 codes are taken with               */
/* pin_e4m3_encode_bits.                                                      */
/* ------------------------------------------------------------------------ */
static float div_device_formula(float a, float s, float r) {
    float q0 = a * r;
    float d = fmaf(q0, s, -a);
    return fmaf(-d, r, q0);
}
static void div_rng(int64_t lo, int64_t hi, void *p, int64_t *cnt) {
    (void)p;
    const float eps = 1e-10f;
    int64_t bad = 0;
    for (int64_t ab = lo; ab < hi; ++ab) {      /* ab: bf16 bits of amax, 0 .. 0x7F7F */
        float amax = fbits((uint32_t)ab << 16);
        float s = (amax > eps ? amax : eps) / 448.0f;
        float r = 1.0f / s;
        for (uint32_t xb = 0; xb <= (uint32_t)ab; ++xb) {
            for (int neg = 0; neg < 2; ++neg) {
                float a = fbits((xb << 16) | (neg ? 0x80000000u : 0u));
                if (pin_e4m3_encode_bits(div_device_formula(a, s, r)) != pin_e4m3_encode_bits(a / s)) ++bad;
            }
        }
    }
    *cnt = bad;
}
/* Returns the number of mismatching (a, amax) pairs over amax bits [lo, hi).
 * Row ab costs about ab steps, so the split balances the cumulative cost. */
int64_t pin_div_correction_mismatches(int64_t lo, int64_t hi, int nt) {
    if (nt < 1) nt = 1;
    if (nt > 128) nt = 128;
    pthread_t th[128];
    struct job jb[128];
    double tot = (double)hi * hi - (double)lo * lo;
    int64_t start = lo;
    for (int t = 0; t < nt; ++t) {
        int64_t end = t == nt - 1 ? hi : (int64_t)sqrt((double)lo * lo + tot * (t + 1) / nt);
        if (end < start) end = start;
        if (end > hi) end = hi;
        jb[t] = (struct job){div_rng, NULL, start, end, 0};
        start = end;
    }
    int64_t total = 0;
    for (int t = 0; t < nt; ++t) pthread_create(&th[t], NULL, tramp, &jb[t]);
    for (int t = 0; t < nt; ++t) { pthread_join(th[t], NULL); total += jb[t].count; }
    return total;
}

/* ------------------------------------------------------------------------ */
/* Exhaustive comparison over every binary32 pattern, against a function    */
/* passed in by address (the oracle's encoder), without Python arrays.       */
/* Returns the number of mismatches; *first gets the first mismatching        */
/* pattern (or 0xFFFFFFFF).                                                   */
/* ------------------------------------------------------------------------ */
typedef uint8_t (*enc8_fn)(float);
typedef uint16_t (*enc16_fn)(double);
struct exh { void *fn; int kind; uint32_t first; pthread_mutex_t mu; };
static void exh_rng(int64_t lo, int64_t hi, void *p, int64_t *cnt) {
    struct exh *c = p;
    int64_t bad = 0;
    uint32_t first = 0xFFFFFFFFu;
    for (int64_t i = lo; i < hi; ++i) {
        float x = fbits((uint32_t)i);
        int differ;
        if (c->kind == 0) {
            differ = ((enc8_fn)c->fn)(x) != pin_e4m3_encode_bits(x);
        } else {
            if (isnan(x)) continue;
            differ = ((enc16_fn)c->fn)((double)x) != pin_bf16_round_bits(x);
        }
        if (differ) { if (!bad) first = (uint32_t)i; ++bad; }
    }
    if (bad) {
        pthread_mutex_lock(&c->mu);
        if (first < c->first) c->first = first;
        pthread_mutex_unlock(&c->mu);
    }
    *cnt = bad;
}
int64_t pin_exhaustive(void *fn, int kind, int nt, uint32_t *first) {
    struct exh c;
    c.fn = fn; c.kind = kind; c.first = 0xFFFFFFFFu;
    pthread_mutex_init(&c.mu, NULL);
    int64_t n = par((int64_t)1 << 32, nt, exh_rng, &c);
    *first = c.first;
    return n;
}

/* ------------------------------------------------------------------------ */
/* The group scale as the GPU kernels compute it: x = max(amax, 1e-10f),     */
/* q0 = RN(x * RN(1/448)), e = fma(-q0, 448, x), s = fma(e, RN(1/448), q0).   */
/* Returns how many bf16 amax values (0 .. largest finite) give a different   */
/* s than the correctly rounded x / 448.                                      */
/* ------------------------------------------------------------------------ */
int64_t pin_scale_formula_mismatches(void) {
    const float c = 1.0f / 448.0f, eps = 1e-10f;
    int64_t bad = 0;
    for (uint32_t b = 0; b < 0x7F80u; ++b) {
        float amax = fbits(b << 16);
        float x = amax > eps ? amax : eps;
        float q0 = x * c;
        float e = fmaf(-q0, 448.0f, x);
        float s = fmaf(e, c, q0);
        if (ubits(s) != ubits(x / 448.0f)) ++bad;
    }
    return bad;
}
