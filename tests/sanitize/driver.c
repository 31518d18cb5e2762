/* Runs every entry point of the CPU oracle (oracle/r9k_oracle.c) and of the
 * independent pins (tests/pins/pins.c) on small inputs, including the edge
 * cases the tests feed them (all-zero and -0 groups, subnormal, infinite and
 * NaN encoder inputs, out-of-range MoE expert ids, sampled GEMM positions),
 * so that a build with -fsanitize=address,undefined checks their memory
 * accesses and arithmetic for undefined behaviour.  Test infrastructure only.
 * Exit status 0 when every call returned and the few facts checked here hold. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* oracle */
double ora_e4m3_value(uint8_t code);
uint8_t ora_e4m3_encode(float x);
void ora_e4m3_encode_array(const float *x, int64_t n, uint8_t *out, int nthreads);
float ora_bf16_value(uint16_t b);
uint16_t ora_bf16_round(double x);
void ora_bf16_round_array(const double *x, int64_t n, uint16_t *out, int nthreads);
void ora_quant_act(const uint16_t *a, int64_t M, int64_t K, uint8_t *q, float *s, int nthreads);
void ora_quant_weight(const uint16_t *w, int64_t N, int64_t K, uint8_t *q, float *s, int nthreads);
void ora_gemm_block(const uint8_t *aq, const float *as, int64_t M, int64_t K, const uint8_t *wq, const float *ws,
                    int64_t N, uint16_t *c, double *c64, int nthreads);
void ora_gemm_block_at(const uint8_t *aq, const float *as, int64_t M, int64_t K, const uint8_t *wq,
                       const float *ws, int64_t N, const int64_t *ms, const int64_t *ns, int64_t cnt, uint16_t *c,
                       double *c64, int nthreads);
void ora_moe_silu_mul(const uint16_t *gu, int64_t P, int64_t I, uint16_t *h);
void ora_moe_decode(const uint16_t *x, int64_t T, int64_t H, const int32_t *ids, const float *w, int64_t topk,
                    const uint8_t *w13q, const float *w13s, const uint8_t *w2q, const float *w2s, int64_t E,
                    int64_t I, uint16_t *out, uint16_t *gu, uint16_t *h, uint8_t *hq, float *hs, double *y,
                    int nthreads);
void ora_moe_down_from_h(const uint16_t *h_in, int64_t T, int64_t H, const int32_t *ids, const float *w,
                         int64_t topk, const uint8_t *w2q, const float *w2s, int64_t E, int64_t I, uint16_t *out,
                         uint8_t *hq, float *hs, double *y, int nthreads);
void ora_moe_route(const float *logits, int64_t T, int64_t E, int64_t topk, int32_t *ids, float *w);
void ora_moe_fold(const double *y, const int32_t *ids, const float *w, int64_t T, int64_t topk, int64_t H,
                  int64_t E, const uint16_t *s, const float *shared_w, uint16_t *out);
void ora_gemm_block_bf16a(const uint16_t *a, int64_t M, int64_t K, const uint8_t *wq, const float *ws, int64_t N,
                          uint16_t *c, double *c64, int nthreads);
/* pins */
uint8_t pin_e4m3_encode_bits(float x);
uint8_t pin_e4m3_encode_search(float x);
uint16_t pin_bf16_round_bits(float x);
void pin_e4m3_encode_bits_array(const float *x, int64_t n, uint8_t *out, int nt);
void pin_e4m3_encode_search_array(const float *x, int64_t n, uint8_t *out, int nt);
void pin_bf16_round_bits_array(const float *x, int64_t n, uint16_t *out, int nt);
int64_t pin_div_correction_mismatches(int64_t lo, int64_t hi, int nt);
int64_t pin_scale_formula_mismatches(void);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) { /* xorshift64*, for test data only */
    g_state ^= g_state >> 12; g_state ^= g_state << 25; g_state ^= g_state >> 27;
    return (uint32_t)((g_state * 0x2545F4914F6CDD1Dull) >> 32);
}
static float uniform(void) { return (float)next_u32() / 4294967296.0f * 2.0f - 1.0f; }
static uint16_t bf16_of(float f) { return ora_bf16_round((double)f); }
static void fill_bf16(uint16_t *p, int64_t n, float scale) {
    for (int64_t i = 0; i < n; ++i) p[i] = bf16_of(uniform() * scale);
}
static int g_fail = 0;
#define CHECK(cond) do { if (!(cond)) { fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); g_fail = 1; } } while (0)

int main(void) {
    const int NT = 4;
    /* codecs, scalar and array forms, on special values */
    const float specials[] = {0.0f, -0.0f, 1.0f, -1.0f, 448.0f, 449.0f, 464.0f, 1e30f, -1e30f, INFINITY, -INFINITY,
                              NAN, 1e-40f, -1e-40f, 0.0009765625f, 0.00146484375f, 2.75f, -3.25f};
    const int NS = (int)(sizeof(specials) / sizeof(specials[0]));
    for (int c = 0; c < 256; ++c) (void)ora_e4m3_value((uint8_t)c);
    uint8_t e1[64], e2[64], e3[64];
    uint16_t b1[64];
    for (int i = 0; i < NS; ++i) {
        CHECK(ora_e4m3_encode(specials[i]) == pin_e4m3_encode_bits(specials[i]));
        (void)pin_e4m3_encode_search(specials[i]);
        (void)pin_bf16_round_bits(specials[i]);
        (void)ora_bf16_round((double)specials[i]);
    }
    ora_e4m3_encode_array(specials, NS, e1, NT);
    pin_e4m3_encode_bits_array(specials, NS, e2, NT);
    pin_e4m3_encode_search_array(specials, NS, e3, NT);
    pin_bf16_round_bits_array(specials, NS, b1, NT);
    for (int i = 0; i < NS; ++i) CHECK(e1[i] == e2[i]);
    double d64[NS];
    uint16_t b2[64];
    for (int i = 0; i < NS; ++i) d64[i] = specials[i];
    ora_bf16_round_array(d64, NS, b2, NT);
    for (int i = 0; i < NS; ++i) if (!isnan(specials[i])) CHECK(b2[i] == b1[i]);

    /* quantisation with an all-zero group, a -0 group and a subnormal group */
    enum { M = 3, K = 384, N = 256 };
    uint16_t *a = malloc(sizeof(uint16_t) * M * K), *w = malloc(sizeof(uint16_t) * N * K);
    fill_bf16(a, M * K, 4.0f);
    fill_bf16(w, N * K, 0.05f);
    for (int k = 0; k < 128; ++k) { a[k] = 0x0000; a[K + k] = 0x8000; a[2 * K + 128 + k] = 0x0001; }
    for (int n = 0; n < 128; ++n) for (int k = 128; k < 256; ++k) w[n * K + k] = 0;
    uint8_t *aq = malloc(M * K), *wq = malloc(N * K);
    float *as = malloc(sizeof(float) * M * (K / 128)), *ws = malloc(sizeof(float) * (N / 128) * (K / 128));
    ora_quant_act(a, M, K, aq, as, NT);
    ora_quant_weight(w, N, K, wq, ws, NT);
    for (int k = 0; k < 128; ++k) CHECK(aq[k] == 0x00 && aq[K + k] == 0x80);

    /* GEMM, full and sampled, and the bf16-activation variant */
    uint16_t *c = malloc(sizeof(uint16_t) * M * N), *c2 = malloc(sizeof(uint16_t) * M * N);
    double *c64 = malloc(sizeof(double) * M * N), *s64 = malloc(sizeof(double) * 16);
    ora_gemm_block(aq, as, M, K, wq, ws, N, c, c64, NT);
    int64_t ms[16], ns[16];
    uint16_t sc[16];
    for (int i = 0; i < 16; ++i) { ms[i] = i % M; ns[i] = (i * 37) % N; }
    ora_gemm_block_at(aq, as, M, K, wq, ws, N, ms, ns, 16, sc, s64, NT);
    for (int i = 0; i < 16; ++i) CHECK(sc[i] == c[ms[i] * N + ns[i]]);
    ora_gemm_block_bf16a(a, M, K, wq, ws, N, c2, c64, NT);

    /* MoE: routing, the decode with out-of-range ids, the down stage from given h, the fold */
    enum { T = 3, H = 256, E = 4, I = 256, TOPK = 2, P = T * TOPK };
    float logits[T * E];
    for (int i = 0; i < T * E; ++i) logits[i] = uniform();
    int32_t ids[P];
    float tw[P];
    ora_moe_route(logits, T, E, TOPK, ids, tw);
    for (int i = 0; i < P; ++i) CHECK(ids[i] >= 0 && ids[i] < E);
    ids[1] = -1;
    ids[4] = E + 2;
    uint16_t *x = malloc(sizeof(uint16_t) * T * H);
    fill_bf16(x, T * H, 3.0f);
    uint16_t *w13 = malloc(sizeof(uint16_t) * E * 2 * I * H), *w2 = malloc(sizeof(uint16_t) * E * H * I);
    fill_bf16(w13, (int64_t)E * 2 * I * H, 0.05f);
    fill_bf16(w2, (int64_t)E * H * I, 0.05f);
    uint8_t *w13q = malloc((size_t)E * 2 * I * H), *w2q = malloc((size_t)E * H * I);
    float *w13s = malloc(sizeof(float) * E * (2 * I / 128) * (H / 128));
    float *w2s = malloc(sizeof(float) * E * (H / 128) * (I / 128));
    for (int e = 0; e < E; ++e) {
        ora_quant_weight(w13 + (int64_t)e * 2 * I * H, 2 * I, H, w13q + (int64_t)e * 2 * I * H,
                         w13s + e * (2 * I / 128) * (H / 128), NT);
        ora_quant_weight(w2 + (int64_t)e * H * I, H, I, w2q + (int64_t)e * H * I, w2s + e * (H / 128) * (I / 128), NT);
    }
    uint16_t *out = malloc(sizeof(uint16_t) * T * H), *out2 = malloc(sizeof(uint16_t) * T * H);
    uint16_t *gu = malloc(sizeof(uint16_t) * P * 2 * I), *hh = malloc(sizeof(uint16_t) * P * I);
    uint16_t *h2 = malloc(sizeof(uint16_t) * P * I);
    uint8_t *hq = malloc(P * I);
    float *hs = malloc(sizeof(float) * P * (I / 128));
    double *y = malloc(sizeof(double) * P * H);
    ora_moe_decode(x, T, H, ids, tw, TOPK, w13q, w13s, w2q, w2s, E, I, out, gu, hh, hq, hs, y, NT);
    for (int n = 0; n < H; ++n) CHECK(y[1 * H + n] == 0.0 && y[4 * H + n] == 0.0);
    ora_moe_decode(x, T, H, ids, tw, TOPK, w13q, w13s, w2q, w2s, E, I, out2, NULL, NULL, NULL, NULL, NULL, NT);
    CHECK(memcmp(out, out2, sizeof(uint16_t) * T * H) == 0);
    ora_moe_silu_mul(gu, P, I, h2);
    for (int p = 0; p < P; ++p)
        if (p != 1 && p != 4) CHECK(memcmp(h2 + p * I, hh + p * I, sizeof(uint16_t) * I) == 0);
    ora_moe_down_from_h(hh, T, H, ids, tw, TOPK, w2q, w2s, E, I, out2, hq, hs, y, NT);
    CHECK(memcmp(out, out2, sizeof(uint16_t) * T * H) == 0);
    uint16_t *shared = malloc(sizeof(uint16_t) * T * H);
    fill_bf16(shared, T * H, 1.0f);
    float gw[T] = {0.5f, -1.0f, 2.0f};
    ora_moe_fold(y, ids, tw, T, TOPK, H, E, NULL, NULL, out2);
    CHECK(memcmp(out, out2, sizeof(uint16_t) * T * H) == 0);
    ora_moe_fold(y, ids, tw, T, TOPK, H, E, shared, gw, out2);
    ora_moe_fold(y, ids, tw, T, TOPK, H, E, shared, NULL, out2);

    /* the pins' own sweeps, over a slice of their ranges */
    CHECK(pin_div_correction_mismatches(0x3F00, 0x3F40, NT) == 0);
    CHECK(pin_scale_formula_mismatches() == 0);

    free(a); free(w); free(aq); free(wq); free(as); free(ws); free(c); free(c2); free(c64); free(s64);
    free(x); free(w13); free(w2); free(w13q); free(w2q); free(w13s); free(w2s); free(out); free(out2);
    free(gu); free(hh); free(h2); free(hq); free(hs); free(y); free(shared);
    if (!g_fail) printf("sanitized oracle and pins: ok\n");
    return g_fail;
}
