/* Exercises every entry point of oracle/oracle.c on small inputs with closed-form answers, so a
 * build with AddressSanitizer and UndefinedBehaviorSanitizer can check the oracle's memory use
 * and arithmetic (multithreaded attention over row subsets, windows and grouped heads included).
 * Prints "ok" and exits 0 when every check holds. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void oracle_decode_e4m3(const uint8_t* in, double* out, int64_t n);
void oracle_decode_bf16(const uint16_t* in, double* out, int64_t n);
void oracle_decode_f16(const uint16_t* in, double* out, int64_t n);
void oracle_rmsnorm(const double* z, const double* gamma, double* out, int64_t rows, int m, double eps);
void oracle_rope(const double* z, const double* angles, double* out, int B, int L, int H, int d, int style);
int oracle_attention(const double* q, const double* k, const double* v, double* out, const int64_t* rows,
                     int64_t nrows, int B, int Hq, int Hkv, int Lq, int Lk, int d, double scale, int64_t win_left,
                     int64_t win_right, int nthreads);
int oracle_attention_spread(const double* q, const double* k, const double* v, double* out, const int64_t* rows,
                            int64_t nrows, int B, int Hq, int Hkv, int Lq, int Lk, int d, double scale,
                            int64_t win_left, int64_t win_right, int nthreads, double* spread_a, double* spread_r,
                            double* span, double tail_binades, double* tail_a, double* tail_w);

static int fails = 0;
#define CHECK(c)                                                             \
    do {                                                                     \
        if (!(c)) {                                                          \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);  \
            ++fails;                                                         \
        }                                                                    \
    } while (0)

static double urand(unsigned* s) {
    *s = *s * 1103515245u + 12345u;
    return ((*s >> 8) & 0xffff) / 32768.0 - 1.0;
}

int main(void) {
    /* every 16-bit pattern and every E4M3 code */
    uint16_t* p16 = malloc(65536 * sizeof *p16);
    double* d16 = malloc(65536 * sizeof *d16);
    for (int i = 0; i < 65536; ++i) p16[i] = (uint16_t)i;
    oracle_decode_bf16(p16, d16, 65536);
    CHECK(d16[0x3f80] == 1.0 && d16[0xc000] == -2.0 && d16[0x0001] == ldexp(1.0, -133));
    oracle_decode_f16(p16, d16, 65536);
    CHECK(d16[0x3c00] == 1.0 && d16[0x7bff] == 65504.0 && d16[0x0001] == ldexp(1.0, -24));
    uint8_t p8[256];
    double d8[256];
    for (int i = 0; i < 256; ++i) p8[i] = (uint8_t)i;
    oracle_decode_e4m3(p8, d8, 256);
    CHECK(d8[0x38] == 1.0 && d8[0x7e] == 448.0 && d8[0x01] == ldexp(1.0, -9) && isnan(d8[0x7f]));
    free(p16);
    free(d16);

    /* RMSNorm with unit weights: every row has unit mean square (up to eps) */
    enum { R = 6, M = 40 };
    double z[R * M], g[M], o[R * M];
    unsigned seed = 1;
    for (int i = 0; i < R * M; ++i) z[i] = urand(&seed) * 3.0;
    for (int i = 0; i < M; ++i) g[i] = 1.0;
    oracle_rmsnorm(z, g, o, R, M, 0.0);
    for (int r = 0; r < R; ++r) {
        double ss = 0.0;
        for (int t = 0; t < M; ++t) ss += o[r * M + t] * o[r * M + t];
        CHECK(fabs(ss / M - 1.0) < 1e-12);
    }

    /* RoPE: position 0 is the identity, every pair keeps its norm (both pairings) */
    enum { B = 2, L = 3, H = 2, D = 8 };
    double x[B * L * H * D], y[B * L * H * D], ang[L * D / 2];
    for (int i = 0; i < B * L * H * D; ++i) x[i] = urand(&seed);
    for (int p = 0; p < L; ++p)
        for (int r = 0; r < D / 2; ++r) ang[p * D / 2 + r] = p * pow(10000.0, -2.0 * r / D);
    for (int style = 1; style <= 2; ++style) {
        oracle_rope(x, ang, y, B, L, H, D, style);
        for (int b = 0; b < B; ++b)
            for (int p = 0; p < L; ++p)
                for (int h = 0; h < H; ++h) {
                    const int64_t base = (((int64_t)b * L + p) * H + h) * D;
                    for (int r = 0; r < D / 2; ++r) {
                        const int ia = style == 1 ? r : 2 * r, ib = style == 1 ? r + D / 2 : 2 * r + 1;
                        const double n0 = x[base + ia] * x[base + ia] + x[base + ib] * x[base + ib];
                        const double n1 = y[base + ia] * y[base + ia] + y[base + ib] * y[base + ib];
                        CHECK(fabs(n0 - n1) < 1e-12);
                        if (p == 0) CHECK(y[base + ia] == x[base + ia] && y[base + ib] == x[base + ib]);
                    }
                }
    }

    /* attention: q = 0 gives the mean of V over the visible keys; a single key returns its value;
       causal row 0 returns v_0; a row subset equals the same rows of the full result */
    enum { AB = 2, HQ = 4, HKV = 2, LQ = 5, LK = 7, AD = 16 };
    double *q = calloc(AB * LQ * HQ * AD, sizeof(double)), *k = malloc(sizeof(double) * AB * LK * HKV * AD),
           *v = malloc(sizeof(double) * AB * LK * HKV * AD), *out = malloc(sizeof(double) * AB * LQ * HQ * AD),
           *sub = malloc(sizeof(double) * 3 * AD);
    for (int i = 0; i < AB * LK * HKV * AD; ++i) {
        k[i] = urand(&seed);
        v[i] = urand(&seed);
    }
    CHECK(oracle_attention(q, k, v, out, NULL, AB * LQ * HQ, AB, HQ, HKV, LQ, LK, AD, 0.25, -1, -1, 3) == 0);
    for (int b = 0; b < AB; ++b)
        for (int i = 0; i < LQ; ++i)
            for (int h = 0; h < HQ; ++h)
                for (int t = 0; t < AD; ++t) {
                    double m = 0.0;
                    for (int j = 0; j < LK; ++j) m += v[(((int64_t)b * LK + j) * HKV + h / 2) * AD + t];
                    CHECK(fabs(out[(((int64_t)b * LQ + i) * HQ + h) * AD + t] - m / LK) < 1e-12);
                }
    for (int i = 0; i < AB * LQ * HQ * AD; ++i) q[i] = urand(&seed) * 4.0;
    /* window (0, 0): each query sees only its own key position i + LK - LQ */
    CHECK(oracle_attention(q, k, v, out, NULL, AB * LQ * HQ, AB, HQ, HKV, LQ, LK, AD, 0.25, 0, 0, 4) == 0);
    for (int b = 0; b < AB; ++b)
        for (int i = 0; i < LQ; ++i)
            for (int h = 0; h < HQ; ++h)
                for (int t = 0; t < AD; ++t)
                    CHECK(out[(((int64_t)b * LQ + i) * HQ + h) * AD + t] ==
                          v[(((int64_t)b * LK + i + LK - LQ) * HKV + h / 2) * AD + t]);
    /* causal with Lq == Lk == LQ (the first LQ*HKV*AD values of each batch as a shorter key
       sequence): row 0 sees key 0 only and returns v_0 */
    CHECK(oracle_attention(q, k, v, out, NULL, AB * LQ * HQ, AB, HQ, HKV, LQ, LQ, AD, 0.25, -1, 0, 2) == 0);
    for (int b = 0; b < AB; ++b)
        for (int h = 0; h < HQ; ++h)
            for (int t = 0; t < AD; ++t)
                CHECK(out[((int64_t)b * LQ * HQ + h) * AD + t] == v[(((int64_t)b * LQ) * HKV + h / 2) * AD + t]);
    const int64_t rows[3] = {7, 0, 39};
    CHECK(oracle_attention(q, k, v, out, NULL, AB * LQ * HQ, AB, HQ, HKV, LQ, LK, AD, 0.25, 2, 1, 1) == 0);
    CHECK(oracle_attention(q, k, v, sub, rows, 3, AB, HQ, HKV, LQ, LK, AD, 0.25, 2, 1, 3) == 0);
    for (int n = 0; n < 3; ++n) CHECK(memcmp(sub + n * AD, out + rows[n] * AD, AD * sizeof(double)) == 0);
    CHECK(oracle_attention(q, k, v, out, NULL, 0, AB, 3, 2, LQ, LK, AD, 0.25, -1, -1, 1) == -1);
    /* spreads over a row subset, threaded: a single visible key (window (0, 0)) has none */
    double *sa = malloc(sizeof(double) * 3 * AD), *sr = malloc(sizeof(double) * 3 * AD), span[3];
    double *ta = malloc(sizeof(double) * 3 * AD), tw[3];
    CHECK(oracle_attention_spread(q, k, v, sub, rows, 3, AB, HQ, HKV, LQ, LK, AD, 0.25, 0, 0, 2, sa, sr, span, 0.5, ta,
                                  tw) == 0);
    for (int i = 0; i < 3 * AD; ++i) CHECK(sa[i] == 0.0 && sr[i] == 0.0 && ta[i] == 0.0);
    CHECK(oracle_attention_spread(q, k, v, sub, rows, 3, AB, HQ, HKV, LQ, LK, AD, 0.25, -1, -1, 3, sa, sr, span, 1e-3,
                                  ta, tw) == 0);
    for (int i = 0; i < 3 * AD; ++i) CHECK(sa[i] > 0.0 && sr[i] > 0.0 && sr[i] <= sa[i] && ta[i] <= sa[i]);
    for (int i = 0; i < 3; ++i) CHECK(span[i] > 0.0 && tw[i] > 0.0 && tw[i] < 1.0);
    free(sa);
    free(sr);
    free(ta);
    free(q);
    free(k);
    free(v);
    free(out);
    free(sub);
    if (fails) return 1;
    printf("ok\n");
    return 0;
}
