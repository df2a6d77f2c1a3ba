/*
 * Reference oracle for streaming multi-head attention: plain, slow, fp64, CPU only.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark load this library. The GPU product path never calls it, links it or shares code
 * with it: the two are independent implementations of the same definitions.
 *
 * Every function restates a definition from the page "flashdreams.accelerated" (developer
 * guide), section "Multi Head Attention Definition":
 *   - 16-bit float decoding is the IEEE-754 binary16 / bfloat16 bit-format definition, and 8-bit
 *     decoding the OCP FP8 E4M3 definition;
 *   - RMSNorm: gamma (.) z / sqrt(mean(z^2) + eps), the RMSNorm equation of that section;
 *   - RoPE: the 2x2 rotation of pair r by angle theta_{p,r} (rotation equation), with the
 *     split-half pairs (r, r + d/2) or interleaved pairs (2r, 2r + 1) named there;
 *   - attention: A_h = softmax(Q_h K_h^T * scale) V_h, the scaled dot-product equation, one
 *     query row at a time, over the full key range (no tiling, no online rescaling).
 * Subtracting the row maximum before exp() is the textbook identity
 * softmax(s) = softmax(s - c); it changes no value in exact arithmetic.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared -pthread oracle.c -lm
 * (no fused multiply-add contraction, so each expression rounds as written).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- 16-bit float decoding */

/* bfloat16: the upper 16 bits of an IEEE-754 binary32 value. */
static double decode_bf16_one(uint16_t h) {
    uint32_t bits = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double decode_f16_one(uint16_t h) {
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double mag;
    if (expo == 0)
        mag = ldexp((double)frac, -24); /* subnormal: frac * 2^-14 * 2^-10 */
    else if (expo == 31)
        mag = frac ? NAN : INFINITY;
    else
        mag = ldexp((double)(1024 + frac), expo - 25); /* (1 + frac/1024) * 2^(expo-15) */
    return sign ? -mag : mag;
}

/* FP8 E4M3 in the OCP 8-bit floating-point format ("e4m3fn"): 1 sign bit, 4 exponent bits
 * (bias 7), 3 fraction bits; exponent 0 holds subnormals frac * 2^-9; there is no infinity, and
 * only exponent 15 with fraction 7 is NaN, so the largest finite magnitude is 1.75 * 2^8 = 448.
 * This is the unscaled float8_e4m3fn the page "flashdreams.accelerated" (section
 * OptimizedMultiHeadAttention, quantized SDPA option) casts Q, K and V to. */
static double decode_e4m3_one(uint8_t x) {
    int sign = (x >> 7) & 1;
    int expo = (x >> 3) & 0xf;
    int frac = x & 0x7;
    double mag;
    if (expo == 0)
        mag = ldexp((double)frac, -9);               /* frac/8 * 2^(1-7) */
    else if (expo == 15 && frac == 7)
        mag = NAN;
    else
        mag = ldexp((double)(8 + frac), expo - 10);  /* (1 + frac/8) * 2^(expo-7) */
    return sign ? -mag : mag;
}

void oracle_decode_e4m3(const uint8_t* in, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = decode_e4m3_one(in[i]);
}

void oracle_decode_bf16(const uint16_t* in, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = decode_bf16_one(in[i]);
}

void oracle_decode_f16(const uint16_t* in, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = decode_f16_one(in[i]);
}

/* ---------------------------------------------------------------- RMSNorm */

/* rows x m matrix z, one RMSNorm per row: out = gamma * z / sqrt((1/m) sum z^2 + eps).
 * Head scope is m = d over rows (b, token, head); inner scope is m = H*d over rows (b, token). */
void oracle_rmsnorm(const double* z, const double* gamma, double* out, int64_t rows, int m, double eps) {
    for (int64_t r = 0; r < rows; ++r) {
        const double* zr = z + r * m;
        double* o = out + r * m;
        double ss = 0.0;
        for (int t = 0; t < m; ++t) ss += zr[t] * zr[t];
        double denom = sqrt(ss / (double)m + eps);
        for (int t = 0; t < m; ++t) o[t] = gamma[t] * (zr[t] / denom);
    }
}

/* ---------------------------------------------------------------- RoPE */

/* z, out: [B, L, H, d]; angles: [L, d/2] (angle of pair r at position p is angles[p*(d/2) + r]).
 * style 1 = split-half pairs (r, r + d/2); style 2 = interleaved pairs (2r, 2r + 1).
 * Rotation: a' = cos*a - sin*b ; b' = sin*a + cos*b. */
void oracle_rope(const double* z, const double* angles, double* out, int B, int L, int H, int d, int style) {
    int half = d / 2;
    for (int b = 0; b < B; ++b)
        for (int p = 0; p < L; ++p)
            for (int h = 0; h < H; ++h) {
                int64_t base = (((int64_t)b * L + p) * H + h) * d;
                const double* zr = z + base;
                double* o = out + base;
                for (int r = 0; r < half; ++r) {
                    int ia = (style == 1) ? r : 2 * r;
                    int ib = (style == 1) ? r + half : 2 * r + 1;
                    double th = angles[(int64_t)p * half + r];
                    double c = cos(th), s = sin(th);
                    double a = zr[ia], bb = zr[ib];
                    o[ia] = c * a - s * bb;
                    o[ib] = s * a + c * bb;
                }
            }
}

/* ---------------------------------------------------------------- attention */

typedef struct {
    const double *q, *k, *v;
    double* out;
    const int64_t* rows; /* flat indices into [B, Lq, Hq]; NULL = all rows in order */
    int64_t nrows;
    int B, Hq, Hkv, Lq, Lk, d;
    int64_t win_left, win_right; /* visible keys of query i: [i+s-win_left, i+s+win_right], s = Lk-Lq; <0 = unbounded */
    double scale;
    int tid, nthreads;
    /* optional per-row outputs (NULL: not computed), for tolerances of kernels that round the
     * softmax weights: spread_a[n*d + t] = sum_j w_j |v_jt - o_t| and spread_r[n*d + t] =
     * sqrt(sum_j w_j^2 (v_jt - o_t)^2) with w_j = p_j / l the exact weights; span[n] = the range
     * of the row's visible scores, max_j s_j - min_j s_j, in base-2 exponent units (times log2 e) */
    double *spread_a, *spread_r, *span;
    /* keys whose score lies more than tail_binades (base-2 units) below the row maximum: their
     * part of spread_a (tail_a[n*d + t]) and their total weight (tail_w[n]) */
    double tail_binades;
    double *tail_a, *tail_w;
} attn_job;

/* One query row: s_j = scale * <q_i, k_j> for every visible key j, then
 * o = sum_j softmax(s)_j v_j. The query block sits at the end of the key sequence: query i is
 * at key position i + (Lk - Lq). Visible keys: j >= i + (Lk - Lq) - win_left (if win_left >= 0)
 * and j <= i + (Lk - Lq) + win_right (if win_right >= 0). Causal is (win_left, win_right) = (-1, 0). */
static void attention_row(const attn_job* J, int64_t row, double* scores, double* o) {
    int64_t h = row % J->Hq;
    int64_t i = (row / J->Hq) % J->Lq;
    int64_t b = row / ((int64_t)J->Hq * J->Lq);
    int group = J->Hq / J->Hkv;
    int64_t hk = h / group;
    int d = J->d;
    const double* qi = J->q + row * d;
    int64_t pos = i + (J->Lk - J->Lq);
    int64_t jlo = 0, jhi = J->Lk - 1;
    if (J->win_left >= 0 && pos - J->win_left > jlo) jlo = pos - J->win_left;
    if (J->win_right >= 0 && pos + J->win_right < jhi) jhi = pos + J->win_right;
    int64_t nvis = jhi >= jlo ? jhi - jlo + 1 : 0;
    double m = -INFINITY;
    for (int64_t n = 0; n < nvis; ++n) {
        int64_t j = jlo + n;
        const double* kj = J->k + (((int64_t)b * J->Lk + j) * J->Hkv + hk) * d;
        double dot = 0.0;
        for (int t = 0; t < d; ++t) dot += qi[t] * kj[t];
        scores[n] = J->scale * dot;
        if (scores[n] > m) m = scores[n];
    }
    double l = 0.0;
    for (int64_t n = 0; n < nvis; ++n) {
        scores[n] = exp(scores[n] - m);
        l += scores[n];
    }
    for (int t = 0; t < d; ++t) o[t] = 0.0;
    for (int64_t n = 0; n < nvis; ++n) {
        const double* vj = J->v + (((int64_t)b * J->Lk + jlo + n) * J->Hkv + hk) * d;
        for (int t = 0; t < d; ++t) o[t] += scores[n] * vj[t];
    }
    for (int t = 0; t < d; ++t) o[t] = o[t] / l;
    if (J->spread_a) {
        const int64_t n_out = o - J->out;   /* this row's offset into the outputs */
        double* a = J->spread_a + n_out;
        double* r = J->spread_r + n_out;
        double* ta = J->tail_a + n_out;
        double tw = 0.0;
        for (int t = 0; t < d; ++t) a[t] = r[t] = ta[t] = 0.0;
        double smin = INFINITY;
        for (int64_t n = 0; n < nvis; ++n) {
            const double w = scores[n] / l;
            const double* vj = J->v + (((int64_t)b * J->Lk + jlo + n) * J->Hkv + hk) * d;
            /* scores[n] = exp(s_n - m): below 2^-tail_binades lies in the tail */
            const int tail = -log2(scores[n]) > J->tail_binades;
            if (tail) tw += w;
            for (int t = 0; t < d; ++t) {
                const double dev = vj[t] - o[t];
                a[t] += w * fabs(dev);
                r[t] += (w * dev) * (w * dev);
                if (tail) ta[t] += w * fabs(dev);
            }
            /* scores[n] holds exp(s_n - m): the smallest gives the row's score range */
            if (scores[n] < smin) smin = scores[n];
        }
        for (int t = 0; t < d; ++t) r[t] = sqrt(r[t]);
        J->span[n_out / d] = nvis > 0 ? -log2(smin) : 0.0;
        J->tail_w[n_out / d] = tw;
    }
}

static void* attention_worker(void* arg) {
    attn_job* J = (attn_job*)arg;
    double* scores = (double*)malloc(sizeof(double) * (size_t)(J->Lk > 0 ? J->Lk : 1));
    if (!scores) return (void*)1;
    for (int64_t n = J->tid; n < J->nrows; n += J->nthreads) {
        int64_t row = J->rows ? J->rows[n] : n;
        attention_row(J, row, scores, J->out + n * J->d);
    }
    free(scores);
    return NULL;
}

/* q: [B, Lq, Hq, d], k and v: [B, Lk, Hkv, d], contiguous fp64. Query head h reads key/value
 * head h / (Hq / Hkv). Visible keys per query as in attention_row (win_left = win_right = -1:
 * all keys; (-1, 0): causal). out: [nrows, d], row n is the attention output of query row rows[n]
 * (flat index (b * Lq + i) * Hq + h), or of row n when rows is NULL (then nrows = B*Lq*Hq).
 * Returns 0 on success, -1 on invalid arguments or allocation failure. */
static int run_attention(const double* q, const double* k, const double* v, double* out, const int64_t* rows,
                         int64_t nrows, int B, int Hq, int Hkv, int Lq, int Lk, int d, double scale,
                         int64_t win_left, int64_t win_right, int nthreads, double* spread_a, double* spread_r,
                         double* span, double tail_binades, double* tail_a, double* tail_w);

int oracle_attention(const double* q, const double* k, const double* v, double* out,
                     const int64_t* rows, int64_t nrows, int B, int Hq, int Hkv, int Lq, int Lk, int d,
                     double scale, int64_t win_left, int64_t win_right, int nthreads) {
    return run_attention(q, k, v, out, rows, nrows, B, Hq, Hkv, Lq, Lk, d, scale, win_left, win_right, nthreads,
                         NULL, NULL, NULL, 0.0, NULL, NULL);
}

/* oracle_attention plus, per output element, the spread of V under the exact softmax weights
 * (spread_a, spread_r: [nrows, d]), per row the range of its scores in base-2 units (span:
 * [nrows]), and the part of spread_a and of the weight that keys more than tail_binades below
 * the row maximum carry (tail_a: [nrows, d], tail_w: [nrows]); see attn_job. Same return values. */
int oracle_attention_spread(const double* q, const double* k, const double* v, double* out,
                            const int64_t* rows, int64_t nrows, int B, int Hq, int Hkv, int Lq, int Lk, int d,
                            double scale, int64_t win_left, int64_t win_right, int nthreads, double* spread_a,
                            double* spread_r, double* span, double tail_binades, double* tail_a, double* tail_w) {
    if (!spread_a || !spread_r || !span || !tail_a || !tail_w) return -1;
    return run_attention(q, k, v, out, rows, nrows, B, Hq, Hkv, Lq, Lk, d, scale, win_left, win_right, nthreads,
                         spread_a, spread_r, span, tail_binades, tail_a, tail_w);
}

static int run_attention(const double* q, const double* k, const double* v, double* out, const int64_t* rows,
                         int64_t nrows, int B, int Hq, int Hkv, int Lq, int Lk, int d, double scale,
                         int64_t win_left, int64_t win_right, int nthreads, double* spread_a, double* spread_r,
                         double* span, double tail_binades, double* tail_a, double* tail_w) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || Lq < 0 || Lk < 0 || d <= 0) return -1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    attn_job jobs[256];
    pthread_t th[256];
    int created[256];
    int rc = 0;
    for (int t = 0; t < nthreads; ++t) {
        attn_job J = {q, k, v, out, rows, nrows, B, Hq, Hkv, Lq, Lk, d, win_left, win_right, scale, t, nthreads,
                      spread_a, spread_r, span, tail_binades, tail_a, tail_w};
        jobs[t] = J;
        created[t] = 0;
    }
    for (int t = 1; t < nthreads; ++t)
        created[t] = pthread_create(&th[t], NULL, attention_worker, &jobs[t]) == 0;
    if (attention_worker(&jobs[0]) != NULL) rc = -1;
    for (int t = 1; t < nthreads; ++t) {
        void* r = NULL;
        if (created[t])
            pthread_join(th[t], &r);
        else
            r = attention_worker(&jobs[t]); /* could not start a thread: do its rows here */
        if (r != NULL) rc = -1;
    }
    return rc;
}
