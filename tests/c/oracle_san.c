/* Drives every function of oracle/oracle.c over a grid of tiny and
 * degenerate shapes, for a build with -fsanitize=address,undefined.
 *
 * Every buffer is allocated at exactly its size, so a read or write one
 * element outside it stops the run (AddressSanitizer), as does undefined
 * behaviour such as signed overflow (UndefinedBehaviorSanitizer).  Optional
 * pointers (biases, lengths, gradient outputs) are passed both set and NULL.
 * Besides running cleanly, the results are checked for two facts that hold
 * whatever the data: a NULL bias gives bit for bit the zero-bias result, and
 * every output frame at or past an item's length is exactly zero.
 *
 * Exit status 0 when every case ran and every check held.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_dwconv1d_fwd(const float *x, const float *w, const float *bias, const int32_t *lengths, double *y,
                        long B, long T, long C, long K, int causal);
int oracle_dwconv2d_fwd(const float *x, const float *w, const float *bias, const int32_t *lengths, double *y,
                        long B, long T, long F, long C, long KH, long KW, long s, long pt0, long pt1, long pf0,
                        long pf1);
int oracle_dwconv2d_bwd(const float *x, const float *w, const int32_t *lengths, const float *dy, double *dx,
                        double *dw, double *db, long B, long T, long F, long C, long KH, long KW, long s, long pt0,
                        long pt1, long pf0, long pf1);
int oracle_dwsub_front_fwd(const float *x, const float *w0, const float *b0, const float *w1, const float *b1,
                           const int32_t *lengths, double *y, long B, long T, long F, long C, int causal);
int oracle_dwsub_front_bwd(const float *x, const float *w0, const float *b0, const float *w1,
                           const int32_t *lengths, const float *dy, double *dw0, double *db0, double *dw1,
                           double *db1, long B, long T, long F, long C, int causal);
int oracle_dwconv1d_bwd(const float *x, const float *w, const int32_t *lengths, const float *dy, double *dx,
                        double *dw, double *db, long B, long T, long C, long K, int causal);
int oracle_dwconv1d_stream_fwd(const float *x, const float *w, const float *bias, const int32_t *lengths,
                               const float *cache_in, double *y, double *cache_out, long B, long Tc, long C, long K);

static int failures = 0;
static long cases = 0;
static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

static uint64_t next_u64(void)
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* A buffer of exactly n floats (at least one byte is allocated so that n = 0
 * still gives a pointer the sanitizer tracks as zero-sized). */
static float *fbuf(long n)
{
    float *p = (float *)malloc(sizeof(float) * (size_t)(n > 0 ? n : 0) + (n > 0 ? 0 : 1));
    for (long i = 0; i < n; ++i) p[i] = (float)((double)(next_u64() >> 11) / 9007199254740992.0 * 2.0 - 1.0);
    return p;
}

static double *dbuf(long n)
{
    double *p = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 0) + (n > 0 ? 0 : 1));
    for (long i = 0; i < n; ++i) p[i] = 12345.0; /* overwritten by the oracle */
    return p;
}

static int32_t *lens(long B, long T)
{
    int32_t *p = (int32_t *)malloc(sizeof(int32_t) * (size_t)(B > 0 ? B : 0) + (B > 0 ? 0 : 1));
    for (long b = 0; b < B; ++b) p[b] = (int32_t)((long)(next_u64() % (uint64_t)(T + 3)) - 1); /* -1 .. T+1 */
    return p;
}

static long clampl(const int32_t *L, long b, long T)
{
    long l = L ? L[b] : T;
    return l < 0 ? 0 : (l > T ? T : l);
}

static void expect(int cond, const char *what, long a, long b, long c, long d)
{
    if (!cond) {
        if (failures < 20) printf("FAIL %s (%ld %ld %ld %ld)\n", what, a, b, c, d);
        ++failures;
    }
}

static int same_bits(const double *a, const double *b, long n)
{
    return n <= 0 || memcmp(a, b, sizeof(double) * (size_t)n) == 0;
}

static long out_len(long n, long k, long s, long pl, long ph)
{
    long v = n + pl + ph - k;
    long q = v >= 0 ? v / s : -((-v + s - 1) / s);
    return q + 1 < 0 ? 0 : q + 1;
}

static void run_1d(long B, long T, long C, long K, int causal)
{
    float *x = fbuf(B * T * C), *w = fbuf(K * C), *bias = fbuf(C), *zero = fbuf(C), *dy = fbuf(B * T * C);
    int32_t *L = lens(B, T);
    double *y = dbuf(B * T * C), *yz = dbuf(B * T * C), *yn = dbuf(B * T * C);
    double *dx = dbuf(B * T * C), *dw = dbuf(K * C), *db = dbuf(C);
    memset(zero, 0, sizeof(float) * (size_t)C);
    expect(oracle_dwconv1d_fwd(x, w, bias, L, y, B, T, C, K, causal) == 0, "1d fwd", B, T, C, K);
    expect(oracle_dwconv1d_fwd(x, w, NULL, L, yn, B, T, C, K, causal) == 0, "1d fwd null bias", B, T, C, K);
    expect(oracle_dwconv1d_fwd(x, w, zero, L, yz, B, T, C, K, causal) == 0, "1d fwd zero bias", B, T, C, K);
    expect(same_bits(yn, yz, B * T * C), "1d null bias is zero bias", B, T, C, K);
    for (long b = 0; b < B; ++b)
        for (long t = clampl(L, b, T); t < T; ++t)
            for (long c = 0; c < C; ++c) expect(y[(b * T + t) * C + c] == 0.0, "1d masked zero", b, t, c, K);
    expect(oracle_dwconv1d_fwd(x, w, bias, NULL, y, B, T, C, K, causal) == 0, "1d fwd null lengths", B, T, C, K);
    expect(oracle_dwconv1d_bwd(x, w, L, dy, dx, dw, db, B, T, C, K, causal) == 0, "1d bwd", B, T, C, K);
    for (long b = 0; b < B; ++b)
        for (long t = clampl(L, b, T); t < T; ++t)
            for (long c = 0; c < C; ++c) expect(dx[(b * T + t) * C + c] == 0.0, "1d dx masked zero", b, t, c, K);
    expect(oracle_dwconv1d_bwd(x, w, NULL, dy, NULL, dw, NULL, B, T, C, K, causal) == 0, "1d bwd dw only", B, T,
           C, K);
    expect(oracle_dwconv1d_bwd(x, w, L, dy, dx, NULL, NULL, B, T, C, K, causal) == 0, "1d bwd dx only", B, T, C, K);
    if (K > 1) {
        float *cache = fbuf(B * (K - 1) * C);
        double *co = dbuf(B * (K - 1) * C), *coz = dbuf(B * (K - 1) * C);
        expect(oracle_dwconv1d_stream_fwd(x, w, bias, L, cache, y, co, B, T, C, K) == 0, "stream", B, T, C, K);
        expect(oracle_dwconv1d_stream_fwd(x, w, NULL, NULL, cache, yn, co, B, T, C, K) == 0, "stream null bias",
               B, T, C, K);
        expect(oracle_dwconv1d_stream_fwd(x, w, zero, NULL, cache, yz, coz, B, T, C, K) == 0, "stream zero bias",
               B, T, C, K);
        expect(same_bits(yn, yz, B * T * C) && same_bits(co, coz, B * (K - 1) * C), "stream null bias is zero",
               B, T, C, K);
        free(cache); free(co); free(coz);
    }
    ++cases;
    free(x); free(w); free(bias); free(zero); free(dy); free(L); free(y); free(yz); free(yn);
    free(dx); free(dw); free(db);
}

static void run_2d(long B, long T, long F, long C, long KH, long KW, long s, long pt0, long pt1, long pf0,
                   long pf1)
{
    long To = out_len(T, KH, s, pt0, pt1), Fo = out_len(F, KW, s, pf0, pf1);
    float *x = fbuf(B * T * F * C), *w = fbuf(KH * KW * C), *bias = fbuf(C), *zero = fbuf(C);
    float *dy = fbuf(B * To * Fo * C);
    int32_t *L = lens(B, T);
    double *y = dbuf(B * To * Fo * C), *yn = dbuf(B * To * Fo * C), *yz = dbuf(B * To * Fo * C);
    double *dx = dbuf(B * T * F * C), *dw = dbuf(KH * KW * C), *db = dbuf(C);
    memset(zero, 0, sizeof(float) * (size_t)C);
    expect(oracle_dwconv2d_fwd(x, w, bias, L, y, B, T, F, C, KH, KW, s, pt0, pt1, pf0, pf1) == 0, "2d fwd", B, T,
           F, C);
    expect(oracle_dwconv2d_fwd(x, w, NULL, L, yn, B, T, F, C, KH, KW, s, pt0, pt1, pf0, pf1) == 0, "2d null bias",
           B, T, F, C);
    expect(oracle_dwconv2d_fwd(x, w, zero, L, yz, B, T, F, C, KH, KW, s, pt0, pt1, pf0, pf1) == 0, "2d zero bias",
           B, T, F, C);
    expect(same_bits(yn, yz, B * To * Fo * C), "2d null bias is zero bias", B, T, F, C);
    expect(oracle_dwconv2d_bwd(x, w, L, dy, dx, dw, db, B, T, F, C, KH, KW, s, pt0, pt1, pf0, pf1) == 0, "2d bwd",
           B, T, F, C);
    for (long b = 0; b < B; ++b)
        for (long t = clampl(L, b, T); t < T; ++t)
            for (long i = 0; i < F * C; ++i) expect(dx[(b * T + t) * F * C + i] == 0.0, "2d dx masked", b, t, i, 0);
    expect(oracle_dwconv2d_bwd(x, w, NULL, dy, NULL, dw, db, B, T, F, C, KH, KW, s, pt0, pt1, pf0, pf1) == 0,
           "2d bwd no dx", B, T, F, C);
    ++cases;
    free(x); free(w); free(bias); free(zero); free(dy); free(L); free(y); free(yn); free(yz);
    free(dx); free(dw); free(db);
}

static void run_front(long B, long T, long F, long C, int causal)
{
    long pl = causal ? 2 : 1;
    long T1 = out_len(T, 3, 2, pl, 1), F1 = out_len(F, 3, 2, pl, 1);
    long T2 = out_len(T1, 3, 2, pl, 1), F2 = out_len(F1, 3, 2, pl, 1);
    long ny = B * T2 * F2 * C;
    float *x = fbuf(B * T * F), *w0 = fbuf(9 * C), *b0 = fbuf(C), *w1 = fbuf(9 * C), *b1 = fbuf(C);
    float *zero = fbuf(C), *dy = fbuf(ny);
    int32_t *L = lens(B, T);
    double *y = dbuf(ny), *yn = dbuf(ny), *yz = dbuf(ny);
    double *g[4] = {dbuf(9 * C), dbuf(C), dbuf(9 * C), dbuf(C)}, *gz[4] = {dbuf(9 * C), dbuf(C), dbuf(9 * C),
                                                                           dbuf(C)};
    memset(zero, 0, sizeof(float) * (size_t)C);
    expect(oracle_dwsub_front_fwd(x, w0, b0, w1, b1, L, y, B, T, F, C, causal) == 0, "front", B, T, F, C);
    for (int m = 1; m < 4; ++m) {
        const float *nb0 = (m & 1) ? NULL : b0, *nb1 = (m & 2) ? NULL : b1;
        const float *zb0 = (m & 1) ? zero : b0, *zb1 = (m & 2) ? zero : b1;
        expect(oracle_dwsub_front_fwd(x, w0, nb0, w1, nb1, L, yn, B, T, F, C, causal) == 0, "front null", B, T, F,
               m);
        expect(oracle_dwsub_front_fwd(x, w0, zb0, w1, zb1, L, yz, B, T, F, C, causal) == 0, "front zero", B, T, F,
               m);
        expect(same_bits(yn, yz, ny), "front null bias is zero bias", B, T, F, m);
    }
    expect(oracle_dwsub_front_fwd(x, w0, b0, w1, b1, NULL, y, B, T, F, C, causal) == 0, "front no lengths", B, T,
           F, C);
    expect(oracle_dwsub_front_bwd(x, w0, NULL, w1, L, dy, g[0], g[1], g[2], g[3], B, T, F, C, causal) == 0,
           "front bwd null b0", B, T, F, C);
    expect(oracle_dwsub_front_bwd(x, w0, zero, w1, L, dy, gz[0], gz[1], gz[2], gz[3], B, T, F, C, causal) == 0,
           "front bwd zero b0", B, T, F, C);
    expect(same_bits(g[0], gz[0], 9 * C) && same_bits(g[1], gz[1], C) && same_bits(g[2], gz[2], 9 * C)
               && same_bits(g[3], gz[3], C), "front bwd null b0 is zero b0", B, T, F, C);
    expect(oracle_dwsub_front_bwd(x, w0, b0, w1, NULL, dy, NULL, g[1], NULL, g[3], B, T, F, C, causal) == 0,
           "front bwd some outputs", B, T, F, C);
    ++cases;
    free(x); free(w0); free(b0); free(w1); free(b1); free(zero); free(dy); free(L); free(y); free(yn); free(yz);
    for (int i = 0; i < 4; ++i) { free(g[i]); free(gz[i]); }
}

int main(void)
{
    static const long Ts[] = {0, 1, 2, 3, 5, 8, 13};
    static const long Ks[] = {1, 2, 3, 4, 5, 9, 15};
    for (long B = 0; B <= 3; ++B)
        for (size_t ti = 0; ti < sizeof Ts / sizeof Ts[0]; ++ti)
            for (long C = 1; C <= 3; C += 2)
                for (size_t ki = 0; ki < sizeof Ks / sizeof Ks[0]; ++ki)
                    for (int causal = 0; causal <= 1; ++causal) run_1d(B, Ts[ti], C, Ks[ki], causal);
    static const long geo[][7] = {
        /* KH KW s pt0 pt1 pf0 pf1 */
        {3, 3, 2, 1, 1, 1, 1}, {3, 3, 2, 2, 1, 2, 1}, {3, 3, 2, 2, 0, 1, 2}, {3, 3, 1, 1, 1, 1, 1},
        {1, 1, 1, 0, 0, 0, 0}, {2, 2, 2, 0, 0, 0, 0}, {5, 3, 3, 2, 2, 1, 1}, {3, 1, 2, 1, 1, 0, 0},
    };
    for (long B = 0; B <= 2; ++B)
        for (size_t ti = 0; ti < sizeof Ts / sizeof Ts[0]; ++ti)
            for (long F = 1; F <= 6; F += 5)
                for (size_t g = 0; g < sizeof geo / sizeof geo[0]; ++g)
                    run_2d(B, Ts[ti], F, 2, geo[g][0], geo[g][1], geo[g][2], geo[g][3], geo[g][4], geo[g][5],
                           geo[g][6]);
    for (long B = 0; B <= 2; ++B)
        for (size_t ti = 0; ti < sizeof Ts / sizeof Ts[0]; ++ti)
            for (long F = 1; F <= 9; F += 4)
                for (int causal = 0; causal <= 1; ++causal) run_front(B, Ts[ti], F, 3, causal);
    /* arguments the oracle refuses */
    float one = 1.0f;
    double out = 0.0;
    expect(oracle_dwconv1d_fwd(&one, &one, NULL, NULL, &out, 1, 1, 1, 0, 0) == -1, "1d K = 0 refused", 0, 0, 0, 0);
    expect(oracle_dwconv1d_fwd(&one, &one, NULL, NULL, &out, -1, 1, 1, 1, 0) == -1, "1d B < 0 refused", 0, 0, 0, 0);
    expect(oracle_dwsub_front_fwd(&one, &one, NULL, &one, NULL, NULL, &out, 1, -1, 1, 1, 0) == -1,
           "front T < 0 refused", 0, 0, 0, 0);
    printf("oracle sanitizer run: %ld cases, %d failures\n", cases, failures);
    return failures == 0 ? 0 : 1;
}
