/*
 * CPU oracle for the depthwise-convolution path.  TEST INFRASTRUCTURE ONLY:
 * the tests, the smoke check and the CPU-baseline leg of the benchmark may
 * call it; the library never does.
 *
 * Plain, single-threaded C.  Inputs are the float32 values the GPU sees
 * (bf16 values are exactly representable as float32); every sum is carried
 * in double and every output is double.  No blocking, no fusion, no
 * reordering beyond what each definition states.  Built with
 * -O2 -fno-fast-math -ffp-contract=off.
 *
 * Layouts (all contiguous, channel fastest):
 *   1-D:  x, y [B][T][C];  w [K][C];  bias [C]
 *   2-D:  x [B][T][F][C];  y, dy [B][T'][F'][C];  w [KH][KW][C];  bias [C]
 *   front: x [B][T][F] (one input channel);  y [B][T2][F2][C]
 * lengths [B] (int32) may be NULL (every item full length); bias may be NULL
 * (zero).  A length is clamped to [0, T].
 *
 * Sources (parakeet.cpp PR #102, "one SSM_CONV for the depthwise conv";
 * NVIDIA NeMo PR #16114, "Use Fused Kernels for Depthwise Striding
 * Subsampler"): cited per function below.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static long clamp_len(const int32_t *lengths, long b, long T)
{
    long l = lengths ? (long)lengths[b] : T;
    if (l < 0) l = 0;
    if (l > T) l = T;
    return l;
}

/* floor(a / b) for b > 0 and any sign of a. */
static long floor_div(long a, long b)
{
    long q = a / b;
    if ((a % b != 0) && (a < 0)) q -= 1;
    return q;
}

/* Output length of a convolution along one axis with pl zeros before the
 * input and ph after it: floor((n + pl + ph - k)/s) + 1, never below zero. */
static long conv_out_len(long n, long k, long s, long pl, long ph)
{
    long o = floor_div(n + pl + ph - k, s) + 1;
    return o < 0 ? 0 : o;
}

/*
 * 1-D depthwise convolution in SSM_CONV form (parakeet.cpp PR #102,
 * "What changes": the conv computed as one SSM_CONV over the input padded to
 * T + K - 1 frames, summing x[t + k, c] * w[k, c] over k, equal to NeMo's
 * depthwise Conv1d for the same left padding, causal or not).
 *
 * Per item b and channel c this builds the padded, pre-masked signal
 *   xp[s] = x[b, s - pL, c]  if 0 <= s - pL < len_b, else 0,   s in [0, T+K-1)
 * with pL = K - 1 (causal) or (K - 1) / 2 (symmetric; an even K puts the
 * extra frame of padding on the right), then
 *   y[b, t, c] = sum_{k=0}^{K-1} xp[t + k] * w[k, c] + bias[c]   for t < len_b
 *   y[b, t, c] = 0                                              for t >= len_b.
 * Returns 0, or -1 on a bad argument or allocation failure.
 */
int oracle_dwconv1d_fwd(const float *x, const float *w, const float *bias,
                        const int32_t *lengths, double *y,
                        long B, long T, long C, long K, int causal)
{
    if (B < 0 || T < 0 || C < 0 || K < 1) return -1;
    long pL = causal ? K - 1 : (K - 1) / 2;
    long P = T + K - 1;
    double *xp = (double *)malloc(sizeof(double) * (size_t)(P > 0 ? P : 1));
    if (!xp) return -1;
    for (long b = 0; b < B; ++b) {
        long len = clamp_len(lengths, b, T);
        for (long c = 0; c < C; ++c) {
            for (long s = 0; s < P; ++s) {
                long t = s - pL;
                xp[s] = (t >= 0 && t < len) ? (double)x[(b * T + t) * C + c] : 0.0;
            }
            for (long t = 0; t < T; ++t) {
                double acc = 0.0;
                if (t < len) {
                    for (long k = 0; k < K; ++k)
                        acc += xp[t + k] * (double)w[k * C + c];
                    acc += bias ? (double)bias[c] : 0.0;
                }
                y[(b * T + t) * C + c] = acc;
            }
        }
    }
    free(xp);
    return 0;
}

/*
 * Depthwise 2-D convolution with length masking (NeMo PR #16114, "What does
 * this PR do": the general depthwise conv2d, with pre- and post-masking
 * fused).  For a KH x KW kernel, stride s, and pt0 zero rows before the
 * input and pt1 after it in time, pf0 and pf1 columns before and after it in
 * frequency (pt0 = pt1 = pf0 = pf1 = p is the symmetric padding; the causal
 * padding the same section names is read as pt0 = KH - 1, pt1 = s - 1, and
 * likewise in frequency):
 *   T' = floor((T + pt0 + pt1 - KH)/s) + 1,  F' = floor((F + pf0 + pf1 - KW)/s) + 1,
 *   len'_b = clamp(floor((len_b + pt0 + pt1 - KH)/s) + 1, 0, T')  (0 for an empty item),
 *   xm[b, t, f, c] = x[b, t, f, c] if t < len_b, else 0 (pre-mask),
 *   y[b, t', f', c] = sum_{i,j} xm[b, s t' + i - pt0, s f' + j - pf0, c] * w[i, j, c]
 *                     + bias[c]                  for t' < len'_b,
 *   y[b, t', f', c] = 0                          for t' >= len'_b (post-mask),
 * where indices outside [0,T) x [0,F) read zero.
 */
int oracle_dwconv2d_fwd(const float *x, const float *w, const float *bias,
                        const int32_t *lengths, double *y,
                        long B, long T, long F, long C,
                        long KH, long KW, long s, long pt0, long pt1, long pf0, long pf1)
{
    if (B < 0 || T < 0 || F < 0 || C < 0 || KH < 1 || KW < 1 || s < 1) return -1;
    if (pt0 < 0 || pt1 < 0 || pf0 < 0 || pf1 < 0) return -1;
    long To = conv_out_len(T, KH, s, pt0, pt1), Fo = conv_out_len(F, KW, s, pf0, pf1);
    for (long b = 0; b < B; ++b) {
        long len = clamp_len(lengths, b, T);
        long leno = conv_out_len(len, KH, s, pt0, pt1);
        if (leno > To) leno = To;
        if (len == 0) leno = 0;
        for (long to = 0; to < To; ++to)
            for (long fo = 0; fo < Fo; ++fo)
                for (long c = 0; c < C; ++c) {
                    double acc = 0.0;
                    if (to < leno) {
                        for (long i = 0; i < KH; ++i) {
                            long t = s * to + i - pt0;
                            if (t < 0 || t >= len) continue; /* padding or pre-masked */
                            for (long j = 0; j < KW; ++j) {
                                long f = s * fo + j - pf0;
                                if (f < 0 || f >= F) continue;
                                acc += (double)x[((b * T + t) * F + f) * C + c] *
                                       (double)w[(i * KW + j) * C + c];
                            }
                        }
                        acc += bias ? (double)bias[c] : 0.0;
                    }
                    y[((b * To + to) * Fo + fo) * C + c] = acc;
                }
    }
    return 0;
}

/*
 * Backward of oracle_dwconv2d_fwd with respect to x, w and bias, given the
 * upstream gradient dy [B][T'][F'][C].  Only dy at unmasked output rows
 * (t' < len'_b) flows back, since masked outputs are constants.  Written in
 * scatter order: every unmasked dy element pushes its contribution to each
 * of the KH*KW input positions it was computed from.
 *   dx[b, t, f, c] += dy[b, t', f', c] * w[i, j, c]     (only where t < len_b:
 *                                                        the pre-mask's derivative)
 *   dw[i, j, c]    += dy[b, t', f', c] * xm[b, t, f, c]
 *   db[c]          += dy[b, t', f', c]
 * with t = s t' + i - pt0, f = s f' + j - pf0 (pads as in the forward).  Any
 * of dx, dw, db may be NULL.
 */
int oracle_dwconv2d_bwd(const float *x, const float *w, const int32_t *lengths,
                        const float *dy, double *dx, double *dw, double *db,
                        long B, long T, long F, long C,
                        long KH, long KW, long s, long pt0, long pt1, long pf0, long pf1)
{
    if (B < 0 || T < 0 || F < 0 || C < 0 || KH < 1 || KW < 1 || s < 1) return -1;
    if (pt0 < 0 || pt1 < 0 || pf0 < 0 || pf1 < 0) return -1;
    long To = conv_out_len(T, KH, s, pt0, pt1), Fo = conv_out_len(F, KW, s, pf0, pf1);
    if (dx) memset(dx, 0, sizeof(double) * (size_t)(B * T * F * C));
    if (dw) memset(dw, 0, sizeof(double) * (size_t)(KH * KW * C));
    if (db) memset(db, 0, sizeof(double) * (size_t)C);
    for (long b = 0; b < B; ++b) {
        long len = clamp_len(lengths, b, T);
        long leno = conv_out_len(len, KH, s, pt0, pt1);
        if (leno > To) leno = To;
        if (len == 0) leno = 0;
        for (long to = 0; to < leno; ++to)
            for (long fo = 0; fo < Fo; ++fo)
                for (long c = 0; c < C; ++c) {
                    double g = (double)dy[((b * To + to) * Fo + fo) * C + c];
                    if (db) db[c] += g;
                    for (long i = 0; i < KH; ++i) {
                        long t = s * to + i - pt0;
                        if (t < 0 || t >= len) continue;
                        for (long j = 0; j < KW; ++j) {
                            long f = s * fo + j - pf0;
                            if (f < 0 || f >= F) continue;
                            size_t xi = (size_t)(((b * T + t) * F + f) * C + c);
                            size_t wi = (size_t)((i * KW + j) * C + c);
                            if (dx) dx[xi] += g * (double)w[wi];
                            if (dw) dw[wi] += g * (double)x[xi];
                        }
                    }
                }
    }
    return 0;
}

/*
 * The depthwise-striding subsampler front (NeMo PR #16114, "What does this
 * PR do": mel input [B,T,F,1] -> conv0 [B,T/2,F/2,256] -> ReLU -> masking ->
 * conv_dw1 [B,T/4,F/4,256]).  Both convolutions pad every axis with pl zeros
 * before and one after: pl = 1 is the symmetric padding, pl = 2 the causal
 * mode (the section's "extra padding layer", read as K - 1 = 2 zeros before
 * and stride - 1 = 1 after).  Computed unfused, stage by stage, with h held
 * in memory:
 *   T1 = floor((T+pl-2)/2) + 1,  F1 = floor((F+pl-2)/2) + 1,
 *   L1_b = floor((len_b+pl-2)/2) + 1 (0 for an empty item): ceil(len_b/2)
 *          for pl = 1, floor(len_b/2) + 1 for pl = 2
 *   h[b,t1,f1,c] = max(0, sum_{i,j<3} xz[b, 2t1+i-pl, 2f1+j-pl] * w0[i,j,c] + b0[c])
 *                  for t1 < L1_b, and 0 for t1 >= L1_b (the time mask)
 *   T2 = floor((T1+pl-2)/2) + 1,  F2 = floor((F1+pl-2)/2) + 1
 *   y[b,t2,f2,c] = sum_{i,j<3} hz[b, 2t2+i-pl, 2f2+j-pl, c] * w1[i,j,c] + b1[c]
 * where xz and hz read zero outside their extents.  The mel input is not
 * length-masked and the output is not masked: the only mask in the chain is
 * the one after the ReLU.
 */
int oracle_dwsub_front_fwd(const float *x, const float *w0, const float *b0,
                           const float *w1, const float *b1, const int32_t *lengths,
                           double *y, long B, long T, long F, long C, int causal)
{
    if (B < 0 || T < 0 || F < 0 || C < 0) return -1;
    long pl = causal ? 2 : 1;
    long T1 = conv_out_len(T, 3, 2, pl, 1), F1 = conv_out_len(F, 3, 2, pl, 1);
    long T2 = conv_out_len(T1, 3, 2, pl, 1), F2 = conv_out_len(F1, 3, 2, pl, 1);
    size_t hn = (size_t)(T1 * F1 * C);
    double *h = (double *)malloc(sizeof(double) * (hn ? hn : 1));
    if (!h) return -1;
    for (long b = 0; b < B; ++b) {
        long len = clamp_len(lengths, b, T);
        long L1 = len > 0 ? conv_out_len(len, 3, 2, pl, 1) : 0;
        /* stage 1: conv0 (one input channel to C), bias, ReLU, time mask */
        for (long t1 = 0; t1 < T1; ++t1)
            for (long f1 = 0; f1 < F1; ++f1)
                for (long c = 0; c < C; ++c) {
                    double v = 0.0;
                    if (t1 < L1) {
                        double acc = 0.0;
                        for (long i = 0; i < 3; ++i) {
                            long t = 2 * t1 + i - pl;
                            if (t < 0 || t >= T) continue;
                            for (long j = 0; j < 3; ++j) {
                                long f = 2 * f1 + j - pl;
                                if (f < 0 || f >= F) continue;
                                acc += (double)x[(b * T + t) * F + f] * (double)w0[(i * 3 + j) * C + c];
                            }
                        }
                        acc += b0 ? (double)b0[c] : 0.0;
                        v = acc > 0.0 ? acc : 0.0;
                    }
                    h[(t1 * F1 + f1) * C + c] = v;
                }
        /* stage 2: depthwise 3x3 stride 2 over h, plus bias */
        for (long t2 = 0; t2 < T2; ++t2)
            for (long f2 = 0; f2 < F2; ++f2)
                for (long c = 0; c < C; ++c) {
                    double acc = 0.0;
                    for (long i = 0; i < 3; ++i) {
                        long t1 = 2 * t2 + i - pl;
                        if (t1 < 0 || t1 >= T1) continue;
                        for (long j = 0; j < 3; ++j) {
                            long f1 = 2 * f2 + j - pl;
                            if (f1 < 0 || f1 >= F1) continue;
                            acc += h[(t1 * F1 + f1) * C + c] * (double)w1[(i * 3 + j) * C + c];
                        }
                    }
                    acc += b1 ? (double)b1[c] : 0.0;
                    y[((b * T2 + t2) * F2 + f2) * C + c] = acc;
                }
    }
    free(h);
    return 0;
}

/*
 * Backward of the subsampler front with respect to its parameters (the
 * training step of NeMo PR #16114, "What does this PR do": the fused kernels
 * speed up the encoder's forward and backward).  The mel input needs no
 * gradient.  With z = conv0(x) + b0 (before the ReLU) and h as in
 * oracle_dwsub_front_fwd, given dy [B][T2][F2][C]:
 *   db1[c]      = sum dy[b,t2,f2,c]
 *   dw1[i,j,c]  = sum dy[b,t2,f2,c] * hz[b, 2t2+i-pl, 2f2+j-pl, c]
 *   dh[b,t1,f1,c] = sum over (t2,i,f2,j) with t1 = 2t2+i-pl, f1 = 2f2+j-pl of
 *                   dy[b,t2,f2,c] * w1[i,j,c]
 *   dz          = dh where t1 < L1_b and z > 0, else 0 (ReLU and mask)
 *   db0[c]      = sum dz
 *   dw0[i,j,c]  = sum dz[b,t1,f1,c] * xz[b, 2t1+i-pl, 2f1+j-pl]
 * (pl, T1 and L1 as in the forward).  Computed unfused: z, h and dh are
 * materialised per item, dh in scatter order.  Any output pointer may be
 * NULL.
 */
int oracle_dwsub_front_bwd(const float *x, const float *w0, const float *b0,
                           const float *w1, const int32_t *lengths, const float *dy,
                           double *dw0, double *db0, double *dw1, double *db1,
                           long B, long T, long F, long C, int causal)
{
    if (B < 0 || T < 0 || F < 0 || C < 0) return -1;
    long pl = causal ? 2 : 1;
    long T1 = conv_out_len(T, 3, 2, pl, 1), F1 = conv_out_len(F, 3, 2, pl, 1);
    long T2 = conv_out_len(T1, 3, 2, pl, 1), F2 = conv_out_len(F1, 3, 2, pl, 1);
    size_t hn = (size_t)(T1 * F1 * C);
    double *z = (double *)malloc(sizeof(double) * (hn ? hn : 1));
    double *h = (double *)malloc(sizeof(double) * (hn ? hn : 1));
    double *dh = (double *)malloc(sizeof(double) * (hn ? hn : 1));
    if (!z || !h || !dh) { free(z); free(h); free(dh); return -1; }
    if (dw0) memset(dw0, 0, sizeof(double) * (size_t)(9 * C));
    if (db0) memset(db0, 0, sizeof(double) * (size_t)C);
    if (dw1) memset(dw1, 0, sizeof(double) * (size_t)(9 * C));
    if (db1) memset(db1, 0, sizeof(double) * (size_t)C);
    for (long b = 0; b < B; ++b) {
        long len = clamp_len(lengths, b, T);
        long L1 = len > 0 ? conv_out_len(len, 3, 2, pl, 1) : 0;
        /* forward again: z = conv0(x) + b0, h = mask * ReLU(z) */
        for (long t1 = 0; t1 < T1; ++t1)
            for (long f1 = 0; f1 < F1; ++f1)
                for (long c = 0; c < C; ++c) {
                    double acc = 0.0;
                    for (long i = 0; i < 3; ++i) {
                        long t = 2 * t1 + i - pl;
                        if (t < 0 || t >= T) continue;
                        for (long j = 0; j < 3; ++j) {
                            long f = 2 * f1 + j - pl;
                            if (f < 0 || f >= F) continue;
                            acc += (double)x[(b * T + t) * F + f] * (double)w0[(i * 3 + j) * C + c];
                        }
                    }
                    acc += b0 ? (double)b0[c] : 0.0;
                    size_t q = (size_t)((t1 * F1 + f1) * C + c);
                    z[q] = acc;
                    h[q] = (t1 < L1 && acc > 0.0) ? acc : 0.0;
                    dh[q] = 0.0;
                }
        /* stage 2 backward, scatter order */
        for (long t2 = 0; t2 < T2; ++t2)
            for (long f2 = 0; f2 < F2; ++f2)
                for (long c = 0; c < C; ++c) {
                    double g = (double)dy[((b * T2 + t2) * F2 + f2) * C + c];
                    if (db1) db1[c] += g;
                    for (long i = 0; i < 3; ++i) {
                        long t1 = 2 * t2 + i - pl;
                        if (t1 < 0 || t1 >= T1) continue;
                        for (long j = 0; j < 3; ++j) {
                            long f1 = 2 * f2 + j - pl;
                            if (f1 < 0 || f1 >= F1) continue;
                            size_t q = (size_t)((t1 * F1 + f1) * C + c);
                            if (dw1) dw1[(i * 3 + j) * C + c] += g * h[q];
                            dh[q] += g * (double)w1[(i * 3 + j) * C + c];
                        }
                    }
                }
        /* through the mask and the ReLU, then conv0's parameters */
        for (long t1 = 0; t1 < T1; ++t1)
            for (long f1 = 0; f1 < F1; ++f1)
                for (long c = 0; c < C; ++c) {
                    size_t q = (size_t)((t1 * F1 + f1) * C + c);
                    if (t1 >= L1) continue; /* masked: contributes nothing (and is never read) */
                    double dz = z[q] > 0.0 ? dh[q] : 0.0;
                    if (db0) db0[c] += dz;
                    if (!dw0) continue;
                    for (long i = 0; i < 3; ++i) {
                        long t = 2 * t1 + i - pl;
                        if (t < 0 || t >= T) continue;
                        for (long j = 0; j < 3; ++j) {
                            long f = 2 * f1 + j - pl;
                            if (f < 0 || f >= F) continue;
                            dw0[(i * 3 + j) * C + c] += dz * (double)x[(b * T + t) * F + f];
                        }
                    }
                }
    }
    free(z);
    free(h);
    free(dh);
    return 0;
}

/*
 * Backward of oracle_dwconv1d_fwd with respect to x, w and bias, given dy
 * [B][T][C] (the conv module's depthwise Conv1d in training; the forward is
 * parakeet.cpp PR #102, "What changes").  Only dy at unmasked output frames
 * (t < len_b) flows back.  Scatter order: every unmasked dy element pushes
 * its contribution to the K padded input frames it was computed from.
 *   db[c]          += dy[b, t, c]
 *   dx[b, u, c]    += dy[b, t, c] * w[k, c]      for u = t + k - pL, 0 <= u < len_b
 *   dw[k, c]       += dy[b, t, c] * x[b, u, c]   (same u)
 * pL as in the forward.  dx at u >= len_b stays 0 (the pre-mask's
 * derivative).  Any of dx, dw, db may be NULL.
 */
int oracle_dwconv1d_bwd(const float *x, const float *w, const int32_t *lengths, const float *dy,
                        double *dx, double *dw, double *db, long B, long T, long C, long K, int causal)
{
    if (B < 0 || T < 0 || C < 0 || K < 1) return -1;
    long pL = causal ? K - 1 : (K - 1) / 2;
    if (dx) memset(dx, 0, sizeof(double) * (size_t)(B * T * C));
    if (dw) memset(dw, 0, sizeof(double) * (size_t)(K * C));
    if (db) memset(db, 0, sizeof(double) * (size_t)C);
    for (long b = 0; b < B; ++b) {
        long len = clamp_len(lengths, b, T);
        for (long t = 0; t < len; ++t)
            for (long c = 0; c < C; ++c) {
                double g = (double)dy[(b * T + t) * C + c];
                if (db) db[c] += g;
                for (long k = 0; k < K; ++k) {
                    long u = t + k - pL;
                    if (u < 0 || u >= len) continue;
                    if (dx) dx[(b * T + u) * C + c] += g * (double)w[k * C + c];
                    if (dw) dw[k * C + c] += g * (double)x[(b * T + u) * C + c];
                }
            }
    }
    return 0;
}

/*
 * Streaming form of the causal 1-D depthwise conv: the conv module of a
 * streaming encoder runs on one chunk of frames per call and keeps a cache of
 * the last K - 1 input frames between calls (parakeet.cpp PR #102, "What
 * changes": the streaming encoder's conv with a cache; the reson8 wiki,
 * "Keep state on the GPU": streaming models carry state between chunks).
 * Per stream b, with len_b = clamp(lengths[b], 0, Tc) valid frames in this
 * chunk, the sequence the call convolves is the cache followed by them:
 *   s[j]              = cache_in[b, j, c]          for j < K - 1
 *   s[K - 1 + u]      = x[b, u, c]                 for u < len_b
 *   y[b, t, c]        = sum_{k<K} s[t + k] * w[k, c] + bias[c]   for t < len_b
 *   y[b, t, c]        = 0                                        for t >= len_b
 *   cache_out[b, j, c] = s[len_b + j]              for j < K - 1
 * (the last K - 1 frames of the cache and the chunk together).  Starting
 * from a zero cache, calling this on consecutive chunks of a sequence gives
 * the causal convolution of the whole sequence.  x, y [B][Tc][C]; caches
 * [B][K-1][C]; cache_out is double and holds input values exactly.
 */
int oracle_dwconv1d_stream_fwd(const float *x, const float *w, const float *bias,
                               const int32_t *lengths, const float *cache_in,
                               double *y, double *cache_out,
                               long B, long Tc, long C, long K)
{
    if (B < 0 || Tc < 0 || C < 0 || K < 1) return -1;
    long S = K - 1 + Tc;
    double *sq = (double *)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
    if (!sq) return -1;
    for (long b = 0; b < B; ++b) {
        long len = clamp_len(lengths, b, Tc);
        for (long c = 0; c < C; ++c) {
            for (long j = 0; j < K - 1; ++j) sq[j] = (double)cache_in[(b * (K - 1) + j) * C + c];
            for (long u = 0; u < len; ++u) sq[K - 1 + u] = (double)x[(b * Tc + u) * C + c];
            for (long t = 0; t < Tc; ++t) {
                double acc = 0.0;
                if (t < len) {
                    for (long k = 0; k < K; ++k)
                        acc += sq[t + k] * (double)w[k * C + c];
                    acc += bias ? (double)bias[c] : 0.0;
                }
                y[(b * Tc + t) * C + c] = acc;
            }
            for (long j = 0; j < K - 1; ++j) cache_out[(b * (K - 1) + j) * C + c] = sq[len + j];
        }
    }
    free(sq);
    return 0;
}
