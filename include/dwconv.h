/*
 * dwconv.h -- C ABI of the depthwise-convolution library for AMD Instinct
 * MI355X (gfx950).
 *
 * What it computes (the pages cited are parakeet.cpp PR #102, "one SSM_CONV
 * for the depthwise conv, less host work per step", and NVIDIA NeMo PR
 * #16114, "Use Fused Kernels for Depthwise Striding Subsampler"):
 *   dwconv1d_fwd     the Conformer conv module's depthwise Conv1d in SSM_CONV
 *                    form (PR #102, "What changes")
 *   dwconv1d_bwd     its gradients dx, dw, db (the conv module in training)
 *   dwconv1d_stream_fwd
 *                    its streaming form with a K-1 frame cache (same PR:
 *                    the streaming encoder's conv with a cache)
 *   dwsub_fused_fwd  the depthwise-striding subsampler front: conv0, bias,
 *                    ReLU, time mask and depthwise conv, fused (PR #16114,
 *                    "What does this PR do", first kernel)
 *   dwconv2d_fwd     the general depthwise conv2d with pre/post masking
 *                    (PR #16114, "What does this PR do", second kernel)
 *   dwsub_fused_bwd  the front's parameter gradients dw0, db0, dw1, db1
 *                    (same section: the kernels serve the training step)
 *   dwconv2d_bwd     its backward: dx, dw, db (same section)
 *   dwconv2d_fwd_ex, dwconv2d_bwd_ex
 *                    the same with per-side padding (the causal padding of
 *                    the same section) and bf16 storage
 *   dwsub_fused_fwd_ex, dwsub_fused_bwd_ex
 *                    the front with its causal mode (same section) and bf16
 *                    storage
 *
 * Conventions shared by every entry point
 *   - Tensors are dense, contiguous and channel-last (channel index fastest):
 *     [B][T][C] for 1-D, [B][T][F][C] for 2-D, [B][T][F] for the one-channel
 *     mel input.  Weights are tap-major: w[K][C] (1-D), w[KH][KW][C] (2-D).
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *     library never allocates, frees or synchronises; all work is enqueued
 *     on `stream` (a hipStream_t; NULL means the default stream) and is
 *     asynchronous with respect to the host.
 *   - lengths[B] (int32, device memory) holds each item's valid number of
 *     input frames; it is read on the device and clamped to [0, T].  NULL
 *     means every item is T frames long.  Frames t >= length are treated as
 *     zero on input (pre-mask) and written as exact zeros on output
 *     (post-mask), where the operation masks.
 *   - A NULL bias means a zero bias.
 *   - Sizes are int64_t.  A forward call with no output elements enqueues
 *     nothing and returns DW_OK without looking at its pointers; a tensor
 *     with no elements may be NULL.
 *   - The kernels address each batch item with 32-bit byte offsets: an item
 *     whose tensors (with a few frames of padding) would reach 2^31 bytes is
 *     refused with DW_ERR_UNSUPPORTED ("sizes too large for one launch"),
 *     and so is any extent (B, T, F, C, K) of 2^31 or more.  These limits
 *     are computed without integer overflow for any int64_t input.  The
 *     batch as a whole may be larger than 2^31 bytes.
 *   - The workspace queries take no storage type.  They return 0 for sizes
 *     that their call refuses in both storage types (invalid, unsupported,
 *     or too large for one launch).  An item within the bf16 call's size
 *     limit but past the float32 call's (which is half as large in bytes
 *     per element) gets its workspace size, and the float32 call then
 *     refuses it.
 *   - Errors: every argument is validated on the host before anything is
 *     enqueued.  A failing call returns a negative dw_status, enqueues
 *     nothing (except DW_ERR_HIP, raised when a launch is rejected) and sets
 *     a thread-local message readable with dw_last_error().  No entry point
 *     aborts, and none falls back to another algorithm.
 *   - The library keeps no mutable global state other than that message, so
 *     calls from several host threads are safe.  Two calls whose output
 *     buffers overlap race, as any two kernels writing the same memory do.
 */
#ifndef DWCONV_H
#define DWCONV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DW_ABI_VERSION 1

typedef enum {
    DW_OK = 0,
    DW_ERR_INVALID_ARG = -1,  /* null required pointer, negative size, aliasing, bad enum */
    DW_ERR_UNSUPPORTED = -2,  /* a geometry, width or size this library does not implement */
    DW_ERR_WORKSPACE = -3,    /* workspace missing or smaller than required */
    DW_ERR_HIP = -4           /* the HIP runtime rejected a launch */
} dw_status;

/* The *_INT32_LO_ and *_INT32_HI_ members are not values to pass: they give
 * each enum the full int32 range, so that an out-of-range value from a
 * caller is a defined value of the type (and refused with
 * DW_ERR_INVALID_ARG) rather than undefined behaviour in the library. */
typedef enum {
    DW_F32 = 0,
    DW_BF16 = 1,
    DW_DTYPE_INT32_LO_ = -2147483647 - 1,
    DW_DTYPE_INT32_HI_ = 2147483647
} dw_dtype;

typedef enum {
    DW_PAD_SYMMETRIC = 0,
    DW_PAD_CAUSAL = 1,
    DW_PAD_INT32_LO_ = -2147483647 - 1,
    DW_PAD_INT32_HI_ = 2147483647
} dw_pad;

/* DW_ABI_VERSION of the built library. */
int dw_abi_version(void);

/* Message describing the last failing call on this host thread ("" if none). */
const char *dw_last_error(void);

/*
 * dwconv1d_fwd -- depthwise Conv1d (groups = C) in SSM_CONV form
 * (parakeet.cpp PR #102, "What changes": one SSM_CONV over the input padded
 * to T + K - 1 frames, summing x[t+k, c] * w[k, c] over k).
 *
 *   pL = K - 1                for DW_PAD_CAUSAL (all padding on the left)
 *   pL = (K - 1) / 2          for DW_PAD_SYMMETRIC (an even K puts the extra
 *                             frame of padding on the right)
 *   xs[b, s, c] = x[b, s - pL, c] if 0 <= s - pL < len_b, else 0
 *   y[b, t, c]  = sum_{k<K} xs[b, t + k, c] * w[k, c] + bias[c]   (t < len_b)
 *   y[b, t, c]  = 0                                               (t >= len_b)
 *
 * x, y: [B][T][C]; w: [K][C]; bias: [C] or NULL; lengths: [B] or NULL.
 * dtype DW_F32: all of x, w, bias, y are float.  DW_BF16: all are bf16
 * (uint16 bit patterns); products and sums are carried in float32 and y is
 * rounded to nearest-even.  Any C >= 1 and any K >= 1 are accepted.
 * Errors: DW_ERR_INVALID_ARG for a null x, w or y, a negative size, K < 1, a
 * bad pad or dtype, or x == y.
 */
dw_status dwconv1d_fwd(const void *x, const void *w, const void *bias, const int32_t *lengths,
                       void *y, int64_t B, int64_t T, int64_t C, int64_t K,
                       dw_pad pad, dw_dtype dtype, void *stream);

/*
 * dwconv1d_stream_fwd -- the causal depthwise conv of a streaming encoder,
 * one chunk per call, with a cache of K - 1 frames per stream between calls
 * (parakeet.cpp PR #102, "What changes": the streaming encoder's conv with a
 * cache).  Per stream b, with len_b = clamp(lengths[b], 0, Tc) valid frames
 * in this chunk and s = cache_in[b] followed by x[b, 0:len_b]:
 *   y[b, t, c]         = sum_{k<K} s[t + k, c] * w[k, c] + bias[c]   for t < len_b, else 0
 *   cache_out[b, j, c] = s[len_b + j, c]                            for j < K - 1
 * (the last K - 1 frames of the cache and the chunk together; a stream with
 * len_b = 0 keeps its cache).  From a zero cache, consecutive calls over the
 * chunks of a sequence give its causal convolution (dwconv1d_fwd with
 * DW_PAD_CAUSAL).
 *
 * x, y: [B][Tc][C]; w: [K][C]; bias: [C] or NULL; cache_in, cache_out:
 * [B][K-1][C] (may be NULL when K = 1), in the same storage type as x.
 * dtype DW_F32 or DW_BF16 (everything bf16; fp32 accumulation; cached values
 * are copied bit for bit).  Any K >= 1.  cache_out must be a different
 * buffer from cache_in (callers alternate two), since the new cache is
 * written while the chunk's first frames are being read from the old one.
 * Tc may be 0 (the cache is then copied).
 * Errors: DW_ERR_INVALID_ARG for a NULL required pointer, a negative size,
 * K < 1, a bad dtype, cache_out == cache_in, or y aliasing x or a cache.
 */
dw_status dwconv1d_stream_fwd(const void *x, const void *w, const void *bias, const int32_t *lengths,
                              const void *cache_in, void *y, void *cache_out, int64_t B, int64_t Tc, int64_t C,
                              int64_t K, dw_dtype dtype, void *stream);

/*
 * Bytes of device workspace dwconv1d_bwd needs when it computes dw or db (0
 * for invalid sizes or a width without a backward kernel).
 */
size_t dwconv1d_bwd_workspace_bytes(int64_t B, int64_t T, int64_t C, int64_t K);

/*
 * dwconv1d_bwd -- gradients of dwconv1d_fwd (the conv module's depthwise
 * Conv1d in training; the forward is parakeet.cpp PR #102, "What changes").
 * With pL as in the forward and g = dy at unmasked frames (t < len_b), 0
 * elsewhere:
 *   dx[b, u, c] = sum_k g[b, u + pL - k, c] * w[k, c]     for u < len_b, else 0
 *   dw[k, c]    = sum_{b,u} g[b, u + pL - k, c] * x[b, u, c]   (x masked at u >= len_b)
 *   db[c]       = sum_{b,t} g[b, t, c]
 * dx is gathered (no atomics); dw and db are accumulated in fp64 and reduced
 * in a fixed order, so repeated calls give bitwise-identical results.
 *
 * x, dy, dx: [B][T][C]; w: [K][C]; dx, dw ([K][C]) and db ([C], float) may be
 * NULL (not computed).  dtype DW_F32: x, w, dy, dx are float; DW_BF16: they
 * are bf16 (dx rounded to nearest even), dw and db stay float, summed in fp64
 * from the exactly widened values.  K must be one of 3, 4, 5, 7, 9, 15, 31,
 * else DW_ERR_UNSUPPORTED.  workspace: at least dwconv1d_bwd_workspace_bytes(...)
 * bytes of device memory when dw or db is requested.
 * Errors: DW_ERR_INVALID_ARG for a null x, w or dy that holds elements, a
 * negative size, K < 1, a bad enum, or dx aliasing x or dy;
 * DW_ERR_WORKSPACE for a missing or short workspace.
 */
dw_status dwconv1d_bwd(const void *x, const void *w, const int32_t *lengths, const void *dy, void *dx,
                       float *dw, float *db, void *workspace, size_t workspace_bytes,
                       int64_t B, int64_t T, int64_t C, int64_t K, dw_pad pad, dw_dtype dtype, void *stream);

/*
 * dwsub_fused_fwd -- the depthwise-striding subsampler front, fused (NeMo PR
 * #16114, "What does this PR do": mel [B,T,F,1] -> conv0 3x3 stride 2
 * [B,T/2,F/2,C] -> ReLU -> masking -> depthwise 3x3 stride 2 conv
 * [B,T/4,F/4,C]).  The intermediate h is never written to memory.
 *
 *   T1 = (T+1)/2, F1 = (F+1)/2, L1_b = (len_b+1)/2, T2 = (T1+1)/2, F2 = (F1+1)/2
 *   h[b,t1,f1,c] = max(0, sum_{i,j<3} x[b, 2t1+i-1, 2f1+j-1] * w0[i,j,c] + b0[c])
 *                  for t1 < L1_b, else 0
 *   y[b,t2,f2,c] = sum_{i,j<3} h[b, 2t2+i-1, 2f2+j-1, c] * w1[i,j,c] + b1[c]
 * with zero padding of one on each side of both stages.  The mel input is
 * not length-masked and y is not masked; the one mask is the one on h.
 *
 * x: [B][T][F] float; w0, w1: [3][3][C] float; b0, b1: [C] float or NULL;
 * lengths: [B] or NULL; y: [B][T2][F2][C] float.  Arithmetic is IEEE fp32
 * fused multiply-add (no reduced-precision products).
 * Errors: DW_ERR_INVALID_ARG for a null x, w0, w1 or y, a negative size or
 * x == y.
 */
dw_status dwsub_fused_fwd(const float *x, const float *w0, const float *b0,
                          const float *w1, const float *b1, const int32_t *lengths,
                          float *y, int64_t B, int64_t T, int64_t F, int64_t C, void *stream);

/*
 * Bytes of device workspace dwsub_fused_bwd needs for these sizes (0 for
 * invalid sizes).
 */
size_t dwsub_fused_bwd_workspace_bytes(int64_t B, int64_t T, int64_t F, int64_t C);

/*
 * dwsub_fused_bwd -- gradients of dwsub_fused_fwd with respect to its
 * parameters, for the training step (NeMo PR #16114, "What does this PR
 * do": the fused kernels speed up the encoder's forward and backward).  The
 * mel input needs no gradient.  With z = conv0(x) + b0 before the ReLU, h
 * and y as in dwsub_fused_fwd, and dy [B][T2][F2][C]:
 *   db1[c]     = sum dy
 *   dw1[i,j,c] = sum_{b,t2,f2} dy[b,t2,f2,c] * h[b, 2t2+i-1, 2f2+j-1, c]
 *   dh         = the depthwise stage's input gradient (dy gathered through w1)
 *   dz         = dh where t1 < ceil(len_b/2) and z > 0, else 0
 *   db0[c]     = sum dz
 *   dw0[i,j,c] = sum_{b,t1,f1} dz[b,t1,f1,c] * x[b, 2t1+i-1, 2f1+j-1]
 * h is recomputed on chip and never written.  z, h, dh, dz and every sum are
 * carried in fp64 (the ReLU derivative's decision on the sign of z is then
 * taken as a full-precision reference takes it), and the sums are added in a
 * fixed order, so repeated calls give bitwise-identical results.
 *
 * x: [B][T][F] float; w0, w1: [3][3][C]; b0: [C] or NULL; lengths: [B] or
 * NULL; dy: [B][T2][F2][C]; dw0, dw1: [3][3][C]; db0, db1: [C] (float, any of
 * the four may be NULL).  workspace: device memory of at least
 * dwsub_fused_bwd_workspace_bytes(...) bytes, contents ignored on entry.
 * Errors: DW_ERR_INVALID_ARG for a null x, w0, w1 or dy that holds elements
 * or a negative size; DW_ERR_WORKSPACE for a missing or short workspace.
 */
dw_status dwsub_fused_bwd(const float *x, const float *w0, const float *b0, const float *w1,
                          const int32_t *lengths, const float *dy, float *dw0, float *db0, float *dw1,
                          float *db1, void *workspace, size_t workspace_bytes,
                          int64_t B, int64_t T, int64_t F, int64_t C, void *stream);

/*
 * dwconv2d_fwd -- depthwise conv2d with pre- and post-masking (NeMo PR
 * #16114, "What does this PR do", the general depthwise conv2d kernel).
 *
 *   T' = (T + 2p - KH)/s + 1,  F' = (F + 2p - KW)/s + 1  (floor division)
 *   len'_b = (len_b + 2p - KH)/s + 1 clamped to [0, T'], and 0 if len_b = 0
 *   y[b,t',f',c] = sum_{i,j} xm[b, s t'+i-p, s f'+j-p, c] * w[i,j,c] + bias[c]
 *                  for t' < len'_b, else 0
 * where xm is x with frames t >= len_b zeroed and indices outside the tensor
 * read zero.  For the 3x3, stride 2, pad 1 geometry len' = ceil(len / 2).
 *
 * x: [B][T][F][C] float; w: [KH][KW][C] float; bias: [C] or NULL; y:
 * [B][T'][F'][C] float.  Implemented geometry: KH = KW = 3, stride 2, pad 1
 * or 2; anything else returns DW_ERR_UNSUPPORTED.  Equal to dwconv2d_fwd_ex
 * with the same pad on every side and DW_F32.
 * Errors: DW_ERR_INVALID_ARG for a null x, w or y, a negative size or x == y.
 */
dw_status dwconv2d_fwd(const float *x, const float *w, const float *bias, const int32_t *lengths,
                       float *y, int64_t B, int64_t T, int64_t F, int64_t C,
                       int64_t KH, int64_t KW, int64_t stride, int64_t pad, void *stream);

/*
 * Bytes of device workspace dwconv2d_bwd needs for these sizes when it
 * computes dw or db (a call that requests neither needs none).  Returns 0
 * for an unsupported geometry or invalid sizes.
 */
size_t dwconv2d_bwd_workspace_bytes(int64_t B, int64_t T, int64_t F, int64_t C,
                                    int64_t KH, int64_t KW, int64_t stride, int64_t pad);

/*
 * dwconv2d_bwd -- gradients of dwconv2d_fwd (NeMo PR #16114, "What does this
 * PR do": the general depthwise conv2d backward).  With g = dy at unmasked
 * output rows (t' < len'_b) and 0 elsewhere:
 *   dx[b,t,f,c] = sum over the (t',f',i,j) with t = s t'+i-p, f = s f'+j-p of
 *                 g[b,t',f',c] * w[i,j,c]          for t < len_b, else 0
 *   dw[i,j,c]   = sum_{b,t',f'} g[b,t',f',c] * xm[b, s t'+i-p, s f'+j-p, c]
 *   db[c]       = sum_{b,t',f'} g[b,t',f',c]
 * dx is written in gather form (no atomics); dw and db are accumulated in
 * fp64 (the fp32 products are exact in fp64) and reduced in a fixed order,
 * so repeated calls give bitwise-identical results.
 *
 * x: [B][T][F][C]; w: [KH][KW][C]; dy: [B][T'][F'][C]; dx: [B][T][F][C] or
 * NULL (not computed); dw: [KH][KW][C] or NULL; db: [C] or NULL (all float).
 * workspace: device memory of at least dwconv2d_bwd_workspace_bytes(...)
 * bytes when dw or db is requested (may be NULL otherwise); its contents on
 * entry are ignored and on return are unspecified.
 * Implemented geometry: KH = KW = 3, stride 2, pad 1 or 2 (else
 * DW_ERR_UNSUPPORTED).
 * An empty batch (B, T or F zero) still writes dw = 0 and db = 0; x and dy
 * may then be NULL.
 * Errors: DW_ERR_INVALID_ARG for a null x, w or dy that holds elements, a
 * negative size, dx aliasing x or dy; DW_ERR_WORKSPACE for a missing or
 * short workspace.
 */
dw_status dwconv2d_bwd(const float *x, const float *w, const int32_t *lengths, const float *dy,
                       float *dx, float *dw, float *db, void *workspace, size_t workspace_bytes,
                       int64_t B, int64_t T, int64_t F, int64_t C,
                       int64_t KH, int64_t KW, int64_t stride, int64_t pad, void *stream);

/*
 * dwsub_fused_fwd_ex -- dwsub_fused_fwd with a padding mode: DW_PAD_SYMMETRIC
 * is dwsub_fused_fwd; DW_PAD_CAUSAL is the front's causal mode (NeMo PR
 * #16114, "What does this PR do": the extra padding layer of causal mode),
 * read as both convolutions padding each axis with 2 zeros before and 1
 * after.  With d = 0 (symmetric) or 1 (causal):
 *   T1 = floor((T - 1 + d)/2) + 1, F1 likewise; T2, F2 the same from T1, F1
 *        (0 for an empty axis when d = 0, 1 when d = 1)
 *   L1_b = floor((len_b - 1 + d)/2) + 1, 0 for an empty item
 *   h[b,t1,f1,c] = max(0, sum_{i,j} x[b, 2t1+i-1-d, 2f1+j-1-d] w0[i,j,c] + b0[c])
 *                  for t1 < L1_b, else 0
 *   y[b,t2,f2,c] = sum_{i,j} h[b, 2t2+i-1-d, 2f2+j-1-d, c] w1[i,j,c] + b1[c]
 * dtype DW_F32: x, w0, b0, w1, b1 and y are float.  DW_BF16: they are bf16
 * (uint16 bit patterns), widened exactly, summed in fp32, y rounded to
 * nearest even.  Arguments, layout and errors otherwise as dwsub_fused_fwd;
 * a bad pad or dtype is DW_ERR_INVALID_ARG.
 */
dw_status dwsub_fused_fwd_ex(const void *x, const void *w0, const void *b0, const void *w1, const void *b1,
                             const int32_t *lengths, void *y, int64_t B, int64_t T, int64_t F, int64_t C,
                             dw_pad pad, dw_dtype dtype, void *stream);

/* Workspace of dwsub_fused_bwd_ex (0 for invalid sizes or pad). */
size_t dwsub_fused_bwd_workspace_bytes_ex(int64_t B, int64_t T, int64_t F, int64_t C, dw_pad pad);

/*
 * dwsub_fused_bwd_ex -- dwsub_fused_bwd for either padding mode and storage
 * type of dwsub_fused_fwd_ex (the same gradients with its T2, F2, L1 and
 * indices).  With DW_BF16, x, w0, b0, w1 and dy are bf16; dw0, db0, dw1, db1
 * are always float (summed in fp64).
 */
dw_status dwsub_fused_bwd_ex(const void *x, const void *w0, const void *b0, const void *w1,
                             const int32_t *lengths, const void *dy, float *dw0, float *db0, float *dw1, float *db1,
                             void *workspace, size_t workspace_bytes, int64_t B, int64_t T, int64_t F, int64_t C,
                             dw_pad pad, dw_dtype dtype, void *stream);

/*
 * dwconv2d_fwd_ex -- dwconv2d_fwd with its padding given per axis and side,
 * and a storage type: the general depthwise conv2d of NeMo PR #16114 ("What
 * does this PR do"), which fuses the masking and the causal padding.
 *
 *   pad_t0 / pad_t1: zero rows before / after the input in time
 *   pad_f0 / pad_f1: zero columns before / after it in frequency
 *   T' = floor((T + pad_t0 + pad_t1 - KH)/s) + 1, F' likewise,
 *   len'_b = floor((len_b + pad_t0 + pad_t1 - KH)/s) + 1 clamped to [0, T'],
 *            and 0 if len_b = 0
 *   y[b,t',f',c] = sum_{i,j} xm[b, s t'+i-pad_t0, s f'+j-pad_f0, c] * w[i,j,c]
 *                  + bias[c]  for t' < len'_b, else 0
 * Symmetric padding is pad 1 everywhere (dwconv2d_fwd's pad = 1).  The causal
 * padding is read as KH - 1 = 2 before and s - 1 = 1 after on each axis
 * (2, 1, 2, 1): output row t' then reads input rows up to 2t' only.
 *
 * dtype DW_F32: x, w, bias, y are float.  DW_BF16: they are bf16 (uint16
 * bit patterns), widened exactly to fp32, accumulated in fp32 and stored
 * rounded to nearest even.
 * Implemented: KH = KW = 3, stride 2, pad_t0 and pad_f0 in {1, 2}, pad_t1
 * and pad_f1 in {0, 1, 2}; other valid geometries return DW_ERR_UNSUPPORTED,
 * negative pads DW_ERR_INVALID_ARG.  Errors otherwise as dwconv2d_fwd.
 */
dw_status dwconv2d_fwd_ex(const void *x, const void *w, const void *bias, const int32_t *lengths, void *y,
                          int64_t B, int64_t T, int64_t F, int64_t C, int64_t KH, int64_t KW, int64_t stride,
                          int64_t pad_t0, int64_t pad_t1, int64_t pad_f0, int64_t pad_f1, dw_dtype dtype,
                          void *stream);

/* Workspace of dwconv2d_bwd_ex for these sizes and pads (0 if unsupported). */
size_t dwconv2d_bwd_workspace_bytes_ex(int64_t B, int64_t T, int64_t F, int64_t C, int64_t KH, int64_t KW,
                                       int64_t stride, int64_t pad_t0, int64_t pad_t1, int64_t pad_f0,
                                       int64_t pad_f1);

/*
 * dwconv2d_bwd_ex -- gradients of dwconv2d_fwd_ex: as dwconv2d_bwd with
 * t = s t'+i-pad_t0, f = s f'+j-pad_f0 and len' as in dwconv2d_fwd_ex.
 * dtype DW_BF16: x, w, dy and dx are bf16; dw and db are always float
 * (accumulated in fp64 from the exactly widened values).  workspace: at
 * least dwconv2d_bwd_workspace_bytes_ex(...) bytes when dw or db is
 * requested.  Implemented geometries and errors as dwconv2d_fwd_ex and
 * dwconv2d_bwd.
 */
dw_status dwconv2d_bwd_ex(const void *x, const void *w, const int32_t *lengths, const void *dy, void *dx,
                          float *dw, float *db, void *workspace, size_t workspace_bytes,
                          int64_t B, int64_t T, int64_t F, int64_t C, int64_t KH, int64_t KW, int64_t stride,
                          int64_t pad_t0, int64_t pad_t1, int64_t pad_f0, int64_t pad_f1, dw_dtype dtype,
                          void *stream);

/*
 * dwconv2d_bwd_noalloc -- dwconv2d_bwd_ex with no workspace argument, for
 * callers that cannot allocate device memory around a call: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * The same gradients, bit for bit, as dwconv2d_bwd_ex with the same
 * arguments (the same kernels run).  The fp64 partial sums of dw and db go to
 * a 16 MiB array that the library holds on each GPU it runs on, for the life
 * of the process; the call itself allocates nothing and frees nothing
 * (callers still pass every input and output).  Every call on one GPU shares
 * that GPU's array, so two calls that overlap in time on the same GPU (on
 * different streams, or from different host threads without ordering) race
 * and may return wrong dw and db; calls ordered on one stream do not.
 * Arguments, layouts, ownership and the other errors are those of
 * dwconv2d_bwd_ex.  Errors: DW_ERR_UNSUPPORTED when dw or db is requested
 * and the partials would not fit the array: they take (P + 4) * 10 * C * 8
 * bytes for P <= 256 workgroup partials (fewer for a small batch), so at
 * most 806 channels fit at any batch size; DW_ERR_HIP if the array's device
 * address cannot be looked up.
 */
dw_status dwconv2d_bwd_noalloc(const void *x, const void *w, const int32_t *lengths, const void *dy, void *dx,
                               float *dw, float *db, int64_t B, int64_t T, int64_t F, int64_t C, int64_t KH,
                               int64_t KW, int64_t stride, int64_t pad_t0, int64_t pad_t1, int64_t pad_f0,
                               int64_t pad_f1, dw_dtype dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DWCONV_H */
