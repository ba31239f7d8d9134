// The library's C ABI (declared in include/dwconv.h): host-side argument
// validation, the thread-local error message, and dispatch to the kernel
// launchers.  Nothing here allocates, frees or synchronises.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/dwconv.h"
#include "launch.h"
#include "scratch.h"

#ifndef DW1D_BF16_VEC
#define DW1D_BF16_VEC 4  // bf16 channels per lane access in the 1-D kernel
#endif

namespace {

thread_local char g_err[512] = "";

dw_status fail(dw_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

dw_status ok() {
    g_err[0] = '\0';
    return DW_OK;
}

dw_status from_hip(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(DW_ERR_HIP, "%s: HIP launch failed: %s", what, hipGetErrorString(e));
}

// The 2-D kernels: a 3x3 kernel, stride 2, and the paddings
// dwconv2d_pads_supported accepts.
dw_status check_geometry_2d(const char* fn, int64_t KH, int64_t KW, int64_t stride, int64_t pt0, int64_t pt1,
                            int64_t pf0, int64_t pf1) {
    if (KH < 1 || KW < 1 || stride < 1 || pt0 < 0 || pt1 < 0 || pf0 < 0 || pf1 < 0)
        return fail(DW_ERR_INVALID_ARG, "%s: kernel %lldx%lld, stride %lld, pads (%lld, %lld, %lld, %lld) are not a "
                    "valid geometry", fn, (long long)KH, (long long)KW, (long long)stride, (long long)pt0,
                    (long long)pt1, (long long)pf0, (long long)pf1);
    if (KH != 3 || KW != 3 || stride != 2 || !dw::dwconv2d_pads_supported(pt0, pt1, pf0, pf1))
        return fail(DW_ERR_UNSUPPORTED, "%s: implemented for a 3x3 kernel, stride 2, padding 1 or 2 before and 0 to 2 "
                    "after on each axis (got %lldx%lld, stride %lld, pads (%lld, %lld, %lld, %lld))", fn,
                    (long long)KH, (long long)KW, (long long)stride, (long long)pt0, (long long)pt1,
                    (long long)pf0, (long long)pf1);
    return DW_OK;
}

// True when every extent is positive: a tensor with these extents holds
// elements.  (Multiplying the extents could overflow.)
template <typename... I>
bool nonempty(I... n) {
    return ((n > 0) && ...);
}

// Whether every extent is below dw::kMaxExtent (the launchers' size checks
// add extents together and need that bound; larger ones cannot fit anyway).
template <typename... I>
bool extents_ok(I... n) {
    return ((n < dw::kMaxExtent) && ...);
}

dw_status too_large(const char* fn) { return fail(DW_ERR_UNSUPPORTED, "%s: sizes too large for one launch", fn); }

bool geometry_ok_2d(int64_t KH, int64_t KW, int64_t stride, int64_t pt0, int64_t pt1, int64_t pf0, int64_t pf1) {
    return KH == 3 && KW == 3 && stride == 2 && dw::dwconv2d_pads_supported(pt0, pt1, pf0, pf1);
}

dw_status check_pad(const char* fn, dw_pad pad) {
    if (pad != DW_PAD_SYMMETRIC && pad != DW_PAD_CAUSAL)
        return fail(DW_ERR_INVALID_ARG, "%s: unknown pad mode %d", fn, (int)pad);
    return DW_OK;
}

}  // namespace

extern "C" {

int dw_abi_version(void) { return DW_ABI_VERSION; }

const char* dw_last_error(void) { return g_err; }

dw_status dwconv1d_fwd(const void* x, const void* w, const void* bias, const int32_t* lengths,
                       void* y, int64_t B, int64_t T, int64_t C, int64_t K,
                       dw_pad pad, dw_dtype dtype, void* stream) {
    const char* fn = "dwconv1d_fwd";
    if (B < 0 || T < 0 || C < 0) return fail(DW_ERR_INVALID_ARG, "%s: negative size (B=%lld T=%lld C=%lld)", fn, (long long)B, (long long)T, (long long)C);
    if (K < 1) return fail(DW_ERR_INVALID_ARG, "%s: kernel width K=%lld must be >= 1", fn, (long long)K);
    if (pad != DW_PAD_SYMMETRIC && pad != DW_PAD_CAUSAL) return fail(DW_ERR_INVALID_ARG, "%s: unknown pad mode %d", fn, (int)pad);
    if (dtype != DW_F32 && dtype != DW_BF16) return fail(DW_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
    if (B == 0 || T == 0 || C == 0) return ok();
    if (!extents_ok(B, T, C, K)) return too_large(fn);
    if (!x || !w || !y) return fail(DW_ERR_INVALID_ARG, "%s: x, w and y must not be NULL", fn);
    if (x == y) return fail(DW_ERR_INVALID_ARG, "%s: y must not alias x", fn);
    const int es = dtype == DW_BF16 ? 2 : 4;
    const void* ptrs[4] = {x, w, bias, y};
    const int vec = dw::pick_vec(C, es, ptrs, 4, dtype == DW_BF16 ? DW1D_BF16_VEC : 4);
    if (!dw::dwconv1d_fwd_fits(B, T, C, K, es, vec))
        return fail(DW_ERR_UNSUPPORTED, "%s: sizes too large for one launch (B=%lld T=%lld C=%lld K=%lld)", fn, (long long)B, (long long)T, (long long)C, (long long)K);
    const int64_t pL = pad == DW_PAD_CAUSAL ? K - 1 : (K - 1) / 2;
    return from_hip(dw::launch_dwconv1d_fwd(x, w, bias, lengths, y, B, T, C, K, pL, dtype == DW_BF16, vec,
                                            (hipStream_t)stream), fn);
}

dw_status dwconv1d_stream_fwd(const void* x, const void* w, const void* bias, const int32_t* lengths,
                              const void* cache_in, void* y, void* cache_out, int64_t B, int64_t Tc, int64_t C,
                              int64_t K, dw_dtype dtype, void* stream) {
    const char* fn = "dwconv1d_stream_fwd";
    if (B < 0 || Tc < 0 || C < 0) return fail(DW_ERR_INVALID_ARG, "%s: negative size", fn);
    if (K < 1) return fail(DW_ERR_INVALID_ARG, "%s: kernel width K=%lld must be >= 1", fn, (long long)K);
    if (dtype != DW_F32 && dtype != DW_BF16) return fail(DW_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
    if (B == 0 || C == 0) return ok();
    if (!extents_ok(B, Tc, C, K)) return too_large(fn);
    const bool has_cache = K > 1;
    if ((!x && Tc > 0) || !w || (!y && Tc > 0) || (has_cache && (!cache_in || !cache_out)))
        return fail(DW_ERR_INVALID_ARG, "%s: x, w, y and the caches must not be NULL (unless empty)", fn);
    if (has_cache && cache_in == (const void*)cache_out)
        return fail(DW_ERR_INVALID_ARG, "%s: cache_out must be a different buffer from cache_in", fn);
    if (Tc > 0 && (x == (const void*)y || (has_cache && (y == cache_in || y == (const void*)cache_out))))
        return fail(DW_ERR_INVALID_ARG, "%s: y must not alias x or a cache", fn);
    const int es = dtype == DW_BF16 ? 2 : 4;
    const void* ptrs[6] = {x, w, bias, y, cache_in, cache_out};
    const int vec = dw::pick_vec(C, es, ptrs, 6, dw::dwconv1d_stream_max_vec(K, dtype == DW_BF16));
    if (!dw::dwconv1d_stream_fits(B, Tc, C, K, es, vec)) return too_large(fn);
    return from_hip(dw::launch_dwconv1d_stream(x, w, bias, lengths, cache_in, y, cache_out, B, Tc, C, K,
                                               dtype == DW_BF16, vec, (hipStream_t)stream), fn);
}

size_t dwconv1d_bwd_workspace_bytes(int64_t B, int64_t T, int64_t C, int64_t K) {
    if (B < 0 || T < 0 || C < 0 || !dw::dwconv1d_bwd_supported(K)) return 0;
    if (!extents_ok(B, T, C) || !dw::dwconv1d_bwd_fits(B, T, C, K, 2)) return 0;
    return dw::dwconv1d_bwd_workspace(B, T, C, K);
}

dw_status dwconv1d_bwd(const void* x, const void* w, const int32_t* lengths, const void* dy, void* dx, float* dw_,
                       float* db, void* workspace, size_t workspace_bytes, int64_t B, int64_t T, int64_t C,
                       int64_t K, dw_pad pad, dw_dtype dtype, void* stream) {
    const char* fn = "dwconv1d_bwd";
    if (B < 0 || T < 0 || C < 0) return fail(DW_ERR_INVALID_ARG, "%s: negative size", fn);
    if (K < 1) return fail(DW_ERR_INVALID_ARG, "%s: kernel width K=%lld must be >= 1", fn, (long long)K);
    if (pad != DW_PAD_SYMMETRIC && pad != DW_PAD_CAUSAL) return fail(DW_ERR_INVALID_ARG, "%s: unknown pad mode %d", fn, (int)pad);
    if (dtype != DW_F32 && dtype != DW_BF16) return fail(DW_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
    if (!dw::dwconv1d_bwd_supported(K))
        return fail(DW_ERR_UNSUPPORTED, "%s: kernel width K=%lld has no backward kernel (3, 4, 5, 7, 9, 15, 31)", fn, (long long)K);
    const bool want_wb = dw_ || db;
    if (!dx && !want_wb) return ok();
    if (C == 0) return ok();
    if ((!x && nonempty(B, T)) || (!dy && nonempty(B, T)) || !w)
        return fail(DW_ERR_INVALID_ARG, "%s: x, w and dy must not be NULL (unless empty)", fn);
    if (dx && (dx == x || dx == dy)) return fail(DW_ERR_INVALID_ARG, "%s: dx must not alias x or dy", fn);
    const int es = dtype == DW_BF16 ? 2 : 4;
    if (!extents_ok(B, T, C) || !dw::dwconv1d_bwd_fits(B, T, C, K, es)) return too_large(fn);
    if (want_wb) {
        const size_t need = dw::dwconv1d_bwd_workspace(B, T, C, K);
        if (!workspace || workspace_bytes < need)
            return fail(DW_ERR_WORKSPACE, "%s: workspace of %zu bytes given, %zu needed", fn, workspace ? workspace_bytes : (size_t)0, need);
    }
    const void* ptrs[4] = {x, w, dy, dx};
    const int vec = dw::pick_vec(C, es, ptrs, 4, dw::dwconv1d_bwd_max_vec(K, dtype == DW_BF16));
    return from_hip(dw::launch_dwconv1d_bwd(x, w, lengths, dy, dx, dw_, db, workspace, B, T, C, K,
                                            pad == DW_PAD_CAUSAL, dtype == DW_BF16, vec, (hipStream_t)stream), fn);
}

dw_status dwsub_fused_fwd_ex(const void* x, const void* w0, const void* b0, const void* w1, const void* b1,
                             const int32_t* lengths, void* y, int64_t B, int64_t T, int64_t F, int64_t C,
                             dw_pad pad, dw_dtype dtype, void* stream) {
    const char* fn = "dwsub_fused_fwd";
    if (B < 0 || T < 0 || F < 0 || C < 0) return fail(DW_ERR_INVALID_ARG, "%s: negative size", fn);
    const dw_status ps = check_pad(fn, pad);
    if (ps != DW_OK) return ps;
    if (dtype != DW_F32 && dtype != DW_BF16) return fail(DW_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
    const bool causal = pad == DW_PAD_CAUSAL;
    if (!extents_ok(B, T, F, C)) return too_large(fn);
    const dw::FrontDims fd = dw::front_dims(T, F, causal ? 1 : 0);
    if (B == 0 || fd.T2 == 0 || fd.F2 == 0 || C == 0) return ok();
    if ((!x && nonempty(T, F)) || !w0 || !w1 || !y)
        return fail(DW_ERR_INVALID_ARG, "%s: x, w0, w1 and y must not be NULL", fn);
    if (x == (const void*)y) return fail(DW_ERR_INVALID_ARG, "%s: y must not alias x", fn);
    const int es = dtype == DW_BF16 ? 2 : 4;
    if (!dw::dwsub_fused_fwd_fits(B, T, F, C, causal, es)) return too_large(fn);
    return from_hip(dw::launch_dwsub_fused_fwd(x, w0, b0, w1, b1, lengths, y, B, T, F, C, causal, dtype == DW_BF16,
                                               (hipStream_t)stream), fn);
}

dw_status dwsub_fused_fwd(const float* x, const float* w0, const float* b0, const float* w1, const float* b1,
                          const int32_t* lengths, float* y, int64_t B, int64_t T, int64_t F, int64_t C,
                          void* stream) {
    return dwsub_fused_fwd_ex(x, w0, b0, w1, b1, lengths, y, B, T, F, C, DW_PAD_SYMMETRIC, DW_F32, stream);
}

size_t dwsub_fused_bwd_workspace_bytes_ex(int64_t B, int64_t T, int64_t F, int64_t C, dw_pad pad) {
    if (B < 0 || T < 0 || F < 0 || C < 0 || (pad != DW_PAD_SYMMETRIC && pad != DW_PAD_CAUSAL)) return 0;
    if (!extents_ok(B, T, F, C) || !dw::dwsub_fused_bwd_fits(B, T, F, C, pad == DW_PAD_CAUSAL, 2)) return 0;
    return dw::dwsub_fused_bwd_workspace(B, T, F, C, pad == DW_PAD_CAUSAL);
}

size_t dwsub_fused_bwd_workspace_bytes(int64_t B, int64_t T, int64_t F, int64_t C) {
    return dwsub_fused_bwd_workspace_bytes_ex(B, T, F, C, DW_PAD_SYMMETRIC);
}

dw_status dwsub_fused_bwd_ex(const void* x, const void* w0, const void* b0, const void* w1, const int32_t* lengths,
                             const void* dy, float* dw0, float* db0, float* dw1, float* db1, void* workspace,
                             size_t workspace_bytes, int64_t B, int64_t T, int64_t F, int64_t C, dw_pad pad,
                             dw_dtype dtype, void* stream) {
    const char* fn = "dwsub_fused_bwd";
    if (B < 0 || T < 0 || F < 0 || C < 0) return fail(DW_ERR_INVALID_ARG, "%s: negative size", fn);
    const dw_status ps = check_pad(fn, pad);
    if (ps != DW_OK) return ps;
    if (dtype != DW_F32 && dtype != DW_BF16) return fail(DW_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
    const bool causal = pad == DW_PAD_CAUSAL;
    if (!dw0 && !db0 && !dw1 && !db1) return ok();
    if (C == 0) return ok();
    if (!extents_ok(B, T, F, C)) return too_large(fn);
    const dw::FrontDims fd = dw::front_dims(T, F, causal ? 1 : 0);
    if ((!x && nonempty(B, T, F)) || (!dy && nonempty(B, fd.T2, fd.F2, C)) || !w0 || !w1)
        return fail(DW_ERR_INVALID_ARG, "%s: x, w0, w1 and dy must not be NULL (unless empty)", fn);
    const int es = dtype == DW_BF16 ? 2 : 4;
    if (!dw::dwsub_fused_bwd_fits(B, T, F, C, causal, es)) return too_large(fn);
    const size_t need = dw::dwsub_fused_bwd_workspace(B, T, F, C, causal);
    if (!workspace || workspace_bytes < need)
        return fail(DW_ERR_WORKSPACE, "%s: workspace of %zu bytes given, %zu needed", fn,
                    workspace ? workspace_bytes : (size_t)0, need);
    return from_hip(dw::launch_dwsub_fused_bwd(x, w0, b0, w1, lengths, dy, dw0, db0, dw1, db1, workspace, B, T, F, C,
                                               causal, dtype == DW_BF16, (hipStream_t)stream), fn);
}

dw_status dwsub_fused_bwd(const float* x, const float* w0, const float* b0, const float* w1,
                          const int32_t* lengths, const float* dy, float* dw0, float* db0, float* dw1, float* db1,
                          void* workspace, size_t workspace_bytes, int64_t B, int64_t T, int64_t F, int64_t C,
                          void* stream) {
    return dwsub_fused_bwd_ex(x, w0, b0, w1, lengths, dy, dw0, db0, dw1, db1, workspace, workspace_bytes, B, T, F, C,
                              DW_PAD_SYMMETRIC, DW_F32, stream);
}

dw_status dwconv2d_fwd_ex(const void* x, const void* w, const void* bias, const int32_t* lengths, void* y,
                          int64_t B, int64_t T, int64_t F, int64_t C, int64_t KH, int64_t KW, int64_t stride,
                          int64_t pad_t0, int64_t pad_t1, int64_t pad_f0, int64_t pad_f1, dw_dtype dtype,
                          void* stream) {
    const char* fn = "dwconv2d_fwd";
    if (B < 0 || T < 0 || F < 0 || C < 0) return fail(DW_ERR_INVALID_ARG, "%s: negative size", fn);
    if (dtype != DW_F32 && dtype != DW_BF16) return fail(DW_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
    const dw_status gs = check_geometry_2d(fn, KH, KW, stride, pad_t0, pad_t1, pad_f0, pad_f1);
    if (gs != DW_OK) return gs;
    if (!extents_ok(B, T, F, C)) return too_large(fn);
    const dw::Conv2dGeom g = dw::conv2d_geom(T, F, C, pad_t0, pad_t1, pad_f0, pad_f1);
    if (B == 0 || g.To == 0 || g.Fo == 0 || C == 0) return ok();
    if ((!x && nonempty(T, F)) || !w || !y) return fail(DW_ERR_INVALID_ARG, "%s: x, w and y must not be NULL", fn);
    if (x == (const void*)y) return fail(DW_ERR_INVALID_ARG, "%s: y must not alias x", fn);
    const int es = dtype == DW_BF16 ? 2 : 4;
    const void* ptrs[4] = {x, w, bias, y};
    const int vec = dw::pick_vec(C, es, ptrs, 4, dtype == DW_BF16 ? 8 : 4);
    if (!dw::dwconv2d_fits(B, g, es)) return too_large(fn);
    return from_hip(dw::launch_dwconv2d_fwd(x, w, bias, lengths, y, B, g, dtype == DW_BF16, vec,
                                            (hipStream_t)stream), fn);
}

dw_status dwconv2d_fwd(const float* x, const float* w, const float* bias, const int32_t* lengths, float* y,
                       int64_t B, int64_t T, int64_t F, int64_t C, int64_t KH, int64_t KW, int64_t stride,
                       int64_t pad, void* stream) {
    return dwconv2d_fwd_ex(x, w, bias, lengths, y, B, T, F, C, KH, KW, stride, pad, pad, pad, pad, DW_F32, stream);
}

size_t dwconv2d_bwd_workspace_bytes_ex(int64_t B, int64_t T, int64_t F, int64_t C, int64_t KH, int64_t KW,
                                       int64_t stride, int64_t pad_t0, int64_t pad_t1, int64_t pad_f0,
                                       int64_t pad_f1) {
    if (B < 0 || T < 0 || F < 0 || C < 0 || !geometry_ok_2d(KH, KW, stride, pad_t0, pad_t1, pad_f0, pad_f1)) return 0;
    if (!extents_ok(B, T, F, C)) return 0;
    const dw::Conv2dGeom g = dw::conv2d_geom(T, F, C, pad_t0, pad_t1, pad_f0, pad_f1);
    if (!dw::dwconv2d_fits(B, g, 2)) return 0;
    return dw::dwconv2d_bwd_workspace(B, g);
}

size_t dwconv2d_bwd_workspace_bytes(int64_t B, int64_t T, int64_t F, int64_t C, int64_t KH, int64_t KW,
                                    int64_t stride, int64_t pad) {
    return dwconv2d_bwd_workspace_bytes_ex(B, T, F, C, KH, KW, stride, pad, pad, pad, pad);
}

// The conv2d backward's checks and launch.  With use_scratch, the fp64
// partials go to the library's own per-device scratch array (allocation-free
// entry point) instead of the caller's workspace.
static dw_status dwconv2d_bwd_impl(const char* fn, const void* x, const void* w, const int32_t* lengths,
                                   const void* dy, void* dx, float* dw_, float* db, void* workspace,
                                   size_t workspace_bytes, bool use_scratch, int64_t B, int64_t T, int64_t F,
                                   int64_t C, int64_t KH, int64_t KW, int64_t stride, int64_t pad_t0,
                                   int64_t pad_t1, int64_t pad_f0, int64_t pad_f1, dw_dtype dtype, void* stream) {
    if (B < 0 || T < 0 || F < 0 || C < 0) return fail(DW_ERR_INVALID_ARG, "%s: negative size", fn);
    if (dtype != DW_F32 && dtype != DW_BF16) return fail(DW_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
    const dw_status gs = check_geometry_2d(fn, KH, KW, stride, pad_t0, pad_t1, pad_f0, pad_f1);
    if (gs != DW_OK) return gs;
    if (!extents_ok(B, T, F, C)) return too_large(fn);
    const dw::Conv2dGeom g = dw::conv2d_geom(T, F, C, pad_t0, pad_t1, pad_f0, pad_f1);
    if ((!x && nonempty(B, T, F, C)) || (!dy && nonempty(B, g.To, g.Fo, C)) || (!w && C > 0))
        return fail(DW_ERR_INVALID_ARG, "%s: x, w and dy must not be NULL (unless empty)", fn);
    if (dx && (dx == x || dx == dy)) return fail(DW_ERR_INVALID_ARG, "%s: dx must not alias x or dy", fn);
    const bool want_wb = dw_ || db;
    const int es = dtype == DW_BF16 ? 2 : 4;
    if (!dw::dwconv2d_fits(B, g, es)) return too_large(fn);
    if (want_wb) {
        const size_t need = dw::dwconv2d_bwd_workspace(B, g);
        if (use_scratch) {
            if (need > dw::kScratchBytes)
                return fail(DW_ERR_UNSUPPORTED, "%s: dw and db need %zu bytes of scratch, more than the %zu bytes "
                            "this allocation-free entry point holds (C = %lld; at most about 800 channels fit)", fn,
                            need, dw::kScratchBytes, (long long)C);
        } else if (!workspace || workspace_bytes < need) {
            return fail(DW_ERR_WORKSPACE, "%s: workspace of %zu bytes given, %zu needed", fn,
                        workspace ? workspace_bytes : (size_t)0, need);
        }
    }
    if (!dx && !want_wb) return ok();
    if (C == 0) return ok();
    if (use_scratch && want_wb) {
        const hipError_t e = dw::scratch_on_current_device(&workspace);
        if (e != hipSuccess)
            return fail(DW_ERR_HIP, "%s: the device address of the library's scratch array: %s", fn,
                        hipGetErrorString(e));
    }
    // An empty batch or item still defines dw = 0 and db = 0; the launcher
    // writes those zeros when there is nothing to reduce.
    const void* ptrs[4] = {x, w, dy, dx};
    const int vec = dw::pick_vec(C, es, ptrs, 4, dtype == DW_BF16 ? 8 : 4);
    return from_hip(dw::launch_dwconv2d_bwd(x, w, lengths, dy, dx, dw_, db, workspace, B, g, dtype == DW_BF16, vec,
                                            (hipStream_t)stream), fn);
}

dw_status dwconv2d_bwd_ex(const void* x, const void* w, const int32_t* lengths, const void* dy, void* dx,
                          float* dw_, float* db, void* workspace, size_t workspace_bytes, int64_t B, int64_t T,
                          int64_t F, int64_t C, int64_t KH, int64_t KW, int64_t stride, int64_t pad_t0,
                          int64_t pad_t1, int64_t pad_f0, int64_t pad_f1, dw_dtype dtype, void* stream) {
    return dwconv2d_bwd_impl("dwconv2d_bwd", x, w, lengths, dy, dx, dw_, db, workspace, workspace_bytes, false, B, T,
                             F, C, KH, KW, stride, pad_t0, pad_t1, pad_f0, pad_f1, dtype, stream);
}

dw_status dwconv2d_bwd_noalloc(const void* x, const void* w, const int32_t* lengths, const void* dy, void* dx,
                               float* dw_, float* db, int64_t B, int64_t T, int64_t F, int64_t C, int64_t KH,
                               int64_t KW, int64_t stride, int64_t pad_t0, int64_t pad_t1, int64_t pad_f0,
                               int64_t pad_f1, dw_dtype dtype, void* stream) {
    return dwconv2d_bwd_impl("dwconv2d_bwd_noalloc", x, w, lengths, dy, dx, dw_, db, nullptr, 0, true, B, T, F, C,
                             KH, KW, stride, pad_t0, pad_t1, pad_f0, pad_f1, dtype, stream);
}

dw_status dwconv2d_bwd(const float* x, const float* w, const int32_t* lengths, const float* dy, float* dx,
                       float* dw_, float* db, void* workspace, size_t workspace_bytes, int64_t B, int64_t T,
                       int64_t F, int64_t C, int64_t KH, int64_t KW, int64_t stride, int64_t pad,
                       void* stream) {
    return dwconv2d_bwd_ex(x, w, lengths, dy, dx, dw_, db, workspace, workspace_bytes, B, T, F, C, KH, KW, stride,
                           pad, pad, pad, pad, DW_F32, stream);
}

}  // extern "C"
