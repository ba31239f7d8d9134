// Host-side launchers of the gfx950 kernels.  The C ABI in capi.hip
// validates every argument and then calls exactly one of these; they assume
// valid, non-empty sizes and only compute launch geometry and enqueue work.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <initializer_list>

namespace dw {

// Every extent the C ABI passes to these launchers (B, T, F, C, K) is below
// this; the *_fits checks rely on it to add extents without overflow.
constexpr int64_t kMaxExtent = (int64_t)1 << 31;

// Whether the product of the non-negative factors is below limit, formed
// without overflow: the running product stays below limit <= 2^63 before
// each multiplication, so it never exceeds 2^126 in 128 bits.
inline bool product_below(int64_t limit, std::initializer_list<int64_t> factors) {
    for (int64_t f : factors)
        if (f == 0) return 0 < limit;
    __int128 p = 1;
    for (int64_t f : factors) {
        p *= f;
        if (p >= limit) return false;
    }
    return true;
}

// Outputs of a partial reduction: output s receives rows
// [first[s], first[s] + count[s]) of the K rows, as [count[s]][C] floats.
struct RowOutputs {
    float* p[4];
    int32_t first[4];
    int32_t count[4];
    int32_t n;
};


// Largest vector width V <= max_vec (channels per access, a power of two)
// such that C is a multiple of V and every pointer given is aligned to V
// elements.
int pick_vec(int64_t C, int elem_bytes, const void* const* ptrs, int nptrs, int max_vec);

// Whether launch_dwconv1d_fwd can address these sizes (32-bit per-item byte
// offsets, 32-bit grid).
bool dwconv1d_fwd_fits(int64_t B, int64_t T, int64_t C, int64_t K, int elem_bytes, int vec);

hipError_t launch_dwconv1d_fwd(const void* x, const void* w, const void* bias, const int32_t* lengths,
                               void* y, int64_t B, int64_t T, int64_t C, int64_t K, int64_t pad_left,
                               bool bf16, int vec, hipStream_t stream);

// Streaming 1-D conv (causal over a K-1 frame cache and the chunk).
bool dwconv1d_stream_fits(int64_t B, int64_t Tc, int64_t C, int64_t K, int elem_bytes, int vec);
int dwconv1d_stream_max_vec(int64_t K, bool bf16);
hipError_t launch_dwconv1d_stream(const void* x, const void* w, const void* bias, const int32_t* lengths,
                                  const void* cache_in, void* y, void* cache_out, int64_t B, int64_t Tc, int64_t C,
                                  int64_t K, bool bf16, int vec, hipStream_t stream);

// 1-D backward: the widths with a kernel, the widest vector each takes, and
// the workspace (fp64 partials) it needs.
bool dwconv1d_bwd_supported(int64_t K);
int dwconv1d_bwd_max_vec(int64_t K, bool bf16);
bool dwconv1d_bwd_fits(int64_t B, int64_t T, int64_t C, int64_t K, int elem_bytes);
size_t dwconv1d_bwd_workspace(int64_t B, int64_t T, int64_t C, int64_t K);
hipError_t launch_dwconv1d_bwd(const void* x, const void* w, const int32_t* lengths, const void* dy, void* dx,
                               float* dw, float* db, void* workspace, int64_t B, int64_t T, int64_t C, int64_t K,
                               bool causal, bool bf16, int vec, hipStream_t stream);

// Sizes of the front's two stages for pad shift d (0 symmetric, 1 causal).
struct FrontDims {
    int64_t T1, F1, T2, F2;
};
FrontDims front_dims(int64_t T, int64_t F, int d);

// The fused front; causal selects its causal padding (2 before, 1 after).
bool dwsub_fused_fwd_fits(int64_t B, int64_t T, int64_t F, int64_t C, bool causal, int elem_bytes);

hipError_t launch_dwsub_fused_fwd(const void* x, const void* w0, const void* b0, const void* w1, const void* b1,
                                  const int32_t* lengths, void* y, int64_t B, int64_t T, int64_t F, int64_t C,
                                  bool causal, bool bf16, hipStream_t stream);

bool dwsub_fused_bwd_fits(int64_t B, int64_t T, int64_t F, int64_t C, bool causal, int elem_bytes);

size_t dwsub_fused_bwd_workspace(int64_t B, int64_t T, int64_t F, int64_t C, bool causal);

hipError_t launch_dwsub_fused_bwd(const void* x, const void* w0, const void* b0, const void* w1,
                                  const int32_t* lengths, const void* dy, float* dw0, float* db0, float* dw1,
                                  float* db1, void* workspace, int64_t B, int64_t T, int64_t F, int64_t C,
                                  bool causal, bool bf16, hipStream_t stream);

// A 3x3, stride-2 depthwise conv2d with pt0 / pt1 zero rows before / after
// the input in time and pf0 / pf1 columns in frequency, and its output extent.
struct Conv2dGeom {
    int64_t T, F, C;
    int64_t pt0, pt1, pf0, pf1;
    int64_t To, Fo;
};
Conv2dGeom conv2d_geom(int64_t T, int64_t F, int64_t C, int64_t pt0, int64_t pt1, int64_t pf0, int64_t pf1);

// The paddings with a kernel: 1 or 2 before, 0 to 2 after, on each axis.
bool dwconv2d_pads_supported(int64_t pt0, int64_t pt1, int64_t pf0, int64_t pf1);

bool dwconv2d_fits(int64_t B, const Conv2dGeom& g, int elem_bytes);

hipError_t launch_dwconv2d_fwd(const void* x, const void* w, const void* bias, const int32_t* lengths, void* y,
                               int64_t B, const Conv2dGeom& g, bool bf16, int vec, hipStream_t stream);

size_t dwconv2d_bwd_workspace(int64_t B, const Conv2dGeom& g);

// Number of fp64 [K][C] rows of scratch launch_partial_reduce needs after the
// P partial rows (at least one).
int64_t partial_reduce_chunks(int64_t P);

// Sum a [P][K][C] fp64 partial matrix over P in a fixed order; chunk_sum is
// scratch of max(1, partial_reduce_chunks(P)) rows of K*C doubles.
hipError_t launch_partial_reduce(const double* partial, int64_t P, int32_t K, int64_t C, double* chunk_sum,
                                 RowOutputs out, hipStream_t stream);

hipError_t launch_dwconv2d_bwd(const void* x, const void* w, const int32_t* lengths, const void* dy, void* dx,
                               float* dw, float* db, void* workspace, int64_t B, const Conv2dGeom& g, bool bf16,
                               int vec, hipStream_t stream);

}  // namespace dw
