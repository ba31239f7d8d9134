// The depthwise-striding subsampler front, fused, for gfx950 (NeMo PR
// #16114, "What does this PR do": mel [B,T,F,1] -> conv0 3x3 stride 2 ->
// ReLU -> masking -> depthwise 3x3 stride 2 conv, with no intermediate
// tensor in memory).
//
//   h[t1,f1,c] = max(0, sum_{i,j} x[2t1+i-1, 2f1+j-1] w0[i,j,c] + b0[c]), zero for t1 >= ceil(len/2)
//   y[t2,f2,c] = sum_{i,j} h[2t2+i-1, 2f2+j-1, c] w1[i,j,c] + b1[c]
//
// Mapping.  The mel input has one channel, so its values are the same for
// every output channel: a workgroup stages the mel patch its outputs need in
// LDS (zero-padded), and its threads read it back as broadcasts.  Each thread
// owns one output channel c of a tile of TY output rows x FC output columns.
// h never leaves the thread: channel c of y needs only channel c of h.  The
// thread walks its columns left to right; at output column f2 it computes the
// 2*TY+1 h rows it needs at h columns 2f2 and 2f2+1 and carries column 2f2+1
// to the next step (as its column 2f2-1).  h rows past the item's time mask,
// and h positions in the padding, are zero; a tile whose h rows are all
// masked stores the output bias without computing.  Only the one h row and
// column shared with neighbouring tiles is computed twice.
//
// Arithmetic is IEEE fp32 FMA throughout, the bias seeding each sum.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace dw {

#ifndef DWSUB_ROWS
#define DWSUB_ROWS 4
#endif
#ifndef DWSUB_COLS
#define DWSUB_COLS 5
#endif
constexpr int kSubBlock = 256;       // channels per workgroup
constexpr int kSubRows = DWSUB_ROWS;  // output rows per thread
constexpr int kSubCols = DWSUB_COLS;  // output columns per thread
// Staged mel patch: rows 4*t0-3 .. 4*t0+4*TY-1, columns 4*f0-5 .. 4*f0+4*FC-1
// (column 4*f0-5 sits at LDS column 0 so that every step reads an aligned
// 16-byte group).
constexpr int kPatchRows = 4 * kSubRows + 3;
constexpr int kPatchCols = 4 * kSubCols + 8;

__global__ __launch_bounds__(kSubBlock) void dwsub_fused_fwd_kernel(
    const float* __restrict__ x, const float* __restrict__ w0, const float* __restrict__ b0,
    const float* __restrict__ w1, const float* __restrict__ b1, const int32_t* __restrict__ lengths,
    float* __restrict__ y, int32_t T, int32_t F, int32_t C, int32_t T1, int32_t F1, int32_t T2, int32_t F2,
    uint32_t n_rt, uint32_t n_ft, uint32_t n_cblk) {
    __shared__ __align__(16) float patch[kPatchRows][kPatchCols];

    // Block -> (item, row tile, column tile, channel block); all uniform.
    const uint32_t blk = xcd_contiguous_block(blockIdx.x, gridDim.x);
    const uint32_t cblk = blk % n_cblk;
    const uint32_t rest = blk / n_cblk;
    const uint32_t ft = rest % n_ft;
    const uint32_t rest2 = rest / n_ft;
    const uint32_t rt = rest2 % n_rt;
    const uint32_t b = rest2 / n_rt;
    const int32_t t0 = (int32_t)rt * kSubRows;  // first output row
    const int32_t f0 = (int32_t)ft * kSubCols;  // first output column
    const int32_t len = (int32_t)item_length(lengths, b, T);
    const int32_t L1 = (len + 1) / 2;

    // Stage the zero-padded mel patch.  The input is not length-masked.
    const float* xb = x + (int64_t)b * T * F;
    for (int i = threadIdx.x; i < kPatchRows * kPatchCols; i += kSubBlock) {
        const int r = i / kPatchCols, q = i % kPatchCols;
        const int32_t t = 4 * t0 - 3 + r, f = 4 * f0 - 5 + q;
        patch[r][q] = (t >= 0 && t < T && f >= 0 && f < F) ? xb[(int64_t)t * F + f] : 0.0f;
    }
    __syncthreads();

    const int32_t c = (int32_t)cblk * kSubBlock + (int32_t)threadIdx.x;
    if (c >= C) return;

    float wa[9], wb[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) {
        wa[k] = w0[(int64_t)k * C + c];
        wb[k] = w1[(int64_t)k * C + c];
    }
    const float ba = b0 ? b0[c] : 0.0f;
    const float bb = b1 ? b1[c] : 0.0f;

    // h rows 2*t0-1+l, l = 0..2*TY, read mel patch rows 2l .. 2l+2.
    // h row validity: inside [0, T1) and before the time mask.
    bool hrow_ok[2 * kSubRows + 1];
    bool any_ok = false;
#pragma unroll
    for (int l = 0; l < 2 * kSubRows + 1; ++l) {
        const int32_t r = 2 * t0 - 1 + l;
        hrow_ok[l] = r >= 0 && r < T1 && r < L1;
        any_ok |= hrow_ok[l];
    }

    const int32_t ncols = min(kSubCols, F2 - f0);
    const uint32_t yrow = (uint32_t)F2 * C * 4;
    const rsrc_t yr = make_rsrc(y + (int64_t)b * T2 * F2 * C, (uint32_t)T2 * yrow);
    if (!any_ok) {
        // Every h row this tile reads is masked or padding: y is the bias.
        for (int s = 0; s < ncols; ++s)
#pragma unroll
            for (int i = 0; i < kSubRows; ++i)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(bb), yr,
                                                      (uint32_t)(t0 + i) * yrow + ((uint32_t)(f0 + s) * C + c) * 4, 0,
                                                      kNonTemporal);
        return;
    }

    // conv0 + bias + ReLU at h row l, for the h column whose three mel
    // columns start at patch column q; zero where the row is masked.  The
    // sum is computed for every row and then selected, so the loads and FMAs
    // of all rows can be scheduled together.
    auto conv0 = [&](int l, int q) -> float {
        float a = ba;
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int j = 0; j < 3; ++j) a = __builtin_fmaf(patch[2 * l + i][q + j], wa[3 * i + j], a);
        return hrow_ok[l] ? fmaxf(a, 0.0f) : 0.0f;
    };

    // Carried h column 2*f0-1 (zero at the left edge).
    float hc[2 * kSubRows + 1];
#pragma unroll
    for (int l = 0; l < 2 * kSubRows + 1; ++l) hc[l] = f0 > 0 ? conv0(l, 2) : 0.0f;

    // One output column: h columns 2f2 and 2f2+1 for every h row, then the
    // depthwise taps.  h column 2f2+1 lies in the padding only at the last
    // output column of an odd-width h, which is peeled off the loop so that
    // the loop body has no condition around its LDS reads.
    auto step = [&](int s, auto odd_valid) {
        const int32_t f2 = f0 + s;
        float he[2 * kSubRows + 1], ho[2 * kSubRows + 1];
#pragma unroll
        for (int l = 0; l < 2 * kSubRows + 1; ++l) {
            he[l] = conv0(l, 4 * s + 4);
            ho[l] = decltype(odd_valid)::value ? conv0(l, 4 * s + 6) : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < kSubRows; ++i) {
            float a = bb;
#pragma unroll
            for (int r = 0; r < 3; ++r) {
                a = __builtin_fmaf(hc[2 * i + r], wb[3 * r + 0], a);
                a = __builtin_fmaf(he[2 * i + r], wb[3 * r + 1], a);
                a = __builtin_fmaf(ho[2 * i + r], wb[3 * r + 2], a);
            }
            const uint32_t off = (uint32_t)(t0 + i) * yrow + ((uint32_t)f2 * C + c) * 4;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(a), yr, off, 0, kNonTemporal);
        }
#pragma unroll
        for (int l = 0; l < 2 * kSubRows + 1; ++l) hc[l] = ho[l];
    };
    const bool last_odd_pad = 2 * (f0 + ncols - 1) + 1 >= F1;
    const int full = last_odd_pad ? ncols - 1 : ncols;
    for (int s = 0; s < full; ++s) step(s, std::true_type{});
    if (last_odd_pad) step(full, std::false_type{});
}

bool dwsub_fused_fwd_fits(int64_t B, int64_t T, int64_t F, int64_t C) {
    const int64_t T2 = ((T + 1) / 2 + 1) / 2, F2 = ((F + 1) / 2 + 1) / 2;
    if ((T2 + kSubRows) * F2 * C * 4 >= ((int64_t)1 << 31)) return false;
    if (T >= ((int64_t)1 << 28) || F >= ((int64_t)1 << 28)) return false;
    const int64_t blocks = B * ((T2 + kSubRows - 1) / kSubRows) * ((F2 + kSubCols - 1) / kSubCols) *
                           ((C + kSubBlock - 1) / kSubBlock);
    return blocks < ((int64_t)1 << 31);
}

hipError_t launch_dwsub_fused_fwd(const float* x, const float* w0, const float* b0, const float* w1,
                                  const float* b1, const int32_t* lengths, float* y,
                                  int64_t B, int64_t T, int64_t F, int64_t C, hipStream_t st) {
    const int64_t T1 = (T + 1) / 2, F1 = (F + 1) / 2, T2 = (T1 + 1) / 2, F2 = (F1 + 1) / 2;
    const uint32_t n_rt = (uint32_t)((T2 + kSubRows - 1) / kSubRows);
    const uint32_t n_ft = (uint32_t)((F2 + kSubCols - 1) / kSubCols);
    const uint32_t n_cblk = (uint32_t)((C + kSubBlock - 1) / kSubBlock);
    const uint64_t blocks = (uint64_t)B * n_rt * n_ft * n_cblk;
    hipLaunchKernelGGL(dwsub_fused_fwd_kernel, dim3((uint32_t)blocks), dim3(kSubBlock), 0, st, x, w0, b0, w1, b1,
                       lengths, y, (int32_t)T, (int32_t)F, (int32_t)C, (int32_t)T1, (int32_t)F1, (int32_t)T2,
                       (int32_t)F2, n_rt, n_ft, n_cblk);
    return hipGetLastError();
}

}  // namespace dw
