// The depthwise-striding subsampler front, fused, for gfx950 (NeMo PR
// #16114, "What does this PR do": mel [B,T,F,1] -> conv0 3x3 stride 2 ->
// ReLU -> masking -> depthwise 3x3 stride 2 conv, with no intermediate
// tensor in memory).
//
//   h[t1,f1,c] = max(0, sum_{i,j} x[2t1+i-pl, 2f1+j-pl] w0[i,j,c] + b0[c]), zero for t1 >= L1
//   y[t2,f2,c] = sum_{i,j} h[2t2+i-pl, 2f2+j-pl, c] w1[i,j,c] + b1[c]
//
// Both convolutions pad each axis with pl zeros before and one after: pl = 1
// is the symmetric front, pl = 2 its causal mode (the page's extra padding
// layer: kernel - 1 before, stride - 1 after).  With d = pl - 1,
// T1 = floor((T - 1 + d)/2) + 1, likewise F1, T2, F2, and
// L1 = floor((len - 1 + d)/2) + 1 (0 for an empty item).  The kernels take d
// as a shift: the mel patch a tile stages starts 3d rows and columns earlier,
// so every index into it is the same in both modes.
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
// Storage is fp32 or bf16 (the mel input, the parameters and y alike); bf16
// values are widened exactly, arithmetic is IEEE fp32 FMA throughout with the
// bias seeding each sum, and a bf16 y is rounded to nearest even.
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
FrontDims front_dims(int64_t T, int64_t F, int d) {
    auto half = [d](int64_t n) { return n > 0 ? (n - 1 + d) / 2 + 1 : (int64_t)d; };
    FrontDims r;
    r.T1 = half(T); r.F1 = half(F); r.T2 = half(r.T1); r.F2 = half(r.F1);
    return r;
}

constexpr int kSubBlock = 256;       // channels per workgroup
constexpr int kSubRows = DWSUB_ROWS;  // output rows per thread
constexpr int kSubCols = DWSUB_COLS;  // output columns per thread
// Staged mel patch: rows 4*t0-3-3d .. 4*t0+4*TY-1-3d, columns
// 4*f0-5-3d .. 4*f0+4*FC-1-3d (column 4*f0-5-3d sits at LDS column 0 so that
// every step reads an aligned 16-byte group).
constexpr int kPatchRows = 4 * kSubRows + 3;
constexpr int kPatchCols = 4 * kSubCols + 8;

template <typename S>
__global__ __launch_bounds__(kSubBlock) void dwsub_fused_fwd_kernel(
    const S* __restrict__ x, const S* __restrict__ w0, const S* __restrict__ b0,
    const S* __restrict__ w1, const S* __restrict__ b1, const int32_t* __restrict__ lengths,
    S* __restrict__ y, int32_t T, int32_t F, int32_t C, int32_t T1, int32_t F1, int32_t T2, int32_t F2,
    int32_t d, uint32_t n_rt, uint32_t n_ft, uint32_t n_cblk) {
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
    const int32_t L1 = len > 0 ? (len - 1 + d) / 2 + 1 : 0;

    // This thread's parameters (channel 0 stands in past C), loaded first so
    // that they arrive with the patch.
    const int32_t cp = min((int32_t)cblk * kSubBlock + (int32_t)threadIdx.x, C - 1);
    S wa_s[9], wb_s[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) {
        wa_s[k] = w0[(int64_t)k * C + cp];
        wb_s[k] = w1[(int64_t)k * C + cp];
    }
    const S ba_s = b0 ? b0[cp] : S(0), bb_s = b1 ? b1[cp] : S(0);

    // Stage the zero-padded mel patch.  The input is not length-masked.
    // Every thread issues its loads before it writes any of them, through a
    // buffer resource: a row above the input wraps to an offset past the
    // item, a row below lies past it, and a column outside [0, F) is sent
    // out of range, so each reads zero with no select on the loaded value.
    constexpr int kPatchN = kPatchRows * kPatchCols;
    constexpr int kPer = (kPatchN + kSubBlock - 1) / kSubBlock;
    constexpr uint32_t esx = sizeof(S);
    const rsrc_t xr = make_rsrc(x + (int64_t)b * T * F, (uint32_t)T * (uint32_t)F * esx);
    float pv[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int i = (int)threadIdx.x + u * kSubBlock;
        const int r = i / kPatchCols, q = i % kPatchCols;
        const int32_t t = 4 * t0 - 3 - 3 * d + r, f = 4 * f0 - 5 - 3 * d + q;
        const uint32_t off = i < kPatchN && f >= 0 && f < F ? (uint32_t)((t * F + f) * (int32_t)esx) : 0x80000000u;
        pv[u] = Buf<S, 1>::load(xr, off).v[0];
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int i = (int)threadIdx.x + u * kSubBlock;
        if (i < kPatchN) patch[i / kPatchCols][i % kPatchCols] = pv[u];
    }
    __syncthreads();

    const int32_t c = (int32_t)cblk * kSubBlock + (int32_t)threadIdx.x;
    if (c >= C) return;

    float wa[9], wb[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) {
        wa[k] = to_f32(wa_s[k]);
        wb[k] = to_f32(wb_s[k]);
    }
    const float ba = to_f32(ba_s), bb = to_f32(bb_s);
    constexpr uint32_t es = sizeof(S);

    // h rows 2*t0-1-d+l, l = 0..2*TY, read mel patch rows 2l .. 2l+2.
    // h row validity: inside [0, T1) and before the time mask.  hlim is the
    // upper clamp of the row's ReLU: +inf for a valid row, 0 for a masked
    // one, so that one median-of-three gives max(z, 0) or 0.
    float hlim[2 * kSubRows + 1];
    bool any_ok = false;
#pragma unroll
    for (int l = 0; l < 2 * kSubRows + 1; ++l) {
        const int32_t r = 2 * t0 - 1 - d + l;
        const bool ok = r >= 0 && r < T1 && r < L1;
        hlim[l] = ok ? __builtin_inff() : 0.0f;
        any_ok |= ok;
    }

    const int32_t ncols = min(kSubCols, F2 - f0);
    const uint32_t yrow = (uint32_t)F2 * C * es;
    const rsrc_t yr = make_rsrc(y + (int64_t)b * T2 * F2 * C, (uint32_t)T2 * yrow);
    auto store = [&](uint32_t off, float v) {
        Vf<1> o;
        o.v[0] = v;
        Buf<S, 1>::store(yr, off, o);
    };
    if (!any_ok) {
        // Every h row this tile reads is masked or padding: y is the bias.
        for (int s = 0; s < ncols; ++s)
#pragma unroll
            for (int i = 0; i < kSubRows; ++i)
                store((uint32_t)(t0 + i) * yrow + ((uint32_t)(f0 + s) * C + c) * es, bb);
        return;
    }

    // conv0 + bias + ReLU at h row l, for the h column whose three mel
    // columns start at patch column q; zero where the row is masked.  The
    // sum is computed for every row and then clamped, so the loads and FMAs
    // of all rows can be scheduled together.  med3(z, 0, hlim) is max(z, 0)
    // for a valid row and 0 for a masked one; a NaN z (from a NaN input)
    // gives 0 either way, as max(NaN, 0) does.
    auto conv0 = [&](int l, int q) -> float {
        float a = ba;
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int j = 0; j < 3; ++j) a = __builtin_fmaf(patch[2 * l + i][q + j], wa[3 * i + j], a);
        return __builtin_amdgcn_fmed3f(a, 0.0f, hlim[l]);
    };

    // Carried h column 2*f0-1-d (zero left of the first h column).  Two
    // carry arrays take turns, so the walk moves no registers between steps.
    float hc[2 * kSubRows + 1], hn[2 * kSubRows + 1];
#pragma unroll
    for (int l = 0; l < 2 * kSubRows + 1; ++l) hc[l] = 2 * f0 - 1 - d >= 0 ? conv0(l, 2) : 0.0f;

    // One output column: h columns 2f2-d and 2f2+1-d for every h row (the
    // odd one lands in `out`, the carry of the next column), then the
    // depthwise taps.  The first lies in the padding only at output column 0
    // of the causal mode, the second only at the last output column when it
    // passes F1; those steps are peeled off the loop so that the loop body
    // has no condition around its LDS reads.
    auto step = [&](int s, const float* in, float* out, auto odd_valid, auto even_valid) {
        const int32_t f2 = f0 + s;
        float he[2 * kSubRows + 1];
#pragma unroll
        for (int l = 0; l < 2 * kSubRows + 1; ++l) {
            he[l] = decltype(even_valid)::value ? conv0(l, 4 * s + 4) : 0.0f;
            out[l] = decltype(odd_valid)::value ? conv0(l, 4 * s + 6) : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < kSubRows; ++i) {
            float a = bb;
#pragma unroll
            for (int r = 0; r < 3; ++r) {
                a = __builtin_fmaf(in[2 * i + r], wb[3 * r + 0], a);
                a = __builtin_fmaf(he[2 * i + r], wb[3 * r + 1], a);
                a = __builtin_fmaf(out[2 * i + r], wb[3 * r + 2], a);
            }
            store((uint32_t)(t0 + i) * yrow + ((uint32_t)f2 * C + c) * es, a);
        }
    };
    const bool first_even_pad = 2 * f0 - d < 0;
    const bool last_odd_pad = 2 * (f0 + ncols - 1) + 1 - d >= F1;
    int s = 0;
    if (first_even_pad) {
        if (ncols == 1 && last_odd_pad) step(0, hc, hn, std::false_type{}, std::false_type{});
        else step(0, hc, hn, std::true_type{}, std::false_type{});
#pragma unroll
        for (int l = 0; l < 2 * kSubRows + 1; ++l) hc[l] = hn[l];
        s = 1;
    }
    const int full = last_odd_pad ? ncols - 1 : ncols;
    for (; s + 1 < full; s += 2) {
        step(s, hc, hn, std::true_type{}, std::true_type{});
        step(s + 1, hn, hc, std::true_type{}, std::true_type{});
    }
    if (s < full) {
        step(s, hc, hn, std::true_type{}, std::true_type{});
#pragma unroll
        for (int l = 0; l < 2 * kSubRows + 1; ++l) hc[l] = hn[l];
        ++s;
    }
    if (last_odd_pad && s < ncols) step(s, hc, hn, std::false_type{}, std::true_type{});
}

bool dwsub_fused_fwd_fits(int64_t B, int64_t T, int64_t F, int64_t C, bool causal, int elem_bytes) {
    const FrontDims fd = front_dims(T, F, causal ? 1 : 0);
    const int64_t T2 = fd.T2, F2 = fd.F2;
    if (T >= ((int64_t)1 << 28) || F >= ((int64_t)1 << 28)) return false;
    if (!product_below((int64_t)1 << 31, {T2 + kSubRows, F2, C, elem_bytes})) return false;
    if (!product_below((int64_t)1 << 31, {T, F, elem_bytes})) return false;  // one item's mel input
    const int64_t blocks = B * ((T2 + kSubRows - 1) / kSubRows) * ((F2 + kSubCols - 1) / kSubCols) *
                           ((C + kSubBlock - 1) / kSubBlock);
    return blocks < ((int64_t)1 << 31);
}

template <typename S>
static hipError_t launch_front_fwd_typed(const S* x, const S* w0, const S* b0, const S* w1, const S* b1,
                                         const int32_t* lengths, S* y, int64_t B, int64_t T, int64_t F, int64_t C,
                                         bool causal, hipStream_t st) {
    const int d = causal ? 1 : 0;
    const FrontDims fd = front_dims(T, F, d);
    const int64_t T1 = fd.T1, F1 = fd.F1, T2 = fd.T2, F2 = fd.F2;
    const uint32_t n_rt = (uint32_t)((T2 + kSubRows - 1) / kSubRows);
    const uint32_t n_ft = (uint32_t)((F2 + kSubCols - 1) / kSubCols);
    const uint32_t n_cblk = (uint32_t)((C + kSubBlock - 1) / kSubBlock);
    const uint64_t blocks = (uint64_t)B * n_rt * n_ft * n_cblk;
    hipLaunchKernelGGL(dwsub_fused_fwd_kernel<S>, dim3((uint32_t)blocks), dim3(kSubBlock), 0, st, x, w0, b0, w1, b1,
                       lengths, y, (int32_t)T, (int32_t)F, (int32_t)C, (int32_t)T1, (int32_t)F1, (int32_t)T2,
                       (int32_t)F2, (int32_t)d, n_rt, n_ft, n_cblk);
    return hipGetLastError();
}

hipError_t launch_dwsub_fused_fwd(const void* x, const void* w0, const void* b0, const void* w1, const void* b1,
                                  const int32_t* lengths, void* y, int64_t B, int64_t T, int64_t F, int64_t C,
                                  bool causal, bool bf16, hipStream_t st) {
    if (bf16)
        return launch_front_fwd_typed<uint16_t>((const uint16_t*)x, (const uint16_t*)w0, (const uint16_t*)b0,
                                                (const uint16_t*)w1, (const uint16_t*)b1, lengths, (uint16_t*)y, B, T,
                                                F, C, causal, st);
    return launch_front_fwd_typed<float>((const float*)x, (const float*)w0, (const float*)b0, (const float*)w1,
                                         (const float*)b1, lengths, (float*)y, B, T, F, C, causal, st);
}


// ---------------------------------------------------------------------------
// Backward of the front with respect to its parameters: dw0, db0, dw1, db1
// (NeMo PR #16114, "What does this PR do": the fused kernels serve the
// encoder's training step).  The mel input needs no gradient.
//
// h is recomputed on chip from the mel patch, never read from memory.  The
// h positions are taken in "quads" (h rows 2t'-d, 2t'+1-d x columns 2f'-d,
// 2f'+1-d; the causal mode's shift d = 1 only moves which h rows a quad
// holds, and quad row or column 0 then holds the padding row or column -1),
// each with the four gradients dy[t'..t'+1, f'..f'+1] it meets, exactly as
// in the conv2d backward:
//   dh[2t',  2f'  ] = g00 w1[1,1]
//   dh[2t',  2f'+1] = g00 w1[1,2] + g01 w1[1,0]
//   dh[2t'+1,2f'  ] = g00 w1[2,1] + g10 w1[0,1]
//   dh[2t'+1,2f'+1] = g00 w1[2,2] + g01 w1[2,0] + g10 w1[0,2] + g11 w1[0,0]
// and each (h, dy) pair above adds h * dy to the dw1 tap it multiplies; every
// pair of the depthwise stage belongs to exactly one quad, and db1 adds g00
// once per quad.  Then dz = dh where the h row is unmasked and z > 0, and
// dw0[i,j] += dz * mel[2r+i-1, 2q+j-1], db0 += dz.
//
// Precision.  Everything from z on is fp64: the ReLU's derivative is a
// decision on the sign of z, and an fp32 z would take it differently from a
// full-precision reference for the few z that sit within an fp32 rounding of
// zero, each such flip moving dw0 by a whole term.  fp64 FMA runs at the
// fp32 vector rate here.  The sums are kept per thread in fp64, written as
// one partial per workgroup and added in a fixed order (reduce.hip).
//
// Mapping.  One thread per channel; a tile is QR quad rows x QC quad columns
// of one item, with its zero-padded mel patch staged in LDS as fp64.  G
// persistent workgroups per channel block take the batch's tiles
// round-robin and keep their sums across tiles.  A tile's loads (its
// (QR+1) x (QC+1) gradients per thread and one mel patch element per thread)
// are issued into registers while the previous tile computes; the patch then
// goes to LDS between two barriers (front backward 33.7 -> 31.8 us in the
// step on MI355X, the same partial sums bit for bit).
// ---------------------------------------------------------------------------

#ifndef DWSUB_BWD_QROWS
#define DWSUB_BWD_QROWS 2
#endif
#ifndef DWSUB_BWD_WGS
#define DWSUB_BWD_WGS 512
#endif
constexpr int kBQR = DWSUB_BWD_QROWS;          // quad rows per tile
constexpr int kBPatchRows = 4 * kBQR + 1;      // mel rows 4*t0-1-3d .. 4*t0+4*QR-1-3d

// Quad columns per tile: 4 where they divide F2, else 5 (measured on MI355X
// within the whole bench step: F2 = 20 with 4 columns 42.6 us, with 5 45.5;
// F2 = 21 with 5 columns 43.2, with 3 45.3).
static int front_bwd_qcols(int64_t F2) { return F2 > 0 && F2 % 4 == 0 ? 4 : 5; }
constexpr int kFrontGrads = 20;                // dw0 (9), db0, dw1 (9), db1

template <typename S, int QC>
__global__ __launch_bounds__(kSubBlock) void dwsub_fused_bwd_kernel(
    const S* __restrict__ x, const S* __restrict__ w0, const S* __restrict__ b0,
    const S* __restrict__ w1, const int32_t* __restrict__ lengths, const S* __restrict__ dy,
    double* __restrict__ partial, int32_t T, int32_t F, int32_t C, int32_t T1, int32_t F1, int32_t T2,
    int32_t F2, int32_t d, uint32_t n_rt, uint32_t n_ft, uint32_t n_tiles, uint32_t n_cblk) {
    constexpr int kBQC = QC;                   // quad columns per tile
    constexpr int kBPatchCols = 4 * kBQC + 1;  // mel columns 4*f0-1-3d .. 4*f0+4*QC-1-3d
    __shared__ double patch[kBPatchRows][kBPatchCols];
    const uint32_t blk = xcd_contiguous_block(blockIdx.x, gridDim.x);
    const uint32_t G = gridDim.x / n_cblk;
    const uint32_t g = blk / n_cblk, cblk = blk - g * n_cblk;
    const int32_t c = (int32_t)cblk * kSubBlock + (int32_t)threadIdx.x;
    const bool active = c < C;

    // Parameters of channel c (channel 0 stands in for a thread past C, which
    // computes nothing), loaded with no condition around each load so that
    // the 19 loads are in flight together: a select per load had made each
    // one wait for the last (front backward 38.6 -> 36.8 us on MI355X).
    const int32_t cp = active ? c : 0;
    S wa_s[9], wb_s[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) {
        wa_s[k] = w0[(int64_t)k * C + cp];
        wb_s[k] = w1[(int64_t)k * C + cp];
    }
    const S ba_s = b0 ? b0[cp] : S(0);
    double wa[9], wb[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) {
        wa[k] = (double)to_f32(wa_s[k]);
        wb[k] = (double)to_f32(wb_s[k]);
    }
    const double ba = (double)to_f32(ba_s);

    double gw0[9], gw1[9], gb0 = 0.0, gb1 = 0.0;
#pragma unroll
    for (int k = 0; k < 9; ++k) gw0[k] = gw1[k] = 0.0;

    constexpr uint32_t es = sizeof(S);
    const uint32_t grow = (uint32_t)F2 * C * es;
    static_assert(kBPatchRows * kBPatchCols <= kSubBlock, "one patch element per thread");
    const uint32_t coff = (uint32_t)(active ? c : 0) * es;
    const int pi = (int)threadIdx.x, pr = pi / kBPatchCols, pq = pi % kBPatchCols;
    // The loads of tile j: its gradients dy[t0 .. t0+QR, f0 .. f0+QC] and this
    // thread's element of the zero-padded mel patch.
    float gtn[kBQR + 1][kBQC + 1], pvn = 0.0f;
    auto fetch = [&](uint32_t j) {
        const uint32_t ft = j % n_ft, rest = j / n_ft;
        const uint32_t rt = rest % n_rt, b = rest / n_rt;
        const int32_t t0 = (int32_t)rt * kBQR, f0 = (int32_t)ft * kBQC;
        const rsrc_t gr = make_rsrc(dy + (int64_t)b * T2 * F2 * C, (uint32_t)T2 * grow);
#pragma unroll
        for (int q = 0; q <= kBQR; ++q)
#pragma unroll
            for (int e = 0; e <= kBQC; ++e)
                gtn[q][e] = Buf<S, 1>::load(gr, (uint32_t)(t0 + q) * grow + (uint32_t)(f0 + e) * C * es + coff).v[0];
        const int32_t t = 4 * t0 - 1 - 3 * d + pr, f = 4 * f0 - 1 - 3 * d + pq;
        const S* xb = x + (int64_t)b * T * F;
        const bool in = pi < kBPatchRows * kBPatchCols && t >= 0 && t < T && f >= 0 && f < F;
        pvn = in ? to_f32(xb[(int64_t)t * F + f]) : 0.0f;
    };
    if (g < n_tiles) fetch(g);
    for (uint32_t j = g; j < n_tiles; j += G) {
        const uint32_t ft = j % n_ft, rest = j / n_ft;
        const uint32_t rt = rest % n_rt, b = rest / n_rt;
        const int32_t t0 = (int32_t)rt * kBQR, f0 = (int32_t)ft * kBQC;  // first quad row / column
        const int32_t len = (int32_t)item_length(lengths, b, T);
        const int32_t hvalid = min(T1, len > 0 ? (len - 1 + d) / 2 + 1 : 0);  // h rows below this are unmasked
        float gt[kBQR + 1][kBQC + 1];
#pragma unroll
        for (int q = 0; q <= kBQR; ++q)
#pragma unroll
            for (int e = 0; e <= kBQC; ++e) gt[q][e] = gtn[q][e];
        const float pv = pvn;
        __syncthreads();  // every thread is done with the previous tile's patch
        if (pi < kBPatchRows * kBPatchCols) patch[pr][pq] = (double)pv;
        __syncthreads();
        if (j + G < n_tiles) fetch(j + G);  // the next tile's loads are in flight during this tile's arithmetic
        if (!active) continue;

        double gc[kBQR + 1];  // dy column f' for quad rows t0 .. t0+QR
#pragma unroll
        for (int q = 0; q <= kBQR; ++q) gc[q] = (double)gt[q][0];
        const int32_t ncols = min(kBQC, F2 - f0);
#pragma unroll
        for (int s = 0; s < kBQC; ++s) {
            if (s >= ncols) break;
            const int32_t f = f0 + s;
            const bool next_ok = f + 1 < F2;     // dy column f'+1 exists
            const bool eok = 2 * f - d >= 0;     // h column 2f'-d exists
            const bool cok = 2 * f + 1 - d < F1; // h column 2f'+1-d exists
            double gn[kBQR + 1];
#pragma unroll
            for (int q = 0; q <= kBQR; ++q) gn[q] = next_ok ? (double)gt[q][s + 1] : 0.0;
#pragma unroll
            for (int q = 0; q < kBQR; ++q) {
                const double g00 = gc[q], g01 = gn[q], g10 = gc[q + 1], g11 = gn[q + 1];
                gb1 += g00;
                const int32_t r0 = 2 * (t0 + q) - d;  // h rows r0, r0 + 1
                // A masked row's mel rows may be anything and are never
                // combined.  Past this test row r0 is unmasked, or it is the
                // padding row -1 of the causal mode, whose staged mel rows
                // are zeros: its terms are then formed and add exact zeros.
                const bool v0 = r0 >= 0 && r0 < hvalid, v1 = r0 + 1 >= 0 && r0 + 1 < hvalid;
                if (r0 >= hvalid) continue;  // both rows masked: no other term
                // The quad's top h row (mel patch rows 4q .. 4q+2), then its
                // bottom row (4q+2 .. 4q+4): three patch rows live at a time.
                double P[3][5];
#pragma unroll
                for (int a = 0; a < 3; ++a)
#pragma unroll
                    for (int e = 0; e < 5; ++e) P[a][e] = patch[4 * q + a][4 * s + e];
                double z00 = ba, z01 = ba;
#pragma unroll
                for (int i = 0; i < 3; ++i)
#pragma unroll
                    for (int k = 0; k < 3; ++k) {
                        z00 = __builtin_fma(P[i][k], wa[3 * i + k], z00);
                        z01 = __builtin_fma(P[i][2 + k], wa[3 * i + k], z01);
                    }
                const bool m00 = v0 && eok && z00 > 0.0, m01 = v0 && cok && z01 > 0.0;
                const double h00 = m00 ? z00 : 0.0, h01 = m01 ? z01 : 0.0;
                // depthwise stage: weight gradient from the (h, dy) pairs of this quad
                gw1[4] = __builtin_fma(g00, h00, gw1[4]);
                gw1[5] = __builtin_fma(g00, h01, gw1[5]);
                gw1[3] = __builtin_fma(g01, h01, gw1[3]);
                // gradient at h, then through the ReLU and the mask
                const double dh00 = g00 * wb[4];
                const double dh01 = __builtin_fma(g01, wb[3], g00 * wb[5]);
                const double dz00 = m00 ? dh00 : 0.0, dz01 = m01 ? dh01 : 0.0;
                gb0 += dz00 + dz01;
#pragma unroll
                for (int i = 0; i < 3; ++i)
#pragma unroll
                    for (int k = 0; k < 3; ++k)
                        gw0[3 * i + k] =
                            __builtin_fma(dz01, P[i][2 + k], __builtin_fma(dz00, P[i][k], gw0[3 * i + k]));
                if (v1) {
#pragma unroll
                    for (int a = 0; a < 3; ++a)
#pragma unroll
                        for (int e = 0; e < 5; ++e) P[a][e] = patch[4 * q + 2 + a][4 * s + e];
                    double z10 = ba, z11 = ba;
#pragma unroll
                    for (int i = 0; i < 3; ++i)
#pragma unroll
                        for (int k = 0; k < 3; ++k) {
                            z10 = __builtin_fma(P[i][k], wa[3 * i + k], z10);
                            z11 = __builtin_fma(P[i][2 + k], wa[3 * i + k], z11);
                        }
                    const bool m10 = eok && z10 > 0.0, m11 = cok && z11 > 0.0;
                    const double h10 = m10 ? z10 : 0.0, h11 = m11 ? z11 : 0.0;
                    gw1[7] = __builtin_fma(g00, h10, gw1[7]);
                    gw1[1] = __builtin_fma(g10, h10, gw1[1]);
                    gw1[8] = __builtin_fma(g00, h11, gw1[8]);
                    gw1[6] = __builtin_fma(g01, h11, gw1[6]);
                    gw1[2] = __builtin_fma(g10, h11, gw1[2]);
                    gw1[0] = __builtin_fma(g11, h11, gw1[0]);
                    const double dh10 = __builtin_fma(g10, wb[1], g00 * wb[7]);
                    const double dh11 =
                        __builtin_fma(g11, wb[0], __builtin_fma(g10, wb[2], __builtin_fma(g01, wb[6], g00 * wb[8])));
                    const double dz10 = m10 ? dh10 : 0.0, dz11 = m11 ? dh11 : 0.0;
                    gb0 += dz10 + dz11;
#pragma unroll
                    for (int i = 0; i < 3; ++i)
#pragma unroll
                        for (int k = 0; k < 3; ++k)
                            gw0[3 * i + k] =
                                __builtin_fma(dz11, P[i][2 + k], __builtin_fma(dz10, P[i][k], gw0[3 * i + k]));
                }
            }
#pragma unroll
            for (int q = 0; q <= kBQR; ++q) gc[q] = gn[q];
        }
    }
    if (!active) return;
    double* out = partial + (int64_t)g * kFrontGrads * C + c;
#pragma unroll
    for (int k = 0; k < 9; ++k) {
        out[(int64_t)k * C] = gw0[k];
        out[(int64_t)(10 + k) * C] = gw1[k];
    }
    out[(int64_t)9 * C] = gb0;
    out[(int64_t)19 * C] = gb1;
}

struct FrontBwdGrid {
    uint32_t n_rt, n_ft, n_tiles, G;
    int qc;
};

// The quad grid is T2 x F2 in both modes: ceil((T1 + d)/2) = T2 quad rows
// cover the h rows, and every dy row is a quad row.
static FrontBwdGrid front_bwd_grid(int64_t B, int64_t T, int64_t F, int d) {
    const FrontDims fd = front_dims(T, F, d);
    const int64_t T2 = fd.T2, F2 = fd.F2;
    FrontBwdGrid g;
    g.qc = front_bwd_qcols(F2);
    g.n_rt = (uint32_t)((T2 + kBQR - 1) / kBQR);
    g.n_ft = (uint32_t)((F2 + g.qc - 1) / g.qc);
    const uint64_t n = (uint64_t)B * g.n_rt * g.n_ft;
    g.n_tiles = (uint32_t)n;
    g.G = (uint32_t)(n < DWSUB_BWD_WGS ? n : DWSUB_BWD_WGS);
    return g;
}

bool dwsub_fused_bwd_fits(int64_t B, int64_t T, int64_t F, int64_t C, bool causal, int elem_bytes) {
    const FrontDims fd = front_dims(T, F, causal ? 1 : 0);
    const int64_t T2 = fd.T2, F2 = fd.F2;
    if (T >= ((int64_t)1 << 28) || F >= ((int64_t)1 << 28) || C >= ((int64_t)1 << 24)) return false;
    if (!product_below((int64_t)1 << 31, {T2 + kBQR + 1, F2, C, elem_bytes})) return false;
    const int qc = front_bwd_qcols(F2);
    return (uint64_t)B * ((T2 + kBQR - 1) / kBQR) * ((F2 + qc - 1) / qc) < ((uint64_t)1 << 31);
}

size_t dwsub_fused_bwd_workspace(int64_t B, int64_t T, int64_t F, int64_t C, bool causal) {
    const int64_t P = front_bwd_grid(B, T, F, causal ? 1 : 0).G;
    const int64_t ch = partial_reduce_chunks(P);
    return (size_t)((P + (ch > 0 ? ch : 1)) * kFrontGrads * C * (int64_t)sizeof(double));
}

hipError_t launch_dwsub_fused_bwd(const void* x, const void* w0, const void* b0, const void* w1,
                                  const int32_t* lengths, const void* dy, float* dw0, float* db0, float* dw1,
                                  float* db1, void* workspace, int64_t B, int64_t T, int64_t F, int64_t C,
                                  bool causal, bool bf16, hipStream_t st) {
    const int d = causal ? 1 : 0;
    const FrontDims fd = front_dims(T, F, d);
    const int64_t T1 = fd.T1, F1 = fd.F1, T2 = fd.T2, F2 = fd.F2;
    const FrontBwdGrid g = front_bwd_grid(B, T, F, d);
    const uint32_t n_cblk = (uint32_t)((C + kSubBlock - 1) / kSubBlock);
    double* partial = (double*)workspace;
    if (g.G > 0) {
        const dim3 grid(g.G * n_cblk), block(kSubBlock);
#define DWSUB_BWD_LAUNCH(QQ)                                                                                   \
    if (bf16)                                                                                                   \
        hipLaunchKernelGGL((dwsub_fused_bwd_kernel<uint16_t, QQ>), grid, block, 0, st, (const uint16_t*)x,        \
                           (const uint16_t*)w0, (const uint16_t*)b0, (const uint16_t*)w1, lengths,                \
                           (const uint16_t*)dy, partial, (int32_t)T, (int32_t)F, (int32_t)C, (int32_t)T1,        \
                           (int32_t)F1, (int32_t)T2, (int32_t)F2, (int32_t)d, g.n_rt, g.n_ft, g.n_tiles, n_cblk); \
    else                                                                                                        \
        hipLaunchKernelGGL((dwsub_fused_bwd_kernel<float, QQ>), grid, block, 0, st, (const float*)x,              \
                           (const float*)w0, (const float*)b0, (const float*)w1, lengths, (const float*)dy,      \
                           partial, (int32_t)T, (int32_t)F, (int32_t)C, (int32_t)T1, (int32_t)F1, (int32_t)T2,  \
                           (int32_t)F2, (int32_t)d, g.n_rt, g.n_ft, g.n_tiles, n_cblk);
        if (g.qc == 4) {
            DWSUB_BWD_LAUNCH(4)
        } else {
            DWSUB_BWD_LAUNCH(5)
        }
#undef DWSUB_BWD_LAUNCH
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    RowOutputs out = {};
    out.n = 4;
    out.p[0] = dw0; out.first[0] = 0; out.count[0] = 9;
    out.p[1] = db0; out.first[1] = 9; out.count[1] = 1;
    out.p[2] = dw1; out.first[2] = 10; out.count[2] = 9;
    out.p[3] = db1; out.first[3] = 19; out.count[3] = 1;
    return launch_partial_reduce(partial, g.G, kFrontGrads, C, partial + (int64_t)g.G * kFrontGrads * C, out, st);
}

}  // namespace dw
