// Depthwise conv2d, 3x3, stride 2, forward and backward, for gfx950 (NeMo PR
// #16114, "What does this PR do": the general depthwise conv2d with the pre-
// and post-masking and the causal padding fused into the kernel, and its
// backward).  fp32 or bf16 storage; arithmetic in fp32, weight gradients in
// fp64.
//
// Layout: x, dx [B][T][F][C], y, dy [B][T'][F'][C]; w [3][3][C]; channel
// fastest.  Padding: pt0 (1 or 2) zero rows before the input and pt1 (0..2)
// after it in time, pf0 and pf1 likewise in frequency; pads of 1 everywhere
// are the symmetric convolution, (2, 1) on an axis its causal padding.  With
// dt = pt0 - 1 and df = pf0 - 1 (0 or 1), output (t', f') reads input rows
// 2t'-1-dt .. 2t'+1-dt and columns 2f'-1-df .. 2f'+1-df;
// T' = floor((T + pt0 + pt1 - 3)/2) + 1, and likewise F'.
//
// Masks through buffer resources: each item's x is read through a resource
// that ends at its valid length (rows t >= len read as zero: the pre-mask)
// and dy through one that ends at len' = floor((len + pt0 + pt1 - 3)/2) + 1
// (masked gradient rows read as zero), and a negative row offset is out of
// range as well, which gives the top padding rows.  The frequency padding
// needs care: a column offset past either edge would land in a neighbouring
// row, so such a column is addressed out of range (kOutOfRange below) or, for
// the backward's dy column, loaded and then selected away.
//
// Forward mapping.  A thread owns V channels of TO consecutive output rows of
// one item and walks left to right over a chunk of the F' output columns.  At
// output column f' it needs input columns 2f'-1-df, 2f'-df, 2f'+1-df; the
// last is carried to the next step as its first, so every input element is
// loaded once per thread, and the one input row shared with the next row
// block comes from L2.
//
// Backward mapping.  dx is gathered, not scattered: output-parity phases.
// Take x rows 2m, 2m+1 and columns 2n, 2n+1 as one "quad" (m, n).  Along an
// axis with one zero before it, output o reads inputs 2o-1 .. 2o+1, so input
// 2n meets tap 1 of output n, and input 2n+1 taps 2 of output n and 0 of
// output n+1; with two zeros before it (the causal padding), output o reads
// 2o-2 .. 2o, so input 2n meets tap 2 of output n and tap 0 of output n+1,
// and input 2n+1 tap 1 of output n+1 (AxisTerms below).  With one zero
// before both axes, writing t' = m, f' = n:
//   dx[2t',  2f'  ] = g[t',f'] w11
//   dx[2t',  2f'+1] = g[t',f'] w12 + g[t',f'+1] w10
//   dx[2t'+1,2f'  ] = g[t',f'] w21 + g[t'+1,f'] w01
//   dx[2t'+1,2f'+1] = g[t',f'] w22 + g[t',f'+1] w20 + g[t'+1,f'] w02 + g[t'+1,f'+1] w00
// and the same (g, x) pairs give the weight gradient: each pair adds
// g * x(quad element) to the tap it multiplies.  Every (input, output) pair
// of the convolution belongs to exactly one quad, so dw is complete and no
// pair is counted twice; db adds g[t',f'] once per quad.  The quad grid
// spans max(ceil(T/2), T') rows, and max(ceil(F/2), F') columns with one
// zero before the columns, so every g element is some quad's g[t',f'].  With
// two zeros before the columns F' can be ceil(F/2) + 1; the grid then keeps
// max(ceil(F/2), F'-1) columns, so that a row splits into equal chunks, and
// the last g column is added to db by the chunk that ends the row.  A thread
// walks a chunk of the quad columns of one row block left to right, carrying
// the g column f'+1 (a chunk starts by loading its first g column).  dw and db
// are accumulated in fp64 from the start (an fp32 x fp32 product is exact in
// fp64, and fp64 FMA runs at the fp32 rate here), because a sum of ~10^6
// terms can cancel to a value far smaller than its terms.  They are summed
// per thread, then across the workgroup's row blocks in a fixed order,
// written as one fp64 partial per workgroup to the workspace, and the
// partials are added in a fixed order (reduce.hip): the result is bitwise
// repeatable.
#include "common.h"
#include "launch.h"

namespace dw {

constexpr int kBlock2d = 256;
constexpr int kLanes2d = 64;                      // channel groups per workgroup row
constexpr int kRowsPerBlock = kBlock2d / kLanes2d;  // row blocks per workgroup

#ifndef DW2D_FWD_ROWS
#define DW2D_FWD_ROWS 1
#endif
#ifndef DW2D_FWD_PERSIST
#define DW2D_FWD_PERSIST 512  // workgroups of the persistent forward grid
#endif
#ifndef DW2D_BWD_XPOL
#define DW2D_BWD_XPOL 2
#endif
// Cache policy of the backward's x loads: every x element is read by exactly
// one quad, so they are loaded non-temporally (2) and leave the cache to the
// g rows that neighbouring quad rows share.
constexpr int kBwdXPolicy = DW2D_BWD_XPOL;
#ifndef DW2D_STORE_POLICY
#define DW2D_STORE_POLICY 18
#endif
// Cache policy of the y and dx stores: non-temporal (2) with the sc1 scope
// bit (16) set.  On MI355X this took the stage backward from 944 to 922 us
// and its causal form from 961 to 941 (non-temporal alone: the previous
// figures; sc1 alone or sc0 with it: the forward 2-10% slower).
constexpr int kStorePolicy2d = DW2D_STORE_POLICY;
#ifndef DW2D_FWD_MIDPOL
#define DW2D_FWD_MIDPOL 2
#endif
// Cache policy of the forward's loads of input rows 2t', which no other
// output row reads: non-temporal (2), leaving the cache to the shared rows.
constexpr int kFwdMidPolicy = DW2D_FWD_MIDPOL;
#ifndef DW2D_BWD_ROWS
#define DW2D_BWD_ROWS 1
#endif
constexpr int kFwdRows = DW2D_FWD_ROWS;   // output rows per thread (forward)
constexpr int kBwdRows = DW2D_BWD_ROWS;   // quad rows per thread (backward)

#ifndef DW2D_BWD_ROWS_BF16
#define DW2D_BWD_ROWS_BF16 2
#endif
#ifndef DW2D_FWD_BF16_VEC
#define DW2D_FWD_BF16_VEC 8  // widest bf16 forward access: 8 channels, 16 bytes
#endif
// quad rows per thread of the backward, per storage type
template <typename S>
constexpr int bwd_rows() { return sizeof(S) == 2 ? DW2D_BWD_ROWS_BF16 : kBwdRows; }

template <int V>
__device__ __forceinline__ void fma_v(Vf<V>& acc, const Vf<V>& a, const Vf<V>& b) {
#pragma unroll
    for (int e = 0; e < V; ++e) acc.v[e] = __builtin_fmaf(a.v[e], b.v[e], acc.v[e]);
}

// acc += a * b in fp64; the product of two floats is exact in fp64.
template <int V>
__device__ __forceinline__ void fma_d(double (&acc)[V], const Vf<V>& a, const Vf<V>& b) {
#pragma unroll
    for (int e = 0; e < V; ++e) acc[e] = __builtin_fma((double)a.v[e], (double)b.v[e], acc[e]);
}

template <int V>
__device__ __forceinline__ Vf<V> select_v(bool keep, const Vf<V>& a) {
    Vf<V> r;
#pragma unroll
    for (int e = 0; e < V; ++e) r.v[e] = keep ? a.v[e] : 0.0f;
    return r;
}

// A column offset past either edge of a row would land in a neighbouring row,
// so such a column is addressed at this offset instead.  Added to any row
// offset the kernels form (at most T + 2 rows, below 2^31 - 2 rows by
// dwconv2d_fits, or a row -1 or -2 that wrapped below 2^32), the sum is at or
// past every resource's size, and the load returns zero.
constexpr uint32_t kOutOfRange = 0x80000000u;

// Geometry handed to the kernels (all sizes fit in 32 bits: dwconv2d_fits).
struct Geo2d {
    int32_t T, F, C, To, Fo;
    int32_t dt, df;     // pad before - 1, per axis (0 or 1)
    int32_t len_add;    // pt0 + pt1 - 3: len' = floor((len + len_add) / 2) + 1
    int32_t NQt, NQf;   // quad rows and columns of the backward
    int32_t fcols;      // output columns per forward thread
    int32_t nqc, qcols; // backward: column chunks of a quad row, quad columns per chunk
};

// Valid output rows of an item with len valid input rows.
__device__ __forceinline__ int32_t out_rows(int32_t len, const Geo2d& g) {
    if (len <= 0) return 0;
    const int32_t o = ((len + g.len_add) >> 1) + 1;  // arithmetic shift: floor division
    return o < 0 ? 0 : (o > g.To ? g.To : o);
}

// ------------------------------------------------------------------ fwd ----

template <typename S, int V, int TO, int LANES>
__global__ __launch_bounds__(kBlock2d) void dwconv2d_fwd_kernel(
    const S* __restrict__ x, const S* __restrict__ w, const S* __restrict__ bias,
    const int32_t* __restrict__ lengths, S* __restrict__ y, Geo2d geo, int32_t B_items,
    uint32_t n_rb, uint32_t CG, uint32_t n_cblk, uint32_t groups_per_item) {
    // A workgroup is kBlock2d / LANES row blocks of LANES channel groups
    // (LANES = 32 when there are at most 32 groups: two row blocks a wave).
    constexpr int32_t es = (int32_t)sizeof(S);
    constexpr uint32_t kRB = kBlock2d / LANES;
    const int32_t T = geo.T, F = geo.F, C = geo.C, To = geo.To, Fo = geo.Fo;
    // The batch's row groups are dealt round-robin to the workgroups of a
    // channel block, so every workgroup gets a like mix of long and short
    // (masked) items.
    const uint32_t blk0 = xcd_contiguous_block(blockIdx.x, gridDim.x);
    const uint32_t G = gridDim.x / n_cblk;
    const uint32_t g0 = blk0 / n_cblk, cb0 = blk0 - g0 * n_cblk;
    const uint32_t cg = cb0 * LANES + threadIdx.x % LANES;
    // A thread keeps its channels for the whole kernel: taps and bias are
    // loaded once.
    Vf<V> wk[9], bv = vzero<V>();
#pragma unroll
    for (int k = 0; k < 9; ++k) wk[k] = vzero<V>();
    if (cg < CG) {
#pragma unroll
        for (int k = 0; k < 9; ++k) wk[k] = load_param<S, V>(w + (int64_t)k * C + (int32_t)cg * V);
        if (bias) bv = load_param<S, V>(bias + (int32_t)cg * V);
    }
    for (uint32_t j = g0; j < (uint32_t)B_items * groups_per_item; j += G) {
        const uint32_t b = j / groups_per_item;
        const uint32_t rb = (j - b * groups_per_item) * kRB + threadIdx.x / LANES;
        if (rb >= n_rb || cg >= CG) continue;
        const int32_t len = (int32_t)item_length(lengths, b, T);
        const int32_t leno = out_rows(len, geo);
        const uint32_t xrow = (uint32_t)(F * C * es), yrow = (uint32_t)(Fo * C * es);
        const int32_t pix = C * es;
        const rsrc_t xr = make_rsrc(x + (int64_t)b * T * F * C, (uint32_t)len * xrow);
        const rsrc_t yr = make_rsrc(y + (int64_t)b * To * Fo * C, (uint32_t)To * yrow);
        const int32_t c0 = (int32_t)cg * V;
        const uint32_t coff = (uint32_t)(c0 * es);
        // row-block index = row block * column chunks + column chunk
        const int32_t nfc = (Fo + geo.fcols - 1) / geo.fcols;
        const int32_t t0 = (int32_t)(rb / nfc) * TO;
        const int32_t fa = (int32_t)(rb % nfc) * geo.fcols, fb = min(Fo, fa + geo.fcols);

        if (t0 >= leno) {
            const Vf<V> z = vzero<V>();
            for (int32_t f = fa; f < fb; ++f)
#pragma unroll
                for (int i = 0; i < TO; ++i)
                    Buf<S, V>::template store<kStorePolicy2d>(yr, (uint32_t)(t0 + i) * yrow + (uint32_t)(f * pix) + coff, z);
            continue;
        }

        // Input rows 2t0-1-dt+r, r = 0 .. 2*TO; byte offset of each row start
        // (a negative row wraps out of range and reads zero).
        uint32_t roff[2 * TO + 1];
#pragma unroll
        for (int r = 0; r < 2 * TO + 1; ++r) roff[r] = (uint32_t)((2 * t0 - 1 - geo.dt + r) * (int32_t)xrow) + coff;

        // Input column 2f'-1-df, carried; zero left of the first column.
        // bf16 loads it out of range there (zeros): a select between the
        // load and zeros made that kernel wait for each load in turn
        // (272 -> 257 us on MI355X).  The fp32 kernel keeps the select, which
        // measured faster there (515 against 531 us).
        const int32_t c_first = 2 * fa - 1 - geo.df;
        Vf<V> carry[2 * TO + 1];
        if constexpr (sizeof(S) == 2) {
            const uint32_t cfo = c_first >= 0 ? (uint32_t)(c_first * pix) : kOutOfRange;
#pragma unroll
            for (int r = 0; r < 2 * TO + 1; ++r) carry[r] = Buf<S, V>::load(xr, roff[r] + cfo);
        } else {
#pragma unroll
            for (int r = 0; r < 2 * TO + 1; ++r)
                carry[r] = c_first >= 0 ? Buf<S, V>::load(xr, roff[r] + (uint32_t)(c_first * pix)) : vzero<V>();
        }

        for (int32_t f = fa; f < fb; ++f) {
            const int32_t ce = 2 * f - geo.df;           // input columns ce, ce + 1
            const uint32_t eo = ce >= 0 && ce < F ? (uint32_t)(ce * pix) : kOutOfRange;
            const uint32_t oo = ce + 1 < F ? (uint32_t)((ce + 1) * pix) : kOutOfRange;
            Vf<V> xe[2 * TO + 1], xo[2 * TO + 1];
#pragma unroll
            for (int r = 0; r < 2 * TO + 1; ++r) {
                // rows 2t' (odd r) are read by this row block alone; the even
                // r are shared with a neighbouring output row
                if (r % 2 == 1 && kFwdMidPolicy != kLoadPolicy) {
                    xe[r] = Buf<S, V>::template load<kFwdMidPolicy>(xr, roff[r] + eo);
                    xo[r] = Buf<S, V>::template load<kFwdMidPolicy>(xr, roff[r] + oo);
                } else {
                    xe[r] = Buf<S, V>::load(xr, roff[r] + eo);
                    xo[r] = Buf<S, V>::load(xr, roff[r] + oo);
                }
            }
#pragma unroll
            for (int i = 0; i < TO; ++i) {
                Vf<V> acc = bv;
#pragma unroll
                for (int a = 0; a < 3; ++a) {
                    fma_v<V>(acc, carry[2 * i + a], wk[3 * a + 0]);
                    fma_v<V>(acc, xe[2 * i + a], wk[3 * a + 1]);
                    fma_v<V>(acc, xo[2 * i + a], wk[3 * a + 2]);
                }
                acc = select_v<V>(t0 + i < leno, acc);
                Buf<S, V>::template store<kStorePolicy2d>(yr, (uint32_t)(t0 + i) * yrow + (uint32_t)(f * pix) + coff, acc);
            }
#pragma unroll
            for (int r = 0; r < 2 * TO + 1; ++r) carry[r] = xo[r];
        }
    }
}

// ------------------------------------------------------------------ bwd ----

// The terms of one axis of the backward's gather.  Input positions 2n and
// 2n+1 form a pair; with padding P+1 before the axis (P = 0 or 1), output o
// reads inputs 2o-1-P .. 2o+1-P through taps 0, 1, 2, so the outputs and taps
// reaching the pair are, as (output - n, tap):
//   P = 0:  2n <- (0, 1);           2n+1 <- (0, 2), (1, 0)
//   P = 1:  2n <- (0, 2), (1, 0);   2n+1 <- (1, 1)
template <int P>
struct AxisTerms {
    static constexpr int count(int e) { return (P == 0) == (e == 0) ? 1 : 2; }
    static constexpr int off(int e, int a) { return P == 0 ? (e == 0 ? 0 : a) : (e == 0 ? a : 1); }
    static constexpr int tap(int e, int a) {
        return P == 0 ? (e == 0 ? 1 : (a == 0 ? 2 : 0)) : (e == 0 ? (a == 0 ? 2 : 0) : 1);
    }
};

// Paired lanes: lane i < 32 holds 8 bf16 channels of column 2n and lane i + 32
// the same 8 channels of column 2n + 1.  Two cross-half swaps give lane i the
// first four channels of both columns (dwords x, y: column 2n; z, w: 2n + 1)
// and lane i + 32 the last four; applied to that layout, the same two swaps
// give back one column's 8 channels per lane.
__device__ __forceinline__ void pair_swap(u32x4& t) {
    const auto a = __builtin_amdgcn_permlane32_swap(t.x, t.z, false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(t.y, t.w, false, false);
    t.x = a[0]; t.z = a[1];
    t.y = b[0]; t.w = b[1];
}

__device__ __forceinline__ Vf<4> widen_bf16x4(uint32_t lo, uint32_t hi) {
    Vf<4> a;
    a.v[0] = bf16_lo(lo); a.v[1] = bf16_hi(lo); a.v[2] = bf16_lo(hi); a.v[3] = bf16_hi(hi);
    return a;
}

// PAIR (bf16 storage, V = 4): the x loads and dx stores move 16 bytes per
// lane instead of 8.  Lanes i and i + 32 of a wave share channels
// 8i .. 8i+7 of the channel block; for x columns 2n, 2n+1, lane i loads them
// at column 2n and lane i + 32 at column 2n+1, and pair_swap leaves lane i
// with channels 8i .. 8i+3 and lane i + 32 with 8i+4 .. 8i+7, of both
// columns: the four-channel layout the arithmetic takes.  Between its load
// and its use a lane's raw 16-byte piece rides in the xe registers of its row,
// bit for bit (xo is not loaded), and the swap is made where it is used.  The
// dx pair is swapped back before its 16-byte store.  A lane whose channels
// are past C runs every load, swap and store (at out-of-range offsets), so
// that every swap sees whole waves.  The host takes this form when C is a
// multiple of 8 and x and dx are 16-byte aligned.
template <typename S, int V, int TQ, int PR, int PC, bool PAIR = false>
__global__ __launch_bounds__(kBlock2d) void dwconv2d_bwd_kernel(
    const S* __restrict__ x, const S* __restrict__ w, const int32_t* __restrict__ lengths,
    const S* __restrict__ dy, S* __restrict__ dx, double* __restrict__ partial, Geo2d geo,
    uint32_t n_rb, uint32_t CG, uint32_t n_cblk, uint32_t groups_per_item, uint32_t n_groups) {
    constexpr int32_t es = (int32_t)sizeof(S);
    const int32_t T = geo.T, F = geo.F, C = geo.C, To = geo.To, Fo = geo.Fo;
    __shared__ double red[kRowsPerBlock - 1][10][kLanes2d * V];
    // Workgroup = kRowsPerBlock waves x kLanes2d channel groups.  The batch's
    // row groups (kRowsPerBlock row blocks each, items one after the other)
    // are dealt round-robin to the G = gridDim.x / n_cblk workgroups of a
    // channel block: group j goes to workgroup j mod G, so every workgroup
    // gets a like mix of long and short (masked) items, and neighbouring
    // workgroups work on neighbouring rows at the same time.  A workgroup
    // keeps one dw/db sum for all of its groups.
    const uint32_t blk = xcd_contiguous_block(blockIdx.x, gridDim.x);
    const uint32_t G = gridDim.x / n_cblk;
    const uint32_t g = blk / n_cblk, cblk = blk - g * n_cblk;
    const uint32_t lane = threadIdx.x % kLanes2d;
    static_assert(!PAIR || (sizeof(S) == 2 && V == 4 && kLanes2d == 64), "paired lanes: bf16, 4 channels, waves of 64");
    const uint32_t cg = PAIR ? cblk * kLanes2d + 2 * (lane % 32) + lane / 32 : cblk * kLanes2d + lane;
    const int32_t c0 = (int32_t)cg * V;
    const bool chan_ok = cg < CG;  // with PAIR, lanes i and i + 32 are both in or both out (C % 8 == 0)

    double gw[9][V], gb[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
        gb[e] = 0.0;
#pragma unroll
        for (int k = 0; k < 9; ++k) gw[k][e] = 0.0;
    }

    // Taps, loaded once: a thread keeps its channels for the whole kernel.
    Vf<V> wk[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) wk[k] = vzero<V>();
    if (chan_ok) {
#pragma unroll
        for (int k = 0; k < 9; ++k) wk[k] = load_param<S, V>(w + (int64_t)k * C + c0);
    }

    for (uint32_t j = g; j < n_groups; j += G) {
        const uint32_t b = j / groups_per_item;
        const uint32_t rb = (j - b * groups_per_item) * kRowsPerBlock + threadIdx.x / kLanes2d;  // one per wave
        if (rb >= n_rb || (!PAIR && !chan_ok)) continue;
        const int32_t len = (int32_t)item_length(lengths, b, T);
        const int32_t leno = out_rows(len, geo);
        const uint32_t xrow = (uint32_t)(F * C * es), grow = (uint32_t)(Fo * C * es);
        const int32_t pix = C * es;
        const int64_t xitem = (int64_t)b * T * F * C;
        const rsrc_t xr = make_rsrc(x + xitem, (uint32_t)len * xrow);
        const rsrc_t gr = make_rsrc(dy + (int64_t)b * To * Fo * C, (uint32_t)leno * grow);
        const rsrc_t dxr = make_rsrc(dx ? dx + xitem : x, dx ? (uint32_t)T * xrow : 0u);
        const uint32_t coff = (uint32_t)(c0 * es);
        const int32_t t0 = (int32_t)(rb / geo.nqc) * TQ;  // first quad row
        const int32_t xr0 = 2 * t0;                        // its first x row
        const int32_t na = (int32_t)(rb % geo.nqc) * geo.qcols;  // quad columns na .. nb-1
        const int32_t nb = min(geo.NQf, na + geo.qcols);
        // PAIR: the offset of this lane's 16-byte piece of x (and dx) columns
        // ce, ce + 1 within a row, out of range where that column or these
        // channels do not exist.
        const uint32_t pair_off = (lane / 32) * (uint32_t)pix + (cblk * kLanes2d + 2 * (lane % 32)) * V * es;
        auto pair_col = [&](int32_t ce) -> uint32_t {
            return chan_ok && ce + (int32_t)(lane / 32) < F ? (uint32_t)(ce * pix) + pair_off : kOutOfRange;
        };

        if (xr0 >= len && t0 >= leno) {
            // Every x row of this block is masked, and so is every g row it
            // adds to db: dx is zero and nothing adds to dw or db.
            if (dx) {
                const int32_t fa = 2 * na, fb = min(F, 2 * nb);
                if constexpr (PAIR) {
                    const u32x4 z = {0u, 0u, 0u, 0u};
                    for (int32_t f = fa; f < fb; f += 2) {
                        const uint32_t po = pair_col(f);
#pragma unroll
                        for (int r = 0; r < 2 * TQ; ++r)
                            __builtin_amdgcn_raw_buffer_store_b128(z, dxr, (uint32_t)(xr0 + r) * xrow + po, 0, kStorePolicy2d);
                    }
                } else {
                    const Vf<V> z = vzero<V>();
                    for (int32_t f = fa; f < fb; ++f)
#pragma unroll
                        for (int r = 0; r < 2 * TQ; ++r)
                            Buf<S, V>::template store<kStorePolicy2d>(dxr, (uint32_t)(xr0 + r) * xrow + (uint32_t)(f * pix) + coff, z);
                }
            }
            continue;
        }
        // g rows t0 .. t0+TQ (the last one belongs to the next block), column na.
        Vf<V> gcur[TQ + 1];
        const uint32_t no0 = na < Fo ? (uint32_t)(na * pix) : kOutOfRange;
#pragma unroll
        for (int q = 0; q <= TQ; ++q) gcur[q] = Buf<S, V>::load(gr, (uint32_t)((t0 + q) * (int32_t)grow) + coff + no0);

        // Loads for quad column n: g column n+1, and x columns 2n and 2n+1,
        // each replaced by an out-of-range offset (which reads zero with no
        // memory traffic) where it does not exist.
        auto load_col = [&](int32_t n, Vf<V>(&gn)[TQ + 1], Vf<V>(&xe)[2 * TQ], Vf<V>(&xo)[2 * TQ]) {
            const int32_t ce = 2 * n;
            // g column n+1 (past the last column it is loaded from the next
            // row, or read as zero past the valid rows, and then discarded)
#pragma unroll
            for (int q = 0; q <= TQ; ++q)
                gn[q] = select_v<V>(n + 1 < Fo,
                                    Buf<S, V>::load(gr, (uint32_t)((t0 + q) * (int32_t)grow + (n + 1) * pix) + coff));
            if constexpr (PAIR) {
                const uint32_t po = pair_col(ce);
#pragma unroll
                for (int r = 0; r < 2 * TQ; ++r) {
                    const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(xr, (uint32_t)((xr0 + r) * (int32_t)xrow) + po, 0,
                                                                          kBwdXPolicy);
                    xe[r].v[0] = __uint_as_float(t.x); xe[r].v[1] = __uint_as_float(t.y);
                    xe[r].v[2] = __uint_as_float(t.z); xe[r].v[3] = __uint_as_float(t.w);
                }
            } else {
                const uint32_t eo = ce < F ? (uint32_t)(ce * pix) : kOutOfRange;
                const uint32_t oo = ce + 1 < F ? (uint32_t)((ce + 1) * pix) : kOutOfRange;
#pragma unroll
                for (int r = 0; r < 2 * TQ; ++r) {
                    const uint32_t ro = (uint32_t)((xr0 + r) * (int32_t)xrow) + coff;
                    xe[r] = Buf<S, V>::template load<kBwdXPolicy>(xr, ro + eo);
                    xo[r] = Buf<S, V>::template load<kBwdXPolicy>(xr, ro + oo);
                }
            }
        };
        // The quads of column n, given its loads; g column n+1 becomes the
        // current column afterwards.  Each pair of x rows and each pair of x
        // columns takes its terms from AxisTerms; db adds g[m][n] once per
        // quad (and the g column past the last quad after the walk).
        auto quads = [&](int32_t n, const Vf<V>(&gnext)[TQ + 1], const Vf<V>(&xe_in)[2 * TQ],
                         const Vf<V>(&xo_in)[2 * TQ]) {
            using R = AxisTerms<PR>;
            using Cc = AxisTerms<PC>;
            const int32_t ce = 2 * n;
            Vf<V> xe[2 * TQ], xo[2 * TQ];
#pragma unroll
            for (int r = 0; r < 2 * TQ; ++r) {
                if constexpr (PAIR) {
                    u32x4 t = {__float_as_uint(xe_in[r].v[0]), __float_as_uint(xe_in[r].v[1]),
                               __float_as_uint(xe_in[r].v[2]), __float_as_uint(xe_in[r].v[3])};
                    pair_swap(t);
                    xe[r] = widen_bf16x4(t.x, t.y);
                    xo[r] = widen_bf16x4(t.z, t.w);
                } else {
                    xe[r] = xe_in[r];
                    xo[r] = xo_in[r];
                }
            }
#pragma unroll
            for (int q = 0; q < TQ; ++q) {
                const Vf<V> G[2][2] = {{gcur[q], gnext[q]}, {gcur[q + 1], gnext[q + 1]}};  // g[m+i][n+j]
                const Vf<V> X[2][2] = {{xe[2 * q], xo[2 * q]}, {xe[2 * q + 1], xo[2 * q + 1]}};
                // dx of the four x elements, then the (g, x) pairs for dw
                Vf<V> D[2][2];
#pragma unroll
                for (int er = 0; er < 2; ++er)
#pragma unroll
                    for (int ec = 0; ec < 2; ++ec) {
                        D[er][ec] = vzero<V>();
#pragma unroll
                        for (int a = 0; a < 2; ++a)
#pragma unroll
                            for (int bb = 0; bb < 2; ++bb)
                                if (a < R::count(er) && bb < Cc::count(ec))  // w[i][j] is tap 3i+j
                                    fma_v<V>(D[er][ec], G[R::off(er, a)][Cc::off(ec, bb)],
                                             wk[3 * R::tap(er, a) + Cc::tap(ec, bb)]);
                    }
#pragma unroll
                for (int er = 0; er < 2; ++er)
#pragma unroll
                    for (int ec = 0; ec < 2; ++ec)
#pragma unroll
                        for (int a = 0; a < 2; ++a)
#pragma unroll
                            for (int bb = 0; bb < 2; ++bb)
                                if (a < R::count(er) && bb < Cc::count(ec))
                                    fma_d<V>(gw[3 * R::tap(er, a) + Cc::tap(ec, bb)],
                                             G[R::off(er, a)][Cc::off(ec, bb)], X[er][ec]);
#pragma unroll
                for (int e = 0; e < V; ++e) gb[e] += (double)G[0][0].v[e];
                if (dx) {
                    // A column at or past F would land in the next row, so
                    // those stores are skipped; rows at or past T are past the
                    // resource and dropped.
                    const int32_t te = xr0 + 2 * q;
                    if constexpr (PAIR) {
                        const uint32_t po = pair_col(ce);
#pragma unroll
                        for (int er = 0; er < 2; ++er) {
                            const Vf<V> de = select_v<V>(te + er < len, D[er][0]);
                            const Vf<V> dd = select_v<V>(te + er < len, D[er][1]);
                            u32x4 t = {pack_bf16x2(de.v[0], de.v[1]), pack_bf16x2(de.v[2], de.v[3]),
                                       pack_bf16x2(dd.v[0], dd.v[1]), pack_bf16x2(dd.v[2], dd.v[3])};
                            pair_swap(t);
                            __builtin_amdgcn_raw_buffer_store_b128(t, dxr, (uint32_t)((te + er) * (int32_t)xrow) + po, 0,
                                                                   kStorePolicy2d);
                        }
                    } else {
                        const bool col_ok[2] = {ce < F, ce + 1 < F};
#pragma unroll
                        for (int ec = 0; ec < 2; ++ec)
#pragma unroll
                            for (int er = 0; er < 2; ++er)
                                if (col_ok[ec])
                                    Buf<S, V>::template store<kStorePolicy2d>(
                                        dxr, (uint32_t)((te + er) * (int32_t)xrow + (ce + ec) * pix) + coff,
                                        select_v<V>(te + er < len, D[er][ec]));
                    }
                }
            }
#pragma unroll
            for (int q = 0; q <= TQ; ++q) gcur[q] = gnext[q];
        };

        // Column n + 1's loads are issued before column n's arithmetic, so a
        // wave keeps two columns of loads in flight.
        Vf<V> ga[TQ + 1], xea[2 * TQ], xoa[2 * TQ];
        load_col(na, ga, xea, xoa);
        for (int32_t n = na; n + 1 < nb; ++n) {
            Vf<V> gb2[TQ + 1], xeb[2 * TQ], xob[2 * TQ];
            load_col(n + 1, gb2, xeb, xob);
            quads(n, ga, xea, xoa);
#pragma unroll
            for (int q = 0; q <= TQ; ++q) ga[q] = gb2[q];
#pragma unroll
            for (int r = 0; r < 2 * TQ; ++r) { xea[r] = xeb[r]; xoa[r] = xob[r]; }
        }
        quads(nb - 1, ga, xea, xoa);

        // With two columns of padding before, F' can be one more than the
        // quad columns: g column NQf then belongs to no quad as its own and is
        // added to db here, by the chunk that ends the row (as zero where it
        // does not exist).
        if constexpr (PC == 1) {
            if (nb == geo.NQf) {
#pragma unroll
                for (int q = 0; q < TQ; ++q)
#pragma unroll
                    for (int e = 0; e < V; ++e) gb[e] += (double)gcur[q].v[e];
            }
        }
    }

    if (!partial) return;  // uniform: dw and db not requested
    // Sum the row blocks of this workgroup in a fixed order (row block 0
    // first), then write one partial per workgroup: partial[p][k][c], k = 0..8
    // the taps, 9 the bias.
    const uint32_t rsub = threadIdx.x / kLanes2d;
    if (rsub > 0) {
#pragma unroll
        for (int e = 0; e < V; ++e) {
#pragma unroll
            for (int k = 0; k < 9; ++k) red[rsub - 1][k][lane * V + e] = gw[k][e];
            red[rsub - 1][9][lane * V + e] = gb[e];
        }
    }
    __syncthreads();
    if (rsub > 0) return;
    const uint32_t p = g;
#pragma unroll
    for (int e = 0; e < V; ++e) {
        const int32_t c = PAIR ? c0 + e : ((int32_t)cblk * kLanes2d + (int32_t)lane) * V + e;
        if (c >= C) continue;
#pragma unroll
        for (int k = 0; k < 10; ++k) {
            double s = k < 9 ? gw[k][e] : gb[e];
#pragma unroll
            for (int q = 0; q < kRowsPerBlock - 1; ++q) s += red[q][k][lane * V + e];
            partial[((int64_t)p * 10 + k) * C + c] = s;
        }
    }
}

// ------------------------------------------------------------- launchers ----

static int64_t floor_half(int64_t n) { return n >= 0 ? n / 2 : (n - 1) / 2; }

Conv2dGeom conv2d_geom(int64_t T, int64_t F, int64_t C, int64_t pt0, int64_t pt1, int64_t pf0, int64_t pf1) {
    Conv2dGeom g;
    g.T = T; g.F = F; g.C = C;
    g.pt0 = pt0; g.pt1 = pt1; g.pf0 = pf0; g.pf1 = pf1;
    const int64_t to = floor_half(T + pt0 + pt1 - 3) + 1, fo = floor_half(F + pf0 + pf1 - 3) + 1;
    g.To = to < 0 ? 0 : to;
    g.Fo = fo < 0 ? 0 : fo;
    return g;
}

bool dwconv2d_pads_supported(int64_t pt0, int64_t pt1, int64_t pf0, int64_t pf1) {
    return pt0 >= 1 && pt0 <= 2 && pf0 >= 1 && pf0 <= 2 && pt1 >= 0 && pt1 <= 2 && pf1 >= 0 && pf1 <= 2;
}

// Column chunking.  A thread walks a chunk of a row left to right; short
// chunks keep the rows that the resident waves touch at one time close
// together in memory, which streams faster than long ones (measured on MI355X
// at [32,1500,64,256]: 4 quad columns per chunk instead of 32 took the
// backward from 1031 to 966 us, 3 output columns instead of 8 the forward
// from 547 to 521), and chunks of unequal width cost more than the imbalance
// suggests (33 quad columns in 9 chunks, the last of width 1: 1109 us; in 11
// of width 3: 1048).  So the width is the first exact divisor from a short
// list of measured choices, else the list's first entry, evened out.
static int32_t chunk_width(int64_t n, const int* pref, int npref) {
    if (n <= 0) return 1;
    for (int i = 0; i < npref; ++i)
        if (pref[i] <= n && n % pref[i] == 0) return pref[i];
    const int64_t chunks = (n + pref[0] - 1) / pref[0];
    return (int32_t)((n + chunks - 1) / chunks);
}

// Output columns per forward thread.
static int32_t fwd_cols(int64_t Fo) {
    static const int pref[] = {4, 3};
    return chunk_width(Fo, pref, 2);
}

// Quad columns per backward chunk, for TQ quad rows per thread.
static int32_t bwd_qcols(int64_t NQf, int tq) {
    static const int pref1[] = {4, 3, 2, 5}, pref2[] = {8, 4, 3, 2};
    return tq >= 2 ? chunk_width(NQf, pref2, 4) : chunk_width(NQf, pref1, 4);
}

// tq: quad rows per backward thread (the backward's column chunks depend on it).
static Geo2d device_geo(const Conv2dGeom& c, int tq) {
    Geo2d g;
    g.T = (int32_t)c.T; g.F = (int32_t)c.F; g.C = (int32_t)c.C;
    g.To = (int32_t)c.To; g.Fo = (int32_t)c.Fo;
    g.dt = (int32_t)(c.pt0 - 1); g.df = (int32_t)(c.pf0 - 1);
    g.len_add = (int32_t)(c.pt0 + c.pt1 - 3);
    // Quads pair x rows 2m, 2m+1 and columns 2n, 2n+1.  Every g row is row
    // m of some quad: NQt = max(ceil(T/2), T').  With one column of padding
    // before, every g column is column n of some quad likewise; with two,
    // F' can be ceil(F/2) + 1 and the last g column is added to db apart
    // (so that a row keeps ceil(F/2) quad columns, which chunk evenly).
    const int64_t nqt = (c.T + 1) / 2, nqf = (c.F + 1) / 2;
    g.NQt = (int32_t)(nqt > c.To ? nqt : c.To);
    if (g.df == 0) {
        g.NQf = (int32_t)(nqf > c.Fo ? nqf : c.Fo);
    } else {
        int64_t q = nqf > c.Fo - 1 ? nqf : c.Fo - 1;
        if (q == 0 && c.Fo > 0) q = 1;
        g.NQf = (int32_t)q;
    }
    g.fcols = fwd_cols(c.Fo);
    g.qcols = bwd_qcols(g.NQf, tq);
    g.nqc = g.NQf > 0 ? (g.NQf + g.qcols - 1) / g.qcols : 1;
    return g;
}

bool dwconv2d_fits(int64_t B, const Conv2dGeom& g, int elem_bytes) {
    // Per-item byte offsets (with two rows of slack on each side) must stay
    // within a signed 32-bit range, and the row groups within 32 bits.
    constexpr int64_t lim = (int64_t)1 << 31;
    if (!product_below(lim, {g.T + 4, g.F, g.C, elem_bytes})) return false;
    if (!product_below(lim, {g.To + 4, g.Fo + 2, g.C, elem_bytes})) return false;
    if (!product_below(lim, {g.F + 4, g.C, elem_bytes})) return false;
    return (uint64_t)B * (uint64_t)(g.T / 2 + 2) * (uint64_t)(g.F / 2 + 2) < ((uint64_t)1 << 31);
}

template <typename S, int V, int LANES>
static hipError_t launch_fwd_lanes(const S* x, const S* w, const S* bias, const int32_t* lengths, S* y, int64_t B,
                                   const Conv2dGeom& c, hipStream_t st) {
    constexpr uint32_t kRB = kBlock2d / LANES;
    const Geo2d geo = device_geo(c, 1);
    const int64_t nfc = (c.Fo + geo.fcols - 1) / geo.fcols;
    const uint32_t n_rb = (uint32_t)(((c.To + kFwdRows - 1) / kFwdRows) * nfc);
    const uint32_t CG = (uint32_t)(c.C / V);
    const uint32_t n_cblk = (CG + LANES - 1) / LANES;
    const uint32_t gpi = (n_rb + kRB - 1) / kRB;  // row groups per item
    const uint64_t ng = (uint64_t)B * gpi;
    if (ng == 0 || n_cblk == 0) return hipSuccess;
    const uint64_t blocks = (ng < DW2D_FWD_PERSIST ? ng : DW2D_FWD_PERSIST) * n_cblk;
    hipLaunchKernelGGL((dwconv2d_fwd_kernel<S, V, kFwdRows, LANES>), dim3((uint32_t)blocks), dim3(kBlock2d), 0, st,
                       x, w, bias, lengths, y, geo, (int32_t)B, n_rb, CG, n_cblk, gpi);
    return hipGetLastError();
}

template <typename S, int V>
static hipError_t launch_fwd_typed(const S* x, const S* w, const S* bias, const int32_t* lengths, S* y, int64_t B,
                                   const Conv2dGeom& c, hipStream_t st) {
    if (c.C / V <= 32) return launch_fwd_lanes<S, V, 32>(x, w, bias, lengths, y, B, c, st);
    return launch_fwd_lanes<S, V, 64>(x, w, bias, lengths, y, B, c, st);
}

template <typename S>
static hipError_t launch_fwd_s(const void* x, const void* w, const void* bias, const int32_t* lengths, void* y,
                               int64_t B, const Conv2dGeom& c, int vec, hipStream_t st) {
    const S* xs = (const S*)x;
    const S* ws = (const S*)w;
    const S* bs = (const S*)bias;
    S* ys = (S*)y;
    switch (vec) {
        case 8:
            if constexpr (sizeof(S) == 2 && DW2D_FWD_BF16_VEC >= 8)
                return launch_fwd_typed<S, 8>(xs, ws, bs, lengths, ys, B, c, st);
            return launch_fwd_typed<S, 4>(xs, ws, bs, lengths, ys, B, c, st);
        case 4: return launch_fwd_typed<S, 4>(xs, ws, bs, lengths, ys, B, c, st);
        case 2: return launch_fwd_typed<S, 2>(xs, ws, bs, lengths, ys, B, c, st);
        default: return launch_fwd_typed<S, 1>(xs, ws, bs, lengths, ys, B, c, st);
    }
}

hipError_t launch_dwconv2d_fwd(const void* x, const void* w, const void* bias, const int32_t* lengths, void* y,
                               int64_t B, const Conv2dGeom& c, bool bf16, int vec, hipStream_t st) {
    return bf16 ? launch_fwd_s<uint16_t>(x, w, bias, lengths, y, B, c, vec, st)
                : launch_fwd_s<float>(x, w, bias, lengths, y, B, c, vec, st);
}

#ifndef DW2D_BWD_TARGET_WGS
#define DW2D_BWD_TARGET_WGS 256
#endif

// Backward grid: G workgroups per channel block share the batch's row groups
// round-robin.  G is about the number of workgroups the chip holds at once
// (2 per CU at this kernel's register use), so every workgroup runs for the
// whole kernel, and there are G dw/db partials to add up afterwards.  G does
// not depend on the vector width: the channel blocks of one workgroup index
// share a partial row.
struct BwdGrid {
    uint32_t n_rb, groups_per_item, n_groups, G;
    int64_t P;
};

static BwdGrid bwd_grid(int64_t B, const Geo2d& geo, int rows) {
    BwdGrid g;  // geo: device_geo(c, rows)
    g.n_rb = (uint32_t)((geo.NQt + rows - 1) / rows) * (uint32_t)geo.nqc;
    g.groups_per_item = (g.n_rb + kRowsPerBlock - 1) / kRowsPerBlock;
    const int64_t n = B * (int64_t)g.groups_per_item;
    g.n_groups = (uint32_t)n;
    g.G = (uint32_t)(n < DW2D_BWD_TARGET_WGS ? n : DW2D_BWD_TARGET_WGS);
    g.P = g.G;
    return g;
}

size_t dwconv2d_bwd_workspace(int64_t B, const Conv2dGeom& c) {
    // [P][10][C] workgroup partials, then [chunks][10][C] chunk sums, fp64
    // (sized for either storage type's grid).
    constexpr int r1 = bwd_rows<float>(), r2 = bwd_rows<uint16_t>();
    const int64_t P1 = bwd_grid(B, device_geo(c, r1), r1).P, P2 = bwd_grid(B, device_geo(c, r2), r2).P;
    const int64_t P = P1 > P2 ? P1 : P2;
    const int64_t rows = P + (partial_reduce_chunks(P) > 0 ? partial_reduce_chunks(P) : 1);
    return (size_t)(rows * 10 * c.C * (int64_t)sizeof(double));
}

template <typename S, int V, bool PAIR = false>
static hipError_t launch_bwd_typed(const S* x, const S* w, const int32_t* lengths, const S* dy, S* dx, float* dw,
                                   float* db, double* partial, int64_t B, const Conv2dGeom& c, hipStream_t st) {
    constexpr int TQ = bwd_rows<S>();
    const Geo2d geo = device_geo(c, TQ);
    const BwdGrid g = bwd_grid(B, geo, TQ);
    const uint32_t CG = (uint32_t)(c.C / V);
    const uint32_t n_cblk = (CG + kLanes2d - 1) / kLanes2d;
    const uint64_t blocks = (uint64_t)g.G * n_cblk;
    if (blocks > 0 && (dx || partial)) {
        const dim3 grid((uint32_t)blocks), block(kBlock2d);
        if (geo.dt == 0 && geo.df == 0)
            hipLaunchKernelGGL((dwconv2d_bwd_kernel<S, V, TQ, 0, 0, PAIR>), grid, block, 0, st, x, w, lengths, dy, dx,
                               partial, geo, g.n_rb, CG, n_cblk, g.groups_per_item, g.n_groups);
        else if (geo.dt == 1 && geo.df == 1)
            hipLaunchKernelGGL((dwconv2d_bwd_kernel<S, V, TQ, 1, 1, PAIR>), grid, block, 0, st, x, w, lengths, dy, dx,
                               partial, geo, g.n_rb, CG, n_cblk, g.groups_per_item, g.n_groups);
        else if (geo.dt == 1)
            hipLaunchKernelGGL((dwconv2d_bwd_kernel<S, V, TQ, 1, 0, PAIR>), grid, block, 0, st, x, w, lengths, dy, dx,
                               partial, geo, g.n_rb, CG, n_cblk, g.groups_per_item, g.n_groups);
        else
            hipLaunchKernelGGL((dwconv2d_bwd_kernel<S, V, TQ, 0, 1, PAIR>), grid, block, 0, st, x, w, lengths, dy, dx,
                               partial, geo, g.n_rb, CG, n_cblk, g.groups_per_item, g.n_groups);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (dw || db) {
        RowOutputs out = {};
        out.n = 2;
        out.p[0] = dw; out.first[0] = 0; out.count[0] = 9;
        out.p[1] = db; out.first[1] = 9; out.count[1] = 1;
        return launch_partial_reduce(partial, g.P, 10, c.C, partial + g.P * 10 * c.C, out, st);
    }
    return hipSuccess;
}

#ifndef DW2D_BWD_VEC
#define DW2D_BWD_VEC 8
#endif

template <typename S>
static hipError_t launch_bwd_s(const void* x, const void* w, const int32_t* lengths, const void* dy, void* dx,
                               float* dw, float* db, double* partial, int64_t B, const Conv2dGeom& c, int vec,
                               hipStream_t st) {
    const S* xs = (const S*)x;
    const S* ws = (const S*)w;
    const S* gs = (const S*)dy;
    S* dxs = (S*)dx;
    if (vec > DW2D_BWD_VEC) vec = DW2D_BWD_VEC;
    switch (vec) {
        case 8:  // bf16 only: 16-byte x and dx accesses through paired lanes
            if constexpr (sizeof(S) == 2)
                return launch_bwd_typed<S, 4, true>(xs, ws, lengths, gs, dxs, dw, db, partial, B, c, st);
            return launch_bwd_typed<S, 4>(xs, ws, lengths, gs, dxs, dw, db, partial, B, c, st);
        case 4: return launch_bwd_typed<S, 4>(xs, ws, lengths, gs, dxs, dw, db, partial, B, c, st);
        case 2: return launch_bwd_typed<S, 2>(xs, ws, lengths, gs, dxs, dw, db, partial, B, c, st);
        default: return launch_bwd_typed<S, 1>(xs, ws, lengths, gs, dxs, dw, db, partial, B, c, st);
    }
}

hipError_t launch_dwconv2d_bwd(const void* x, const void* w, const int32_t* lengths, const void* dy, void* dx,
                               float* dw, float* db, void* workspace, int64_t B, const Conv2dGeom& c, bool bf16,
                               int vec, hipStream_t st) {
    double* partial = (dw || db) ? (double*)workspace : nullptr;
    return bf16 ? launch_bwd_s<uint16_t>(x, w, lengths, dy, dx, dw, db, partial, B, c, vec, st)
                : launch_bwd_s<float>(x, w, lengths, dy, dx, dw, db, partial, B, c, vec, st);
}

}  // namespace dw
