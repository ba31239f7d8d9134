// Depthwise conv2d, 3x3, stride 2, pad 1, forward and backward, for gfx950
// (NeMo PR #16114, "What does this PR do": the general depthwise conv2d with
// the pre- and post-masking fused into the kernel, and its backward).
//
// Layout: x, dx [B][T][F][C], y, dy [B][T'][F'][C] with T' = ceil(T/2),
// F' = ceil(F/2); w [3][3][C]; channel fastest.
//
// Masks through buffer resources: each item's x is read through a resource
// that ends at its valid length (rows t >= len read as zero: the pre-mask)
// and dy through one that ends at len' = ceil(len/2) (masked gradient rows
// read as zero), and a negative row offset is out of range as well, which
// gives the top padding row.  Only the frequency padding (column -1, and
// column F when F is odd) needs an explicit zero.
//
// Forward mapping.  A thread owns V channels of TO consecutive output rows of
// one item and walks left to right over the F' output columns (or a chunk of
// them).  At output
// column f' it needs input columns 2f'-1, 2f', 2f'+1 of the 2*TO+1 input rows
// 2t0-1 .. 2t0+2*TO-1; column 2f'+1 is carried to the next step as its
// column 2(f'+1)-1, so every input element is loaded once per thread, and
// the one input row shared with the next row block comes from L2.
//
// Backward mapping.  dx is gathered, not scattered: output-parity phases.
// With x rows 2t', 2t'+1 and columns 2f', 2f'+1 as one "quad" (t', f'):
//   dx[2t',  2f'  ] = g[t',f'] w11
//   dx[2t',  2f'+1] = g[t',f'] w12 + g[t',f'+1] w10
//   dx[2t'+1,2f'  ] = g[t',f'] w21 + g[t'+1,f'] w01
//   dx[2t'+1,2f'+1] = g[t',f'] w22 + g[t',f'+1] w20 + g[t'+1,f'] w02 + g[t'+1,f'+1] w00
// and the same (g, x) pairs give the weight gradient: each pair above adds
// g * x(quad element) to the tap it multiplies.  Every (input, output) pair
// of the convolution belongs to exactly one quad, so dw is complete and no
// pair is counted twice; db adds g[t',f'] once per quad.  A thread walks one
// row block of quads left to right, carrying the g column f'+1.  dw and db
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
#define DW2D_FWD_PERSIST 512  // workgroups of a persistent forward grid; 0 = one workgroup per tile
#endif
#ifndef DW2D_FWD_COLS
#define DW2D_FWD_COLS 8  // output columns per thread in the forward; 0 = all of them
#endif
#ifndef DW2D_BWD_ROWS
#define DW2D_BWD_ROWS 1
#endif
constexpr int kFwdRows = DW2D_FWD_ROWS;   // output rows per thread (forward)
constexpr int kFwdCols = DW2D_FWD_COLS;   // output columns per thread (forward), 0 = all
constexpr int kBwdRows = DW2D_BWD_ROWS;   // quad rows per thread (backward)

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

// Block decode shared by the forward and backward kernels: the workgroup is
// kRowsPerBlock row blocks x kLanes2d channel groups of one item.
struct Tile2d {
    uint32_t b, rb, cg;
    bool valid;
};

__device__ __forceinline__ Tile2d decode_2d(uint32_t n_rb, uint32_t CG, uint32_t n_cblk, uint32_t wg_per_item) {
    const uint32_t blk = xcd_contiguous_block(blockIdx.x, gridDim.x);
    Tile2d d;
    d.b = blk / wg_per_item;
    const uint32_t r = blk - d.b * wg_per_item;
    const uint32_t rgroup = r / n_cblk, cblk = r - rgroup * n_cblk;
    d.rb = rgroup * kRowsPerBlock + threadIdx.x / kLanes2d;
    d.cg = cblk * kLanes2d + threadIdx.x % kLanes2d;
    d.valid = d.rb < n_rb && d.cg < CG;
    return d;
}

// ------------------------------------------------------------------ fwd ----

template <int V, int TO>
__global__ __launch_bounds__(kBlock2d) void dwconv2d_fwd_kernel(
    const float* __restrict__ x, const float* __restrict__ w, const float* __restrict__ bias,
    const int32_t* __restrict__ lengths, float* __restrict__ y, int32_t B_items,
    int32_t T, int32_t F, int32_t C, int32_t To, int32_t Fo,
    uint32_t n_rb, uint32_t CG, uint32_t n_cblk, uint32_t wg_per_item) {
#if DW2D_FWD_PERSIST
    // wg_per_item here is the number of row groups per item; the batch's row
    // groups are dealt round-robin to the workgroups of a channel block.
    const uint32_t blk0 = xcd_contiguous_block(blockIdx.x, gridDim.x);
    const uint32_t G = gridDim.x / n_cblk;
    const uint32_t g0 = blk0 / n_cblk, cb0 = blk0 - g0 * n_cblk;
    for (uint32_t j = g0; j < (uint32_t)B_items * wg_per_item; j += G) {
    Tile2d d;
    d.b = j / wg_per_item;
    d.rb = (j - d.b * wg_per_item) * kRowsPerBlock + threadIdx.x / kLanes2d;
    d.cg = cb0 * kLanes2d + threadIdx.x % kLanes2d;
    d.valid = d.rb < n_rb && d.cg < CG;
    if (!d.valid) continue;
#else
    const Tile2d d = decode_2d(n_rb, CG, n_cblk, wg_per_item);
    if (!d.valid) return;
#endif
    const int32_t len = (int32_t)item_length(lengths, d.b, T);
    const int32_t leno = (len + 1) / 2;
    const uint32_t xrow = (uint32_t)F * C * 4, yrow = (uint32_t)Fo * C * 4, pix = (uint32_t)C * 4;
    const rsrc_t xr = make_rsrc(x + (int64_t)d.b * T * F * C, (uint32_t)len * xrow);
    const rsrc_t yr = make_rsrc(y + (int64_t)d.b * To * Fo * C, (uint32_t)To * yrow);
    const int32_t c0 = (int32_t)d.cg * V;
    const uint32_t coff = (uint32_t)c0 * 4;
    // row-block index = row block * column chunks + column chunk
    const int32_t fch = kFwdCols > 0 ? kFwdCols : Fo;
    const int32_t nfc = (Fo + fch - 1) / fch;
    const int32_t t0 = (int32_t)(d.rb / nfc) * TO;
    const int32_t fa = (int32_t)(d.rb % nfc) * fch, fb = min(Fo, fa + fch);

    if (t0 >= leno) {
        const Vf<V> z = vzero<V>();
        for (int32_t f = fa; f < fb; ++f)
#pragma unroll
            for (int i = 0; i < TO; ++i) Buf<float, V>::store(yr, (uint32_t)(t0 + i) * yrow + f * pix + coff, z);
#if DW2D_FWD_PERSIST
        continue;
#else
        return;
#endif
    }

    Vf<V> wk[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) wk[k] = load_param<float, V>(w + (int64_t)k * C + c0);
    const Vf<V> bv = bias ? load_param<float, V>(bias + c0) : vzero<V>();

    // Input rows 2t0-1+r, r = 0 .. 2*TO; byte offset of each row start (a
    // negative row wraps out of range and reads zero).
    uint32_t roff[2 * TO + 1];
#pragma unroll
    for (int r = 0; r < 2 * TO + 1; ++r) roff[r] = (uint32_t)((2 * t0 - 1 + r) * (int32_t)xrow) + coff;

    Vf<V> carry[2 * TO + 1];  // input column 2f'-1 (zero left of the first column)
#pragma unroll
    for (int r = 0; r < 2 * TO + 1; ++r)
        carry[r] = fa > 0 ? Buf<float, V>::load(xr, roff[r] + (uint32_t)(2 * fa - 1) * pix) : vzero<V>();

    for (int32_t f = fa; f < fb; ++f) {
        const uint32_t c_even = (uint32_t)(2 * f) * pix;
        const bool odd_ok = 2 * f + 1 < F;  // column 2f'+1 exists
        Vf<V> ce[2 * TO + 1], co[2 * TO + 1];
#pragma unroll
        for (int r = 0; r < 2 * TO + 1; ++r) {
            ce[r] = Buf<float, V>::load(xr, roff[r] + c_even);
            co[r] = Buf<float, V>::load(xr, roff[r] + c_even + pix);
        }
#pragma unroll
        for (int r = 0; r < 2 * TO + 1; ++r) co[r] = select_v<V>(odd_ok, co[r]);
#pragma unroll
        for (int i = 0; i < TO; ++i) {
            Vf<V> acc = bv;
#pragma unroll
            for (int a = 0; a < 3; ++a) {
                fma_v<V>(acc, carry[2 * i + a], wk[3 * a + 0]);
                fma_v<V>(acc, ce[2 * i + a], wk[3 * a + 1]);
                fma_v<V>(acc, co[2 * i + a], wk[3 * a + 2]);
            }
            acc = select_v<V>(t0 + i < leno, acc);
            Buf<float, V>::store(yr, (uint32_t)(t0 + i) * yrow + f * pix + coff, acc);
        }
#pragma unroll
        for (int r = 0; r < 2 * TO + 1; ++r) carry[r] = co[r];
    }
#if DW2D_FWD_PERSIST
    }  // row groups
#endif
}

#ifdef DW2D_FWD_PIXEL
// Experimental: one output pixel (V channels) per thread, 9 loads through L2.
template <int V>
__global__ __launch_bounds__(kBlock2d) void dwconv2d_fwd_pixel_kernel(
    const float* __restrict__ x, const float* __restrict__ w, const float* __restrict__ bias,
    const int32_t* __restrict__ lengths, float* __restrict__ y,
    int32_t T, int32_t F, int32_t C, int32_t To, int32_t Fo, uint32_t CG, uint32_t blocks_per_item) {
    const uint32_t blk = xcd_contiguous_block(blockIdx.x, gridDim.x);
    const uint32_t b = blk / blocks_per_item;
    const uint32_t local = (blk - b * blocks_per_item) * kBlock2d + threadIdx.x;
    const uint32_t pixel = local / CG, cg = local - pixel * CG;
    if (pixel >= (uint32_t)(To * Fo)) return;
    const int32_t to = (int32_t)(pixel / Fo), fo = (int32_t)(pixel % Fo);
    const int32_t len = (int32_t)item_length(lengths, b, T);
    const int32_t leno = (len + 1) / 2;
    const uint32_t xrow = (uint32_t)F * C * 4, pix = (uint32_t)C * 4;
    const rsrc_t xr = make_rsrc(x + (int64_t)b * T * F * C, (uint32_t)len * xrow);
    const rsrc_t yr = make_rsrc(y + (int64_t)b * To * Fo * C, (uint32_t)To * Fo * pix);
    const int32_t c0 = (int32_t)cg * V;
    const uint32_t coff = (uint32_t)c0 * 4;
    const uint32_t yo = (uint32_t)pixel * pix + coff;
    if (to >= leno) { Buf<float, V>::store(yr, yo, vzero<V>()); return; }
    Vf<V> xv[9];
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int32_t f = 2 * fo + j - 1;
            xv[3 * i + j] = Buf<float, V>::load(xr, (uint32_t)((2 * to + i - 1) * (int32_t)xrow + f * (int32_t)pix) + coff);
            if (f < 0 || f >= F) xv[3 * i + j] = vzero<V>();
        }
    Vf<V> acc = bias ? load_param<float, V>(bias + c0) : vzero<V>();
#pragma unroll
    for (int k = 0; k < 9; ++k) fma_v<V>(acc, xv[k], load_param<float, V>(w + (int64_t)k * C + c0));
    Buf<float, V>::store(yr, yo, acc);
}
#endif

// ------------------------------------------------------------------ bwd ----

template <int V, int TQ>
__global__ __launch_bounds__(kBlock2d) void dwconv2d_bwd_kernel(
    const float* __restrict__ x, const float* __restrict__ w, const int32_t* __restrict__ lengths,
    const float* __restrict__ dy, float* __restrict__ dx, double* __restrict__ partial,
    int32_t T, int32_t F, int32_t C, int32_t To, int32_t Fo,
    uint32_t n_rb, uint32_t CG, uint32_t n_cblk, uint32_t groups_per_item, uint32_t n_groups) {
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
    const uint32_t cg = cblk * kLanes2d + threadIdx.x % kLanes2d;
    const int32_t c0 = (int32_t)cg * V;

    double gw[9][V], gb[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
        gb[e] = 0.0;
#pragma unroll
        for (int k = 0; k < 9; ++k) gw[k][e] = 0.0;
    }

    for (uint32_t j = g; j < n_groups; j += G) {
    Tile2d d;
    d.b = j / groups_per_item;
    d.cg = cg;
    d.rb = (j - d.b * groups_per_item) * kRowsPerBlock + threadIdx.x / kLanes2d;
    d.valid = d.rb < n_rb && d.cg < CG;
    if (d.valid) {
        const int32_t len = (int32_t)item_length(lengths, d.b, T);
        const int32_t leno = (len + 1) / 2;
        const uint32_t xrow = (uint32_t)F * C * 4, grow = (uint32_t)Fo * C * 4, pix = (uint32_t)C * 4;
        const int64_t xitem = (int64_t)d.b * T * F * C;
        const rsrc_t xr = make_rsrc(x + xitem, (uint32_t)len * xrow);
        const rsrc_t gr = make_rsrc(dy + (int64_t)d.b * To * Fo * C, (uint32_t)leno * grow);
        const rsrc_t dxr = make_rsrc(dx ? dx + xitem : x, dx ? (uint32_t)T * xrow : 0u);
        const uint32_t coff = (uint32_t)c0 * 4;
        const int32_t t0 = (int32_t)d.rb * TQ;  // first quad row

        if (2 * t0 >= len) {
            // Every x row of this block is masked, so is every g row it
            // touches: dx is zero and nothing adds to dw or db.
            if (dx) {
                const Vf<V> z = vzero<V>();
                for (int32_t f = 0; f < F; ++f)
#pragma unroll
                    for (int r = 0; r < 2 * TQ; ++r)
                        Buf<float, V>::store(dxr, (uint32_t)(2 * t0 + r) * xrow + f * pix + coff, z);
            }
        } else {
            Vf<V> wk[9];
#pragma unroll
            for (int k = 0; k < 9; ++k) wk[k] = load_param<float, V>(w + (int64_t)k * C + c0);
            // g rows t0 .. t0+TQ (the last one belongs to the next block).
            Vf<V> gcur[TQ + 1];
#pragma unroll
            for (int q = 0; q <= TQ; ++q)
                gcur[q] = Buf<float, V>::load(gr, (uint32_t)((t0 + q) * (int32_t)grow) + coff);
            for (int32_t f = 0; f < Fo; ++f) {
                const bool next_ok = f + 1 < Fo;      // g column f'+1 exists
                const bool odd_ok = 2 * f + 1 < F;    // x column 2f'+1 exists
                Vf<V> gnext[TQ + 1], xe[2 * TQ], xo[2 * TQ];
#pragma unroll
                for (int q = 0; q <= TQ; ++q)
                    gnext[q] = Buf<float, V>::load(gr, (uint32_t)((t0 + q) * (int32_t)grow) + (f + 1) * pix + coff);
#pragma unroll
                for (int r = 0; r < 2 * TQ; ++r) {
                    const uint32_t ro = (uint32_t)(2 * t0 + r) * xrow + (uint32_t)(2 * f) * pix + coff;
                    xe[r] = Buf<float, V>::load(xr, ro);
                    xo[r] = Buf<float, V>::load(xr, ro + pix);
                }
#pragma unroll
                for (int q = 0; q <= TQ; ++q) gnext[q] = select_v<V>(next_ok, gnext[q]);
#pragma unroll
                for (int r = 0; r < 2 * TQ; ++r) xo[r] = select_v<V>(odd_ok, xo[r]);
#pragma unroll
                for (int q = 0; q < TQ; ++q) {
                    const Vf<V>& g00 = gcur[q];       // g[t', f']
                    const Vf<V>& g01 = gnext[q];      // g[t', f'+1]
                    const Vf<V>& g10 = gcur[q + 1];   // g[t'+1, f']
                    const Vf<V>& g11 = gnext[q + 1];  // g[t'+1, f'+1]
                    const Vf<V>& x00 = xe[2 * q];
                    const Vf<V>& x01 = xo[2 * q];
                    const Vf<V>& x10 = xe[2 * q + 1];
                    const Vf<V>& x11 = xo[2 * q + 1];
                    // tap index k = 3*i + j of w[i][j]
                    Vf<V> d00 = vzero<V>(), d01 = vzero<V>(), d10 = vzero<V>(), d11 = vzero<V>();
                    fma_v<V>(d00, g00, wk[4]);
                    fma_v<V>(d01, g00, wk[5]); fma_v<V>(d01, g01, wk[3]);
                    fma_v<V>(d10, g00, wk[7]); fma_v<V>(d10, g10, wk[1]);
                    fma_v<V>(d11, g00, wk[8]); fma_v<V>(d11, g01, wk[6]);
                    fma_v<V>(d11, g10, wk[2]); fma_v<V>(d11, g11, wk[0]);
                    fma_d<V>(gw[4], g00, x00);
                    fma_d<V>(gw[5], g00, x01); fma_d<V>(gw[3], g01, x01);
                    fma_d<V>(gw[7], g00, x10); fma_d<V>(gw[1], g10, x10);
                    fma_d<V>(gw[8], g00, x11); fma_d<V>(gw[6], g01, x11);
                    fma_d<V>(gw[2], g10, x11); fma_d<V>(gw[0], g11, x11);
#pragma unroll
                    for (int e = 0; e < V; ++e) gb[e] += (double)g00.v[e];
                    if (dx) {
                        const int32_t te = 2 * (t0 + q);
                        const uint32_t o = (uint32_t)te * xrow + (uint32_t)(2 * f) * pix + coff;
                        Buf<float, V>::store(dxr, o, select_v<V>(te < len, d00));
                        Buf<float, V>::store(dxr, o + xrow, select_v<V>(te + 1 < len, d10));
                        if (odd_ok) {
                            Buf<float, V>::store(dxr, o + pix, select_v<V>(te < len, d01));
                            Buf<float, V>::store(dxr, o + xrow + pix, select_v<V>(te + 1 < len, d11));
                        }
                    }
                }
#pragma unroll
                for (int q = 0; q <= TQ; ++q) gcur[q] = gnext[q];
            }
        }
    }

    }  // row groups

    if (!partial) return;  // uniform: dw and db not requested
    // Sum the row blocks of this workgroup in a fixed order (row block 0
    // first), then write one partial per workgroup: partial[p][k][c], k = 0..8
    // the taps, 9 the bias.
    const uint32_t lane = threadIdx.x % kLanes2d, rsub = threadIdx.x / kLanes2d;
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
        const int32_t c = ((int32_t)cblk * kLanes2d + (int32_t)lane) * V + e;
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

struct Grid2d {
    uint32_t n_rb, CG, n_cblk, wg_per_item;
    uint64_t blocks;
};

static Grid2d grid_2d(int64_t B, int64_t rows, int rows_per_thread, int64_t C, int vec) {
    Grid2d g;
    g.n_rb = (uint32_t)((rows + rows_per_thread - 1) / rows_per_thread);
    g.CG = (uint32_t)(C / vec);
    g.n_cblk = (g.CG + kLanes2d - 1) / kLanes2d;
    const uint32_t rgroups = (g.n_rb + kRowsPerBlock - 1) / kRowsPerBlock;
    g.wg_per_item = rgroups * g.n_cblk;
    g.blocks = (uint64_t)B * g.wg_per_item;
    return g;
}

bool dwconv2d_fits(int64_t B, int64_t T, int64_t F, int64_t C, int vec) {
    // Per-item byte offsets (with one row of slack on each side) must stay
    // within a signed 32-bit range.
    if ((T + 2) * F * C * 4 >= ((int64_t)1 << 31)) return false;
    const int64_t To = (T + 1) / 2;
    const Grid2d g = grid_2d(B, To, 1, C, vec);
    return g.blocks < ((uint64_t)1 << 31);
}

template <int V>
static hipError_t launch_fwd_typed(const float* x, const float* w, const float* bias, const int32_t* lengths,
                                   float* y, int64_t B, int64_t T, int64_t F, int64_t C, hipStream_t st) {
    const int64_t To = (T + 1) / 2, Fo = (F + 1) / 2;
#ifdef DW2D_FWD_PIXEL
    {
        const uint32_t CG = (uint32_t)(C / V);
        const uint32_t bpi = (uint32_t)(((uint64_t)To * Fo * CG + kBlock2d - 1) / kBlock2d);
        hipLaunchKernelGGL((dwconv2d_fwd_pixel_kernel<V>), dim3((uint32_t)(B * bpi)), dim3(kBlock2d), 0, st, x, w,
                           bias, lengths, y, (int32_t)T, (int32_t)F, (int32_t)C, (int32_t)To, (int32_t)Fo, CG, bpi);
        return hipGetLastError();
    }
#endif
    const int64_t nfc = kFwdCols > 0 ? (Fo + kFwdCols - 1) / kFwdCols : 1;
    Grid2d g = grid_2d(B, To, kFwdRows, C, V);
    if (nfc > 1) g = grid_2d(B, ((To + kFwdRows - 1) / kFwdRows) * nfc * kFwdRows, kFwdRows, C, V);
#if DW2D_FWD_PERSIST
    const uint32_t gpi = g.wg_per_item / g.n_cblk;  // row groups per item
    const uint64_t ng = (uint64_t)B * gpi;
    g.blocks = (ng < DW2D_FWD_PERSIST ? ng : DW2D_FWD_PERSIST) * g.n_cblk;
    g.wg_per_item = gpi;
#endif
    hipLaunchKernelGGL((dwconv2d_fwd_kernel<V, kFwdRows>), dim3((uint32_t)g.blocks), dim3(kBlock2d), 0, st, x, w,
                       bias, lengths, y, (int32_t)B, (int32_t)T, (int32_t)F, (int32_t)C, (int32_t)To, (int32_t)Fo,
                       g.n_rb, g.CG, g.n_cblk, g.wg_per_item);
    return hipGetLastError();
}

hipError_t launch_dwconv2d_fwd(const float* x, const float* w, const float* bias, const int32_t* lengths,
                               float* y, int64_t B, int64_t T, int64_t F, int64_t C, int vec, hipStream_t st) {
    switch (vec) {
        case 4: return launch_fwd_typed<4>(x, w, bias, lengths, y, B, T, F, C, st);
        case 2: return launch_fwd_typed<2>(x, w, bias, lengths, y, B, T, F, C, st);
        default: return launch_fwd_typed<1>(x, w, bias, lengths, y, B, T, F, C, st);
    }
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

static BwdGrid bwd_grid(int64_t B, int64_t T) {
    BwdGrid g;
    const int64_t To = (T + 1) / 2;
    g.n_rb = (uint32_t)((To + kBwdRows - 1) / kBwdRows);
    g.groups_per_item = (g.n_rb + kRowsPerBlock - 1) / kRowsPerBlock;
    const int64_t n = B * (int64_t)g.groups_per_item;
    g.n_groups = (uint32_t)n;
    g.G = (uint32_t)(n < DW2D_BWD_TARGET_WGS ? n : DW2D_BWD_TARGET_WGS);
    g.P = g.G;
    return g;
}

size_t dwconv2d_bwd_workspace(int64_t B, int64_t T, int64_t F, int64_t C) {
    (void)F;
    // [P][10][C] workgroup partials, then [chunks][10][C] chunk sums, fp64.
    const int64_t P = bwd_grid(B, T).P;
    const int64_t rows = P + (partial_reduce_chunks(P) > 0 ? partial_reduce_chunks(P) : 1);
    return (size_t)(rows * 10 * C * (int64_t)sizeof(double));
}

template <int V>
static hipError_t launch_bwd_typed(const float* x, const float* w, const int32_t* lengths, const float* dy,
                                   float* dx, float* dw, float* db, double* partial, int64_t B, int64_t T,
                                   int64_t F, int64_t C, hipStream_t st) {
    const int64_t To = (T + 1) / 2, Fo = (F + 1) / 2;
    const BwdGrid g = bwd_grid(B, T);
    const uint32_t CG = (uint32_t)(C / V);
    const uint32_t n_cblk = (CG + kLanes2d - 1) / kLanes2d;
    const uint64_t blocks = (uint64_t)g.G * n_cblk;
    if (blocks > 0 && (dx || partial)) {
        hipLaunchKernelGGL((dwconv2d_bwd_kernel<V, kBwdRows>), dim3((uint32_t)blocks), dim3(kBlock2d), 0, st, x,
                           w, lengths, dy, dx, partial, (int32_t)T, (int32_t)F, (int32_t)C, (int32_t)To,
                           (int32_t)Fo, g.n_rb, CG, n_cblk, g.groups_per_item, g.n_groups);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (dw || db) {
        RowOutputs out = {};
        out.n = 2;
        out.p[0] = dw; out.first[0] = 0; out.count[0] = 9;
        out.p[1] = db; out.first[1] = 9; out.count[1] = 1;
        return launch_partial_reduce(partial, g.P, 10, C, partial + g.P * 10 * C, out, st);
    }
    return hipSuccess;
}

#ifndef DW2D_BWD_VEC
#define DW2D_BWD_VEC 4
#endif

hipError_t launch_dwconv2d_bwd(const float* x, const float* w, const int32_t* lengths, const float* dy,
                               float* dx, float* dw, float* db, void* workspace, int64_t B, int64_t T,
                               int64_t F, int64_t C, int vec, hipStream_t st) {
    double* partial = (dw || db) ? (double*)workspace : nullptr;
    if (vec > DW2D_BWD_VEC) vec = DW2D_BWD_VEC;
    switch (vec) {
        case 4: return launch_bwd_typed<4>(x, w, lengths, dy, dx, dw, db, partial, B, T, F, C, st);
        case 2: return launch_bwd_typed<2>(x, w, lengths, dy, dx, dw, db, partial, B, T, F, C, st);
        default: return launch_bwd_typed<1>(x, w, lengths, dy, dx, dw, db, partial, B, T, F, C, st);
    }
}

}  // namespace dw
