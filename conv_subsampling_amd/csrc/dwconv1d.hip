// Depthwise Conv1d in SSM_CONV form for gfx950 (parakeet.cpp PR #102,
// "What changes": y[t, c] = sum_k x[t + k, c] * w[k, c] over the input
// padded to T + K - 1 frames, with per-item length masking).
//
// Mapping.  Each workgroup serves one batch item; within it, one thread owns
// V consecutive channels (one vector access) of TT consecutive output frames.
// Thread ids run channel-group fastest, so a wavefront's loads of one frame
// are contiguous in memory, and neighbouring time tiles of the same channels
// sit in the same or the next workgroup; blocks are renumbered so those land
// on one XCD and the K - 1 halo frames they share are served from its L2.
//
// Masking and padding cost nothing: the item's input is read through a
// buffer resource that ends at the item's valid length, so frames at or past
// the length, and the left padding (negative offsets), load as zero with no
// branch and no memory traffic; the output resource ends at T, so stores of
// a ragged last tile are dropped.  Per thread, the TT + K - 1 input frames
// the tile needs are loaded into a register window with back-to-back
// independent loads, the K taps slide over it with fp32 FMAs (the bias seeds
// each sum), and frames at or past the length are stored as exact zeros.  A
// tile that lies wholly past the length stores zeros without loading.
// Output uses non-temporal stores: nothing here reads it back.  fp32 at the
// compiled widths (3, 4, 5, 9, 15) with at least 32 channel groups stages the
// window through LDS instead: with 16-byte lanes a persistent workgroup
// streams its tiles through two LDS buffers (the persistent form below), with
// narrower lanes (a pointer off 16-byte alignment) each workgroup stages one
// tile (the LDS-staged form below).
#include "common.h"
#include "launch.h"

namespace dw {

constexpr int kBlock1d = 256;

struct Tile1d {
    uint32_t b, tile, cg;
    bool valid;
};

// Decode (item, time tile, channel group) from the block and thread index;
// the item depends on the block alone, so it is uniform across the wave.
__device__ __forceinline__ Tile1d decode_1d(uint32_t n_tiles, uint32_t CG, uint32_t blocks_per_item) {
    const uint32_t blk = xcd_contiguous_block(blockIdx.x, gridDim.x);
    Tile1d d;
    d.b = blk / blocks_per_item;
    const uint32_t local = (blk - d.b * blocks_per_item) * kBlock1d + threadIdx.x;
    d.tile = local / CG;
    d.cg = local - d.tile * CG;
    d.valid = d.tile < n_tiles;
    return d;
}

template <typename S, int V, int K, int TT>
__global__ __launch_bounds__(kBlock1d) void dwconv1d_fwd_kernel(
    const S* __restrict__ x, const S* __restrict__ w, const S* __restrict__ bias,
    const int32_t* __restrict__ lengths, S* __restrict__ y,
    int32_t T, int32_t C, int32_t pL, uint32_t n_tiles, uint32_t CG, uint32_t blocks_per_item) {
    const Tile1d d = decode_1d(n_tiles, CG, blocks_per_item);
    if (!d.valid) return;
    const int32_t len = (int32_t)item_length(lengths, d.b, T);
    const uint32_t row = (uint32_t)C * sizeof(S);
    const int64_t item = (int64_t)d.b * T * C;
    const rsrc_t xr = make_rsrc(x + item, (uint32_t)len * row);
    const rsrc_t yr = make_rsrc(y + item, (uint32_t)T * row);
    const int32_t c0 = (int32_t)d.cg * V;
    const uint32_t coff = (uint32_t)c0 * sizeof(S);
    const int32_t t0 = (int32_t)d.tile * TT;

    if (t0 >= len) {
        const Vf<V> z = vzero<V>();
#pragma unroll
        for (int i = 0; i < TT; ++i) Buf<S, V>::store(yr, (uint32_t)(t0 + i) * row + coff, z);
        return;
    }

    Vf<V> win[TT + K - 1];
#pragma unroll
    for (int r = 0; r < TT + K - 1; ++r)
        win[r] = Buf<S, V>::load(xr, (uint32_t)((t0 - pL + r) * (int32_t)row) + coff);
    Vf<V> wk[K];
#pragma unroll
    for (int k = 0; k < K; ++k) wk[k] = load_param<S, V>(w + (int64_t)k * C + c0);
    const Vf<V> bv = bias ? load_param<S, V>(bias + c0) : vzero<V>();

#pragma unroll
    for (int i = 0; i < TT; ++i) {
        Vf<V> acc = bv;
#pragma unroll
        for (int k = 0; k < K; ++k)
#pragma unroll
            for (int e = 0; e < V; ++e) acc.v[e] = __builtin_fmaf(win[i + k].v[e], wk[k].v[e], acc.v[e]);
        const bool keep = t0 + i < len;
#pragma unroll
        for (int e = 0; e < V; ++e) acc.v[e] = keep ? acc.v[e] : 0.0f;
        Buf<S, V>::store(yr, (uint32_t)(t0 + i) * row + coff, acc);
    }
}

// LDS-staged form, for the fp32 kernels: a workgroup owns TW output
// frames of 64 channel groups (one slab).  Its four waves stage the
// TW + K - 1 input frames the tile needs into LDS once (each wave a quarter
// of the rows, one vector per lane per row), then each wave computes TW / 4
// of the output frames from LDS.  The K - 1 halo frames are then read once
// per 32 output frames instead of once per thread tile: at K = 15 a thread
// tile of 12 frames reads 26, 2.2 times its share, against 1.4 times here
// (measured on MI355X at [32,1500,512]: K15 40.2 -> 37.5 us, K9 37.2 -> 36.7;
// in bf16 the register window stays ahead).
constexpr int kLdsTile1d = 32;
template <int V>
__device__ __forceinline__ void lds_put(float* p, const Vf<V>& a) {
    if constexpr (V == 4) {
        *reinterpret_cast<f32x4*>(p) = f32x4{a.v[0], a.v[1], a.v[2], a.v[3]};
    } else {
#pragma unroll
        for (int e = 0; e < V; ++e) p[e] = a.v[e];
    }
}
template <int V>
__device__ __forceinline__ Vf<V> lds_get(const float* p) {
    Vf<V> a;
    if constexpr (V == 4) {
        const f32x4 t = *reinterpret_cast<const f32x4*>(p);
        a.v[0] = t.x; a.v[1] = t.y; a.v[2] = t.z; a.v[3] = t.w;
    } else {
#pragma unroll
        for (int e = 0; e < V; ++e) a.v[e] = p[e];
    }
    return a;
}

template <typename S, int V, int K, int TW>
__global__ __launch_bounds__(kBlock1d) void dwconv1d_fwd_lds_kernel(
    const S* __restrict__ x, const S* __restrict__ w, const S* __restrict__ bias,
    const int32_t* __restrict__ lengths, S* __restrict__ y,
    int32_t T, int32_t C, int32_t pL, uint32_t n_ttiles, uint32_t n_slabs, uint32_t CG) {
    constexpr int R = TW + K - 1;            // staged frames
    constexpr int TT = TW / 4;               // output frames per wave
    constexpr int W = kBlock1d / 64;         // waves
    __shared__ __align__(16) float tile[R][64 * V];
    const uint32_t blk = xcd_contiguous_block(blockIdx.x, gridDim.x);
    const uint32_t slab = blk % n_slabs, rest = blk / n_slabs;
    const uint32_t tt = rest % n_ttiles, b = rest / n_ttiles;
    const int32_t len = (int32_t)item_length(lengths, b, T);
    const uint32_t row = (uint32_t)C * sizeof(S);
    const int64_t item = (int64_t)b * T * C;
    const rsrc_t yr = make_rsrc(y + item, (uint32_t)T * row);
    const uint32_t lane = threadIdx.x % 64, wv = threadIdx.x / 64;
    // Lanes past the last channel group (a partial last slab) address out of
    // range: their loads read zero and their stores are dropped.
    const bool active = slab * 64 + lane < CG;
    const int32_t c0 = active ? (int32_t)(slab * 64 + lane) * V : 0;
    const uint32_t coff = active ? (uint32_t)c0 * sizeof(S) : 0x80000000u;
    const int32_t t0 = (int32_t)tt * TW;
    const int32_t tw = t0 + (int32_t)wv * TT;  // this wave's first output frame
    if (t0 >= len) {  // uniform: the whole tile is past the length
        const Vf<V> z = vzero<V>();
#pragma unroll
        for (int i = 0; i < TT; ++i) Buf<S, V>::store(yr, (uint32_t)(tw + i) * row + coff, z);
        return;
    }
    const rsrc_t xr = make_rsrc(x + item, (uint32_t)len * row);
    // Taps first, then every staged row's load, all in flight together: a
    // row past the tile (only in the last round, where R is not a multiple
    // of the wave count) is loaded out of range and not written.
    Vf<V> wk[K];
#pragma unroll
    for (int k = 0; k < K; ++k) wk[k] = load_param<S, V>(w + (int64_t)k * C + c0);
    const Vf<V> bv = bias ? load_param<S, V>(bias + c0) : vzero<V>();
    constexpr int kRounds = (R + W - 1) / W;
    Vf<V> st[kRounds];
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
        const int r = (int)wv + W * j;
        const uint32_t ro = (R % W == 0 || r < R) ? (uint32_t)((t0 - pL + r) * (int32_t)row) + coff : 0x80000000u;
        st[j] = Buf<S, V>::load(xr, ro);
    }
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
        const int r = (int)wv + W * j;
        if (R % W == 0 || r < R) lds_put<V>(&tile[r][lane * V], st[j]);
    }
    __syncthreads();
    Vf<V> win[TT + K - 1];
#pragma unroll
    for (int r = 0; r < TT + K - 1; ++r) win[r] = lds_get<V>(&tile[(int)wv * TT + r][lane * V]);
#pragma unroll
    for (int i = 0; i < TT; ++i) {
        Vf<V> acc = bv;
#pragma unroll
        for (int k = 0; k < K; ++k)
#pragma unroll
            for (int e = 0; e < V; ++e) acc.v[e] = __builtin_fmaf(win[i + k].v[e], wk[k].v[e], acc.v[e]);
        const bool keep = tw + i < len;
#pragma unroll
        for (int e = 0; e < V; ++e) acc.v[e] = keep ? acc.v[e] : 0.0f;
        Buf<S, V>::store(yr, (uint32_t)(tw + i) * row + coff, acc);
    }
}

// Persistent, double-buffered form (fp32 at the compiled widths with 16-byte
// lanes and at least 32 channel groups).  The one-shot form above loads its
// tile, waits, computes and exits, so within a workgroup the loads never
// overlap the FMAs and stores, and tens of thousands of short workgroups
// leave gaps between them.  Here a fixed grid of workgroups walks the time
// tiles (16 frames; 32 at K = 15) of its channel slab (tile g, g + G, ...),
// and while it computes one tile the rows of its next tile are already on
// their way into a second LDS buffer, by buffer-to-LDS loads
// (buffer_load_dwordx4 ... lds) that hold no registers: lane i of a wave
// writes its 16 bytes at byte 16 i of the LDS row named by M0, so a wave's
// load of one frame fills one 1 KiB row.  Out-of-range frames arrive as zeros,
// as everywhere here.
//
// The two buffers are separate arrays, and the loop body is written out once
// per buffer, so that waits for one buffer's loads do not cover the other's.
// The workgroup syncs with a bare s_barrier after an explicit wait: vmcnt(kR)
// leaves this wave's kR just-issued loads of the next tile in flight and
// retires everything older, which includes this tile's loads, since loads
// return in issue order; a __syncthreads fence would wait for all of them.
// Before a buffer is refilled, each wave waits for its own LDS reads
// (lgkmcnt(0)) and the workgroup meets at a barrier.
//
// Measured in the full step on MI355X at [32,1500,512] causal: K3 35.5 ->
// 33.4 us, K4 35.5 -> 32.0, K5 35.0 -> 32.2, K9 36.2 -> 34.9; K15 with
// 32-frame tiles 37.0 -> 35.5 (with 16-frame tiles, 30 staged rows per 16
// frames, it lost); [32,1500,200] K9 19.8 -> 19.2 on 512 workgroups (it lost
// on 256, and on 1024).
typedef __attribute__((address_space(3))) void* lds_ptr_t;
// s_waitcnt immediates (gfx9 layout: vmcnt in bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8): vmcnt(n) alone, and lgkmcnt(0) alone.
constexpr int vmcnt_wait(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }
constexpr int kWaitLds = 0xC07F;
// Frames per tile: 16, and 32 at K = 15, where a 16-frame tile would stage
// 30 rows for 16 outputs.
constexpr int pipe_tile_1d(int K) { return K >= 15 ? 32 : 16; }
// Stores of the persistent form: non-temporal with the sc1 scope bit (18);
// measured ahead of non-temporal alone (2) in the full step.
constexpr int kPipeStorePolicy = 18;

template <int K>
struct Pipe1d {
    static constexpr int TW = pipe_tile_1d(K), R = TW + K - 1, W = kBlock1d / 64, TT = TW / W;
    static constexpr int kR = (R + W - 1) / W;  // rows each wave loads; rows past R land in spare rows
    static constexpr int kRows = kR * W;
};

// Issue the buffer-to-LDS loads of tile j (item b, frames t0 - pL ...) into
// `tile`; false (and nothing issued) when the tile lies wholly past the length.
template <int K>
__device__ __forceinline__ bool pipe1d_issue(float (*tile)[256], uint32_t j, uint32_t n_tt, const float* x,
                                             const int32_t* lengths, int32_t T, int32_t C, int32_t pL,
                                             uint32_t row, uint32_t coff, uint32_t wv) {
    using P = Pipe1d<K>;
    const uint32_t b = j / n_tt, tt = j - b * n_tt;
    const int32_t len = (int32_t)item_length(lengths, b, T);
    const int32_t t0 = (int32_t)tt * P::TW;
    if (t0 >= len) return false;
    const rsrc_t xr = make_rsrc(x + (int64_t)b * T * C, (uint32_t)len * row);
#pragma unroll
    for (int q = 0; q < P::kR; ++q) {
        const int r = (int)wv + P::W * q;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)&tile[r][0], 16,
                                                 (uint32_t)((t0 - pL + r) * (int32_t)row) + coff, 0, 0, 0);
    }
    return true;
}

// This wave's TT output frames of tile j from the staged rows.
template <int K>
__device__ __forceinline__ void pipe1d_compute(const float (*tile)[256], uint32_t j, uint32_t n_tt, float* y,
                                               const int32_t* lengths, int32_t T, int32_t C, uint32_t row,
                                               uint32_t coff, uint32_t lane, uint32_t wv, const Vf<4>* wk,
                                               const Vf<4>& bv) {
    using P = Pipe1d<K>;
    constexpr int V = 4, TT = P::TT;
    const uint32_t b = j / n_tt, tt = j - b * n_tt;
    const int32_t len = (int32_t)item_length(lengths, b, T);
    const int32_t t0 = (int32_t)tt * P::TW, tw = t0 + (int32_t)wv * TT;
    const rsrc_t yr = make_rsrc(y + (int64_t)b * T * C, (uint32_t)T * row);
    if (t0 >= len) {  // uniform: the whole tile is past the length
        const Vf<V> z = vzero<V>();
#pragma unroll
        for (int i = 0; i < TT; ++i)
            Buf<float, V>::template store<kPipeStorePolicy>(yr, (uint32_t)(tw + i) * row + coff, z);
        return;
    }
    Vf<V> win[TT + K - 1];
#pragma unroll
    for (int r = 0; r < TT + K - 1; ++r) win[r] = lds_get<V>(&tile[(int)wv * TT + r][lane * V]);
#pragma unroll
    for (int i = 0; i < TT; ++i) {
        Vf<V> acc = bv;
#pragma unroll
        for (int k = 0; k < K; ++k)
#pragma unroll
            for (int e = 0; e < V; ++e) acc.v[e] = __builtin_fmaf(win[i + k].v[e], wk[k].v[e], acc.v[e]);
        const bool keep = tw + i < len;
#pragma unroll
        for (int e = 0; e < V; ++e) acc.v[e] = keep ? acc.v[e] : 0.0f;
        Buf<float, V>::template store<kPipeStorePolicy>(yr, (uint32_t)(tw + i) * row + coff, acc);
    }
}

// grid: G workgroups per slab of 64 channel groups (block = slab + n_slabs * g)
template <int K>
__global__ __launch_bounds__(kBlock1d) void dwconv1d_fwd_pipe_kernel(
    const float* __restrict__ x, const float* __restrict__ w, const float* __restrict__ bias,
    const int32_t* __restrict__ lengths, float* __restrict__ y, int32_t T, int32_t C, int32_t pL,
    uint32_t n_ttiles, uint32_t n_slabs, uint32_t CG, uint32_t ntiles) {
    using P = Pipe1d<K>;
    constexpr int V = 4;
    __shared__ __align__(16) float ta[P::kRows][64 * V];
    __shared__ __align__(16) float tb[P::kRows][64 * V];
    const uint32_t blk = xcd_contiguous_block(blockIdx.x, gridDim.x);
    const uint32_t slab = blk % n_slabs, g = blk / n_slabs;
    const uint32_t G = gridDim.x / n_slabs;
    const uint32_t row = (uint32_t)C * sizeof(float);
    const uint32_t lane = threadIdx.x % 64, wv = threadIdx.x / 64;
    const bool active = slab * 64 + lane < CG;
    const int32_t c0 = active ? (int32_t)(slab * 64 + lane) * V : 0;
    const uint32_t coff = active ? (uint32_t)c0 * sizeof(float) : 0x80000000u;
    Vf<V> wk[K];
#pragma unroll
    for (int k = 0; k < K; ++k) wk[k] = load_param<float, V>(w + (int64_t)k * C + c0);
    const Vf<V> bv = bias ? load_param<float, V>(bias + c0) : vzero<V>();
    uint32_t j = g;  // uniform over the workgroup, as is every branch below
    if (j >= ntiles) return;
    pipe1d_issue<K>(ta, j, n_ttiles, x, lengths, T, C, pL, row, coff, wv);
    for (;;) {
        // tile j is in ta (or needs no rows); stage tile j + G into tb
        uint32_t jn = j + G;
        bool more = jn < ntiles && pipe1d_issue<K>(tb, jn, n_ttiles, x, lengths, T, C, pL, row, coff, wv);
        if (more) __builtin_amdgcn_s_waitcnt(vmcnt_wait(P::kR));
        else __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
        __builtin_amdgcn_s_barrier();
        pipe1d_compute<K>(ta, j, n_ttiles, y, lengths, T, C, row, coff, lane, wv, wk, bv);
        __builtin_amdgcn_s_waitcnt(kWaitLds);
        __builtin_amdgcn_s_barrier();
        j = jn;
        if (j >= ntiles) break;
        // tile j is in tb; stage tile j + G into ta
        jn = j + G;
        more = jn < ntiles && pipe1d_issue<K>(ta, jn, n_ttiles, x, lengths, T, C, pL, row, coff, wv);
        if (more) __builtin_amdgcn_s_waitcnt(vmcnt_wait(P::kR));
        else __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
        __builtin_amdgcn_s_barrier();
        pipe1d_compute<K>(tb, j, n_ttiles, y, lengths, T, C, row, coff, lane, wv, wk, bv);
        __builtin_amdgcn_s_waitcnt(kWaitLds);
        __builtin_amdgcn_s_barrier();
        j = jn;
        if (j >= ntiles) break;
    }
}

// Any K: the same tiling, with the taps read through the cache instead of a
// register window whose size would have to be known at compile time.
template <typename S, int V, int TT>
__global__ __launch_bounds__(kBlock1d) void dwconv1d_fwd_anyk_kernel(
    const S* __restrict__ x, const S* __restrict__ w, const S* __restrict__ bias,
    const int32_t* __restrict__ lengths, S* __restrict__ y,
    int32_t T, int32_t C, int32_t K, int32_t pL, uint32_t n_tiles, uint32_t CG, uint32_t blocks_per_item) {
    const Tile1d d = decode_1d(n_tiles, CG, blocks_per_item);
    if (!d.valid) return;
    const int32_t len = (int32_t)item_length(lengths, d.b, T);
    const uint32_t row = (uint32_t)C * sizeof(S);
    const int64_t item = (int64_t)d.b * T * C;
    const rsrc_t xr = make_rsrc(x + item, (uint32_t)len * row);
    const rsrc_t yr = make_rsrc(y + item, (uint32_t)T * row);
    const int32_t c0 = (int32_t)d.cg * V;
    const uint32_t coff = (uint32_t)c0 * sizeof(S);
    const int32_t t0 = (int32_t)d.tile * TT;
    const Vf<V> bv = bias ? load_param<S, V>(bias + c0) : vzero<V>();

    for (int i = 0; i < TT; ++i) {
        const int32_t t = t0 + i;
        Vf<V> acc = bv;
        if (t < len) {
            for (int k = 0; k < K; ++k) {
                const Vf<V> xv = Buf<S, V>::load(xr, (uint32_t)((t - pL + k) * (int32_t)row) + coff);
                const Vf<V> wv = load_param<S, V>(w + (int64_t)k * C + c0);
#pragma unroll
                for (int e = 0; e < V; ++e) acc.v[e] = __builtin_fmaf(xv.v[e], wv.v[e], acc.v[e]);
            }
        } else {
            acc = vzero<V>();
        }
        Buf<S, V>::store(yr, (uint32_t)t * row + coff, acc);
    }
}

// Time-tile length per thread for each specialised width (register window of
// TT + K - 1 channel vectors).
// Time-tile length per thread (outputs per thread; the register window holds
// TT + K - 1 channel vectors).  Chosen per width from measurements on MI355X:
// short tiles re-read more halo through L2, long tiles hold more registers.
#ifndef DW1D_TILE
#define DW1D_TILE 0  // 0: the per-width choice below; otherwise one tile for every width
#endif
template <int K>
constexpr int tile_1d_f32() { return DW1D_TILE > 0 ? DW1D_TILE : (K <= 3 ? 4 : K == 4 ? 6 : K <= 9 ? 8 : 12); }
#ifndef DW1D_TILE_BF16
#define DW1D_TILE_BF16 0  // 0: the per-width choice below
#endif
template <int K>
constexpr int tile_1d_bf16() {
    return DW1D_TILE > 0 ? DW1D_TILE : DW1D_TILE_BF16 > 0 ? DW1D_TILE_BF16 : (K <= 4 ? 8 : 12);
}
constexpr int kTileAnyK = 8;

// (The tile depends on the storage type and K only, so host and device agree
// for every vector width.)
template <typename S, int K, int V>
constexpr int tile_of() { return sizeof(S) == 2 ? tile_1d_bf16<K>() : tile_1d_f32<K>(); }

static int tile_for(int64_t K, bool bf16) {
    switch (K) {
        case 3: return bf16 ? tile_of<uint16_t, 3, 4>() : tile_of<float, 3, 4>();
        case 4: return bf16 ? tile_of<uint16_t, 4, 4>() : tile_of<float, 4, 4>();
        case 5: return bf16 ? tile_of<uint16_t, 5, 4>() : tile_of<float, 5, 4>();
        case 9: return bf16 ? tile_of<uint16_t, 9, 4>() : tile_of<float, 9, 4>();
        case 15: return bf16 ? tile_of<uint16_t, 15, 4>() : tile_of<float, 15, 4>();
        default: return kTileAnyK;
    }
}

// The fp32 forward stages through LDS at the compiled widths (3, 4, 5, 9, 15)
// when there are at least 32 channel groups; a last slab of fewer than
// 64 groups leaves its other lanes idle (C = 200: 21.5 -> 19.9 us against the
// register form).  At K <= 5 it is ahead since its loads are issued together
// (K5 36.6 -> 34.7 us, K3 35.5 -> 35.0 at [32,1500,512] on MI355X; figures
// of the one-shot form).
static bool lds_form_1d(int64_t K, int64_t CG) {
    return (K == 3 || K == 4 || K == 5 || K == 9 || K == 15) && CG >= 32;
}

// With 16-byte lanes those take the persistent, double-buffered form instead.
// Its grid: 256 workgroups (one per CU) when the channels span two or more
// slabs, 512 when they fit one and K < 15 (two per CU; a K = 15 workgroup's
// 96 KiB of LDS leaves room for one).  Measured: [32,1500,512] 33.1 us on 256
// against 35.0 on 512 (K3; K9 34.2 against 35.1); [32,1500,200] K9 19.2 on
// 512 against 23.2 on 256 and 21.5 on 1024.
static bool pipe_form_1d(int64_t K, int64_t CG) { return lds_form_1d(K, CG); }
static uint32_t pipe_workgroups_1d(int64_t K, uint32_t n_slabs) { return n_slabs == 1 && K < 15 ? 512 : 256; }

bool dwconv1d_fwd_fits(int64_t B, int64_t T, int64_t C, int64_t K, int elem_bytes, int vec) {
    // Per-item byte offsets, including the left padding as a negative
    // offset, must stay within a signed 32-bit range.
    if (!product_below((int64_t)1 << 31, {T + K + 32, C, elem_bytes})) return false;
    const int64_t tt = tile_for(K, elem_bytes == 2);
    const int64_t per_item = ((T + tt - 1) / tt) * (C / vec);
    int64_t blocks = B * ((per_item + kBlock1d - 1) / kBlock1d);
    if (elem_bytes == 4 && lds_form_1d(K, C / vec))
        blocks = B * ((T + kLdsTile1d - 1) / kLdsTile1d) * ((C / vec + 63) / 64);
    // the persistent form counts its tiles, B * ceil(T / 16), in 32 bits
    if (elem_bytes == 4 && vec == 4 && pipe_form_1d(K, C / vec)) blocks = B * ((T + 15) / 16);
    return blocks < ((int64_t)1 << 31);
}

template <typename S, int V>
static hipError_t launch_typed(const S* x, const S* w, const S* bias, const int32_t* lengths, S* y,
                               int64_t B, int64_t T, int64_t C, int64_t K, int64_t pL, hipStream_t st) {
    const int tt = tile_for(K, sizeof(S) == 2);
    const uint32_t n_tiles = (uint32_t)((T + tt - 1) / tt);
    const uint32_t CG = (uint32_t)(C / V);
    const uint32_t bpi = (uint32_t)(((uint64_t)n_tiles * CG + kBlock1d - 1) / kBlock1d);
    const dim3 grid((uint32_t)(B * bpi)), block(kBlock1d);
    const int32_t T32 = (int32_t)T, C32 = (int32_t)C, p32 = (int32_t)pL;
    if constexpr (sizeof(S) == 4 && V == 4) {
        if (pipe_form_1d(K, (int64_t)CG)) {
            const int64_t TW = pipe_tile_1d((int)K);
            const uint32_t n_tt = (uint32_t)((T + TW - 1) / TW), n_sl = (CG + 63) / 64;
            const uint32_t ntiles = (uint32_t)B * n_tt;
            if (ntiles == 0) return hipSuccess;
            uint32_t G = pipe_workgroups_1d(K, n_sl) / n_sl;
            G = G < 1 ? 1 : (G > ntiles ? ntiles : G);
            const dim3 pgrid(G * n_sl);
            if (K == 3)
                hipLaunchKernelGGL((dwconv1d_fwd_pipe_kernel<3>), pgrid, block, 0, st, x, w, bias, lengths, y, T32,
                                   C32, p32, n_tt, n_sl, CG, ntiles);
            else if (K == 4)
                hipLaunchKernelGGL((dwconv1d_fwd_pipe_kernel<4>), pgrid, block, 0, st, x, w, bias, lengths, y, T32,
                                   C32, p32, n_tt, n_sl, CG, ntiles);
            else if (K == 5)
                hipLaunchKernelGGL((dwconv1d_fwd_pipe_kernel<5>), pgrid, block, 0, st, x, w, bias, lengths, y, T32,
                                   C32, p32, n_tt, n_sl, CG, ntiles);
            else if (K == 9)
                hipLaunchKernelGGL((dwconv1d_fwd_pipe_kernel<9>), pgrid, block, 0, st, x, w, bias, lengths, y, T32,
                                   C32, p32, n_tt, n_sl, CG, ntiles);
            else
                hipLaunchKernelGGL((dwconv1d_fwd_pipe_kernel<15>), pgrid, block, 0, st, x, w, bias, lengths, y, T32,
                                   C32, p32, n_tt, n_sl, CG, ntiles);
            return hipGetLastError();
        }
    }
    if constexpr (sizeof(S) == 4) {
        if (lds_form_1d(K, (int64_t)CG)) {
            constexpr int TW = kLdsTile1d;
            const uint32_t n_tt = (uint32_t)((T + TW - 1) / TW), n_sl = (CG + 63) / 64;
            const dim3 lgrid((uint32_t)(B * n_tt * n_sl));
            if (K == 3)
                hipLaunchKernelGGL((dwconv1d_fwd_lds_kernel<S, V, 3, TW>), lgrid, block, 0, st, x, w, bias,
                                   lengths, y, T32, C32, p32, n_tt, n_sl, CG);
            else if (K == 4)
                hipLaunchKernelGGL((dwconv1d_fwd_lds_kernel<S, V, 4, TW>), lgrid, block, 0, st, x, w, bias,
                                   lengths, y, T32, C32, p32, n_tt, n_sl, CG);
            else if (K == 5)
                hipLaunchKernelGGL((dwconv1d_fwd_lds_kernel<S, V, 5, TW>), lgrid, block, 0, st, x, w, bias,
                                   lengths, y, T32, C32, p32, n_tt, n_sl, CG);
            else if (K == 9)
                hipLaunchKernelGGL((dwconv1d_fwd_lds_kernel<S, V, 9, TW>), lgrid, block, 0, st, x, w, bias,
                                   lengths, y, T32, C32, p32, n_tt, n_sl, CG);
            else
                hipLaunchKernelGGL((dwconv1d_fwd_lds_kernel<S, V, 15, TW>), lgrid, block, 0, st, x, w, bias,
                                   lengths, y, T32, C32, p32, n_tt, n_sl, CG);
            return hipGetLastError();
        }
    }
#define DW1D_CASE(KK)                                                                            \
    case KK:                                                                                     \
        hipLaunchKernelGGL((dwconv1d_fwd_kernel<S, V, KK, tile_of<S, KK, V>()>), grid, block, 0, st, x, \
                           w, bias, lengths, y, T32, C32, p32, n_tiles, CG, bpi);                  \
        break;
    switch (K) {
        DW1D_CASE(3)
        DW1D_CASE(4)
        DW1D_CASE(5)
        DW1D_CASE(9)
        DW1D_CASE(15)
        default:
            hipLaunchKernelGGL((dwconv1d_fwd_anyk_kernel<S, V, kTileAnyK>), grid, block, 0, st, x, w,
                               bias, lengths, y, T32, C32, (int32_t)K, p32, n_tiles, CG, bpi);
    }
#undef DW1D_CASE
    return hipGetLastError();
}

hipError_t launch_dwconv1d_fwd(const void* x, const void* w, const void* bias, const int32_t* lengths,
                               void* y, int64_t B, int64_t T, int64_t C, int64_t K, int64_t pad_left,
                               bool bf16, int vec, hipStream_t st) {
    if (bf16) {
        auto X = (const uint16_t*)x; auto W = (const uint16_t*)w; auto Bi = (const uint16_t*)bias;
        auto Y = (uint16_t*)y;
        switch (vec) {
            case 8: return launch_typed<uint16_t, 8>(X, W, Bi, lengths, Y, B, T, C, K, pad_left, st);
            case 4: return launch_typed<uint16_t, 4>(X, W, Bi, lengths, Y, B, T, C, K, pad_left, st);
            case 2: return launch_typed<uint16_t, 2>(X, W, Bi, lengths, Y, B, T, C, K, pad_left, st);
            default: return launch_typed<uint16_t, 1>(X, W, Bi, lengths, Y, B, T, C, K, pad_left, st);
        }
    }
    auto X = (const float*)x; auto W = (const float*)w; auto Bi = (const float*)bias;
    auto Y = (float*)y;
    switch (vec) {
        case 4: return launch_typed<float, 4>(X, W, Bi, lengths, Y, B, T, C, K, pad_left, st);
        case 2: return launch_typed<float, 2>(X, W, Bi, lengths, Y, B, T, C, K, pad_left, st);
        default: return launch_typed<float, 1>(X, W, Bi, lengths, Y, B, T, C, K, pad_left, st);
    }
}

int pick_vec(int64_t C, int elem_bytes, const void* const* ptrs, int nptrs, int max_vec) {
    for (int v = max_vec; v > 1; v /= 2) {
        if (C % v) continue;
        bool ok = true;
        for (int i = 0; i < nptrs; ++i)
            if (ptrs[i] && ((uintptr_t)ptrs[i] % (uintptr_t)(v * elem_bytes))) ok = false;
        if (ok) return v;
    }
    return 1;
}


// ---------------------------------------------------------------------------
// Streaming form (the streaming encoder's conv with a cache: parakeet.cpp PR
// #102, "What changes"; state kept on the GPU between chunks).  Per stream,
// the sequence convolved is the K - 1 cached frames followed by the chunk's
// len valid frames, s = cache ++ x[:len], causally:
//   y[t] = sum_k s[t + k] w[k] + bias   (t < len; 0 after)
//   cache_out[j] = s[len + j]           (j < K - 1: the last K - 1 frames)
// The grid is the forward's (item, time tile, channel group), plus one tile
// per item whose threads write the new cache.  Frame s[i] is x frame
// i - (K - 1) when i >= K - 1 and cache frame i otherwise; where a window or
// the cache update may need either, both are loaded through their resources
// (the one out of range reads zero, with no traffic) and a select picks the
// right one, so cached values are copied bit for bit.  Only tiles with
// t0 < K - 1 read the cache.  The output cache is a different buffer from the
// input cache, since the update runs beside the tiles that read it.
// ---------------------------------------------------------------------------

template <typename S, int V>
__device__ __forceinline__ Vf<V> stream_frame(rsrc_t xr, rsrc_t cr, int32_t i, int32_t Km1, uint32_t row,
                                              uint32_t coff) {
    const Vf<V> xv = Buf<S, V>::load(xr, (uint32_t)((i - Km1) * (int32_t)row) + coff);
    const Vf<V> cv = Buf<S, V>::load(cr, (uint32_t)(i * (int32_t)row) + coff);
    Vf<V> r;
#pragma unroll
    for (int e = 0; e < V; ++e) r.v[e] = i < Km1 ? cv.v[e] : xv.v[e];
    return r;
}

// K > 0: a compile-time width with a register window; K = 0: any width,
// given at run time, taps read through the cache.
template <typename S, int V, int K, int TT>
__global__ __launch_bounds__(kBlock1d) void dwconv1d_stream_kernel(
    const S* __restrict__ x, const S* __restrict__ w, const S* __restrict__ bias,
    const int32_t* __restrict__ lengths, const S* __restrict__ cache_in, S* __restrict__ y,
    S* __restrict__ cache_out, int32_t Tc, int32_t C, int32_t Kr, uint32_t n_tiles, uint32_t CG,
    uint32_t blocks_per_item) {
    const int32_t Kw = K > 0 ? K : Kr;
    const int32_t Km1 = Kw - 1;
    const Tile1d d = decode_1d(n_tiles + 1, CG, blocks_per_item);
    if (!d.valid) return;
    const int32_t len = (int32_t)item_length(lengths, d.b, Tc);
    const uint32_t row = (uint32_t)C * sizeof(S);
    const rsrc_t xr = make_rsrc(x + (int64_t)d.b * Tc * C, (uint32_t)len * row);
    const rsrc_t cr = make_rsrc(cache_in + (int64_t)d.b * Km1 * C, (uint32_t)Km1 * row);
    const int32_t c0 = (int32_t)d.cg * V;
    const uint32_t coff = (uint32_t)c0 * sizeof(S);

    if (d.tile == n_tiles) {
        // The new cache: s[len + j], j < K - 1.
        const rsrc_t co = make_rsrc(cache_out + (int64_t)d.b * Km1 * C, (uint32_t)Km1 * row);
        if constexpr (K > 0) {
            Vf<V> v[K > 1 ? K - 1 : 1];
#pragma unroll
            for (int j = 0; j < K - 1; ++j) v[j] = stream_frame<S, V>(xr, cr, len + j, Km1, row, coff);
#pragma unroll
            for (int j = 0; j < K - 1; ++j) Buf<S, V>::store(co, (uint32_t)j * row + coff, v[j]);
        } else {
            for (int32_t j = 0; j < Km1; ++j)
                Buf<S, V>::store(co, (uint32_t)j * row + coff, stream_frame<S, V>(xr, cr, len + j, Km1, row, coff));
        }
        return;
    }

    const rsrc_t yr = make_rsrc(y + (int64_t)d.b * Tc * C, (uint32_t)Tc * row);
    const int32_t t0 = (int32_t)d.tile * TT;
    if (t0 >= len) {
        const Vf<V> z = vzero<V>();
#pragma unroll
        for (int i = 0; i < TT; ++i) Buf<S, V>::store(yr, (uint32_t)(t0 + i) * row + coff, z);
        return;
    }
    const Vf<V> bv = bias ? load_param<S, V>(bias + c0) : vzero<V>();
    if constexpr (K > 0) {
        Vf<V> win[TT + K - 1];
        if (t0 == 0) {
            // the first tile: window frames 0 .. K-2 are the cache, the rest the chunk
#pragma unroll
            for (int r = 0; r < TT + K - 1; ++r)
                win[r] = r < K - 1 ? Buf<S, V>::load(cr, (uint32_t)r * row + coff)
                                   : Buf<S, V>::load(xr, (uint32_t)(r - (K - 1)) * row + coff);
        } else if (t0 < K - 1) {
#pragma unroll
            for (int r = 0; r < TT + K - 1; ++r) win[r] = stream_frame<S, V>(xr, cr, t0 + r, K - 1, row, coff);
        } else {
#pragma unroll
            for (int r = 0; r < TT + K - 1; ++r)
                win[r] = Buf<S, V>::load(xr, (uint32_t)((t0 + r - (K - 1)) * (int32_t)row) + coff);
        }
        Vf<V> wk[K];
#pragma unroll
        for (int k = 0; k < K; ++k) wk[k] = load_param<S, V>(w + (int64_t)k * C + c0);
#pragma unroll
        for (int i = 0; i < TT; ++i) {
            Vf<V> acc = bv;
#pragma unroll
            for (int k = 0; k < K; ++k)
#pragma unroll
                for (int e = 0; e < V; ++e) acc.v[e] = __builtin_fmaf(win[i + k].v[e], wk[k].v[e], acc.v[e]);
            const bool keep = t0 + i < len;
#pragma unroll
            for (int e = 0; e < V; ++e) acc.v[e] = keep ? acc.v[e] : 0.0f;
            Buf<S, V>::store(yr, (uint32_t)(t0 + i) * row + coff, acc);
        }
    } else {
        for (int i = 0; i < TT; ++i) {
            const int32_t t = t0 + i;
            Vf<V> acc = vzero<V>();
            if (t < len) {
                acc = bv;
                for (int32_t k = 0; k < Kw; ++k) {
                    const Vf<V> sv = stream_frame<S, V>(xr, cr, t + k, Km1, row, coff);
                    const Vf<V> wv = load_param<S, V>(w + (int64_t)k * C + c0);
#pragma unroll
                    for (int e = 0; e < V; ++e) acc.v[e] = __builtin_fmaf(sv.v[e], wv.v[e], acc.v[e]);
                }
            }
            Buf<S, V>::store(yr, (uint32_t)t * row + coff, acc);
        }
    }
}


// Streaming chunks are short: a chunk of at most kStreamShort frames takes a
// tile of that length instead of the forward's (a longer tile would only
// compute frames past the chunk).
#ifndef DW1S_SHORT_TILE
#define DW1S_SHORT_TILE 8
#endif
constexpr int kStreamShort = DW1S_SHORT_TILE;

// Persistent streaming form (compiled widths, 16-byte lanes, chunks of at
// most kStreamShort frames, at least 32 channel groups).  The form above
// gives each stream a workgroup that loads, computes and stores once, and a
// second set of threads that loads the same frames again for the new cache.
// Here a fixed grid of workgroups (G per 64-group slab) walks the streams
// b = g, g + G, ... of its slab: stream b's sequence s = cache ++ chunk, all
// K - 1 + Tc rows of it, is staged once in LDS by buffer-to-LDS loads (rows
// past the chunk's valid length arrive as zeros), double-buffered as in the
// persistent 1-D forward, so the next stream's rows are in flight while this
// one's outputs are written.  Wave v computes y frames v, v + 4, ... from
// LDS, and copies the new cache rows s[len + j], j = v, v + 4, ..., from LDS
// at the run-time offset len, as raw bytes.  Every wave issues the same
// number of row loads (rows past K - 1 + Tc are sent out of range), so the
// wait counts are compile-time constants.  Measured in the full step on
// MI355X at 1024 streams x 8 frames x 1024 channels, K = 9, bf16:
// 21.3 -> 18.7 us on 512 workgroups (23.8 on 256, 19.8 on 1024).
template <typename S, int K>
struct StreamPipe {
    static constexpr int V = 16 / (int)sizeof(S), W = kBlock1d / 64;
    static constexpr int RMAX = kStreamShort + K - 1, kR = (RMAX + W - 1) / W, kRows = kR * W;
};

template <typename S, int K>
__device__ __forceinline__ void stream_pipe_issue(uint32_t (*tile)[256], uint32_t b, const S* x, const S* cache_in,
                                                  const int32_t* lengths, int32_t Tc, int32_t C, uint32_t row,
                                                  uint32_t coff, uint32_t wv) {
    using P = StreamPipe<S, K>;
    constexpr int Km1 = K - 1;
    const int32_t len = (int32_t)item_length(lengths, b, Tc);
    const rsrc_t xr = make_rsrc(x + (int64_t)b * Tc * C, (uint32_t)len * row);
    const rsrc_t cr = make_rsrc(cache_in + (int64_t)b * Km1 * C, (uint32_t)Km1 * row);
#pragma unroll
    for (int q = 0; q < P::kR; ++q) {
        const int r = (int)wv + P::W * q;  // rows at or past K - 1 + Tc read zero and are never used
        const bool cached = r < Km1;       // uniform over the wave
        const uint32_t off = cached ? (uint32_t)r * row + coff : (uint32_t)((r - Km1) * (int32_t)row) + coff;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(cached ? cr : xr, (lds_ptr_t)&tile[r][0], 16, off, 0, 0, 0);
    }
}

template <typename S, int K>
__device__ __forceinline__ void stream_pipe_compute(const uint32_t (*tile)[256], uint32_t b, S* y, S* cache_out,
                                                    const int32_t* lengths, int32_t Tc, int32_t C, uint32_t row,
                                                    uint32_t coff, uint32_t lane, uint32_t wv,
                                                    const Vf<StreamPipe<S, K>::V>* wk,
                                                    const Vf<StreamPipe<S, K>::V>& bv) {
    using P = StreamPipe<S, K>;
    constexpr int V = P::V, Km1 = K - 1;
    const int32_t len = (int32_t)item_length(lengths, b, Tc);
    const rsrc_t yr = make_rsrc(y + (int64_t)b * Tc * C, (uint32_t)Tc * row);
    for (int32_t t = (int32_t)wv; t < Tc; t += P::W) {
        Vf<V> acc = bv;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const u32x4 raw = *reinterpret_cast<const u32x4*>(&tile[t + k][lane * 4]);
            Vf<V> sv;
            if constexpr (sizeof(S) == 2) {
                sv.v[0] = bf16_lo(raw.x); sv.v[1] = bf16_hi(raw.x); sv.v[2] = bf16_lo(raw.y); sv.v[3] = bf16_hi(raw.y);
                sv.v[4] = bf16_lo(raw.z); sv.v[5] = bf16_hi(raw.z); sv.v[6] = bf16_lo(raw.w); sv.v[7] = bf16_hi(raw.w);
            } else {
                sv.v[0] = __uint_as_float(raw.x); sv.v[1] = __uint_as_float(raw.y);
                sv.v[2] = __uint_as_float(raw.z); sv.v[3] = __uint_as_float(raw.w);
            }
#pragma unroll
            for (int e = 0; e < V; ++e) acc.v[e] = __builtin_fmaf(sv.v[e], wk[k].v[e], acc.v[e]);
        }
        const bool keep = t < len;
#pragma unroll
        for (int e = 0; e < V; ++e) acc.v[e] = keep ? acc.v[e] : 0.0f;
        Buf<S, V>::store(yr, (uint32_t)t * row + coff, acc);
    }
    if (cache_out) {
        const rsrc_t co = make_rsrc(cache_out + (int64_t)b * Km1 * C, (uint32_t)Km1 * row);
        for (int32_t j = (int32_t)wv; j < Km1; j += P::W) {
            const u32x4 raw = *reinterpret_cast<const u32x4*>(&tile[len + j][lane * 4]);
            __builtin_amdgcn_raw_buffer_store_b128(raw, co, (uint32_t)j * row + coff, 0, kNonTemporal);
        }
    }
}

// grid: G workgroups per slab of 64 channel groups (block = slab + n_slabs * g)
template <typename S, int K>
__global__ __launch_bounds__(kBlock1d) void dwconv1d_stream_pipe_kernel(
    const S* __restrict__ x, const S* __restrict__ w, const S* __restrict__ bias,
    const int32_t* __restrict__ lengths, const S* __restrict__ cache_in, S* __restrict__ y,
    S* __restrict__ cache_out, int32_t Tc, int32_t C, uint32_t n_slabs, uint32_t CG, uint32_t B) {
    using P = StreamPipe<S, K>;
    constexpr int V = P::V;
    __shared__ __align__(16) uint32_t ta[P::kRows][256];
    __shared__ __align__(16) uint32_t tb[P::kRows][256];
    const uint32_t blk = xcd_contiguous_block(blockIdx.x, gridDim.x);
    const uint32_t slab = blk % n_slabs, g = blk / n_slabs, G = gridDim.x / n_slabs;
    const uint32_t row = (uint32_t)C * sizeof(S);
    const uint32_t lane = threadIdx.x % 64, wv = threadIdx.x / 64;
    const bool active = slab * 64 + lane < CG;
    const int32_t c0 = active ? (int32_t)(slab * 64 + lane) * V : 0;
    const uint32_t coff = active ? (uint32_t)c0 * sizeof(S) : 0x80000000u;
    Vf<V> wk[K];
#pragma unroll
    for (int k = 0; k < K; ++k) wk[k] = load_param<S, V>(w + (int64_t)k * C + c0);
    const Vf<V> bv = bias ? load_param<S, V>(bias + c0) : vzero<V>();
    uint32_t b = g;  // uniform over the workgroup, as is every branch below
    if (b >= B) return;
    stream_pipe_issue<S, K>(ta, b, x, cache_in, lengths, Tc, C, row, coff, wv);
    for (;;) {
        // stream b is in ta; stage stream b + G into tb
        uint32_t bn = b + G;
        if (bn < B) {
            stream_pipe_issue<S, K>(tb, bn, x, cache_in, lengths, Tc, C, row, coff, wv);
            __builtin_amdgcn_s_waitcnt(vmcnt_wait(P::kR));
        } else {
            __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
        }
        __builtin_amdgcn_s_barrier();
        stream_pipe_compute<S, K>(ta, b, y, cache_out, lengths, Tc, C, row, coff, lane, wv, wk, bv);
        __builtin_amdgcn_s_waitcnt(kWaitLds);
        __builtin_amdgcn_s_barrier();
        b = bn;
        if (b >= B) break;
        // stream b is in tb; stage stream b + G into ta
        bn = b + G;
        if (bn < B) {
            stream_pipe_issue<S, K>(ta, bn, x, cache_in, lengths, Tc, C, row, coff, wv);
            __builtin_amdgcn_s_waitcnt(vmcnt_wait(P::kR));
        } else {
            __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
        }
        __builtin_amdgcn_s_barrier();
        stream_pipe_compute<S, K>(tb, b, y, cache_out, lengths, Tc, C, row, coff, lane, wv, wk, bv);
        __builtin_amdgcn_s_waitcnt(kWaitLds);
        __builtin_amdgcn_s_barrier();
        b = bn;
        if (b >= B) break;
    }
}

static int stream_tile(int64_t K, bool bf16, int64_t Tc) {
    const int tt = tile_for(K, bf16);
    const bool specialised = K == 3 || K == 4 || K == 5 || K == 9 || K == 15;
    return (kStreamShort > 0 && specialised && Tc <= kStreamShort && kStreamShort < tt) ? kStreamShort : tt;
}

bool dwconv1d_stream_fits(int64_t B, int64_t Tc, int64_t C, int64_t K, int elem_bytes, int vec) {
    if (!product_below((int64_t)1 << 31, {Tc + 2 * K + 32, C, elem_bytes})) return false;
    const int64_t tt = stream_tile(K, elem_bytes == 2, Tc);
    const int64_t per_item = ((Tc + tt - 1) / tt + 1) * (C / vec);
    return B * ((per_item + kBlock1d - 1) / kBlock1d) < ((int64_t)1 << 31);
}

// bf16 streaming takes 16-byte lanes (8 channels) up to this width; wider
// kernels keep 8-byte lanes, whose register window fits two waves per SIMD.
#ifndef DW1S_BF16_VEC
#define DW1S_BF16_VEC 8
#endif
constexpr int kStreamWideMaxK = 9;

int dwconv1d_stream_max_vec(int64_t K, bool bf16) {
    return bf16 ? (DW1S_BF16_VEC >= 8 && K <= kStreamWideMaxK ? 8 : 4) : 4;
}

// The persistent streaming form: compiled widths, 16-byte lanes, chunks of at
// most kStreamShort frames and at least 32 channel groups, on 512 workgroups.
static bool stream_pipe_form(int64_t K, int64_t Tc, int64_t CG) {
    return (K == 3 || K == 4 || K == 5 || K == 9 || K == 15) && Tc <= kStreamShort && CG >= 32;
}
constexpr uint32_t kStreamPipeWorkgroups = 512;

template <typename S, int V>
static hipError_t launch_stream_typed(const S* x, const S* w, const S* bias, const int32_t* lengths,
                                      const S* cache_in, S* y, S* cache_out, int64_t B, int64_t Tc, int64_t C,
                                      int64_t K, hipStream_t st) {
    if constexpr (sizeof(S) * V == 16) {
        const uint32_t CGp = (uint32_t)(C / V);
        if (stream_pipe_form(K, Tc, (int64_t)CGp)) {
            const uint32_t n_sl = (CGp + 63) / 64;
            uint32_t G = kStreamPipeWorkgroups / n_sl;
            G = G < 1 ? 1 : (G > (uint64_t)B ? (uint32_t)B : G);
            const dim3 pgrid(G * n_sl), pblock(kBlock1d);
            const int32_t T32 = (int32_t)Tc, C32 = (int32_t)C;
#define DW1SP_CASE(KK)                                                                                        \
    case KK:                                                                                                 \
        hipLaunchKernelGGL((dwconv1d_stream_pipe_kernel<S, KK>), pgrid, pblock, 0, st, x, w, bias, lengths, \
                           cache_in, y, cache_out, T32, C32, n_sl, CGp, (uint32_t)B);                        \
        break;
            switch (K) {
                DW1SP_CASE(3)
                DW1SP_CASE(4)
                DW1SP_CASE(5)
                DW1SP_CASE(9)
                DW1SP_CASE(15)
                default: return hipErrorInvalidValue;
            }
#undef DW1SP_CASE
            return hipGetLastError();
        }
    }
    const int tt = stream_tile(K, sizeof(S) == 2, Tc);
    const bool short_tile = kStreamShort > 0 && tt == kStreamShort;
    const uint32_t n_tiles = (uint32_t)((Tc + tt - 1) / tt);
    const uint32_t CG = (uint32_t)(C / V);
    const uint32_t bpi = (uint32_t)(((uint64_t)(n_tiles + 1) * CG + kBlock1d - 1) / kBlock1d);
    const dim3 grid((uint32_t)(B * bpi)), block(kBlock1d);
    const int32_t T32 = (int32_t)Tc, C32 = (int32_t)C, K32 = (int32_t)K;
    constexpr int TS = kStreamShort > 0 ? kStreamShort : 1;
#define DW1S_CASE(KK)                                                                                    \
    case KK:                                                                                             \
        if (short_tile)                                                                                  \
            hipLaunchKernelGGL((dwconv1d_stream_kernel<S, V, KK, TS>), grid, block, 0, st, x, w, bias,   \
                               lengths, cache_in, y, cache_out, T32, C32, K32, n_tiles, CG, bpi);        \
        else                                                                                             \
            hipLaunchKernelGGL((dwconv1d_stream_kernel<S, V, KK, tile_of<S, KK, V>()>), grid, block, 0, st, x, \
                               w, bias, lengths, cache_in, y, cache_out, T32, C32, K32, n_tiles, CG, bpi); \
        break;
    switch (K) {
        DW1S_CASE(3)
        DW1S_CASE(4)
        DW1S_CASE(5)
        DW1S_CASE(9)
        DW1S_CASE(15)
        default:
            hipLaunchKernelGGL((dwconv1d_stream_kernel<S, V, 0, kTileAnyK>), grid, block, 0, st, x, w, bias,
                               lengths, cache_in, y, cache_out, T32, C32, K32, n_tiles, CG, bpi);
    }
#undef DW1S_CASE
    return hipGetLastError();
}

hipError_t launch_dwconv1d_stream(const void* x, const void* w, const void* bias, const int32_t* lengths,
                                  const void* cache_in, void* y, void* cache_out, int64_t B, int64_t Tc, int64_t C,
                                  int64_t K, bool bf16, int vec, hipStream_t st) {
    if (bf16) {
        auto X = (const uint16_t*)x; auto W = (const uint16_t*)w; auto Bi = (const uint16_t*)bias;
        auto Ci = (const uint16_t*)cache_in; auto Y = (uint16_t*)y; auto Co = (uint16_t*)cache_out;
        switch (vec) {
            case 8:
                if constexpr (DW1S_BF16_VEC >= 8)
                    return launch_stream_typed<uint16_t, 8>(X, W, Bi, lengths, Ci, Y, Co, B, Tc, C, K, st);
                return launch_stream_typed<uint16_t, 4>(X, W, Bi, lengths, Ci, Y, Co, B, Tc, C, K, st);
            case 4: return launch_stream_typed<uint16_t, 4>(X, W, Bi, lengths, Ci, Y, Co, B, Tc, C, K, st);
            case 2: return launch_stream_typed<uint16_t, 2>(X, W, Bi, lengths, Ci, Y, Co, B, Tc, C, K, st);
            default: return launch_stream_typed<uint16_t, 1>(X, W, Bi, lengths, Ci, Y, Co, B, Tc, C, K, st);
        }
    }
    auto X = (const float*)x; auto W = (const float*)w; auto Bi = (const float*)bias;
    auto Ci = (const float*)cache_in; auto Y = (float*)y; auto Co = (float*)cache_out;
    switch (vec) {
        case 4: return launch_stream_typed<float, 4>(X, W, Bi, lengths, Ci, Y, Co, B, Tc, C, K, st);
        case 2: return launch_stream_typed<float, 2>(X, W, Bi, lengths, Ci, Y, Co, B, Tc, C, K, st);
        default: return launch_stream_typed<float, 1>(X, W, Bi, lengths, Ci, Y, Co, B, Tc, C, K, st);
    }
}


// ---------------------------------------------------------------------------
// Backward of the 1-D depthwise conv (the conv module in training): with
// g = dy at unmasked frames (t < len) and 0 elsewhere,
//   dx[u, c] = [u < len] sum_k g[u + pL - k, c] w[k, c]
//   dw[k, c] = sum_{b,u} g[u + pL - k, c] x[u, c]      (x masked at u >= len)
//   db[c]    = sum_{b,t} g[t, c]
// Gather form, no atomics: the thread that owns input frame u forms dx[u]
// and every (g, x[u]) pair of dw, so each pair is counted once.  One thread
// owns V channels of TT input frames; a register window holds the TT + K - 1
// gradient frames those need (through the same length-bounded buffer
// resources as the forward, which give the masks and the padding).  dw and
// db are accumulated in fp64 (the fp32 products are exact there), summed
// across the workgroup's 4 time sub-blocks in a fixed order, and written as
// one partial per persistent workgroup for the fixed-order reduction of
// reduce.hip.
// ---------------------------------------------------------------------------

constexpr int kLanes1b = 64, kSubs1b = kBlock1d / kLanes1b;
#ifndef DW1B_VMAX_K9
#define DW1B_VMAX_K9 4
#endif
// Widest lane access of the backward per width (fp64 accumulators for K + 1
// sums per channel must fit beside the K + 7 frame window).
constexpr int bwd1d_vmax(int K) { return K <= 5 ? 4 : (K == 9 ? DW1B_VMAX_K9 : (K <= 15 ? 2 : 1)); }
constexpr int kBwdTile1d = 8;
#ifndef DW1D_BWD_WGS
#define DW1D_BWD_WGS 256
#endif
#ifndef DW1D_BWD_XPOL
#define DW1D_BWD_XPOL 2
#endif
// Cache policy of the backward's x loads: each x frame is read by one tile
// only, so non-temporally (2); the dy frames, which neighbouring tiles share,
// keep the default.
constexpr int kBwdXPolicy1d = DW1D_BWD_XPOL;

template <typename S, int V, int K, bool CAUSAL, int TT>
__global__ __launch_bounds__(kBlock1d) void dwconv1d_bwd_kernel(
    const S* __restrict__ x, const S* __restrict__ w, const int32_t* __restrict__ lengths,
    const S* __restrict__ dy, S* __restrict__ dx, double* __restrict__ partial, int32_t T, int32_t C,
    uint32_t n_tb, uint32_t CG, uint32_t n_cblk, uint32_t groups_per_item, uint32_t n_groups) {
    constexpr int pL = CAUSAL ? K - 1 : (K - 1) / 2;
    __shared__ double red[kSubs1b - 1][K + 1][kLanes1b * V];
    const uint32_t blk = xcd_contiguous_block(blockIdx.x, gridDim.x);
    const uint32_t G = gridDim.x / n_cblk;
    const uint32_t g = blk / n_cblk, cblk = blk - g * n_cblk;
    const uint32_t lane = threadIdx.x % kLanes1b, sub = threadIdx.x / kLanes1b;
    const uint32_t cg = cblk * kLanes1b + lane;
    const bool cvalid = cg < CG;
    const int32_t c0 = (int32_t)(cvalid ? cg : 0) * V;
    const uint32_t row = (uint32_t)C * sizeof(S), coff = (uint32_t)c0 * sizeof(S);

    Vf<V> wk[K];
#pragma unroll
    for (int k = 0; k < K; ++k) wk[k] = load_param<S, V>(w + (int64_t)k * C + c0);
    double gw[K][V], gb[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
        gb[e] = 0.0;
#pragma unroll
        for (int k = 0; k < K; ++k) gw[k][e] = 0.0;
    }

    for (uint32_t j = g; j < n_groups; j += G) {
        const uint32_t b = j / groups_per_item;
        const uint32_t tb = (j - b * groups_per_item) * kSubs1b + sub;
        if (!cvalid || tb >= n_tb) continue;
        const int32_t len = (int32_t)item_length(lengths, b, T);
        const int32_t u0 = (int32_t)tb * TT;
        const int64_t item = (int64_t)b * T * C;
        const rsrc_t dxr = make_rsrc(dx ? dx + item : x, dx ? (uint32_t)T * row : 0u);
        if (u0 >= len) {
            // masked input frames: dx is zero, and there is nothing to add
            if (dx) {
#pragma unroll
                for (int i = 0; i < TT; ++i) Buf<S, V>::store(dxr, (uint32_t)(u0 + i) * row + coff, vzero<V>());
            }
            continue;
        }
        const rsrc_t gr = make_rsrc(dy + item, (uint32_t)len * row);
        const rsrc_t xr = make_rsrc(x + item, (uint32_t)len * row);
        Vf<V> gwin[TT + K - 1], xv[TT];
#pragma unroll
        for (int r = 0; r < TT + K - 1; ++r)
            gwin[r] = Buf<S, V>::load(gr, (uint32_t)((u0 + pL - (K - 1) + r) * (int32_t)row) + coff);
#pragma unroll
        for (int i = 0; i < TT; ++i) xv[i] = Buf<S, V>::template load<kBwdXPolicy1d>(xr, (uint32_t)(u0 + i) * row + coff);
#pragma unroll
        for (int i = 0; i < TT; ++i) {
            Vf<V> d = vzero<V>();
#pragma unroll
            for (int k = 0; k < K; ++k)
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const float gv = gwin[i + K - 1 - k].v[e];
                    d.v[e] = __builtin_fmaf(gv, wk[k].v[e], d.v[e]);
                    gw[k][e] = __builtin_fma((double)gv, (double)xv[i].v[e], gw[k][e]);
                }
#pragma unroll
            for (int e = 0; e < V; ++e) {
                gb[e] += (double)gwin[i + K - 1 - pL].v[e];
                d.v[e] = u0 + i < len ? d.v[e] : 0.0f;
            }
            if (dx) Buf<S, V>::store(dxr, (uint32_t)(u0 + i) * row + coff, d);
        }
    }

    if (!partial) return;  // uniform: dw and db not requested
    if (sub > 0) {
#pragma unroll
        for (int e = 0; e < V; ++e) {
#pragma unroll
            for (int k = 0; k < K; ++k) red[sub - 1][k][lane * V + e] = gw[k][e];
            red[sub - 1][K][lane * V + e] = gb[e];
        }
    }
    __syncthreads();
    if (sub > 0 || !cvalid) return;
#pragma unroll
    for (int e = 0; e < V; ++e) {
        const int32_t c = c0 + e;
#pragma unroll
        for (int k = 0; k <= K; ++k) {
            double s = k < K ? gw[k][e] : gb[e];
#pragma unroll
            for (int q = 0; q < kSubs1b - 1; ++q) s += red[q][k][lane * V + e];
            partial[((int64_t)g * (K + 1) + k) * C + c] = s;
        }
    }
}

// Lane groups (16-byte-aligned tensors, the widths below): Q = 2 or 4 lanes
// share one 16-byte piece of P channels (4 fp32 or 8 bf16), so each lane
// computes V = P / Q channels and keeps that many channels' fp64 sums, while
// every x and dy load and every dx store still moves 16 bytes.  The Q lanes
// of a group sit 64 / Q apart (lane l + r * 64 / Q, r = 0 .. Q-1, holds the
// piece P (cblk * 64 / Q + l) .. +P-1).  Of each run of Q consecutive
// frames, lane r of the group loads frame r, and a transpose of the group's
// Q x 4 dwords by cross-lane swaps leaves lane r with its 4 / Q dwords (its
// V channels) at all Q frames: for Q = 2 one swap of the wave's halves
// (v_permlane32_swap) per dword pair; for Q = 4 the same, then a swap of
// neighbouring 16-lane rows (v_permlane16_swap).  dx goes back through the
// same swaps in reverse order before lane r stores frame r of the run.  The
// arithmetic is the V-channel form's, term for term.  A lane whose channels
// are past C runs every load, swap and store at out-of-range offsets, so
// that the swaps see whole waves.
template <int Q>
__device__ __forceinline__ void group_transpose(u32x4& t) {
    // halves: lanes l and l + 32 exchange dwords z, w of the low half with x, y of the high half
    const auto a = __builtin_amdgcn_permlane32_swap(t.x, t.z, false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(t.y, t.w, false, false);
    t.x = a[0]; t.z = a[1];
    t.y = b[0]; t.w = b[1];
    if constexpr (Q == 4) {
        // rows: lanes l and l + 16 (within each half) exchange dword y of the
        // even row with x of the odd row, and w with z
        const auto c = __builtin_amdgcn_permlane16_swap(t.x, t.y, false, false);
        const auto d = __builtin_amdgcn_permlane16_swap(t.z, t.w, false, false);
        t.x = c[0]; t.y = c[1];
        t.z = d[0]; t.w = d[1];
    }
}

// The inverse of group_transpose: each stage is its own inverse, taken in
// reverse order.
template <int Q>
__device__ __forceinline__ void group_untranspose(u32x4& t) {
    if constexpr (Q == 4) {
        const auto c = __builtin_amdgcn_permlane16_swap(t.x, t.y, false, false);
        const auto d = __builtin_amdgcn_permlane16_swap(t.z, t.w, false, false);
        t.x = c[0]; t.y = c[1];
        t.z = d[0]; t.w = d[1];
    }
    const auto a = __builtin_amdgcn_permlane32_swap(t.x, t.z, false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(t.y, t.w, false, false);
    t.x = a[0]; t.z = a[1];
    t.y = b[0]; t.w = b[1];
}

// The V channels of frame i of a transposed run, widened to float: dwords
// (x, y) or (z, w) for Q = 2, one dword for Q = 4; a dword holds one fp32 or
// two bf16 channels.
template <typename S, int Q>
__device__ __forceinline__ Vf<16 / (int)sizeof(S) / Q> group_frame(const u32x4& t, int i) {
    constexpr int V = 16 / (int)sizeof(S) / Q;
    uint32_t u[4 / Q];
    if constexpr (Q == 2) {
        u[0] = i == 0 ? t.x : t.z;
        u[1] = i == 0 ? t.y : t.w;
    } else {
        u[0] = i == 0 ? t.x : (i == 1 ? t.y : (i == 2 ? t.z : t.w));
    }
    Vf<V> a;
#pragma unroll
    for (int k = 0; k < 4 / Q; ++k) {
        if constexpr (sizeof(S) == 2) {
            a.v[2 * k] = bf16_lo(u[k]);
            a.v[2 * k + 1] = bf16_hi(u[k]);
        } else {
            a.v[k] = __uint_as_float(u[k]);
        }
    }
    return a;
}

// Dword k of a V-channel value in storage form (bf16 rounded to nearest even).
template <typename S, int V>
__device__ __forceinline__ uint32_t group_dword(const Vf<V>& a, int k) {
    if constexpr (sizeof(S) == 2) return pack_bf16x2(a.v[2 * k], a.v[2 * k + 1]);
    else return __float_as_uint(a.v[k]);
}

template <typename S, int K, bool CAUSAL, int TT, int Q>
__global__ __launch_bounds__(kBlock1d) void dwconv1d_bwd_group_kernel(
    const S* __restrict__ x, const S* __restrict__ w, const int32_t* __restrict__ lengths,
    const S* __restrict__ dy, S* __restrict__ dx, double* __restrict__ partial, int32_t T, int32_t C,
    uint32_t n_tb, uint32_t CG, uint32_t n_cblk, uint32_t groups_per_item, uint32_t n_groups) {
    constexpr int P = 16 / (int)sizeof(S);                                 // channels per piece
    constexpr int V = P / Q, NW = TT + K - 1, NR = (NW + Q - 1) / Q;  // window frames, runs of Q loaded
    static_assert((Q == 2 || Q == 4) && TT % Q == 0, "frames are loaded in runs of Q");
    constexpr int pL = CAUSAL ? K - 1 : (K - 1) / 2;
    constexpr uint32_t span = 64 / Q;  // lanes between the members of a group
    __shared__ double red[kSubs1b - 1][K + 1][kLanes1b * V];
    const uint32_t blk = xcd_contiguous_block(blockIdx.x, gridDim.x);
    const uint32_t G = gridDim.x / n_cblk;
    const uint32_t g = blk / n_cblk, cblk = blk - g * n_cblk;
    const uint32_t lane = threadIdx.x % kLanes1b, sub = threadIdx.x / kLanes1b;
    const uint32_t r = lane / span;  // this lane's member index in its group
    // CG counts V-channel groups; the members of a piece hold Q consecutive
    // ones (all valid or none, since C % P == 0)
    const uint32_t cg = (cblk * span + lane % span) * Q + r;
    const bool cvalid = cg < CG;
    const int32_t c0 = (int32_t)(cvalid ? cg : 0) * V;
    const uint32_t row = (uint32_t)C * sizeof(S);
    // this lane's 16-byte piece of a frame: its group's P channels
    const uint32_t qoff = cvalid ? (uint32_t)(c0 - (int32_t)r * V) * (uint32_t)sizeof(S) : 0x80000000u;

    Vf<V> wk[K];
#pragma unroll
    for (int k = 0; k < K; ++k) wk[k] = load_param<S, V>(w + (int64_t)k * C + c0);
    double gw[K][V], gb[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
        gb[e] = 0.0;
#pragma unroll
        for (int k = 0; k < K; ++k) gw[k][e] = 0.0;
    }

    for (uint32_t j = g; j < n_groups; j += G) {
        const uint32_t b = j / groups_per_item;
        const uint32_t tb = (j - b * groups_per_item) * kSubs1b + sub;  // one per wave
        if (tb >= n_tb) continue;
        const int32_t len = (int32_t)item_length(lengths, b, T);
        const int32_t u0 = (int32_t)tb * TT;
        const int64_t item = (int64_t)b * T * C;
        const rsrc_t dxr = make_rsrc(dx ? dx + item : x, dx ? (uint32_t)T * row : 0u);
        if (u0 >= len) {
            // masked input frames: dx is zero, and there is nothing to add
            if (dx) {
                const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int p = 0; p < TT / Q; ++p)
                    __builtin_amdgcn_raw_buffer_store_b128(z, dxr, (uint32_t)(u0 + Q * p + (int32_t)r) * row + qoff, 0,
                                                           kNonTemporal);
            }
            continue;
        }
        const rsrc_t gr = make_rsrc(dy + item, (uint32_t)len * row);
        const rsrc_t xr = make_rsrc(x + item, (uint32_t)len * row);
        const int32_t gs = u0 + pL - (K - 1);  // first gradient frame of the window
        u32x4 graw[NR], xraw[TT / Q];
#pragma unroll
        for (int p = 0; p < NR; ++p)
            graw[p] = __builtin_amdgcn_raw_buffer_load_b128(gr, (uint32_t)((gs + Q * p + (int32_t)r) * (int32_t)row) + qoff,
                                                            0, kLoadPolicy);
#pragma unroll
        for (int p = 0; p < TT / Q; ++p)
            xraw[p] = __builtin_amdgcn_raw_buffer_load_b128(xr, (uint32_t)(u0 + Q * p + (int32_t)r) * row + qoff, 0,
                                                            kBwdXPolicy1d);
        Vf<V> gwin[NR * Q], xv[TT];
#pragma unroll
        for (int p = 0; p < NR; ++p) {
            u32x4 t = graw[p];
            group_transpose<Q>(t);
#pragma unroll
            for (int i = 0; i < Q; ++i) gwin[Q * p + i] = group_frame<S, Q>(t, i);
        }
#pragma unroll
        for (int p = 0; p < TT / Q; ++p) {
            u32x4 t = xraw[p];
            group_transpose<Q>(t);
#pragma unroll
            for (int i = 0; i < Q; ++i) xv[Q * p + i] = group_frame<S, Q>(t, i);
        }
#pragma unroll
        for (int p = 0; p < TT / Q; ++p) {
            Vf<V> d[Q];
#pragma unroll
            for (int h = 0; h < Q; ++h) {
                const int i = Q * p + h;
                d[h] = vzero<V>();
#pragma unroll
                for (int k = 0; k < K; ++k)
#pragma unroll
                    for (int e = 0; e < V; ++e) {
                        const float gv = gwin[i + K - 1 - k].v[e];
                        d[h].v[e] = __builtin_fmaf(gv, wk[k].v[e], d[h].v[e]);
                        gw[k][e] = __builtin_fma((double)gv, (double)xv[i].v[e], gw[k][e]);
                    }
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    gb[e] += (double)gwin[i + K - 1 - pL].v[e];
                    d[h].v[e] = u0 + i < len ? d[h].v[e] : 0.0f;
                }
            }
            if (dx) {
                u32x4 t;
                if constexpr (Q == 2) {
                    t = u32x4{group_dword<S, V>(d[0], 0), group_dword<S, V>(d[0], 1), group_dword<S, V>(d[1], 0),
                              group_dword<S, V>(d[1], 1)};
                } else {
                    t = u32x4{group_dword<S, V>(d[0], 0), group_dword<S, V>(d[1], 0), group_dword<S, V>(d[2], 0),
                              group_dword<S, V>(d[3], 0)};
                }
                group_untranspose<Q>(t);
                __builtin_amdgcn_raw_buffer_store_b128(t, dxr, (uint32_t)(u0 + Q * p + (int32_t)r) * row + qoff, 0,
                                                       kNonTemporal);
            }
        }
    }

    if (!partial) return;  // uniform: dw and db not requested
    if (sub > 0) {
#pragma unroll
        for (int e = 0; e < V; ++e) {
#pragma unroll
            for (int k = 0; k < K; ++k) red[sub - 1][k][lane * V + e] = gw[k][e];
            red[sub - 1][K][lane * V + e] = gb[e];
        }
    }
    __syncthreads();
    if (sub > 0 || !cvalid) return;
#pragma unroll
    for (int e = 0; e < V; ++e) {
        const int32_t c = c0 + e;
#pragma unroll
        for (int k = 0; k <= K; ++k) {
            double s = k < K ? gw[k][e] : gb[e];
#pragma unroll
            for (int q = 0; q < kSubs1b - 1; ++q) s += red[q][k][lane * V + e];
            partial[((int64_t)g * (K + 1) + k) * C + c] = s;
        }
    }
}

struct Bwd1dGrid {
    uint32_t n_tb, groups_per_item, n_groups, G;
};

// The lane width a launch takes for the caller's widest aligned width vec.
static int bwd1d_vec(int vec, int64_t K) {
    const int vm = bwd1d_vmax((int)K);
    return vec >= 4 && vm >= 4 ? 4 : (vec >= 2 && vm >= 2 ? 2 : 1);
}

#ifndef DW1B_PAIR
#define DW1B_PAIR 1
#endif
#ifndef DW1B_PAIR_WGS
#define DW1B_PAIR_WGS 512
#endif
#ifndef DW1B_Q9
#define DW1B_Q9 2
#endif
#ifndef DW1B_Q15
#define DW1B_Q15 2
#endif
#ifndef DW1B_Q31
#define DW1B_Q31 4
#endif
// Lanes per 16-byte piece (2 or 4) for the widths that take the lane-group
// kernel, 0 for the others.  Those widths are wide enough that the
// four-channel form runs short of registers or lanes (measured on MI355X at
// [32,1500,512], causal, cold caches: K7 67.7 -> 63.9 us with pairs against
// two-channel 8-byte lanes, while K3 and K5 stay faster with four channels
// and 16-byte lanes, 59.6 and 60.5 against 62.0 and 62.9).
constexpr int bwd1d_group_q(int64_t K) {
    return K == 7 ? 2 : (K == 9 ? DW1B_Q9 : (K == 15 ? DW1B_Q15 : (K == 31 ? DW1B_Q31 : 0)));
}
#ifndef DW1B_QB
#define DW1B_QB 4
#endif
// The same for bf16 storage (8 channels per piece): groups of DW1B_QB lanes at
// K = 7, 9 and 15; at K = 31 even two channels per lane would not fit.
constexpr int bwd1d_group_q_bf16(int64_t K) { return K == 7 || K == 9 || K == 15 ? DW1B_QB : 0; }
// The lane-group size a call with 16-byte-aligned tensors takes, or 0.
static int bwd1d_group(int vec, int64_t K, bool bf16) {
    if (!DW1B_PAIR) return 0;
    return bf16 ? (vec >= 8 ? bwd1d_group_q_bf16(K) : 0) : (vec >= 4 ? bwd1d_group_q(K) : 0);
}
// Channels per lane of the lane-group form.
static int bwd1d_group_v(int q, bool bf16) { return (bf16 ? 8 : 4) / q; }

// Persistent grid: G workgroups per channel block.  With 16-byte lanes
// about DW1D_BWD_WGS workgroups in all (one per CU), with narrower lanes
// DW1D_BWD_WGS per channel block (measured on MI355X at [32..128,1500,512]:
// K9 and K5 on 16-byte lanes 2-6% faster with 256 in all than with 512;
// K15 on 8-byte lanes 3% slower with 512 in all than with 1024).
// The lane-group form (V channels per lane, 16-byte accesses) takes about
// DW1B_PAIR_WGS workgroups in all.
static Bwd1dGrid bwd1d_grid(int64_t B, int64_t T, int64_t C, int V, bool group = false) {
    Bwd1dGrid g;
    g.n_tb = (uint32_t)((T + kBwdTile1d - 1) / kBwdTile1d);
    g.groups_per_item = (g.n_tb + kSubs1b - 1) / kSubs1b;
    const uint64_t n = (uint64_t)B * g.groups_per_item;
    g.n_groups = (uint32_t)n;
    const int64_t n_cblk = ((C + V - 1) / V + kLanes1b - 1) / kLanes1b;
    const int64_t wide = group ? DW1B_PAIR_WGS : DW1D_BWD_WGS;
    const int64_t per = V >= 4 || group ? (n_cblk > 0 ? (wide + n_cblk - 1) / n_cblk : 1) : DW1D_BWD_WGS;
    g.G = (uint32_t)(n < (uint64_t)per ? n : (uint64_t)per);
    return g;
}

bool dwconv1d_bwd_supported(int64_t K) {
    return K == 3 || K == 4 || K == 5 || K == 7 || K == 9 || K == 15 || K == 31;
}

// The lane-group form takes 16-byte accesses whatever its lane width: 4 fp32
// or 8 bf16 channels.
int dwconv1d_bwd_max_vec(int64_t K, bool bf16) {
    if (DW1B_PAIR && (bf16 ? bwd1d_group_q_bf16(K) : bwd1d_group_q(K)) > 0) return bf16 ? 8 : 4;
    return bwd1d_vmax((int)K);
}

bool dwconv1d_bwd_fits(int64_t B, int64_t T, int64_t C, int64_t K, int elem_bytes) {
    if (!product_below((int64_t)1 << 31, {T + K + 32, C, elem_bytes})) return false;
    return (uint64_t)B * ((T + kBwdTile1d - 1) / kBwdTile1d) < ((uint64_t)1 << 31);
}

size_t dwconv1d_bwd_workspace(int64_t B, int64_t T, int64_t C, int64_t K) {
    // enough for whichever lane width the pointers' alignment allows
    int64_t P = 0;
    for (int v : {1, 2, 4})
        for (bool group : {false, true}) {
            const int64_t p = bwd1d_grid(B, T, C, v, group).G;
            P = p > P ? p : P;
        }
    const int64_t ch = partial_reduce_chunks(P);
    return (size_t)((P + (ch > 0 ? ch : 1)) * (K + 1) * C * (int64_t)sizeof(double));
}

template <typename S, int V, int K, bool CAUSAL>
static hipError_t launch_bwd1d_typed(const S* x, const S* w, const int32_t* lengths, const S* dy, S* dx,
                                     double* partial, int64_t B, int64_t T, int64_t C, hipStream_t st) {
    const Bwd1dGrid g = bwd1d_grid(B, T, C, V);
    const uint32_t CG = (uint32_t)(C / V);
    const uint32_t n_cblk = (CG + kLanes1b - 1) / kLanes1b;
    if (g.G == 0 || (!dx && !partial)) return hipSuccess;
    hipLaunchKernelGGL((dwconv1d_bwd_kernel<S, V, K, CAUSAL, kBwdTile1d>), dim3(g.G * n_cblk), dim3(kBlock1d), 0, st, x,
                       w, lengths, dy, dx, partial, (int32_t)T, (int32_t)C, g.n_tb, CG, n_cblk, g.groups_per_item,
                       g.n_groups);
    return hipGetLastError();
}

template <typename S, int K, bool CAUSAL, int Q>
static hipError_t launch_bwd1d_group(const S* x, const S* w, const int32_t* lengths, const S* dy, S* dx,
                                     double* partial, int64_t B, int64_t T, int64_t C, hipStream_t st) {
    constexpr int V = 16 / (int)sizeof(S) / Q;
    const Bwd1dGrid g = bwd1d_grid(B, T, C, V, true);
    const uint32_t CG = (uint32_t)(C / V);
    const uint32_t n_cblk = (CG + kLanes1b - 1) / kLanes1b;
    if (g.G == 0 || (!dx && !partial)) return hipSuccess;
    hipLaunchKernelGGL((dwconv1d_bwd_group_kernel<S, K, CAUSAL, kBwdTile1d, Q>), dim3(g.G * n_cblk), dim3(kBlock1d),
                       0, st, x, w, lengths, dy, dx, partial, (int32_t)T, (int32_t)C, g.n_tb, CG, n_cblk,
                       g.groups_per_item, g.n_groups);
    return hipGetLastError();
}

template <typename S, int K, bool CAUSAL>
static hipError_t launch_bwd1d_k(int vec, const void* xv, const void* wv, const int32_t* lengths, const void* dyv,
                                 void* dxv, double* partial, int64_t B, int64_t T, int64_t C, hipStream_t st) {
    constexpr int VMAX = bwd1d_vmax(K);
    const S* x = (const S*)xv;
    const S* w = (const S*)wv;
    const S* dy = (const S*)dyv;
    S* dx = (S*)dxv;
    constexpr int Q = sizeof(S) == 2 ? bwd1d_group_q_bf16(K) : bwd1d_group_q(K);
    if constexpr (Q > 0) {
        if (bwd1d_group(vec, K, sizeof(S) == 2))
            return launch_bwd1d_group<S, K, CAUSAL, Q>(x, w, lengths, dy, dx, partial, B, T, C, st);
    }
    if (vec >= 4 && VMAX >= 4) return launch_bwd1d_typed<S, (VMAX >= 4 ? 4 : 1), K, CAUSAL>(x, w, lengths, dy, dx, partial, B, T, C, st);
    if (vec >= 2 && VMAX >= 2) return launch_bwd1d_typed<S, (VMAX >= 2 ? 2 : 1), K, CAUSAL>(x, w, lengths, dy, dx, partial, B, T, C, st);
    return launch_bwd1d_typed<S, 1, K, CAUSAL>(x, w, lengths, dy, dx, partial, B, T, C, st);
}

hipError_t launch_dwconv1d_bwd(const void* x, const void* w, const int32_t* lengths, const void* dy, void* dx,
                               float* dw, float* db, void* workspace, int64_t B, int64_t T, int64_t C, int64_t K,
                               bool causal, bool bf16, int vec, hipStream_t st) {
    double* partial = (dw || db) ? (double*)workspace : nullptr;
    hipError_t e = hipSuccess;
#define DW1B_CASE(KK)                                                                                        \
    case KK:                                                                                                 \
        if (bf16)                                                                                            \
            e = causal ? launch_bwd1d_k<uint16_t, KK, true>(vec, x, w, lengths, dy, dx, partial, B, T, C, st)   \
                       : launch_bwd1d_k<uint16_t, KK, false>(vec, x, w, lengths, dy, dx, partial, B, T, C, st); \
        else                                                                                                 \
            e = causal ? launch_bwd1d_k<float, KK, true>(vec, x, w, lengths, dy, dx, partial, B, T, C, st)      \
                       : launch_bwd1d_k<float, KK, false>(vec, x, w, lengths, dy, dx, partial, B, T, C, st);    \
        break;
    switch (K) {
        DW1B_CASE(3)
        DW1B_CASE(4)
        DW1B_CASE(5)
        DW1B_CASE(7)
        DW1B_CASE(9)
        DW1B_CASE(15)
        DW1B_CASE(31)
        default: return hipErrorInvalidValue;
    }
#undef DW1B_CASE
    if (e != hipSuccess || !partial) return e;
    const int q = bwd1d_group(vec, K, bf16);
    const int64_t P = (q ? bwd1d_grid(B, T, C, bwd1d_group_v(q, bf16), true) : bwd1d_grid(B, T, C, bwd1d_vec(vec, K))).G;
    RowOutputs out = {};
    out.n = 2;
    out.p[0] = dw; out.first[0] = 0; out.count[0] = (int32_t)K;
    out.p[1] = db; out.first[1] = (int32_t)K; out.count[1] = 1;
    return launch_partial_reduce(partial, P, (int32_t)(K + 1), C, partial + P * (K + 1) * C, out, st);
}

}  // namespace dw
