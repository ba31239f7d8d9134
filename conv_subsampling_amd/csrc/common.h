// Shared device helpers for the gfx950 depthwise-convolution kernels:
// native vector types, bf16 <-> fp32 conversion, per-item length clamping
// and the XCD-aware block order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dw {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// MI355X dispatches consecutive workgroups round-robin over its 8 XCDs, each
// with a private L2.  Kernels whose neighbouring tiles share halo rows
// renumber their blocks so that every XCD works through one contiguous range
// of logical tiles, and the shared rows are found in that XCD's L2.
constexpr int kNumXcd = 8;

#ifndef DW_XCD_REMAP
#define DW_XCD_REMAP 1
#endif
__device__ __forceinline__ uint32_t xcd_contiguous_block(uint32_t bid, uint32_t nblocks) {
    if (!DW_XCD_REMAP) return bid;
    uint32_t q = nblocks / kNumXcd, r = nblocks % kNumXcd;
    uint32_t x = bid % kNumXcd, j = bid / kNumXcd;
    return x * q + (x < r ? x : r) + j;
}

__device__ __forceinline__ int64_t item_length(const int32_t* lengths, int64_t b, int64_t T) {
    int64_t l = lengths ? (int64_t)lengths[b] : T;
    return l < 0 ? 0 : (l > T ? T : l);
}

// bf16 is the upper half of an IEEE binary32, so widening is exact.
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Round two binary32 values to bf16, nearest-even, packed low/high.  On gfx950
// this is the single hardware conversion v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint32_t bf16_bits_rne(float f) { return pack_bf16x2(f, 0.0f) & 0xffffu; }

// ---------------------------------------------------------------------------
// A group of V consecutive channels, held as floats in registers.
// V * sizeof(storage) is the width of one memory access (at most 16 bytes).
// ---------------------------------------------------------------------------
template <int V>
struct Vf {
    float v[V];
};

// Raw buffer resources.  A buffer load whose byte offset is at or beyond the
// resource's size returns zero without touching memory, and a store there is
// dropped.  A negative 32-bit offset wraps to a huge unsigned one, so it is
// out of range too.  The kernels give each batch item its own resource whose
// size ends at the item's valid length: frames beyond the length, and frames
// left of zero, then read as the zeros the masks and the padding call for,
// with no branch and no memory traffic.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kBufferFlags = 0x00020000;  // dword 3 of a raw (untyped) gfx9 buffer resource
#ifndef DW_STORE_NT
#define DW_STORE_NT 1
#endif
constexpr int kNonTemporal = DW_STORE_NT ? 2 : 0;  // store cache policy: 2 = no reuse expected
#ifndef DW_LOAD_POLICY
#define DW_LOAD_POLICY 0
#endif
constexpr int kLoadPolicy = DW_LOAD_POLICY;      // load cache policy of the streamed operands

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferFlags);
}

template <typename S, int V>
struct Buf;

template <int V>
struct Buf<float, V> {
    static_assert(V == 1 || V == 2 || V == 4, "float vectors are 4, 8 or 16 bytes");
    // P: the cache policy bits of the load (the streamed operands' default).
    template <int P = kLoadPolicy>
    static __device__ __forceinline__ Vf<V> load(rsrc_t r, uint32_t off) {
        Vf<V> a;
        if constexpr (V == 4) {
            u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, P);
            a.v[0] = __uint_as_float(t.x); a.v[1] = __uint_as_float(t.y);
            a.v[2] = __uint_as_float(t.z); a.v[3] = __uint_as_float(t.w);
        } else if constexpr (V == 2) {
            u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, P);
            a.v[0] = __uint_as_float(t.x); a.v[1] = __uint_as_float(t.y);
        } else {
            a.v[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, P));
        }
        return a;
    }
    // P: the cache policy bits of the store (non-temporal by default).
    template <int P = kNonTemporal>
    static __device__ __forceinline__ void store(rsrc_t r, uint32_t off, const Vf<V>& a) {
        if constexpr (V == 4) {
            u32x4 t = {__float_as_uint(a.v[0]), __float_as_uint(a.v[1]), __float_as_uint(a.v[2]),
                       __float_as_uint(a.v[3])};
            __builtin_amdgcn_raw_buffer_store_b128(t, r, off, 0, P);
        } else if constexpr (V == 2) {
            u32x2 t = {__float_as_uint(a.v[0]), __float_as_uint(a.v[1])};
            __builtin_amdgcn_raw_buffer_store_b64(t, r, off, 0, P);
        } else {
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(a.v[0]), r, off, 0, P);
        }
    }
};

template <int V>
struct Buf<uint16_t, V> {
    static_assert(V == 1 || V == 2 || V == 4 || V == 8, "bf16 vectors are 2 to 16 bytes");
    // P: the cache policy bits of the load (the streamed operands' default).
    template <int P = kLoadPolicy>
    static __device__ __forceinline__ Vf<V> load(rsrc_t r, uint32_t off) {
        Vf<V> a;
        if constexpr (V == 8) {
            u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, P);
            a.v[0] = bf16_lo(t.x); a.v[1] = bf16_hi(t.x); a.v[2] = bf16_lo(t.y); a.v[3] = bf16_hi(t.y);
            a.v[4] = bf16_lo(t.z); a.v[5] = bf16_hi(t.z); a.v[6] = bf16_lo(t.w); a.v[7] = bf16_hi(t.w);
        } else if constexpr (V == 4) {
            u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, P);
            a.v[0] = bf16_lo(t.x); a.v[1] = bf16_hi(t.x); a.v[2] = bf16_lo(t.y); a.v[3] = bf16_hi(t.y);
        } else if constexpr (V == 2) {
            uint32_t t = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, P);
            a.v[0] = bf16_lo(t); a.v[1] = bf16_hi(t);
        } else {
            a.v[0] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, P) << 16);
        }
        return a;
    }
    // P: the cache policy bits of the store (non-temporal by default).
    template <int P = kNonTemporal>
    static __device__ __forceinline__ void store(rsrc_t r, uint32_t off, const Vf<V>& a) {
        if constexpr (V == 8) {
            u32x4 t = {pack_bf16x2(a.v[0], a.v[1]), pack_bf16x2(a.v[2], a.v[3]),
                       pack_bf16x2(a.v[4], a.v[5]), pack_bf16x2(a.v[6], a.v[7])};
            __builtin_amdgcn_raw_buffer_store_b128(t, r, off, 0, P);
        } else if constexpr (V == 4) {
            u32x2 t = {pack_bf16x2(a.v[0], a.v[1]), pack_bf16x2(a.v[2], a.v[3])};
            __builtin_amdgcn_raw_buffer_store_b64(t, r, off, 0, P);
        } else if constexpr (V == 2) {
            __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(a.v[0], a.v[1]), r, off, 0, P);
        } else {
            __builtin_amdgcn_raw_buffer_store_b16((unsigned short)bf16_bits_rne(a.v[0]), r, off, 0, P);
        }
    }
};

// Loads of small, reused operands (weights, biases) through the cache.  The
// host only picks a vector width V when these pointers are aligned to V
// elements, so the vector loads below are aligned.
template <typename S, int V>
__device__ __forceinline__ Vf<V> load_param(const S* p) {
    Vf<V> a;
    if constexpr (sizeof(S) == 4 && V == 4) {
        f32x4 t = *reinterpret_cast<const f32x4*>(p);
        a.v[0] = t.x; a.v[1] = t.y; a.v[2] = t.z; a.v[3] = t.w;
    } else if constexpr (sizeof(S) == 4 && V == 2) {
        f32x2 t = *reinterpret_cast<const f32x2*>(p);
        a.v[0] = t.x; a.v[1] = t.y;
    } else if constexpr (sizeof(S) == 2 && V == 8) {
        u32x4 t = *reinterpret_cast<const u32x4*>(p);
        a.v[0] = bf16_lo(t.x); a.v[1] = bf16_hi(t.x); a.v[2] = bf16_lo(t.y); a.v[3] = bf16_hi(t.y);
        a.v[4] = bf16_lo(t.z); a.v[5] = bf16_hi(t.z); a.v[6] = bf16_lo(t.w); a.v[7] = bf16_hi(t.w);
    } else if constexpr (sizeof(S) == 2 && V == 4) {
        u32x2 t = *reinterpret_cast<const u32x2*>(p);
        a.v[0] = bf16_lo(t.x); a.v[1] = bf16_hi(t.x); a.v[2] = bf16_lo(t.y); a.v[3] = bf16_hi(t.y);
    } else if constexpr (sizeof(S) == 2 && V == 2) {
        uint32_t t = *reinterpret_cast<const uint32_t*>(p);
        a.v[0] = bf16_lo(t); a.v[1] = bf16_hi(t);
    } else {
#pragma unroll
        for (int i = 0; i < V; ++i) {
            if constexpr (sizeof(S) == 4) a.v[i] = p[i];
            else a.v[i] = __uint_as_float((uint32_t)p[i] << 16);
        }
    }
    return a;
}

// One stored value (fp32, or bf16 bits) widened exactly to fp32.
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

template <int V>
__device__ __forceinline__ Vf<V> vzero() {
    Vf<V> r;
#pragma unroll
    for (int i = 0; i < V; ++i) r.v[i] = 0.0f;
    return r;
}

}  // namespace dw
