// HBM streaming probe for gfx950: moves an exact number of bytes with the
// plainest streaming kernel (one 16-byte access per thread, a huge grid).
// Measurement only; see include/dwprobe.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dwprobe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kBufferFlags = 0x00020000;  // dword 3 of a raw (untyped) gfx9 buffer resource
constexpr int kBlock = 256;
constexpr int64_t kChunk = (int64_t)kBlock * 16;  // bytes per workgroup

// Each workgroup owns one 4 KiB chunk of the transfer and addresses it
// through buffer resources sized to what is left of each side: a load past
// read_bytes returns zero with no traffic, a store past write_bytes is
// dropped.  So the grid covers max(read, write) with no branch.
template <int PL, int PS>
__global__ __launch_bounds__(kBlock) void stream_probe_kernel(const uint8_t* __restrict__ src,
                                                              uint8_t* __restrict__ dst, int64_t nr, int64_t nw) {
    const int64_t base = (int64_t)blockIdx.x * kChunk;
    const int64_t r = nr - base, w = nw - base;
    const uint32_t rb = (uint32_t)(r <= 0 ? 0 : (r > kChunk ? kChunk : r));
    const uint32_t wb = (uint32_t)(w <= 0 ? 0 : (w > kChunk ? kChunk : w));
    const rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src + (rb ? base : 0)), (short)0,
                                                        (int)rb, kBufferFlags);
    const rsrc_t dr = __builtin_amdgcn_make_buffer_rsrc(dst + (wb ? base : 0), (short)0, (int)wb, kBufferFlags);
    const uint32_t off = threadIdx.x * 16u;
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(sr, off, 0, PL);
    __builtin_amdgcn_raw_buffer_store_b128(v, dr, off, 0, PS);
}

}  // namespace

extern "C" int dw_probe_stream(const void* src, void* dst, int64_t read_bytes, int64_t write_bytes, int policy,
                               void* stream) {
    if (read_bytes < 0 || write_bytes < 0 || read_bytes > ((int64_t)1 << 42) || write_bytes > ((int64_t)1 << 42))
        return -1;
    const int64_t nr = read_bytes & ~(int64_t)15, nw = write_bytes & ~(int64_t)15;
    if ((nr && !src) || (nw && !dst)) return -1;
    if (((uintptr_t)src & 15u) || ((uintptr_t)dst & 15u)) return -1;
    if (policy < 0 || policy > 2) return -1;
    const int64_t n = nr > nw ? nr : nw;
    if (n == 0) return 0;
    const dim3 grid((uint32_t)((n + kChunk - 1) / kChunk)), block(kBlock);
    const hipStream_t st = (hipStream_t)stream;
    auto s = (const uint8_t*)src;
    auto d = (uint8_t*)dst;
    if (policy == 0)
        hipLaunchKernelGGL((stream_probe_kernel<0, 0>), grid, block, 0, st, s, d, nr, nw);
    else if (policy == 1)
        hipLaunchKernelGGL((stream_probe_kernel<2, 2>), grid, block, 0, st, s, d, nr, nw);
    else
        hipLaunchKernelGGL((stream_probe_kernel<2, 18>), grid, block, 0, st, s, d, nr, nw);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}
