// Fixed-order reduction of per-workgroup fp64 partials, shared by the
// backward kernels.  The partials form a [P][K][C] fp64 matrix (one row of
// K*C sums per workgroup); the result is its sum over P, rounded to float and
// written to up to four outputs, each taking a range of the K rows.
//
// Up to 2048 partials are summed in one pass (16 sub-rows per column).
// Beyond that, two levels, so that enough workgroups share the reading: level 1 sums
// chunks of up to kSumChunk partial rows and writes one fp64 row per chunk;
// level 2 sums the chunk rows.  Each level's workgroup is kSumRows sub-rows x
// kSumCols columns: sub-row q adds rows q, q + kSumRows, ... of its chunk,
// then the sub-rows are added in order through LDS.  The order of every
// addition is fixed, so the result is bitwise repeatable.
#include "common.h"
#include "launch.h"

namespace dw {

constexpr int kSumCols = 64, kSumRows = 4, kSumChunk = 64;

__device__ __forceinline__ double sum_chunk(const double* __restrict__ in, int32_t ncol, int32_t r0, int32_t r1,
                                            int32_t col, double (*acc)[kSumCols]) {
    const int32_t sub = threadIdx.x / kSumCols, lane = threadIdx.x % kSumCols;
    double s = 0.0;
    if (col < ncol) {
#pragma unroll 4
        for (int32_t r = r0 + sub; r < r1; r += kSumRows) s += in[(int64_t)r * ncol + col];
    }
    acc[sub][lane] = s;
    __syncthreads();
    double t = acc[0][lane];
#pragma unroll
    for (int q = 1; q < kSumRows; ++q) t += acc[q][lane];
    return t;
}

__global__ __launch_bounds__(kSumCols* kSumRows) void partial_reduce1_kernel(
    const double* __restrict__ partial, double* __restrict__ chunk_sum, int32_t ncol, int32_t P) {
    __shared__ double acc[kSumRows][kSumCols];
    const int32_t col = blockIdx.x * kSumCols + threadIdx.x % kSumCols;  // column = k * C + c
    const int32_t p0 = blockIdx.y * kSumChunk, p1 = min(P, p0 + kSumChunk);
    const double t = sum_chunk(partial, ncol, p0, p1, col, acc);
    if (threadIdx.x < kSumCols && col < ncol) chunk_sum[(int64_t)blockIdx.y * ncol + col] = t;
}

__global__ __launch_bounds__(kSumCols* kSumRows) void partial_reduce2_kernel(
    const double* __restrict__ chunk_sum, RowOutputs out, int32_t K, int32_t C, int32_t nchunk) {
    __shared__ double acc[kSumRows][kSumCols];
    const int32_t ncol = K * C;
    const int32_t col = blockIdx.x * kSumCols + threadIdx.x % kSumCols;
    const double t = sum_chunk(chunk_sum, ncol, 0, nchunk, col, acc);
    if (threadIdx.x >= kSumCols || col >= ncol) return;
    const int32_t k = col / C, c = col % C;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        if (s < out.n && out.p[s] && k >= out.first[s] && k < out.first[s] + out.count[s])
            out.p[s][(int64_t)(k - out.first[s]) * C + c] = (float)t;
    }
}

// One pass for up to kOnePassMax partials: kOnePassRows sub-rows x kSumCols
// columns per workgroup, sub-row q adding rows q, q + kOnePassRows, ...
constexpr int kOnePassRows = 16, kOnePassMax = 2048;

__global__ __launch_bounds__(kSumCols* kOnePassRows) void partial_reduce_onepass_kernel(
    const double* __restrict__ partial, RowOutputs out, int32_t K, int32_t C, int32_t P) {
    __shared__ double acc[kOnePassRows][kSumCols];
    const int32_t ncol = K * C;
    const int32_t lane = threadIdx.x % kSumCols, sub = threadIdx.x / kSumCols;
    const int32_t col = blockIdx.x * kSumCols + lane;
    double s = 0.0;
    if (col < ncol) {
#pragma unroll 4
        for (int32_t r = sub; r < P; r += kOnePassRows) s += partial[(int64_t)r * ncol + col];
    }
    acc[sub][lane] = s;
    __syncthreads();
    if (sub != 0 || col >= ncol) return;
    double t = acc[0][lane];
#pragma unroll
    for (int q = 1; q < kOnePassRows; ++q) t += acc[q][lane];
    const int32_t k = col / C, c = col % C;
#pragma unroll
    for (int o = 0; o < 4; ++o) {
        if (o < out.n && out.p[o] && k >= out.first[o] && k < out.first[o] + out.count[o])
            out.p[o][(int64_t)(k - out.first[o]) * C + c] = (float)t;
    }
}

int64_t partial_reduce_chunks(int64_t P) { return (P + kSumChunk - 1) / kSumChunk; }

hipError_t launch_partial_reduce(const double* partial, int64_t P, int32_t K, int64_t C, double* chunk_sum,
                                 RowOutputs out, hipStream_t st) {
    const int32_t ncol = (int32_t)(K * C);
    const int32_t nchunk = (int32_t)partial_reduce_chunks(P);
    const uint32_t ncblk = (uint32_t)((ncol + kSumCols - 1) / kSumCols);
    if (P <= kOnePassMax) {
        hipLaunchKernelGGL(partial_reduce_onepass_kernel, dim3(ncblk), dim3(kSumCols * kOnePassRows), 0, st, partial,
                           out, K, (int32_t)C, (int32_t)P);
        return hipGetLastError();
    }
    if (nchunk > 0) {
        hipLaunchKernelGGL(partial_reduce1_kernel, dim3(ncblk, (uint32_t)nchunk), dim3(kSumCols * kSumRows), 0, st,
                           partial, chunk_sum, ncol, (int32_t)P);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(partial_reduce2_kernel, dim3(ncblk), dim3(kSumCols * kSumRows), 0, st, chunk_sum, out, K,
                       (int32_t)C, nchunk);
    return hipGetLastError();
}

}  // namespace dw
