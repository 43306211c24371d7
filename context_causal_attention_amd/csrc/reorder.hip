// Chunk reorder between the all-gather's rank order and global sequence order.
// "On Context Parallelism", section All-gather: gathering the zigzag shards in rank order
// yields chunks 0, 2C-1, 1, 2C-2, ... (0,7,1,6,2,5,3,4 at C=4); attention needs them in
// sequence order, and the backward needs the inverse.  Gathered slot k holds chunk k/2
// for even k and chunk 2C-1-(k-1)/2 for odd k.
//
// A pure byte copy of B*2C contiguous chunks of t*row_bytes bytes each, bandwidth-bound:
// each block copies a contiguous span of one destination chunk, one 16-byte access per lane
// (byte accesses when sizes or pointers are not 16-byte aligned); the 16-byte path streams
// (stream_access.h).  All offsets are 64-bit.
#include "cpattn_internal.h"
#include "stream_access.h"

namespace cpattn {
namespace {

constexpr int kThreads = 256;
constexpr int kVecPerThread = 1;


__device__ inline int64_t slot_of_chunk(int64_t c, int64_t C) {
    return c < C ? 2 * c : 2 * (2 * C - 1 - c) + 1;
}
__device__ inline int64_t chunk_of_slot(int64_t k, int64_t C) {
    return (k % 2 == 0) ? k / 2 : 2 * C - 1 - (k - 1) / 2;
}

// grid.x = blocks per chunk, grid.y = 2C destination chunks, grid.z = batch
template <typename T>
__global__ void __launch_bounds__(kThreads) reorder_kernel(const T* __restrict__ in, T* __restrict__ out,
                                                           int64_t chunk_elems, int64_t seq_elems,
                                                           int32_t C, int32_t dir) {
    const int64_t dst = blockIdx.y;
    const int64_t src = (dir == 0) ? slot_of_chunk(dst, C) : chunk_of_slot(dst, C);
    const int64_t b = blockIdx.z;
    const T* s = in + b * seq_elems + src * chunk_elems;
    T* d = out + b * seq_elems + dst * chunk_elems;
    const int64_t base = (int64_t)blockIdx.x * (kThreads * kVecPerThread) + threadIdx.x;
    T tmp[kVecPerThread];
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
        const int64_t e = base + (int64_t)u * kThreads;
        if (e < chunk_elems) tmp[u] = load_stream(s + e);
    }
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
        const int64_t e = base + (int64_t)u * kThreads;
        if (e < chunk_elems) store_stream(d + e, tmp[u]);
    }
}

}  // namespace

hipError_t launch_reorder_gathered(const void* in, void* out, int32_t batch, int64_t seq_len,
                                   int64_t row_bytes, int32_t cp_size, int32_t dir,
                                   hipStream_t stream) {
    const int64_t chunk_bytes = (seq_len / (2 * (int64_t)cp_size)) * row_bytes;
    const bool vec = (chunk_bytes % 16 == 0) && ((uintptr_t)in % 16 == 0) && ((uintptr_t)out % 16 == 0);
    const int64_t elem = vec ? 16 : 1;
    const int64_t chunk_elems = chunk_bytes / elem;
    const int64_t seq_elems = seq_len * row_bytes / elem;
    const int64_t per_block = kThreads * kVecPerThread;
    const int64_t bx = (chunk_elems + per_block - 1) / per_block;
    const dim3 grid((unsigned)bx, (unsigned)(2 * cp_size), (unsigned)batch);
    if (vec)
        hipLaunchKernelGGL(reorder_kernel<v4u>, grid, dim3(kThreads), 0, stream,
                           (const v4u*)in, (v4u*)out, chunk_elems, seq_elems, cp_size, dir);
    else
        hipLaunchKernelGGL(reorder_kernel<uint8_t>, grid, dim3(kThreads), 0, stream,
                           (const uint8_t*)in, (uint8_t*)out, chunk_elems, seq_elems, cp_size, dir);
    return hipGetLastError();
}

}  // namespace cpattn
