// Zigzag positions of one rank's local tokens (or of every rank's, one row per rank).
// "On Context Parallelism", section All-gather: 2C chunks of t tokens; rank r holds chunk r
// then chunk 2C-1-r.  The positions are written in that local order.
#include "cpattn_internal.h"

namespace cpattn {
namespace {

__global__ void __launch_bounds__(256) zigzag_index_kernel(int64_t t, int64_t early, int64_t late,
                                                           int64_t* __restrict__ out) {
    const int64_t n = 2 * t;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        out[i] = (i < t) ? early * t + i : late * t + (i - t);
    }
}

// Every rank's positions at once: row r of out (2t entries) is rank r's local order; the
// rank is the grid's second dimension.
__global__ void __launch_bounds__(256) zigzag_index_all_kernel(int64_t t, int64_t n_chunks,
                                                               int64_t* __restrict__ out) {
    const int64_t r = blockIdx.y;
    const int64_t n = 2 * t;
    int64_t* row = out + r * n;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        row[i] = (i < t) ? r * t + i : (n_chunks - 1 - r) * t + (i - t);
    }
}

}  // namespace

hipError_t launch_zigzag_index_all(int64_t chunk_len, int32_t cp_size, int64_t* positions,
                                   hipStream_t stream) {
    const int64_t n = 2 * chunk_len;
    const int64_t blocks = (n + 255) / 256;
    const unsigned grid = (unsigned)(blocks < 65536 ? blocks : 65536);
    hipLaunchKernelGGL(zigzag_index_all_kernel, dim3(grid, (unsigned)cp_size), dim3(256), 0, stream,
                       chunk_len, 2 * (int64_t)cp_size, positions);
    return hipGetLastError();
}

hipError_t launch_zigzag_index(int64_t chunk_len, int64_t early_chunk, int64_t late_chunk,
                               int64_t* positions, hipStream_t stream) {
    const int64_t n = 2 * chunk_len;
    const int64_t blocks = (n + 255) / 256;
    const unsigned grid = (unsigned)(blocks < 65536 ? blocks : 65536);
    hipLaunchKernelGGL(zigzag_index_kernel, dim3(grid), dim3(256), 0, stream, chunk_len,
                       early_chunk, late_chunk, positions);
    return hipGetLastError();
}

}  // namespace cpattn
