// Zigzag positions of one rank's local tokens.
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

}  // namespace

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
