// In-place merge of a completed partial attention result into an accumulator, with the
// arithmetic of merge_math.h ("On Context Parallelism", section Peer-to-peer).
//
// Bandwidth-bound: per row of head_dim floats it reads out and out_tile and writes out.
// A block owns kRows consecutive (b, i, h) rows: it first turns their lse pairs into the two
// weights (in LDS), then streams the rows with 16-byte non-temporal accesses, one per lane
// (stream_access.h).
#include "cpattn_internal.h"
#include "merge_math.h"
#include "stream_access.h"

#include <math.h>

namespace cpattn {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 8;   // 8 rows x 128 floats = one 16-byte access per lane

__global__ void __launch_bounds__(kThreads) lse_merge_kernel(
    float* __restrict__ out, float* __restrict__ lse, const float* __restrict__ out_t,
    const float* __restrict__ lse_t, int64_t seq, int32_t heads, int32_t head_dim, int64_t n_rows) {
    __shared__ float w_old[kRows];
    __shared__ float w_new[kRows];
    const int64_t row0 = (int64_t)blockIdx.x * kRows;
    const int tid = threadIdx.x;
    if (tid < kRows && row0 + tid < n_rows) {
        // row = (b*seq + i)*heads + h  <->  lse index (b*heads + h)*seq + i
        const int64_t row = row0 + tid;
        const int64_t h = row % heads;
        const int64_t bi = row / heads;
        const int64_t i = bi % seq, b = bi / seq;
        const int64_t li = (b * heads + h) * seq + i;
        const MergeWeights mw = merge_weights(lse[li], lse_t[li]);
        w_old[tid] = mw.w_old;
        w_new[tid] = mw.w_new;
        lse[li] = mw.lse;
    }
    __syncthreads();
    const int vec_per_row = head_dim / 4;
    const int rows_here = (int)((n_rows - row0) < kRows ? (n_rows - row0) : kRows);
    const int n_vec = rows_here * vec_per_row;
    v4f* o4 = reinterpret_cast<v4f*>(out + row0 * head_dim);
    const v4f* t4 = reinterpret_cast<const v4f*>(out_t + row0 * head_dim);
    for (int e = tid; e < n_vec; e += kThreads) {
        const int r = e / vec_per_row;
        const float a = w_old[r], c = w_new[r];
        const v4f x = load_stream(o4 + e), y = load_stream(t4 + e);
        v4f z;
        z.x = merge_value(x.x, y.x, a, c);
        z.y = merge_value(x.y, y.y, a, c);
        z.z = merge_value(x.z, y.z, a, c);
        z.w = merge_value(x.w, y.w, a, c);
        store_stream(o4 + e, z);
    }
}

}  // namespace

hipError_t launch_lse_merge(float* out, float* lse, const float* out_tile, const float* lse_tile,
                            int32_t batch, int64_t seq, int32_t heads, int32_t head_dim,
                            hipStream_t stream) {
    const int64_t n_rows = (int64_t)batch * seq * heads;
    const int64_t blocks = (n_rows + kRows - 1) / kRows;
    hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, out, lse,
                       out_tile, lse_tile, seq, heads, head_dim, n_rows);
    return hipGetLastError();
}

}  // namespace cpattn
