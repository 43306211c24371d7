// fp32 block attention on the vector ALUs (the exact-precision path).
// Computes, for each query row i and head h, the softmax over the keys of this block whose
// global position is not later than the query's ("Context parallelism -- splitting the
// sequence across GPUs", attention definition with j <= i; "On Context Parallelism",
// section Peer-to-peer / Forward: attention on global positions returning (out, lse)).
//
// One wave per block; each lane owns one query row of one head and keeps q, the running
// output, the running max m and the running sum l in registers.  K/V tiles of 64 keys and
// their positions are staged in LDS and read by broadcast.  Only tiles whose first key is
// visible to the block's last query are visited.
#include "cpattn_internal.h"
#include "merge_math.h"

#include <math.h>

namespace cpattn {
namespace {

constexpr int kRows = 64;   // queries per block (one per lane)
constexpr int kTile = 64;   // keys per LDS tile
constexpr int kSub = 16;    // keys folded per online-softmax update

template <int D>
__global__ void __launch_bounds__(kRows) block_fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const int64_t* __restrict__ q_pos, const int64_t* __restrict__ kv_pos, float* __restrict__ out,
    float* __restrict__ lse, int64_t seq_q, int64_t seq_kv, int32_t heads_q, int32_t heads_kv,
    float scale, int merge) {
    __shared__ float ks[kTile][D];
    __shared__ float vs[kTile][D];
    __shared__ int64_t ps[kTile];

    const int lane = threadIdx.x;
    const int64_t h = blockIdx.y, b = blockIdx.z;
    const int64_t kvh = h / (heads_q / heads_kv);
    const int64_t row0 = (int64_t)blockIdx.x * kRows;
    const int64_t i = row0 + lane;
    const bool valid = i < seq_q;
    const int64_t last = (row0 + kRows < seq_q ? row0 + kRows : seq_q) - 1;
    const int64_t p_last = q_pos[last];
    const int64_t p = valid ? q_pos[i] : INT64_MIN;

    // number of keys whose position is <= the block's last query position
    int64_t lo = 0, hi = seq_kv;
    while (lo < hi) {
        const int64_t mid = (lo + hi) / 2;
        if (kv_pos[mid] <= p_last) lo = mid + 1; else hi = mid;
    }
    const int64_t n_keys = lo;

    float qr[D], o[D];
    const float* qrow = q + ((b * seq_q + (valid ? i : 0)) * heads_q + h) * D;
#pragma unroll
    for (int d = 0; d < D; ++d) { qr[d] = valid ? qrow[d] : 0.f; o[d] = 0.f; }
    float m = -INFINITY, l = 0.f;

    for (int64_t j0 = 0; j0 < n_keys; j0 += kTile) {
        __syncthreads();
        for (int e = lane; e < kTile * D; e += kRows) {
            const int r = e / D, d = e % D;
            const int64_t j = j0 + r;
            const bool in = j < seq_kv;
            const int64_t off = ((b * seq_kv + (in ? j : 0)) * heads_kv + kvh) * D + d;
            ks[r][d] = in ? k[off] : 0.f;
            vs[r][d] = in ? v[off] : 0.f;
        }
        if (lane < kTile) ps[lane] = (j0 + lane < seq_kv) ? kv_pos[j0 + lane] : INT64_MAX;
        __syncthreads();
        // keys of the tile in sub-blocks of kSub, each folded in with the running max
#pragma unroll 1
        for (int r0 = 0; r0 < kTile; r0 += kSub) {
            float sc[kSub];
            float tmax = -INFINITY;
#pragma unroll
            for (int r = 0; r < kSub; ++r) {
                float dot = 0.f;
#pragma unroll
                for (int d = 0; d < D; ++d) dot = fmaf(qr[d], ks[r0 + r][d], dot);
                sc[r] = (ps[r0 + r] <= p) ? dot * scale : -INFINITY;
                tmax = fmaxf(tmax, sc[r]);
            }
            const float m_new = fmaxf(m, tmax);
            if (m_new == -INFINITY) continue;  // nothing visible to this row yet
            const float alpha = expf(m - m_new);
            l *= alpha;
#pragma unroll
            for (int d = 0; d < D; ++d) o[d] *= alpha;
#pragma unroll
            for (int r = 0; r < kSub; ++r) {
                const float w = expf(sc[r] - m_new);
                l += w;
#pragma unroll
                for (int d = 0; d < D; ++d) o[d] = fmaf(w, vs[r0 + r][d], o[d]);
            }
            m = m_new;
        }
    }
    if (!valid) return;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* orow = out + ((b * seq_q + i) * heads_q + h) * D;
    float* lrow = lse + (b * heads_q + h) * seq_q + i;
    const float lse_t = l > 0.f ? m + logf(l) : -INFINITY;
    if (merge) {
        const MergeWeights mw = merge_weights(*lrow, lse_t);
#pragma unroll
        for (int d = 0; d < D; ++d) orow[d] = merge_value(orow[d], o[d] * inv, mw.w_old, mw.w_new);
        *lrow = mw.lse;
    } else {
#pragma unroll
        for (int d = 0; d < D; ++d) orow[d] = o[d] * inv;
        *lrow = lse_t;
    }
}

// A block with no keys at all: every row is empty (out = 0, lse = -inf).
__global__ void __launch_bounds__(256) empty_rows_kernel(float* __restrict__ out, float* __restrict__ lse,
                                                         int64_t n_out, int64_t n_lse) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n_out; e += stride) out[e] = 0.f;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n_lse; e += stride) lse[e] = -INFINITY;
}

// Merging an empty result (0, -inf) into an accumulator: one thread per (b, h, i) row.
// Rows with a finite lse keep their bits; rows at -inf become (0, -inf).
__global__ void __launch_bounds__(256) merge_empty_kernel(float* __restrict__ out, float* __restrict__ lse,
                                                          int64_t seq, int32_t heads, int32_t head_dim,
                                                          int64_t n_rows) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t li = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; li < n_rows; li += stride) {
        // lse index (b*heads + h)*seq + i  <->  out row (b*seq + i)*heads + h
        const int64_t i = li % seq, bh = li / seq;
        const int64_t h = bh % heads, b = bh / heads;
        const MergeWeights mw = merge_weights(lse[li], -INFINITY);
        float* orow = out + ((b * seq + i) * heads + h) * head_dim;
        for (int d = 0; d < head_dim; ++d) orow[d] = merge_value(orow[d], 0.f, mw.w_old, mw.w_new);
        lse[li] = mw.lse;
    }
}

}  // namespace

hipError_t launch_block_fwd_empty(const BlockFwdArgs& a, hipStream_t stream) {
    const int64_t n_lse = (int64_t)a.batch * a.heads_q * a.seq_q;
    if (a.merge) {
        const int64_t rb = (n_lse + 255) / 256;
        hipLaunchKernelGGL(merge_empty_kernel, dim3((unsigned)(rb < 16384 ? rb : 16384)), dim3(256), 0, stream,
                           a.out, a.lse, a.seq_q, a.heads_q, a.head_dim, n_lse);
        return hipGetLastError();
    }
    const int64_t n_out = n_lse * a.head_dim;
    const int64_t blocks = (n_out + 255) / 256;
    hipLaunchKernelGGL(empty_rows_kernel, dim3((unsigned)(blocks < 16384 ? blocks : 16384)), dim3(256), 0,
                       stream, a.out, a.lse, n_out, n_lse);
    return hipGetLastError();
}

hipError_t launch_block_fwd_f32(const BlockFwdArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)((a.seq_q + kRows - 1) / kRows), (unsigned)a.heads_q, (unsigned)a.batch);
    const float* q = (const float*)a.q;
    const float* k = (const float*)a.k;
    const float* v = (const float*)a.v;
    if (a.head_dim == 64)
        hipLaunchKernelGGL(block_fwd_f32_kernel<64>, grid, dim3(kRows), 0, stream, q, k, v, a.q_pos,
                           a.kv_pos, a.out, a.lse, a.seq_q, a.seq_kv, a.heads_q, a.heads_kv, a.scale, (int)a.merge);
    else
        hipLaunchKernelGGL(block_fwd_f32_kernel<128>, grid, dim3(kRows), 0, stream, q, k, v, a.q_pos,
                           a.kv_pos, a.out, a.lse, a.seq_q, a.seq_kv, a.heads_q, a.heads_kv, a.scale, (int)a.merge);
    return hipGetLastError();
}

}  // namespace cpattn
