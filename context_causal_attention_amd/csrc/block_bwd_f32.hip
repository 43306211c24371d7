// Attention backward helpers and the fp32 block backward (vector ALUs).
//
// delta: D_i = <dout_i, out_i> per (b, h, i), the row term of the softmax derivative
// ("On Context Parallelism", section Peer-to-peer / Backward: the backward of each step uses
// the saved output; the chain rule of the softmax gives ds_ij = p_ij (dp_ij - D_i)).
// Bandwidth-bound and small (once per rank share): 16 lanes per row, 16-byte reads of out.
//
// fp32 block backward, same arithmetic as the bf16 path without any rounding to bf16:
//   dq kernel: one lane per query row (q, dout, dq in registers); K/V tiles in LDS, read by
//   broadcast.  dk/dv kernel: one lane per key row (k, v, dk, dv in registers); Q/dout tiles
//   of every query head of the group in LDS.  Only tiles with a visible pair are visited.
#include "cpattn_internal.h"
#include "stream_access.h"

#include <math.h>

namespace cpattn {
namespace {

constexpr int kRows = 64;  // rows (queries or keys) per block, one per lane
constexpr int kTile = 32;  // rows of the other side staged per LDS tile

template <typename T>
__device__ inline float to_f(T x) { return (float)x; }

// One row of head_dim values per 16 lanes (head_dim a multiple of 4): each lane takes every
// 16th group of 4 consecutive values, so a wave reads four rows with contiguous accesses.
template <typename T>
__device__ inline float4 load4(const T* p);
template <>
__device__ inline float4 load4<float>(const float* p) { return *(const float4*)p; }
template <>
__device__ inline float4 load4<__bf16>(const __bf16* p) {
    // four bf16 in one 8-byte streaming read; a bf16 is the top half of the fp32 it widens to
    const uint64_t u = __builtin_nontemporal_load((const uint64_t*)p);
    const uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);  // elements 0,1 and 2,3
    return make_float4(__uint_as_float(lo << 16), __uint_as_float(lo & 0xFFFF0000u), __uint_as_float(hi << 16),
                       __uint_as_float(hi & 0xFFFF0000u));
}

template <typename T>
__global__ void __launch_bounds__(256) delta_kernel(const float* __restrict__ out, const T* __restrict__ dout,
                                                    float* __restrict__ delta, int64_t seq, int32_t heads,
                                                    int32_t D, int64_t n_rows) {
    const int64_t r = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 4;  // (b*seq + i)*heads + h
    const int sub = threadIdx.x & 15;
    float s = 0.f;
    if (r < n_rows) {
        const float* o = out + r * D;
        const T* g = dout + r * D;
        for (int d = 4 * sub; d < D; d += 64) {
            const v4f a4 = load_stream((const v4f*)(o + d));
            const float4 a = make_float4(a4.x, a4.y, a4.z, a4.w);
            const float4 b = load4<T>(g + d);
            s = fmaf(a.x, b.x, s);
            s = fmaf(a.y, b.y, s);
            s = fmaf(a.z, b.z, s);
            s = fmaf(a.w, b.w, s);
        }
    }
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) s += __shfl_xor(s, o, 16);
    if (r < n_rows && sub == 0) {
        const int64_t h = r % heads, bi = r / heads;
        const int64_t i = bi % seq, b = bi / seq;
        delta[(b * heads + h) * seq + i] = s;
    }
}

template <int D>
__global__ void __launch_bounds__(kRows) bwd_dq_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dout, const int64_t* __restrict__ qpos, const int64_t* __restrict__ kvpos,
    const float* __restrict__ lse, const float* __restrict__ delta, float* __restrict__ dq, int64_t seq_q,
    int64_t seq_kv, int32_t heads_q, int32_t heads_kv, float scale, int write) {
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
    const int64_t p_last = qpos[last];
    const int64_t mypos = valid ? qpos[i] : INT64_MIN;
    int64_t lo = 0, hi = seq_kv;  // keys visible to the block's last query
    while (lo < hi) {
        const int64_t mid = (lo + hi) / 2;
        if (kvpos[mid] <= p_last) lo = mid + 1; else hi = mid;
    }
    const int64_t n_keys = lo;
    const int64_t qr = ((b * seq_q + (valid ? i : 0)) * heads_q + h) * D;
    float qv[D], gv[D], acc[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        qv[d] = valid ? q[qr + d] : 0.f;
        gv[d] = valid ? dout[qr + d] : 0.f;
        acc[d] = 0.f;
    }
    const int64_t li = (b * heads_q + h) * seq_q + (valid ? i : 0);
    const float l = valid ? lse[li] : -INFINITY;
    const float dl = valid ? delta[li] : 0.f;
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
        if (lane < kTile) ps[lane] = (j0 + lane < seq_kv) ? kvpos[j0 + lane] : INT64_MAX;
        __syncthreads();
        if (l == -INFINITY) continue;  // no visible key anywhere: no gradient
        for (int r = 0; r < kTile; ++r) {
            if (ps[r] > mypos) continue;
            float s = 0.f, dp = 0.f;
#pragma unroll
            for (int d = 0; d < D; ++d) {
                s = fmaf(qv[d], ks[r][d], s);
                dp = fmaf(gv[d], vs[r][d], dp);
            }
            const float pv = expf(s * scale - l);
            const float ds = pv * (dp - dl);
#pragma unroll
            for (int d = 0; d < D; ++d) acc[d] = fmaf(ds, ks[r][d], acc[d]);
        }
    }
    if (!valid) return;
#pragma unroll
    for (int d = 0; d < D; ++d) dq[qr + d] = (write ? 0.f : dq[qr + d]) + scale * acc[d];
}

template <int D>
__global__ void __launch_bounds__(kRows) bwd_dkdv_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dout, const int64_t* __restrict__ qpos, const int64_t* __restrict__ kvpos,
    const float* __restrict__ lse, const float* __restrict__ delta, float* __restrict__ dk,
    float* __restrict__ dv, int64_t seq_q, int64_t seq_kv, int32_t heads_q, int32_t heads_kv, float scale,
    int write) {
    __shared__ float qs[kTile][D];
    __shared__ float gs[kTile][D];
    __shared__ float ls[kTile];
    __shared__ float dls[kTile];
    __shared__ int64_t ps[kTile];
    const int lane = threadIdx.x;
    const int64_t c = blockIdx.y, b = blockIdx.z;
    const int32_t G = heads_q / heads_kv;
    const int64_t row0 = (int64_t)blockIdx.x * kRows;
    const int64_t j = row0 + lane;
    const bool valid = j < seq_kv;
    const int64_t kp = valid ? kvpos[j] : INT64_MAX;
    // queries that see the block's first key: from the first with position >= it
    const int64_t k_first = kvpos[row0];
    int64_t lo = 0, hi = seq_q;
    while (lo < hi) {
        const int64_t mid = (lo + hi) / 2;
        if (qpos[mid] < k_first) lo = mid + 1; else hi = mid;
    }
    const int64_t i_begin = lo;
    const int64_t kr = ((b * seq_kv + (valid ? j : 0)) * heads_kv + c) * D;
    float kv_[D], vv[D], ak[D], av[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        kv_[d] = valid ? k[kr + d] : 0.f;
        vv[d] = valid ? v[kr + d] : 0.f;
        ak[d] = 0.f;
        av[d] = 0.f;
    }
    for (int32_t hh = 0; hh < G; ++hh) {
        const int64_t h = c * G + hh;
        for (int64_t i0 = i_begin; i0 < seq_q; i0 += kTile) {
            __syncthreads();
            for (int e = lane; e < kTile * D; e += kRows) {
                const int r = e / D, d = e % D;
                const int64_t i = i0 + r;
                const bool in = i < seq_q;
                const int64_t off = ((b * seq_q + (in ? i : 0)) * heads_q + h) * D + d;
                qs[r][d] = in ? q[off] : 0.f;
                gs[r][d] = in ? dout[off] : 0.f;
            }
            if (lane < kTile) {
                const int64_t i = i0 + lane;
                const bool in = i < seq_q;
                ps[lane] = in ? qpos[i] : INT64_MIN;
                ls[lane] = in ? lse[(b * heads_q + h) * seq_q + i] : -INFINITY;
                dls[lane] = in ? delta[(b * heads_q + h) * seq_q + i] : 0.f;
            }
            __syncthreads();
            for (int r = 0; r < kTile; ++r) {
                if (ps[r] < kp || ls[r] == -INFINITY) continue;
                float s = 0.f, dp = 0.f;
#pragma unroll
                for (int d = 0; d < D; ++d) {
                    s = fmaf(qs[r][d], kv_[d], s);
                    dp = fmaf(gs[r][d], vv[d], dp);
                }
                const float pv = expf(s * scale - ls[r]);
                const float ds = pv * (dp - dls[r]);
#pragma unroll
                for (int d = 0; d < D; ++d) {
                    ak[d] = fmaf(ds, qs[r][d], ak[d]);
                    av[d] = fmaf(pv, gs[r][d], av[d]);
                }
            }
        }
    }
    if (!valid) return;
#pragma unroll
    for (int d = 0; d < D; ++d) {
        dk[kr + d] = (write ? 0.f : dk[kr + d]) + scale * ak[d];
        dv[kr + d] = (write ? 0.f : dv[kr + d]) + av[d];
    }
}

template <int D>
hipError_t launch_f32(const BlockBwdArgs& a, hipStream_t stream) {
    const float* q = (const float*)a.q;
    const float* k = (const float*)a.k;
    const float* v = (const float*)a.v;
    const float* g = (const float*)a.dout;
    const dim3 gq((unsigned)((a.seq_q + kRows - 1) / kRows), (unsigned)a.heads_q, (unsigned)a.batch);
    hipLaunchKernelGGL(bwd_dq_f32_kernel<D>, gq, dim3(kRows), 0, stream, q, k, v, g, a.q_pos, a.kv_pos, a.lse,
                       a.delta, a.dq, a.seq_q, a.seq_kv, a.heads_q, a.heads_kv, a.scale, (int)a.write_dq);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 gk((unsigned)((a.seq_kv + kRows - 1) / kRows), (unsigned)a.heads_kv, (unsigned)a.batch);
    hipLaunchKernelGGL(bwd_dkdv_f32_kernel<D>, gk, dim3(kRows), 0, stream, q, k, v, g, a.q_pos, a.kv_pos, a.lse,
                       a.delta, a.dk, a.dv, a.seq_q, a.seq_kv, a.heads_q, a.heads_kv, a.scale,
                       (int)a.write_dkv);
    return hipGetLastError();
}

__global__ void __launch_bounds__(256) zero_kernel(float* __restrict__ p, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += stride) p[e] = 0.f;
}

}  // namespace

hipError_t launch_zero_fill(float* p, int64_t n, hipStream_t stream) {
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)(blocks < 16384 ? blocks : 16384)), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

hipError_t launch_attn_bwd_delta(const float* out, const void* dout, bool bf16, int32_t batch, int64_t seq,
                                 int32_t heads, int32_t head_dim, float* delta, hipStream_t stream) {
    const int64_t n_rows = (int64_t)batch * seq * heads;
    const dim3 grid((unsigned)((n_rows * 16 + 255) / 256));
    if (bf16)
        hipLaunchKernelGGL(delta_kernel<__bf16>, grid, dim3(256), 0, stream, out, (const __bf16*)dout, delta, seq,
                           heads, head_dim, n_rows);
    else
        hipLaunchKernelGGL(delta_kernel<float>, grid, dim3(256), 0, stream, out, (const float*)dout, delta, seq,
                           heads, head_dim, n_rows);
    return hipGetLastError();
}

hipError_t launch_block_bwd_f32(const BlockBwdArgs& a, hipStream_t stream) {
    return a.head_dim == 64 ? launch_f32<64>(a, stream) : launch_f32<128>(a, stream);
}

}  // namespace cpattn
