// Local layout change of Ulysses context parallelism for one head group.
// "Appendix F: Context Parallelism and MoE Parallel Folding", Eq. (96): [B, S/C, H, d] per
// rank becomes [B, S, H/C, d]; "On Context Parallelism", section All-to-all; "Context
// parallelism: Ring Attention and Ulysses", section Ulysses: group g = heads
// [g*H/C, (g+1)*H/C), and sequence shard src supplies rows [src*S/C, (src+1)*S/C).
//
// Zigzag shards (rank src holds chunks src and 2C-1-src of t = S/(2C) tokens, "On Context
// Parallelism", section All-gather): the same exchange with the chunk reorder folded in, so
// that the grouped tensor comes out in global sequence order ("On Context Parallelism",
// section All-to-all: the gathered sequence is in rank order and must be put back in order
// before causal attention).  Shard row i < t goes to global row src*t + i, row i >= t to
// (2C-1-src)*t + i - t.
//
// For one (src, b) pair the move is a 2-D copy of s = S/C rows of one head-group segment
// (H/C * D * elem bytes): in the stacked shards [C][B][S/C][H][D] the rows are H*D*elem
// apart, in the grouped tensor [B][S][H/C][D] they are packed.  grid.y enumerates (src, b),
// grid.x spans the s*seg elements of that copy.  Bandwidth-bound: 16-byte streaming accesses
// when sizes and pointers allow (stream_access.h; byte accesses otherwise), NV per lane with
// all loads issued before the first store.  The gather (seq -> heads: strided reads, packed
// writes) runs fastest with one access per lane and many small blocks, the scatter (heads ->
// seq: packed reads, strided writes) with four per lane (measured with the caches flushed:
// 4.4 -> 5.2 TB/s on a 512 MiB scatter, while four per lane cost the gather 5-8 %).  The
// row/offset split uses a 32-bit division by an invariant divisor (multiply-high with a
// precomputed magic number).
#include "cpattn_internal.h"
#include "stream_access.h"

namespace cpattn {
namespace {

constexpr int kThreads = 256;

// Exact n / d for 0 <= n < 2^31 and 1 <= d < 2^31 (Granlund & Montgomery, "Division by
// invariant integers using multiplication", 1994): l = ceil(log2 d),
// m = floor(2^32 (2^l - d) / d) + 1, q = (mulhi(n, m) + n) >> l.
struct FastDiv {
    uint32_t m, l, d;
};

FastDiv make_fastdiv(uint32_t d) {
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    const uint64_t m = ((1ull << 32) * ((1ull << l) - d)) / d + 1;
    return FastDiv{(uint32_t)m, l, d};
}

__device__ inline uint32_t fast_div(uint32_t n, FastDiv f) {
    return (__umulhi(n, f.m) + n) >> f.l;
}

template <typename T, int NV>
__global__ void __launch_bounds__(kThreads) ulysses_kernel(const T* __restrict__ in, T* __restrict__ out,
                                                           uint32_t span, FastDiv seg, int64_t row,
                                                           int64_t head_off, int64_t S, int64_t s,
                                                           int64_t B, int32_t dir, int64_t zz_t,
                                                           int64_t zz_last) {
    const int64_t sb = blockIdx.y;          // src * B + b
    const int64_t src = sb / B, b = sb - src * B;
    const int64_t stacked_base = sb * s * row + head_off;          // row i at + i*row
    const int64_t grouped_b = b * S * (int64_t)seg.d;
    const uint32_t base = blockIdx.x * (uint32_t)(kThreads * NV) + threadIdx.x;
    int64_t from[NV], to[NV];
    T val[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
        const uint32_t e = base + (uint32_t)u * kThreads;
        const uint32_t i = fast_div(e, seg);
        const uint32_t w = e - i * seg.d;
        // destination row: contiguous shards keep their order; zigzag shards split in two
        const int64_t grow = (zz_t == 0) ? src * s + i
                             : ((int64_t)i < zz_t ? src * zz_t + i : (zz_last - src) * zz_t + (i - zz_t));
        const int64_t so = stacked_base + (int64_t)i * row + w;
        const int64_t go = grouped_b + grow * (int64_t)seg.d + w;
        from[u] = dir == 0 ? so : go;
        to[u] = dir == 0 ? go : so;
    }
#pragma unroll
    for (int u = 0; u < NV; ++u)
        if (base + (uint32_t)u * kThreads < span) val[u] = load_stream(in + from[u]);
#pragma unroll
    for (int u = 0; u < NV; ++u)
        if (base + (uint32_t)u * kThreads < span) store_stream(out + to[u], val[u]);
}

}  // namespace

hipError_t launch_ulysses_permute(const void* in, void* out, int32_t elem_bytes, int32_t batch,
                                  int64_t seq_len, int32_t heads, int32_t head_dim,
                                  int32_t cp_size, int32_t group, int32_t dir, bool zigzag,
                                  hipStream_t stream) {
    const int64_t hg = heads / cp_size;
    const int64_t seg_bytes = hg * head_dim * (int64_t)elem_bytes;
    const int64_t row_bytes = (int64_t)heads * head_dim * elem_bytes;
    const int64_t off_bytes = (int64_t)group * seg_bytes;
    const bool vec = (seg_bytes % 16 == 0) && (row_bytes % 16 == 0) && ((uintptr_t)in % 16 == 0) &&
                     ((uintptr_t)out % 16 == 0);
    const int64_t el = vec ? 16 : 1;
    const int64_t s = seq_len / cp_size;
    const int64_t seg = seg_bytes / el;
    const int64_t span = s * seg;  // elements of one (src, b) copy; the ABI layer bounds it < 2^31
    const FastDiv fd = make_fastdiv((uint32_t)seg);
    const int64_t zz_t = zigzag ? seq_len / (2 * (int64_t)cp_size) : 0;
    const int64_t zz_last = 2 * (int64_t)cp_size - 1;
    auto launch = [&](auto nv) {
        constexpr int NV = decltype(nv)::value;
        const int64_t per_block = kThreads * NV;
        const dim3 grid((unsigned)((span + per_block - 1) / per_block), (unsigned)(cp_size * batch));
        if (vec)
            hipLaunchKernelGGL((ulysses_kernel<v4u, NV>), grid, dim3(kThreads), 0, stream, (const v4u*)in,
                               (v4u*)out, (uint32_t)span, fd, row_bytes / el, off_bytes / el, seq_len,
                               s, (int64_t)batch, dir, zz_t, zz_last);
        else
            hipLaunchKernelGGL((ulysses_kernel<uint8_t, NV>), grid, dim3(kThreads), 0, stream,
                               (const uint8_t*)in, (uint8_t*)out, (uint32_t)span, fd, row_bytes,
                               off_bytes, seq_len, s, (int64_t)batch, dir, zz_t, zz_last);
    };
    if (dir == 0) launch(std::integral_constant<int, 1>{});
    else launch(std::integral_constant<int, 4>{});
    return hipGetLastError();
}

}  // namespace cpattn
