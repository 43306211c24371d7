// Internal launch interface between the C ABI layer (api.hip) and the kernels.
// Every launcher assumes its arguments were validated by the ABI layer and only enqueues
// work on `stream`; it returns the launch status from hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpattn {

hipError_t launch_zigzag_index_all(int64_t chunk_len, int32_t cp_size, int64_t* positions,
                                   hipStream_t stream);
hipError_t launch_zigzag_index(int64_t chunk_len, int64_t early_chunk, int64_t late_chunk,
                               int64_t* positions, hipStream_t stream);

hipError_t launch_lse_merge(float* out, float* lse, const float* out_tile, const float* lse_tile,
                            int32_t batch, int64_t seq, int32_t heads, int32_t head_dim,
                            hipStream_t stream);

hipError_t launch_reorder_gathered(const void* in, void* out, int32_t batch, int64_t seq_len,
                                   int64_t row_bytes, int32_t cp_size, int32_t dir,
                                   hipStream_t stream);

hipError_t launch_ulysses_permute(const void* in, void* out, int32_t elem_bytes, int32_t batch,
                                  int64_t seq_len, int32_t heads, int32_t head_dim,
                                  int32_t cp_size, int32_t group, int32_t dir, bool zigzag,
                                  hipStream_t stream);

constexpr int kMaxRingBlocks = 16;  // K/V blocks one ring-share launch can take

struct KVBlockArg {
    const void* k;
    const void* v;
    const int64_t* pos;
    int64_t seq;
};

struct BlockFwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const int64_t* q_pos;
    const int64_t* kv_pos;
    float* out;
    float* lse;
    int32_t batch;
    int64_t seq_q;
    int64_t seq_kv;
    int32_t heads_q;
    int32_t heads_kv;
    int32_t head_dim;
    float scale;
    // false: write the block's (out, lse).  true: (out, lse) hold an accumulator and the
    // block's result is merged into it in the epilogue, with the arithmetic of merge_math.h.
    bool merge;
    // bf16 path: the K/V blocks attended in turn (one softmax over all their keys); a single
    // block call fills blk[0] from k, v, kv_pos, seq_kv
    int32_t n_blk;
    KVBlockArg blk[kMaxRingBlocks];
    // bf16 path: elements between consecutive sequence rows of q, of every K/V block, and of
    // out (heads are contiguous within a row); 0 means dense rows (heads * head_dim)
    int64_t q_row_stride = 0;
    int64_t kv_row_stride = 0;
    int64_t out_row_stride = 0;
};

// No keys: writes out = 0 and lse = -inf for every row (merge: merges that empty result).
hipError_t launch_block_fwd_empty(const BlockFwdArgs& a, hipStream_t stream);
// fp32 inputs, fp32 arithmetic on the vector ALUs.
hipError_t launch_block_fwd_f32(const BlockFwdArgs& a, hipStream_t stream);
// bf16 inputs, bf16 matrix-core products with fp32 accumulation.
hipError_t launch_block_fwd_bf16(const BlockFwdArgs& a, hipStream_t stream);

struct BlockBwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* dout;
    const int64_t* q_pos;
    const int64_t* kv_pos;
    const float* lse;
    const float* delta;
    float* dq;
    float* dk;
    float* dv;
    int32_t batch;
    int64_t seq_q;
    int64_t seq_kv;
    int32_t heads_q;
    int32_t heads_kv;
    int32_t head_dim;
    float scale;
    bool write_dq;   // overwrite dq instead of adding to it
    bool write_dkv;  // overwrite dk and dv instead of adding to them
};

// delta[b][h][i] = <dout[b][i][h], out[b][i][h]> (dout bf16 or fp32, out fp32).
hipError_t launch_attn_bwd_delta(const float* out, const void* dout, bool bf16, int32_t batch, int64_t seq,
                                 int32_t heads, int32_t head_dim, float* delta, hipStream_t stream);
// One block's backward, accumulated into dq, dk, dv (fp32 and bf16 paths).
hipError_t launch_block_bwd_f32(const BlockBwdArgs& a, hipStream_t stream);
hipError_t launch_block_bwd_bf16(const BlockBwdArgs& a, hipStream_t stream);
// A ring share's backward over n_blk blocks (bf16): dq written with the sum over the blocks,
// each block's dk and dv written to its own buffers.  a supplies the query side (q, dout,
// q_pos, lse, delta, dq, shapes, scale); its k, v, kv_pos, seq_kv, dk, dv are not used.
struct RingBwdBlock {
    const void* k;
    const void* v;
    const int64_t* pos;
    int64_t seq_kv;
    float* dk;
    float* dv;
};
hipError_t launch_ring_bwd_bf16(const BlockBwdArgs& a, int32_t n_blk, const RingBwdBlock* blocks,
                                hipStream_t stream);
// n floats of p set to 0 (an accumulator that no block writes)
hipError_t launch_zero_fill(float* p, int64_t n, hipStream_t stream);

}  // namespace cpattn
