/*
 * cpattn.h -- C ABI of libcpattn.so: one context-parallel rank's share of causal
 * attention, computed blockwise on one AMD Instinct MI355X (gfx950), plus the layout
 * companions of the all-gather and Ulysses variants.
 *
 * Sources (web pages; cited by title and section):
 *   [CP]    "On Context Parallelism" (jonahsamost.bearblog.dev)
 *   [DAY74] "Context parallelism -- splitting the sequence across GPUs" (llmdaily.org)
 *   [RING]  "Context Parallelism & Ring Attention" (Distributed Training from First Principles)
 *   [HB]    "Context parallelism: Ring Attention and Ulysses" (AI infra handbook)
 *   [OLMO]  "Appendix F: Context Parallelism and MoE Parallel Folding" (olmo-core MoE report)
 *
 * Conventions shared by every call
 * --------------------------------
 * - All tensor pointers are DEVICE pointers owned by the caller.  The library never
 *   allocates, frees or synchronises; every call only enqueues kernels on `stream`
 *   (a hipStream_t passed as void*; NULL means the null stream) and returns.
 * - Tensors are dense, row-major, in the layouts stated per call (cpattn_block_fwd_rows
 *   alone takes row strides).  Outputs must not alias inputs, except where a call is
 *   documented as in place.
 * - Every argument is validated on the host before anything is enqueued.  A call that
 *   returns an error has enqueued nothing and touched no memory.  CPATTN_ERR_HIP is
 *   returned when the HIP runtime reports an error for a launch.
 *   cpattn_last_error() gives a human-readable reason for the last failure on the
 *   calling thread.
 * - Sizes are int64 and address arithmetic is 64-bit (tensors above 2^31 elements are
 *   supported), except a lane's offset within one tile of up to 128 rows, which the bf16
 *   kernels form in 32 bits: their calls bound a row at 2^24 elements.
 * - The library keeps no state between calls except small arrays of work counters in
 *   device memory (32 KB per device, part of the loaded code, never allocated).  A long
 *   bf16 launch lets its workgroups take their work from queues counted there, so that
 *   the chip's XCDs, which hold different clocks under load, end together: a forward of
 *   at least 1024 workgroups, a backward dq launch of at least 4096, a dk/dv launch of at
 *   least 2048.  Successive launches take the arrays' 256 slots in turn, and a kernel on
 *   the call's stream zeroes the slot first (no memset, so such a call can be captured in
 *   a graph).  Results do not depend on which workgroup takes which item.  Calls on
 *   different streams may run concurrently as long as their buffers do not overlap and
 *   fewer than 256 such launches are in flight on one device at a time (a slot reused by
 *   a launch still running would be shared).
 */
#ifndef CPATTN_H
#define CPATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CPATTN_OK = 0,
    CPATTN_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, bad enum, bad scale */
    CPATTN_ERR_SHAPE = 2,       /* a divisibility or size relation between arguments fails */
    CPATTN_ERR_UNSUPPORTED = 3, /* well-formed but not implemented (head_dim, dtype) */
    CPATTN_ERR_HIP = 4          /* the HIP runtime reported an error */
} cpattn_status_t;

typedef enum { CPATTN_F32 = 0, CPATTN_BF16 = 1 } cpattn_dtype_t;

/* flags of cpattn_block_bwd */
#define CPATTN_BWD_WRITE_DQ 1u  /* dq = this block's part instead of dq += it */
#define CPATTN_BWD_WRITE_DKV 2u /* the same for dk and dv */

typedef enum {
    CPATTN_RANK_TO_SEQ = 0, /* all-gather (rank) order -> global sequence order */
    CPATTN_SEQ_TO_RANK = 1  /* global sequence order -> all-gather (rank) order */
} cpattn_reorder_dir_t;

typedef enum {
    CPATTN_SEQ_TO_HEADS = 0, /* [C][B][S/C][H][D] rank shards -> [B][S][H/C][D] of one group */
    CPATTN_HEADS_TO_SEQ = 1  /* the inverse */
} cpattn_permute_dir_t;

/* Static string naming a status code. */
const char* cpattn_status_string(cpattn_status_t status);

/* Reason for the last failed call on this thread ("" if none).  Valid until the next
 * call on the same thread. */
const char* cpattn_last_error(void);

/* ABI version of this header: 1. */
int32_t cpattn_abi_version(void);

/*
 * cpattn_zigzag_index -- global positions of rank `rank`'s local tokens under zigzag
 * sharding.  [CP] "All-gather" (and [RING] "The zigzag fix", [HB] "The zigzag
 * partition"): the sequence is cut into 2C chunks of t = S/(2C) tokens and rank r holds
 * chunk r followed by chunk 2C-1-r.
 *
 *   positions  out, int64 [seq_len / cp_size]: positions[i] = r*t + i for i < t,
 *              (2C-1-r)*t + (i - t) otherwise.  Strictly increasing.
 * Errors: SHAPE if seq_len % (2*cp_size) != 0; INVALID_ARG if seq_len <= 0, cp_size <= 0,
 * rank outside [0, cp_size) or positions is NULL.
 */
cpattn_status_t cpattn_zigzag_index(int64_t seq_len, int32_t cp_size, int32_t rank,
                                    int64_t* positions, void* stream);

/*
 * cpattn_zigzag_index_all -- the same positions for every rank in one launch (the ring
 * forward of [CP] "Peer-to-peer" needs each ring step's owner's positions, i.e. all ranks').
 *
 *   positions  out, int64 [cp_size][seq_len / cp_size], caller-owned: row r equals what
 *              cpattn_zigzag_index(seq_len, cp_size, r, ...) writes.  Rows are contiguous.
 * Errors: as cpattn_zigzag_index (no rank argument); UNSUPPORTED if cp_size > 65535 (one
 * grid row per rank).
 */
cpattn_status_t cpattn_zigzag_index_all(int64_t seq_len, int32_t cp_size, int64_t* positions,
                                        void* stream);

/*
 * cpattn_block_fwd -- attention of local queries against one K/V block under a causal
 * mask on GLOBAL positions, returning the block's normalised output and its log-sum-exp.
 * This is the per-step attention call of the ring forward in [CP] "Peer-to-peer" /
 * "Forward" (and the single call of [CP] "All-gather" / "Forward"):
 *
 *   s_ij  = scale * <q_i, k_j>            for kv_positions[j] <= q_positions[i]
 *   lse_i = ln sum_j exp(s_ij)            (natural log; [CP] "Peer-to-peer", the lse
 *                                          definition in the merge discussion)
 *   out_i = sum_j exp(s_ij - lse_i) v_j
 *
 * A query with no visible key in this block gets out_i = 0 and lse_i = -inf, which the
 * merge treats as "no contribution".  Grouped-query attention: query head h reads K/V
 * head h / (heads_q / heads_kv).
 *
 *   q             in  [batch][seq_q][heads_q][head_dim], dtype
 *   k, v          in  [batch][seq_kv][heads_kv][head_dim], dtype
 *   q_positions   in  int64 [seq_q], strictly increasing (precondition, not checked;
 *                     violating it gives unspecified values, never an out-of-bounds access)
 *   kv_positions  in  int64 [seq_kv], strictly increasing (same)
 *   scale         finite and > 0 (e.g. 1/sqrt(head_dim))
 *   out           out fp32 [batch][seq_q][heads_q][head_dim]
 *   lse           out fp32 [batch][heads_q][seq_q]
 *
 * dtype CPATTN_BF16: bf16 inputs, products accumulated in fp32 on the matrix cores; the
 * softmax weights are rounded to bf16 (round to nearest even) before the second product;
 * the row sums are kept in fp32.  dtype CPATTN_F32: fp32 throughout.
 * head_dim must be 64 or 128, for both dtypes.  seq_q == 0 is a no-op (pointers may be
 * NULL); seq_kv == 0 writes out = 0, lse = -inf (k, v, kv_positions may be NULL).
 * bf16: q, k, v, out 16-byte aligned, and a K/V row (heads_kv * head_dim elements) at most
 * 2^24 elements, since the kernels form offsets within a tile of rows in 32 bits.
 * Errors: INVALID_ARG (NULL pointer, batch/heads <= 0, seq < 0, bad scale or dtype),
 * SHAPE (heads_q % heads_kv != 0), UNSUPPORTED (head_dim not 64/128, misalignment, a K/V
 * row above 2^24 elements, a launch grid too large).
 */
cpattn_status_t cpattn_block_fwd(const void* q, const void* k, const void* v, cpattn_dtype_t dtype,
                                 int32_t batch, int64_t seq_q, int64_t seq_kv, int32_t heads_q,
                                 int32_t heads_kv, int32_t head_dim, const int64_t* q_positions,
                                 const int64_t* kv_positions, float scale, float* out, float* lse,
                                 void* stream);

/*
 * cpattn_block_fwd_merge -- cpattn_block_fwd with its result folded into an accumulator
 * in the same launch.  A ring step of [CP] "Peer-to-peer" / "Forward" computes one block's
 * (out_tile, lse_tile) and merges it into the running result (the merge discussion of the
 * same section); here the kernel's epilogue does the merge, so the tile never reaches
 * memory.  With (o, l) the values cpattn_block_fwd would write for the same arguments:
 *
 *   merged = ln(exp(lse) + exp(l))
 *   out    = exp(lse - merged) * out + exp(l - merged) * o
 *   lse    = merged
 *
 * with the rounding of cpattn_lse_merge: the result has the same bits as cpattn_block_fwd
 * into a scratch tile followed by cpattn_lse_merge into (out, lse).
 *
 *   q, k, v, positions, scale, dtype   as for cpattn_block_fwd
 *   out   in/out fp32 [batch][seq_q][heads_q][head_dim], the accumulator
 *   lse   in/out fp32 [batch][heads_q][seq_q], the accumulator (-inf marks "nothing yet";
 *         out must then hold finite values, e.g. 0)
 * seq_q == 0 is a no-op; seq_kv == 0 merges an empty result (rows at -inf become out = 0).
 * Errors as for cpattn_block_fwd.
 */
cpattn_status_t cpattn_block_fwd_merge(const void* q, const void* k, const void* v,
                                       cpattn_dtype_t dtype, int32_t batch, int64_t seq_q,
                                       int64_t seq_kv, int32_t heads_q, int32_t heads_kv,
                                       int32_t head_dim, const int64_t* q_positions,
                                       const int64_t* kv_positions, float scale, float* out,
                                       float* lse, void* stream);

/*
 * cpattn_block_fwd_rows -- cpattn_block_fwd (bf16, batch 1, head_dim 64 or 128) on strided
 * rows: q, k, v and out are sequences of rows whose consecutive rows lie q_row_stride,
 * kv_row_stride and out_row_stride elements apart; within a row the heads are contiguous
 * (head h at h * head_dim; the lines below write 128 for head_dim).  This lets Ulysses' head group be read in place from the stacked
 * rank shards and its output written back into them: with B = 1 and contiguous shards,
 * the exchange of [HB] "Ulysses" / [OLMO] Eq. (96) maps global row i of group g to row i
 * of the stacked buffer at head offset g * H/C, so q = Q_st + g*(Hq/C)*128 with
 * q_row_stride = Hq*128 (likewise k, v and out), and the sequence->heads permute and its
 * inverse need no separate pass.  Results have the same bits as cpattn_block_fwd on dense
 * copies of the same rows.
 *   q        in  bf16 rows of heads_q*128 values, seq_q rows
 *   k, v     in  bf16 rows of heads_kv*128 values, seq_kv rows
 *   q_row_stride, kv_row_stride   in elements: >= heads*128, multiples of 8, <= 2^24
 *   q_positions, kv_positions, scale   as for cpattn_block_fwd
 *   out      out fp32 rows, out_row_stride elements apart (>= heads_q*128, multiple of 4);
 *                only each row's heads_q*128 values are written
 *   lse      out fp32 [heads_q][seq_q] (dense)
 * seq_q == 0 is a no-op; seq_kv == 0 gives out = 0 and lse = -inf (k, v, kv_positions may
 * then be NULL).  Pointers 16-byte aligned.
 * Errors: INVALID_ARG (NULL pointer, heads <= 0, seq < 0, bad scale), SHAPE (heads_q %
 * heads_kv != 0), UNSUPPORTED (head_dim not 64/128, a stride too small, too large or not a
 * multiple of its unit, misalignment).
 */
cpattn_status_t cpattn_block_fwd_rows(const void* q, int64_t q_row_stride, const void* k,
                                      const void* v, int64_t kv_row_stride, int64_t seq_q,
                                      int64_t seq_kv, int32_t heads_q, int32_t heads_kv,
                                      int32_t head_dim, const int64_t* q_positions,
                                      const int64_t* kv_positions, float scale, float* out,
                                      int64_t out_row_stride, float* lse, void* stream);

/*
 * cpattn_ring_share_fwd -- a rank's whole share in one launch: the queries against C K/V
 * blocks taken in the given (ring) order, as [CP] "Peer-to-peer" / "Forward" computes them
 * step by step with the merge of attention tiles.  Here each workgroup walks the blocks'
 * visible tiles one after another with a single running softmax, so the per-step results
 * are never formed: the output is the merge of the C block results (equal in exact
 * arithmetic; rounded once instead of C times).  This is the persistent launch over all
 * ring blocks; on one GPU it removes the per-step launches, their tails and the merges.
 *
 *   q, q_positions, scale, out, lse   as for cpattn_block_fwd (out, lse are written)
 *   k_blocks, v_blocks   host arrays of n_blocks DEVICE pointers, block o of shape
 *                        [batch][seq_kv[o]][heads_kv][head_dim], dtype
 *   kv_positions         host array of n_blocks DEVICE pointers to int64 [seq_kv[o]],
 *                        each strictly increasing
 *   seq_kv               host array of n_blocks lengths (0: the block is skipped)
 *   n_blocks             1 .. 16
 * dtype CPATTN_BF16: one launch (head_dim 64 or 128).  CPATTN_F32: cpattn_block_fwd on the
 * first block and cpattn_block_fwd_merge on the others; every block is validated before
 * the first of them is launched.
 * Errors: as for cpattn_block_fwd, and INVALID_ARG for n_blocks outside [1, 16] or NULL
 * arrays.  A call that returns an error has enqueued nothing, for either dtype.
 */
cpattn_status_t cpattn_ring_share_fwd(const void* q, const void* const* k_blocks,
                                      const void* const* v_blocks, const int64_t* const* kv_positions,
                                      const int64_t* seq_kv, int32_t n_blocks, cpattn_dtype_t dtype,
                                      int32_t batch, int64_t seq_q, int32_t heads_q, int32_t heads_kv,
                                      int32_t head_dim, const int64_t* q_positions, float scale,
                                      float* out, float* lse, void* stream);

/*
 * cpattn_lse_merge -- fold one completed partial result into an accumulator, in place.
 * [CP] "Peer-to-peer" (merging attention tiles) and [HB] "Ring Attention":
 *
 *   merged = ln(exp(lse) + exp(lse_tile))
 *   out    = exp(lse - merged) * out + exp(lse_tile - merged) * out_tile
 *   lse    = merged
 *
 * A side whose lse is -inf has weight 0; two empty sides give (0, -inf) and never NaN.
 * The result is symmetric in its two operands.
 *
 *   out       in/out fp32 [batch][seq][heads][head_dim]
 *   lse       in/out fp32 [batch][heads][seq]
 *   out_tile  in     fp32 [batch][seq][heads][head_dim]
 *   lse_tile  in     fp32 [batch][heads][seq]
 * Errors: INVALID_ARG (NULL pointer, batch/heads/head_dim <= 0, seq < 0), SHAPE
 * (head_dim % 4 != 0).  seq == 0 is a no-op.
 */
cpattn_status_t cpattn_lse_merge(float* out, float* lse, const float* out_tile,
                                 const float* lse_tile, int32_t batch, int64_t seq,
                                 int32_t heads, int32_t head_dim, void* stream);

/*
 * cpattn_attn_bwd_delta -- the row term of the attention backward, D_i = <dout_i, out_i>.
 * [CP] "Peer-to-peer" / "Backward" (and "All-gather" / "Backward"): the backward of every
 * ring step starts from the saved output and its gradient; the softmax derivative needs
 * this per-row dot product (ds_ij = p_ij (dp_ij - D_i)), which is the same for all steps,
 * so it is computed once per rank share.
 *
 *   out    in  fp32 [batch][seq][heads][head_dim] (the complete forward output)
 *   dout   in  [batch][seq][heads][head_dim], dtype (bf16 or fp32)
 *   delta  out fp32 [batch][heads][seq]
 * Errors: INVALID_ARG (NULL pointer, sizes <= 0, seq < 0, bad dtype), SHAPE (head_dim % 4
 * != 0), UNSUPPORTED (out not 16-byte aligned, dout not 16-byte (fp32) or 8-byte (bf16)
 * aligned).  seq == 0 is a no-op.
 */
cpattn_status_t cpattn_attn_bwd_delta(const float* out, const void* dout, cpattn_dtype_t dtype,
                                      int32_t batch, int64_t seq, int32_t heads, int32_t head_dim,
                                      float* delta, void* stream);

/*
 * cpattn_block_bwd -- the backward of one block, ADDED into gradient accumulators.
 * [CP] "Peer-to-peer" / "Backward": each ring step computes tile_dq, tile_dk, tile_dv of
 * the local queries against one K/V block from the saved output and lse; dq accumulates
 * locally over the steps, dk and dv accumulate in the buffers that travel with the block.
 * With lse the complete (merged) log-sum-exp of each query row:
 *   p_ij  = exp(scale <q_i, k_j> - lse_i)  for kv_positions[j] <= q_positions[i], else 0
 *   ds_ij = p_ij (<dout_i, v_j> - delta_i)
 *   dq_i += scale sum_j ds_ij k_j;  dk_j += scale sum_i ds_ij q_i;  dv_j += sum_i p_ij dout_i
 * (chain rule of the attention definition of cpattn_block_fwd).  Grouped-query attention:
 * dk, dv of kv head c sum over the query heads h with h / (heads_q/heads_kv) == c.
 *
 *   q, dout      in  [batch][seq_q][heads_q][head_dim], dtype
 *   k, v         in  [batch][seq_kv][heads_kv][head_dim], dtype
 *   positions    in  int64, strictly increasing (precondition, as for cpattn_block_fwd)
 *   lse          in  fp32 [batch][heads_q][seq_q] (from the forward; -inf: no visible key)
 *   delta        in  fp32 [batch][heads_q][seq_q] (cpattn_attn_bwd_delta)
 *   dq           in/out fp32 [batch][seq_q][heads_q][head_dim]   (+= this block's part)
 *   dk, dv       in/out fp32 [batch][seq_kv][heads_kv][head_dim] (+= this block's part)
 *   flags        CPATTN_BWD_WRITE_DQ: dq = this block's part (no prior contents read);
 *                CPATTN_BWD_WRITE_DKV: the same for dk and dv.  A ring share passes
 *                WRITE_DQ on its first step, so no accumulator needs clearing.
 * dtype CPATTN_BF16: bf16 products with fp32 accumulation; p and ds are rounded to bf16
 * (RNE) before the products that use them.  CPATTN_F32: fp32 throughout.  head_dim 64 or
 * 128 for both dtypes (bf16: a Q row of heads_q * head_dim elements at most 2^24).  seq_q == 0
 * or seq_kv == 0 adds nothing.
 * Errors: INVALID_ARG (also unknown flag bits), SHAPE, UNSUPPORTED as for cpattn_block_fwd.
 */
cpattn_status_t cpattn_block_bwd(const void* q, const void* k, const void* v, const void* dout,
                                 cpattn_dtype_t dtype, int32_t batch, int64_t seq_q, int64_t seq_kv,
                                 int32_t heads_q, int32_t heads_kv, int32_t head_dim,
                                 const int64_t* q_positions, const int64_t* kv_positions, float scale,
                                 const float* lse, const float* delta, float* dq, float* dk, float* dv,
                                 uint32_t flags, void* stream);

/*
 * cpattn_ring_share_bwd -- a rank's whole backward share: the gradients from the queries
 * against C K/V blocks, as [CP] "Peer-to-peer" / "Backward" computes them step by step
 * (cpattn_block_bwd once per block, dq summed locally over the steps, each block's dk and dv
 * going to the buffers that travel with it).  The same arithmetic as those calls with
 * CPATTN_BWD_WRITE_DKV on every block and CPATTN_BWD_WRITE_DQ on the first; for bf16 the
 * dk and dv of all blocks come from one launch, so that the blocks' key ranges fill the chip
 * together (one launch per block leaves it partly empty wherever half a block's keys are
 * hidden from every query, as in the zigzag ring steps).
 *
 *   q, dout, q_positions, scale, lse, delta   as for cpattn_block_bwd
 *   k_blocks, v_blocks, kv_positions, seq_kv, n_blocks   as for cpattn_ring_share_fwd
 *   dq          out fp32 [batch][seq_q][heads_q][head_dim]: the sum of the blocks' parts
 *   dk_blocks, dv_blocks   host arrays of n_blocks DEVICE pointers, block o's dk and dv,
 *               out fp32 [batch][seq_kv[o]][heads_kv][head_dim] (written)
 * dk, dv of every block and dq are the same bits as the per-block calls give.  Every block is
 * validated before anything is enqueued.
 * Errors: as for cpattn_block_bwd on each block, and INVALID_ARG for n_blocks outside [1, 16]
 * or NULL arrays.
 */
cpattn_status_t cpattn_ring_share_bwd(const void* q, const void* dout, const void* const* k_blocks,
                                      const void* const* v_blocks, const int64_t* const* kv_positions,
                                      const int64_t* seq_kv, int32_t n_blocks, cpattn_dtype_t dtype,
                                      int32_t batch, int64_t seq_q, int32_t heads_q, int32_t heads_kv,
                                      int32_t head_dim, const int64_t* q_positions, float scale,
                                      const float* lse, const float* delta, float* dq,
                                      float* const* dk_blocks, float* const* dv_blocks, void* stream);

/*
 * cpattn_reorder_gathered -- chunk reorder between the all-gather's rank order and the
 * global sequence order.  [CP] "All-gather": the gather concatenates the ranks' zigzag
 * shards in rank order (at C=4: chunks 0,7,1,6,2,5,3,4), and K/V must be put back in
 * sequence order before attention; the backward applies the inverse permutation.
 * Gathered slot k holds chunk k/2 (k even) or 2C-1-(k-1)/2 (k odd).
 *
 *   in, out    [batch][seq_len][row_bytes] (rows are opaque bytes, e.g. heads*D*2)
 *   dir        CPATTN_RANK_TO_SEQ: out[b][chunk c] = in[b][slot of c]
 *              CPATTN_SEQ_TO_RANK: out[b][slot k] = in[b][chunk of k]
 * Bit-exact byte copy.  Errors: INVALID_ARG (NULL pointer, sizes <= 0, bad dir, in == out),
 * SHAPE (seq_len % (2*cp_size) != 0).
 */
cpattn_status_t cpattn_reorder_gathered(const void* in, void* out, int32_t batch, int64_t seq_len,
                                        int64_t row_bytes, int32_t cp_size,
                                        cpattn_reorder_dir_t dir, void* stream);

/*
 * cpattn_ulysses_permute -- the local layout change around Ulysses' all-to-all, for head
 * group `group`.  [OLMO] Eq. (96), [CP] "All-to-all", [HB] "Ulysses: transposing between
 * the sequence and the heads": [B, S/C, H, D] per rank becomes [B, S, H/C, D] holding
 * heads [g*H/C, (g+1)*H/C) for the whole sequence; sequence shard src supplies rows
 * [src*S/C, (src+1)*S/C) (contiguous sharding).
 *
 *   CPATTN_SEQ_TO_HEADS: in  = the C rank shards stacked, [C][B][S/C][H][D]
 *                        out = [B][S][H/C][D];
 *                        out[b][src*S/C + i][h][d] = in[src][b][i][g*H/C + h][d]
 *   CPATTN_HEADS_TO_SEQ: in  = [B][S][H/C][D], out = stacked [C][B][S/C][H][D]; writes
 *                        only group g's heads of out (the rest is left untouched).
 * Elements are opaque byte strings of elem_bytes (2 for bf16, 4 for fp32).  Bit-exact.
 * Errors: INVALID_ARG (NULL pointer, sizes <= 0, bad dir, group outside [0, C), in == out),
 * SHAPE (seq_len % C != 0 or heads % C != 0; C must divide the head count, [CP]
 * "All-to-all" and [HB] "How to choose").
 */
cpattn_status_t cpattn_ulysses_permute(const void* in, void* out, int32_t elem_bytes,
                                       int32_t batch, int64_t seq_len, int32_t heads,
                                       int32_t head_dim, int32_t cp_size, int32_t group,
                                       cpattn_permute_dir_t dir, void* stream);

/*
 * cpattn_ulysses_permute_zigzag -- cpattn_ulysses_permute for zigzag shards, with the chunk
 * reorder folded in so that the grouped side is in global sequence order.  Rank src holds
 * chunks src and 2C-1-src of t = S/(2C) tokens ([CP] "All-gather"); the all-to-all
 * concatenates shards in rank order, which causal attention cannot use until the chunks are
 * put back in order ([CP] "All-to-all", [CP] "All-gather" for the rank-order layout).
 * With C = A this is also the per-group exchange of the two-dimensional mesh of [CP]
 * "Peer-to-peer + All-to-all": an A2A group's A zigzag shards come out as the group's
 * tokens in increasing position order.
 *
 *   CPATTN_SEQ_TO_HEADS: in = stacked [C][B][S/C][H][D], out = [B][S][H/C][D] with
 *                        out[b][p][h][d] = in[src][b][i][g*H/C + h][d] where shard row
 *                        i < t holds position p = src*t + i and row i >= t holds
 *                        p = (2C-1-src)*t + (i - t)
 *   CPATTN_HEADS_TO_SEQ: the inverse; writes only group g's heads of the stacked out.
 * Bit-exact.  Errors as for cpattn_ulysses_permute, and SHAPE if seq_len % (2*C) != 0.
 */
cpattn_status_t cpattn_ulysses_permute_zigzag(const void* in, void* out, int32_t elem_bytes,
                                              int32_t batch, int64_t seq_len, int32_t heads,
                                              int32_t head_dim, int32_t cp_size, int32_t group,
                                              cpattn_permute_dir_t dir, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CPATTN_H */
