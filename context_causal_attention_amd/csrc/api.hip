// C ABI of libcpattn.so: argument validation on the host, then one or more kernel launches
// on the caller's stream.  Nothing here allocates, frees or synchronises.  A call that fails
// validation returns before touching the GPU.  See include/cpattn.h for the contract of
// each entry point.
#include "cpattn.h"
#include "cpattn_internal.h"

#include <math.h>

#include <algorithm>
#include <stdarg.h>
#include <stdio.h>

#define CPATTN_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_last_error[512] = "";

cpattn_status_t fail(cpattn_status_t s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

cpattn_status_t ok() {
    g_last_error[0] = '\0';
    return CPATTN_OK;
}

cpattn_status_t from_hip(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(CPATTN_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

constexpr int64_t kMaxGrid = 2147483647;  // grid.x limit

}  // namespace

CPATTN_API const char* cpattn_status_string(cpattn_status_t s) {
    switch (s) {
        case CPATTN_OK: return "CPATTN_OK";
        case CPATTN_ERR_INVALID_ARG: return "CPATTN_ERR_INVALID_ARG";
        case CPATTN_ERR_SHAPE: return "CPATTN_ERR_SHAPE";
        case CPATTN_ERR_UNSUPPORTED: return "CPATTN_ERR_UNSUPPORTED";
        case CPATTN_ERR_HIP: return "CPATTN_ERR_HIP";
    }
    return "CPATTN_ERR_UNKNOWN";
}

CPATTN_API const char* cpattn_last_error(void) { return g_last_error; }

CPATTN_API int32_t cpattn_abi_version(void) { return 1; }

CPATTN_API cpattn_status_t cpattn_zigzag_index(int64_t seq_len, int32_t cp_size, int32_t rank,
                                               int64_t* positions, void* stream) {
    if (seq_len <= 0) return fail(CPATTN_ERR_INVALID_ARG, "zigzag_index: seq_len must be > 0");
    if (cp_size <= 0) return fail(CPATTN_ERR_INVALID_ARG, "zigzag_index: cp_size must be > 0");
    if (rank < 0 || rank >= cp_size)
        return fail(CPATTN_ERR_INVALID_ARG, "zigzag_index: rank %d outside [0, %d)", rank, cp_size);
    if (!positions) return fail(CPATTN_ERR_INVALID_ARG, "zigzag_index: positions is NULL");
    if (seq_len % (2 * (int64_t)cp_size) != 0)
        return fail(CPATTN_ERR_SHAPE, "zigzag_index: seq_len %lld not divisible by 2*cp_size = %lld",
                    (long long)seq_len, 2LL * cp_size);
    const int64_t t = seq_len / (2 * (int64_t)cp_size);
    return from_hip(cpattn::launch_zigzag_index(t, rank, 2 * (int64_t)cp_size - 1 - rank, positions,
                                                (hipStream_t)stream),
                    "zigzag_index");
}

CPATTN_API cpattn_status_t cpattn_zigzag_index_all(int64_t seq_len, int32_t cp_size, int64_t* positions,
                                                   void* stream) {
    if (seq_len <= 0) return fail(CPATTN_ERR_INVALID_ARG, "zigzag_index_all: seq_len must be > 0");
    if (cp_size <= 0) return fail(CPATTN_ERR_INVALID_ARG, "zigzag_index_all: cp_size must be > 0");
    if (cp_size > 65535) return fail(CPATTN_ERR_UNSUPPORTED, "zigzag_index_all: cp_size above 65535");
    if (!positions) return fail(CPATTN_ERR_INVALID_ARG, "zigzag_index_all: positions is NULL");
    if (seq_len % (2 * (int64_t)cp_size) != 0)
        return fail(CPATTN_ERR_SHAPE, "zigzag_index_all: seq_len %lld not divisible by 2*cp_size = %lld",
                    (long long)seq_len, 2LL * cp_size);
    const int64_t t = seq_len / (2 * (int64_t)cp_size);
    return from_hip(cpattn::launch_zigzag_index_all(t, cp_size, positions, (hipStream_t)stream),
                    "zigzag_index_all");
}

namespace {

// The bf16 kernels form each lane's byte offset within a K/V (or Q) tile of up to 128 rows in
// 32 bits: 127 rows times the row pitch must stay below 2^32 bytes, so a row (heads * head_dim
// elements of 2 bytes) is bounded at 2^24 elements.
constexpr int64_t kMaxRowElems = 1LL << 24;

// Validation of one block attention call (cpattn_block_fwd, cpattn_block_fwd_merge and each
// block of the fp32 ring share).  Returns CPATTN_OK when the call may launch; *empty is set
// when there is nothing to launch (no query rows).  `name` prefixes the error messages.
cpattn_status_t block_fwd_check(const char* name, const void* q, const void* k, const void* v,
                                cpattn_dtype_t dtype, int32_t batch, int64_t seq_q, int64_t seq_kv,
                                int32_t heads_q, int32_t heads_kv, int32_t head_dim,
                                const int64_t* q_positions, const int64_t* kv_positions, float scale,
                                float* out, float* lse, bool* empty) {
    *empty = false;
    if (dtype != CPATTN_F32 && dtype != CPATTN_BF16)
        return fail(CPATTN_ERR_INVALID_ARG, "%s: unknown dtype %d", name, (int)dtype);
    if (batch <= 0 || heads_q <= 0 || heads_kv <= 0)
        return fail(CPATTN_ERR_INVALID_ARG, "%s: batch and head counts must be > 0", name);
    if (seq_q < 0 || seq_kv < 0)
        return fail(CPATTN_ERR_INVALID_ARG, "%s: sequence lengths must be >= 0", name);
    if (!(scale > 0.f) || !isfinite(scale))
        return fail(CPATTN_ERR_INVALID_ARG, "%s: scale must be finite and > 0", name);
    if (heads_q % heads_kv != 0)
        return fail(CPATTN_ERR_SHAPE, "%s: heads_q %d not a multiple of heads_kv %d", name, heads_q,
                    heads_kv);
    if (head_dim != 64 && head_dim != 128)
        return fail(CPATTN_ERR_UNSUPPORTED, "%s: head_dim %d (supported: 64, 128)", name, head_dim);
    if (dtype == CPATTN_BF16 && (int64_t)heads_kv * head_dim > kMaxRowElems)
        return fail(CPATTN_ERR_UNSUPPORTED, "%s: heads_kv * head_dim = %lld above 2^24", name,
                    (long long)heads_kv * head_dim);
    if (seq_q == 0) {
        *empty = true;
        return ok();
    }
    if (!q || !q_positions || !out || !lse)
        return fail(CPATTN_ERR_INVALID_ARG, "%s: q, q_positions, out and lse must be non-NULL", name);
    if (seq_kv > 0 && (!k || !v || !kv_positions))
        return fail(CPATTN_ERR_INVALID_ARG, "%s: k, v and kv_positions must be non-NULL", name);
    if (dtype == CPATTN_BF16 &&
        (!aligned16(q) || (seq_kv > 0 && (!aligned16(k) || !aligned16(v))) || !aligned16(out)))
        return fail(CPATTN_ERR_UNSUPPORTED, "%s: bf16 path needs 16-byte aligned q, k, v, out", name);
    if (dtype == CPATTN_F32 && ((seq_q + 63) / 64 > kMaxGrid || heads_q > 65535 || batch > 65535))
        return fail(CPATTN_ERR_UNSUPPORTED, "%s: launch grid too large", name);
    // every bf16 forward variant launches ceil(seq_q / pq) * batch * heads_q / G blocks with
    // pq >= 32 query positions per block, so this bound holds for all of them
    if (dtype == CPATTN_BF16 && (seq_q + 31) / 32 * (int64_t)batch * heads_q > kMaxGrid)
        return fail(CPATTN_ERR_UNSUPPORTED, "%s: launch grid too large", name);
    return ok();
}

// Launch of one validated block attention call.
cpattn_status_t block_fwd_launch(const char* name, bool merge, const void* q, const void* k, const void* v,
                                 cpattn_dtype_t dtype, int32_t batch, int64_t seq_q, int64_t seq_kv,
                                 int32_t heads_q, int32_t heads_kv, int32_t head_dim,
                                 const int64_t* q_positions, const int64_t* kv_positions, float scale,
                                 float* out, float* lse, void* stream) {
    cpattn::BlockFwdArgs a{q,     k,      v,       q_positions, kv_positions, out,      lse,
                           batch, seq_q, seq_kv, heads_q,     heads_kv,     head_dim, scale, merge};
    a.n_blk = 1;
    a.blk[0] = cpattn::KVBlockArg{k, v, kv_positions, seq_kv};
    if (seq_kv == 0) {
        // no keys at all: every row is empty (out = 0, lse = -inf)
        return from_hip(cpattn::launch_block_fwd_empty(a, (hipStream_t)stream), name);
    }
    const hipError_t e = (dtype == CPATTN_BF16) ? cpattn::launch_block_fwd_bf16(a, (hipStream_t)stream)
                                                : cpattn::launch_block_fwd_f32(a, (hipStream_t)stream);
    return from_hip(e, name);
}

// cpattn_block_fwd (merge = false) and cpattn_block_fwd_merge (merge = true).
cpattn_status_t block_fwd_common(const char* name, bool merge, const void* q, const void* k,
                                 const void* v, cpattn_dtype_t dtype, int32_t batch, int64_t seq_q,
                                 int64_t seq_kv, int32_t heads_q, int32_t heads_kv, int32_t head_dim,
                                 const int64_t* q_positions, const int64_t* kv_positions, float scale,
                                 float* out, float* lse, void* stream) {
    bool empty = false;
    const cpattn_status_t st = block_fwd_check(name, q, k, v, dtype, batch, seq_q, seq_kv, heads_q, heads_kv,
                                               head_dim, q_positions, kv_positions, scale, out, lse, &empty);
    if (st != CPATTN_OK || empty) return st;
    return block_fwd_launch(name, merge, q, k, v, dtype, batch, seq_q, seq_kv, heads_q, heads_kv, head_dim,
                            q_positions, kv_positions, scale, out, lse, stream);
}

}  // namespace

CPATTN_API cpattn_status_t cpattn_block_fwd(const void* q, const void* k, const void* v,
                                            cpattn_dtype_t dtype, int32_t batch, int64_t seq_q,
                                            int64_t seq_kv, int32_t heads_q, int32_t heads_kv,
                                            int32_t head_dim, const int64_t* q_positions,
                                            const int64_t* kv_positions, float scale, float* out,
                                            float* lse, void* stream) {
    return block_fwd_common("block_fwd", false, q, k, v, dtype, batch, seq_q, seq_kv, heads_q, heads_kv,
                            head_dim, q_positions, kv_positions, scale, out, lse, stream);
}

CPATTN_API cpattn_status_t cpattn_block_fwd_merge(const void* q, const void* k, const void* v,
                                                  cpattn_dtype_t dtype, int32_t batch, int64_t seq_q,
                                                  int64_t seq_kv, int32_t heads_q, int32_t heads_kv,
                                                  int32_t head_dim, const int64_t* q_positions,
                                                  const int64_t* kv_positions, float scale, float* out,
                                                  float* lse, void* stream) {
    return block_fwd_common("block_fwd_merge", true, q, k, v, dtype, batch, seq_q, seq_kv, heads_q,
                            heads_kv, head_dim, q_positions, kv_positions, scale, out, lse, stream);
}

CPATTN_API cpattn_status_t cpattn_block_fwd_rows(const void* q, int64_t q_row_stride, const void* k,
                                                 const void* v, int64_t kv_row_stride, int64_t seq_q,
                                                 int64_t seq_kv, int32_t heads_q, int32_t heads_kv,
                                                 int32_t head_dim, const int64_t* q_positions,
                                                 const int64_t* kv_positions, float scale, float* out,
                                                 int64_t out_row_stride, float* lse, void* stream) {
    const char* name = "block_fwd_rows";
    if (heads_q <= 0 || heads_kv <= 0) return fail(CPATTN_ERR_INVALID_ARG, "%s: head counts must be > 0", name);
    if (seq_q < 0 || seq_kv < 0) return fail(CPATTN_ERR_INVALID_ARG, "%s: sequence lengths must be >= 0", name);
    if (!(scale > 0.f) || !isfinite(scale))
        return fail(CPATTN_ERR_INVALID_ARG, "%s: scale must be finite and > 0", name);
    if (heads_q % heads_kv != 0)
        return fail(CPATTN_ERR_SHAPE, "%s: heads_q %d not a multiple of heads_kv %d", name, heads_q, heads_kv);
    if (head_dim != 64 && head_dim != 128)
        return fail(CPATTN_ERR_UNSUPPORTED, "%s: head_dim %d (supported: 64, 128)", name, head_dim);
    const int64_t qw = (int64_t)heads_q * head_dim, kw = (int64_t)heads_kv * head_dim;
    if (q_row_stride < qw || q_row_stride % 8 != 0 || q_row_stride > (1LL << 24) || kv_row_stride < kw ||
        kv_row_stride % 8 != 0 || kv_row_stride > (1LL << 24) || out_row_stride < qw || out_row_stride % 4 != 0)
        return fail(CPATTN_ERR_UNSUPPORTED,
                    "%s: row strides must cover the row (q %lld, kv %lld, out %lld elements), be multiples "
                    "of 8 (q, kv) or 4 (out) and at most 2^24 (q, kv)",
                    name, (long long)qw, (long long)kw, (long long)qw);
    if (seq_q == 0) return ok();
    if (!q || !q_positions || !out || !lse)
        return fail(CPATTN_ERR_INVALID_ARG, "%s: q, q_positions, out and lse must be non-NULL", name);
    if (seq_kv > 0 && (!k || !v || !kv_positions))
        return fail(CPATTN_ERR_INVALID_ARG, "%s: k, v and kv_positions must be non-NULL", name);
    if (!aligned16(q) || !aligned16(out) || (seq_kv > 0 && (!aligned16(k) || !aligned16(v))))
        return fail(CPATTN_ERR_UNSUPPORTED, "%s: q, k, v and out must be 16-byte aligned", name);
    if ((seq_q + 31) / 32 * (int64_t)heads_q > kMaxGrid)  // as for block_fwd
        return fail(CPATTN_ERR_UNSUPPORTED, "%s: launch grid too large", name);
    // batch 1; no keys is the same kernel with an empty block (it reads no K/V)
    cpattn::BlockFwdArgs a{q,     k,     v,       q_positions, kv_positions, out,      lse,
                           1,     seq_q, seq_kv, heads_q,     heads_kv,     head_dim, scale, false};
    a.n_blk = 1;
    a.blk[0] = cpattn::KVBlockArg{k, v, kv_positions, seq_kv};
    a.q_row_stride = q_row_stride;
    a.kv_row_stride = kv_row_stride;
    a.out_row_stride = out_row_stride;
    return from_hip(cpattn::launch_block_fwd_bf16(a, (hipStream_t)stream), name);
}

CPATTN_API cpattn_status_t cpattn_attn_bwd_delta(const float* out, const void* dout, cpattn_dtype_t dtype,
                                                 int32_t batch, int64_t seq, int32_t heads, int32_t head_dim,
                                                 float* delta, void* stream) {
    if (dtype != CPATTN_F32 && dtype != CPATTN_BF16)
        return fail(CPATTN_ERR_INVALID_ARG, "attn_bwd_delta: unknown dtype %d", (int)dtype);
    if (batch <= 0 || heads <= 0 || head_dim <= 0)
        return fail(CPATTN_ERR_INVALID_ARG, "attn_bwd_delta: batch, heads and head_dim must be > 0");
    if (seq < 0) return fail(CPATTN_ERR_INVALID_ARG, "attn_bwd_delta: seq must be >= 0");
    if (seq == 0) return ok();
    if (!out || !dout || !delta) return fail(CPATTN_ERR_INVALID_ARG, "attn_bwd_delta: NULL pointer");
    if (head_dim % 4 != 0)
        return fail(CPATTN_ERR_SHAPE, "attn_bwd_delta: head_dim %d not a multiple of 4", head_dim);
    if (!aligned16(out)) return fail(CPATTN_ERR_UNSUPPORTED, "attn_bwd_delta: out must be 16-byte aligned");
    // dout is read four elements at a time: 16 bytes (fp32) or 8 bytes (bf16)
    if ((uintptr_t)dout % (dtype == CPATTN_BF16 ? 8 : 16) != 0)
        return fail(CPATTN_ERR_UNSUPPORTED, "attn_bwd_delta: dout must be %d-byte aligned",
                    dtype == CPATTN_BF16 ? 8 : 16);
    if (((int64_t)batch * seq * heads * 16 + 255) / 256 > kMaxGrid)
        return fail(CPATTN_ERR_UNSUPPORTED, "attn_bwd_delta: launch grid too large");
    return from_hip(cpattn::launch_attn_bwd_delta(out, dout, dtype == CPATTN_BF16, batch, seq, heads, head_dim,
                                                  delta, (hipStream_t)stream),
                    "attn_bwd_delta");
}

// Validation of one block's backward call, enqueueing nothing.  *empty: no (query, key) pair
// (seq_q == 0 or seq_kv == 0), when only the accumulators to overwrite are touched (zeroed).
static cpattn_status_t block_bwd_check(const char* name, const void* q, const void* k, const void* v,
                                       const void* dout, cpattn_dtype_t dtype, int32_t batch, int64_t seq_q,
                                       int64_t seq_kv, int32_t heads_q, int32_t heads_kv, int32_t head_dim,
                                       const int64_t* q_positions, const int64_t* kv_positions, float scale,
                                       const float* lse, const float* delta, const float* dq, const float* dk,
                                       const float* dv, bool wdq, bool wdkv, bool* empty) {
    if (dtype != CPATTN_F32 && dtype != CPATTN_BF16)
        return fail(CPATTN_ERR_INVALID_ARG, "%s: unknown dtype %d", name, (int)dtype);
    if (batch <= 0 || heads_q <= 0 || heads_kv <= 0)
        return fail(CPATTN_ERR_INVALID_ARG, "%s: batch and head counts must be > 0", name);
    if (seq_q < 0 || seq_kv < 0)
        return fail(CPATTN_ERR_INVALID_ARG, "%s: sequence lengths must be >= 0", name);
    if (!(scale > 0.f) || !isfinite(scale))
        return fail(CPATTN_ERR_INVALID_ARG, "%s: scale must be finite and > 0", name);
    if (heads_q % heads_kv != 0)
        return fail(CPATTN_ERR_SHAPE, "%s: heads_q %d not a multiple of heads_kv %d", name, heads_q, heads_kv);
    if (head_dim != 64 && head_dim != 128)
        return fail(CPATTN_ERR_UNSUPPORTED, "%s: head_dim %d (supported: 64, 128)", name, head_dim);
    if (dtype == CPATTN_BF16 && (int64_t)heads_q * head_dim > kMaxRowElems)
        return fail(CPATTN_ERR_UNSUPPORTED, "%s: heads_q * head_dim = %lld above 2^24", name,
                    (long long)heads_q * head_dim);
    *empty = (seq_q == 0 || seq_kv == 0);
    if (*empty) {
        if ((wdq && seq_q > 0 && !dq) || (wdkv && seq_kv > 0 && (!dk || !dv)))
            return fail(CPATTN_ERR_INVALID_ARG, "%s: NULL pointer", name);
        return ok();
    }
    if (!q || !k || !v || !dout || !q_positions || !kv_positions || !lse || !delta || !dq || !dk || !dv)
        return fail(CPATTN_ERR_INVALID_ARG, "%s: NULL pointer", name);
    if (dtype == CPATTN_BF16 && (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) ||
                                 !aligned16(dq) || !aligned16(dk) || !aligned16(dv)))
        return fail(CPATTN_ERR_UNSUPPORTED, "%s: bf16 path needs 16-byte aligned q, k, v, dout, dq, dk, dv", name);
    if ((seq_q + 31) / 32 * (int64_t)batch * heads_q > kMaxGrid ||
        (seq_kv + 31) / 32 * (int64_t)batch * heads_kv > kMaxGrid || heads_q > 65535 || batch > 65535)
        return fail(CPATTN_ERR_UNSUPPORTED, "%s: launch grid too large", name);
    return ok();
}

// A call without pairs: the accumulators to overwrite become zero.
static cpattn_status_t block_bwd_empty(const char* name, int32_t batch, int64_t seq_q, int64_t seq_kv,
                                       int32_t heads_q, int32_t heads_kv, int32_t head_dim, float* dq, float* dk,
                                       float* dv, bool wdq, bool wdkv, void* stream) {
    if (wdq && seq_q > 0) {
        const hipError_t e =
            cpattn::launch_zero_fill(dq, (int64_t)batch * seq_q * heads_q * head_dim, (hipStream_t)stream);
        if (e != hipSuccess) return from_hip(e, name);
    }
    if (wdkv && seq_kv > 0) {
        const int64_t n = (int64_t)batch * seq_kv * heads_kv * head_dim;
        hipError_t e = cpattn::launch_zero_fill(dk, n, (hipStream_t)stream);
        if (e == hipSuccess) e = cpattn::launch_zero_fill(dv, n, (hipStream_t)stream);
        if (e != hipSuccess) return from_hip(e, name);
    }
    return ok();
}

CPATTN_API cpattn_status_t cpattn_block_bwd(const void* q, const void* k, const void* v, const void* dout,
                                            cpattn_dtype_t dtype, int32_t batch, int64_t seq_q, int64_t seq_kv,
                                            int32_t heads_q, int32_t heads_kv, int32_t head_dim,
                                            const int64_t* q_positions, const int64_t* kv_positions,
                                            float scale, const float* lse, const float* delta, float* dq,
                                            float* dk, float* dv, uint32_t flags, void* stream) {
    const char* name = "block_bwd";
    if (flags & ~(uint32_t)(CPATTN_BWD_WRITE_DQ | CPATTN_BWD_WRITE_DKV))
        return fail(CPATTN_ERR_INVALID_ARG, "%s: unknown flags 0x%x", name, flags);
    const bool wdq = (flags & CPATTN_BWD_WRITE_DQ) != 0, wdkv = (flags & CPATTN_BWD_WRITE_DKV) != 0;
    bool empty = false;
    const cpattn_status_t st =
        block_bwd_check(name, q, k, v, dout, dtype, batch, seq_q, seq_kv, heads_q, heads_kv, head_dim,
                        q_positions, kv_positions, scale, lse, delta, dq, dk, dv, wdq, wdkv, &empty);
    if (st != CPATTN_OK) return st;
    if (empty) return block_bwd_empty(name, batch, seq_q, seq_kv, heads_q, heads_kv, head_dim, dq, dk, dv, wdq, wdkv,
                                      stream);
    cpattn::BlockBwdArgs a{q,  k,     v,     dout,   q_positions, kv_positions, lse,      delta, dq, dk,
                           dv, batch, seq_q, seq_kv, heads_q,     heads_kv,     head_dim, scale, wdq, wdkv};
    const hipError_t e = (dtype == CPATTN_BF16) ? cpattn::launch_block_bwd_bf16(a, (hipStream_t)stream)
                                                : cpattn::launch_block_bwd_f32(a, (hipStream_t)stream);
    return from_hip(e, name);
}

CPATTN_API cpattn_status_t cpattn_ring_share_bwd(const void* q, const void* dout, const void* const* k_blocks,
                                                 const void* const* v_blocks,
                                                 const int64_t* const* kv_positions, const int64_t* seq_kv,
                                                 int32_t n_blocks, cpattn_dtype_t dtype, int32_t batch,
                                                 int64_t seq_q, int32_t heads_q, int32_t heads_kv,
                                                 int32_t head_dim, const int64_t* q_positions, float scale,
                                                 const float* lse, const float* delta, float* dq,
                                                 float* const* dk_blocks, float* const* dv_blocks, void* stream) {
    const char* name = "ring_share_bwd";
    if (n_blocks <= 0 || n_blocks > cpattn::kMaxRingBlocks)
        return fail(CPATTN_ERR_INVALID_ARG, "%s: n_blocks %d outside [1, %d]", name, n_blocks,
                    cpattn::kMaxRingBlocks);
    if (!k_blocks || !v_blocks || !kv_positions || !seq_kv || !dk_blocks || !dv_blocks)
        return fail(CPATTN_ERR_INVALID_ARG, "%s: NULL block array", name);
    // every block validated as a single-block call (dq written by the first, dk and dv by
    // their own block) before anything is enqueued
    bool any_pairs = false;
    for (int32_t o = 0; o < n_blocks; ++o) {
        bool empty = false;
        const cpattn_status_t st = block_bwd_check(name, q, k_blocks[o], v_blocks[o], dout, dtype, batch, seq_q,
                                                   seq_kv[o], heads_q, heads_kv, head_dim, q_positions,
                                                   kv_positions[o], scale, lse, delta, dq, dk_blocks[o],
                                                   dv_blocks[o], o == 0, true, &empty);
        if (st != CPATTN_OK) return st;
        any_pairs = any_pairs || !empty;
    }
    if (!any_pairs) {
        // no pair in any block: dq and every block's dk, dv become zero
        for (int32_t o = 0; o < n_blocks; ++o) {
            const cpattn_status_t st = block_bwd_empty(name, batch, seq_q, seq_kv[o], heads_q, heads_kv, head_dim,
                                                       dq, dk_blocks[o], dv_blocks[o], o == 0, true, stream);
            if (st != CPATTN_OK) return st;
        }
        return ok();
    }
    if (dtype != CPATTN_BF16) {
        // fp32: the per-step calls, the first writing dq and each block writing its dk, dv
        for (int32_t o = 0; o < n_blocks; ++o) {
            const cpattn_status_t st = cpattn_block_bwd(
                q, k_blocks[o], v_blocks[o], dout, dtype, batch, seq_q, seq_kv[o], heads_q, heads_kv, head_dim,
                q_positions, kv_positions[o], scale, lse, delta, dq, dk_blocks[o], dv_blocks[o],
                CPATTN_BWD_WRITE_DKV | (o == 0 ? CPATTN_BWD_WRITE_DQ : 0u), stream);
            if (st != CPATTN_OK) return st;
        }
        return ok();
    }
    // the dk/dv launch: (longest block's 128-key blocks) x (blocks) x (batch, kv head) workgroups
    int64_t max_kb = 0;
    for (int32_t o = 0; o < n_blocks; ++o) max_kb = std::max(max_kb, (seq_kv[o] + 127) / 128);
    if (max_kb * n_blocks * batch * heads_kv > kMaxGrid)
        return fail(CPATTN_ERR_UNSUPPORTED, "%s: launch grid too large", name);
    cpattn::RingBwdBlock blocks[cpattn::kMaxRingBlocks];
    for (int32_t o = 0; o < n_blocks; ++o)
        blocks[o] = cpattn::RingBwdBlock{k_blocks[o], v_blocks[o], kv_positions[o], seq_kv[o], dk_blocks[o],
                                         dv_blocks[o]};
    const cpattn::BlockBwdArgs a{q,       nullptr, nullptr, dout,     q_positions, nullptr, lse,   delta,
                                 dq,      nullptr, nullptr, batch,    seq_q,       0,       heads_q, heads_kv,
                                 head_dim, scale,  true,    true};
    return from_hip(cpattn::launch_ring_bwd_bf16(a, n_blocks, blocks, (hipStream_t)stream), name);
}

CPATTN_API cpattn_status_t cpattn_ring_share_fwd(const void* q, const void* const* k_blocks,
                                                 const void* const* v_blocks,
                                                 const int64_t* const* kv_positions, const int64_t* seq_kv,
                                                 int32_t n_blocks, cpattn_dtype_t dtype, int32_t batch,
                                                 int64_t seq_q, int32_t heads_q, int32_t heads_kv,
                                                 int32_t head_dim, const int64_t* q_positions, float scale,
                                                 float* out, float* lse, void* stream) {
    const char* name = "ring_share_fwd";
    if (n_blocks <= 0 || n_blocks > cpattn::kMaxRingBlocks)
        return fail(CPATTN_ERR_INVALID_ARG, "%s: n_blocks %d outside [1, %d]", name, n_blocks,
                    cpattn::kMaxRingBlocks);
    if (!k_blocks || !v_blocks || !kv_positions || !seq_kv)
        return fail(CPATTN_ERR_INVALID_ARG, "%s: NULL block array", name);
    for (int32_t o = 0; o < n_blocks; ++o)
        if (seq_kv[o] < 0) return fail(CPATTN_ERR_INVALID_ARG, "%s: seq_kv[%d] < 0", name, o);
    if (dtype != CPATTN_BF16) {
        // fp32: one block at a time, the later ones merged in the epilogue.  Every block is
        // validated before the first launch, so a call that fails has enqueued nothing.
        for (int32_t o = 0; o < n_blocks; ++o) {
            bool empty = false;
            const cpattn_status_t st =
                block_fwd_check(name, q, k_blocks[o], v_blocks[o], dtype, batch, seq_q, seq_kv[o], heads_q,
                                heads_kv, head_dim, q_positions, kv_positions[o], scale, out, lse, &empty);
            if (st != CPATTN_OK) return st;
            if (empty) return ok();  // no query rows: nothing to do for any block
        }
        for (int32_t o = 0; o < n_blocks; ++o) {
            const cpattn_status_t st =
                block_fwd_launch(name, o > 0, q, k_blocks[o], v_blocks[o], dtype, batch, seq_q, seq_kv[o],
                                 heads_q, heads_kv, head_dim, q_positions, kv_positions[o], scale, out, lse,
                                 stream);
            if (st != CPATTN_OK) return st;
        }
        return ok();
    }
    // validate every block as a single-block call would, without launching
    for (int32_t o = 0; o < n_blocks; ++o) {
        if (seq_kv[o] > 0 && (!k_blocks[o] || !v_blocks[o] || !kv_positions[o]))
            return fail(CPATTN_ERR_INVALID_ARG, "%s: block %d has a NULL pointer", name, o);
        if (seq_kv[o] > 0 && (!aligned16(k_blocks[o]) || !aligned16(v_blocks[o])))
            return fail(CPATTN_ERR_UNSUPPORTED, "%s: block %d not 16-byte aligned", name, o);
    }
    if (batch <= 0 || heads_q <= 0 || heads_kv <= 0)
        return fail(CPATTN_ERR_INVALID_ARG, "%s: batch and head counts must be > 0", name);
    if (seq_q < 0) return fail(CPATTN_ERR_INVALID_ARG, "%s: seq_q must be >= 0", name);
    if (!(scale > 0.f) || !isfinite(scale))
        return fail(CPATTN_ERR_INVALID_ARG, "%s: scale must be finite and > 0", name);
    if (heads_q % heads_kv != 0)
        return fail(CPATTN_ERR_SHAPE, "%s: heads_q %d not a multiple of heads_kv %d", name, heads_q, heads_kv);
    if (head_dim != 64 && head_dim != 128)
        return fail(CPATTN_ERR_UNSUPPORTED, "%s: head_dim %d (supported: 64, 128)", name, head_dim);
    if ((int64_t)heads_kv * head_dim > kMaxRowElems)
        return fail(CPATTN_ERR_UNSUPPORTED, "%s: heads_kv * head_dim = %lld above 2^24", name,
                    (long long)heads_kv * head_dim);
    if (seq_q == 0) return ok();
    if (!q || !q_positions || !out || !lse)
        return fail(CPATTN_ERR_INVALID_ARG, "%s: q, q_positions, out and lse must be non-NULL", name);
    if (!aligned16(q) || !aligned16(out))
        return fail(CPATTN_ERR_UNSUPPORTED, "%s: bf16 path needs 16-byte aligned q and out", name);
    if ((seq_q + 31) / 32 * (int64_t)batch * heads_q > kMaxGrid)  // as for block_fwd
        return fail(CPATTN_ERR_UNSUPPORTED, "%s: launch grid too large", name);
    cpattn::BlockFwdArgs a{q, nullptr, nullptr, q_positions, nullptr, out,      lse,   batch,
                           seq_q, 0,   heads_q, heads_kv,    head_dim, scale,   false};
    a.n_blk = 0;
    for (int32_t o = 0; o < n_blocks; ++o) {
        if (seq_kv[o] == 0) continue;  // no keys: contributes nothing
        a.blk[a.n_blk++] = cpattn::KVBlockArg{k_blocks[o], v_blocks[o], kv_positions[o], seq_kv[o]};
    }
    if (a.n_blk == 0) return from_hip(cpattn::launch_block_fwd_empty(a, (hipStream_t)stream), name);
    a.k = a.blk[0].k;
    a.seq_kv = a.blk[0].seq;
    return from_hip(cpattn::launch_block_fwd_bf16(a, (hipStream_t)stream), name);
}

CPATTN_API cpattn_status_t cpattn_lse_merge(float* out, float* lse, const float* out_tile,
                                            const float* lse_tile, int32_t batch, int64_t seq,
                                            int32_t heads, int32_t head_dim, void* stream) {
    if (batch <= 0 || heads <= 0 || head_dim <= 0)
        return fail(CPATTN_ERR_INVALID_ARG, "lse_merge: batch, heads and head_dim must be > 0");
    if (seq < 0) return fail(CPATTN_ERR_INVALID_ARG, "lse_merge: seq must be >= 0");
    if (head_dim % 4 != 0) return fail(CPATTN_ERR_SHAPE, "lse_merge: head_dim %d not a multiple of 4", head_dim);
    if (head_dim > 4096) return fail(CPATTN_ERR_UNSUPPORTED, "lse_merge: head_dim %d above 4096", head_dim);
    if (seq == 0) return ok();
    if (!out || !lse || !out_tile || !lse_tile)
        return fail(CPATTN_ERR_INVALID_ARG, "lse_merge: NULL pointer");
    if (!aligned16(out) || !aligned16(out_tile))
        return fail(CPATTN_ERR_UNSUPPORTED, "lse_merge: out and out_tile must be 16-byte aligned");
    if (out == out_tile || lse == lse_tile)
        return fail(CPATTN_ERR_INVALID_ARG, "lse_merge: the tile must not alias the accumulator");
    if (((int64_t)batch * seq * heads + 7) / 8 > kMaxGrid)  // 8 rows per block
        return fail(CPATTN_ERR_UNSUPPORTED, "lse_merge: launch grid too large");
    return from_hip(cpattn::launch_lse_merge(out, lse, out_tile, lse_tile, batch, seq, heads, head_dim,
                                             (hipStream_t)stream),
                    "lse_merge");
}

CPATTN_API cpattn_status_t cpattn_reorder_gathered(const void* in, void* out, int32_t batch,
                                                   int64_t seq_len, int64_t row_bytes,
                                                   int32_t cp_size, cpattn_reorder_dir_t dir,
                                                   void* stream) {
    if (batch <= 0 || seq_len <= 0 || row_bytes <= 0 || cp_size <= 0)
        return fail(CPATTN_ERR_INVALID_ARG, "reorder_gathered: sizes must be > 0");
    if (dir != CPATTN_RANK_TO_SEQ && dir != CPATTN_SEQ_TO_RANK)
        return fail(CPATTN_ERR_INVALID_ARG, "reorder_gathered: unknown direction %d", (int)dir);
    if (!in || !out) return fail(CPATTN_ERR_INVALID_ARG, "reorder_gathered: NULL pointer");
    if (in == out) return fail(CPATTN_ERR_INVALID_ARG, "reorder_gathered: in and out must differ");
    if (seq_len % (2 * (int64_t)cp_size) != 0)
        return fail(CPATTN_ERR_SHAPE, "reorder_gathered: seq_len %lld not divisible by 2*cp_size = %lld",
                    (long long)seq_len, 2LL * cp_size);
    if (2LL * cp_size > 65535 || batch > 65535)
        return fail(CPATTN_ERR_UNSUPPORTED, "reorder_gathered: cp_size or batch too large");
    const int64_t chunk_bytes = seq_len / (2 * (int64_t)cp_size) * row_bytes;
    if (chunk_bytes / 256 + 1 > kMaxGrid)  // the byte path copies 256 bytes per block
        return fail(CPATTN_ERR_UNSUPPORTED, "reorder_gathered: chunk too large");
    return from_hip(cpattn::launch_reorder_gathered(in, out, batch, seq_len, row_bytes, cp_size, (int32_t)dir,
                                                    (hipStream_t)stream),
                    "reorder_gathered");
}

namespace {

cpattn_status_t ulysses_common(const char* name, bool zigzag, const void* in, void* out, int32_t elem_bytes,
                               int32_t batch, int64_t seq_len, int32_t heads, int32_t head_dim,
                               int32_t cp_size, int32_t group, cpattn_permute_dir_t dir, void* stream) {
    if (elem_bytes <= 0 || batch <= 0 || seq_len <= 0 || heads <= 0 || head_dim <= 0 || cp_size <= 0)
        return fail(CPATTN_ERR_INVALID_ARG, "%s: sizes must be > 0", name);
    if (dir != CPATTN_SEQ_TO_HEADS && dir != CPATTN_HEADS_TO_SEQ)
        return fail(CPATTN_ERR_INVALID_ARG, "%s: unknown direction %d", name, (int)dir);
    if (group < 0 || group >= cp_size)
        return fail(CPATTN_ERR_INVALID_ARG, "%s: group %d outside [0, %d)", name, group, cp_size);
    if (!in || !out) return fail(CPATTN_ERR_INVALID_ARG, "%s: NULL pointer", name);
    if (in == out) return fail(CPATTN_ERR_INVALID_ARG, "%s: in and out must differ", name);
    const int64_t div = zigzag ? 2 * (int64_t)cp_size : cp_size;
    if (seq_len % div != 0)
        return fail(CPATTN_ERR_SHAPE, "%s: seq_len %lld not divisible by %s %lld", name, (long long)seq_len,
                    zigzag ? "2*cp_size =" : "cp_size", (long long)div);
    if (heads % cp_size != 0)
        return fail(CPATTN_ERR_SHAPE, "%s: heads %d not divisible by cp_size %d", name, heads, cp_size);
    const int64_t seg_bytes = (int64_t)(heads / cp_size) * head_dim * elem_bytes;
    const int64_t span_bytes = seq_len / cp_size * seg_bytes;
    if (span_bytes >= (1LL << 31) || (int64_t)cp_size * batch > 65535)
        return fail(CPATTN_ERR_UNSUPPORTED, "%s: one shard's head group exceeds 2 GiB or "
                                            "cp_size*batch exceeds 65535", name);
    return from_hip(cpattn::launch_ulysses_permute(in, out, elem_bytes, batch, seq_len, heads, head_dim,
                                                   cp_size, group, (int32_t)dir, zigzag, (hipStream_t)stream),
                    name);
}

}  // namespace

CPATTN_API cpattn_status_t cpattn_ulysses_permute(const void* in, void* out, int32_t elem_bytes,
                                                  int32_t batch, int64_t seq_len, int32_t heads,
                                                  int32_t head_dim, int32_t cp_size, int32_t group,
                                                  cpattn_permute_dir_t dir, void* stream) {
    return ulysses_common("ulysses_permute", false, in, out, elem_bytes, batch, seq_len, heads, head_dim,
                          cp_size, group, dir, stream);
}

CPATTN_API cpattn_status_t cpattn_ulysses_permute_zigzag(const void* in, void* out, int32_t elem_bytes,
                                                         int32_t batch, int64_t seq_len, int32_t heads,
                                                         int32_t head_dim, int32_t cp_size, int32_t group,
                                                         cpattn_permute_dir_t dir, void* stream) {
    return ulysses_common("ulysses_permute_zigzag", true, in, out, elem_bytes, batch, seq_len, heads,
                          head_dim, cp_size, group, dir, stream);
}
