// bf16 attention backward of one block on the gfx950 matrix cores.
//
// What it computes ("On Context Parallelism", section Peer-to-peer / Backward: each ring step
// yields tile_dq, tile_dk, tile_dv of the local queries against one K/V block from the saved
// output and lse; the formulas are the chain rule of the attention definition):
//   p_ij = exp(scale <q_i,k_j> - lse_i) on visible pairs, D_i = <dout_i, out_i> (given),
//   ds_ij = p_ij (<dout_i, v_j> - D_i),
//   dq_i += scale sum_j ds_ij k_j,  dk_j += scale sum_i ds_ij q_i,  dv_j += sum_i p_ij dout_i.
// lse is the row's complete log-sum-exp, so p is the global softmax weight and the blocks'
// contributions add up to the whole gradient.
//
// Two kernels, each with bf16 matrix-core products (v_mfma_f32_32x32x16_bf16) and fp32
// accumulation; p and ds are rounded to bf16 (RNE) before the products that consume them.
//
// dq kernel: a block of 4 waves owns G query heads sharing one K/V head times 128/G query
// positions; each lane holds one query row (its q and dout as matrix operands).  K/V tiles
// of 64 keys are staged in LDS (direct global->LDS loads, two stages).  Per 32-key block of a
// tile: S^T = K Q^T and dP^T - D = V dO^T - D (K, V rows read from LDS; the products start from
// -D), p and ds per lane (one query: lse and D are per-lane scalars), dQ^T += K^T dS^T (K read
// transposed, ds_read_b64_tr_b16).
//   Launches too small to fill the chip take 8 waves instead, two per 32-row query group, each
//   over one 32-key half of every tile (block_bwd_dq_kernel<2>).
// dk/dv kernel: a block of 8 waves owns 128 keys of one K/V head, in 4 groups of 32 (one key
// per lane; k as a matrix operand in registers, the block's v rows in LDS), and walks the
// query tiles of 64 rows that see them, for every query head of the group.  Q, dO, lse and D
// tiles are staged in LDS.  Each key group has two waves, one per 32-query half of every
// tile, so two waves share each SIMD and one's products run beside the other's p/ds math.
// Per wave and tile:
//   S = Q K^T and dP = dO V^T (Q, dO, V rows from LDS), p and ds (lse and D per accumulator
//   row, read from LDS), dV^T += dO^T P and dK^T += Q^T dS (Q, dO read transposed).
// At the end the second-half waves hand their partial dK, dV to the first-half waves through
// LDS, which add them and write the result.
// The causal structure is used as in the forward: tiles entirely hidden are skipped, tiles
// entirely visible need no mask, and on partly visible tiles the packed bf16 weights of hidden
// pairs are cleared, by comparing row indices with a count found once by binary search over
// the positions.
// cpattn_ring_share_bwd runs the dq kernel once per K/V block and the dk/dv kernel once over
// all the blocks (each workgroup one block's 128 keys of one K/V head).
// Launches of at least eight rounds of workgroups take their items from queues at run time
// (one per XCD, taking the others' last items once its own run out), as the forward does:
// the XCDs hold different clocks under load, and equal shares would end at different times.
#include "cpattn_internal.h"

#include <atomic>
#include <math.h>

namespace cpattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int kTile = 64;                   // keys (dq kernel) or queries (dk/dv kernel) per tile
constexpr int kNW = 4;                      // waves per block
constexpr int kThreads = 64 * kNW;
constexpr float kLog2e = 1.4426950408889634f;

// One K/V block of a dk/dv launch: its keys, values, positions and gradient buffers.
struct BwdKV {
    const __bf16* k;
    const __bf16* v;
    const int64_t* kvpos;
    float* dk;
    float* dv;
    int64_t seq_kv;
    int64_t n_kb;  // key blocks of 128 keys
};

struct BwdParams {
    const __bf16* q;
    const __bf16* k;
    const __bf16* v;
    const __bf16* dout;
    const int64_t* qpos;
    const int64_t* kvpos;
    const float* lse;
    const float* delta;
    float* dq;
    float* dk;
    float* dv;
    int64_t seq_q;
    int64_t seq_kv;
    int32_t batch;
    int32_t heads_q;
    int32_t heads_kv;
    int32_t ratio;      // heads_q / heads_kv
    float c;            // scale * log2(e)
    float scale;
    // dq grid: G query heads per block, pq positions, n_hg head groups, n_cols columns
    int32_t G;
    int32_t pq;
    int32_t n_hg;
    int32_t n_cols;
    int64_t n_qt;
    int32_t xcd_cols;
    // dk/dv grid: key blocks of 128 keys, columns (b, kv head)
    int64_t n_kb;
    int32_t kv_cols;
    int32_t kv_xcd_cols;
    int32_t write_dq;   // overwrite instead of adding
    int32_t write_dkv;
    // dk/dv launch: the K/V blocks it covers (a single-block call fills kv[0] from k, v,
    // kvpos, dk, dv); workgroups take key block kb of block o in the order (o, kb): the
    // workgroups running at one time mostly share a block, so they stream the same query
    // tiles through L2 (interleaving the blocks by key block lost 6% on the 256K share), and
    // the launch has no gap between one block's last workgroups and the next block's
    int32_t n_blk;
    int64_t max_n_kb;
    BwdKV kv[kMaxRingBlocks];
    // work taken from queues at run time (per_q > 0; set by each launch for its own grid):
    // n_queues queues (8: one per XCD, holding its columns' work; 1: all of it) of per_q
    // items each, counted in counter slot `slot`
    int32_t n_queues;
    int32_t slot;
    int64_t per_q;
};

// Work counters of the launches that take their items from queues: a slot per launch, taken
// in turn, 16 counters per slot, zeroed by a one-workgroup kernel on the launch's stream.
// Device code reaches the array by name; host code never uses it.
constexpr int kCtrSlots = 256;
__device__ int g_bwd_ctr[kCtrSlots * 16];

__global__ void bwd_ctr_reset_kernel(int slot) { g_bwd_ctr[slot * 16 + threadIdx.x] = 0; }

// The item a workgroup works on when its launch uses queues: the next one of its XCD's queue
// (the hardware deals consecutive workgroups to the 8 XCDs in turn, and the XCDs hold
// different clocks under load, so equal shares would end at different times), or, once that
// queue is empty, of the next queue that is not.  Returns false when every queue is empty (the
// whole workgroup then has nothing to do).  Each item is done by exactly one workgroup, with
// the same code wherever it runs.
__device__ inline bool claim_item(const BwdParams& p, int& queue, int64_t& item) {
    __shared__ int claim[2];
    if (threadIdx.x == 0) {
        const int home = p.n_queues > 1 ? (int)(blockIdx.x & 7) : 0;
        int q = -1, it = 0;
        for (int y = 0; y < p.n_queues; ++y) {
            const int qq = (home + y) % p.n_queues;
            const int i = atomicAdd(&g_bwd_ctr[p.slot * 16 + qq], 1);
            if (i < p.per_q) {
                q = qq;
                it = i;
                break;
            }
        }
        claim[0] = q;
        claim[1] = it;
    }
    __syncthreads();
    queue = claim[0];
    item = claim[1];
    return queue >= 0;
}

__device__ inline int wave_sum(int x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

__device__ inline bf16x8 lds_b128(const LDS_AS char* p) { return *(const LDS_AS bf16x8*)p; }

__device__ inline bf16x8 lds_tr_pair(const LDS_AS char* p0, const LDS_AS char* p1) {
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)p0);
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)p1);
    const s16x8 c = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_bit_cast(bf16x8, c);
}

// Buffer descriptor over `bytes` bytes from `base` (raw, no stride; word 3 as gfx9 wants).
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// One 16-byte direct load into LDS: this lane's 16 bytes come from the descriptor's base +
// voff and land at lds_base + 16*lane.  A buffer load, unlike global_load_lds, is not a flat
// access, so LDS reads issued while it is in flight keep exact lgkm counts.
__device__ inline void load_lds16(__amdgpu_buffer_rsrc_t r, uint32_t voff, LDS_AS void* lds_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_base, 16, voff, 0, 0, 0);
}

__device__ inline bf16x8 load_row16(const __bf16* p, bool valid) {
    const u32x4 raw = valid ? *(const u32x4*)p : u32x4{0, 0, 0, 0};
    return __builtin_bit_cast(bf16x8, raw);
}

__device__ inline f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Masking after the fact on a partly visible tile.  The weights are computed for every pair
// of the tile and packed to bf16 two per register (element 2m in the low half, 2m + 1 in the
// high half); a hidden pair's weight may be anything, inf or NaN included, and its 16 bits are
// replaced whole by +0, so the products see exactly what a weight of 0 would give.  n is how
// many of the register's two elements are kept, counted from the low half (keep_low) or from
// the high half (keep_high); any n outside 0..2 is clamped.
__device__ inline uint32_t keep_low(int n) { return n >= 2 ? 0xFFFFFFFFu : (n == 1 ? 0x0000FFFFu : 0u); }
__device__ inline uint32_t keep_high(int n) { return n >= 2 ? 0xFFFFFFFFu : (n == 1 ? 0xFFFF0000u : 0u); }
__device__ inline bf16x8 and_mask(const bf16x8& x, const u32x4& m) {
    return __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, x) & m);
}

// Scheduling hint for a loop of N steps, each of M matrix-core products fed by R LDS reads:
// issue the reads A steps ahead of the products that use them (sync group G).  X more LDS
// reads, which the first products need, go out with the first group, and Y more, which the
// vector work after the products needs, with the last one.
template <int N, int M, int R, int G, int A = 2, int X = 0, int Y = 0>
__device__ inline void sched_reads_ahead() {
    __builtin_amdgcn_sched_group_barrier(0x100, R * A + X, G);
#pragma unroll
    for (int i = 0; i < N - A - 1; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, M, G);
        __builtin_amdgcn_sched_group_barrier(0x100, R, G);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, M, G);
    __builtin_amdgcn_sched_group_barrier(0x100, R + Y, G);
    __builtin_amdgcn_sched_group_barrier(0x008, M * A, G);
}

// Tiles in LDS are row-major (D bf16 per row) with 16-byte chunk c of row r stored at chunk
// c ^ swz(r).
//   D = 128 (256-byte rows, one per bank row): swz(r) = ((r & 3) << 2) | ((r >> 2) & 3).  Over
//   16 aligned rows swz is a permutation of 0..15, so a row read of 16 consecutive rows at one
//   chunk touches 16 distinct chunk slots; over 4 aligned rows its top two bits differ, so a
//   transposed read of 4 rows x 4 chunks (one 32-lane pass) also touches 16 distinct slots.
//   D = 64 (128-byte rows, two per bank row: even rows in its first half, odd rows in its
//   second): swz(r) = (((r >> 1) & 1) << 2) | ((r >> 2) & 3).  Over 16 aligned rows it is a
//   permutation of 0..7 on the even rows and on the odd rows, so a row read again touches 16
//   distinct slots; in 4 aligned rows the two even (and the two odd) rows differ in its top
//   bit, so a transposed read's 4 aligned chunks land in the two halves of the bank row.
// Both access patterns are free of bank conflicts at either width.
struct TrOff {
    uint32_t a, b;
};
template <int D> struct BwdGeom {
    static_assert(D == 64 || D == 128, "head dim 64 or 128");
    static constexpr int kRowBytes = D * 2;
    static constexpr int kTileBytes = kTile * kRowBytes;
    static constexpr int kChunks = D / 8;              // 16-byte chunks per row
    static constexpr int kRowsPerLoad = 64 / kChunks;  // rows one 64-lane 16-byte load fills
    __device__ static inline int swz(int r) {
        return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
    }
    // Row-read offsets (matrix-core A operand, 32 rows x 16 columns, lane = row l32 holding
    // columns 16*ks + 8*half .. +7): row l32 of a 32-row block.
    __device__ static inline uint32_t row_off(int lane, int ks) {
        const int l32 = lane & 31, half = lane >> 5;
        return l32 * kRowBytes + (((2 * ks + half) ^ swz(l32)) << 4);
    }
    // Transposed-read offsets (A operand = columns 32*db .. +31 as rows, 16 tile rows as k):
    // the k order is the accumulator's row order 16*ks2 + 8*(j/4) + 4*half + j%4, so that an
    // operand packed straight from an accumulator lines up.  Two 8-byte reads per operand:
    // tile rows vkey and vkey + 8 of the 16-row step.
    __device__ static inline TrOff tr_off(int lane, int db) {
        const int half = lane >> 5, grp = lane >> 4, s16 = lane & 15;
        const int vkey = 4 * half + (s16 >> 2);
        const int chunk = 4 * db + 2 * (grp & 1) + ((s16 & 3) >> 1);
        const uint32_t lo = (s16 & 1) << 3;
        return TrOff{vkey * kRowBytes + ((chunk ^ swz(vkey)) << 4) + lo,
                     (vkey + 8) * kRowBytes + ((chunk ^ swz(vkey + 8)) << 4) + lo};
    }
};

// ------------------------------------------------------------------------------------------
// dq kernel
// ------------------------------------------------------------------------------------------
// KS = 1: 4 waves, each over both 32-key halves of every K/V tile.  KS = 2 (launches too small
// to fill the chip): 8 waves, two per 32-row query group, one per 32-key half of every tile,
// each with its own partial dQ; the second-half waves hand theirs over through LDS at the end.
template <int D, int KS>
__global__ void __launch_bounds__(64 * kNW * KS, 1) block_bwd_dq_kernel(const BwdParams p) {
    using BG = BwdGeom<D>;
    constexpr int kD = D;
    constexpr int kRowBytes = BG::kRowBytes;
    constexpr int kTileBytes = BG::kTileBytes;
    constexpr int kRPL = BG::kRowsPerLoad;
    constexpr int NW = kNW * KS;
    constexpr int kThr = 64 * NW;
    constexpr int kRowsW = kTile / NW;  // tile rows each wave loads
    static_assert(kRowsW % kRPL == 0, "whole loads per wave");
    constexpr int kLd = kRowsW / kRPL;
    constexpr int NKB = 2 / KS;         // 32-key halves of a tile each wave takes
    __shared__ __attribute__((aligned(16))) char lds_stage0[2 * kTileBytes];  // [K|V]
    __shared__ __attribute__((aligned(16))) char lds_stage1[2 * kTileBytes];
    __shared__ int red[2 * NW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = KS > 1 ? __builtin_amdgcn_readfirstlane(tid >> 6) : (tid >> 6);
    const int qg = KS > 1 ? w % kNW : w;     // query group: rows 32*qg .. +31 of the block
    const int khalf = KS > 1 ? w / kNW : 0;  // with KS = 2: the 32-key half of each tile
    const int half = lane >> 5;
    const int l32 = lane & 31;

    int col;
    int64_t qt_rank;
    if (p.per_q > 0) {
        int q;
        int64_t it;
        if (!claim_item(p, q, it)) return;
        if (p.n_queues > 1) {
            qt_rank = it / p.xcd_cols;
            col = q + 8 * (int)(it % p.xcd_cols);
        } else {
            col = (int)(it % p.n_cols);
            qt_rank = it / p.n_cols;
        }
    } else if (p.xcd_cols > 0) {
        const int x = blockIdx.x & 7;
        const int64_t kk = blockIdx.x >> 3;
        qt_rank = kk / p.xcd_cols;
        col = x + 8 * (int)(kk % p.xcd_cols);
    } else {
        col = (int)(blockIdx.x % p.n_cols);
        qt_rank = blockIdx.x / p.n_cols;
    }
    const int64_t qt = p.n_qt - 1 - qt_rank;  // late queries (most keys) first
    const int hg = col % p.n_hg;
    const int kvh = (col / p.n_hg) % p.heads_kv;
    const int64_t b = col / (p.n_hg * p.heads_kv);

    const int64_t q0 = qt * p.pq;
    const int64_t q_last = (q0 + p.pq < p.seq_q ? q0 + p.pq : p.seq_q) - 1;
    const int64_t pmin = p.qpos[q0];
    const int64_t pmax = p.qpos[q_last];

    // visible key tiles (a prefix) and tiles visible to every query of the block
    const int64_t n_tiles = (p.seq_kv + kTile - 1) / kTile;
    int c_ne = 0, c_full = 0;
    for (int64_t t = tid; t < n_tiles; t += kThr) {
        c_ne += (p.kvpos[t * kTile] <= pmax) ? 1 : 0;
        const int64_t lk = t * kTile + kTile - 1;
        c_full += (lk < p.seq_kv && p.kvpos[lk] <= pmin) ? 1 : 0;
    }
    c_ne = wave_sum(c_ne);
    c_full = wave_sum(c_full);
    if (lane == 0) {
        red[w] = c_ne;
        red[NW + w] = c_full;
    }
    __syncthreads();
    int n_ne = 0, n_full = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        n_ne += red[i];
        n_full += red[NW + i];
    }
    n_ne = __builtin_amdgcn_readfirstlane(n_ne);  // the same in every lane: scalar registers
    n_full = __builtin_amdgcn_readfirstlane(n_full);

    // K/V tile loads (both tensors row-read, same swizzle)
    const int64_t kvstride = (int64_t)p.heads_kv * kD;
    const char* kbase = (const char*)(p.k + (b * p.seq_kv * p.heads_kv + kvh) * (int64_t)kD);
    const char* vbase = (const char*)(p.v + (b * p.seq_kv * p.heads_kv + kvh) * (int64_t)kD);
    const int64_t tile_bytes_g = (int64_t)kTile * kvstride * 2;
    const int ld_row_in = lane / BG::kChunks;
    const int ld_chunk = lane % BG::kChunks;
    uint32_t koff[kLd];
#pragma unroll
    for (int i = 0; i < kLd; ++i) {
        const int row = w * kRowsW + kRPL * i + ld_row_in;
        koff[i] = (uint32_t)(row * kvstride * 2) + ((ld_chunk ^ BG::swz(row)) << 4);
    }
    auto issue_tile = [&](int jt, LDS_AS char* kt) {
        LDS_AS char* vt = kt + kTileBytes;
        const char* kb_t = kbase + (int64_t)jt * tile_bytes_g;
        const char* vb_t = vbase + (int64_t)jt * tile_bytes_g;
        const int64_t rmax = p.seq_kv - 1 - (int64_t)jt * kTile;  // last valid row of the tile
        // the descriptors cover the tile's rows that exist (a tile spans < 4 GiB)
        const uint32_t span = (uint32_t)((rmax < kTile - 1 ? rmax : kTile - 1) * kvstride * 2 + kRowBytes);
        const __amdgpu_buffer_rsrc_t kr = make_rsrc(kb_t, span);
        const __amdgpu_buffer_rsrc_t vr = make_rsrc(vb_t, span);
#pragma unroll
        for (int i = 0; i < kLd; ++i) {
            const int row = w * kRowsW + kRPL * i + ld_row_in;
            // rows past the end re-read the last key (finite data the mask hides)
            const uint32_t back = (row > rmax) ? (uint32_t)((row - rmax) * kvstride * 2) : 0u;
            load_lds16(kr, koff[i] - back, kt + (w * kRowsW + kRPL * i) * kRowBytes);
            load_lds16(vr, koff[i] - back, vt + (w * kRowsW + kRPL * i) * kRowBytes);
        }
    };

    // this lane's query row: q and dout as B operands, lse (log2 domain) and D as scalars
    const int row0 = qg * 32;
    const int hs = row0 / p.pq;
    const int64_t i = q0 + (row0 % p.pq) + l32;
    const int64_t head = (int64_t)kvh * p.ratio + (int64_t)hg * p.G + hs;
    const bool valid = i < p.seq_q;
    const int64_t mypos = valid ? p.qpos[i] : INT64_MIN;
    const int64_t qrow = (b * p.seq_q + (valid ? i : 0)) * p.heads_q + head;
    bf16x8 qreg[kD / 16], doreg[kD / 16];
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) {
        qreg[ks] = load_row16(p.q + qrow * kD + 16 * ks + 8 * half, valid);
        doreg[ks] = load_row16(p.dout + qrow * kD + 16 * ks + 8 * half, valid);
    }
    const int64_t li = (b * p.heads_q + head) * p.seq_q + (valid ? i : 0);
    const float lse_v = valid ? p.lse[li] : INFINITY;
    // a row with no visible key anywhere has lse = -inf and every pair masked
    const float lse2 = (lse_v == -INFINITY) ? INFINITY : lse_v * kLog2e;
    const float dlt = valid ? p.delta[li] : 0.f;
    f32x16 ndlt;  // -D in every entry: the dP products accumulate onto it
#pragma unroll
    for (int v = 0; v < 16; ++v) ndlt[v] = -dlt;

    int64_t vis = 0;  // keys visible to this row, needed only when some tile is partly visible
    if (n_full < n_ne) {
        int64_t lo = (int64_t)n_full * kTile;
        int64_t hi = (int64_t)n_ne * kTile < p.seq_kv ? (int64_t)n_ne * kTile : p.seq_kv;
        while (lo < hi) {
            const int64_t mid = (lo + hi) >> 1;
            if (p.kvpos[mid] <= mypos) lo = mid + 1; else hi = mid;
        }
        vis = lo;
    }

    f32x16 acc[kD / 32];
#pragma unroll
    for (int db = 0; db < kD / 32; ++db) acc[db] = f32x16{};

    uint32_t off_r[kD / 16];
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) off_r[ks] = BG::row_off(lane, ks);
    TrOff off_t[kD / 32];
#pragma unroll
    for (int db = 0; db < kD / 32; ++db) off_t[db] = BG::tr_off(lane, db);

    LDS_AS char* st0 = (LDS_AS char*)lds_stage0;
    LDS_AS char* st1 = (LDS_AS char*)lds_stage1;

    auto tile = [&](int jt, const LDS_AS char* kt, LDS_AS char* nxt) {
        const LDS_AS char* vt = kt + kTileBytes;
        if (jt + 1 < n_ne) issue_tile(jt + 1, nxt);

        // The wave's 32-key blocks of the tile one after the other (key block kb = khalf * NKB
        // + kk): S^T = K Q^T and dP^T - D = V dO^T - D (the products accumulate onto -D), ds,
        // then dQ^T += K^T dS^T.  One block at a time leaves the registers for the -D operand
        // (the subtraction per weight goes) and splits the vector work into shorter runs.
#pragma unroll
        for (int kk = 0; kk < NKB; ++kk) {
            const int kb = khalf * NKB + kk;
            f32x16 s = f32x16{}, dp = ndlt;
#pragma unroll
            for (int ks = 0; ks < kD / 16; ++ks) {
                const bf16x8 ka = lds_b128(kt + kb * 32 * kRowBytes + off_r[ks]);
                const bf16x8 va = lds_b128(vt + kb * 32 * kRowBytes + off_r[ks]);
                s = mfma(ka, qreg[ks], s);
                dp = mfma(va, doreg[ks], dp);
            }
            sched_reads_ahead<8, 2, 2, 1>();

            // ds = p (dp - D); entry v is key 32*kb + 8*(v/4) + 4*half + v%4 of the tile
            bf16x8 dsb[2];
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float pv = __builtin_amdgcn_exp2f(fmaf(s[v], p.c, -lse2));
                dsb[v >> 3][v & 7] = (__bf16)(pv * dp[v]);
            }
            // A partly visible tile (a uniform branch, taken by few tiles): the row sees keys
            // below lim of the tile, so each packed pair keeps lim - (its first key) elements
            // from its low half.  Masking here rather than per weight keeps the compares and
            // selects out of the other tiles.
            if (jt >= n_full) {
                // an empty volatile statement: the branch cannot be turned into selects
                // executed on every tile
                asm volatile("");
                const int64_t rel = vis - (int64_t)jt * kTile - 4 * half;
                const int lim = rel < 0 ? 0 : (rel > kTile ? kTile : (int)rel);
#pragma unroll
                for (int h8 = 0; h8 < 2; ++h8) {
                    // element 2m of dsb[h8] is entry v = 8*h8 + 2m
                    const int kfirst = 32 * kb + 16 * h8;
                    const u32x4 m = {keep_low(lim - kfirst), keep_low(lim - kfirst - 2),
                                     keep_low(lim - kfirst - 8), keep_low(lim - kfirst - 10)};
                    dsb[h8] = and_mask(dsb[h8], m);
                }
            }

            // dQ^T += K^T dS^T
#pragma unroll
            for (int db = 0; db < kD / 32; ++db)
#pragma unroll
                for (int ks2 = 0; ks2 < 2; ++ks2) {
                    const LDS_AS char* base = kt + (32 * kb + 16 * ks2) * kRowBytes;
                    const bf16x8 a = lds_tr_pair(base + off_t[db].a, base + off_t[db].b);
                    acc[db] = mfma(a, dsb[ks2], acc[db]);
                }
            sched_reads_ahead<8, 1, 2, 2>();
        }

        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the next tile has landed
        __syncthreads();
    };

    if (n_ne > 0) issue_tile(0, st0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    for (int jt = 0; jt < n_ne; jt += 2) {
        tile(jt, st0, st1);
        if (jt + 1 < n_ne) tile(jt + 1, st1, st0);
    }

    if constexpr (KS > 1) {
        // the key halves' partial sums meet in the first-half waves (each stage holds two
        // waves' partials, D/2 KB each; the stages are free after the loop)
        LDS_AS float* xch = (LDS_AS float*)((qg >> 1) ? lds_stage1 : lds_stage0) + (qg & 1) * ((kD / 32) * 16 * 64);
        if (khalf == 1) {
#pragma unroll
            for (int db = 0; db < kD / 32; ++db)
#pragma unroll
                for (int v = 0; v < 16; ++v) xch[(db * 16 + v) * 64 + lane] = acc[db][v];
        }
        __syncthreads();
        if (khalf != 0) return;
#pragma unroll
        for (int db = 0; db < kD / 32; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[db][v] += xch[(db * 16 + v) * 64 + lane];
    }
    // dq += scale * dQ; accumulator entry v of block db is dimension 32*db + 8*(v/4) + 4*half + v%4
    if (!valid) return;
    float* drow = p.dq + qrow * kD;
#pragma unroll
    for (int db = 0; db < kD / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            float4* dst = (float4*)(drow + 32 * db + 8 * g + 4 * half);
            float4 x = p.write_dq ? make_float4(0.f, 0.f, 0.f, 0.f) : *dst;
            x.x += p.scale * acc[db][4 * g + 0];
            x.y += p.scale * acc[db][4 * g + 1];
            x.z += p.scale * acc[db][4 * g + 2];
            x.w += p.scale * acc[db][4 * g + 3];
            *dst = x;
        }
}

// ------------------------------------------------------------------------------------------
// dk/dv kernel
// ------------------------------------------------------------------------------------------
constexpr int kNWkv = 8;                       // dk/dv waves: 4 key groups x 2 query halves
constexpr int kThreadsKv = 64 * kNWkv;
constexpr int kRowsPerWaveKv = kTile / kNWkv;  // tile rows each wave loads

template <int D>
__global__ void __launch_bounds__(kThreadsKv, 1) block_bwd_dkdv_kernel(const BwdParams p) {
    using BG = BwdGeom<D>;
    constexpr int kD = D;
    constexpr int kRowBytes = BG::kRowBytes;
    constexpr int kTileBytes = BG::kTileBytes;
    constexpr int kRPL = BG::kRowsPerLoad;
    constexpr int kStageBytes = 2 * kTileBytes + 2 * kTile * 4;  // [Q | dO | lse2 | D]
    static_assert(kRowsPerWaveKv % kRPL == 0, "whole loads per wave");
    constexpr int kLoadsKv = kRowsPerWaveKv / kRPL;
    __shared__ __attribute__((aligned(256))) char lds_stage0[kStageBytes];
    __shared__ __attribute__((aligned(256))) char lds_stage1[kStageBytes];
    __shared__ int red[2 * kNWkv];
    // the block's V rows, key group g at rows 32*(g+1): the 32 rows of slack in front keep the
    // read base below (shifted back by the wave's query-half offset) inside the array
    __shared__ __attribute__((aligned(16))) char lds_v[5 * 32 * kRowBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in a scalar register
    const int kg = w & 3;   // key group: keys 32*kg .. +31 of the block
    const int qhalf = w >> 2;  // the 32-row half of each query tile this wave takes
    const int half = lane >> 5;
    const int l32 = lane & 31;

    int col;
    int64_t kb_rank;
    if (p.per_q > 0) {
        int q;
        int64_t it;
        if (!claim_item(p, q, it)) return;
        if (p.n_queues > 1) {
            kb_rank = it / p.kv_xcd_cols;
            col = q + 8 * (int)(it % p.kv_xcd_cols);
        } else {
            col = (int)(it % p.kv_cols);
            kb_rank = it / p.kv_cols;
        }
    } else if (p.kv_xcd_cols > 0) {
        const int x = blockIdx.x & 7;
        const int64_t kk = blockIdx.x >> 3;
        kb_rank = kk / p.kv_xcd_cols;
        col = x + 8 * (int)(kk % p.kv_xcd_cols);
    } else {
        col = (int)(blockIdx.x % p.kv_cols);
        kb_rank = blockIdx.x / p.kv_cols;
    }
    // the blocks one after another, each with its early keys (most queries) first (the grid
    // stays below 2^31)
    const int o = (int)((uint32_t)kb_rank / (uint32_t)p.max_n_kb);
    const int64_t kblk = (int64_t)((uint32_t)kb_rank % (uint32_t)p.max_n_kb);
    const BwdKV& blk = p.kv[o];
    if (kblk >= blk.n_kb) return;  // a shorter block: nothing here (the whole workgroup)
    const __bf16* const kbuf = blk.k;
    const __bf16* const vbuf = blk.v;
    const int64_t* const kvpos = blk.kvpos;
    const int64_t seq_kv = blk.seq_kv;
    const int kvh = col % p.heads_kv;
    const int64_t b = col / p.heads_kv;

    const int64_t k0 = kblk * (32 * kNW);
    const int64_t k_last = (k0 + 32 * kNW < seq_kv ? k0 + 32 * kNW : seq_kv) - 1;
    const int64_t kmin = kvpos[k0];
    const int64_t kmax = kvpos[k_last];

    // query tiles that see some key of the block (a suffix, from qt_lo) and tiles whose every
    // query sees every key of the block (a shorter suffix, from qt_full)
    const int64_t n_qt = (p.seq_q + kTile - 1) / kTile;
    int c_hidden = 0, c_part = 0;
    for (int64_t t = tid; t < n_qt; t += kThreadsKv) {
        const int64_t lq = (t * kTile + kTile - 1 < p.seq_q) ? t * kTile + kTile - 1 : p.seq_q - 1;
        c_hidden += (p.qpos[lq] < kmin) ? 1 : 0;
        c_part += (p.qpos[t * kTile] < kmax) ? 1 : 0;
    }
    c_hidden = wave_sum(c_hidden);
    c_part = wave_sum(c_part);
    if (lane == 0) {
        red[w] = c_hidden;
        red[kNWkv + w] = c_part;
    }
    __syncthreads();
    int qt_lo = 0, qt_full = 0;
#pragma unroll
    for (int ii = 0; ii < kNWkv; ++ii) {
        qt_lo += red[ii];
        qt_full += red[kNWkv + ii];
    }
    qt_lo = __builtin_amdgcn_readfirstlane(qt_lo);  // the same in every lane: scalar registers
    qt_full = __builtin_amdgcn_readfirstlane(qt_full);
    const int nq_vis = (int)n_qt - qt_lo;
    const int n_steps = nq_vis > 0 ? nq_vis * p.ratio : 0;  // (query head, query tile) pairs
    const int64_t h0 = (int64_t)kvh * p.ratio;

    // this lane's key row: k and v as B operands
    const int64_t key = k0 + kg * 32 + l32;
    const bool kvalid = key < seq_kv;
    const int64_t krow = (b * seq_kv + (kvalid ? key : 0)) * p.heads_kv + kvh;
    bf16x8 kreg[kD / 16];
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) kreg[ks] = load_row16(kbuf + krow * kD + 16 * ks + 8 * half, kvalid);
    // V rows go to LDS once (the first-half waves write their key group's rows) and are read
    // as the dP operand with the same swizzled row offsets as the Q and dO tiles
    LDS_AS char* vl = (LDS_AS char*)lds_v + (kg + 1) * 32 * kRowBytes;
    if (qhalf == 0) {
#pragma unroll
        for (int ks = 0; ks < kD / 16; ++ks)
            *(LDS_AS bf16x8*)(vl + BG::row_off(lane, ks)) = load_row16(vbuf + krow * kD + 16 * ks + 8 * half, kvalid);
    }
    // first query row that sees this key (rows before it are masked), when some tile is partial
    int64_t first = 0;
    if (qt_lo < qt_full) {
        const int64_t kp = kvalid ? kvpos[key] : INT64_MAX;
        int64_t lo = (int64_t)qt_lo * kTile;
        int64_t hi = (int64_t)qt_full * kTile < p.seq_q ? (int64_t)qt_full * kTile : p.seq_q;
        while (lo < hi) {
            const int64_t mid = (lo + hi) >> 1;
            if (p.qpos[mid] < kp) lo = mid + 1; else hi = mid;
        }
        first = kvalid ? lo : INT64_MAX;
    }

    // Q/dO tile loads: step u is query head h0 + u / nq_vis, query tile qt_lo + u % nq_vis
    const int64_t qstride = (int64_t)p.heads_q * kD;
    const int64_t qtile_bytes_g = (int64_t)kTile * qstride * 2;
    const int ld_row_in = lane / BG::kChunks;
    const int ld_chunk = lane % BG::kChunks;
    uint32_t qoff[kLoadsKv];
#pragma unroll
    for (int ii = 0; ii < kLoadsKv; ++ii) {
        const int row = w * kRowsPerWaveKv + kRPL * ii + ld_row_in;
        qoff[ii] = (uint32_t)(row * qstride * 2) + ((ld_chunk ^ BG::swz(row)) << 4);
    }
    auto step_of = [&](int u, int64_t& h, int64_t& qt) {
        h = h0 + u / nq_vis;
        qt = qt_lo + u % nq_vis;
    };
    auto issue_tile = [&](int u, LDS_AS char* st) {
        int64_t h, qt;
        step_of(u, h, qt);
        const char* qb_t = (const char*)(p.q + (b * p.seq_q * p.heads_q + h) * (int64_t)kD) + qt * qtile_bytes_g;
        const char* gb_t = (const char*)(p.dout + (b * p.seq_q * p.heads_q + h) * (int64_t)kD) + qt * qtile_bytes_g;
        const int64_t rmax = p.seq_q - 1 - qt * kTile;
        const uint32_t span = (uint32_t)((rmax < kTile - 1 ? rmax : kTile - 1) * qstride * 2 + kRowBytes);
        const __amdgpu_buffer_rsrc_t qr = make_rsrc(qb_t, span);
        const __amdgpu_buffer_rsrc_t gr = make_rsrc(gb_t, span);
#pragma unroll
        for (int ii = 0; ii < kLoadsKv; ++ii) {
            const int row = w * kRowsPerWaveKv + kRPL * ii + ld_row_in;
            // rows past the end re-read the last query; their lse is +inf, so p = 0
            const uint32_t back = (row > rmax) ? (uint32_t)((row - rmax) * qstride * 2) : 0u;
            load_lds16(qr, qoff[ii] - back, st + (w * kRowsPerWaveKv + kRPL * ii) * kRowBytes);
            load_lds16(gr, qoff[ii] - back, st + kTileBytes + (w * kRowsPerWaveKv + kRPL * ii) * kRowBytes);
        }
    };
    // lse (log2 domain, +inf past the end or for rows with no visible key) and -D of a step,
    // one value per thread of the first two waves, fetched a step ahead through registers.
    // The raw value is converted only when it is stored at the end of the step, so that the
    // wave does not wait for the load (and the tile loads issued before it) at the start.
    auto fetch_rowvals = [&](int u) -> float {
        int64_t h, qt;
        step_of(u, h, qt);
        // wave 0 fetches lse, wave 1 D (kTile = 64 rows: one per lane); wave-uniform choices,
        // so the base pointers stay scalar
        const int64_t row = qt * kTile + lane;
        if (w >= 2) return 0.f;
        const int64_t li = (b * p.heads_q + h) * p.seq_q + row;
        if (w == 0) return (row < p.seq_q) ? p.lse[li] : INFINITY;
        return (row < p.seq_q) ? p.delta[li] : 0.f;
    };
    auto store_rowvals = [&](LDS_AS char* st, float x) {
        x = (w == 0) ? ((x == -INFINITY) ? INFINITY : x * kLog2e) : -x;
        if (w < 2) ((LDS_AS float*)(st + 2 * kTileBytes))[tid] = x;
    };

    f32x16 dk[kD / 32], dv[kD / 32];
#pragma unroll
    for (int db = 0; db < kD / 32; ++db) {
        dk[db] = f32x16{};
        dv[db] = f32x16{};
    }
    // Operand offsets include the wave's query half (rows 32*qhalf of each staged tile), so the
    // Q and dO reads address a stage, whose base is a constant, with no add in the loop; the V
    // rows are read from a base shifted back by the same amount.
    const uint32_t qbase = (uint32_t)(qhalf * 32 * kRowBytes);
    uint32_t off_r[kD / 16];
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) off_r[ks] = BG::row_off(lane, ks) + qbase;
    TrOff off_t[kD / 32];
#pragma unroll
    for (int db = 0; db < kD / 32; ++db) {
        off_t[db] = BG::tr_off(lane, db);
        off_t[db].a += qbase;
        off_t[db].b += qbase;
    }
    const LDS_AS char* vq = (const LDS_AS char*)lds_v + (kg + 1 - qhalf) * 32 * kRowBytes;

    LDS_AS char* st0 = (LDS_AS char*)lds_stage0;
    LDS_AS char* st1 = (LDS_AS char*)lds_stage1;

    auto step = [&](int u, const LDS_AS char* st, LDS_AS char* nxt) {
        const LDS_AS char* qt_l = st;
        const LDS_AS char* gt_l = st + kTileBytes;
        const LDS_AS float* lse_l = (const LDS_AS float*)(st + 2 * kTileBytes);
        const LDS_AS float* dlt_l = lse_l + kTile;
        float nextv = 0.f;
        if (u + 1 < n_steps) {
            issue_tile(u + 1, nxt);
            nextv = fetch_rowvals(u + 1);
        }
        int64_t h, qt;
        step_of(u, h, qt);
        const bool masked = qt < qt_full;
        {
            const int qb = qhalf;
            // S = Q K^T and dP - D = dO V^T - D for 32 queries x this wave's 32 keys: the dP
            // products accumulate onto -D of each accumulator row (entry v is query row
            // qb*32 + 8*(v/4) + 4*half + v%4 of the tile, key l32), so no subtraction follows
            f32x16 s = f32x16{}, dp;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 nd = *(const LDS_AS f32x4*)(dlt_l + qb * 32 + 8 * g + 4 * half);
#pragma unroll
                for (int e = 0; e < 4; ++e) dp[4 * g + e] = nd[e];
            }
            f32x4 lv[4];
#pragma unroll
            for (int ks = 0; ks < kD / 16; ++ks) {
                const bf16x8 qa = lds_b128(qt_l + off_r[ks]);
                const bf16x8 ga = lds_b128(gt_l + off_r[ks]);
                const bf16x8 va = lds_b128(vq + off_r[ks]);
                s = mfma(qa, kreg[ks], s);
                dp = mfma(ga, va, dp);
                if (ks == kD / 16 - 1) {
#pragma unroll
                    for (int g = 0; g < 4; ++g) lv[g] = *(const LDS_AS f32x4*)(lse_l + qb * 32 + 8 * g + 4 * half);
                }
            }
            // the row values go out with the last operand reads, ahead of the final products
            sched_reads_ahead<8, 2, 3, 3, 2, 4, 4>();
            bf16x8 pb[2], dsb[2];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int v = 4 * g + e;
                    const float pv = __builtin_amdgcn_exp2f(fmaf(s[v], p.c, -lv[g][e]));
                    pb[v >> 3][v & 7] = (__bf16)pv;
                    dsb[v >> 3][v & 7] = (__bf16)(pv * dp[v]);
                }
            }
            // A partly visible tile (a uniform branch, taken by few steps): rows below lim of
            // this half do not see the key, so each packed pair keeps (its first row) + 2 - lim
            // elements from its high half.  Masking here rather than per weight keeps the
            // compares and selects out of the other steps.
            if (masked) {
                asm volatile("");  // keeps the branch a branch (see the dq kernel)
                const int64_t rel = first - qt * kTile - qb * 32 - 4 * half;
                const int lim = rel < 0 ? 0 : (rel > 32 ? 32 : (int)rel);
#pragma unroll
                for (int h8 = 0; h8 < 2; ++h8) {
                    // element 2m of pb[h8] and dsb[h8] is entry v = 8*h8 + 2m
                    const int r = 16 * h8 + 2 - lim;
                    const u32x4 m = {keep_high(r), keep_high(r + 2), keep_high(r + 8), keep_high(r + 10)};
                    pb[h8] = and_mask(pb[h8], m);
                    dsb[h8] = and_mask(dsb[h8], m);
                }
            }
            // dV^T += dO^T P and dK^T += Q^T dS
#pragma unroll
            for (int db = 0; db < kD / 32; ++db)
#pragma unroll
                for (int ks2 = 0; ks2 < 2; ++ks2) {
                    const int rb = 16 * ks2 * kRowBytes;
                    const bf16x8 ga = lds_tr_pair(gt_l + rb + off_t[db].a, gt_l + rb + off_t[db].b);
                    const bf16x8 qa = lds_tr_pair(qt_l + rb + off_t[db].a, qt_l + rb + off_t[db].b);
                    dv[db] = mfma(ga, pb[ks2], dv[db]);
                    dk[db] = mfma(qa, dsb[ks2], dk[db]);
                }
            sched_reads_ahead<8, 2, 4, 4>();
        }
        // every wave is done with this stage; the next one (tiles and row values) is in place
        if (u + 1 < n_steps) store_rowvals(nxt, nextv);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
    };

    if (n_steps > 0) {
        issue_tile(0, st0);
        store_rowvals(st0, fetch_rowvals(0));
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    for (int u = 0; u < n_steps; u += 2) {
        step(u, st0, st1);
        if (u + 1 < n_steps) step(u + 1, st1, st0);
    }

    // the two query halves' partial sums: the second-half waves hand theirs to the first-half
    // waves through LDS (one tensor at a time; each stage holds two waves' 16 KB)
    {
        LDS_AS float* xch = (LDS_AS float*)((kg >> 1) ? lds_stage1 : lds_stage0) + (kg & 1) * ((kD / 32) * 16 * 64);
        auto combine = [&](f32x16(&acc)[kD / 32]) {
            if (qhalf == 1) {
#pragma unroll
                for (int db = 0; db < kD / 32; ++db)
#pragma unroll
                    for (int v = 0; v < 16; ++v) xch[(db * 16 + v) * 64 + lane] = acc[db][v];
            }
            __syncthreads();
            if (qhalf == 0) {
#pragma unroll
                for (int db = 0; db < kD / 32; ++db)
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[db][v] += xch[(db * 16 + v) * 64 + lane];
            }
            __syncthreads();
        };
        combine(dk);
        combine(dv);
    }
    // dk += scale * dK, dv += dV; entry v of block db is dimension 32*db + 8*(v/4) + 4*half + v%4
    if (!kvalid || qhalf != 0) return;
    float* krow_k = blk.dk + krow * kD;
    float* krow_v = blk.dv + krow * kD;
#pragma unroll
    for (int db = 0; db < kD / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            float4* dst = (float4*)(krow_k + 32 * db + 8 * g + 4 * half);
            float4 x = p.write_dkv ? make_float4(0.f, 0.f, 0.f, 0.f) : *dst;
            x.x += p.scale * dk[db][4 * g + 0];
            x.y += p.scale * dk[db][4 * g + 1];
            x.z += p.scale * dk[db][4 * g + 2];
            x.w += p.scale * dk[db][4 * g + 3];
            *dst = x;
            float4* dsv = (float4*)(krow_v + 32 * db + 8 * g + 4 * half);
            float4 y = p.write_dkv ? make_float4(0.f, 0.f, 0.f, 0.f) : *dsv;
            y.x += dv[db][4 * g + 0];
            y.y += dv[db][4 * g + 1];
            y.z += dv[db][4 * g + 2];
            y.w += dv[db][4 * g + 3];
            *dsv = y;
        }
}

std::atomic<uint32_t> g_next_slot{0};

// A launch of at least `min_items` workgroups (eight rounds of the chip) takes its work from
// queues: one per XCD when the columns divide by 8 (xcd_cols > 0), else one, and a grid of a
// quarter more workgroups than items (at least 64 more per XCD), so that the XCDs that finish
// their own queue early have workgroups left to take the others' last items.  Returns the grid.
int64_t use_queues(BwdParams& p, int64_t items, int64_t xcd_cols, int64_t min_items, hipStream_t stream) {
    p.n_queues = 1;
    p.slot = 0;
    p.per_q = 0;
    if (items < min_items) return items;
    const int nq = xcd_cols > 0 ? 8 : 1;
    const int64_t per_q = items / nq;  // exact: with 8 queues, the columns are 8 * xcd_cols
    const int64_t grid = nq * per_q + 8 * (per_q / 4 + 64);
    if (grid > INT32_MAX) return items;
    p.n_queues = nq;
    p.per_q = per_q;
    p.slot = (int32_t)(g_next_slot.fetch_add(1, std::memory_order_relaxed) % kCtrSlots);
    hipLaunchKernelGGL(bwd_ctr_reset_kernel, dim3(1), dim3(16), 0, stream, p.slot);
    return grid;
}

template <int D>
hipError_t launch_dq(BwdParams p, hipStream_t stream) {
    const int64_t items = p.n_qt * p.n_cols;
    // launches of fewer than two blocks per CU split each tile's keys over two wave groups
    if (items < 512) {
        p.per_q = 0;
        hipLaunchKernelGGL((block_bwd_dq_kernel<D, 2>), dim3((unsigned)items), dim3(2 * kThreads), 0, stream, p);
    } else {
        // two 4-wave blocks per CU: eight rounds are 4096 blocks
        const int64_t grid = use_queues(p, items, p.xcd_cols, 4096, stream);
        hipLaunchKernelGGL((block_bwd_dq_kernel<D, 1>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
    }
    return hipGetLastError();
}

template <int D>
hipError_t launch_dkdv(BwdParams p, hipStream_t stream) {
    const int64_t items = p.max_n_kb * p.n_blk * p.kv_cols;
    // one 8-wave block per CU: eight rounds are 2048 blocks (at four, the 8K share's launch
    // of 1024 blocks lost 7% to the spare blocks and claims)
    const int64_t grid = use_queues(p, items, p.kv_xcd_cols, 2048, stream);
    hipLaunchKernelGGL(block_bwd_dkdv_kernel<D>, dim3((unsigned)grid), dim3(kThreadsKv), 0, stream, p);
    return hipGetLastError();
}

// The parameters of one block's call (dq and dk/dv of that block).
BwdParams block_params(const BlockBwdArgs& a) {
    BwdParams p;
    p.q = (const __bf16*)a.q;
    p.k = (const __bf16*)a.k;
    p.v = (const __bf16*)a.v;
    p.dout = (const __bf16*)a.dout;
    p.qpos = a.q_pos;
    p.kvpos = a.kv_pos;
    p.lse = a.lse;
    p.delta = a.delta;
    p.dq = a.dq;
    p.dk = a.dk;
    p.dv = a.dv;
    p.seq_q = a.seq_q;
    p.seq_kv = a.seq_kv;
    p.batch = a.batch;
    p.heads_q = a.heads_q;
    p.heads_kv = a.heads_kv;
    p.ratio = a.heads_q / a.heads_kv;
    p.c = a.scale * kLog2e;
    p.scale = a.scale;
    p.G = (p.ratio % 4 == 0) ? 4 : (p.ratio % 2 == 0) ? 2 : 1;
    p.n_hg = p.ratio / p.G;
    p.n_cols = a.batch * a.heads_kv * p.n_hg;
    p.xcd_cols = (p.n_cols % 8 == 0) ? p.n_cols / 8 : 0;
    p.pq = 32 * kNW / p.G;
    p.n_qt = (a.seq_q + p.pq - 1) / p.pq;
    p.n_kb = (a.seq_kv + 32 * kNW - 1) / (32 * kNW);
    p.kv_cols = a.batch * a.heads_kv;
    p.kv_xcd_cols = (p.kv_cols % 8 == 0) ? p.kv_cols / 8 : 0;
    p.write_dq = a.write_dq ? 1 : 0;
    p.write_dkv = a.write_dkv ? 1 : 0;
    p.n_blk = 1;
    p.max_n_kb = p.n_kb;
    p.kv[0] = BwdKV{p.k, p.v, p.kvpos, p.dk, p.dv, p.seq_kv, p.n_kb};
    p.n_queues = 1;  // set by each launch
    p.slot = 0;
    p.per_q = 0;
    return p;
}

}  // namespace

hipError_t launch_block_bwd_bf16(const BlockBwdArgs& a, hipStream_t stream) {
    const BwdParams p = block_params(a);
    hipError_t e = a.head_dim == 64 ? launch_dq<64>(p, stream) : launch_dq<128>(p, stream);
    if (e != hipSuccess) return e;
    return a.head_dim == 64 ? launch_dkdv<64>(p, stream) : launch_dkdv<128>(p, stream);
}

hipError_t launch_ring_bwd_bf16(const BlockBwdArgs& a, int32_t n_blk, const RingBwdBlock* blocks,
                                hipStream_t stream) {
    // dq: the blocks one launch after another, the first that has keys writing, the others
    // adding (as the per-step calls do); blocks without keys add nothing
    bool first = true;
    for (int32_t o = 0; o < n_blk; ++o) {
        if (blocks[o].seq_kv == 0) continue;
        BlockBwdArgs b = a;
        b.k = blocks[o].k;
        b.v = blocks[o].v;
        b.kv_pos = blocks[o].pos;
        b.seq_kv = blocks[o].seq_kv;
        b.write_dq = first;
        first = false;
        const BwdParams p = block_params(b);
        const hipError_t e = a.head_dim == 64 ? launch_dq<64>(p, stream) : launch_dq<128>(p, stream);
        if (e != hipSuccess) return e;
    }
    // dk, dv: every block's key blocks in one launch (each written)
    BwdParams p = block_params(a);
    p.write_dkv = 1;
    p.n_blk = 0;
    p.max_n_kb = 0;
    for (int32_t o = 0; o < n_blk; ++o) {
        if (blocks[o].seq_kv == 0) continue;
        const int64_t n_kb = (blocks[o].seq_kv + 32 * kNW - 1) / (32 * kNW);
        p.kv[p.n_blk++] = BwdKV{(const __bf16*)blocks[o].k, (const __bf16*)blocks[o].v, blocks[o].pos,
                                blocks[o].dk, blocks[o].dv, blocks[o].seq_kv, n_kb};
        if (n_kb > p.max_n_kb) p.max_n_kb = n_kb;
    }
    if (p.n_blk == 0) return hipSuccess;
    return a.head_dim == 64 ? launch_dkdv<64>(p, stream) : launch_dkdv<128>(p, stream);
}

}  // namespace cpattn
