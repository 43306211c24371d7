// bf16 block attention on the gfx950 matrix cores.
//
// What it computes ("On Context Parallelism", section Peer-to-peer / Forward: the attention
// call of one ring step on global positions, returning the normalised block output and its
// log-sum-exp; "Context Parallelism & Ring Attention", section Softmax is decomposable:
// the running max / sum / output recurrence over key blocks):
//   for each (b, query head h, local row i), over keys j of this block with
//   kv_pos[j] <= q_pos[i]:  out_i = softmax_j(scale <q_i, k_j>) v_j,  lse_i = ln sum_j e^(s_ij).
//
// Work decomposition.  A block of NW waves owns G query heads that share one K/V head
// (G = 4, 2 or 1, whichever divides heads_q/heads_kv) times PQ = 32*(NW/KS)*NB/G query
// positions (KS: the key split below, else 1).  Each wave owns NB column blocks of 32 query rows; every lane holds one query
// row of each column block.  With NW = 8 two waves share a SIMD, so one wave's matrix
// products overlap the other's softmax; with NW = 12, three.  At three waves per SIMD a wave
// has 168 registers, too few for a whole tile's scores and weights, so that variant takes
// each tile in two passes of 32 keys (KBP = 1 key block per pass; KBP = 2 is the whole
// tile).  The first 8 waves (or all, when fewer) fill the LDS stages.
//
// Key split (KS = 2, for launches too small to fill the chip): the NW waves form KS groups of
// NW/KS waves over the same rows.  Group g takes tiles g, g+KS, ... of the block's tile
// sequence, with its own LDS stages, running softmax and accumulator; at the end the groups'
// states meet in group 0, rescaled to the larger reference (the same exact combine as the
// merge of two blocks), before the epilogue.
//
// Per K/V tile of 64 keys (per pass of 32*KBP keys):
//   S^T = K Q^T    with v_mfma_f32_32x32x16_bf16: A = 32 keys x 16 dims of K (LDS),
//                  B = 16 dims x 32 queries of Q (registers, loaded once).  The accumulator
//                  gives each lane 16 keys of ONE query, so the row max is lane-local plus
//                  one exchange with the other half-wave.
//   softmax in the log2 domain (scores times scale*log2(e), exp2) against a running
//                  reference m that is not necessarily the row max: the result is the same
//                  for any reference.  Each tile first takes the weights against the current
//                  m.  Only when some lane's sum of them exceeds 2^kLazy (or m is still unset)
//                  does the wave compute the row max, raise m to it, rescale the accumulator
//                  and recompute; so weights stay <= 2^kLazy and most tiles need no max.
//   P rounded to bf16 (RNE) straight from the weights; the row sum adds the fp32 weights
//                  (rounding them first would cost lse up to 2^-9 on short rows).
//   O^T += V^T P^T with A = 32 dims x 16 keys of V read transposed from the row-major LDS
//                  tile by ds_read_b64_tr_b16, B = P^T (registers).  The key order inside a
//                  16-key step is the accumulator's own order, applied to V's addresses.
// K and V tiles go from global memory straight into LDS (buffer_load_dwordx4 ... lds; each
// lane lands 16 bytes at base + 16*lane, so the XOR-swizzled layout is chosen by which chunk
// each lane fetches).  Two LDS stages: the next tile is in flight while the current one is
// used (issued at the start of the tile, or between the passes in the two-pass variant).  Buffer loads rather than global_load_lds: the compiler treats a pending global LDS
// load as a flat access and then waits for every outstanding LDS read (lgkmcnt(0)) before
// each product, instead of only for the read the product needs.
//
// Causal skip ("Context parallelism: Ring Attention and Ulysses", Ring Attention: blocks
// later than the query are skipped whole): with strictly increasing positions the visible
// tiles of a block are a prefix, and the tiles entirely visible to every query of the block
// are a shorter prefix; only the tiles in between are masked element by element, against
// each row's count of visible keys (found once by binary search over the key positions).
// Rows with no visible key end with out = 0 and lse = -inf.
//
// Block order: heaviest query tiles first, a K/V head's columns on one XCD.  Launches of at
// least four rounds of blocks take their tiles from queues at run time (an atomic add per
// block; one queue per XCD, taking the others' last tiles once its own run out), since the
// XCDs hold different clocks under load and equal shares would end at different times.
#include "cpattn_internal.h"
#include "merge_math.h"

#include <atomic>
#include <math.h>

namespace cpattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int kBN = 64;             // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.0f;       // raise the running max only past this margin (log2)
constexpr float kLazyWeight = 256.0f;  // 2^kLazy
constexpr int kMaxBlocks = kMaxRingBlocks;  // K/V blocks of one launch
constexpr int64_t kQueueMinBlocks = 1024;    // launches with at least 4 rounds of blocks use the queues
constexpr int kVisKeys = 256;               // key positions a wave searches in LDS

// One K/V block: keys [B][seq][heads_kv][D] and their positions.
struct KVBlock {
    const __bf16* k;
    const __bf16* v;
    const int64_t* pos;
    int64_t seq;
};

struct Params {
    const __bf16* q;
    const int64_t* qpos;
    float* out;
    float* lse;
    int64_t seq_q;
    int64_t n_qt;      // query tiles of PQ positions
    int32_t heads_q;
    int32_t heads_kv;
    int32_t ratio;     // heads_q / heads_kv
    int32_t G;         // query heads per block
    int32_t pq;        // query positions per block
    int32_t n_hg;      // ratio / G head groups per kv head
    int32_t n_cols;    // batch * heads_kv * n_hg
    int32_t xcd_cols;  // n_cols / 8 when n_cols % 8 == 0, else 0
    float c;           // scale * log2(e)
    int32_t merge;     // merge into (out, lse) instead of overwriting them
    int32_t n_blk;     // K/V blocks attended in turn, as one softmax over all their keys
    int64_t q_rs;      // elements between consecutive rows of q, K/V and out (heads within a
    int64_t kv_rs;     // row are contiguous: dense rows have heads * D)
    int64_t out_rs;
    KVBlock blk[kMaxBlocks];
    // work taken from queues at run time (per_q > 0) instead of by block index: n_queues
    // queues (8: one per XCD, holding its columns' tiles; 1: all tiles) of per_q tiles each,
    // counted in counter slot `slot`
    int32_t n_queues;
    int32_t slot;
    int64_t per_q;
};

// Work counters of the launches that take their tiles from queues: a slot per call, taken in
// turn (so calls in flight on different streams use different slots), 16 counters per slot
// (one per queue), set to zero by a one-workgroup kernel on the call's stream before the
// attention launch.  Device code reaches the array by name; host code never uses it.
constexpr int kCtrSlots = 256;
__device__ int g_fwd_ctr[kCtrSlots * 16];

__global__ void fwd_ctr_reset_kernel(int slot) { g_fwd_ctr[slot * 16 + threadIdx.x] = 0; }

__device__ inline int wave_sum(int x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

// Combine a value with the other half-wave's (lane ^ 32): both outputs of the half-swap
// hold {ours, theirs}.
__device__ inline float half_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float half_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline bf16x8 lds_b128(const LDS_AS char* p) { return *(const LDS_AS bf16x8*)p; }

__device__ inline bf16x8 lds_tr_pair(const LDS_AS char* p0, const LDS_AS char* p1) {
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)p0);
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)p1);
    const s16x8 c = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_bit_cast(bf16x8, c);
}

// Head-dim dependent layout of a K/V tile in LDS: one row of D bf16 is D/8 chunks of 16 bytes,
// and chunk c of row r is stored at chunk c ^ swz(r).
//   K (row reads: 16 lanes read one chunk of 16 consecutive keys, which must fall in 16
//   distinct 16-byte bank groups of the 256-byte bank row):
//     D = 128 (one row per bank row): r & 15
//     D = 64 (two rows per bank row): (r >> 1) & 7
//   V (transposed reads: each 32-lane half reads 4 consecutive keys x 4 chunks, which must
//   cover all 64 banks):
//     D = 128: (r & 3) << 2
//     D = 64: ((r >> 1) & 1) << 2
// Both are unchanged by adding a multiple of 8 rows, which the operand reads rely on.
template <int D> struct TileGeom {
    static_assert(D == 64 || D == 128, "head dim 64 or 128");
    static constexpr int kRowBytes = D * 2;
    static constexpr int kTileBytes = kBN * kRowBytes;
    static constexpr int kChunks = D / 8;             // 16-byte chunks per row
    static constexpr int kRowsPerLoad = 64 / kChunks; // rows one 64-lane 16-byte load fills
    __device__ static inline int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
    __device__ static inline int swz_v(int r) { return D == 128 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2); }
};

// Buffer descriptor over `bytes` bytes from `base` (raw, no stride; word 3 as gfx9 wants).
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// One 16-byte direct load into LDS through a buffer descriptor: this lane's 16 bytes come from
// base + voff and land at lds_base + 16*lane.  (A buffer load, unlike a global one, is not a
// flat access, so LDS reads issued while it is in flight keep exact lgkm counts.)
__device__ inline void load_lds16(__amdgpu_buffer_rsrc_t r, uint32_t voff, LDS_AS void* lds_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_base, 16, voff, 0, 0, 0);
}

// LDS operand reads kept in flight ahead of the matrix products (K: one read per MFMA,
// V: two transposed reads per MFMA).  The two-pass variant (168 registers) keeps K two ahead:
// same speed on the ring share, +1.5% on Ulysses, and no registers spilled.
constexpr int kReadAheadK = 4;
constexpr int kReadAheadV = 2;
constexpr int kReadAheadK2 = 2;

template <int D, int NW, int NB, int KBP, int KS>
__global__ void __launch_bounds__(64 * NW, 1) block_fwd_bf16_kernel(const Params p) {
    static_assert(KS == 1 || NB == 1, "the key split combines one column block per wave");
    using TG = TileGeom<D>;
    constexpr int kD = D;
    constexpr int kRowBytes = TG::kRowBytes;
    constexpr int kTileBytes = TG::kTileBytes;
    constexpr int kRAK = KBP == 1 ? kReadAheadK2 : kReadAheadK;
    constexpr int kThreads = 64 * NW;
    constexpr int NWR = NW / KS;  // waves per row group (all waves unless the keys are split)
    // K/V tile row r, 16-byte chunk c is stored at chunk c ^ swz(r) (TileGeom);
    // two stages in two distinct arrays, so that the compiler can tell the stage being read
    // from the stage being filled and does not wait for the fill before reading
    // (with the keys split over KS wave groups, each group has its own pair of stages)
    __shared__ __attribute__((aligned(16))) char lds_stage0[KS * 2 * kTileBytes];  // [group][K|V][tile]
    __shared__ __attribute__((aligned(16))) char lds_stage1[KS * 2 * kTileBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = KS > 1 ? __builtin_amdgcn_readfirstlane(tid >> 6) : (tid >> 6);
    const int wr = KS > 1 ? w % NWR : w;  // wave within its row group
    const int ksg = KS > 1 ? w / NWR : 0;  // key group: takes tiles ksg, ksg + KS, ... of the sequence
    const int half = lane >> 5;
    const int l32 = lane & 31;

    // ---- which (b, kv head, head group, query tile) this block owns; heavy tiles first
    int col;
    int64_t qt_rank;
    if (p.per_q > 0) {
        // From the queues: the hardware deals consecutive blocks to the 8 XCDs in turn, and
        // the XCDs run at different clocks under load, so equal shares of blocks end at
        // different times.  A block takes the next tile of its XCD's queue (its columns, heavy
        // tiles first), or, once that is empty, of the next queue that is not; a block that
        // finds every queue empty has nothing to do.  Each tile is computed by exactly one
        // block, with the same code wherever it runs.
        __shared__ int claim[2];
        if (threadIdx.x == 0) {
            const int home = p.n_queues > 1 ? (int)(blockIdx.x & 7) : 0;
            int q = -1, it = 0;
            for (int y = 0; y < p.n_queues; ++y) {
                const int qq = (home + y) % p.n_queues;
                const int i = atomicAdd(&g_fwd_ctr[p.slot * 16 + qq], 1);
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
        const int q = claim[0];
        if (q < 0) return;  // the whole block
        const int64_t it = claim[1];
        if (p.n_queues > 1) {
            qt_rank = it / p.xcd_cols;
            col = q + 8 * (int)(it % p.xcd_cols);
        } else {
            col = (int)(it % p.n_cols);
            qt_rank = it / p.n_cols;
        }
    } else if (p.xcd_cols > 0) {
        // consecutive blocks are dealt round-robin to the 8 XCDs: keep one XCD on the same
        // columns (same K/V head) so its L2 serves all of them
        const int x = blockIdx.x & 7;
        const int64_t kk = blockIdx.x >> 3;
        qt_rank = kk / p.xcd_cols;
        col = x + 8 * (int)(kk % p.xcd_cols);
    } else {
        col = (int)(blockIdx.x % p.n_cols);
        qt_rank = blockIdx.x / p.n_cols;
    }
    const int64_t qt = p.n_qt - 1 - qt_rank;
    const int hg = col % p.n_hg;
    const int kvh = (col / p.n_hg) % p.heads_kv;
    const int64_t b = col / (p.n_hg * p.heads_kv);

    const int64_t q0 = qt * p.pq;
    const int64_t q_last = (q0 + p.pq < p.seq_q ? q0 + p.pq : p.seq_q) - 1;
    const int64_t pmin = p.qpos[q0];
    const int64_t pmax = p.qpos[q_last];

    // ---- per K/V block: visible tiles (a prefix) and tiles visible to every query of this
    // workgroup, wave w counting blocks w, w + NW, ... in one pass (four tiles per lane in
    // flight); then the tile sequence runs over the blocks in turn
    __shared__ int blk_ne[kMaxBlocks], blk_full[kMaxBlocks];
    __shared__ int64_t vis_keys[NW][kVisKeys];  // each wave's copy of a block's diagonal positions
    for (int o = w; o < p.n_blk; o += NW) {
        const int64_t* kp = p.blk[o].pos;
        const int64_t seq_o = p.blk[o].seq;
        const int64_t n_tiles = (seq_o + kBN - 1) / kBN;
        int c_ne = 0, c_full = 0;
        for (int64_t t0 = lane; t0 < n_tiles; t0 += 4 * 64) {
            int64_t first[4], last[4];
            bool has_f[4], has_l[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t t = t0 + 64 * u;
                const int64_t lk = t * kBN + kBN - 1;
                has_f[u] = t < n_tiles;
                has_l[u] = has_f[u] && lk < seq_o;
                first[u] = has_f[u] ? kp[t * kBN] : 0;
                last[u] = has_l[u] ? kp[lk] : 0;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                c_ne += (has_f[u] && first[u] <= pmax) ? 1 : 0;
                c_full += (has_l[u] && last[u] <= pmin) ? 1 : 0;
            }
        }
        c_ne = wave_sum(c_ne);
        c_full = wave_sum(c_full);
        if (lane == 0) {
            blk_ne[o] = c_ne;
            blk_full[o] = c_full;
        }
    }
    __syncthreads();
    int n_total = 0;  // tiles over all blocks
    for (int o = 0; o < p.n_blk; ++o) n_total += blk_ne[o];

    // ---- K/V tile loads: each wave fills (64 / NW) rows of K and of V per tile, 1 KB (four
    // rows of D = 128, eight of D = 64) per instruction; lane -> row (lane / chunks per row),
    // stored chunk (lane % chunks per row).  The source
    // address is a wave-uniform tile base plus a per-lane byte offset fixed for the kernel;
    // only a ragged last tile clamps its rows (to the last key, finite data the mask hides).
    const int64_t kvstride = p.kv_rs;  // elements between consecutive keys
    const int64_t tile_bytes_g = (int64_t)kBN * kvstride * 2;  // global bytes between tiles
    auto kbase_of = [&](int o) {
        return (const char*)(p.blk[o].k + b * p.blk[o].seq * p.kv_rs + kvh * (int64_t)kD);
    };
    auto vbase_of = [&](int o) {
        return (const char*)(p.blk[o].v + b * p.blk[o].seq * p.kv_rs + kvh * (int64_t)kD);
    };
    constexpr int kLW = NWR < 8 ? NWR : 8;  // waves of a row group that load (all, or the first 8)
    constexpr int kRowsPerWave = kBN / kLW;
    constexpr int kRPL = TG::kRowsPerLoad;
    static_assert(kRowsPerWave % kRPL == 0, "whole loads per wave");
    constexpr int kLoadsPerWave = kRowsPerWave / kRPL;
    const int ld_row_in = lane / TG::kChunks;   // row within the slab of one load
    const int ld_chunk = lane % TG::kChunks;    // stored chunk
    uint32_t koff[kLoadsPerWave], voff[kLoadsPerWave];
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i) {
        const int row = wr * kRowsPerWave + kRPL * i + ld_row_in;
        koff[i] = (uint32_t)(row * kvstride * 2) + ((ld_chunk ^ TG::swz_k(row)) << 4);
        voff[i] = (uint32_t)(row * kvstride * 2) + ((ld_chunk ^ TG::swz_v(row)) << 4);
    }
    // cursors: the tile being computed (block oc, tile jt of its ne_c visible tiles; n_full
    // of oc) and the next one to load (block on, tile jn of ne_n, the tile's K and V
    // addresses and the block's length; on == p.n_blk when there is none).  All are uniform
    // and live in scalar registers: a step within a block only counts and adds, and the
    // per-block counts (LDS) and addresses (kernel arguments) are read when a cursor enters
    // a new block, so no memory round trip sits between a barrier and the next tile.
    int oc = 0, jt = 0, ne_c = 0, n_full = 0;
    int on = p.n_blk, jn = 0, ne_n = 0;  // no load until set_load (a key group may have no tile)
    const char* kb_n = nullptr;
    const char* vb_n = nullptr;
    int64_t seq_n = 0;
    auto ne_of = [&](int o) { return o < p.n_blk ? __builtin_amdgcn_readfirstlane(blk_ne[o]) : 0; };
    auto next_block = [&](int o) {
        do { ++o; } while (o < p.n_blk && blk_ne[o] == 0);
        return o;
    };
    auto set_load = [&](int o, int j) {
        on = o;
        jn = j;
        ne_n = ne_of(o);
        if (o < p.n_blk) {
            kb_n = kbase_of(o) + (int64_t)j * tile_bytes_g;
            vb_n = vbase_of(o) + (int64_t)j * tile_bytes_g;
            seq_n = p.blk[o].seq;
        }
    };
    auto adv_c = [&]() {
        if (++jt >= ne_c) {
            jt = 0;
            oc = next_block(oc);
            ne_c = ne_of(oc);
        }
    };
    auto adv_n = [&]() {
        kb_n += tile_bytes_g;
        vb_n += tile_bytes_g;
        if (++jn >= ne_n) set_load(next_block(on), 0);
    };
    // the load cursor's tile into the stage at kt
    auto issue_tile = [&](LDS_AS char* kt) {
        LDS_AS char* vt = kt + kTileBytes;
        const char* kb_t = kb_n;
        const char* vb_t = vb_n;
        const int64_t seq_o = seq_n;
        const int jt = jn;
        // the descriptor covers this tile's rows that exist (a tile spans < 4 GiB)
        const int64_t rows = seq_o - (int64_t)jt * kBN < kBN ? seq_o - (int64_t)jt * kBN : kBN;
        if (rows <= 0) return;  // never a tile without rows (the cursor stays within its block)
        const uint32_t span = (uint32_t)((rows - 1) * kvstride * 2 + kRowBytes);
        const __amdgpu_buffer_rsrc_t kr = make_rsrc(kb_t, span);
        const __amdgpu_buffer_rsrc_t vr = make_rsrc(vb_t, span);
        if (NWR > kLW && wr >= kLW) return;
        if ((int64_t)(jt + 1) * kBN <= seq_o) {
#pragma unroll
            for (int i = 0; i < kLoadsPerWave; ++i) {
                load_lds16(kr, koff[i], kt + (wr * kRowsPerWave + kRPL * i) * kRowBytes);
                load_lds16(vr, voff[i], vt + (wr * kRowsPerWave + kRPL * i) * kRowBytes);
            }
        } else {
#pragma unroll
            for (int i = 0; i < kLoadsPerWave; ++i) {
                const int row = wr * kRowsPerWave + kRPL * i + ld_row_in;
                const int64_t j = (int64_t)jt * kBN + row;
                const uint32_t over = (j >= seq_o) ? (uint32_t)((j - (seq_o - 1)) * kvstride * 2) : 0u;
                load_lds16(kr, koff[i] - over, kt + (wr * kRowsPerWave + kRPL * i) * kRowBytes);
                load_lds16(vr, voff[i] - over, vt + (wr * kRowsPerWave + kRPL * i) * kRowBytes);
            }
        }
    };

    // ---- this lane's query rows; Q as MFMA B operands (16 dims x 32 queries per step)
    // ---- the first tile of this (key group's) sequence goes out now, so that its latency
    // overlaps the reads of the query rows and of the diagonal positions below
    LDS_AS char* st0 = (LDS_AS char*)lds_stage0 + ksg * 2 * kTileBytes;
    LDS_AS char* st1 = (LDS_AS char*)lds_stage1 + ksg * 2 * kTileBytes;
    while (oc < p.n_blk && blk_ne[oc] == 0) ++oc;  // first block with a visible tile
    ne_c = ne_of(oc);
    // key group g starts at tile g of the sequence
    for (int s2 = 0; s2 < ksg; ++s2)
        if (oc < p.n_blk) adv_c();
    if (oc < p.n_blk) {
        set_load(oc, jt);
        issue_tile(st0);
        if (KS == 1) {
            adv_n();
        } else {
#pragma unroll
            for (int s2 = 0; s2 < KS; ++s2)
                if (on < p.n_blk) adv_n();
        }
    }

    bf16x8 qreg[NB][kD / 16];
    int64_t myq[NB];
    int64_t myh[NB];
    int64_t mypos[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int row0 = (wr * NB + nb) * 32;
        const int hs = row0 / p.pq;
        const int64_t i = q0 + (row0 % p.pq) + l32;
        const int64_t head = (int64_t)kvh * p.ratio + (int64_t)hg * p.G + hs;
        myq[nb] = i;
        myh[nb] = head;
        const bool valid = i < p.seq_q;
        mypos[nb] = valid ? p.qpos[i] : INT64_MIN;
        const __bf16* qrow = p.q + (b * p.seq_q + (valid ? i : 0)) * p.q_rs + head * kD + 8 * half;
#pragma unroll
        for (int ks = 0; ks < kD / 16; ++ks) {
            u32x4 raw = valid ? *(const u32x4*)(qrow + 16 * ks) : u32x4{0, 0, 0, 0};
            qreg[nb][ks] = __builtin_bit_cast(bf16x8, raw);
        }
    }

    // number of keys of block o visible to each of this lane's query rows, needed only when
    // some tile of o is partly visible: positions increase, so it is found by binary search
    // within the keys of the partly visible tiles [n_full*kBN, min(n_ne*kBN, seq))
    // within the keys of the partly visible tiles [n_full*kBN, min(n_ne*kBN, seq)).  At the
    // start (use_lds), when they are few (at most kVisKeys: a block's diagonal), the wave
    // copies their positions into its own slice of LDS once and searches there; otherwise,
    // and for blocks entered later (whose rows are in the zigzag shares all or nothing, so
    // no search runs), it searches global memory.
    int64_t vis[NB];
    auto find_vis = [&](int o, bool use_lds) {
        const int ne = blk_ne[o], full = blk_full[o];
        const int64_t seq_o = p.blk[o].seq;
        const int64_t* kp = p.blk[o].pos;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) vis[nb] = 0;
        if (full >= ne) return;
        const int64_t lo0 = (int64_t)full * kBN;
        const int64_t hi0 = (int64_t)ne * kBN < seq_o ? (int64_t)ne * kBN : seq_o;
        const int n = (int)(hi0 - lo0 < kVisKeys + 1 ? hi0 - lo0 : kVisKeys + 1);
        if (use_lds && n <= kVisKeys) {
            LDS_AS int64_t* vk = (LDS_AS int64_t*)&vis_keys[w][0];
            for (int i = lane; i < n; i += 64) vk[i] = kp[lo0 + i];
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's copies are in LDS
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                int lo = 0, hi = n;
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    if (vk[mid] <= mypos[nb]) lo = mid + 1; else hi = mid;
                }
                vis[nb] = lo0 + lo;
            }
            return;
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            int64_t lo = lo0, hi = hi0;
            while (lo < hi) {
                const int64_t mid = (lo + hi) >> 1;
                if (kp[mid] <= mypos[nb]) lo = mid + 1; else hi = mid;
            }
            vis[nb] = lo;
        }
    };

    f32x16 acc_o[NB][kD / 32];
    // m_run: the reference (log2 domain; -inf until the row has a visible key); nm: -m_run as
    // the fast path adds it, NaN while m_run is unset, so that the fast path's weights and
    // sum come out NaN and its one bound test also sends an unset row to the exact path
    float m_run[NB], l_run[NB], nm[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        m_run[nb] = -INFINITY;
        nm[nb] = __builtin_nanf("");
        l_run[nb] = 0.f;
#pragma unroll
        for (int db = 0; db < kD / 32; ++db) acc_o[nb][db] = f32x16{};
    }

    // ---- per-lane LDS read offsets
    // K (row reads): key = 32*kb + l32, chunk (2*ks + half) stored at chunk ^ swz_k(key)
    uint32_t off_k[kD / 16];
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks)
        off_k[ks] = l32 * kRowBytes + (((2 * ks + half) ^ TG::swz_k(l32)) << 4);
    // V (transposed reads): in each 16-lane group, lane s reads 4 dims starting at
    // 16*(group&1) + 4*(s&3) of key (s>>2) + 4*half (+8 for the second read)
    const int grp = lane >> 4, s16 = lane & 15;
    const int vkey = 4 * half + (s16 >> 2);
    const int vsw = TG::swz_v(vkey);
    uint32_t off_v[kD / 32];
#pragma unroll
    for (int db = 0; db < kD / 32; ++db) {
        const int chunk = 4 * db + 2 * (grp & 1) + ((s16 & 3) >> 1);
        off_v[db] = vkey * kRowBytes + ((chunk ^ vsw) << 4) + ((s16 & 1) << 3);
    }


    // one tile: prefetch the next tile into `nxt`, compute the current one from `cur`
    auto tile = [&](const LDS_AS char* kt, LDS_AS char* nxt) {
        const LDS_AS char* vt = kt + kTileBytes;
        // The next tile's loads go out at the start of the tile, or, in the two-pass variant,
        // between the passes: right after the barrier all twelve waves start their score
        // products at once, and issuing the loads there too slowed the kernel (between the
        // passes: +2-4%, the loads still land within the second pass).
        if (KBP != 1 && on < p.n_blk) issue_tile(nxt);

        // the tile in 2 / KBP passes of 32 * KBP keys each: scores, mask, softmax, PV (with the
        // keys split, a group whose share has run out only keeps the barriers)
#pragma unroll
        for (int ps = 0; ps < ((KS == 1 || oc < p.n_blk) ? 2 / KBP : 0); ++ps) {
            if (KBP == 1 && ps == 1 && on < p.n_blk) issue_tile(nxt);
            // S^T = K Q^T
            f32x16 s[NB][KBP];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int kk = 0; kk < KBP; ++kk) s[nb][kk] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < kD / 16; ++ks) {
#pragma unroll
                for (int kk = 0; kk < KBP; ++kk) {
                    const bf16x8 a = lds_b128(kt + (ps * KBP + kk) * 32 * kRowBytes + off_k[ks]);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        s[nb][kk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[nb][ks], s[nb][kk], 0, 0, 0);
                }
            }
            // keep the operand reads kRAK ahead of the matrix products
            __builtin_amdgcn_sched_group_barrier(0x100, kRAK, 1);
#pragma unroll
            for (int i = 0; i < (kD / 16) * KBP - kRAK; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, NB, 1);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, NB * kRAK, 1);

            // element mask on tiles not entirely visible: key index of accumulator entry v of
            // key block kb is 32*kb + 8*(v/4) + 4*half + v%4 within the tile; visible iff below
            // the row's count
            if (jt >= n_full) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const int64_t rel = vis[nb] - (int64_t)jt * kBN - 4 * half;
                    const int lim = rel < 0 ? 0 : (rel > kBN ? kBN : (int)rel);
#pragma unroll
                    for (int kk = 0; kk < KBP; ++kk)
#pragma unroll
                        for (int v = 0; v < 16; ++v)
                            if (32 * (ps * KBP + kk) + 8 * (v / 4) + v % 4 >= lim) s[nb][kk][v] = -INFINITY;
                }
            }

            // softmax in the log2 domain against the running reference m.  Fast path: weights
            // against the current m; they stay bounded (each at most 2^kLazy) whenever this
            // lane's sum of them does, so no row max is needed.  Otherwise (or while m is unset,
            // which makes the sum NaN) the wave takes the slow path: row max, raise m to it,
            // rescale O and l, recompute.  The sums start from their first term (0 + e == e:
            // every weight is >= +0).
            bf16x8 pb[NB][KBP][2];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                float ts = 0.f;
#pragma unroll
                for (int kk = 0; kk < KBP; ++kk)
#pragma unroll
                    for (int h8 = 0; h8 < 2; ++h8)
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const float e = __builtin_amdgcn_exp2f(fmaf(s[nb][kk][8 * h8 + j], p.c, nm[nb]));
                            ts = (kk == 0 && h8 == 0 && j == 0) ? e : ts + e;
                            pb[nb][kk][h8][j] = (__bf16)e;
                        }
                if (__builtin_amdgcn_ballot_w64(!(ts <= kLazyWeight)) != 0) {
                    float mx = -INFINITY;
#pragma unroll
                    for (int kk = 0; kk < KBP; ++kk)
#pragma unroll
                        for (int vv = 0; vv < 16; ++vv) mx = fmaxf(mx, s[nb][kk][vv]);
                    const float mt = half_max(mx) * p.c;
                    const float m_new = fmaxf(m_run[nb], mt);
                    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
                    const float alpha = __builtin_amdgcn_exp2f(m_run[nb] - m_use);
                    l_run[nb] *= alpha;
#pragma unroll
                    for (int db = 0; db < kD / 32; ++db) acc_o[nb][db] *= alpha;
                    m_run[nb] = m_new;
                    nm[nb] = (m_new == -INFINITY) ? __builtin_nanf("") : -m_new;
#pragma unroll
                    for (int kk = 0; kk < KBP; ++kk)
#pragma unroll
                        for (int h8 = 0; h8 < 2; ++h8)
#pragma unroll
                            for (int j = 0; j < 8; ++j) {
                                const float e = __builtin_amdgcn_exp2f(fmaf(s[nb][kk][8 * h8 + j], p.c, -m_use));
                                ts = (kk == 0 && h8 == 0 && j == 0) ? e : ts + e;
                                pb[nb][kk][h8][j] = (__bf16)e;
                            }
                }
                l_run[nb] += ts;
            }

            // O^T += V^T P^T (the four accumulators interleaved: a product never waits on the
            // one just issued).  The wave issues these at raised priority: when several waves of
            // a SIMD are ready, the arbiter takes the one with output products to issue, so the
            // matrix pipe stays fed while the others' softmax fills the gaps (+1.6% on the ring
            // share and the Ulysses group at the same or a lower clock; the same raise around
            // the score products, or around both, gained less or lost)
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int kk = 0; kk < KBP; ++kk) {
#pragma unroll
                for (int ks2 = 0; ks2 < 2; ++ks2) {
#pragma unroll
                    for (int db = 0; db < kD / 32; ++db) {
                        const LDS_AS char* base = vt + (32 * (ps * KBP + kk) + 16 * ks2) * kRowBytes + off_v[db];
                        const bf16x8 a = lds_tr_pair(base, base + 8 * kRowBytes);
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
                            acc_o[nb][db] =
                                __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[nb][kk][ks2], acc_o[nb][db], 0, 0, 0);
                    }
                }
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * kReadAheadV, 2);
#pragma unroll
            for (int i = 0; i < (kD / 16) * KBP - kReadAheadV; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, NB, 2);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 2);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, NB * kReadAheadV, 2);
            __builtin_amdgcn_s_setprio(0);
        }
        // the next tile has landed in LDS (own loads) and every wave is done with this one
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), visible to the compiler
        __syncthreads();
        const int o_prev = oc;
        if (KS == 1) {
            adv_c();
            if (on < p.n_blk) adv_n();
        } else {
#pragma unroll
            for (int s2 = 0; s2 < KS; ++s2) {
                if (oc < p.n_blk) adv_c();
                if (on < p.n_blk) adv_n();
            }
        }
        if (oc != o_prev && oc < p.n_blk) {
            n_full = __builtin_amdgcn_readfirstlane(blk_full[oc]);
            find_vis(oc, false);
        }
    };

    if (oc < p.n_blk) {
        n_full = __builtin_amdgcn_readfirstlane(blk_full[oc]);
        find_vis(oc, true);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), visible to the compiler
    __syncthreads();
    const int n_it = (n_total + KS - 1) / KS;  // tiles per key group, rounded up
    for (int u = 0; u < n_it; u += 2) {
        tile(st0, st1);
        if (u + 1 < n_it) tile(st1, st0);
    }

    if constexpr (KS > 1) {
        // the key groups' partial softmax states (accumulator, reference m, sums l) meet in
        // group 0: group 1 hands its own over through LDS (the stages are free now) and group
        // 0 rescales both to the larger reference
        LDS_AS float* xa = (LDS_AS float*)lds_stage0 + wr * (16 * (kD / 32) * 64);
        LDS_AS float* xm = (LDS_AS float*)lds_stage1 + wr * (2 * 64);
        if (ksg == 1) {
#pragma unroll
            for (int db = 0; db < kD / 32; ++db)
#pragma unroll
                for (int v = 0; v < 16; ++v) xa[(db * 16 + v) * 64 + lane] = acc_o[0][db][v];
            xm[lane] = m_run[0];
            xm[64 + lane] = l_run[0];
        }
        __syncthreads();
        if (ksg != 0) return;
        const float mb = xm[lane], lb = xm[64 + lane];
        const float m = fmaxf(m_run[0], mb);
        const float fa = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run[0] - m);
        const float fb = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mb - m);
        l_run[0] = l_run[0] * fa + lb * fb;
#pragma unroll
        for (int db = 0; db < kD / 32; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc_o[0][db][v] = acc_o[0][db][v] * fa + xa[(db * 16 + v) * 64 + lane] * fb;
        m_run[0] = m;
    }

    // ---- epilogue: combine the half-wave row sums, normalise, store (or merge into out, lse)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const float l_tot = half_sum(l_run[nb]);
        const bool any = l_tot > 0.f;
        const float inv = any ? 1.f / l_tot : 0.f;
        if (myq[nb] >= p.seq_q) continue;
        float* orow = p.out + (b * p.seq_q + myq[nb]) * p.out_rs + myh[nb] * kD;
        float* lrow = p.lse + (b * p.heads_q + myh[nb]) * p.seq_q + myq[nb];
        const float lse_t = any ? (m_run[nb] + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
        if (p.merge) {
            // both half-waves read the accumulator's lse before either writes it back
            const MergeWeights mw = merge_weights(*lrow, lse_t);
#pragma unroll
            for (int db = 0; db < kD / 32; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float4* dst = (float4*)(orow + 32 * db + 8 * g + 4 * half);
                    const float4 x = *dst;
                    float4 o4;
                    o4.x = merge_value(x.x, acc_o[nb][db][4 * g + 0] * inv, mw.w_old, mw.w_new);
                    o4.y = merge_value(x.y, acc_o[nb][db][4 * g + 1] * inv, mw.w_old, mw.w_new);
                    o4.z = merge_value(x.z, acc_o[nb][db][4 * g + 2] * inv, mw.w_old, mw.w_new);
                    o4.w = merge_value(x.w, acc_o[nb][db][4 * g + 3] * inv, mw.w_old, mw.w_new);
                    *dst = o4;
                }
            if (half == 0) *lrow = mw.lse;
            continue;
        }
#pragma unroll
        for (int db = 0; db < kD / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float4 o4;
                o4.x = acc_o[nb][db][4 * g + 0] * inv;
                o4.y = acc_o[nb][db][4 * g + 1] * inv;
                o4.z = acc_o[nb][db][4 * g + 2] * inv;
                o4.w = acc_o[nb][db][4 * g + 3] * inv;
                *(float4*)(orow + 32 * db + 8 * g + 4 * half) = o4;
            }
        if (half == 0) *lrow = lse_t;
    }
}

std::atomic<uint32_t> g_next_slot{0};

template <int D, int NW, int NB, int KBP, int KS>
hipError_t launch_variant(Params p, int64_t seq_q, hipStream_t stream) {
    p.pq = 32 * (NW / KS) * NB / p.G;
    p.n_qt = (seq_q + p.pq - 1) / p.pq;
    const int64_t blocks = p.n_qt * p.n_cols;
    int64_t grid = blocks;
    p.n_queues = 1;
    p.slot = 0;
    p.per_q = 0;
    // Launches of at least four rounds of blocks take their tiles from queues, with a quarter
    // more blocks (and at least 64 more per XCD) than tiles, so that the XCDs that finish
    // their own queue early have blocks left to take the others' last tiles with.
    if (blocks >= kQueueMinBlocks) {
        p.n_queues = p.xcd_cols > 0 ? 8 : 1;
        p.per_q = blocks / p.n_queues;  // exact: with 8 queues, n_cols = 8 * xcd_cols
        const int64_t extra = p.per_q / 4 + 64;
        grid = p.n_queues * p.per_q + 8 * extra;
        if (grid > INT32_MAX) {
            grid = blocks;
            p.per_q = 0;
            p.n_queues = 1;
        }
    }
    if (p.per_q > 0) {
        p.slot = (int32_t)(g_next_slot.fetch_add(1, std::memory_order_relaxed) % kCtrSlots);
        hipLaunchKernelGGL(fwd_ctr_reset_kernel, dim3(1), dim3(16), 0, stream, p.slot);
    }
    hipLaunchKernelGGL((block_fwd_bf16_kernel<D, NW, NB, KBP, KS>), dim3((unsigned)grid), dim3(64 * NW), 0, stream, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_head_dim(const BlockFwdArgs& a, Params p, hipStream_t stream) {
    // When 8-wave blocks would leave the chip less than half full: 8 waves over 128 rows with
    // the keys split between two wave groups (two waves per SIMD on every CU, where plain
    // 4-wave blocks would have one).  Otherwise 12 waves (three per SIMD: more of each wave's
    // softmax runs under the other waves' products; +5-7% on causal launches) when the
    // blocks' work differs, i.e. the launch walks several K/V blocks or the queries and keys
    // share one positions array (a causal triangle): the heavy blocks run first, so the last
    // round of blocks is light.  Launches of equal-work blocks (queries against another
    // shard's keys) keep 8 waves: 12-wave blocks hold 384/G positions (96 for G = 4), which
    // split a power-of-two shard into a part-filled last round of the 256 CUs, while
    // 64-position blocks divide it evenly.
    const int64_t blocks8 = ((a.seq_q + 256 / p.G - 1) / (256 / p.G)) * p.n_cols;
    if (blocks8 < 512) return launch_variant<D, 8, 1, 2, 2>(p, a.seq_q, stream);
    if (a.n_blk > 1 || a.blk[0].pos == a.q_pos) {
        // head dim 64: 16 waves, four per SIMD (the 64-dim kernel needs 110 registers).  The
        // softmax's vector work per score is the same as at 128 while the products per score
        // halve, so the kernel is bound by vector work, and a fourth wave per SIMD gives it
        // more to run beside (+2.8% on a 64K causal block, +4-7% on a 16K one).
        if constexpr (D == 64) return launch_variant<D, 16, 1, 1, 1>(p, a.seq_q, stream);
        else return launch_variant<D, 12, 1, 1, 1>(p, a.seq_q, stream);
    }
    return launch_variant<D, 8, 1, 2, 1>(p, a.seq_q, stream);
}

}  // namespace

hipError_t launch_block_fwd_bf16(const BlockFwdArgs& a, hipStream_t stream) {
    Params p;
    p.q = (const __bf16*)a.q;
    p.qpos = a.q_pos;
    p.out = a.out;
    p.lse = a.lse;
    p.seq_q = a.seq_q;
    p.n_blk = a.n_blk;
    p.q_rs = a.q_row_stride > 0 ? a.q_row_stride : (int64_t)a.heads_q * a.head_dim;
    p.kv_rs = a.kv_row_stride > 0 ? a.kv_row_stride : (int64_t)a.heads_kv * a.head_dim;
    p.out_rs = a.out_row_stride > 0 ? a.out_row_stride : (int64_t)a.heads_q * a.head_dim;
    for (int o = 0; o < a.n_blk; ++o)
        p.blk[o] = KVBlock{(const __bf16*)a.blk[o].k, (const __bf16*)a.blk[o].v, a.blk[o].pos, a.blk[o].seq};
    p.heads_q = a.heads_q;
    p.heads_kv = a.heads_kv;
    p.ratio = a.heads_q / a.heads_kv;
    p.G = (p.ratio % 4 == 0) ? 4 : (p.ratio % 2 == 0) ? 2 : 1;
    p.n_hg = p.ratio / p.G;
    p.n_cols = a.batch * a.heads_kv * p.n_hg;
    p.xcd_cols = (p.n_cols % 8 == 0) ? p.n_cols / 8 : 0;
    p.c = a.scale * kLog2e;
    p.merge = a.merge ? 1 : 0;
    return a.head_dim == 64 ? launch_head_dim<64>(a, p, stream) : launch_head_dim<128>(a, p, stream);
}

}  // namespace cpattn
