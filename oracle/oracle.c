/*
 * oracle.c -- plain, slow, fp64 CPU reference for one context-parallel rank's share
 * of causal attention and its layout companions.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's
 * cpu_baseline leg load this library.  The product library (context_causal_attention_amd)
 * never includes, links or calls it, and this file includes nothing from there.
 *
 * Every routine is the plain definition written out with loops: no blocking, no fusion,
 * no reordering beyond what the definition states.  Floating-point work is fp64.
 * Inputs arrive as fp32 arrays; bf16 inputs are passed as their exact fp32 upcast.
 *
 * Sources (web pages; cited by title and section):
 *   [CP]   "On Context Parallelism" (jonahsamost.bearblog.dev)
 *   [DAY74]"Context parallelism -- splitting the sequence across GPUs" (llmdaily.org, day 74)
 *   [RING] "Context Parallelism & Ring Attention" (Distributed Training from First Principles)
 *   [HB]   "Context parallelism: Ring Attention and Ulysses" (AI infra handbook)
 *   [OLMO] "Appendix F: Context Parallelism and MoE Parallel Folding" (olmo-core MoE report)
 *
 * Build: gcc -O2 -std=c11 -shared -fPIC oracle.c -o liboracle.so -lm -lpthread
 * (no -ffast-math: the arithmetic must be IEEE fp64 as written).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_BAD -1

/* ------------------------------------------------------------------------------------ */
/* Zigzag ownership.                                                                       */
/* [CP] section "All-gather": the sequence of S tokens is cut into 2C chunks of t = S/(2C); */
/* rank r holds chunk r followed by chunk 2C-r-1.  [RING] "The zigzag fix" and [HB] "The  */
/* zigzag partition" state the same pairing.  Output: the s = 2t global positions of the  */
/* rank's local tokens in local order.                                                    */
/* ------------------------------------------------------------------------------------ */
int orc_zigzag_positions(int64_t S, int32_t C, int32_t r, int64_t* out) {
    if (C <= 0 || S <= 0 || S % (2 * (int64_t)C) != 0 || r < 0 || r >= C) return ORC_BAD;
    const int64_t t = S / (2 * (int64_t)C);
    const int64_t early = r, late = 2 * (int64_t)C - r - 1;
    for (int64_t i = 0; i < t; ++i) out[i] = early * t + i;
    for (int64_t i = 0; i < t; ++i) out[t + i] = late * t + i;
    return ORC_OK;
}

/* Contiguous ownership ([RING] "The last remaining axis"; [DAY74] "What exactly gets
 * sharded?"): device p of P holds positions [p*S/P, (p+1)*S/P). */
int orc_contiguous_positions(int64_t S, int32_t P, int32_t p, int64_t* out) {
    if (P <= 0 || S <= 0 || S % P != 0 || p < 0 || p >= P) return ORC_BAD;
    const int64_t s = S / P;
    for (int64_t i = 0; i < s; ++i) out[i] = (int64_t)p * s + i;
    return ORC_OK;
}

/* ------------------------------------------------------------------------------------ */
/* All-gather reorder.  [CP] section "All-gather": the gather concatenates every rank's   */
/* whole local tensor in rank order, so gathered row i holds the token whose global       */
/* position is gathered_pos[i] = (zigzag positions of rank 0) ++ (rank 1) ++ ...           */
/* Direction 0 (rank order -> sequence order): out[b][gathered_pos[i]] = in[b][i].        */
/* Direction 1 (sequence order -> rank order): out[b][i] = in[b][gathered_pos[i]].        */
/* Rows are opaque byte strings of row_bytes.                                              */
/* ------------------------------------------------------------------------------------ */
int orc_gathered_positions(int64_t S, int32_t C, int64_t* out) {
    if (C <= 0 || S <= 0 || S % (2 * (int64_t)C) != 0) return ORC_BAD;
    const int64_t s = S / C;
    for (int32_t r = 0; r < C; ++r)
        if (orc_zigzag_positions(S, C, r, out + (int64_t)r * s) != ORC_OK) return ORC_BAD;
    return ORC_OK;
}

int orc_reorder(const uint8_t* in, uint8_t* out, int32_t B, int64_t S, int64_t row_bytes,
                int32_t C, int32_t dir) {
    if (B <= 0 || row_bytes <= 0 || (dir != 0 && dir != 1)) return ORC_BAD;
    int64_t* gp = (int64_t*)malloc(sizeof(int64_t) * (size_t)S);
    if (!gp) return ORC_BAD;
    if (orc_gathered_positions(S, C, gp) != ORC_OK) { free(gp); return ORC_BAD; }
    for (int64_t b = 0; b < B; ++b) {
        const uint8_t* src = in + b * S * row_bytes;
        uint8_t* dst = out + b * S * row_bytes;
        for (int64_t i = 0; i < S; ++i) {
            if (dir == 0) memcpy(dst + gp[i] * row_bytes, src + i * row_bytes, (size_t)row_bytes);
            else          memcpy(dst + i * row_bytes, src + gp[i] * row_bytes, (size_t)row_bytes);
        }
    }
    free(gp);
    return ORC_OK;
}

/* ------------------------------------------------------------------------------------ */
/* Ulysses layout change, done locally for one head group.                                */
/* [OLMO] Eq. (96): [B, S/C, H, d] -> [B, S, H/C, d]; [CP] section "All-to-all"; [HB]     */
/* "Ulysses: transposing between the sequence and the heads": after the exchange, the     */
/* rank of group g holds heads [g*H/C, (g+1)*H/C) for every sequence shard, and the       */
/* shard that came from rank src supplies sequence rows [src*S/C, (src+1)*S/C).           */
/* Input of dir 0: the C ranks' local tensors stacked, [C][B][S/C][H][D].                 */
/* dir 0 (sequence -> heads): out[b][src*S/C + i][h][d] = in[src][b][i][g*H/C + h][d],     */
/*   out is [B][S][H/C][D].                                                                */
/* dir 1 (heads -> sequence): the inverse assignment, in = [B][S][H/C][D], out = stacked   */
/*   [C][B][S/C][H][D]; only group g's heads of out are written.                           */
/* Elements are opaque byte strings of elem_bytes.                                         */
/* ------------------------------------------------------------------------------------ */
int orc_ulysses_permute(const uint8_t* in, uint8_t* out, int32_t elem_bytes, int32_t B, int64_t S,
                        int32_t H, int32_t D, int32_t C, int32_t g, int32_t dir) {
    if (elem_bytes <= 0 || B <= 0 || S <= 0 || H <= 0 || D <= 0 || C <= 0) return ORC_BAD;
    if (S % C != 0 || H % C != 0 || g < 0 || g >= C || (dir != 0 && dir != 1)) return ORC_BAD;
    const int64_t s = S / C, hg = H / C, e = elem_bytes;
    for (int64_t src = 0; src < C; ++src)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t i = 0; i < s; ++i)
                for (int64_t h = 0; h < hg; ++h)
                    for (int64_t d = 0; d < D; ++d) {
                        const int64_t stacked = ((((src * B + b) * s + i) * H + (g * hg + h)) * D + d) * e;
                        const int64_t grouped = (((b * S + src * s + i) * hg + h) * D + d) * e;
                        if (dir == 0) memcpy(out + grouped, in + stacked, (size_t)e);
                        else          memcpy(out + stacked, in + grouped, (size_t)e);
                    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------------------ */
/* Causal attention by its definition, for any subset of query rows.                      */
/* [DAY74] "Why long contexts stress training memory": s_ij = <q_i, k_j> * scale and      */
/* o_i = sum_{j visible} softmax_j(s_ij) v_j, with key j visible to query i iff its global */
/* position is not later than the query's ([HB] cp_common's mask hides k > q).             */
/* [CP] section "Peer-to-peer", the merge discussion: lse = m + ln(sum_j exp(s_j - m)),    */
/* natural log, m the row maximum.                                                         */
/* Layouts: q [B][Sq][Hq][D], k and v [B][Skv][Hkv][D] (fp32 values), positions int64.      */
/* Query head h reads kv head h / (Hq/Hkv) (grouped-query attention).                      */
/* Outputs for the selected rows: out [B][nrows][Hq][D], lse [B][Hq][nrows], fp64.         */
/* A row with no visible key gets out = 0 and lse = -inf (no contribution).                */
/* ------------------------------------------------------------------------------------ */
typedef struct {
    const float *q, *k, *v;
    int64_t B, Sq, Skv, Hq, Hkv, D;
    const int64_t *qpos, *kvpos, *rows;
    int64_t nrows;
    double scale;
    double *out, *lse;
    int64_t next;  /* work counter, guarded by mu */
    pthread_mutex_t mu;
} attn_job_t;

static void attend_one(attn_job_t* J, int64_t b, int64_t h, int64_t ri, double* sc) {
    const int64_t D = J->D, i = J->rows[ri], kh = h / (J->Hq / J->Hkv);
    const float* qi = J->q + ((b * J->Sq + i) * J->Hq + h) * D;
    const int64_t p = J->qpos[i];
    double* o = J->out + ((b * J->nrows + ri) * J->Hq + h) * D;
    double m = -INFINITY;
    int64_t nvis = 0;
    /* pass 1: scores of visible keys and their maximum */
    for (int64_t j = 0; j < J->Skv; ++j) {
        if (J->kvpos[j] > p) { sc[j] = NAN; continue; }
        const float* kj = J->k + ((b * J->Skv + j) * J->Hkv + kh) * D;
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += (double)qi[d] * (double)kj[d];
        sc[j] = dot * J->scale;
        if (sc[j] > m) m = sc[j];
        ++nvis;
    }
    for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
    double* lse = J->lse + (b * J->Hq + h) * J->nrows + ri;
    if (nvis == 0) { *lse = -INFINITY; return; }
    /* pass 2: unnormalised weights, their sum and the weighted value sum */
    double l = 0.0;
    for (int64_t j = 0; j < J->Skv; ++j) {
        if (J->kvpos[j] > p) continue;
        const double w = exp(sc[j] - m);
        l += w;
        const float* vj = J->v + ((b * J->Skv + j) * J->Hkv + kh) * D;
        for (int64_t d = 0; d < D; ++d) o[d] += w * (double)vj[d];
    }
    for (int64_t d = 0; d < D; ++d) o[d] /= l;
    *lse = m + log(l);
}

static void* attn_worker(void* arg) {
    attn_job_t* J = (attn_job_t*)arg;
    double* sc = (double*)malloc(sizeof(double) * (size_t)(J->Skv > 0 ? J->Skv : 1));
    const int64_t total = J->B * J->Hq * J->nrows;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        const int64_t w = J->next++;
        pthread_mutex_unlock(&J->mu);
        if (w >= total) break;
        const int64_t ri = w % J->nrows, h = (w / J->nrows) % J->Hq, b = w / (J->nrows * J->Hq);
        attend_one(J, b, h, ri, sc);
    }
    free(sc);
    return NULL;
}

int orc_attention_rows(const float* q, const float* k, const float* v, int32_t B, int64_t Sq,
                       int64_t Skv, int32_t Hq, int32_t Hkv, int32_t D, const int64_t* qpos,
                       const int64_t* kvpos, double scale, const int64_t* rows, int64_t nrows,
                       double* out, double* lse, int32_t nthreads) {
    if (B <= 0 || Sq < 0 || Skv < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || nrows < 0) return ORC_BAD;
    if (Hq % Hkv != 0) return ORC_BAD;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= Sq) return ORC_BAD;
    attn_job_t J = {q, k, v, B, Sq, Skv, Hq, Hkv, D, qpos, kvpos, rows, nrows, scale, out, lse, 0};
    pthread_mutex_init(&J.mu, NULL);
    if (nthreads < 1) nthreads = 1;
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    for (int32_t t = 0; t < nthreads; ++t) pthread_create(&th[t], NULL, attn_worker, &J);
    for (int32_t t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
    free(th);
    pthread_mutex_destroy(&J.mu);
    return ORC_OK;
}

/* ------------------------------------------------------------------------------------ */
/* Per-block softmax statistics, [DAY74] "How do partial softmax results combine?":        */
/* for one query row and one block of keys, m_r = max s_j, l_r = sum exp(s_j - m_r),      */
/* z_r = sum exp(s_j - m_r) v_j (unnormalised).  A block with no visible key gives         */
/* m_r = -inf, l_r = 0, z_r = 0.  Layouts as orc_attention_rows; m, l [B][Hq][nrows],       */
/* z [B][nrows][Hq][D].  Single-threaded: used on small cases only.                        */
/* ------------------------------------------------------------------------------------ */
int orc_block_stats(const float* q, const float* k, const float* v, int32_t B, int64_t Sq,
                    int64_t Skv, int32_t Hq, int32_t Hkv, int32_t D, const int64_t* qpos,
                    const int64_t* kvpos, double scale, const int64_t* rows, int64_t nrows,
                    double* m_out, double* l_out, double* z_out) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0) return ORC_BAD;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < Hq; ++h)
            for (int64_t ri = 0; ri < nrows; ++ri) {
                const int64_t i = rows[ri], kh = h / (Hq / Hkv);
                const float* qi = q + ((b * Sq + i) * Hq + h) * D;
                double m = -INFINITY;
                for (int64_t j = 0; j < Skv; ++j) {
                    if (kvpos[j] > qpos[i]) continue;
                    const float* kj = k + ((b * Skv + j) * Hkv + kh) * D;
                    double dot = 0.0;
                    for (int64_t d = 0; d < D; ++d) dot += (double)qi[d] * (double)kj[d];
                    if (dot * scale > m) m = dot * scale;
                }
                double l = 0.0;
                double* z = z_out + ((b * nrows + ri) * Hq + h) * D;
                for (int64_t d = 0; d < D; ++d) z[d] = 0.0;
                if (m != -INFINITY) {
                    for (int64_t j = 0; j < Skv; ++j) {
                        if (kvpos[j] > qpos[i]) continue;
                        const float* kj = k + ((b * Skv + j) * Hkv + kh) * D;
                        const float* vj = v + ((b * Skv + j) * Hkv + kh) * D;
                        double dot = 0.0;
                        for (int64_t d = 0; d < D; ++d) dot += (double)qi[d] * (double)kj[d];
                        const double w = exp(dot * scale - m);
                        l += w;
                        for (int64_t d = 0; d < D; ++d) z[d] += w * (double)vj[d];
                    }
                }
                m_out[(b * Hq + h) * nrows + ri] = m;
                l_out[(b * Hq + h) * nrows + ri] = l;
            }
    return ORC_OK;
}

/* ------------------------------------------------------------------------------------ */
/* Merge of two completed partial results, [CP] section "Peer-to-peer" (the LSE merge of  */
/* attention tiles) and [HB] "Ring Attention": merged = log(e^lse + e^lse_t);              */
/* out <- e^(lse - merged) * out + e^(lse_t - merged) * out_t; lse <- merged.               */
/* A side with lse = -inf carries zero weight; two empty sides give (0, -inf).             */
/* In place on out [B][s][H][D] and lse [B][H][s].                                          */
/* ------------------------------------------------------------------------------------ */
static double log_add_exp(double x, double y) {
    if (x == -INFINITY) return y;
    if (y == -INFINITY) return x;
    const double mx = x > y ? x : y;
    return mx + log(exp(x - mx) + exp(y - mx));
}

int orc_merge(double* out, double* lse, const double* out_t, const double* lse_t, int32_t B,
              int64_t s, int32_t H, int32_t D) {
    if (B <= 0 || s < 0 || H <= 0 || D <= 0) return ORC_BAD;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < H; ++h)
            for (int64_t i = 0; i < s; ++i) {
                double* L = lse + (b * H + h) * s + i;
                const double Lt = lse_t[(b * H + h) * s + i];
                const double merged = log_add_exp(*L, Lt);
                const double a = (merged == -INFINITY) ? 0.0 : exp(*L - merged);
                const double c = (merged == -INFINITY) ? 0.0 : exp(Lt - merged);
                double* o = out + ((b * s + i) * H + h) * D;
                const double* ot = out_t + ((b * s + i) * H + h) * D;
                for (int64_t d = 0; d < D; ++d) o[d] = a * o[d] + c * ot[d];
                *L = merged;
            }
    return ORC_OK;
}

/* ------------------------------------------------------------------------------------ */
/* Closed-form combine of R blocks, [DAY74] "How do partial softmax results combine?":     */
/* m = max_r m_r;  o = sum_r e^(m_r - m) z_r / sum_r e^(m_r - m) l_r;                        */
/* and lse = m + ln(sum_r e^(m_r - m) l_r).                                                 */
/* m, l: [R][n]; z: [R][n][D]; out [n][D]; lse [n].  Rows with no visible key anywhere      */
/* (all m_r = -inf) give out = 0, lse = -inf.                                               */
/* ------------------------------------------------------------------------------------ */
int orc_combine_blocks(const double* m, const double* l, const double* z, int32_t R, int64_t n,
                       int32_t D, double* out, double* lse) {
    if (R <= 0 || n < 0 || D <= 0) return ORC_BAD;
    for (int64_t i = 0; i < n; ++i) {
        double mm = -INFINITY;
        for (int32_t r = 0; r < R; ++r) if (m[(int64_t)r * n + i] > mm) mm = m[(int64_t)r * n + i];
        double* o = out + i * D;
        for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
        if (mm == -INFINITY) { lse[i] = -INFINITY; continue; }
        double den = 0.0;
        for (int32_t r = 0; r < R; ++r) {
            const double mr = m[(int64_t)r * n + i];
            if (mr == -INFINITY) continue;
            const double w = exp(mr - mm);
            den += w * l[(int64_t)r * n + i];
            const double* zr = z + ((int64_t)r * n + i) * D;
            for (int64_t d = 0; d < D; ++d) o[d] += w * zr[d];
        }
        for (int64_t d = 0; d < D; ++d) o[d] /= den;
        lse[i] = mm + log(den);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------------------ */
/* Backward of one block.  [CP] section "Peer-to-peer" / "Backward": each ring step takes  */
/* the local queries, one K/V block, the saved output and lse and the output gradient,    */
/* and yields tile_dq, tile_dk, tile_dv; dq adds up over the steps and dk, dv over the     */
/* ranks.  The pages do not print the formulas; they are the chain rule applied to the     */
/* attention definition above.  With lse_i the row's complete log-sum-exp (all blocks):    */
/*   p_ij  = exp(scale <q_i, k_j> - lse_i) for visible pairs, 0 otherwise                  */
/*   D_i   = sum_d dout_i,d out_i,d                                                         */
/*   dp_ij = <dout_i, v_j>,   ds_ij = p_ij (dp_ij - D_i)                                    */
/*   dq_i  = scale sum_j ds_ij k_j,  dk_j = scale sum_i ds_ij q_i,  dv_j = sum_i p_ij dout_i */
/* Grouped-query attention: dk and dv of kv head c sum over the query heads reading it.    */
/* Layouts: q, dout [B][Sq][Hq][D]; k, v [B][Skv][Hkv][D] (fp32 values); out [B][Sq][Hq][D] */
/* and lse [B][Hq][Sq] fp64.  Outputs for the selected query rows qrows and key rows krows: */
/* dq [B][nq][Hq][D], dk and dv [B][nk][Hkv][D], fp64, overwritten.                        */
/* ------------------------------------------------------------------------------------ */
typedef struct {
    const float *q, *k, *v, *dout;
    const double *out, *lse;
    int64_t B, Sq, Skv, Hq, Hkv, D;
    const int64_t *qpos, *kvpos, *qrows, *krows;
    int64_t nq, nk;
    double scale;
    double *dq, *dk, *dv;
    int32_t bf16_pds;
    int64_t next;
    pthread_mutex_t mu;
} bwd_job_t;

static double bwd_delta(const bwd_job_t* J, int64_t b, int64_t h, int64_t i) {
    const float* g = J->dout + ((b * J->Sq + i) * J->Hq + h) * J->D;
    const double* o = J->out + ((b * J->Sq + i) * J->Hq + h) * J->D;
    double s = 0.0;
    for (int64_t d = 0; d < J->D; ++d) s += (double)g[d] * o[d];
    return s;
}

/* x rounded to the nearest bf16 value, ties to even (bf16: 8 significant bits, the fp32
 * exponent range, subnormals below 2^-126 in steps of 2^-133).  Exact for finite x of
 * magnitude below the largest bf16; nearbyint rounds ties to even in the default mode. */
static double round_bf16(double x) {
    if (x == 0.0 || !isfinite(x)) return x;
    if (fabs(x) < ldexp(1.0, -126)) return nearbyint(ldexp(x, 133)) * ldexp(1.0, -133);
    int e;
    const double m = frexp(x, &e); /* x = m 2^e, 0.5 <= |m| < 1 */
    return ldexp(nearbyint(ldexp(m, 8)), e - 8);
}

int orc_round_bf16(const double* x, double* y, int64_t n) {
    if (n < 0) return ORC_BAD;
    for (int64_t i = 0; i < n; ++i) y[i] = round_bf16(x[i]);
    return ORC_OK;
}

/* p_ij and ds_ij of one visible pair (query row i of head h, key row j of kv head c).
 * With bf16_pds set (a model of a bf16 backward that rounds the two matrix-product
 * operands it forms itself), p is rounded to bf16 for its use in dv, and ds is rounded
 * after being formed from the unrounded p; all else stays fp64. */
static void bwd_pair(const bwd_job_t* J, int64_t b, int64_t h, int64_t i, int64_t c, int64_t j,
                     double delta, double* p, double* ds) {
    const int64_t D = J->D;
    const float* qi = J->q + ((b * J->Sq + i) * J->Hq + h) * D;
    const float* gi = J->dout + ((b * J->Sq + i) * J->Hq + h) * D;
    const float* kj = J->k + ((b * J->Skv + j) * J->Hkv + c) * D;
    const float* vj = J->v + ((b * J->Skv + j) * J->Hkv + c) * D;
    double s = 0.0, dp = 0.0;
    for (int64_t d = 0; d < D; ++d) {
        s += (double)qi[d] * (double)kj[d];
        dp += (double)gi[d] * (double)vj[d];
    }
    *p = exp(s * J->scale - J->lse[(b * J->Hq + h) * J->Sq + i]);
    *ds = *p * (dp - delta);
    if (J->bf16_pds) {
        *p = round_bf16(*p);
        *ds = round_bf16(*ds);
    }
}

static void* bwd_worker(void* arg) {
    bwd_job_t* J = (bwd_job_t*)arg;
    const int64_t D = J->D, G = J->Hq / J->Hkv;
    const int64_t nq_jobs = J->B * J->Hq * J->nq, total = nq_jobs + J->B * J->Hkv * J->nk;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        const int64_t w = J->next++;
        pthread_mutex_unlock(&J->mu);
        if (w >= total) break;
        if (w < nq_jobs) {
            /* dq of one query row */
            const int64_t ri = w % J->nq, h = (w / J->nq) % J->Hq, b = w / (J->nq * J->Hq);
            const int64_t i = J->qrows[ri], c = h / G;
            double* dq = J->dq + ((b * J->nq + ri) * J->Hq + h) * D;
            for (int64_t d = 0; d < D; ++d) dq[d] = 0.0;
            if (J->lse[(b * J->Hq + h) * J->Sq + i] == -INFINITY) continue;
            const double delta = bwd_delta(J, b, h, i);
            for (int64_t j = 0; j < J->Skv; ++j) {
                if (J->kvpos[j] > J->qpos[i]) continue;
                double p, ds;
                bwd_pair(J, b, h, i, c, j, delta, &p, &ds);
                const float* kj = J->k + ((b * J->Skv + j) * J->Hkv + c) * D;
                for (int64_t d = 0; d < D; ++d) dq[d] += J->scale * ds * (double)kj[d];
            }
        } else {
            /* dk and dv of one key row */
            const int64_t u = w - nq_jobs;
            const int64_t rj = u % J->nk, c = (u / J->nk) % J->Hkv, b = u / (J->nk * J->Hkv);
            const int64_t j = J->krows[rj];
            double* dk = J->dk + ((b * J->nk + rj) * J->Hkv + c) * D;
            double* dv = J->dv + ((b * J->nk + rj) * J->Hkv + c) * D;
            for (int64_t d = 0; d < D; ++d) { dk[d] = 0.0; dv[d] = 0.0; }
            for (int64_t h = c * G; h < (c + 1) * G; ++h)
                for (int64_t i = 0; i < J->Sq; ++i) {
                    if (J->kvpos[j] > J->qpos[i]) continue;
                    if (J->lse[(b * J->Hq + h) * J->Sq + i] == -INFINITY) continue;
                    double p, ds;
                    bwd_pair(J, b, h, i, c, j, bwd_delta(J, b, h, i), &p, &ds);
                    const float* qi = J->q + ((b * J->Sq + i) * J->Hq + h) * D;
                    const float* gi = J->dout + ((b * J->Sq + i) * J->Hq + h) * D;
                    for (int64_t d = 0; d < D; ++d) {
                        dk[d] += J->scale * ds * (double)qi[d];
                        dv[d] += p * (double)gi[d];
                    }
                }
        }
    }
    return NULL;
}

int orc_block_bwd(const float* q, const float* k, const float* v, const float* dout, const double* out,
                  const double* lse, int32_t B, int64_t Sq, int64_t Skv, int32_t Hq, int32_t Hkv, int32_t D,
                  const int64_t* qpos, const int64_t* kvpos, double scale, const int64_t* qrows,
                  int64_t nq, const int64_t* krows, int64_t nk, double* dq, double* dk, double* dv,
                  int32_t bf16_pds, int32_t nthreads) {
    if (B <= 0 || Sq < 0 || Skv < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0) return ORC_BAD;
    if (nq < 0 || nk < 0) return ORC_BAD;
    for (int64_t r = 0; r < nq; ++r) if (qrows[r] < 0 || qrows[r] >= Sq) return ORC_BAD;
    for (int64_t r = 0; r < nk; ++r) if (krows[r] < 0 || krows[r] >= Skv) return ORC_BAD;
    bwd_job_t J = {q, k, v, dout, out, lse, B, Sq, Skv, Hq, Hkv, D, qpos, kvpos, qrows, krows,
                   nq, nk, scale, dq, dk, dv, bf16_pds ? 1 : 0, 0};
    pthread_mutex_init(&J.mu, NULL);
    if (nthreads < 1) nthreads = 1;
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    for (int32_t t = 0; t < nthreads; ++t) pthread_create(&th[t], NULL, bwd_worker, &J);
    for (int32_t t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
    free(th);
    pthread_mutex_destroy(&J.mu);
    return ORC_OK;
}
