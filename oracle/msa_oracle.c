/*
 * msa_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, double-precision CPU implementation of MSA sparse-layer
 * decode attention (block scores over a paged index cache, top-k block
 * selection, attention over the selected pages).  It exists to check the HIP
 * library and is called only from the tests, the smoke check and the bench's
 * CPU-baseline leg.  It shares no code with the GPU path.
 *
 * Sources (the pages, cited by title and section):
 *  - Cacheon "Kernel ABI", section "Attention block slots":
 *      attention.decode         -- attend exactly the supplied nonnegative block
 *                                  ids; -1 entries and tokens at or beyond
 *                                  seq_lens are excluded; GQA head expansion as
 *                                  in attention.sdpa (Hq divisible by Hkv).
 *      attention.msa_block_score -- a block-max score sheet per query.
 *      attention.msa_prefill_block_score -- per-query selection, unused output
 *                                  cells are -1.
 *  - Cacheon "Kernel ABI", section "Correctness is target-owned": block
 *    selections are graded as sets (index order is not semantic).
 *  - vLLM design note "MiniMax-M3 decode through the ATOM kernel library",
 *    section "Supported experiment": FP8 main and index caches, block size 128,
 *    static scalar K/V scales, 1 + 3 speculative tokens per row.
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes of the repository):
 *  - score[n][j] = idx_scale * max over the visible tokens s of block j of
 *    sum_d q_idx[n][d] * code(index_k[page(j)][s][d]); -inf if block j has no
 *    visible token.  The pages leave the score function open.
 *  - Query token n = r*T + t of row r sees key positions [0, V(n)) with
 *    V(n) = max(0, seq_lens[r] - (T-1-t)): causal within the row, the row's T
 *    new tokens already in the cache.
 *  - Selection: candidates are scores that are neither -inf nor NaN; order by
 *    (score descending, block id ascending) with -0 equal to +0; take
 *    min(k, #candidates); emit in ascending block id; pad with -1.
 *  - Attention logit = sm_scale * k_scale * sum_d q*code(k); weights
 *    exp(logit - max); out = v_scale * sum p*code(v) / sum p; 0 when the
 *    selection holds no visible token.
 *  - E4M3FN per the OCP 8-bit floating point format: 1 sign, 4 exponent bits
 *    (bias 7), 3 mantissa bits, no infinities, S.1111.111 is NaN, max 448.
 *
 * All functions return 0 on success and a positive code when an input breaks a
 * precondition (the tests rely on that to catch generator mistakes).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_E4M3FN = 2 };
enum { ORC_OK = 0, ORC_EARG = 1, ORC_EPAGE = 2, ORC_ELEN = 3, ORC_EDUP = 4, ORC_ENAN = 5 };

/* ---------------------------------------------------------------- decoding */

double orc_e4m3fn_value(uint8_t code)
{
    int sign = code >> 7;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);               /* subnormal: m/8 * 2^(1-7) */
    else
        v = ldexp(1.0 + m / 8.0, e - 7);        /* normal: 1.m * 2^(e-7) */
    return sign ? -v : v;
}

double orc_bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;          /* bf16 is the top half of fp32 */
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double elem(const void *base, int dtype, int64_t i)
{
    switch (dtype) {
    case ORC_F32:    return (double)((const float *)base)[i];
    case ORC_BF16:   return orc_bf16_value(((const uint16_t *)base)[i]);
    case ORC_E4M3FN: return orc_e4m3fn_value(((const uint8_t *)base)[i]);
    }
    return NAN;
}

/* Keys visible to query token n. */
static int64_t visible(const int32_t *seq_lens, int64_t T, int64_t n)
{
    int64_t r = n / T, t = n % T;
    int64_t v = (int64_t)seq_lens[r] - (T - 1 - t);
    return v > 0 ? v : 0;
}

static int check_lens(const int32_t *seq_lens, int64_t R, int64_t MB, int64_t B)
{
    for (int64_t r = 0; r < R; r++)
        if (seq_lens[r] < 0 || (int64_t)seq_lens[r] > MB * B)
            return ORC_ELEN;
    return ORC_OK;
}

/* ------------------------------------------------------------ block scores */

/*
 * Score sheet rows n in [n_begin, n_end).  q_idx [N, Di]; index_k [P, B, Di];
 * block_table [R, MB]; seq_lens [R]; scores [N, MB] (row-major, doubles).
 */
int orc_block_score(const void *q_idx, int q_dtype, const void *index_k, int k_dtype,
                    const int32_t *block_table, const int32_t *seq_lens,
                    int64_t R, int64_t T, int64_t MB, int64_t P, int64_t B, int64_t Di,
                    double idx_scale, int64_t n_begin, int64_t n_end, double *scores)
{
    if (T < 1 || B < 1 || Di < 1 || MB < 1 || n_begin < 0 || n_end > R * T || !(idx_scale > 0))
        return ORC_EARG;
    if (check_lens(seq_lens, R, MB, B))
        return ORC_ELEN;
    for (int64_t n = n_begin; n < n_end; n++) {
        int64_t r = n / T;
        int64_t vis = visible(seq_lens, T, n);
        for (int64_t j = 0; j < MB; j++) {
            int64_t lo = j * B, hi = (j + 1) * B < vis ? (j + 1) * B : vis;
            double best = -INFINITY;
            if (lo < hi) {
                int64_t page = block_table[r * MB + j];
                if (page < 0 || page >= P)
                    return ORC_EPAGE;
                for (int64_t s = lo; s < hi; s++) {
                    double dot = 0.0;
                    for (int64_t d = 0; d < Di; d++)
                        dot += elem(q_idx, q_dtype, n * Di + d) *
                               elem(index_k, k_dtype, (page * B + (s - lo)) * Di + d);
                    if (isnan(dot))
                        return ORC_ENAN;
                    if (dot > best)
                        best = dot;
                }
                best *= idx_scale;
            }
            scores[n * MB + j] = best;
        }
    }
    return ORC_OK;
}

/* --------------------------------------------------------------- selection */

typedef struct { double s; int32_t j; } cand_t;

static int by_score_then_id(const void *a, const void *b)
{
    const cand_t *x = a, *y = b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->j > y->j) - (x->j < y->j);
}

static int by_id(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/* topk_idx [N, k] from scores [N, MB]. */
int orc_select_topk(const double *scores, int64_t N, int64_t MB, int64_t k, int32_t *topk_idx)
{
    if (N < 0 || MB < 1 || k < 1)
        return ORC_EARG;
    cand_t *c = malloc(sizeof(cand_t) * (size_t)MB);
    int32_t *ids = malloc(sizeof(int32_t) * (size_t)MB);
    if (!c || !ids) { free(c); free(ids); return ORC_EARG; }
    for (int64_t n = 0; n < N; n++) {
        int64_t nc = 0;
        for (int64_t j = 0; j < MB; j++) {
            double s = scores[n * MB + j];
            if (isnan(s) || s == -INFINITY)
                continue;
            c[nc].s = (s == 0.0) ? 0.0 : s;   /* -0 counts as +0 */
            c[nc].j = (int32_t)j;
            nc++;
        }
        qsort(c, (size_t)nc, sizeof(cand_t), by_score_then_id);
        int64_t take = nc < k ? nc : k;
        for (int64_t i = 0; i < take; i++)
            ids[i] = c[i].j;
        qsort(ids, (size_t)take, sizeof(int32_t), by_id);
        for (int64_t i = 0; i < k; i++)
            topk_idx[n * k + i] = i < take ? ids[i] : -1;
    }
    free(c);
    free(ids);
    return ORC_OK;
}

/* -------------------------------------------------- prefill score + select */

/*
 * Score-to-selection over a ragged prefill batch, one call per batch
 * (Cacheon "Kernel ABI", "Attention block slots",
 * attention.msa_prefill_block_score).  Readings where the page is silent:
 *  - request b (block_table row slot_ids[b]) has new query tokens
 *    q[cu_seqlens[b] .. cu_seqlens[b+1]); its query block qb (block_size_q
 *    tokens, the last one possibly short) sees the keys
 *    [0, V) with V = min(seq_lens[b], prefix_lens[b] + qb * block_size_q),
 *    the keys before the block's first token;
 *  - score(h, qb, j) = scale * max over the block's tokens t and the visible
 *    keys s of block j of sum_d q[t][h][d] * code(index_k[page(j)][s][d]);
 *    the candidates are the blocks j < ceil(V / B);
 *  - forced blocks: the first init_blocks and the last local_blocks
 *    candidates; the selection takes the forced blocks (lower ids first when
 *    they exceed topk), then the highest-scoring other candidates (ties to
 *    the lower id, -0 equal to +0), emits ascending ids, pads with -1;
 *  - out_topk [Hq, all_qb, topk] row cu_seqblocks_q[b] + qb; rows no query
 *    block owns hold -1.
 * scores, when not NULL, receives [Hq, all_qb, MB] (-inf where no candidate).
 * rows, when not NULL, is a [Hq, all_qb] mask: only the rows it marks are
 * computed (the others stay -1 / -inf), so that large batches can be sampled.
 */
int orc_prefill_select(const void *q, int q_dtype, int64_t total_q, int64_t Hq, int64_t Di,
                       const void *index_k, int k_dtype, int64_t P, int64_t B,
                       const int32_t *block_table, int64_t nslots, int64_t MB,
                       const int32_t *slot_ids, const int32_t *cu_seqlens, const int32_t *seq_lens,
                       const int32_t *prefix_lens, int64_t batch, int64_t bsq, int64_t topk,
                       int64_t init_blocks, int64_t local_blocks, double scale,
                       const int32_t *cu_seqblocks_q, int64_t all_qb, int64_t h_begin, int64_t h_end,
                       const uint8_t *rows, int32_t *out_topk, double *scores)
{
    if (Hq < 1 || Di < 1 || B < 1 || MB < 1 || bsq < 1 || topk < 1 || init_blocks < 0 ||
        local_blocks < 0 || !(scale > 0) || h_begin < 0 || h_end > Hq || batch < 0)
        return ORC_EARG;
    for (int64_t i = 0; i < Hq * all_qb * topk; i++)
        if (i / (all_qb * topk) >= h_begin && i / (all_qb * topk) < h_end)
            out_topk[i] = -1;
    if (scores)
        for (int64_t i = h_begin * all_qb * MB; i < h_end * all_qb * MB; i++)
            scores[i] = -INFINITY;
    cand_t *c = malloc(sizeof(cand_t) * (size_t)MB);
    int32_t *ids = malloc(sizeof(int32_t) * (size_t)MB);
    double *sc = malloc(sizeof(double) * (size_t)MB);
    char *forced = malloc((size_t)MB);
    if (!c || !ids || !sc || !forced) { free(c); free(ids); free(sc); free(forced); return ORC_EARG; }
    int rc = ORC_OK;
    for (int64_t b = 0; b < batch && rc == ORC_OK; b++) {
        const int64_t q0 = cu_seqlens[b], nq = (int64_t)cu_seqlens[b + 1] - q0;
        const int64_t nqb = (nq + bsq - 1) / bsq;
        const int64_t row0 = cu_seqblocks_q[b];
        const int64_t slot = slot_ids[b];
        if (nq < 0 || q0 < 0 || q0 + nq > total_q || slot < 0 || slot >= nslots ||
            (int64_t)cu_seqblocks_q[b + 1] - row0 != nqb || row0 < 0 || row0 + nqb > all_qb ||
            prefix_lens[b] < 0 || seq_lens[b] < 0 || (int64_t)seq_lens[b] > MB * B) {
            rc = ORC_EARG;
            break;
        }
        for (int64_t h = h_begin; h < h_end && rc == ORC_OK; h++) {
            for (int64_t qb = 0; qb < nqb && rc == ORC_OK; qb++) {
                if (rows && !rows[h * all_qb + row0 + qb])
                    continue;                     /* row not asked for: stays -1 / -inf */
                int64_t V = (int64_t)prefix_lens[b] + qb * bsq;
                if (V > seq_lens[b])
                    V = seq_lens[b];
                const int64_t ncand = (V + B - 1) / B;
                const int64_t t1 = (qb + 1) * bsq < nq ? (qb + 1) * bsq : nq;
                for (int64_t j = 0; j < ncand; j++) {
                    const int64_t page = block_table[slot * MB + j];
                    if (page < 0 || page >= P) { rc = ORC_EPAGE; break; }
                    const int64_t s1 = (j + 1) * B < V ? (j + 1) * B : V;
                    double best = -INFINITY;
                    for (int64_t t = qb * bsq; t < t1; t++)
                        for (int64_t s = j * B; s < s1; s++) {
                            double dot = 0.0;
                            for (int64_t d = 0; d < Di; d++)
                                dot += elem(q, q_dtype, ((q0 + t) * Hq + h) * Di + d) *
                                       elem(index_k, k_dtype, (page * B + (s - j * B)) * Di + d);
                            if (isnan(dot)) rc = ORC_ENAN;
                            if (dot > best) best = dot;
                        }
                    sc[j] = scale * best;
                    if (scores)
                        scores[(h * all_qb + row0 + qb) * MB + j] = sc[j];
                }
                if (rc != ORC_OK)
                    break;
                /* forced blocks first (lower ids first), then by score */
                int64_t take = 0;
                for (int64_t j = 0; j < ncand; j++)
                    forced[j] = (j < init_blocks) || (j >= ncand - local_blocks);
                for (int64_t j = 0; j < ncand && take < topk; j++)
                    if (forced[j])
                        ids[take++] = (int32_t)j;
                int64_t nc = 0;
                for (int64_t j = 0; j < ncand; j++)
                    if (!forced[j]) {
                        c[nc].s = (sc[j] == 0.0) ? 0.0 : sc[j];
                        c[nc].j = (int32_t)j;
                        nc++;
                    }
                qsort(c, (size_t)nc, sizeof(cand_t), by_score_then_id);
                for (int64_t i = 0; i < nc && take < topk; i++)
                    ids[take++] = c[i].j;
                qsort(ids, (size_t)take, sizeof(int32_t), by_id);
                int32_t *dst = out_topk + (h * all_qb + row0 + qb) * topk;
                for (int64_t i = 0; i < topk; i++)
                    dst[i] = i < take ? ids[i] : -1;
            }
        }
    }
    free(c);
    free(ids);
    free(sc);
    free(forced);
    return rc;
}

/* --------------------------------------------------------------- attention */

/*
 * Sparse attention for query tokens n in [n_begin, n_end).
 * q [N, Hq, D]; k_cache, v_cache [P, B, Hkv, D]; topk_idx [N, K];
 * out [N, Hq, D] doubles.  Query head h reads KV head h / (Hq / Hkv).
 */
int orc_sparse_decode(const void *q, int q_dtype, const void *k_cache, const void *v_cache,
                      int kv_dtype, const int32_t *block_table, const int32_t *seq_lens,
                      const int32_t *topk_idx, int64_t R, int64_t T, int64_t MB, int64_t P,
                      int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t K,
                      double sm_scale, double k_scale, double v_scale,
                      int64_t n_begin, int64_t n_end, double *out)
{
    if (T < 1 || B < 1 || D < 1 || K < 1 || Hkv < 1 || Hq % Hkv || n_begin < 0 || n_end > R * T)
        return ORC_EARG;
    if (check_lens(seq_lens, R, MB, B))
        return ORC_ELEN;
    int64_t G = Hq / Hkv;
    double *logit = malloc(sizeof(double) * (size_t)(K * B));
    int64_t *slot = malloc(sizeof(int64_t) * (size_t)(K * B));   /* page*B + offset */
    double *acc = malloc(sizeof(double) * (size_t)D);
    if (!logit || !slot || !acc) { free(logit); free(slot); free(acc); return ORC_EARG; }
    int rc = ORC_OK;

    for (int64_t n = n_begin; n < n_end && rc == ORC_OK; n++) {
        int64_t r = n / T;
        int64_t vis = visible(seq_lens, T, n);
        /* the visible keys of the selected blocks */
        int64_t nkeys = 0;
        for (int64_t i = 0; i < K; i++) {
            int64_t j = topk_idx[n * K + i];
            if (j < 0 || j >= MB)
                continue;                         /* -1 (or out of range) = none */
            for (int64_t i2 = 0; i2 < i; i2++)
                if (topk_idx[n * K + i2] == j)
                    rc = ORC_EDUP;
            int64_t lo = j * B, hi = (j + 1) * B < vis ? (j + 1) * B : vis;
            if (lo >= hi)
                continue;
            int64_t page = block_table[r * MB + j];
            if (page < 0 || page >= P)
                rc = ORC_EPAGE;
            for (int64_t s = lo; s < hi && rc == ORC_OK; s++)
                slot[nkeys++] = page * B + (s - lo);
        }
        if (rc != ORC_OK)
            break;
        for (int64_t h = 0; h < Hq; h++) {
            int64_t g = h / G;
            const int64_t qoff = (n * Hq + h) * D;
            double mx = -INFINITY;
            for (int64_t e = 0; e < nkeys; e++) {
                const int64_t koff = (slot[e] * Hkv + g) * D;
                double dot = 0.0;
                for (int64_t d = 0; d < D; d++)
                    dot += elem(q, q_dtype, qoff + d) * elem(k_cache, kv_dtype, koff + d);
                logit[e] = sm_scale * k_scale * dot;
                if (isnan(logit[e]))
                    rc = ORC_ENAN;
                if (logit[e] > mx)
                    mx = logit[e];
            }
            double denom = 0.0;
            for (int64_t d = 0; d < D; d++)
                acc[d] = 0.0;
            for (int64_t e = 0; e < nkeys; e++) {
                double p = exp(logit[e] - mx);
                const int64_t voff = (slot[e] * Hkv + g) * D;
                denom += p;
                for (int64_t d = 0; d < D; d++)
                    acc[d] += p * elem(v_cache, kv_dtype, voff + d);
            }
            for (int64_t d = 0; d < D; d++)
                out[qoff + d] = nkeys ? v_scale * acc[d] / denom : 0.0;
        }
    }
    free(logit);
    free(slot);
    free(acc);
    return rc;
}

/*
 * Dense attention over every visible key of each query token, through a
 * separate path: the visible keys and values are first gathered into
 * contiguous arrays in position order, then a textbook softmax is applied.
 * With a selection holding every block it must agree with orc_sparse_decode.
 */
int orc_dense_attention(const void *q, int q_dtype, const void *k_cache, const void *v_cache,
                        int kv_dtype, const int32_t *block_table, const int32_t *seq_lens,
                        int64_t R, int64_t T, int64_t MB, int64_t P, int64_t B,
                        int64_t Hq, int64_t Hkv, int64_t D,
                        double sm_scale, double k_scale, double v_scale,
                        int64_t n_begin, int64_t n_end, double *out)
{
    if (T < 1 || B < 1 || D < 1 || Hkv < 1 || Hq % Hkv || n_begin < 0 || n_end > R * T)
        return ORC_EARG;
    if (check_lens(seq_lens, R, MB, B))
        return ORC_ELEN;
    int64_t G = Hq / Hkv;
    int64_t Lmax = MB * B;
    double *Kd = malloc(sizeof(double) * (size_t)(Lmax * D));
    double *Vd = malloc(sizeof(double) * (size_t)(Lmax * D));
    double *w = malloc(sizeof(double) * (size_t)Lmax);
    if (!Kd || !Vd || !w) { free(Kd); free(Vd); free(w); return ORC_EARG; }
    int rc = ORC_OK;
    for (int64_t n = n_begin; n < n_end && rc == ORC_OK; n++) {
        int64_t r = n / T;
        int64_t vis = visible(seq_lens, T, n);
        for (int64_t h = 0; h < Hq && rc == ORC_OK; h++) {
            int64_t g = h / G;
            for (int64_t s = 0; s < vis; s++) {
                int64_t page = block_table[r * MB + s / B];
                if (page < 0 || page >= P) { rc = ORC_EPAGE; break; }
                for (int64_t d = 0; d < D; d++) {
                    int64_t off = ((page * B + s % B) * Hkv + g) * D + d;
                    Kd[s * D + d] = k_scale * elem(k_cache, kv_dtype, off);
                    Vd[s * D + d] = v_scale * elem(v_cache, kv_dtype, off);
                }
            }
            if (rc != ORC_OK)
                break;
            double mx = -INFINITY, sum = 0.0;
            for (int64_t s = 0; s < vis; s++) {
                double dot = 0.0;
                for (int64_t d = 0; d < D; d++)
                    dot += elem(q, q_dtype, (n * Hq + h) * D + d) * Kd[s * D + d];
                w[s] = sm_scale * dot;
                mx = w[s] > mx ? w[s] : mx;
            }
            for (int64_t s = 0; s < vis; s++) {
                w[s] = exp(w[s] - mx);
                sum += w[s];
            }
            for (int64_t d = 0; d < D; d++) {
                double o = 0.0;
                for (int64_t s = 0; s < vis; s++)
                    o += (w[s] / sum) * Vd[s * D + d];
                out[(n * Hq + h) * D + d] = vis ? o : 0.0;
            }
        }
    }
    free(Kd);
    free(Vd);
    free(w);
    return rc;
}
