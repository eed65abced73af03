// Ragged prefill score-to-selection: Cacheon "Kernel ABI", "Attention block
// slots", attention.msa_prefill_block_score.  For every request b of a
// ragged batch, query head h and query block qb of the request's new tokens:
// the blocks that can be selected are the logical blocks holding keys before
// position V = min(seq_lens[b], prefix_lens[b] + qb * block_size_q); block j
// scores scale * max over the block's tokens t and the visible keys s of block
// j of q[t][h] . index_k[s]; the first init_blocks and the last local_blocks of
// those blocks are taken first (lower ids first), the rest by score with ties
// to the lower id; ids are written ascending into out_topk[h][row(b, qb)] and
// padded with -1, and rows no request owns are all -1.
//
// Two launches on the caller's stream, no host synchronisation:
//  1. scoring (one persistent workgroup per CU).  The work is cut into chunks
//     of (token, head) columns of one request (kPrefillCols at most, whole
//     query blocks where they fit), and each chunk into its visible blocks
//     ("pages"), in the order request, query-block group, head group, part.
//     Every workgroup first derives the page count of every request from the
//     offsets alone (a prologue over the batch, in LDS), then takes the
//     contiguous page range [r*T/nwg, (r+1)*T/nwg) of the T pages: the shares
//     differ by at most one page whatever the mix of lengths.  It walks its
//     range in tiles of at most kPMaxPC pages of one chunk (prefill_tile: MFMA
//     over LDS-staged bf16 pages) and reduces each tile to the max over each
//     query block's tokens, written to the [Hq, all_qb, NP, MB] sheet in the
//     workspace.  XCD x holds the ranges of 1/8 of the pages, so neighbouring
//     chunks of one request (same pages) and the tiles of one chunk (same
//     queries) share its L2.  The prologue also records which request owns
//     each query-block row.
//  2. selection (one wave per (head, query-block row)): forced blocks become
//     the largest keys, the others their order-preserving score keys, and the
//     wave-level radix select of select_unit.h takes the topk.
#include "device_util.h"
#include "msa_internal.h"
#include "prefill_tile.h"
#include "select_unit.h"

namespace msa {

namespace {

// keys visible to query block qb of a request: min(seq, prefix + qb*bsq),
// never below 0 (seqc is already clamped to [0, MB*B])
__device__ __forceinline__ int qb_visible(int seqc, int pre, int64_t qb, int64_t bsq) {
    const int64_t v = min((int64_t)pre + qb * bsq, (int64_t)seqc);
    return (int)max(v, (int64_t)0);
}

__device__ __forceinline__ int ld(const int32_t *a, int64_t s, int64_t i) { return a[i * s]; }

// the query-block sheet is written and read with device-coherent (agent
// scope) accesses: the workgroup that selects a group's rows reads what the
// other workgroups of the launch wrote, possibly on another XCD
__device__ __forceinline__ void st_sheet(float *a, float v) {
    __hip_atomic_store((uint32_t *)a, __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_sheet(const float *a) {
    return __uint_as_float(__hip_atomic_load((const uint32_t *)a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// exclusive prefix sum over the NT threads of the workgroup; total gets the
// sum of all.  wsum: NT/64 ints of LDS.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int x, int *wsum, int &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int inc = wave_prefix_sum(x);
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const int v = wsum[w];
        base += w < wave ? v : 0;
        tot += v;
    }
    __syncthreads();                                   // wsum is reused by the next scan
    total = tot;
    return base + inc - x;
}

// what the kernels read of request b
struct Req {
    int q0, nq, nqb, row0, seqc, pre, slot;
    int nqcs;      // query-block groups: ceil(nqb / nqc)
};

__device__ __forceinline__ Req load_req(const PrefillSelParams &p, int b) {
    Req r;
    r.q0 = ld(p.cu_seqlens, p.s_cu, b);
    r.nq = max(0, ld(p.cu_seqlens, p.s_cu, b + 1) - r.q0);
    r.row0 = ld(p.cu_qb, p.s_cq, b);
    r.nqb = min(max(ld(p.cu_qb, p.s_cq, b + 1) - r.row0, 0), p.all_qb);
    r.seqc = min(max(ld(p.seq_lens, p.s_sl, b), 0), p.MB * kBlock);
    r.pre = ld(p.prefix_lens, p.s_pl, b);
    r.slot = ld(p.slot_ids, p.s_slot, b);
    r.nqcs = (r.nqb + p.g.nqc - 1) / p.g.nqc;
    return r;
}

// tokens [tok0, tok1) of chunk (query-block group qc, part) of a request
__device__ __forceinline__ void chunk_tokens(const PrefillSelParams &p, const Req &r, int qc, int part,
                                             int64_t &tok0, int64_t &tok1) {
    const int64_t bsq = p.bsq, qstart = (int64_t)qc * p.g.nqc * bsq;
    tok0 = qstart + (int64_t)part * kPrefillCols;
    tok1 = qstart + min((int64_t)p.g.nqc * bsq, (int64_t)(part + 1) * kPrefillCols);
    tok1 = min(tok1, min((int64_t)r.nq, (int64_t)r.nqb * bsq));
}

// pages of a chunk: the blocks its last query block sees (0 for no tokens).
// Division-free (it runs once per chunk in every workgroup's prologue): the
// last query block of group qc is min(nqb, (qc+1)*nqc) - 1, and a part of a
// query block (NP > 1, nqc = 1) belongs to query block qc.
__device__ __forceinline__ int chunk_pages(const PrefillSelParams &p, const Req &r, int qc, int part) {
    const int64_t bsq = p.bsq;
    const int64_t tok0 = (int64_t)qc * p.g.nqc * bsq + (int64_t)part * kPrefillCols;
    if (tok0 >= min((int64_t)r.nq, (int64_t)r.nqb * bsq)) return 0;
    const int qbl = p.g.NP > 1 ? qc : min(r.nqb - 1, (qc + 1) * p.g.nqc - 1);
    return (qb_visible(r.seqc, r.pre, qbl, bsq) + kBlock - 1) / kBlock;
}

// The selection of row (head h, query block qb of request r, out_topk row g)
// from the query-block sheet: forced blocks become the largest keys, the other
// candidates their score keys, and the wave-level radix select takes topk.
// The sheet is read with device-coherent loads (it may have been written by
// other workgroups of the same launch).
template <int KPL>
__device__ __forceinline__ void select_prefill_row(const PrefillSelParams &p, const Req &r, int h, int g, int qb,
                                                   int *hist) {
    const int lane = threadIdx.x & 63;
    const int64_t bsq = p.bsq;
    int32_t *dst = p.out + (int64_t)h * p.o_sh + (int64_t)g * p.o_sq;
    const int V = qb_visible(r.seqc, r.pre, qb, bsq);
    const int ncand = (V + kBlock - 1) / kBlock;
    // parts of the query block that hold tokens (more than one only when
    // block_size_q exceeds a chunk)
    const int64_t ntq = min(bsq, (int64_t)r.nq - qb * bsq);
    const int npv = max(1, min(p.g.NP, (int)((ntq + kPrefillCols - 1) / kPrefillCols)));
    const float *src = p.ws + ((int64_t)h * p.all_qb + g) * p.g.NP * p.MB;
    uint32_t key[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const int j = i * 64 + lane;
        key[i] = 0u;
        if (j < ncand) {
            float s = ld_sheet(src + j);
            for (int q = 1; q < npv; ++q) s = fmaxf(s, ld_sheet(src + (int64_t)q * p.MB + j));
            const bool forced = j < p.init_blocks || j >= ncand - p.local_blocks;
            key[i] = forced ? 0xffffffffu : score_key(s);
        }
    }
    select_keys<KPL>(key, p.topk, hist, [&](int pos, int id) { dst[(int64_t)pos * p.o_si] = id; });
}

// out_topk rows of query block qb of request r for heads [h0, h1): -1
__device__ __forceinline__ void fill_rows_none(const PrefillSelParams &p, int g, int h0, int h1, int tid, int nt) {
    for (int i = tid; i < (h1 - h0) * p.topk; i += nt) {
        const int h = h0 + i / p.topk, k = i - (i / p.topk) * p.topk;
        p.out[(int64_t)h * p.o_sh + (int64_t)g * p.o_sq + (int64_t)k * p.o_si] = -1;
    }
}

// blocks per scoring tile: as many as LDS holds next to the four page
// buffers, so that most workgroups' shares are one tile
constexpr int kRaggedPC = 14;
// requests whose fields the prologue keeps in LDS (larger batches re-read them)
constexpr int kLdsReqs = 512;
// page buffers of a scoring workgroup: two groups of two pages, one barrier
// per pair (two 4-wave workgroups per CU with one page per barrier and
// 256-column chunks were measured slower: every page is staged per chunk)
constexpr int kRaggedBufs = 4;
// the fixed cost of a tile (queries and first pages on their way), in pages
constexpr int kRampWeight = 3;

template <int DI>
__global__ __launch_bounds__(64 * kPrefillWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_score_ragged_kernel(PrefillSelParams p) {
    constexpr int QT = kPrefillCols / (16 * kPrefillWaves);
    constexpr int NT = 64 * kPrefillWaves;
    using Lds = PrefillLds<DI, QT, kRaggedPC, kPrefillWaves, kRaggedBufs>;
    static_assert(Lds::PQ == kPrefillCols, "chunk columns = tile columns");
    static_assert(sizeof(Lds::kb) >= 4 * (kPlanMaxBatch + 4 + 8 * kLdsReqs), "prologue tables in the page buffers");
    __shared__ Lds lds;
    __shared__ int wsum[NT / 64];
    const int tid = threadIdx.x, lane = tid & 63;
    const PrefillGeom g = p.g;
    const int64_t bsq = p.bsq;
    // XCD x (= blockIdx % 8) holds the ranges x*nwg/8 .. (x+1)*nwg/8 - 1
    const int rng = (int)(blockIdx.x % 8) * (p.nwg / 8) + (int)(blockIdx.x / 8);
    // the rows of request rng (written at the end, read now)
    const int ri_row0 = rng < p.batch ? ld(p.cu_qb, p.s_cq, rng) : 0;
    const int ri_end = rng < p.batch ? ld(p.cu_qb, p.s_cq, rng + 1) : 0;
    const int rows_owned = ld(p.cu_qb, p.s_cq, p.batch);

    // weight of every request, prefix-summed into PS, and the request fields
    // for small batches, in the page buffers (before any page is staged).  A
    // chunk with pages weighs its pages plus kRampWeight, the cost of loading
    // its queries and first pages: shares that start a new chunk hold fewer
    // pages.
    int *PS = (int *)&lds.kb[0][0];
    int *RQ = PS + ((kPlanMaxBatch + 4) & ~3);          // 16-byte aligned
    const bool rq_lds = p.batch <= kLdsReqs;
    int run = 0;
    for (int base = 0; base < p.batch; base += NT) {
        const int b = base + tid;
        int n = 0;
        if (b < p.batch) {
            const Req r = load_req(p, b);
            for (int qc = 0; qc < r.nqcs; ++qc)
                for (int part = 0; part < g.NP; ++part) {
                    const int l = chunk_pages(p, r, qc, part);
                    n += l ? l + kRampWeight : 0;
                }
            n *= g.HG;
            if (rq_lds) {
                *(int4 *)(RQ + 8 * b) = make_int4(r.q0, r.nq, r.nqb, r.row0);
                *(int4 *)(RQ + 8 * b + 4) = make_int4(r.seqc, r.pre, r.slot, r.nqcs);
            }
        }
        int tot;
        const int ex = block_excl_scan<NT>(n, wsum, tot);
        if (b < p.batch) PS[b] = run + ex;
        run += tot;
    }
    __syncthreads();                                   // PS and RQ complete
    auto req_lds = [&](int b) {
        if (!rq_lds) return load_req(p, b);
        const int4 a = *(const int4 *)(RQ + 8 * b), c = *(const int4 *)(RQ + 8 * b + 4);
        Req r;
        r.q0 = __builtin_amdgcn_readfirstlane(a.x); r.nq = __builtin_amdgcn_readfirstlane(a.y);
        r.nqb = __builtin_amdgcn_readfirstlane(a.z); r.row0 = __builtin_amdgcn_readfirstlane(a.w);
        r.seqc = __builtin_amdgcn_readfirstlane(c.x); r.pre = __builtin_amdgcn_readfirstlane(c.y);
        r.slot = __builtin_amdgcn_readfirstlane(c.z); r.nqcs = __builtin_amdgcn_readfirstlane(c.w);
        return r;
    };
    // The share is the weight range [w0, w1).  A weight position w falls in
    // the chunk whose range [cum, cum + pages + kRampWeight) holds it, at page
    // max(0, w - cum - kRampWeight); the share takes the pages from the
    // position of w0 up to that of w1, so every page goes to exactly one share.
    const int W = run;
    const int w0 = (int)((int64_t)rng * W / p.nwg), w1 = (int)((int64_t)(rng + 1) * W / p.nwg);
    const int per_qc = g.HG * g.NP;                    // chunks per query-block group
    int b = 0, qc = 0, hg = 0, part = 0, lp = 0, j = 0;
    int cum = 0;                                       // weight position of the current chunk
    Req rq{};
    bool have = false;                                 // a current chunk
    // (a share with no weight still locates the chunk at its position: it
    // arrives at that chunk's group without work, see below)
    if (w0 < W) {
        // the request holding w0 (the last b with PS[b] <= w0), then its chunk
        // holding w0: the request's chunk weights prefix-summed across a wave,
        // 64 chunks at a time
        int lo = 0, hi = p.batch - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (PS[mid] <= w0) lo = mid; else hi = mid - 1;
        }
        b = __builtin_amdgcn_readfirstlane(lo);
        const int psb = __builtin_amdgcn_readfirstlane(PS[b]);
        const int off = w0 - psb;
        rq = req_lds(b);
        const int nch = rq.nqcs * per_qc;
        int base = 0;
        for (int kb = 0; kb < nch; kb += 64) {
            const int k = kb + lane;
            int wt = 0;
            if (k < nch) {
                const int l = chunk_pages(p, rq, k / per_qc, k % g.NP);
                wt = l ? l + kRampWeight : 0;
            }
            const int inc = wave_prefix_sum(wt);
            const uint64_t m = __ballot(k < nch && base + inc > off);
            if (m) {
                const int L = __builtin_ctzll(m);
                const int k0 = kb + L;
                qc = k0 / per_qc;
                hg = (k0 - qc * per_qc) / g.NP;
                part = k0 % g.NP;
                cum = psb + base + __builtin_amdgcn_readlane(inc - wt, L);
                have = true;
                break;
            }
            base += __builtin_amdgcn_readlane(inc, 63);
        }
        if (have) {
            lp = chunk_pages(p, rq, qc, part);
            j = max(0, w0 - cum - kRampWeight);
        }
    }
    __syncthreads();                                   // the prologue tables are dead

    // next chunk of the batch, in chunk order (query-block group, head group,
    // part)
    auto advance = [&]() {
        if (++part == g.NP) {
            part = 0;
            if (++hg == g.HG) {
                hg = 0;
                ++qc;
            }
        }
        while (qc >= rq.nqcs) {                        // past the request's chunks
            if (++b >= p.batch) return false;
            rq = load_req(p, b);
            qc = hg = part = 0;
        }
        lp = chunk_pages(p, rq, qc, part);
        return true;
    };
    const int hc = g.hc;
    // Selection inside the launch (p.fused): a group (request, query-block
    // group, head group) is done when every share whose weight range meets
    // the group's has written its pages' maxima; each such share then adds
    // one to the group's counter, and the one that completes the count
    // selects the group's rows and clears the counter.  The number of such
    // shares follows from the weight positions alone: the shares whose range
    // starts inside [g0w, g1w), plus the one that holds g0w when g0w is not
    // a share start.
    auto seg_count = [&](int g0w, int g1w) {
        const int64_t n = p.nwg;
        const int64_t c0 = ((int64_t)g0w * n + W - 1) / W, c1 = ((int64_t)g1w * n + W - 1) / W;
        const bool start = c0 < n && (c0 * W / n) == g0w;
        return (int)(c1 - c0) + (start ? 0 : 1);
    };
    // weight range of the current chunk's group (its NP parts are
    // consecutive chunks)
    auto group_span = [&](int &g0w, int &g1w) {
        int before = 0, from = 0;
        for (int pp = 0; pp < g.NP; ++pp) {
            const int l = chunk_pages(p, rq, qc, pp);
            const int w = l ? l + kRampWeight : 0;
            if (pp < part) before += w; else from += w;
        }
        g0w = cum - before;
        g1w = cum + from;
    };
    __shared__ int s_last;
    auto arrive = [&](const Req &gr, int gqc, int ghg, int g0w, int g1w) {
        const int grow0 = gr.row0 + gqc * g.nqc;       // the group's first out_topk row
        if (grow0 < 0 || grow0 >= p.all_qb) return;   // (inconsistent offsets: nothing to select)
        const int gh0 = ghg * hc;
        int *ctr = p.counters + (int64_t)gh0 * p.all_qb + grow0;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this thread's sheet stores are done
        __syncthreads();
        if (tid == 0)
            s_last = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                     seg_count(g0w, g1w) - 1;
        __syncthreads();
        if (!s_last) return;
        const int wave = tid >> 6;
        const int qb0 = gqc * g.nqc, nqbg = min(gr.nqb, qb0 + g.nqc) - qb0;
        const int nh = min(p.Hq, gh0 + hc) - gh0;
        int *hist = (int *)&lds.kb[0][0] + 256 * wave;   // the page buffers are idle here
        for (int i = wave; i < nqbg * nh; i += kPrefillWaves) {
            const int ql = i / nh, h = gh0 + (i - ql * nh);
            if (grow0 + ql < p.all_qb) select_prefill_row<2>(p, gr, h, grow0 + ql, qb0 + ql, hist);
        }
        if (tid == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();                               // the page buffers are reused
    };
    while (have) {
        const int wt = lp + kRampWeight;               // lp > 0 here
        const bool last = w1 <= cum + wt;              // the share ends in this chunk
        const int jend = last ? min(lp, max(0, w1 - cum - kRampWeight)) : lp;
        for (; j < jend;) {
            const int n = min(kRaggedPC, jend - j);
            int64_t tok0l, tok1l;
            chunk_tokens(p, rq, qc, part, tok0l, tok1l);
            const int tok0 = (int)tok0l, ntok = (int)(tok1l - tok0l), h0 = hg * hc;
            const int qbf = tok0 / p.bsq, qbl = (int)(tok1l - 1) / p.bsq;   // token offsets fit in int
            const int64_t qrow0 = max((int64_t)rq.q0 + tok0l, (int64_t)0);
            const int seqc = rq.seqc, pre = rq.pre, row0 = rq.row0;
            PrefillPages pg;
            pg.index_k = p.index_k; pg.k_sp = p.k_sp; pg.k_sb = p.k_sb; pg.P = p.P;
            pg.bt_row = (rq.slot >= 0 && rq.slot < p.nslots) ? p.bt + (int64_t)rq.slot * p.bt_sr : nullptr;
            pg.bt_sj = p.bt_sj;
            pg.j0 = j; pg.npg = n;
            pg.vmin = qb_visible(seqc, pre, qbf, bsq);
            pg.vmax = qb_visible(seqc, pre, qbl, bsq);
            pg.scale = p.scale;
            // column col = (token tok0 + col / hc, head h0 + col % hc); columns
            // past the chunk read its last valid row and see no key
            auto qrow = [&](int col) {
                const int tl = col / hc, hl = col - tl * hc;
                const int t = min(ntok - 1, tl), h = min(p.Hq - 1, h0 + hl);
                const int64_t row = min((int64_t)p.total_q - 1, qrow0 + t);
                return p.q + row * p.q_st + (int64_t)h * p.q_sh;
            };
            auto vis = [&](int col) {
                const int tl = col / hc, hl = col - tl * hc;
                if (tl >= ntok || h0 + hl >= p.Hq) return 0;
                return qb_visible(seqc, pre, (tok0 + tl) / p.bsq, bsq);
            };
            prefill_tile<DI, QT, kRaggedPC>(pg, qrow, vis, lds);

            // max over each query block's tokens: output (query block qbf + o /
            // hc, head h0 + o % hc) x block j + pi, S lanes per pair
            const int O = (qbl - qbf + 1) * hc, NPR = O * n;
            int S = 64;
            while (S > 1 && NPR * S > NT) S >>= 1;
            const int sub = lane & (S - 1);
            for (int pr = tid / S; pr < NPR; pr += NT / S) {
                const int o = pr / n, pi = pr - o * n;
                const int ql = o / hc, hl = o - ql * hc;
                const int64_t qb = qbf + ql;
                const int t_lo = (int)(max((int64_t)tok0, qb * bsq) - tok0);
                const int t_hi = (int)(min((int64_t)tok0 + ntok, (qb + 1) * bsq) - tok0);
                float m = -INFINITY;
                for (int t = t_lo + sub; t < t_hi; t += S) m = fmaxf(m, lds.sbuf[t * hc + hl][pi]);
                for (int o2 = S >> 1; o2 >= 1; o2 >>= 1) m = fmaxf(m, __shfl_xor(m, o2));
                const int h = h0 + hl;
                const int64_t row = row0 + qb;
                if (sub == 0 && h < p.Hq && row >= 0 && row < p.all_qb)
                    st_sheet(p.ws + (((int64_t)h * p.all_qb + row) * g.NP + part) * p.MB + j + pi, m);
            }
            __syncthreads();                               // sbuf and the page buffers are reused
            j += n;
        }
        int g0w = 0, g1w = 0;
        if (p.fused) group_span(g0w, g1w);
        if (last) {
            if (p.fused) arrive(rq, qc, hg, g0w, g1w);
            break;
        }
        const Req grq = rq;
        const int gb = b, gqc = qc, ghg = hg;
        cum += wt;                                     // next chunk that has pages
        do {
            have = advance();
        } while (have && lp == 0);
        j = 0;
        if (p.fused && (!have || b != gb || qc != gqc || hg != ghg))   // left the group
            arrive(grq, gqc, ghg, g0w, g1w);
    }

    // owners of the query-block rows: requests rng, rng + nwg, ...; -1 for
    // the rows past the last request's
    for (int bb = rng; bb < p.batch; bb += p.nwg) {
        const int row0 = bb == rng ? ri_row0 : ld(p.cu_qb, p.s_cq, bb);
        const int rend = bb == rng ? ri_end : ld(p.cu_qb, p.s_cq, bb + 1);
        for (int r = row0 + tid; r < rend; r += NT)
            if (r >= 0 && r < p.all_qb) p.rowinfo[r] = bb;
    }
    for (int r = max(rows_owned, 0) + rng * NT + tid; r < p.all_qb; r += p.nwg * NT) p.rowinfo[r] = -1;
    if (!p.fused) return;
    // rows that no share selects: groups without pages (every query block
    // sees no key) and rows past the last request's
    for (int bb = rng; bb < p.batch; bb += p.nwg) {
        const Req r = load_req(p, bb);
        for (int gq = 0; gq < r.nqcs; ++gq) {
            int w = 0;
            for (int pp = 0; pp < g.NP; ++pp) w += chunk_pages(p, r, gq, pp);
            if (w) continue;
            for (int q = gq * g.nqc; q < min(r.nqb, gq * g.nqc + g.nqc); ++q)
                if (r.row0 + q >= 0 && r.row0 + q < p.all_qb) fill_rows_none(p, r.row0 + q, 0, p.Hq, tid, NT);
        }
    }
    for (int r = max(rows_owned, 0) + rng; r < p.all_qb; r += p.nwg) fill_rows_none(p, r, 0, p.Hq, tid, NT);
}

template <int KPL>
__global__ __launch_bounds__(256) void prefill_select_kernel(PrefillSelParams p) {
    __shared__ __attribute__((aligned(16))) int hist[4][256];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t rowid = (int64_t)blockIdx.x * 4 + wave;
    if (rowid >= (int64_t)p.Hq * p.all_qb) return;    // no barriers in this kernel
    const int h = (int)(rowid / p.all_qb), g = (int)(rowid - (int64_t)h * p.all_qb);
    const int b = p.rowinfo[g];
    if (b < 0 || b >= p.batch) {
        fill_rows_none(p, g, h, h + 1, lane, 64);
        return;
    }
    const Req r = load_req(p, b);
    select_prefill_row<KPL>(p, r, h, g, g - r.row0, hist[wave]);
}

template <int KPL>
hipError_t launch_select(const PrefillSelParams &p, hipStream_t s) {
    const int64_t rows = (int64_t)p.Hq * p.all_qb;
    hipLaunchKernelGGL((prefill_select_kernel<KPL>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace

PrefillGeom prefill_geom(int64_t batch, int64_t Hq, int64_t all_qb, int64_t MB, int64_t bsq) {
    PrefillGeom g{};
    const int64_t PQ = kPrefillCols;
    if (bsq * Hq <= PQ) {
        g.hc = (int32_t)Hq; g.nqc = (int32_t)(PQ / (bsq * Hq)); g.NP = 1;
    } else if (bsq <= PQ) {
        g.hc = (int32_t)(PQ / bsq); g.nqc = 1; g.NP = 1;
    } else {
        g.hc = 1; g.nqc = 1; g.NP = (int32_t)((bsq + PQ - 1) / PQ);
    }
    g.HG = (int32_t)((Hq + g.hc - 1) / g.hc);
    g.Cmax = ((all_qb + g.nqc - 1) / g.nqc + batch) * g.HG * g.NP;
    g.Wmax = g.Cmax * (MB + kRampWeight);
    return g;
}

namespace {
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
}  // namespace

size_t prefill_workspace_bytes(int64_t batch, int64_t Hq, int64_t all_qb, int64_t MB, int64_t bsq) {
    const PrefillGeom g = prefill_geom(batch, Hq, all_qb, MB, bsq);
    return align256(4 * (size_t)(Hq * all_qb)) + align256(4 * (size_t)all_qb) +
           align256(4 * (size_t)(Hq * all_qb * g.NP * MB));
}

void prefill_carve_workspace(void *ws, int64_t batch, int64_t Hq, int64_t all_qb, int64_t MB, int64_t bsq,
                             PrefillSelParams &p) {
    p.g = prefill_geom(batch, Hq, all_qb, MB, bsq);
    // selection inside the scoring launch when a group's rows fit a few
    // selections per wave and a score row fits two keys per lane
    p.fused = MB <= 128 && (int64_t)p.g.nqc * p.g.hc <= 4 * kPrefillWaves;
    uint8_t *b = (uint8_t *)ws;
    p.counters = (int32_t *)b;
    b += align256(4 * (size_t)(Hq * all_qb));
    p.rowinfo = (int32_t *)b;
    b += align256(4 * (size_t)all_qb);
    p.ws = (float *)b;
}

hipError_t launch_prefill_select(const PrefillSelParams &p, int Di, hipStream_t s) {
    if ((int64_t)p.Hq * p.all_qb == 0) return hipSuccess;
    if (Di == 128)
        hipLaunchKernelGGL(prefill_score_ragged_kernel<128>, dim3(p.nwg), dim3(64 * kPrefillWaves), 0, s, p);
    else
        hipLaunchKernelGGL(prefill_score_ragged_kernel<64>, dim3(p.nwg), dim3(64 * kPrefillWaves), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.fused) return e;
    if (p.MB <= 64) return launch_select<1>(p, s);
    if (p.MB <= 128) return launch_select<2>(p, s);
    if (p.MB <= 256) return launch_select<4>(p, s);
    if (p.MB <= 512) return launch_select<8>(p, s);
    if (p.MB <= 1024) return launch_select<16>(p, s);
    if (p.MB <= 2048) return launch_select<32>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace msa
