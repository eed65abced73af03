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
// Three launches on the caller's stream, no host synchronisation:
//  1. plan (one workgroup): cuts the batch into chunks of (token, head)
//     columns of one request (kPrefillCols at most) and each chunk's visible
//     blocks into units of G consecutive blocks, with G chosen from the live
//     totals so that the units fill the CUs evenly; writes the chunk and unit
//     tables and the owner of every query-block row to the workspace.
//  2. scoring (one persistent workgroup per CU): each unit is one
//     prefill_tile (MFMA over LDS-staged bf16 pages) followed by the max over
//     each query block's tokens, written to the [Hq, all_qb, NP, MB] sheet in
//     the workspace.  Consecutive units (same chunk, then neighbouring chunks
//     of one request) run on one XCD so that they share its L2.
//  3. selection (one wave per (head, query-block row)): forced blocks become
//     the largest keys, the others their order-preserving score keys, and the
//     wave-level radix select of select_unit.h takes the topk.
#include "device_util.h"
#include "msa_internal.h"
#include "prefill_tile.h"
#include "select_unit.h"

namespace msa {

namespace {

constexpr int kPlanThreads = 1024;

// keys visible to query block qb of a request: min(seq, prefix + qb*bsq),
// never below 0 (seqc is already clamped to [0, MB*B])
__device__ __forceinline__ int qb_visible(int seqc, int pre, int64_t qb, int64_t bsq) {
    const int64_t v = min((int64_t)pre + qb * bsq, (int64_t)seqc);
    return (int)max(v, (int64_t)0);
}

__device__ __forceinline__ int ld(const int32_t *a, int64_t s, int64_t i) { return a[i * s]; }

// exclusive prefix sum over the kPlanThreads threads of the workgroup; total
// gets the sum of all.  wsum: 16 ints of LDS.
__device__ __forceinline__ int block_excl_scan(int x, int *wsum, int &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int inc = wave_prefix_sum(x);
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kPlanThreads / 64; ++w) {
        const int v = wsum[w];
        base += w < wave ? v : 0;
        tot += v;
    }
    __syncthreads();                                   // wsum is reused by the next scan
    total = tot;
    return base + inc - x;
}

__global__ __launch_bounds__(kPlanThreads) void prefill_plan_kernel(PrefillSelParams p) {
    __shared__ int cs[kPlanMaxBatch + 1];              // first chunk of each request
    __shared__ int wsum[kPlanThreads / 64];
    __shared__ int gsum[8][kPlanThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const PrefillGeom g = p.g;
    const int64_t bsq = p.bsq;
    const int per_qc = g.HG * g.NP;                   // chunks per group of nqc query blocks

    for (int r = tid; r < p.all_qb; r += kPlanThreads) p.rowinfo[r] = -1;

    // chunks per request, prefix-summed into cs
    int run = 0;
    for (int base = 0; base < p.batch; base += kPlanThreads) {
        const int b = base + tid;
        int n = 0;
        if (b < p.batch) {
            const int nqb = min(max(ld(p.cu_qb, p.s_cq, b + 1) - ld(p.cu_qb, p.s_cq, b), 0), p.all_qb);
            n = (nqb + g.nqc - 1) / g.nqc * per_qc;
        }
        int tot;
        const int ex = block_excl_scan(n, wsum, tot);
        if (b < p.batch) cs[b] = run + ex;
        run += tot;
    }
    const int C = (int)min((int64_t)run, g.Cmax);
    if (tid == 0) cs[p.batch] = run;
    __syncthreads();                                   // cs complete, rowinfo cleared

    // chunk descriptors; units per chunk for every G in 1..8
    int ucount[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int c = tid; c < C; c += kPlanThreads) {
        // the request: the last b with cs[b] <= c (it has cs[b+1] > c)
        int lo = 0, hi = p.batch - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (cs[mid] <= c) lo = mid; else hi = mid - 1;
        }
        const int b = lo, k = c - cs[b];
        const int qc = k / per_qc, rem = k - qc * per_qc, hg = rem / g.NP, part = rem - hg * g.NP;
        const int q0 = ld(p.cu_seqlens, p.s_cu, b);
        const int nq = max(0, ld(p.cu_seqlens, p.s_cu, b + 1) - q0);
        const int row0 = ld(p.cu_qb, p.s_cq, b);
        const int nqb = min(max(ld(p.cu_qb, p.s_cq, b + 1) - row0, 0), p.all_qb);
        const int seqc = min(max(ld(p.seq_lens, p.s_sl, b), 0), p.MB * kBlock);
        const int pre = ld(p.prefix_lens, p.s_pl, b);
        const int slot = ld(p.slot_ids, p.s_slot, b);
        const int64_t qstart = (int64_t)qc * g.nqc * bsq;
        const int64_t tok0 = qstart + (int64_t)part * kPrefillCols;
        int64_t tok1 = qstart + min((int64_t)g.nqc * bsq, (int64_t)(part + 1) * kPrefillCols);
        tok1 = min(tok1, min((int64_t)nq, (int64_t)nqb * bsq));
        const int ntok = (int)max(tok1 - tok0, (int64_t)0);
        const int lp = ntok > 0 ? (qb_visible(seqc, pre, (tok1 - 1) / bsq, bsq) + kBlock - 1) / kBlock : 0;
        p.chunks[3 * (int64_t)c] = make_int4(slot, (int)min((int64_t)q0 + tok0, (int64_t)0x7fffffff), ntok,
                                             hg * g.hc);
        p.chunks[3 * (int64_t)c + 1] = make_int4((int)min(tok0, (int64_t)0x7fffffff), seqc, pre, row0);
        p.chunks[3 * (int64_t)c + 2] = make_int4(part, lp, 0, 0);
#pragma unroll
        for (int G = 1; G <= 8; ++G) ucount[G - 1] += (lp + G - 1) / G;
        if (hg == 0 && part == 0)
            for (int qb = qc * g.nqc; qb < min(nqb, qc * g.nqc + g.nqc); ++qb)
                if (row0 + qb >= 0 && row0 + qb < p.all_qb) p.rowinfo[row0 + qb] = b;
    }

    // G: fewest rounds of units over the workgroups, each round priced at G
    // pages plus the fixed cost of a unit (its queries, its first pages'
    // latency), about 1.5 pages
#pragma unroll
    for (int G = 0; G < 8; ++G) {
        int v = ucount[G];
        v += __shfl_xor(v, 1); v += __shfl_xor(v, 2); v += __shfl_xor(v, 4);
        v += __shfl_xor(v, 8); v += __shfl_xor(v, 16); v += __shfl_xor(v, 32);
        if (lane == 0) gsum[G][wave] = v;
    }
    __syncthreads();
    int G = 8;
    int64_t best = -1;
    for (int c = 1; c <= 8; ++c) {
        int64_t L = 0;
        for (int w = 0; w < kPlanThreads / 64; ++w) L += gsum[c - 1][w];
        if (L > g.Umax) continue;
        const int64_t cost = (L + p.nwg - 1) / p.nwg * (2 * c + 3);
        if (best < 0 || cost <= best) { best = cost; G = c; }
    }

    // unit table: chunk c's units are consecutive, in block order
    run = 0;
    for (int base = 0; base < C; base += kPlanThreads) {
        const int c = base + tid;
        const int lp = c < C ? p.chunks[3 * (int64_t)c + 2].y : 0;   // written by this thread above
        const int n = (lp + G - 1) / G;
        int tot;
        const int ex = block_excl_scan(n, wsum, tot);
        for (int i = 0; i < n; ++i) {
            const int64_t u = (int64_t)run + ex + i;
            if (u < g.Umax) p.units[u] = make_int4(c, i * G, min(G, lp - i * G), 0);
        }
        run += tot;
    }
    if (tid == 0) {
        p.hdr[0] = (int)min((int64_t)run, g.Umax);
        p.hdr[1] = G;
        p.hdr[2] = C;
    }
}

template <int DI>
__global__ __launch_bounds__(64 * kPWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_score_ragged_kernel(PrefillSelParams p) {
    constexpr int QT = kPrefillCols / (16 * kPWaves);
    constexpr int NT = 64 * kPWaves;
    static_assert(PrefillLds<DI, QT>::PQ == kPrefillCols, "chunk columns = tile columns");
    __shared__ PrefillLds<DI, QT> lds;
    const int tid = threadIdx.x, lane = tid & 63;
    const int L = p.hdr[0];
    // XCD x (= blockIdx % 8) takes the units [x*per, (x+1)*per) of every
    // round of nwg units
    const int per = p.nwg / 8;
    const int first = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
    const int hc = p.g.hc, NP = p.g.NP;
    const int64_t bsq = p.bsq;
    for (int u = first; u < L; u += p.nwg) {
        const int4 un = p.units[u];
        const int4 d0 = p.chunks[3 * (int64_t)un.x], d1 = p.chunks[3 * (int64_t)un.x + 1];
        const int part = p.chunks[3 * (int64_t)un.x + 2].x;
        const int slot = d0.x, qrow0 = max(d0.y, 0), ntok = d0.z, h0 = d0.w;
        const int tok0 = d1.x, seqc = d1.y, pre = d1.z, row0 = d1.w;
        const int qbf = (int)(tok0 / bsq), qbl = (int)((tok0 + ntok - 1) / bsq);
        PrefillPages pg;
        pg.index_k = p.index_k; pg.k_sp = p.k_sp; pg.k_sb = p.k_sb; pg.P = p.P;
        pg.bt_row = (slot >= 0 && slot < p.nslots) ? p.bt + (int64_t)slot * p.bt_sr : nullptr;
        pg.bt_sj = p.bt_sj;
        pg.j0 = un.y; pg.npg = un.z;
        pg.vmin = qb_visible(seqc, pre, qbf, bsq);
        pg.vmax = qb_visible(seqc, pre, qbl, bsq);
        pg.scale = p.scale;
        // column col = (token tok0 + col / hc, head h0 + col % hc); columns
        // past the chunk read its last valid row and see no key
        auto qrow = [&](int col) {
            const int tl = col / hc, hl = col - tl * hc;
            const int t = min(ntok - 1, tl), h = min(p.Hq - 1, h0 + hl);
            const int64_t row = min((int64_t)p.total_q - 1, (int64_t)qrow0 + t);
            return p.q + row * p.q_st + (int64_t)h * p.q_sh;
        };
        auto vis = [&](int col) {
            const int tl = col / hc, hl = col - tl * hc;
            if (tl >= ntok || h0 + hl >= p.Hq) return 0;
            return qb_visible(seqc, pre, (tok0 + tl) / bsq, bsq);
        };
        prefill_tile<DI, QT>(pg, qrow, vis, lds);

        // max over each query block's tokens: output (query block qbf + o /
        // hc, head h0 + o % hc) x block j0 + pi, S lanes per pair
        const int npg = pg.npg, O = (qbl - qbf + 1) * hc, NPR = O * npg;
        int S = 64;
        while (S > 1 && NPR * S > NT) S >>= 1;
        const int sub = lane & (S - 1);
        for (int pr = tid / S; pr < NPR; pr += NT / S) {
            const int o = pr / npg, pi = pr - o * npg;
            const int ql = o / hc, hl = o - ql * hc;
            const int64_t qb = qbf + ql;
            const int t_lo = (int)(max((int64_t)tok0, qb * bsq) - tok0);
            const int t_hi = (int)(min((int64_t)tok0 + ntok, (qb + 1) * bsq) - tok0);
            float m = -INFINITY;
            for (int t = t_lo + sub; t < t_hi; t += S) m = fmaxf(m, lds.sbuf[t * hc + hl][pi]);
            for (int off = S >> 1; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
            const int h = h0 + hl;
            const int64_t row = row0 + qb;
            if (sub == 0 && h < p.Hq && row >= 0 && row < p.all_qb)
                p.ws[(((int64_t)h * p.all_qb + row) * NP + part) * p.MB + pg.j0 + pi] = m;
        }
        __syncthreads();                               // sbuf and the page buffers are reused
    }
}

template <int KPL>
__global__ __launch_bounds__(256) void prefill_select_kernel(PrefillSelParams p) {
    __shared__ __attribute__((aligned(16))) int hist[4][256];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t rowid = (int64_t)blockIdx.x * 4 + wave;
    if (rowid >= (int64_t)p.Hq * p.all_qb) return;    // no barriers in this kernel
    const int h = (int)(rowid / p.all_qb), g = (int)(rowid - (int64_t)h * p.all_qb);
    int32_t *dst = p.out + (int64_t)h * p.o_sh + (int64_t)g * p.o_sq;
    const int b = p.rowinfo[g];
    if (b < 0) {
        for (int i = lane; i < p.topk; i += 64) dst[(int64_t)i * p.o_si] = -1;
        return;
    }
    const int64_t bsq = p.bsq;
    const int qb = g - ld(p.cu_qb, p.s_cq, b);
    const int nq = ld(p.cu_seqlens, p.s_cu, b + 1) - ld(p.cu_seqlens, p.s_cu, b);
    const int seqc = min(max(ld(p.seq_lens, p.s_sl, b), 0), p.MB * kBlock);
    const int V = qb_visible(seqc, ld(p.prefix_lens, p.s_pl, b), qb, bsq);
    const int ncand = (V + kBlock - 1) / kBlock;
    // parts of the query block that hold tokens (more than one only when
    // block_size_q exceeds a chunk)
    const int64_t ntq = min(bsq, (int64_t)nq - qb * bsq);
    const int npv = max(1, min(p.g.NP, (int)((ntq + kPrefillCols - 1) / kPrefillCols)));
    const float *src = p.ws + ((int64_t)h * p.all_qb + g) * p.g.NP * p.MB;
    uint32_t key[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const int j = i * 64 + lane;
        key[i] = 0u;
        if (j < ncand) {
            float s = src[j];
            for (int q = 1; q < npv; ++q) s = fmaxf(s, src[(int64_t)q * p.MB + j]);
            const bool forced = j < p.init_blocks || j >= ncand - p.local_blocks;
            key[i] = forced ? 0xffffffffu : score_key(s);
        }
    }
    select_keys<KPL>(key, p.topk, hist[wave], [&](int pos, int id) { dst[(int64_t)pos * p.o_si] = id; });
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
    g.Umax = 2 * g.Cmax * ((MB + kPMaxPC - 1) / kPMaxPC);
    return g;
}

namespace {
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
}  // namespace

size_t prefill_workspace_bytes(int64_t batch, int64_t Hq, int64_t all_qb, int64_t MB, int64_t bsq) {
    const PrefillGeom g = prefill_geom(batch, Hq, all_qb, MB, bsq);
    return 256 + align256(4 * (size_t)all_qb) + align256(48 * (size_t)g.Cmax) + align256(16 * (size_t)g.Umax) +
           align256(4 * (size_t)(Hq * all_qb * g.NP * MB));
}

void prefill_carve_workspace(void *ws, int64_t batch, int64_t Hq, int64_t all_qb, int64_t MB, int64_t bsq,
                             PrefillSelParams &p) {
    p.g = prefill_geom(batch, Hq, all_qb, MB, bsq);
    uint8_t *b = (uint8_t *)ws;
    p.hdr = (int32_t *)b;
    b += 256;
    p.rowinfo = (int32_t *)b;
    b += align256(4 * (size_t)all_qb);
    p.chunks = (int4 *)b;
    b += align256(48 * (size_t)p.g.Cmax);
    p.units = (int4 *)b;
    b += align256(16 * (size_t)p.g.Umax);
    p.ws = (float *)b;
}

hipError_t launch_prefill_select(const PrefillSelParams &p, int Di, hipStream_t s) {
    if ((int64_t)p.Hq * p.all_qb == 0) return hipSuccess;
    hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (Di == 128)
        hipLaunchKernelGGL(prefill_score_ragged_kernel<128>, dim3(p.nwg), dim3(64 * kPWaves), 0, s, p);
    else
        hipLaunchKernelGGL(prefill_score_ragged_kernel<64>, dim3(p.nwg), dim3(64 * kPWaves), 0, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (p.MB <= 64) return launch_select<1>(p, s);
    if (p.MB <= 128) return launch_select<2>(p, s);
    if (p.MB <= 256) return launch_select<4>(p, s);
    if (p.MB <= 512) return launch_select<8>(p, s);
    if (p.MB <= 1024) return launch_select<16>(p, s);
    if (p.MB <= 2048) return launch_select<32>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace msa
