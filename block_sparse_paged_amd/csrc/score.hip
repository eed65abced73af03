// Stage 1: block scores over the paged index cache.
//
// scores[n][j] = idx_scale * max over the keys s of block j visible to query
// token n of sum_d q_idx[n][d] * index_k[page(j)][s][d]   (-inf when none).
// Cacheon "Kernel ABI", "Attention block slots": attention.msa_block_score
// (decode score sheet) and attention.msa_prefill_block_score (prefill).
//
// Two kernels:
//  * score_valu  -- decode rows (T < 16 query tokens per row).  One wave per
//    (row, group of <= 4 tokens, block).  The wave streams the 128-token page
//    with coalesced 16-byte loads (8 lanes per 128-byte index row for FP8
//    Di=128), decodes FP8 in registers to bf16 and accumulates with
//    v_dot2_f32_bf16; the partial dots of a row are summed across its lanes
//    with DPP, masked by visibility and max-reduced.
//  * score_mfma  -- prefill rows (T >= 16).  A workgroup owns 128 query tokens
//    of one row and a run of blocks; each page is staged once in LDS (FP8,
//    XOR-swizzled) and every wave multiplies its 32 queries against it with
//    v_mfma_f32_16x16x32_bf16 after exact FP8 -> bf16 decoding.
#include "device_util.h"
#include "msa_internal.h"
#include "score_unit.h"

namespace msa {

namespace {



// ------------------------------------------------------------------ VALU path

template <bool QBF16, bool KFP8, int DI>
__global__ __launch_bounds__(256) void score_valu_kernel(ScoreParams p) {
    constexpr int ESZ = KFP8 ? 1 : 4;
    constexpr int ROWB = DI * ESZ;           // bytes per index row
    constexpr int LPT = ROWB / 16;           // lanes per token row
    constexpr int TPL = 64 / LPT;            // tokens per wave-wide load
    constexpr int NLOAD = kBlock / TPL;      // loads per page per lane
    constexpr int EPL = 16 / ESZ;            // elements per lane per load
    constexpr int CH = NLOAD < 16 ? NLOAD : 16;
    constexpr int TQ = kTokGroup;
    static_assert(LPT >= 1 && LPT <= 64 && (64 % LPT) == 0, "row size");

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int TG = (p.T + TQ - 1) / TQ;
    const int JC = (p.MB + 3) >> 2;
    int bid = blockIdx.x;
    const int jc = bid % JC;
    bid /= JC;
    const int tg = bid % TG;
    const int r = bid / TG;
    const int j = jc * 4 + wave;
    if (j >= p.MB) return;                   // no barriers below: a wave may leave

    const int t0 = tg * TQ;
    const int nt = min(TQ, p.T - t0);
    const int L = clamp_len(p.seq_lens[(int64_t)r * p.sl_s], p.MB);
    int vis[TQ];
#pragma unroll
    for (int t = 0; t < TQ; ++t) vis[t] = (t < nt) ? max(0, L - (p.T - 1 - (t0 + t))) : 0;
    const int vmax = max(0, L - (p.T - t0 - nt));   // the group's last token sees most
    const int64_t n0 = (int64_t)r * p.T + t0;

    float best[TQ];
#pragma unroll
    for (int t = 0; t < TQ; ++t) best[t] = -INFINITY;
    bool bad_page = false;

    if (j * kBlock < vmax) {
        const int pid = p.bt[(int64_t)r * p.bt_sr + (int64_t)j * p.bt_sj];
        if (pid < 0 || pid >= p.P) {
            bad_page = true;
        } else {
            const int dchunk = lane % LPT;
            const int grp = lane / LPT;
            // query fragments: elements [dchunk*EPL, +EPL) of each token's q_idx row
            constexpr int QW = (QBF16 && KFP8) ? EPL / 2 : EPL;   // words per token
            uint32_t qf[TQ][QW];
#pragma unroll
            for (int t = 0; t < TQ; ++t) {
                if (t < nt) {
                    const char *qrow = (const char *)p.q_idx +
                                       (n0 + t) * p.q_sn * (QBF16 ? 2 : 4);
                    if constexpr (QBF16 && KFP8) {
                        const uint4 *src = (const uint4 *)(qrow + dchunk * EPL * 2);
#pragma unroll
                        for (int w = 0; w < QW / 4; ++w) {
                            uint4 v = src[w];
                            qf[t][4 * w + 0] = v.x; qf[t][4 * w + 1] = v.y;
                            qf[t][4 * w + 2] = v.z; qf[t][4 * w + 3] = v.w;
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < EPL; ++e) {
                            float f;
                            if constexpr (QBF16)
                                f = __uint_as_float((uint32_t)((const uint16_t *)qrow)[dchunk * EPL + e] << 16);
                            else
                                f = ((const float *)qrow)[dchunk * EPL + e];
                            qf[t][e] = __float_as_uint(f);
                        }
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < QW; ++e) qf[t][e] = 0u;
                }
            }

            const char *page = (const char *)p.index_k + (int64_t)pid * p.k_sp * ESZ;
            const int kbase = j * kBlock;
#pragma unroll
            for (int c0 = 0; c0 < NLOAD; c0 += CH) {
                uint4 buf[CH];
#pragma unroll
                for (int i = 0; i < CH; ++i) {
                    const int s = (c0 + i) * TPL + grp;
                    buf[i] = *(const uint4 *)(page + (int64_t)s * p.k_sb * ESZ + dchunk * 16);
                }
#pragma unroll
                for (int i = 0; i < CH; ++i) {
                    const int s = (c0 + i) * TPL + grp;
                    float dot[TQ];
#pragma unroll
                    for (int t = 0; t < TQ; ++t) dot[t] = 0.f;
                    const uint32_t w4[4] = {buf[i].x, buf[i].y, buf[i].z, buf[i].w};
                    if constexpr (KFP8 && QBF16) {
#pragma unroll
                        for (int w = 0; w < 4; ++w) {
                            const bf16x2 k01 = __builtin_bit_cast(bf16x2, fp8x2_to_bf16x2<false>(w4[w]));
                            const bf16x2 k23 = __builtin_bit_cast(bf16x2, fp8x2_to_bf16x2<true>(w4[w]));
#pragma unroll
                            for (int t = 0; t < TQ; ++t) {
                                dot[t] = __builtin_amdgcn_fdot2_f32_bf16(
                                    k01, __builtin_bit_cast(bf16x2, qf[t][2 * w]), dot[t], false);
                                dot[t] = __builtin_amdgcn_fdot2_f32_bf16(
                                    k23, __builtin_bit_cast(bf16x2, qf[t][2 * w + 1]), dot[t], false);
                            }
                        }
                    } else if constexpr (KFP8) {
#pragma unroll
                        for (int w = 0; w < 4; ++w) {
                            const f32x2 a = fp8x2_to_f32x2<false>(w4[w]);
                            const f32x2 b = fp8x2_to_f32x2<true>(w4[w]);
#pragma unroll
                            for (int t = 0; t < TQ; ++t) {
                                dot[t] = fmaf(a.x, __uint_as_float(qf[t][4 * w + 0]), dot[t]);
                                dot[t] = fmaf(a.y, __uint_as_float(qf[t][4 * w + 1]), dot[t]);
                                dot[t] = fmaf(b.x, __uint_as_float(qf[t][4 * w + 2]), dot[t]);
                                dot[t] = fmaf(b.y, __uint_as_float(qf[t][4 * w + 3]), dot[t]);
                            }
                        }
                    } else {
#pragma unroll
                        for (int w = 0; w < 4; ++w) {
#pragma unroll
                            for (int t = 0; t < TQ; ++t)
                                dot[t] = fmaf(__uint_as_float(w4[w]), __uint_as_float(qf[t][w]), dot[t]);
                        }
                    }
                    const int pos = kbase + s;
#pragma unroll
                    for (int t = 0; t < TQ; ++t) {
                        const float d = group_sum<LPT>(dot[t]);
                        best[t] = (pos < vis[t]) ? fmaxf(best[t], d) : best[t];
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < TQ; ++t) best[t] = max_across_groups<LPT>(best[t]);
        }
    }
    if (lane < nt) {
        float v = best[0];
#pragma unroll
        for (int t = 1; t < TQ; ++t) v = (lane == t) ? best[t] : v;
        v = bad_page ? __builtin_nanf("") : v * p.idx_scale;
        p.scores[(n0 + lane) * p.sc_sn + (int64_t)j * p.sc_sj] = v;
    }
}

// ------------------------------------------------------------- MFMA decode path

template <int DI>
__global__ __launch_bounds__(256) void score_mfma_decode_kernel(ScoreParams p) {
    const int wave = threadIdx.x >> 6;
    const int JC = (p.MB + 3) >> 2;
    int r, jc;
    if (p.R >= 8) {
        // workgroup b runs on XCD b % 8: the row's workgroups all go to XCD r % 8,
        // where the attention workgroups of its tokens run (block table and
        // score row stay in that XCD's L2)
        const int x = blockIdx.x & 7, i = blockIdx.x >> 3;
        r = x + 8 * (i / JC);
        jc = i % JC;
        if (r >= p.R) return;
    } else {
        r = blockIdx.x / JC;
        jc = blockIdx.x % JC;
    }
    const int j = jc * 4 + wave;
    if (j >= p.MB) return;                      // no barriers in this kernel
    score_page<DI>(p, r, j);
}

// ------------------------------------------------------------------ MFMA path
//
// Prefill rows (T > 16): a GEMM per row, S = Q_r K_r^T over the row's visible
// keys, reduced to block maxima.  A workgroup of 8 waves (two per SIMD, one
// workgroup per CU) owns 128*QT query tokens of a row (16*QT per wave = QT
// MFMA column tiles of 16) and an even share of the blocks those tokens see
// (at most kPMaxPC consecutive ones); the tiles are laid out so that the
// workgroups of one query chunk run on one XCD.  The query rows are read
// coalesced and transposed into the MFMA operand layout through LDS.
//
// Each live page is read once per workgroup with coalesced 16-byte loads
// (every thread a 32-byte slice of a key row), decoded FP8 -> bf16 once and
// stored to a bf16 page buffer in LDS, from which all 8 waves read their A
// operands ready to use: the decode costs 16 VALU instructions per wave and
// page instead of one per MFMA, and VALU issue does not overlap MFMA issue
// well on a SIMD.  Pages go through LDS two at a time (four page buffers, one
// barrier per pair); the next pair's slices are loaded into registers while
// the current pair is multiplied, and decoded and stored after it.  Pages
// that every token sees whole skip the causal mask.  The running block max
// per (query, block) is staged in LDS and written out coalesced at the end.

constexpr int kPWaves = 8;        // waves per workgroup, two per SIMD
constexpr int kPMaxPC = 8;        // blocks per workgroup, at most
constexpr int kPTargetWGs = 256;  // workgroups aimed for (one per CU)

// max of three as IEEE maximum (v_maximum3_f32, no quieting of the operands
// first, unlike fmaxf); the operands are dot products, never NaN (a NaN dot
// product is outside the contract)
__device__ __forceinline__ float max3f(float a, float b, float c) {
    return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// bf16 A operands of the 16-key tile kt of the page in `buf`: key 16*kt +
// lane%16; k-step ks covers d = 32*ks .. +31, lane group grp its d = 32*ks +
// 8*grp .. +7: 16-byte unit 4*ks + grp of the key's bf16 row, stored
// XOR-swizzled by the key.
template <int DI>
__device__ __forceinline__ void prefill_frag(const uint8_t *buf, int kt, int li, int grp, uint4 (&a)[DI / 32]) {
    constexpr int KS = DI / 32, UPR = DI / 8;
    const int key = kt * 16 + li;
    const uint8_t *krow = buf + key * (DI * 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) a[ks] = *(const uint4 *)(krow + (((4 * ks + grp) ^ (key & (UPR - 1))) << 4));
}

// S^T tile of those keys against the wave's QT query tiles: acc[qt][e] =
// q . k for key 16*kt + 4*grp + e and query column lane%16.
template <int DI, int QT>
__device__ __forceinline__ void prefill_mma(const uint4 (&a)[DI / 32], const uint4 (&qf)[QT][DI / 32],
                                            f32x4 (&acc)[QT]) {
    constexpr int KS = DI / 32;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) acc[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
            acc[qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, a[ks]), __builtin_bit_cast(bf16x8, qf[qt][ks]), acc[qt], 0, 0, 0);
}

template <int DI, int QT>
__global__ __launch_bounds__(64 * kPWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void score_prefill_kernel(ScoreParams p, int WPC) {
    constexpr int KS = DI / 32;                 // MFMA k-steps per 16-key tile
    constexpr int NT = 64 * kPWaves;            // threads per workgroup
    constexpr int PQ = 16 * QT * kPWaves;       // query tokens per workgroup
    constexpr int RB = DI * 2;                  // bytes per bf16 row (query or key)
    constexpr int UPR = DI / 8;                 // 16-byte units per bf16 row
    constexpr int VPT = kBlock * DI / (16 * NT) > 0 ? kBlock * DI / (16 * NT) : 1;  // 16-byte FP8 loads per slice
    constexpr int TPK = DI / (16 * VPT);        // slices per key row
    constexpr int NLD = TPK * kBlock;           // threads holding a slice (whole waves)
    static_assert(NLD <= NT && NLD % 64 == 0 && TPK * 16 * VPT == DI, "page slicing");
    __shared__ __attribute__((aligned(16))) uint8_t kb[4][kBlock * RB];   // two pairs of pages
    __shared__ float sbuf[PQ][kPMaxPC + 1];
    static_assert(kPWaves * 16 * RB <= 2 * kBlock * RB, "query transpose area inside the first pair");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = lane >> 4, li = lane & 15;
    const int QC = (p.T + PQ - 1) / PQ;
    // Query chunk c = r*QC + qc has WPC workgroups, tiles u = c*WPC + w.
    // Workgroups are dispatched round-robin over the 8 XCDs (XCD = blockIdx %
    // 8), each with its own L2; XCD x runs the contiguous tile range [x*U8,
    // (x+1)*U8), so the workgroups of one query chunk (and of one row's pages)
    // share an L2 instead of every XCD fetching every chunk.
    const int U = p.R * QC * WPC, U8 = (U + 7) / 8;
    const int u = (int)(blockIdx.x % 8) * U8 + (int)(blockIdx.x / 8);
    if (u >= U) return;                                    // whole workgroup, before any barrier
    const int c = u / WPC, qc = c % QC, r = c / QC, w = u % WPC;
    const int L = clamp_len(p.seq_lens[(int64_t)r * p.sl_s], p.MB);
    const int tq0 = qc * PQ, tq1 = min(p.T, tq0 + PQ);
    const int vmin = max(0, L - (p.T - 1 - tq0));        // keys seen by the WG's first token
    const int vmax = max(0, L - (p.T - 1 - (tq1 - 1)));  // ... by its last
    const int64_t nrow = (int64_t)r * p.T;
    // Blocks the chunk's last token sees: 0 .. lp-1.  They are split evenly
    // over the chunk's workgroups (at most kPMaxPC each, by the choice of
    // WPC); blocks from lp on are seen by no token of the chunk: -inf, written
    // by workgroup w for every WPC-th of them.
    const int lp = min(p.MB, (vmax + kBlock - 1) / kBlock);
    const int j0 = (int)((int64_t)w * lp / WPC), npg = (int)((int64_t)(w + 1) * lp / WPC) - j0;
    for (int jd = lp + w; jd < p.MB; jd += WPC)
        for (int qq = tid; qq < tq1 - tq0; qq += NT)
            p.scores[(nrow + tq0 + qq) * p.sc_sn + (int64_t)jd * p.sc_sj] = -INFINITY;

    // page table of the share: lane i holds block j0 + i (npg <= 8 < 64)
    const int pid_l = lane < npg ? p.bt[(int64_t)r * p.bt_sr + (int64_t)(j0 + lane) * p.bt_sj] : -1;
    const bool vis_l = lane < npg && (j0 + lane) * kBlock < vmax;
    const bool ok_l = pid_l >= 0 && pid_l < p.P;
    uint64_t todo = __ballot(vis_l && ok_l);               // live pages, in block order
    auto next_live = [&]() {
        if (!todo) return -1;
        const int pi = __builtin_ctzll(todo);
        todo &= todo - 1;
        return pi;
    };
    // this thread's slice of a page (threads below NLD): key tid / TPK, bytes
    // 16*VPT*(tid % TPK) ..
    const int skey = tid / TPK, spart = tid % TPK;
    uint4 pv[2][VPT];                                      // the slices of the next pair of pages
    auto load_page = [&](int pi, uint4 (&v)[VPT]) {
        if (NLD < NT && tid >= NLD) return;
        const int pid = __builtin_amdgcn_readlane(pid_l, pi);
        const uint8_t *src = (const uint8_t *)p.index_k + (int64_t)pid * p.k_sp + (int64_t)skey * p.k_sb +
                             16 * VPT * spart;
#pragma unroll
        for (int h = 0; h < VPT; ++h) v[h] = *(const uint4 *)(src + 16 * h);
    };
    auto store_page = [&](const uint4 (&pv)[VPT], uint8_t *dst) {   // decode the slice to bf16 into dst
        if (NLD < NT && tid >= NLD) return;
        uint8_t *row = dst + skey * RB;
#pragma unroll
        for (int h = 0; h < VPT; ++h) {
            const int u0 = 2 * (VPT * spart + h);          // bf16 unit of the slice's first 8 codes
            uint4 lo, hi;
            lo.x = fp8x2_to_bf16x2<false>(pv[h].x); lo.y = fp8x2_to_bf16x2<true>(pv[h].x);
            lo.z = fp8x2_to_bf16x2<false>(pv[h].y); lo.w = fp8x2_to_bf16x2<true>(pv[h].y);
            hi.x = fp8x2_to_bf16x2<false>(pv[h].z); hi.y = fp8x2_to_bf16x2<true>(pv[h].z);
            hi.z = fp8x2_to_bf16x2<false>(pv[h].w); hi.w = fp8x2_to_bf16x2<true>(pv[h].w);
            *(uint4 *)(row + ((u0 ^ (skey & (UPR - 1))) << 4)) = lo;
            *(uint4 *)(row + (((u0 + 1) ^ (skey & (UPR - 1))) << 4)) = hi;
        }
    };
    // Pages go through LDS two at a time (one barrier per pair).  The first
    // pair is requested before the query rows: the other order was measured
    // to be far slower.
    int c0 = next_live(), c1 = next_live();
    if (c0 >= 0) load_page(c0, pv[0]);
    if (c1 >= 0) load_page(c1, pv[1]);

    // Query rows, read coalesced.  In the MFMA operand layout consecutive
    // lanes hold different query rows, and a global load in that layout
    // touches a separate cache line for every lane of a 4-lane quad, several
    // times slower than quads reading 64 contiguous bytes.  So each wave reads
    // its 16*QT rows with whole rows across consecutive lanes and transposes
    // them through 16 rows' worth of LDS of its own (below).  Columns past
    // the row's last token read that token again; their scores are never
    // stored, and no reduction mixes columns.
    constexpr int RPL = 64 / UPR;               // rows per coalesced load
    constexpr int LPT = 16 / RPL;               // loads per 16-row tile
    uint4 qraw[QT][LPT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int l = 0; l < LPT; ++l) {
            const int t = min(p.T - 1, tq0 + 16 * QT * wave + 16 * qt + l * RPL + lane / UPR);
            qraw[qt][l] = *(const uint4 *)((const uint16_t *)p.q_idx + (nrow + t) * p.q_sn + 8 * (lane % UPR));
        }

    // blocks without a live page: -inf for tokens that see none of their keys,
    // NaN for tokens that see keys of a block whose page id is out of range
    const uint64_t live = __ballot(vis_l && ok_l);
    for (int idx = tid; idx < PQ * npg; idx += NT) {
        const int qq = idx / npg, pi = idx % npg;
        if (!((live >> pi) & 1)) {
            const int v = max(0, L - (p.T - 1 - (tq0 + qq)));
            const int pid = __shfl(pid_l, pi);
            const bool bad = (j0 + pi) * kBlock < v && !(pid >= 0 && pid < p.P);
            sbuf[qq][pi] = bad ? __builtin_nanf("") : -INFINITY;
        }
    }

    // B operand of S^T = K Q^T: for tile qt and k-step ks the lane holds query
    // tq0 + 16*QT*wave + 16*qt + lane%16 at d = 32*ks + 8*(lane/16) .. +7.
    // Each wave transposes through 16 rows of LDS of its own (inside the page
    // buffers, before any page is stored there), 16-byte units XOR-swizzled
    // by row so that neither side has bank conflicts.  LDS accesses of one
    // wave complete in order, so the wave needs no barrier of its own.
    uint8_t *const stage = &kb[0][0] + wave * (16 * RB);
    uint4 qf[QT][KS];
    int vt[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const int t = tq0 + 16 * QT * wave + 16 * qt + li;
        vt[qt] = (t < p.T) ? max(0, L - (p.T - 1 - t)) : 0;
#pragma unroll
        for (int l = 0; l < LPT; ++l) {
            const int row = l * RPL + lane / UPR, unit = lane % UPR;
            *(uint4 *)(stage + row * RB + ((unit ^ (row & (UPR - 1))) << 4)) = qraw[qt][l];
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int unit = 4 * ks + grp;
            qf[qt][ks] = *(const uint4 *)(stage + li * RB + ((unit ^ (li & (UPR - 1))) << 4));
        }
    }

    // first pair to LDS (once every wave is done with its transpose area);
    // the next pair's slices on their way
    __syncthreads();
    if (c0 >= 0) store_page(pv[0], kb[0]);
    if (c1 >= 0) store_page(pv[1], kb[1]);
    int n0 = next_live(), n1 = next_live();
    if (n0 >= 0) load_page(n0, pv[0]);
    if (n1 >= 0) load_page(n1, pv[1]);
    __syncthreads();

    const float scale = p.idx_scale;
    auto compute_page = [&](const uint8_t *buf, int cur) {
        const int kbase = (j0 + cur) * kBlock;
        float best[QT];
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) best[qt] = -INFINITY;
        if (kbase + kBlock <= vmin) {                      // every key visible to every token
            // tile kt+1's operands are read before tile kt's MFMAs, and tile
            // kt's max is taken after tile kt+1's MFMAs are issued, so that
            // neither the LDS latency nor the MFMA latency sits in the way
            f32x4 acc[2][QT];
            uint4 af[2][KS];
            prefill_frag<DI>(buf, 0, li, grp, af[0]);
#pragma unroll
            for (int kt = 0; kt <= 8; ++kt) {
                if (kt + 1 < 8) prefill_frag<DI>(buf, kt + 1, li, grp, af[(kt + 1) & 1]);
                if (kt < 8) prefill_mma<DI, QT>(af[kt & 1], qf, acc[kt & 1]);
                if (kt >= 1) {
                    const f32x4 *done = acc[(kt - 1) & 1];
#pragma unroll
                    for (int qt = 0; qt < QT; ++qt) {
                        best[qt] = max3f(best[qt], done[qt][0], done[qt][1]);
                        best[qt] = max3f(best[qt], done[qt][2], done[qt][3]);
                    }
                }
            }
        } else {                                           // causal edge: mask key >= V(token)
            int lim[QT];
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) lim[qt] = vt[qt] - kbase - 4 * grp;
            for (int kt = 0; kt < 8; ++kt) {
                uint4 a[KS];
                prefill_frag<DI>(buf, kt, li, grp, a);
                f32x4 acc[QT];
                prefill_mma<DI, QT>(a, qf, acc);
#pragma unroll
                for (int qt = 0; qt < QT; ++qt) {
                    float m[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) m[e] = (kt * 16 + e < lim[qt]) ? acc[qt][e] : -INFINITY;
                    best[qt] = max3f(best[qt], m[0], m[1]);
                    best[qt] = max3f(best[qt], m[2], m[3]);
                }
            }
        }
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            const float v = max_across_groups<16>(best[qt]);
            if (grp == 0) sbuf[16 * QT * wave + 16 * qt + li][cur] = v * scale;
        }
    };
    for (int i = 0; c0 >= 0; ++i) {
        const int b = 2 * (i & 1);
        compute_page(kb[b], c0);
        if (c1 >= 0) compute_page(kb[b + 1], c1);
        // the other pair of buffers held the previous pair, done by every
        // wave before the last barrier
        const int nb = 2 - b;
        if (n0 >= 0) store_page(pv[0], kb[nb]);
        if (n1 >= 0) store_page(pv[1], kb[nb + 1]);
        const int a0 = next_live(), a1 = next_live();
        if (a0 >= 0) load_page(a0, pv[0]);
        if (a1 >= 0) load_page(a1, pv[1]);
        __syncthreads();
        c0 = n0; c1 = n1;
        n0 = a0; n1 = a1;
    }
    for (int idx = tid; idx < (tq1 - tq0) * npg; idx += NT) {
        const int qq = idx / npg, pi = idx % npg;
        p.scores[(nrow + tq0 + qq) * p.sc_sn + (int64_t)(j0 + pi) * p.sc_sj] = sbuf[qq][pi];
    }
}

template <bool QB, bool KF, int DI>
hipError_t launch_valu(const ScoreParams &p, hipStream_t s) {
    const int TG = (p.T + kTokGroup - 1) / kTokGroup;
    const int JC = (p.MB + 3) / 4;
    const int64_t grid = (int64_t)p.R * TG * JC;
    hipLaunchKernelGGL((score_valu_kernel<QB, KF, DI>), dim3((unsigned)grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

template <int DI>
hipError_t launch_mfma_decode(const ScoreParams &p, hipStream_t s) {
    const int64_t JC = (p.MB + 3) / 4;
    // R >= 8: 8 XCDs x ceil(R / 8) rows each x JC (see the kernel)
    const int64_t grid = p.R >= 8 ? 8 * ((p.R + 7) / 8) * JC : (int64_t)p.R * JC;
    hipLaunchKernelGGL((score_mfma_decode_kernel<DI>), dim3((unsigned)grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

template <int DI, int QT>
hipError_t launch_prefill(const ScoreParams &p, hipStream_t s) {
    const int64_t QC = (p.T + 16 * QT * kPWaves - 1) / (16 * QT * kPWaves), chunks = (int64_t)p.R * QC;
    // workgroups per query chunk: enough for kPTargetWGs in all, and enough
    // that none holds more than kPMaxPC blocks; no more than there are blocks
    int64_t WPC = (kPTargetWGs + chunks - 1) / chunks;
    WPC = WPC < (p.MB + kPMaxPC - 1) / kPMaxPC ? (p.MB + kPMaxPC - 1) / kPMaxPC : WPC;
    WPC = WPC > p.MB ? p.MB : WPC;
    const int64_t U = chunks * WPC;
    const int64_t grid = 8 * ((U + 7) / 8);               // tile ranges per XCD (see the kernel)
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;   // the kernel indexes tiles in int
    hipLaunchKernelGGL((score_prefill_kernel<DI, QT>), dim3((unsigned)grid), dim3(64 * kPWaves), 0, s, p, (int)WPC);
    return hipGetLastError();
}

// 4 query tiles per wave (512 tokens per workgroup) once a row has more than
// 256 query tokens, else 2
template <int DI>
hipError_t launch_mfma(const ScoreParams &p, hipStream_t s) {
    return p.T > 256 ? launch_prefill<DI, 4>(p, s) : launch_prefill<DI, 2>(p, s);
}

template <bool QB, bool KF>
hipError_t launch_valu_di(const ScoreParams &p, int Di, hipStream_t s) {
    switch (Di) {
    case 32: return launch_valu<QB, KF, 32>(p, s);
    case 64: return launch_valu<QB, KF, 64>(p, s);
    case 128: return launch_valu<QB, KF, 128>(p, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool score_supported(int q_type, int k_type, int Di) {
    return (q_type == E_F32 || q_type == E_BF16) && (k_type == E_F32 || k_type == E_FP8) &&
           (Di == 32 || Di == 64 || Di == 128);
}

hipError_t launch_score(const ScoreParams &p, int q_type, int k_type, int Di, hipStream_t s) {
    const bool qb = q_type == E_BF16, kf = k_type == E_FP8;
    if (p.R == 0 || p.T == 0) return hipSuccess;
    if (qb && kf && p.T > 16 && (Di == 64 || Di == 128))
        return Di == 64 ? launch_mfma<64>(p, s) : launch_mfma<128>(p, s);
    if (qb && kf && (Di == 64 || Di == 128))
        return Di == 64 ? launch_mfma_decode<64>(p, s) : launch_mfma_decode<128>(p, s);
    if (qb && kf) return launch_valu_di<true, true>(p, Di, s);
    if (qb) return launch_valu_di<true, false>(p, Di, s);
    if (kf) return launch_valu_di<false, true>(p, Di, s);
    return launch_valu_di<false, false>(p, Di, s);
}

}  // namespace msa
