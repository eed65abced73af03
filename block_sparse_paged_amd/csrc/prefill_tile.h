// One prefill score tile on MFMA: up to 512 query columns (bf16 rows of Di)
// against a run of at most MPC consecutive logical blocks of one request's
// FP8 index pages, reduced to the per-(column, block) maximum of the dot
// products over the keys the column sees.  Shared by the prefill path of
// msa_block_score (columns = query tokens of one row) and by the ragged
// prefill score-to-selection call (columns = (token, query head) pairs of one
// request), which differ only in which q row a column reads and how many keys
// it sees.
//
// A workgroup of 8 waves (two per SIMD, one workgroup per CU) holds the tile.
// The query rows are read coalesced and transposed into the MFMA operand
// layout through LDS.  Each live page is read once per workgroup with
// coalesced 16-byte loads (every thread a 32-byte slice of a key row),
// decoded FP8 -> bf16 once and stored to a bf16 page buffer in LDS, from which
// all 8 waves read their A operands ready to use: the decode costs 16 VALU
// instructions per wave and page instead of one per MFMA, and VALU issue does
// not overlap MFMA issue well on a SIMD.  Pages go through LDS two at a time
// (four page buffers, one barrier per pair); the next pair's slices are loaded
// into registers while the current pair is multiplied, and decoded and stored
// after it.  Pages that every column sees whole skip the visibility mask.
#pragma once

#include "device_util.h"
#include "msa_internal.h"

namespace msa {

constexpr int kPWaves = 8;        // waves per workgroup, two per SIMD
constexpr int kPMaxPC = 8;        // blocks per tile of the prefill score sheet, at most

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

// LDS of one tile of at most MPC blocks, worked by NW waves: NB bf16 page
// buffers (two groups of NB/2 pages) and the block maxima.
template <int DI, int QT, int MPC, int NW = kPWaves, int NB = 4>
struct PrefillLds {
    static constexpr int PQ = 16 * QT * NW;         // query columns
    static constexpr int MaxPages = MPC;
    static constexpr int Waves = NW;
    __attribute__((aligned(16))) uint8_t kb[NB][kBlock * DI * 2];
    float sbuf[PQ][MPC + 1];
};

// The pages of a tile: blocks j0 .. j0+npg-1 of a request whose block table
// row is bt_row (nullptr: no valid row, every block's page is invalid).
struct PrefillPages {
    const uint8_t *index_k;
    int64_t k_sp, k_sb;       // bytes per page, per key row
    int P;
    const int32_t *bt_row;
    int64_t bt_sj;
    int j0, npg;              // npg <= the tile's MPC (< 64)
    int vmin, vmax;           // keys seen by every column, by the column that sees most
    float scale;
};

// Fills lds.sbuf[col][pi] (col < PQ, pi < npg) with scale * max over the keys
// of block j0 + pi visible to column col of its dot products; -inf where the
// column sees none of them, NaN where it sees some and the block's page id
// lies outside [0, P) (the page is not read).  qrow(col) gives the column's bf16
// query row (any valid address for columns that are not used), vis(col) the
// number of keys the column sees (0 for unused columns).  Every thread of the
// workgroup calls it; it ends with a barrier, after which sbuf is complete.
template <int DI, int QT, int MPC, int NW, int NB, class QRow, class Vis>
__device__ __forceinline__ void prefill_tile(const PrefillPages &pg, QRow qrow, Vis vis,
                                             PrefillLds<DI, QT, MPC, NW, NB> &lds) {
    constexpr int KS = DI / 32;                 // MFMA k-steps per 16-key tile
    constexpr int NT = 64 * NW;                 // threads per workgroup
    constexpr int G = NB / 2;                   // pages per group (one barrier per group)
    constexpr int RB = DI * 2;                  // bytes per bf16 row (query or key)
    constexpr int UPR = DI / 8;                 // 16-byte units per bf16 row
    constexpr int VPT = kBlock * DI / (16 * NT) > 0 ? kBlock * DI / (16 * NT) : 1;  // 16-byte FP8 loads per slice
    constexpr int TPK = DI / (16 * VPT);        // slices per key row
    constexpr int NLD = TPK * kBlock;           // threads holding a slice (whole waves)
    constexpr int PQ = PrefillLds<DI, QT, MPC, NW, NB>::PQ;
    static_assert(MPC < 64, "page ids live one per lane");
    static_assert(NB == 2 || NB == 4, "one or two pages per group");
    static_assert(NLD <= NT && NLD % 64 == 0 && TPK * 16 * VPT == DI, "page slicing");
    static_assert(NW * 16 * RB <= G * kBlock * RB, "query transpose area inside the second group");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = lane >> 4, li = lane & 15;
    const int j0 = pg.j0, npg = pg.npg, vmin = pg.vmin, vmax = pg.vmax;

    // page table of the tile: lane i holds block j0 + i (npg < 64)
    const int pid_l = (lane < npg && pg.bt_row) ? pg.bt_row[(int64_t)(j0 + lane) * pg.bt_sj] : -1;
    const bool vis_l = lane < npg && (j0 + lane) * kBlock < vmax;
    const bool ok_l = pid_l >= 0 && pid_l < pg.P;
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
    uint4 pv[G][VPT];                                      // the slices of the next group of pages
    auto load_page = [&](int pi, uint4 (&v)[VPT]) {
        if (NLD < NT && tid >= NLD) return;
        const int pid = __builtin_amdgcn_readlane(pid_l, pi);
        const uint8_t *src = pg.index_k + (int64_t)pid * pg.k_sp + (int64_t)skey * pg.k_sb + 16 * VPT * spart;
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
    // Pages go through LDS G at a time (one barrier per group).  The first
    // group is requested before the query rows: the other order was measured
    // to be slower.
    int cur[G];
#pragma unroll
    for (int u = 0; u < G; ++u) {
        cur[u] = next_live();
        if (cur[u] >= 0) load_page(cur[u], pv[u]);
    }

    // Query rows, read coalesced.  In the MFMA operand layout consecutive
    // lanes hold different query rows, and a global load in that layout
    // touches a separate cache line for every lane of a 4-lane quad, several
    // times slower than quads reading 64 contiguous bytes.  So each wave reads
    // its 16*QT rows with whole rows across consecutive lanes and transposes
    // them through 16 rows' worth of LDS of its own (below).
    constexpr int RPL = 64 / UPR;               // rows per coalesced load
    constexpr int LPT = 16 / RPL;               // loads per 16-row tile
    uint4 qraw[QT][LPT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int l = 0; l < LPT; ++l) {
            const int col = 16 * QT * wave + 16 * qt + l * RPL + lane / UPR;
            qraw[qt][l] = *(const uint4 *)(qrow(col) + 8 * (lane % UPR));
        }

    // blocks without a live page: -inf for columns that see none of their
    // keys, NaN for columns that see keys of a block whose page id is out of
    // range
    const uint64_t live = __ballot(vis_l && ok_l);
    for (int idx = tid; idx < PQ * npg; idx += NT) {
        const int qq = idx / npg, pi = idx % npg;
        if (!((live >> pi) & 1)) {
            const int v = vis(qq);
            const int pid = __shfl(pid_l, pi);
            const bool bad = (j0 + pi) * kBlock < v && !(pid >= 0 && pid < pg.P);
            lds.sbuf[qq][pi] = bad ? __builtin_nanf("") : -INFINITY;
        }
    }

    // The first group to LDS as soon as its slices have landed, while the
    // query rows are still on their way (they were requested after it); the
    // next group's slices follow.  The second group's buffers stay free until
    // the first group has been multiplied, so the query transpose below uses
    // them and the first group's decode does not wait for it.
#pragma unroll
    for (int u = 0; u < G; ++u)
        if (cur[u] >= 0) store_page(pv[u], lds.kb[u]);
    int nxt[G];
#pragma unroll
    for (int u = 0; u < G; ++u) {
        nxt[u] = next_live();
        if (nxt[u] >= 0) load_page(nxt[u], pv[u]);
    }

    // B operand of S^T = K Q^T: for tile qt and k-step ks the lane holds
    // column 16*QT*wave + 16*qt + lane%16 at d = 32*ks + 8*(lane/16) .. +7.
    // Each wave transposes through 16 rows of LDS of its own (inside the
    // second group's page buffers), 16-byte units XOR-swizzled by row so that
    // neither side has bank conflicts.  LDS accesses of one wave complete in
    // order, so the wave needs no barrier of its own.
    uint8_t *const stage = &lds.kb[G][0] + wave * (16 * RB);
    uint4 qf[QT][KS];
    int vt[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        vt[qt] = vis(16 * QT * wave + 16 * qt + li);
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

    // the fewest and the most keys any column of the wave sees: key tiles of a
    // page that no column sees are skipped, and only tiles that some column
    // sees in part are masked
    int vminw, vmaxw;
    {
        int mn = vt[0], mx = vt[0];
#pragma unroll
        for (int qt = 1; qt < QT; ++qt) {
            mn = min(mn, vt[qt]);
            mx = max(mx, vt[qt]);
        }
        vminw = __builtin_amdgcn_readfirstlane(-(int)group_max<16>(-(float)mn));
        vmaxw = __builtin_amdgcn_readfirstlane((int)group_max<16>((float)mx));
    }

    // the first group is in LDS and every wave's transpose is done (the
    // loop's first stores go to the transpose area)
    __syncthreads();

    const float scale = pg.scale;
    auto compute_page = [&](const uint8_t *buf, int pidx) {
        const int kbase = (j0 + pidx) * kBlock;
        float best[QT];
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) best[qt] = -INFINITY;
        // lane (li, grp) holds keys 16*kt + 4*grp + e of tile kt; key k of
        // the page is visible to the lane's column of tile qt when
        // k < vt[qt] - kbase, i.e. e < lim[qt] - 16*kt
        int lim[QT];
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) lim[qt] = vt[qt] - kbase - 4 * grp;
        const int lo = vminw - kbase, hi = vmaxw - kbase;
        // One pass over the page's 8 key tiles: tile kt+1's operands are read
        // before tile kt's MFMAs, and tile kt-1's maxima are taken after them,
        // so that neither the LDS latency nor the MFMA latency sits in the
        // way; scheduling barriers keep that order (left to itself the
        // compiler moved each read next to its first use, measured 3 %
        // slower).  EDGE: a page some column sees only in part.
        auto run = [&](auto EDGE_) {
            constexpr bool EDGE = decltype(EDGE_)::value;
            auto live = [&](int kt) { return !EDGE || kt * 16 < hi; };   // some column sees the tile
            f32x4 acc[2][QT];
            uint4 af[2][KS];
            prefill_frag<DI>(buf, 0, li, grp, af[0]);
            // a raised issue priority while the wave streams its MFMAs: the
            // other wave of the SIMD takes the gaps for its loads, decodes and
            // maxima instead of interleaving with them (measured 3-4 % faster)
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int kt = 0; kt <= 8; ++kt) {
                __builtin_amdgcn_sched_barrier(0);
                if (kt + 1 < 8 && live(kt + 1)) prefill_frag<DI>(buf, kt + 1, li, grp, af[(kt + 1) & 1]);
                __builtin_amdgcn_sched_barrier(0);
                if (kt < 8 && live(kt)) prefill_mma<DI, QT>(af[kt & 1], qf, acc[kt & 1]);
                __builtin_amdgcn_sched_barrier(0);
                if (kt >= 1 && live(kt - 1)) {
                    const int k0 = (kt - 1) * 16;
                    const f32x4 *done = acc[(kt - 1) & 1];
                    if (EDGE && k0 + 16 > lo) {
                        // some column sees the tile in part: mask its keys
#pragma unroll
                        for (int qt = 0; qt < QT; ++qt) {
                            float m[4];
#pragma unroll
                            for (int e = 0; e < 4; ++e) m[e] = (k0 + e < lim[qt]) ? done[qt][e] : -INFINITY;
                            best[qt] = max3f(best[qt], m[0], m[1]);
                            best[qt] = max3f(best[qt], m[2], m[3]);
                        }
                    } else {
#pragma unroll
                        for (int qt = 0; qt < QT; ++qt) {
                            best[qt] = max3f(best[qt], done[qt][0], done[qt][1]);
                            best[qt] = max3f(best[qt], done[qt][2], done[qt][3]);
                        }
                    }
                }
            }
            __builtin_amdgcn_s_setprio(0);
        };
        if (kbase + kBlock <= vmin) run(Int<0>{});   // every key visible to every column
        else run(Int<1>{});
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            const float v = max_across_groups<16>(best[qt]);
            if (grp == 0) lds.sbuf[16 * QT * wave + 16 * qt + li][pidx] = v * scale;
        }
    };
    for (int i = 0; cur[0] >= 0; ++i) {
        const int b = G * (i & 1);
#pragma unroll
        for (int u = 0; u < G; ++u)
            if (cur[u] >= 0) compute_page(lds.kb[b + u], cur[u]);
        // the other group of buffers held the previous group, done by every
        // wave before the last barrier
        const int nb = G - b;
#pragma unroll
        for (int u = 0; u < G; ++u)
            if (nxt[u] >= 0) store_page(pv[u], lds.kb[nb + u]);
        int aft[G];
#pragma unroll
        for (int u = 0; u < G; ++u) {
            aft[u] = next_live();
            if (aft[u] >= 0) load_page(aft[u], pv[u]);
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < G; ++u) {
            cur[u] = nxt[u];
            nxt[u] = aft[u];
        }
    }
}

}  // namespace msa
