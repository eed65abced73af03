// Decode block scoring of one page by one wave (the score kernel for T <= 16).
#pragma once

#include "attn_unit.h"
#include "device_util.h"
#include "msa_internal.h"

namespace msa {

//
// Decode rows (T <= 16 tokens): one wave per (row, page).  The row's T query
// tokens are the 16 columns of v_mfma_f32_16x16x32_bf16 (unused columns are
// zero); the page's 128 keys are its rows.  With STAGE the wave brings its
// 16 KiB page into LDS of its own with direct-to-LDS loads of 1 KiB, each
// covering whole key rows (an operand layout straight from HBM puts 16 rows in
// every load instruction, twice the cache lines of a contiguous one: with
// every CU streaming, measurably slower), 16-byte units XOR-swizzled by key as
// in the attention unit, and reads each 16-key tile back in the operand layout
// as soon as its loads have landed.  Without STAGE (launches of fewer than two
// waves per CU, bound by latency, where the LDS round trip costs more than
// the address unit saves) the lanes load the operand layout straight into
// registers.  The VALU only decodes FP8 -> bf16 (exact) and takes the masked
// maximum; the dot products run on the matrix cores.

// 16-byte load with the non-temporal cache policy (index pages are read once)
__device__ __forceinline__ uint4 load_nt16(const uint8_t *ptr) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load((const u32x4 *)ptr);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// One wave scores page j of row r for the row's T <= 16 tokens; spg (STAGE):
// 128 * DI bytes of LDS owned by the wave.
template <int DI, bool STAGE>
__device__ __forceinline__ void score_page(const ScoreParams &p, const int r, const int j, uint8_t *spg) {
    constexpr int KS = DI / 32;                 // k-steps per 16-key tile
    constexpr int CPR = DI / 16;                // 16-byte units per key row
    constexpr int KPL = 64 / CPR;               // key rows per 1 KiB load
    constexpr int LPT = 16 / KPL;               // loads per 16-key tile
    constexpr int NLD = 8 * LPT;                // loads per page
    static_assert(KS >= 2 && KS % 2 == 0 && LPT >= 1, "index dim");
    const int lane = threadIdx.x & 63;
    const int grp = lane >> 4, li = lane & 15;
    // seq_len, this page's id and the query fragments are independent: one round trip
    const int Lraw = p.seq_lens[(int64_t)r * p.sl_s];
    const int pid = p.bt[(int64_t)r * p.bt_sr + (int64_t)j * p.bt_sj];
    const int64_t n0 = (int64_t)r * p.T;
    const bool tok = li < p.T;
    // B operand of k-step ks: token li, d = 64*(ks/2) + 16*grp + 8*(ks%2) .. +8
    // (bf16), the d order of the K operand below
    uint4 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int d = 64 * (ks >> 1) + 16 * grp + 8 * (ks & 1);
        qf[ks] = tok ? *(const uint4 *)((const uint16_t *)p.q_idx + (n0 + li) * p.q_sn + d) : make_uint4(0, 0, 0, 0);
    }
    const int L = clamp_len(Lraw, p.MB);
    const int vmax = max(0, L);                 // the row's last token sees L keys
    const int vmin = max(0, L - (p.T - 1));     // and its first L - (T - 1)
    const int vt = tok ? max(0, L - (p.T - 1 - li)) : 0;
    float best = -INFINITY;
    bool bad_page = false;
    if (j * kBlock < vmax) {
        if (pid < 0 || pid >= p.P) {
            bad_page = true;
        } else {
            const uint8_t *pg = (const uint8_t *)p.index_k + (int64_t)pid * p.k_sp;
            // tile kt: A operand of k-step ks, key 16*kt + li, d = 64*(ks/2) +
            // 16*grp + 8*(ks%2): unit grp + 4*(ks/2) of the row
            uint4 kf[STAGE ? 1 : 8][KS / 2];
            if constexpr (STAGE) {
                // nothing but the page loads may be in the wave's load queue:
                // the waits below count positions in it
                __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
                // load l: key rows KPL*l .. +KPL, lane -> (row KPL*l + lane /
                // CPR, unit slot lane % CPR), global unit slot ^ kswz(row)
                const int key0 = lane / CPR, slot = lane % CPR;
#pragma unroll
                for (int l = 0; l < NLD; ++l) {
                    const int key = l * KPL + key0;
                    dma16_nt(pg + (int64_t)key * p.k_sb + ((slot ^ kswz<CPR>(key)) << 4), spg + l * 1024);
                }
            } else {
#pragma unroll
                for (int kt = 0; kt < 8; ++kt)
#pragma unroll
                    for (int h = 0; h < KS / 2; ++h)
                        kf[kt][h] = load_nt16(pg + (int64_t)(16 * kt + li) * p.k_sb + 16 * (grp + 4 * h));
            }
            f32x4 acc[8];
            static_for<0, 8>([&](auto KT) {
                constexpr int kt = decltype(KT)::value;
                const int key = 16 * kt + li;
                const uint8_t *krow = spg + key * DI;
                if constexpr (STAGE) wait_vmcnt<NLD - LPT * (kt + 1)>();
                acc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int h = 0; h < KS / 2; ++h) {
                    uint4 raw;
                    if constexpr (STAGE) raw = *(const uint4 *)(krow + (((grp + 4 * h) ^ kswz<CPR>(key)) << 4));
                    else raw = kf[kt][h];
                    acc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, fp8x8_to_bf16x8(raw.x, raw.y)),
                        __builtin_bit_cast(bf16x8, qf[2 * h]), acc[kt], 0, 0, 0);
                    acc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, fp8x8_to_bf16x8(raw.z, raw.w)),
                        __builtin_bit_cast(bf16x8, qf[2 * h + 1]), acc[kt], 0, 0, 0);
                }
            });
            // acc[kt][e] = dot of key 16*kt + 4*grp + e with token li
            const int kbase = j * kBlock;
            if (kbase + kBlock <= vmin) {
                // the whole page is visible to every token of the row (one
                // branch for the wave); the products of a visible key are dot
                // products of finite codes (a NaN code there is outside the
                // contract), so the maximum needs no NaN quieting
#pragma unroll
                for (int kt = 0; kt < 8; ++kt)
                    best = max3f(best, max3f(acc[kt][0], acc[kt][1], acc[kt][2]), acc[kt][3]);
            } else {
#pragma unroll
                for (int kt = 0; kt < 8; ++kt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int pos = kbase + kt * 16 + 4 * grp + e;
                        best = (pos < vt) ? fmaxf(best, acc[kt][e]) : best;
                    }
            }
            best = max_across_groups<16>(best);
            if (!tok) best = -INFINITY;                 // unused columns
        }
    }
    if (p.per_row) {
        // one row per request: the max over the row's tokens (columns past
        // T hold -inf)
        best = group_max<16>(best);
        if (lane == 0) {
            const float v = bad_page ? __builtin_nanf("") : best * p.idx_scale;
            p.scores[(int64_t)r * p.sc_sn + (int64_t)j * p.sc_sj] = v;
        }
    } else if (grp == 0 && tok) {
        const float v = bad_page ? __builtin_nanf("") : best * p.idx_scale;
        p.scores[(n0 + li) * p.sc_sn + (int64_t)j * p.sc_sj] = v;
    }
}

}  // namespace msa
