// Decode block scoring of one page by one wave (the score kernel for T <= 16).
#pragma once

#include "attn_unit.h"
#include "device_util.h"
#include "msa_internal.h"

namespace msa {

// 16-byte load with the non-temporal cache policy (index pages are read once)
__device__ __forceinline__ uint4 load_nt16(const uint8_t *ptr) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load((const u32x4 *)ptr);
    return make_uint4(v.x, v.y, v.z, v.w);
}

//
// Decode rows (T <= 16 tokens): one wave per (row, page).  The row's T query
// tokens are the 16 columns of v_mfma_f32_16x16x32_bf16 (unused columns are
// zero); the page's 128 keys are its rows.  Each lane pulls its operand bytes
// straight from HBM -- key 16*kt + lane%16, Di/4 contiguous bytes at
// d = (Di/4)*(lane/16) -- so a wave keeps the whole 16 KiB page in flight in
// 64 registers, and the VALU only decodes FP8 -> bf16 (exact) and takes the
// masked running max.  The dot products themselves run on the matrix cores.

// One wave scores page j of row r for the row's T <= 16 tokens.
template <int DI>
__device__ __forceinline__ void score_page(const ScoreParams &p, const int r, const int j) {
    constexpr int KS = DI / 32;                 // k-steps per 16-key tile
    constexpr int LB = DI / 4;                  // bytes per lane per key row
    constexpr int NL = LB / 16;                 // 16-byte loads per key tile
    static_assert(NL >= 1, "index dim");
    const int lane = threadIdx.x & 63;
    const int grp = lane >> 4, li = lane & 15;
    // seq_len, this page's id and the query fragments are independent: one round trip
    const int Lraw = p.seq_lens[(int64_t)r * p.sl_s];
    const int pid = p.bt[(int64_t)r * p.bt_sr + (int64_t)j * p.bt_sj];
    const int64_t n0 = (int64_t)r * p.T;
    const bool tok = li < p.T;
    // B operand: token li, d = LB*grp + 8*ks .. +8 (bf16)
    uint4 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        qf[ks] = tok ? *(const uint4 *)((const uint16_t *)p.q_idx + (n0 + li) * p.q_sn + LB * grp + 8 * ks)
                     : make_uint4(0, 0, 0, 0);
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
            uint4 kf[8][NL];
#pragma unroll
            for (int kt = 0; kt < 8; ++kt)
#pragma unroll
                for (int h = 0; h < NL; ++h)
                    kf[kt][h] = load_nt16(pg + (int64_t)(kt * 16 + li) * p.k_sb + LB * grp + 16 * h);
            // eight independent accumulators (one per 16-key tile), so that no
            // tile waits for the previous tile's products before its own
            f32x4 acc[8];
#pragma unroll
            for (int kt = 0; kt < 8; ++kt) {
                acc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const uint4 raw = kf[kt][ks >> 1];
                    const uint32_t lo = (ks & 1) ? raw.z : raw.x, hi = (ks & 1) ? raw.w : raw.y;
                    uint4 a;
                    a.x = fp8x2_to_bf16x2<false>(lo); a.y = fp8x2_to_bf16x2<true>(lo);
                    a.z = fp8x2_to_bf16x2<false>(hi); a.w = fp8x2_to_bf16x2<true>(hi);
                    acc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                                      __builtin_bit_cast(bf16x8, qf[ks]), acc[kt],
                                                                      0, 0, 0);
                }
            }
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
