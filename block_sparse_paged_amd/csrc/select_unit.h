// Per-row top-k block selection by one wave, shared by the standalone top-k
// kernel and the attention launch of msa_decode_step (which selects its
// token's blocks from the score row itself).
//
// Scores become order-preserving unsigned keys (-0 folded onto +0; -inf and
// NaN become key 0 = not a candidate).  The wave finds the k-th largest key
// tau two bits at a time from the top (tau = the largest x with
// #{key >= x} >= k), counting with ballots: no LDS and no barrier (it stops
// early once exactly k keys are >= tau).  Keys above tau are taken, and keys equal to tau in
// ascending block id until k are taken, so ties go to the lower id; output positions come from ballot prefix counts, which keeps the
// ids ascending.  Positions past the candidates get -1.
#pragma once

#include "device_util.h"
#include "msa_internal.h"

namespace msa {

__device__ __forceinline__ uint32_t score_key(float s) {
    if (s != s || s == -INFINITY) return 0u;
    uint32_t u = __float_as_uint(s == 0.f ? 0.f : s);   // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// key[i] of lane l is the key of block i*64 + l (0 past MB).  emit(pos, id) is
// called for pos in [0, k): the selected ids ascending, then -1.
template <int KPL, class Emit>
__device__ __forceinline__ void select_keys(const uint32_t (&key)[KPL], const int k, Emit emit) {
    const int lane = threadIdx.x & 63;
    int ncand = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i) ncand += __popcll(__ballot(key[i] != 0u));
    const bool take_all = ncand <= k;

    // Two bits of tau per round: the largest of tau|11, tau|10, tau|01 (else
    // tau|00) that still has >= k keys at or above it (the counts fall as the
    // trial rises).  Once exactly k keys are >= tau, those k are the selection
    // whatever the lower bits of the k-th key are: the search stops there (the
    // (k+1)-th key already lies below tau, so no tie crosses the cut).
    uint32_t tau = 0u;
    if (!take_all) {
#pragma unroll 1
        for (int b = 30; b >= 0; b -= 2) {
            const uint32_t t1 = tau | (1u << b), t2 = tau | (2u << b), t3 = tau | (3u << b);
            int c1 = 0, c2 = 0, c3 = 0;
#pragma unroll
            for (int i = 0; i < KPL; ++i) {
                c1 += __popcll(__ballot(key[i] >= t1));
                c2 += __popcll(__ballot(key[i] >= t2));
                c3 += __popcll(__ballot(key[i] >= t3));
            }
            const int c = c3 >= k ? c3 : c2 >= k ? c2 : c1 >= k ? c1 : 0;
            tau = c3 >= k ? t3 : c2 >= k ? t2 : c1 >= k ? t1 : tau;
            if (c == k) break;
        }
    }
    int above = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i) above += __popcll(__ballot(key[i] > tau));
    const int need = k - above;                          // keys equal to tau to take
    int eq_base = 0, out_base = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const uint64_t eq = __ballot(!take_all && key[i] == tau && key[i] != 0u);
        const int eq_rank = eq_base + lanes_below(eq);
        eq_base += __popcll(eq);
        const bool sel = take_all ? key[i] != 0u
                                  : (key[i] > tau || (key[i] == tau && eq_rank < need));
        const uint64_t sm = __ballot(sel);
        if (sel) emit(out_base + lanes_below(sm), i * 64 + lane);
        out_base += __popcll(sm);
    }
    for (int q = out_base + lane; q < k; q += 64) emit(q, -1);
}

// Score row n of the sheet -> topk row n.
template <int KPL>
__device__ __forceinline__ void select_row(const TopkParams &p, const int64_t n) {
    const int lane = threadIdx.x & 63;
    uint32_t key[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const int id = i * 64 + lane;
        key[i] = id < p.MB ? score_key(p.scores[n * p.sc_sn + (int64_t)id * p.sc_sj]) : 0u;
    }
    int32_t *dst = p.topk + n * p.tk_sn;
    select_keys<KPL>(key, p.k, [&](int pos, int id) { dst[(int64_t)pos * p.tk_si] = id; });
}

// Scores already in registers (v[i] of lane l = score of block i*64 + l) ->
// slots[0..k) (LDS).
template <int KPL>
__device__ __forceinline__ void select_from_values(const float (&v)[KPL], const int MB, const int k,
                                                   int *slots) {
    const int lane = threadIdx.x & 63;
    uint32_t key[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) key[i] = (i * 64 + lane < MB) ? score_key(v[i]) : 0u;
    select_keys<KPL>(key, k, [&](int pos, int id) { slots[pos] = id; });
}

}  // namespace msa
