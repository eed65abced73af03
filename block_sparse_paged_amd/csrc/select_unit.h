// Per-row top-k block selection by one wave, shared by the standalone top-k
// kernel and the attention launch of msa_decode_step (which selects its
// token's blocks from the score row itself).
//
// Scores become order-preserving unsigned keys (-0 folded onto +0; -inf and
// NaN become key 0 = not a candidate).  A threshold tau -- the k-th largest
// key, or a value that exactly k keys reach -- is found bit by bit from the
// top with ballot counts (up to 256 keys a row, see kth_largest_key_bits) or
// by a radix select over the bytes of the keys (LDS histograms, see
// kth_largest_key); keys above tau are taken, and keys equal to tau in
// ascending block id until k are taken, so ties go to the lower id;
// output positions come from ballot prefix counts, which keeps the ids
// ascending.
// Positions past the candidates get -1.  Integer work only: exact and
// deterministic.
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

// The k-th largest candidate key (key 0 excluded; there are more than k
// candidates), found one byte at a time from the top: each pass counts the
// candidates that match the bytes found so far into a 256-bin histogram in
// LDS (hist: 256 ints owned by the wave), and the bin holding the
// need-th largest of them gives the next byte.  It stops early when that
// bin's keys are exactly the ones still needed; the value returned then has
// the remaining bytes zero, and exactly k keys are >= it.
template <int KPL>
__device__ __forceinline__ uint32_t kth_largest_key(const uint32_t (&key)[KPL], const int k, int *hist) {
    const int lane = threadIdx.x & 63;
    uint32_t prefix = 0u, pmask = 0u;
    int need = k;
#pragma unroll 1
    for (int shift = 24; shift >= 0; shift -= 8) {
        *(int4 *)(hist + 4 * lane) = make_int4(0, 0, 0, 0);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
        for (int i = 0; i < KPL; ++i)
            if (key[i] != 0u && (key[i] & pmask) == prefix)
                __hip_atomic_fetch_add(hist + ((key[i] >> shift) & 255u), 1, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WAVEFRONT);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // lane l holds bins 255-4l (h.w) down to 252-4l (h.x)
        const int4 h = *(const int4 *)(hist + 252 - 4 * lane);
        const int t = h.x + h.y + h.z + h.w;
        const int above_lane = wave_prefix_sum(t) - t;         // candidates in bins > 255-4l
        // S(b): candidates in bins >= b
        const int sa = above_lane + h.w, sb = sa + h.z, sc = sb + h.y, sd = sc + h.x;
        const uint64_t m = __ballot(sd >= need);               // nonzero: lane 63 counts all
        const int L = __builtin_ctzll(m);                      // lane of the top bin with S >= need
        const int jj = sa >= need ? 0 : sb >= need ? 1 : sc >= need ? 2 : 3;
        const int sj = jj == 0 ? sa : jj == 1 ? sb : jj == 2 ? sc : sd;
        const int hj = jj == 0 ? h.w : jj == 1 ? h.z : jj == 2 ? h.y : h.x;
        const int bin = 255 - 4 * L - __builtin_amdgcn_readlane(jj, L);
        const int s_bin = __builtin_amdgcn_readlane(sj, L), h_bin = __builtin_amdgcn_readlane(hj, L);
        need -= s_bin - h_bin;                                 // the keys in higher bins are taken
        prefix |= (uint32_t)bin << shift;
        pmask |= 255u << shift;
        if (h_bin == need) break;                              // all of this bin is taken
    }
    return prefix;
}

// One step of the bitwise search below: candidate c = prefix | bit, n = the
// number of keys >= c; c is kept (prefix = c, cnt = n) when n >= k.  Written
// as one block of assembly so that the KPL compares go into SGPR pairs of
// their own and issue back to back, and the scalar counts wait for them once
// (compiled from C, every compare and count went through the same pair, two
// vector-to-scalar waits a step).  KPL is 1, 2 or 4.
template <int KPL>
__device__ __forceinline__ void kth_bit_step(uint32_t &prefix, int &cnt, const uint32_t bit,
                                             const uint32_t (&key)[KPL], const int k) {
    uint32_t c, n, t1, t2, t3;
    uint64_t m0, m1, m2, m3;
    if constexpr (KPL == 1) {
        asm volatile(
            "s_or_b32 %[c], %[p], %[b]\n\t"
            "v_cmp_le_u32_e64 %[m0], %[c], %[k0]\n\t"
            "s_bcnt1_i32_b64 %[n], %[m0]\n\t"
            "s_cmp_ge_u32 %[n], %[k]\n\t"
            "s_cselect_b32 %[p], %[c], %[p]\n\t"
            "s_cselect_b32 %[cnt], %[n], %[cnt]"
            : [p] "+s"(prefix), [cnt] "+s"(cnt), [c] "=&s"(c), [n] "=&s"(n), [m0] "=&s"(m0)
            : [b] "s"(bit), [k0] "v"(key[0]), [k] "s"(k)
            : "scc");
    } else if constexpr (KPL == 2) {
        asm volatile(
            "s_or_b32 %[c], %[p], %[b]\n\t"
            "v_cmp_le_u32_e64 %[m0], %[c], %[k0]\n\t"
            "v_cmp_le_u32_e64 %[m1], %[c], %[k1]\n\t"
            "s_bcnt1_i32_b64 %[n], %[m0]\n\t"
            "s_bcnt1_i32_b64 %[t1], %[m1]\n\t"
            "s_add_u32 %[n], %[n], %[t1]\n\t"
            "s_cmp_ge_u32 %[n], %[k]\n\t"
            "s_cselect_b32 %[p], %[c], %[p]\n\t"
            "s_cselect_b32 %[cnt], %[n], %[cnt]"
            : [p] "+s"(prefix), [cnt] "+s"(cnt), [c] "=&s"(c), [n] "=&s"(n), [t1] "=&s"(t1), [m0] "=&s"(m0),
              [m1] "=&s"(m1)
            : [b] "s"(bit), [k0] "v"(key[0]), [k1] "v"(key[1]), [k] "s"(k)
            : "scc");
    } else {
        static_assert(KPL == 4, "KPL 1, 2 or 4");
        asm volatile(
            "s_or_b32 %[c], %[p], %[b]\n\t"
            "v_cmp_le_u32_e64 %[m0], %[c], %[k0]\n\t"
            "v_cmp_le_u32_e64 %[m1], %[c], %[k1]\n\t"
            "v_cmp_le_u32_e64 %[m2], %[c], %[k2]\n\t"
            "v_cmp_le_u32_e64 %[m3], %[c], %[k3]\n\t"
            "s_bcnt1_i32_b64 %[n], %[m0]\n\t"
            "s_bcnt1_i32_b64 %[t1], %[m1]\n\t"
            "s_bcnt1_i32_b64 %[t2], %[m2]\n\t"
            "s_bcnt1_i32_b64 %[t3], %[m3]\n\t"
            "s_add_u32 %[n], %[n], %[t1]\n\t"
            "s_add_u32 %[t2], %[t2], %[t3]\n\t"
            "s_add_u32 %[n], %[n], %[t2]\n\t"
            "s_cmp_ge_u32 %[n], %[k]\n\t"
            "s_cselect_b32 %[p], %[c], %[p]\n\t"
            "s_cselect_b32 %[cnt], %[n], %[cnt]"
            : [p] "+s"(prefix), [cnt] "+s"(cnt), [c] "=&s"(c), [n] "=&s"(n), [t1] "=&s"(t1), [t2] "=&s"(t2),
              [t3] "=&s"(t3), [m0] "=&s"(m0), [m1] "=&s"(m1), [m2] "=&s"(m2), [m3] "=&s"(m3)
            : [b] "s"(bit), [k0] "v"(key[0]), [k1] "v"(key[1]), [k2] "v"(key[2]), [k3] "v"(key[3]), [k] "s"(k)
            : "scc");
    }
}

// The threshold of the k largest candidate keys (there are more than k
// candidates), built from the top bit down: a bit is kept when at least k keys
// are >= the value with it set.  Ballot counts only (no LDS, no atomics,
// whose conflicts serialise the histogram passes when the scores share their
// top bytes).  The search stops as soon as exactly k keys are >= the value
// built so far (the k-th and (k+1)-th largest keys first differ in the last
// bit kept): the value returned then has the remaining bits zero, and exactly
// k keys are >= it; otherwise it is the k-th largest key.  Selection from it
// (keys above it, then keys equal to it by ascending id) is the same either
// way.
template <int KPL>
__device__ __forceinline__ uint32_t kth_largest_key_bits(const uint32_t (&key)[KPL], const int k) {
    constexpr int KP = KPL <= 1 ? 1 : KPL <= 2 ? 2 : 4;     // registers searched (padding keys are 0)
    uint32_t kp[KP];
#pragma unroll
    for (int i = 0; i < KP; ++i) kp[i] = i < KPL ? key[i] : 0u;
    uint32_t prefix = 0u;
    int cnt = 64 * KP;                               // keys >= 0; more than k
#pragma unroll
    for (int b = 31; b >= 0; --b) {
        kth_bit_step<KP>(prefix, cnt, 1u << b, kp, k);
        if (cnt == k) break;
    }
    return prefix;
}

// The selection of a row as lane masks: key[i] of lane l is the key of block
// i*64 + l (0 past MB); bit l of selm[i] is set when that block is selected.
// The selected ids, ascending, are the set bits in order of (i, lane); there
// are min(k, candidates) of them.  hist: 256 ints of LDS owned by the wave
// (used only for KPL > 4).
template <int KPL>
__device__ __forceinline__ void select_masks(const uint32_t (&key)[KPL], const int k, int *hist,
                                             uint64_t (&selm)[KPL]) {
    int ncand = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i) ncand += __popcll(__ballot(key[i] != 0u));
    const bool take_all = ncand <= k;
    uint32_t tau = 0u;
    if (!take_all) {
        if constexpr (KPL <= 4) tau = kth_largest_key_bits<KPL>(key, k);
        else tau = kth_largest_key<KPL>(key, k, hist);
    }
    int above = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i) above += __popcll(__ballot(key[i] > tau));
    const int need = k - above;                          // keys equal to tau to take
    int eq_base = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const uint64_t eq = __ballot(!take_all && key[i] == tau && key[i] != 0u);
        const int eq_rank = eq_base + lanes_below(eq);
        eq_base += __popcll(eq);
        const bool sel = take_all ? key[i] != 0u
                                  : (key[i] > tau || (key[i] == tau && eq_rank < need));
        selm[i] = __ballot(sel);
    }
}

// emit(pos, id) for pos in [0, k): the ids of the masks ascending, then -1.
template <int KPL, class Emit>
__device__ __forceinline__ void emit_selection(const uint64_t (&selm)[KPL], const int k, Emit emit) {
    const int lane = threadIdx.x & 63;
    int out_base = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const uint64_t sm = selm[i];
        if ((sm >> lane) & 1u) emit(out_base + lanes_below(sm), i * 64 + lane);
        out_base += __popcll(sm);
    }
    for (int q = out_base + lane; q < k; q += 64) emit(q, -1);
}

// key[i] of lane l is the key of block i*64 + l (0 past MB).  emit(pos, id) is
// called for pos in [0, k): the selected ids ascending, then -1.  hist: 256
// ints of LDS owned by the wave.
template <int KPL, class Emit>
__device__ __forceinline__ void select_keys(const uint32_t (&key)[KPL], const int k, int *hist, Emit emit) {
    uint64_t selm[KPL];
    select_masks<KPL>(key, k, hist, selm);
    emit_selection<KPL>(selm, k, emit);
}

// Score row n of the sheet -> topk row n.
template <int KPL>
__device__ __forceinline__ void select_row(const TopkParams &p, const int64_t n, int *hist) {
    const int lane = threadIdx.x & 63;
    uint32_t key[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const int id = i * 64 + lane;
        key[i] = id < p.MB ? score_key(p.scores[n * p.sc_sn + (int64_t)id * p.sc_sj]) : 0u;
    }
    int32_t *dst = p.topk + n * p.tk_sn;
    select_keys<KPL>(key, p.k, hist, [&](int pos, int id) { dst[(int64_t)pos * p.tk_si] = id; });
}

// Scores already in registers (v[i] of lane l = score of block i*64 + l) ->
// slots[0..k) (LDS).
template <int KPL>
__device__ __forceinline__ void select_from_values(const float (&v)[KPL], const int MB, const int k,
                                                   int *slots, int *hist) {
    const int lane = threadIdx.x & 63;
    uint32_t key[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) key[i] = (i * 64 + lane < MB) ? score_key(v[i]) : 0u;
    select_keys<KPL>(key, k, hist, [&](int pos, int id) { slots[pos] = id; });
}

}  // namespace msa
