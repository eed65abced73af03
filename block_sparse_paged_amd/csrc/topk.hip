// Stage 2: per-row top-k block selection.
//
// Cacheon "Kernel ABI", "Attention block slots": attention.decode takes the
// selected nonnegative block ids with -1 meaning none, and
// attention.msa_prefill_block_score leaves unused cells at -1; "Correctness is
// target-owned": selections are graded as sets, so the order within a row is
// free and this library writes ascending block ids.
//
// One wave per score row.  Scores become order-preserving unsigned keys
// (-0 folded onto +0; -inf and NaN become key 0 = not a candidate).  A radix
// select over the 32-bit keys, one bit per step from the top with wave-wide
// ballot counts, finds the k-th largest key tau; keys above tau are taken,
// and keys equal to tau in ascending block id until k are taken, so ties go to
// the lower id.  Output positions come from ballot prefix counts, which keeps
// the ids ascending.  Everything is integer work: the result is exact and
// deterministic.
#include "device_util.h"
#include "msa_internal.h"

namespace msa {

namespace {

__device__ __forceinline__ uint32_t score_key(float s) {
    if (s != s || s == -INFINITY) return 0u;
    uint32_t u = __float_as_uint(s == 0.f ? 0.f : s);   // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// One wave per score row; the wave finds the k-th largest key tau bit by bit
// from the top (tau = the largest x with #{key >= x} >= k), counting with
// ballots, so no LDS and no barrier is involved.
template <int KPL>
__global__ __launch_bounds__(256) void topk_kernel(TopkParams p) {
    const int lane = threadIdx.x & 63;
    const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (n >= p.N) return;

    uint32_t key[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const int id = i * 64 + lane;
        key[i] = (id < p.MB) ? score_key(p.scores[n * p.sc_sn + (int64_t)id * p.sc_sj]) : 0u;
    }
    int ncand = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i) ncand += __popcll(__ballot(key[i] != 0u));
    const bool take_all = ncand <= p.k;

    uint32_t tau = 0u;
    if (!take_all) {
#pragma unroll 1
        for (int b = 31; b >= 0; --b) {
            const uint32_t trial = tau | (1u << b);
            int cnt = 0;
#pragma unroll
            for (int i = 0; i < KPL; ++i) cnt += __popcll(__ballot(key[i] >= trial));
            if (cnt >= p.k) tau = trial;
        }
    }
    int above = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i) above += __popcll(__ballot(key[i] > tau));
    const int need = p.k - above;                          // keys equal to tau to take
    int eq_base = 0, out_base = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const uint64_t eq = __ballot(!take_all && key[i] == tau && key[i] != 0u);
        const int eq_rank = eq_base + lanes_below(eq);
        eq_base += __popcll(eq);
        const bool sel = take_all ? key[i] != 0u
                                  : (key[i] > tau || (key[i] == tau && eq_rank < need));
        const uint64_t sm = __ballot(sel);
        if (sel) p.topk[n * p.tk_sn + (int64_t)(out_base + lanes_below(sm)) * p.tk_si] = i * 64 + lane;
        out_base += __popcll(sm);
    }
    for (int q = out_base + lane; q < p.k; q += 64) p.topk[n * p.tk_sn + (int64_t)q * p.tk_si] = -1;
}

template <int KPL>
hipError_t launch(const TopkParams &p, hipStream_t s) {
    const int grid = (p.N + 3) / 4;
    hipLaunchKernelGGL((topk_kernel<KPL>), dim3(grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(const TopkParams &p, hipStream_t s) {
    if (p.N == 0) return hipSuccess;
    if (p.MB <= 64) return launch<1>(p, s);
    if (p.MB <= 128) return launch<2>(p, s);
    if (p.MB <= 256) return launch<4>(p, s);
    if (p.MB <= 512) return launch<8>(p, s);
    if (p.MB <= 1024) return launch<16>(p, s);
    if (p.MB <= 2048) return launch<32>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace msa
