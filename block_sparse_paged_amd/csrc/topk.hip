// Stage 2: per-row top-k block selection.
//
// Cacheon "Kernel ABI", "Attention block slots": attention.decode takes the
// selected nonnegative block ids with -1 meaning none, and
// attention.msa_prefill_block_score leaves unused cells at -1; "Correctness is
// target-owned": selections are graded as sets, so the order within a row is
// free and this library writes ascending block ids.
//
// One wave per score row.  Scores become order-preserving unsigned keys
// (-0 folded onto +0; -inf and NaN become key 0 = not a candidate).  An
// 8-bit-digit radix select over the 32-bit keys (four passes, a 256-bin
// histogram per wave in LDS) finds the k-th largest key tau and how many keys
// equal to tau still fit.  Keys above tau are taken, and keys equal to tau in
// ascending block id until k are taken, so ties go to the lower id.  Output
// positions come from ballot prefix counts, which keeps the ids ascending.
// Everything is integer work: the result is exact and deterministic.
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

template <int KPL>
__global__ __launch_bounds__(256) void topk_kernel(TopkParams p) {
    __shared__ uint32_t hist[4][256];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t n = (int64_t)blockIdx.x * 4 + wave;
    const bool active = n < p.N;

    uint32_t key[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const int id = i * 64 + lane;
        key[i] = 0u;
        if (active && id < p.MB) key[i] = score_key(p.scores[n * p.sc_sn + (int64_t)id * p.sc_sj]);
    }
    int ncand = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i) ncand += __popcll(__ballot(key[i] != 0u));

    // radix select for the k-th largest key among the candidates
    uint32_t prefix = 0u, pmask = 0u;
    int remaining = p.k;
#pragma unroll 1
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int b = lane; b < 256; b += 64) hist[wave][b] = 0u;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < KPL; ++i)
            if (key[i] != 0u && (key[i] & pmask) == prefix)
                atomicAdd(&hist[wave][(key[i] >> shift) & 255u], 1u);
        __syncthreads();
        const uint32_t h0 = hist[wave][4 * lane + 0], h1 = hist[wave][4 * lane + 1];
        const uint32_t h2 = hist[wave][4 * lane + 2], h3 = hist[wave][4 * lane + 3];
        const int lsum = (int)(h0 + h1 + h2 + h3);
        int incl = lsum;                                   // sum over lanes >= this one
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int v = __shfl_down(incl, off);
            if (lane + off < 64) incl += v;
        }
        const int s3 = incl - lsum + (int)h3;              // keys with digit >= 4*lane+3
        const int s2 = s3 + (int)h2, s1 = s2 + (int)h1, s0 = s1 + (int)h0;
        const uint64_t m = __ballot(s0 >= remaining);
        const int top = m ? 63 - __clzll((long long)m) : 0;
        int digit, above;
        if (s3 >= remaining)      { digit = 4 * lane + 3; above = s3 - (int)h3; }
        else if (s2 >= remaining) { digit = 4 * lane + 2; above = s2 - (int)h2; }
        else if (s1 >= remaining) { digit = 4 * lane + 1; above = s1 - (int)h1; }
        else                      { digit = 4 * lane + 0; above = s0 - (int)h0; }
        digit = __shfl(digit, top);
        above = __shfl(above, top);
        remaining -= above;
        prefix |= (uint32_t)digit << shift;
        pmask |= 0xffu << shift;
        __syncthreads();
    }
    if (!active) return;

    const bool take_all = ncand <= p.k;
    const uint32_t tau = prefix;
    const int need = remaining;                            // keys equal to tau to take
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
