// Stage 3: sparse attention over the selected pages, split-K + reduction.
//
// Cacheon "Kernel ABI", "Attention block slots", attention.decode: attend
// exactly the supplied nonnegative block ids, excluding -1 entries and keys at
// or beyond the query's visibility; GQA as in attention.sdpa (query head h
// reads KV head h / (Hq/Hkv)).  Static scalar K/V scales and FP8 caches as in
// the vLLM design note "MiniMax-M3 decode through the ATOM kernel library",
// "Supported experiment".
//
// Work split.  A workgroup owns (row r, KV head g, group of <= 4 query tokens
// of the row, split s).  It builds the union of the group's selected blocks in
// LDS (ascending block id) and takes the s-th contiguous slice of that union,
// so every selected page is read from HBM once per row even when several of
// the row's speculative tokens chose it.  Wave w serves token w of the group
// and skips blocks its token did not select.  Each split leaves a partial
// (running max m in log2 units, sum l, unnormalised acc) per (token, head); a
// second kernel merges the splits in a fixed order.
//
// MFMA path (16 query heads per KV head, bf16 queries, FP8 K/V): each page is
// decoded once to bf16 in LDS -- K row-major, V transposed -- and every wave
// runs S^T = K * Q^T and O^T += V^T * P^T on v_mfma_f32_16x16x32_bf16 tiles,
// whose 16 columns are the 16 heads of its token.  The softmax statistics then
// live in the lane's column (head = lane % 16) for both products, and the PV
// k-index is permuted inside each 32-key chunk so that P leaves the QK
// accumulator already in the PV operand layout (no cross-lane moves).
#include "attn_unit.h"
#include "device_util.h"
#include "msa_internal.h"

namespace msa {

namespace {


struct Group {
    int r, g, t0, nt, s, L;
};

// keys visible to token t of the group
__device__ __forceinline__ int token_vis(const AttnParams &p, const Group &q, int t) {
    return max(0, q.L - (p.T - 1 - (q.t0 + t)));
}

// order LDS traffic between the lanes of one wave
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ Group decode_group(const AttnParams &p) {
    Group q;
    const int TG = (p.T + kTokGroup - 1) / kTokGroup;
    int bid = blockIdx.x;
    q.s = bid % p.splits;
    bid /= p.splits;
    const int tg = bid % TG;
    bid /= TG;
    q.g = bid % p.Hkv;
    q.r = bid / p.Hkv;
    q.t0 = tg * kTokGroup;
    q.nt = min(kTokGroup, p.T - q.t0);
    q.L = clamp_len(p.seq_lens[(int64_t)q.r * p.sl_s], p.MB);
    return q;
}

// Union of the group's selections.  sel[t] is token t's bitmask over logical
// blocks (only ids in [0, MB) with a visible key and a valid page id); ulist
// gets the union in ascending order.  Returns the union size (uniform).
__device__ int build_union(const AttnParams &p, const Group &q, uint32_t (*sel)[kMaxMB / 32],
                           uint16_t *ulist, int *ucount) {
    const int tid = threadIdx.x;
    const int MBW = (p.MB + 31) >> 5;
    for (int w = tid; w < kTokGroup * (kMaxMB / 32); w += 256) (&sel[0][0])[w] = 0u;
    __syncthreads();
    const int64_t n0 = (int64_t)q.r * p.T + q.t0;
    for (int e = tid; e < q.nt * p.k; e += 256) {
        const int t = e / p.k, i = e - t * p.k;
        const int64_t row = p.sel_per_row ? (int64_t)q.r : n0 + t;
        const int j = p.topk[(int64_t)q.g * p.tk_sg + row * p.tk_sn + (int64_t)i * p.tk_si];
        if (j < 0 || j >= p.MB || j * kBlock >= token_vis(p, q, t)) continue;
        const int pid = p.bt[(int64_t)q.r * p.bt_sr + (int64_t)j * p.bt_sj];
        if (pid < 0 || pid >= p.P) continue;
        atomicOr(&sel[t][j >> 5], 1u << (j & 31));
    }
    __syncthreads();
    if (tid < 64) {                                 // wave 0: one 32-block word per lane
        int base = 0;
        for (int w0 = 0; w0 < MBW; w0 += 64) {
            const int w = w0 + tid;
            uint32_t u = 0u;
            if (w < MBW) u = sel[0][w] | sel[1][w] | sel[2][w] | sel[3][w];
            const int c = __popc(u);
            int incl = c;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int v = __shfl_up(incl, off);
                if (tid >= off) incl += v;
            }
            int pos = base + incl - c;
            while (u) {
                const int b = __ffs(u) - 1;
                u &= u - 1u;
                ulist[pos++] = (uint16_t)(w * 32 + b);
            }
            base += __shfl(incl, 63);
        }
        if (tid == 0) *ucount = base;
    }
    __syncthreads();
    return *ucount;
}

__device__ __forceinline__ void split_range(int U, int S, int s, int &beg, int &end) {
    beg = (int)(((int64_t)U * s) / S);
    end = (int)(((int64_t)U * (s + 1)) / S);
}

// ------------------------------------------------------------------ MFMA path
//
// Launches of the per-token MFMA attention unit (attn_unit.h, which describes
// the chunk pipeline and the split merge): one workgroup per (query token n,
// KV head g, split s of n's selection list), placed by decode_token_slot.

struct TokenSlot {
    int n, g, s;
    bool live;
};

// Workgroup -> (token, KV head, split) with XCD-aware placement: workgroup id b
// runs on XCD b % 8.
__device__ __forceinline__ TokenSlot decode_token_slot(const AttnParams &p) {
    TokenSlot q;
    const int x = blockIdx.x & 7;
    const int local = blockIdx.x >> 3;
    const int S = p.splits;
    const int sidx = local % S;
    const int unit_local = local / S;            // index among this XCD's units
    const int N = p.R * p.T;
    int n, g;
    if (p.R >= 8) {                              // a row's units stay on XCD r % 8
        const int per_row = p.T * p.Hkv;
        const int rr = unit_local / per_row;
        const int rem = unit_local % per_row;
        const int r = x + 8 * rr;
        n = r * p.T + rem / p.Hkv;
        g = rem % p.Hkv;
        q.live = r < p.R;
    } else {                                     // unit u = n*Hkv + g on XCD u % 8
        const int u = x + 8 * unit_local;
        n = u / p.Hkv;
        g = u % p.Hkv;
        q.live = n < N;
    }
    q.n = n;
    q.g = g;
    q.s = sidx;
    return q;
}

template <int D, int KV>
__global__ __launch_bounds__(kAttnWaves * 64, 1) void attn_token_kernel(AttnParams p) {
    const TokenSlot q = decode_token_slot(p);
    if (!q.live) return;                         // uniform over the workgroup
    attn_unit<D, false, KV>(p, q.n, q.g, q.s);
}

// The same, selecting the token's blocks from its score row first (MB <= 128).
template <int D, int KV>
__global__ __launch_bounds__(kAttnWaves * 64, 1) void attn_token_select_kernel(AttnParams p) {
    const TokenSlot q = decode_token_slot(p);
    if (!q.live) return;
    attn_unit<D, true, KV>(p, q.n, q.g, q.s);
}

// ------------------------------------------------------------------ VALU path

// one K/V element of type KVT (E_FP8 code, bf16 or f32) as float (exact)
template <int KVT>
__device__ __forceinline__ float load_elem(const void *base, int64_t i) {
    if constexpr (KVT == E_FP8) {
        const uint8_t c = ((const uint8_t *)base)[i];
        return fp8x2_to_f32x2<false>((uint32_t)c).x;
    } else if constexpr (KVT == E_BF16) {
        return __uint_as_float((uint32_t)((const uint16_t *)base)[i] << 16);
    } else {
        return ((const float *)base)[i];
    }
}

template <bool QBF16, int KVT, int D>
__global__ __launch_bounds__(256) void attn_valu_kernel(AttnParams p) {
    constexpr int DPL = D / 64;                    // output dims per lane
    constexpr int GMAX = 16;
    __shared__ uint32_t sel[kTokGroup][kMaxMB / 32];
    __shared__ uint16_t ulist[kMaxMB];
    __shared__ int ucount;
    __shared__ float qs[kTokGroup][D];
    __shared__ float pbuf[kTokGroup][kBlock];
    __shared__ float st_m[kTokGroup][GMAX], st_l[kTokGroup][GMAX];
    __shared__ float st_acc[kTokGroup][GMAX][D];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const Group q = decode_group(p);
    const int U = build_union(p, q, sel, ulist, &ucount);
    int beg, end;
    split_range(U, p.splits, q.s, beg, end);
    const int G = p.Hq / p.Hkv;
    const bool tok_active = wave < q.nt;
    const int64_t n = (int64_t)q.r * p.T + q.t0 + wave;
    const int vis = token_vis(p, q, wave);
    const int w = wave;
    const float scale2 = p.sm_scale * p.k_scale * kLog2e;
    if (tok_active) {
        for (int h = 0; h < G; ++h) {
            if (lane == 0) { st_m[w][h] = -INFINITY; st_l[w][h] = 0.f; }
            for (int d = lane; d < D; d += 64) st_acc[w][h][d] = 0.f;
        }
        wave_sync();
    }
    bool any = false;
    for (int b = beg; b < end; ++b) {
        const int j = ulist[b];
        if (!tok_active || !((sel[w][j >> 5] >> (j & 31)) & 1u)) continue;   // wave-uniform
        any = true;
        const int pid = p.bt[(int64_t)q.r * p.bt_sr + (int64_t)j * p.bt_sj];
        const int nk = min(kBlock, vis - j * kBlock);
        const int64_t kpage = (int64_t)pid * p.k_sp + (int64_t)q.g * p.k_sh;
        const int64_t vpage = (int64_t)pid * p.v_sp + (int64_t)q.g * p.v_sh;
        for (int hh = 0; hh < G; ++hh) {
            const int h = q.g * G + hh;
            for (int d = lane; d < D; d += 64) {
                float f;
                if constexpr (QBF16)
                    f = __uint_as_float((uint32_t)((const uint16_t *)p.q)[n * p.q_sn + h * p.q_sh + d] << 16);
                else
                    f = ((const float *)p.q)[n * p.q_sn + h * p.q_sh + d];
                qs[w][d] = f;
            }
            wave_sync();
            float lg[2];
            float bmax = -INFINITY;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int key = lane + 64 * e;
                float dot = 0.f;
                if (key < nk) {
                    for (int d = 0; d < D; ++d)
                        dot = fmaf(qs[w][d], load_elem<KVT>(p.k_cache, kpage + key * p.k_sb + d), dot);
                    lg[e] = dot * scale2;
                } else {
                    lg[e] = -INFINITY;
                }
                bmax = fmaxf(bmax, lg[e]);
            }
            bmax = group_max<64>(bmax);
            const float m_old = st_m[w][hh];
            const float m_new = fmaxf(m_old, bmax);
            const float alpha = exp2f(m_old - m_new);
            float ps = 0.f;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float pr = exp2f(lg[e] - m_new);
                pbuf[w][lane + 64 * e] = pr;
                ps += pr;
            }
            ps = group_sum<64>(ps);
            wave_sync();
#pragma unroll
            for (int e = 0; e < DPL; ++e) {
                const int d = lane + 64 * e;
                float a = st_acc[w][hh][d] * alpha;
                for (int key = 0; key < nk; ++key)
                    a = fmaf(pbuf[w][key], load_elem<KVT>(p.v_cache, vpage + key * p.v_sb + d), a);
                st_acc[w][hh][d] = a;
            }
            if (lane == 0) {
                st_m[w][hh] = m_new;
                st_l[w][hh] = st_l[w][hh] * alpha + ps;
            }
            wave_sync();
        }
    }
    if (!tok_active) return;
    const int64_t N = (int64_t)p.R * p.T;
    for (int hh = 0; hh < G; ++hh) {
        const int h = q.g * G + hh;
        if (lane == 0) {
            float *ml = p.part_ml + part_ml_index(q.s, n, h, N, p.Hq);
            ml[0] = any ? st_m[w][hh] : -INFINITY;
            ml[1] = any ? st_l[w][hh] : 0.f;
        }
        if (any)
            for (int d = lane; d < D; d += 64)
                p.part_acc[part_acc_index(q.s, n, h, d, N, p.Hq, D)] = st_acc[w][hh][d];
    }
}

// ------------------------------------------------------------------ reduction

// Split merge: four threads per (query token, head, 8 consecutive d), thread
// group q of the workgroup folding splits q, q + 4, q + 8, ... (all of its
// partial loads issued before they are combined, so that a merge costs about
// one memory round trip whatever the split count), then the four groups'
// results combined in group order through LDS.  The order is fixed
// (deterministic).  A split that saw no key has m = -inf and its acc is never
// read into the sum.
constexpr int kReduceOuts = 64;              // outputs (8-wide d groups) per workgroup
constexpr int kReduceGroups = 4;             // split groups per output

struct Fold {
    float m, l, a[8];
};

__device__ __forceinline__ void fold_in(Fold &f, float mu, float lu, const f32x4 &lo, const f32x4 &hi) {
    // mu = -inf: nothing to add (acc not read)
    const bool live = mu != -INFINITY;
    const float mn = fmaxf(f.m, live ? mu : -INFINITY);
    const float wo = (f.m == -INFINITY) ? 0.f : exp2_fast(f.m - mn);
    const float wn = live ? exp2_fast(mu - mn) : 0.f;
    f.l = f.l * wo + (live ? lu : 0.f) * wn;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f.a[e] = f.a[e] * wo + (live ? lo[e] : 0.f) * wn;
        f.a[4 + e] = f.a[4 + e] * wo + (live ? hi[e] : 0.f) * wn;
    }
    f.m = mn;
}

__global__ __launch_bounds__(kReduceOuts * kReduceGroups) void attn_reduce_kernel(ReduceParams p) {
    // thread -> (token n, 8-wide d group dq, head h), h fastest: the partial
    // loads of consecutive threads are contiguous
    __shared__ float sf[kReduceGroups - 1][10][kReduceOuts];
    const int DQ = p.D >> 3;
    const int o = threadIdx.x % kReduceOuts, q = threadIdx.x / kReduceOuts;
    const int64_t idx = (int64_t)blockIdx.x * kReduceOuts + o;
    const int64_t N = p.N;
    const bool live = idx < N * p.Hq * DQ;
    const int h = live ? (int)(idx % p.Hq) : 0;
    const int dq = live ? (int)((idx / p.Hq) % DQ) : 0;
    const int64_t n = live ? idx / ((int64_t)p.Hq * DQ) : 0;
    Fold f;
    f.m = -INFINITY;
    f.l = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f.a[e] = 0.f;
    if (live) {
        for (int s0 = q; s0 < p.splits; s0 += 4 * kReduceGroups) {
            f32x2 ml[4];
            f32x4 lo[4], hi[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int sp = min(s0 + u * kReduceGroups, p.splits - 1);
                ml[u] = *(const f32x2 *)(p.part_ml + part_ml_index(sp, n, h, N, p.Hq));
                const f32x4 *src = (const f32x4 *)(p.part_acc + part_acc_index(sp, n, h, dq * 8, N, p.Hq, p.D));
                lo[u] = src[0];
                hi[u] = src[1];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                fold_in(f, s0 + u * kReduceGroups < p.splits ? ml[u].x : -INFINITY, ml[u].y, lo[u], hi[u]);
        }
    }
    if (q > 0) {
        float *d = &sf[q - 1][0][o];
        d[0] = f.m;
        d[kReduceOuts] = f.l;
#pragma unroll
        for (int e = 0; e < 8; ++e) d[(2 + e) * kReduceOuts] = f.a[e];
    }
    __syncthreads();
    if (q > 0 || !live) return;
#pragma unroll
    for (int g = 0; g < kReduceGroups - 1; ++g) {
        const float *d = &sf[g][0][o];
        fold_in(f, d[0], d[kReduceOuts], f32x4{d[2 * kReduceOuts], d[3 * kReduceOuts], d[4 * kReduceOuts],
                                               d[5 * kReduceOuts]},
                f32x4{d[6 * kReduceOuts], d[7 * kReduceOuts], d[8 * kReduceOuts], d[9 * kReduceOuts]});
    }
    const float inv = (f.l > 0.f) ? p.v_scale / f.l : 0.f;
    const int64_t base = n * p.o_sn + (int64_t)h * p.o_sh + (int64_t)(dq * 8) * p.o_sd;
    if (p.out_bf16) {
        uint16_t *op = (uint16_t *)p.out;
        if (p.o_sd == 1) {
            uint4 v;
            v.x = cvt_pk_bf16(f.a[0] * inv, f.a[1] * inv);
            v.y = cvt_pk_bf16(f.a[2] * inv, f.a[3] * inv);
            v.z = cvt_pk_bf16(f.a[4] * inv, f.a[5] * inv);
            v.w = cvt_pk_bf16(f.a[6] * inv, f.a[7] * inv);
            *(uint4 *)(op + base) = v;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) op[base + e * p.o_sd] = (uint16_t)cvt_pk_bf16(f.a[e] * inv, 0.f);
        }
    } else {
        float *op = (float *)p.out;
#pragma unroll
        for (int e = 0; e < 8; ++e) op[base + e * p.o_sd] = f.a[e] * inv;
    }
}

// grid of the token kernels: 8 XCDs x units per XCD x splits (see decode_token_slot)
static int64_t token_grid(const AttnParams &p) {
    const int64_t N = (int64_t)p.R * p.T;
    const int64_t units_per_xcd = (p.R >= 8) ? (int64_t)((p.R + 7) / 8) * p.T * p.Hkv
                                             : (N * p.Hkv + 7) / 8;
    return 8 * units_per_xcd * p.splits;
}

// dynamic LDS of the token kernel: the selection row, block table and
// first-entry tables for selections of more than 256 entries or tables of
// more than 128 blocks (see attn_unit)
static size_t token_xtab_bytes(const AttnParams &p) {
    return (p.k > 256 || p.MB > 128) ? (size_t)3 * kMaxMB * sizeof(int) : 0;
}

template <int D, int KV>
hipError_t launch_token(const AttnParams &p, hipStream_t s) {
    hipLaunchKernelGGL((attn_token_kernel<D, KV>), dim3((unsigned)token_grid(p)), dim3(kAttnWaves * 64),
                       token_xtab_bytes(p), s, p);
    return hipGetLastError();
}

template <int D, int KV>
hipError_t launch_token_select(const AttnParams &p, hipStream_t s) {
    hipLaunchKernelGGL((attn_token_select_kernel<D, KV>), dim3((unsigned)token_grid(p)), dim3(kAttnWaves * 64), 0, s, p);
    return hipGetLastError();
}

template <bool QB, int KVT, int D>
hipError_t launch_valu(const AttnParams &p, int64_t grid, hipStream_t s) {
    hipLaunchKernelGGL((attn_valu_kernel<QB, KVT, D>), dim3((unsigned)grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_valu_types(const AttnParams &p, int qt, int kt, int64_t grid, hipStream_t s) {
    const bool qb = qt == E_BF16;
    switch (kt) {
    case E_FP8: return qb ? launch_valu<true, E_FP8, D>(p, grid, s) : launch_valu<false, E_FP8, D>(p, grid, s);
    case E_BF16: return qb ? launch_valu<true, E_BF16, D>(p, grid, s) : launch_valu<false, E_BF16, D>(p, grid, s);
    case E_F32: return qb ? launch_valu<true, E_F32, D>(p, grid, s) : launch_valu<false, E_F32, D>(p, grid, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

// union VALU path: enough (row, KV head, token group, split) workgroups for the chip
static int union_splits(int32_t R, int32_t T, int32_t Hkv, int32_t k) {
    const int64_t TG = (T + kTokGroup - 1) / kTokGroup;
    const int64_t groups = (int64_t)R * Hkv * TG;
    const int64_t maxU = (int64_t)min(T, kTokGroup) * k;
    int64_t S = groups > 0 ? (kSplitTargetWGs + groups - 1) / groups : 1;
    S = S > maxU ? maxU : S;
    return (int)(S < 1 ? 1 : S);
}

// token path: 4 page slots per workgroup, bpw selected pages per slot, and
// about one workgroup per CU: S splits of epw selection entries per (token,
// KV head) unit, at most kTokenMaxSplits (the last workgroup of a unit merges
// all S partials).  A slot streams its pages back to back, so one round of
// workgroups with several pages per slot costs less than several rounds; a
// small batch takes fewer than 4 entries per split (down to two pages per
// workgroup at the cap of 8 splits: more splits would leave each token's last
// workgroup taking in more partials than it streams pages) so that its few
// units still spread over many CUs.
static void token_split(int64_t units, int32_t k, int32_t *S, int32_t *bpw, int32_t *epw) {
    int64_t s = units > 0 ? (kSplitTargetWGs + units - 1) / units : 1;
    s = s > k ? k : s;
    s = s > kTokenMaxSplits ? kTokenMaxSplits : s;
    s = s < 1 ? 1 : s;
    int64_t e = (k + s - 1) / s;                 // entries per split
    e = e < 1 ? 1 : e;
    *epw = (int32_t)e;
    *bpw = (int32_t)((e + 3) / 4);
    *S = (int32_t)((k + e - 1) / e);
    *S = *S < 1 ? 1 : *S;
}

bool attention_uses_mfma(int q_type, int kv_type, int G) {
    return G == 16 && q_type == E_BF16 && (kv_type == E_FP8 || kv_type == E_BF16);
}

AttnPlan attn_plan(int32_t R, int32_t T, int32_t Hq, int32_t Hkv, int32_t D, int32_t MB, int32_t k,
                   bool sel_per_row, float score_scale, int q_type, int kv_type) {
    AttnPlan pl;
    pl.mfma = attention_uses_mfma(q_type, kv_type, Hq / Hkv);
    pl.row = attention_row_eligible(q_type, kv_type, D, Hq / Hkv, T, MB, k, sel_per_row, score_scale);
    if (pl.row) {
        pl.splits = row_splits(R, Hkv);
        pl.bpw = 1;
        pl.epw = 0;
    } else if (pl.mfma) {
        token_split((int64_t)R * T * Hkv, k, &pl.splits, &pl.bpw, &pl.epw);
    } else {
        pl.splits = union_splits(R, T, Hkv, k);
        pl.bpw = 1;
        pl.epw = 4;
    }
    return pl;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// [counters N*Hkv x 256 B][(m, l) S*N*Hq pairs][acc S*N*Hq*D], each 256-byte aligned.
// The size covers both paths (the query does not know the element types).
size_t attn_workspace_bytes(int32_t R, int32_t T, int32_t Hq, int32_t Hkv, int32_t D, int32_t k) {
    int32_t St, bpw, epw;
    token_split((int64_t)R * T * Hkv, k, &St, &bpw, &epw);
    const int32_t Su = union_splits(R, T, Hkv, k);
    size_t S = (size_t)(St > Su ? St : Su);
    // the row-level kernel's splits (it may serve 2 <= T <= 4 with k <= 128)
    if (T >= 2 && T <= 4 && k <= kSelSlots) S = S > (size_t)row_splits(R, Hkv) ? S : (size_t)row_splits(R, Hkv);
    const size_t N = (size_t)R * T;
    const size_t rows = S * N * Hq;
    return N * Hkv * kCounterStride * 4 + align256(rows * 8) + align256(rows * D * 4);
}

// The same layout for a plan with S splits (what the call actually touches),
// with room for at least `counter_slots` arrival counters.
size_t attn_workspace_bytes_for_splits(int32_t S, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                                       int32_t counter_slots) {
    const size_t rows = (size_t)S * N * Hq;
    const size_t ctr = (size_t)(N * Hkv > counter_slots ? N * Hkv : counter_slots);
    return ctr * kCounterStride * 4 + align256(rows * 8) + align256(rows * D * 4);
}

// counter_slots: the counter region holds max(N*Hkv, counter_slots) counters
// (a fixed region keeps the counters of calls of different sizes in one place)
void attn_carve_workspace(void *ws, int32_t S, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                          int32_t counter_slots, float **ml, float **acc, int32_t **counters) {
    const size_t rows = (size_t)S * N * Hq;
    const size_t ctr = (size_t)(N * Hkv > counter_slots ? N * Hkv : counter_slots);
    char *b = (char *)ws;
    *counters = (int32_t *)b;
    b += ctr * kCounterStride * 4;
    *ml = (float *)b;
    *acc = (float *)(b + align256(rows * 8));
    (void)D;
}

bool attention_supported(int q_type, int kv_type, int D, int G) {
    if (!((q_type == E_F32 || q_type == E_BF16) && (kv_type == E_F32 || kv_type == E_BF16 || kv_type == E_FP8)))
        return false;
    if (!(D == 64 || D == 128)) return false;
    return G >= 1 && G <= 16;
}

hipError_t launch_attention(const AttnParams &p, int q_type, int kv_type, int D, hipStream_t s) {
    const int TG = (p.T + kTokGroup - 1) / kTokGroup;
    const int64_t grid = (int64_t)p.R * p.Hkv * TG * p.splits;
    if (grid == 0) return hipSuccess;
    const int G = p.Hq / p.Hkv;
    if (attention_uses_mfma(q_type, kv_type, G)) {
        if (kv_type == E_BF16) return D == 64 ? launch_token<64, E_BF16>(p, s) : launch_token<128, E_BF16>(p, s);
        return D == 64 ? launch_token<64, E_FP8>(p, s) : launch_token<128, E_FP8>(p, s);
    }
    return D == 64 ? launch_valu_types<64>(p, q_type, kv_type, grid, s)
                   : launch_valu_types<128>(p, q_type, kv_type, grid, s);
}

hipError_t launch_attention_select(const AttnParams &p, int D, int kv_type, hipStream_t s) {
    if ((int64_t)p.R * p.T * p.Hkv == 0) return hipSuccess;
    if (p.MB > kSelSlots || p.k > p.MB) return hipErrorInvalidValue;
    if (kv_type == E_BF16)
        return D == 64 ? launch_token_select<64, E_BF16>(p, s) : launch_token_select<128, E_BF16>(p, s);
    return D == 64 ? launch_token_select<64, E_FP8>(p, s) : launch_token_select<128, E_FP8>(p, s);
}

hipError_t launch_reduce(const ReduceParams &p, hipStream_t s) {
    const int64_t total = (int64_t)p.N * p.Hq * (p.D / 8);
    if (total == 0) return hipSuccess;
    const int64_t grid = (total + kReduceOuts - 1) / kReduceOuts;
    // v_scale is applied at the merge: out = v_scale * sum w acc / sum w l
    hipLaunchKernelGGL(attn_reduce_kernel, dim3((unsigned)grid), dim3(kReduceOuts * kReduceGroups), 0, s, p);
    return hipGetLastError();
}

}  // namespace msa
