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
#include "device_util.h"
#include "msa_internal.h"

namespace msa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int clamp_len(int L, int MB) { return max(0, min(L, MB * kBlock)); }

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
        const int j = p.topk[(n0 + t) * p.tk_sn + (int64_t)i * p.tk_si];
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
// One workgroup per (query token n, KV head g, split s of n's selection list);
// wave w of the workgroup takes selection entries s*4*bpw + w*bpw .. +bpw.  A
// wave's page goes
//   K -> straight from HBM into MFMA A-operand registers (lane = key row,
//        32 contiguous bytes of d per lane), decoded FP8 -> bf16 per k-step;
//   V -> straight from HBM into the wave's LDS slot (direct-to-LDS 16-byte
//        loads, row-major, 16-byte chunks XOR-swizzled by key), then read back
//        with ds_read_b64_tr_b8, which hands each lane 8 keys at one d: the
//        A operand of O^T = V^T P^T.
// The 4 waves merge their softmax partials in LDS; the splits of a token merge
// through a per-(token, KV head) arrival counter in the workspace: the last
// workgroup to arrive combines the S partials in a fixed order and writes the
// output, then resets the counter to zero (so the counters are zero again
// after every call).  Workgroups are placed so that all those of a row (at
// least 8 rows) or of a token run on one XCD and share its L2: a page chosen
// by several of a row's tokens is then fetched from HBM once.  Correctness
// does not depend on the placement (the hand-off below is device-coherent).

typedef int v2i __attribute__((ext_vector_type(2)));

// cache policy of the page loads: non-temporal (each page is used once per call)
constexpr int kNonTemporal = 2;

// Device-coherent single-element accesses (relaxed, agent scope): sc1 loads and
// stores, no cache-maintenance fences.
__device__ __forceinline__ void st_coherent(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// V page in LDS: [128 keys][D bytes], 16-byte chunk c of key k stored at c ^ swz(k).
// swz separates the 8 keys one ds_read_b64_tr_b8 group touches (keys 4a..4a+3 and
// 16+4a..16+4a+3 of a 32-key chunk) onto distinct chunk positions.
__device__ __forceinline__ int vswz(int key) { return (key & 3) | (((key >> 4) & 1) << 2); }

// PV k-order inside a 32-key chunk: MFMA k index 8*grp + e holds key
//   e < 4 : 4*grp + e            (QK accumulator tile 2c,   row 4*grp + e)
//   e >= 4: 16 + 4*grp + (e - 4) (QK accumulator tile 2c+1, row 4*grp + e - 4)
__device__ __forceinline__ int pv_key(int grp, int e) {
    return (e < 4) ? 4 * grp + e : 16 + 4 * grp + (e - 4);
}

__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
    uint4 r;
    r.x = fp8x2_to_bf16x2<false>(lo);
    r.y = fp8x2_to_bf16x2<true>(lo);
    r.z = fp8x2_to_bf16x2<false>(hi);
    r.w = fp8x2_to_bf16x2<true>(hi);
    return r;
}

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

template <int D>
__global__ __launch_bounds__(256, 1) void attn_token_kernel(AttnParams p) {
    constexpr int KS = D / 32;          // k-steps of the QK product
    constexpr int DT = D / 16;          // 16-row d tiles of the PV product
    constexpr int PB = kBlock * D;      // bytes of one K or V page (one KV head)
    constexpr int LOADS = PB / 1024;    // 1 KiB direct-to-LDS loads per page
    constexpr int CPR = D / 16;         // 16-byte chunks per key row
    // per wave: [K page | V page]; the 4-wave merge reuses the space afterwards
    __shared__ __attribute__((aligned(16))) uint8_t lds[4][2 * PB];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const TokenSlot q = decode_token_slot(p);
    if (!q.live) return;                         // uniform over the workgroup
    const int n = q.n, g = q.g;
    const int r = n / p.T, t = n % p.T;
    const int per_wg = 4 * p.bpw;
    const int e0 = q.s * per_wg;
    const int e1 = min(p.k, e0 + per_wg);

    // One round trip for the small inputs: seq_len, the selection row up to e1
    // (lane l holds entries l + 64c) and the row's block table (lane l holds
    // logical blocks l and l + 64).
    const int64_t trow = (int64_t)n * p.tk_sn;
    int tkv[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int idx = lane + 64 * c;
        tkv[c] = idx < e1 ? p.topk[trow + (int64_t)idx * p.tk_si] : -1;
    }
    int btv[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int jj = lane + 64 * c;
        btv[c] = jj < p.MB ? p.bt[(int64_t)r * p.bt_sr + (int64_t)jj * p.bt_sj] : -1;
    }
    const int L = clamp_len(p.seq_lens[(int64_t)r * p.sl_s], p.MB);
    const int vis = max(0, L - (p.T - 1 - t));

    const int h0 = g * 16;
    // B operand of S^T = K Q^T for k-step ks: lane holds q[n][h0 + lane%16][d],
    // d = (D/4)*(lane/16) + 8*ks + e   (the same d order as the K operand below)
    uint4 qf[KS];
    {
        const uint16_t *qp = (const uint16_t *)p.q + (int64_t)n * p.q_sn + (int64_t)(h0 + (lane & 15)) * p.q_sh;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = *(const uint4 *)(qp + (D / 4) * (lane >> 4) + 8 * ks);
    }
    const float scale2 = p.sm_scale * p.k_scale * kLog2e;
    float m_run = -INFINITY, l_run = 0.f;
    f32x4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint8_t *kw = lds[wave];
    uint8_t *vw = lds[wave] + PB;
    const int grp = lane >> 4, li = lane & 15;
    for (int b = 0; b < p.bpw; ++b) {
        const int i = e0 + wave * p.bpw + b;
        if (i >= e1) break;
        // entry i and duplicate check against entries [0, i)  (wave-uniform)
        int j;
        bool dup = false;
        if (i < 256) {
            const int c = i >> 6;
            const int src = c == 0 ? tkv[0] : c == 1 ? tkv[1] : c == 2 ? tkv[2] : tkv[3];
            j = __builtin_amdgcn_readlane(src, i & 63);
#pragma unroll
            for (int c2 = 0; c2 < 4; ++c2) dup |= __ballot(lane + 64 * c2 < i && tkv[c2] == j) != 0;
        } else {
            j = p.topk[trow + (int64_t)i * p.tk_si];
            for (int c2 = 0; c2 * 64 < i; ++c2) {
                const int idx = c2 * 64 + lane;
                const int v = (idx < i) ? p.topk[trow + (int64_t)idx * p.tk_si] : -1;
                dup |= __ballot(idx < i && v == j) != 0;
            }
        }
        if (dup || j < 0 || j >= p.MB || j * kBlock >= vis) continue;
        int pid;
        if (j < 128) {
            pid = __builtin_amdgcn_readlane(j < 64 ? btv[0] : btv[1], j & 63);
        } else {
            pid = p.bt[(int64_t)r * p.bt_sr + (int64_t)j * p.bt_sj];
        }
        if (pid < 0 || pid >= p.P) continue;
        const uint8_t *kp = (const uint8_t *)p.k_cache + (int64_t)pid * p.k_sp + (int64_t)g * p.k_sh;
        const uint8_t *vp = (const uint8_t *)p.v_cache + (int64_t)pid * p.v_sp + (int64_t)g * p.v_sh;
        // K then V into the wave's LDS slots: load ld covers keys 64*ld/CPR .. and
        // lane -> (key, chunk slot); K chunks swizzled by key & 7, V by vswz(key).
        // For a given lane the key advances by 64/CPR per load and the swizzle
        // depends only on the lane (K) or on the lane and bit 1 of ld (V, D=128).
        {
            constexpr int KPL = 64 / CPR;                       // keys per load
            const int key0 = lane / CPR, slot = lane % CPR;
            const uint8_t *ka = kp + (int64_t)key0 * p.k_sb + ((slot ^ (key0 & (CPR - 1) & 7)) << 4);
            const int64_t kstep = (int64_t)KPL * p.k_sb;
#pragma unroll
            for (int ld = 0; ld < LOADS; ++ld)
                __builtin_amdgcn_global_load_lds((const void *)(ka + ld * kstep),
                                                 (__attribute__((address_space(3))) void *)(kw + ld * 1024),
                                                 16, 0, kNonTemporal);
            const int64_t vstep = (int64_t)KPL * p.v_sb;
#pragma unroll
            for (int ld = 0; ld < LOADS; ++ld) {
                const int key = ld * KPL + key0;
                const uint8_t *va = vp + (int64_t)key0 * p.v_sb + ((slot ^ (vswz(key) & (CPR - 1))) << 4);
                __builtin_amdgcn_global_load_lds((const void *)(va + ld * vstep),
                                                 (__attribute__((address_space(3))) void *)(vw + ld * 1024),
                                                 16, 0, kNonTemporal);
            }
        }
        // K landed when at most the V loads are outstanding
        if constexpr (LOADS == 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        // S^T tiles: acc[kt][e] = q . k for key 16*kt + 4*grp + e, head h0 + lane%16.
        // A operand: key 16*kt + lane%16, d = (D/4)*grp + 8*ks .. +8
        const int kbase = j * kBlock;
        f32x4 sacc[8];
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) {
            const int key = kt * 16 + li;
            const uint8_t *krow = kw + key * D;
            const int ksw = key & (CPR - 1) & 7;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kp2 = 0; kp2 < KS / 2; ++kp2) {
                const int chunk = ((D / 4) * grp) / 16 + kp2;
                const uint4 raw = *(const uint4 *)(krow + ((chunk ^ ksw) << 4));
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, fp8x8_to_bf16x8(raw.x, raw.y)),
                    __builtin_bit_cast(bf16x8, qf[2 * kp2]), acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, fp8x8_to_bf16x8(raw.z, raw.w)),
                    __builtin_bit_cast(bf16x8, qf[2 * kp2 + 1]), acc, 0, 0, 0);
            }
            sacc[kt] = acc * scale2;
        }
        // visibility mask only where the page is not entirely visible (uniform)
        const bool full = kbase + kBlock <= vis;
        if (!full) {
#pragma unroll
            for (int kt = 0; kt < 8; ++kt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sacc[kt][e] = (kbase + kt * 16 + 4 * grp + e < vis) ? sacc[kt][e] : -INFINITY;
        }
        float bmax = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 8; ++kt)
            bmax = fmaxf(bmax, fmaxf(fmaxf(sacc[kt][0], sacc[kt][1]), fmaxf(sacc[kt][2], sacc[kt][3])));
        bmax = max_across_groups<16>(bmax);
        const float m_new = fmaxf(m_run, bmax);
        const float alpha = exp2_fast(m_run - m_new);
        m_run = m_new;
        // P rounded to bf16 (hardware RNE); l sums the rounded values so that the
        // weights used in PV and in the normaliser are the same numbers
        uint32_t pb[8][2];
        float lsum = 0.f;
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) {
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const uint32_t w = cvt_pk_bf16(exp2_fast(sacc[kt][2 * h2] - m_new),
                                               exp2_fast(sacc[kt][2 * h2 + 1] - m_new));
                pb[kt][h2] = w;
                lsum += __uint_as_float(w << 16) + __uint_as_float(w & 0xffff0000u);
            }
        }
        l_run = l_run * alpha + lsum;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
        // V rows past seq_len hold arbitrary bytes (NaN poison in the tests);
        // their P is 0, but 0 * NaN would poison the sum, so such keys are
        // dropped from the operand (only the page holding seq_len needs it).
        const int vvalid = L - kbase;
        const bool vfull = vvalid >= kBlock;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint4 bp = make_uint4(pb[2 * c][0], pb[2 * c][1], pb[2 * c + 1][0], pb[2 * c + 1][1]);
            // lanes 2b, 2b+1 of a 16-lane group read the two 8-byte halves of
            // key pv_key(grp, b)'s 16-byte chunk dt
            const int key = 32 * c + pv_key(grp, li >> 1);
            const uint8_t *vrow = vw + key * D + 8 * (li & 1);
            const int vsw = vswz(key) & (CPR - 1);
            uint32_t kill_lo = 0u, kill_hi = 0u;
            if (!vfull) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const bool dead = 32 * c + pv_key(grp, e) >= vvalid;
                    if (e < 4) kill_lo |= dead ? (0xffu << (8 * e)) : 0u;
                    else kill_hi |= dead ? (0xffu << (8 * (e - 4))) : 0u;
                }
            }
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const v2i raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (__attribute__((address_space(3))) v2i *)(vrow + ((dt ^ vsw) << 4)));
                const uint4 a = fp8x8_to_bf16x8((uint32_t)raw.x & ~kill_lo, (uint32_t)raw.y & ~kill_hi);
                o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                                __builtin_bit_cast(bf16x8, bp), o[dt], 0, 0, 0);
            }
        }
    }
    // full per-head sum over the wave's four lane groups
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);

    // ---- merge the 4 waves (LDS), then either write out or a split partial
    __syncthreads();                                   // all K/V reads done
    float *mo = (float *)&lds[0][0];                   // [4 waves][D][16 heads]
    float *mm = mo + 4 * D * 16;                       // [4 waves][16]
    float *ml = mm + 4 * 16;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) mo[(wave * D + dt * 16 + 4 * grp + e) * 16 + li] = o[dt][e];
    if (lane < 16) {
        mm[wave * 16 + lane] = m_run;
        ml[wave * 16 + lane] = l_tot;
    }
    __syncthreads();
    // thread -> (head hh, 8-wide d group dq); D/8 groups x 16 heads = 256 (D=128)
    constexpr int DQ = D / 8;
    const int hh = tid & 15, dq = tid >> 4;
    const bool active = dq < DQ;
    float mw[4], wsum = 0.f, mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) { mw[w] = mm[w * 16 + hh]; mx = fmaxf(mx, mw[w]); }
    float acc8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc8[e] = 0.f;
    float lm = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float wgt = exp2_fast(mw[w] - mx);       // -inf -> 0
            lm += wgt * ml[w * 16 + hh];
            wsum += wgt;
            if (active)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc8[e] += wgt * mo[(w * D + dq * 8 + e) * 16 + hh];
        }
    }
    (void)wsum;
    const int h = h0 + hh;
    auto write_out = [&](const float *a, float lsum) {
        const float inv = (lsum > 0.f) ? p.v_scale / lsum : 0.f;
        const int64_t base = (int64_t)n * p.o_sn + (int64_t)h * p.o_sh + (int64_t)(dq * 8) * p.o_sd;
        if (p.out_bf16) {
            uint16_t *op = (uint16_t *)p.out;
#pragma unroll
            for (int e = 0; e < 8; ++e) op[base + e * p.o_sd] = (uint16_t)cvt_pk_bf16(lsum > 0.f ? a[e] * inv : 0.f, 0.f);
        } else {
            float *op = (float *)p.out;
#pragma unroll
            for (int e = 0; e < 8; ++e) op[base + e * p.o_sd] = lsum > 0.f ? a[e] * inv : 0.f;
        }
    };
    if (p.splits == 1) {
        if (active) write_out(acc8, lm);
        return;
    }
    // Split hand-off.  Partials are written and read with device-coherent
    // (sc1) accesses and the arrival counter is a device-scope atomic, so the
    // workgroups of one token may sit on different XCDs; no fence (which would
    // write back and invalidate the whole L2) is needed: each writer waits for
    // its stores to complete before the workgroup's single counter increment.
    const int64_t N = (int64_t)p.R * p.T;
    const int64_t row = (int64_t)n * p.Hq + h;
    if (active) {
        float *dst = p.part_acc + ((int64_t)q.s * N * p.Hq + row) * D + dq * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) st_coherent(dst + e, acc8[e]);
        if (dq == 0) {
            st_coherent(p.part_m + (int64_t)q.s * N * p.Hq + row, mx);
            st_coherent(p.part_l + (int64_t)q.s * N * p.Hq + row, lm);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    __shared__ int last;
    int *ctr = p.counters + (int64_t)n * p.Hkv + g;
    if (tid == 0) {
        const int old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = (old == p.splits - 1);
    }
    __syncthreads();
    if (!last) return;
    if (active) {
        // every split wrote (m, l, acc) (m = -inf, l = 0, acc = 0 when empty):
        // load them all at once, weight with selects, sum in split order
        const int S = p.splits;
        float m2 = -INFINITY, l2 = 0.f, a2[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) a2[e] = 0.f;
        for (int s0 = 0; s0 < S; s0 += 4) {
            float ms[4], ls[4], as[4][8];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int sp = min(s0 + u, S - 1);
                const int64_t srow = (int64_t)sp * N * p.Hq + row;
                ms[u] = (s0 + u < S) ? ld_coherent(p.part_m + srow) : -INFINITY;
                ls[u] = ld_coherent(p.part_l + srow);
#pragma unroll
                for (int e = 0; e < 8; ++e) as[u][e] = ld_coherent(p.part_acc + srow * D + dq * 8 + e);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float mn = fmaxf(m2, ms[u]);
                const float wo = (m2 == -INFINITY) ? 0.f : exp2_fast(m2 - mn);
                const float wn = (ms[u] == -INFINITY) ? 0.f : exp2_fast(ms[u] - mn);
                l2 = l2 * wo + ls[u] * wn;
#pragma unroll
                for (int e = 0; e < 8; ++e) a2[e] = a2[e] * wo + as[u][e] * wn;
                m2 = mn;
            }
        }
        write_out(a2, l2);
    }
    if (tid == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ VALU path

template <bool QBF16, bool KVFP8>
__device__ __forceinline__ float load_elem(const void *base, int64_t i) {
    if constexpr (KVFP8) {
        const uint8_t c = ((const uint8_t *)base)[i];
        return fp8x2_to_f32x2<false>((uint32_t)c).x;
    } else {
        return ((const float *)base)[i];
    }
}

template <bool QBF16, bool KVFP8, int D>
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
                        dot = fmaf(qs[w][d], load_elem<QBF16, KVFP8>(p.k_cache, kpage + key * p.k_sb + d), dot);
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
                    a = fmaf(pbuf[w][key], load_elem<QBF16, KVFP8>(p.v_cache, vpage + key * p.v_sb + d), a);
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
    for (int hh = 0; hh < G; ++hh) {
        const int64_t row = ((int64_t)q.s * (p.R * p.T) + n) * p.Hq + q.g * G + hh;
        if (lane == 0) {
            p.part_m[row] = any ? st_m[w][hh] : -INFINITY;
            p.part_l[row] = any ? st_l[w][hh] : 0.f;
        }
        if (any)
            for (int d = lane; d < D; d += 64) p.part_acc[row * D + d] = st_acc[w][hh][d];
    }
}

// ------------------------------------------------------------------ reduction

__global__ __launch_bounds__(256) void attn_reduce_kernel(ReduceParams p) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)p.N * p.Hq * p.D;
    if (idx >= total) return;
    const int d = (int)(idx % p.D);
    const int64_t nh = idx / p.D;                 // n * Hq + h
    const int h = (int)(nh % p.Hq);
    const int64_t n = nh / p.Hq;
    const int64_t NH = (int64_t)p.N * p.Hq;
    float mx = -INFINITY;
    for (int s = 0; s < p.splits; ++s) mx = fmaxf(mx, p.part_m[s * NH + nh]);
    float num = 0.f, den = 0.f;
    if (mx != -INFINITY) {
        for (int s = 0; s < p.splits; ++s) {
            const float ms = p.part_m[s * NH + nh];
            if (ms == -INFINITY) continue;
            const float wgt = exp2f(ms - mx);
            num = fmaf(wgt, p.part_acc[(s * NH + nh) * p.D + d], num);
            den = fmaf(wgt, p.part_l[s * NH + nh], den);
        }
    }
    const float o = (den > 0.f) ? p.v_scale * (num / den) : 0.f;
    const int64_t off = n * p.o_sn + (int64_t)h * p.o_sh + (int64_t)d * p.o_sd;
    if (p.out_bf16)
        ((uint16_t *)p.out)[off] = (uint16_t)f32_to_bf16_rne(o);
    else
        ((float *)p.out)[off] = o;
}

template <int D>
hipError_t launch_token(const AttnParams &p, hipStream_t s) {
    const int64_t N = (int64_t)p.R * p.T;
    const int64_t units_per_xcd = (p.R >= 8) ? (int64_t)((p.R + 7) / 8) * p.T * p.Hkv
                                             : (N * p.Hkv + 7) / 8;
    const int64_t grid = 8 * units_per_xcd * p.splits;
    hipLaunchKernelGGL((attn_token_kernel<D>), dim3((unsigned)grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

template <bool QB, bool KF, int D>
hipError_t launch_valu(const AttnParams &p, int64_t grid, hipStream_t s) {
    hipLaunchKernelGGL((attn_valu_kernel<QB, KF, D>), dim3((unsigned)grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_valu_types(const AttnParams &p, int qt, int kt, int64_t grid, hipStream_t s) {
    const bool qb = qt == E_BF16, kf = kt == E_FP8;
    if (qb && kf) return launch_valu<true, true, D>(p, grid, s);
    if (qb) return launch_valu<true, false, D>(p, grid, s);
    if (kf) return launch_valu<false, true, D>(p, grid, s);
    return launch_valu<false, false, D>(p, grid, s);
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

// token path: one selected page per wave while k <= 64, 4 waves per workgroup
static void token_split(int32_t k, int32_t *S, int32_t *bpw) {
    *bpw = (k + 63) / 64;
    *S = (k + 4 * *bpw - 1) / (4 * *bpw);
}

bool attention_uses_mfma(int q_type, int kv_type, int G) {
    return G == 16 && q_type == E_BF16 && kv_type == E_FP8;
}

AttnPlan attn_plan(int32_t R, int32_t T, int32_t Hq, int32_t Hkv, int32_t k, int q_type, int kv_type) {
    AttnPlan pl;
    pl.mfma = attention_uses_mfma(q_type, kv_type, Hq / Hkv);
    if (pl.mfma) {
        token_split(k, &pl.splits, &pl.bpw);
    } else {
        pl.splits = union_splits(R, T, Hkv, k);
        pl.bpw = 1;
    }
    return pl;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// [counters N*Hkv i32][m S*N*Hq][l S*N*Hq][acc S*N*Hq*D], each 256-byte aligned.
// The size covers both paths (the query does not know the element types).
size_t attn_workspace_bytes(int32_t R, int32_t T, int32_t Hq, int32_t Hkv, int32_t D, int32_t k) {
    int32_t St, bpw;
    token_split(k, &St, &bpw);
    const int32_t Su = union_splits(R, T, Hkv, k);
    const size_t S = (size_t)(St > Su ? St : Su);
    const size_t N = (size_t)R * T;
    const size_t rows = S * N * Hq;
    return align256(N * Hkv * 4) + 2 * align256(rows * 4) + align256(rows * D * 4);
}

void attn_carve_workspace(void *ws, int32_t S, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                          float **m, float **l, float **acc, int32_t **counters) {
    const size_t rows = (size_t)S * N * Hq;
    char *b = (char *)ws;
    *counters = (int32_t *)b;
    b += align256((size_t)N * Hkv * 4);
    *m = (float *)b;
    *l = (float *)(b + align256(rows * 4));
    *acc = (float *)(b + 2 * align256(rows * 4));
    (void)D;
}

bool attention_supported(int q_type, int kv_type, int D, int G) {
    if (!((q_type == E_F32 || q_type == E_BF16) && (kv_type == E_F32 || kv_type == E_FP8)))
        return false;
    if (!(D == 64 || D == 128)) return false;
    return G >= 1 && G <= 16;
}

hipError_t launch_attention(const AttnParams &p, int q_type, int kv_type, int D, hipStream_t s) {
    const int TG = (p.T + kTokGroup - 1) / kTokGroup;
    const int64_t grid = (int64_t)p.R * p.Hkv * TG * p.splits;
    if (grid == 0) return hipSuccess;
    const int G = p.Hq / p.Hkv;
    if (attention_uses_mfma(q_type, kv_type, G))
        return D == 64 ? launch_token<64>(p, s) : launch_token<128>(p, s);
    return D == 64 ? launch_valu_types<64>(p, q_type, kv_type, grid, s)
                   : launch_valu_types<128>(p, q_type, kv_type, grid, s);
}

hipError_t launch_reduce(const ReduceParams &p, hipStream_t s) {
    const int64_t total = (int64_t)p.N * p.Hq * p.D;
    if (total == 0) return hipSuccess;
    const int64_t grid = (total + 255) / 256;
    // v_scale is applied at the merge: out = v_scale * sum w acc / sum w l
    hipLaunchKernelGGL(attn_reduce_kernel, dim3((unsigned)grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace msa
