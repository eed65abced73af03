// The per-token MFMA attention unit behind msa_sparse_decode and the
// attention launch of msa_decode_step (see attend.hip for the work split).
#pragma once

#include "device_util.h"
#include "msa_internal.h"
#include "select_unit.h"

namespace msa {

__device__ __forceinline__ int clamp_len(int L, int MB) { return max(0, min(L, MB * kBlock)); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kSelSlots = 128;      // per-wave selection slots (k <= MB <= 128)

//
// One workgroup per (query token n, KV head g, split s of n's selection list);
// wave w of the workgroup takes selection entries s*4*bpw + w*bpw .. +bpw.  A
// wave's K and V pages go straight from HBM into the wave's LDS slots
// (direct-to-LDS 16-byte non-temporal loads, row-major, 16-byte chunks
// XOR-swizzled by key), then
//   K -> read back row-wise as the MFMA A operand of S^T = K Q^T (lane = key
//        row), decoded FP8 -> bf16 per k-step;
//   V -> read back with ds_read_b64_tr_b8, which hands each lane 8 keys at one
//        d: the A operand of O^T = V^T P^T.
// The 4 waves merge their softmax partials in LDS.  The splits of a token are
// then merged either by the separate merge kernel (each workgroup leaves a
// partial) or in this launch through a per-(token, KV head) arrival counter in
// the workspace: the last workgroup to arrive combines the S partials in a
// fixed order, writes the output and resets the counter to zero (so the
// counters are zero again after every call).  Workgroups are placed so that
// all those of a row (at least 8 rows) or of a token run on one XCD and share
// its L2: a page chosen by several of a row's tokens is then fetched from HBM
// once.  Correctness does not depend on the placement.

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

// MERGE: splits of a token are combined in this launch by the last workgroup
// to arrive; otherwise each workgroup leaves its partial for the separate
// merge kernel.
// SEL: the token's selection is computed here from its score row (MB <= 128;
// every wave redundantly, into its slots) instead of read from topk_idx, and
// the workgroup of split 0, KV head 0 writes it to topk_idx.
template <int D, bool MERGE, bool SEL>
__device__ __forceinline__ void attn_unit(const AttnParams &p, uint8_t (*lds)[2 * kBlock * D],
                                          const int n, const int g, const int qs,
                                          int (*slots)[kSelSlots] = nullptr) {
    constexpr int KS = D / 32;          // k-steps of the QK product
    constexpr int DT = D / 16;          // 16-row d tiles of the PV product
    constexpr int PB = kBlock * D;      // bytes of one K or V page (one KV head)
    constexpr int LOADS = PB / 1024;    // 1 KiB direct-to-LDS loads per page
    constexpr int CPR = D / 16;         // 16-byte chunks per key row
    // lds: per wave [K page | V page]; the 4-wave merge reuses the space afterwards
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = n / p.T, t = n % p.T;
    const int per_wg = 4 * p.bpw;
    const int e0 = qs * per_wg;
    const int e1 = min(p.k, e0 + per_wg);

    // One round trip for the small inputs: seq_len, the selection row up to e1
    // (lane l holds entries l + 64c) and the row's block table (lane l holds
    // logical blocks l and l + 64).
    const int64_t trow = (int64_t)n * p.tk_sn;
    int tkv[4];
    float srow[2];
    if constexpr (SEL) {
        // the score row, issued together with the other small loads below
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int jj = lane + 64 * c;
            srow[c] = jj < p.MB ? p.scores[(int64_t)n * p.sc_sn + (int64_t)jj * p.sc_sj] : 0.f;
        }
    } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int idx = lane + 64 * c;
            tkv[c] = idx < e1 ? p.topk[trow + (int64_t)idx * p.tk_si] : -1;
        }
    }
    int btv[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int jj = lane + 64 * c;
        btv[c] = jj < p.MB ? p.bt[(int64_t)r * p.bt_sr + (int64_t)jj * p.bt_sj] : -1;
    }
    const int L = clamp_len(p.seq_lens[(int64_t)r * p.sl_s], p.MB);
    const int vis = max(0, L - (p.T - 1 - t));
    if constexpr (SEL) {
        int *sl = slots[wave];
        select_from_values<2>(srow, p.MB, p.k, sl);
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int idx = lane + 64 * c;
            tkv[c] = idx < e1 ? sl[idx] : -1;
        }
        if (qs == 0 && g == 0 && wave == 0)
            for (int i = lane; i < p.k; i += 64) p.topk_out[trow + (int64_t)i * p.tk_si] = sl[i];
    }

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
    if constexpr (!MERGE) {
        // partial for the merge kernel: m, l per head, unnormalised acc
        const int64_t N = (int64_t)p.R * p.T;
        const int64_t row = (int64_t)qs * N * p.Hq + (int64_t)n * p.Hq + h;
        if (active) {
            float *dst = p.part_acc + row * D + dq * 8;
            *(f32x4 *)dst = f32x4{acc8[0], acc8[1], acc8[2], acc8[3]};
            *(f32x4 *)(dst + 4) = f32x4{acc8[4], acc8[5], acc8[6], acc8[7]};
            if (dq == 0) {
                p.part_m[row] = mx;
                p.part_l[row] = lm;
            }
        }
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
        float *dst = p.part_acc + ((int64_t)qs * N * p.Hq + row) * D + dq * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) st_coherent(dst + e, acc8[e]);
        if (dq == 0) {
            st_coherent(p.part_m + (int64_t)qs * N * p.Hq + row, mx);
            st_coherent(p.part_l + (int64_t)qs * N * p.Hq + row, lm);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    __shared__ int last;
    int *ctr = p.counters + ((int64_t)n * p.Hkv + g) * kCounterStride;
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


}  // namespace msa
