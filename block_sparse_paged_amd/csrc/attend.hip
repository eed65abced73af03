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

// K in LDS: [128 keys][D bf16], 16-byte units XOR-swizzled by key.
template <int D>
__device__ __forceinline__ int k_off(int key, int unit) {
    constexpr int U = D / 8;
    return key * (D * 2) + ((unit ^ (key & (U - 1))) << 4);
}
// V^T in LDS: [D rows][128 keys bf16 in PV k-order], 16-byte units swizzled by d.
__device__ __forceinline__ int v_off(int d, int unit) {
    return d * (kBlock * 2) + ((unit ^ (d & 15) ^ (((d >> 4) & 3) << 2)) << 4);
}

template <int D>
__global__ __launch_bounds__(256) void attn_mfma_kernel(AttnParams p) {
    constexpr int KS = D / 32;          // k-steps of the QK product
    constexpr int DT = D / 16;          // 16-row d tiles of the PV product
    constexpr int KCH = kBlock * D / 16 / 256;          // 16-byte K chunks per thread
    constexpr int VITEMS = 32 * (D / 16);               // (4-key group, 16-d chunk) items
    __shared__ __attribute__((aligned(16))) uint8_t kbuf[2][kBlock * D * 2];
    __shared__ __attribute__((aligned(16))) uint8_t vbuf[2][D * kBlock * 2];
    __shared__ uint32_t sel[kTokGroup][kMaxMB / 32];
    __shared__ uint16_t ulist[kMaxMB];
    __shared__ int ucount;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const Group q = decode_group(p);
    const int U = build_union(p, q, sel, ulist, &ucount);
    int beg, end;
    split_range(U, p.splits, q.s, beg, end);

    const bool tok_active = wave < q.nt;
    const int64_t n = (int64_t)q.r * p.T + q.t0 + wave;
    const int vis = token_vis(p, q, wave);
    const int h0 = q.g * 16;

    // B operand of S^T = K Q^T: lane holds q[n][h0 + lane%16][32*ks + 8*(lane/16) .. +8]
    uint4 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        if (tok_active) {
            const uint16_t *qp = (const uint16_t *)p.q + n * p.q_sn + (int64_t)(h0 + (lane & 15)) * p.q_sh;
            qf[ks] = *(const uint4 *)(qp + 32 * ks + 8 * (lane >> 4));
        } else {
            qf[ks] = make_uint4(0, 0, 0, 0);
        }
    }
    const float scale2 = p.sm_scale * p.k_scale * kLog2e;

    float m_run = -INFINITY, l_run = 0.f;
    f32x4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    bool any = false;

    // register staging of the next page
    uint4 kst[KCH];
    uint4 vst[4];
    const int vdc = tid % (D / 16);
    const int vkg = tid / (D / 16);
    auto load = [&](int b) {
        const int j = ulist[b];
        const int pid = p.bt[(int64_t)q.r * p.bt_sr + (int64_t)j * p.bt_sj];
        const uint8_t *kp = (const uint8_t *)p.k_cache + (int64_t)pid * p.k_sp + (int64_t)q.g * p.k_sh;
        const uint8_t *vp = (const uint8_t *)p.v_cache + (int64_t)pid * p.v_sp + (int64_t)q.g * p.v_sh;
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
            const int chunk = tid + 256 * c;
            const int key = chunk / (D / 16);
            const int col = (chunk % (D / 16)) * 16;
            kst[c] = *(const uint4 *)(kp + (int64_t)key * p.k_sb + col);
        }
        if (tid < VITEMS) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                vst[e] = *(const uint4 *)(vp + (int64_t)(4 * vkg + e) * p.v_sb + vdc * 16);
        }
    };
    auto store = [&](int b, int buf) {
        const int j = ulist[b];
        const int valid = q.L - j * kBlock;          // keys of this page inside seq_len
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
            const int chunk = tid + 256 * c;
            const int key = chunk / (D / 16);
            const int unit = (chunk % (D / 16)) * 2;
            uint4 lo, hi;
            lo.x = fp8x2_to_bf16x2<false>(kst[c].x); lo.y = fp8x2_to_bf16x2<true>(kst[c].x);
            lo.z = fp8x2_to_bf16x2<false>(kst[c].y); lo.w = fp8x2_to_bf16x2<true>(kst[c].y);
            hi.x = fp8x2_to_bf16x2<false>(kst[c].z); hi.y = fp8x2_to_bf16x2<true>(kst[c].z);
            hi.z = fp8x2_to_bf16x2<false>(kst[c].w); hi.w = fp8x2_to_bf16x2<true>(kst[c].w);
            *(uint4 *)&kbuf[buf][k_off<D>(key, unit)] = lo;
            *(uint4 *)&kbuf[buf][k_off<D>(key, unit + 1)] = hi;
        }
        if (tid < VITEMS) {
            // 4 keys x 16 d -> bf16, keys past seq_len zeroed (P is 0 there, and
            // 0 * NaN would poison the PV product)
            uint32_t kv[4][8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool ok = 4 * vkg + e < valid;
                const uint32_t w[4] = {vst[e].x, vst[e].y, vst[e].z, vst[e].w};
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    kv[e][2 * m] = ok ? fp8x2_to_bf16x2<false>(w[m]) : 0u;
                    kv[e][2 * m + 1] = ok ? fp8x2_to_bf16x2<true>(w[m]) : 0u;
                }
            }
            // position of keys 4*vkg..+3 in the PV k-order of their 32-key chunk
            const int c32 = vkg >> 3, a = vkg & 7;
            const int unit = 4 * c32 + (a & 3);
            const int half = (a >> 2) * 8;
#pragma unroll
            for (int m = 0; m < 8; ++m) {
#pragma unroll
                for (int hbit = 0; hbit < 2; ++hbit) {
                    const int d = vdc * 16 + 2 * m + hbit;
                    uint2 w2;
                    if (hbit == 0) {
                        w2.x = (kv[0][m] & 0xffffu) | (kv[1][m] << 16);
                        w2.y = (kv[2][m] & 0xffffu) | (kv[3][m] << 16);
                    } else {
                        w2.x = (kv[0][m] >> 16) | (kv[1][m] & 0xffff0000u);
                        w2.y = (kv[2][m] >> 16) | (kv[3][m] & 0xffff0000u);
                    }
                    *(uint2 *)&vbuf[buf][v_off(d, unit) + half] = w2;
                }
            }
        }
    };

    if (beg < end) load(beg);
    int buf = 0;
    for (int b = beg; b < end; ++b) {
        store(b, buf);
        __syncthreads();
        if (b + 1 < end) load(b + 1);
        const int j = ulist[b];
        const bool mine = tok_active && ((sel[wave][j >> 5] >> (j & 31)) & 1u);
        if (mine) {
            any = true;
            const int kbase = j * kBlock;
            float s[8][4];
            float bmax = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 8; ++kt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                const int key = kt * 16 + (lane & 15);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const uint4 a = *(const uint4 *)&kbuf[buf][k_off<D>(key, 4 * ks + (lane >> 4))];
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, qf[ks]), acc, 0, 0, 0);
                }
                // acc[i] = S^T[key 16*kt + 4*(lane/16) + i][head lane%16]
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int pos = kbase + kt * 16 + 4 * (lane >> 4) + i;
                    const float x = acc[i] * scale2;
                    s[kt][i] = (pos < vis) ? x : -INFINITY;
                    bmax = fmaxf(bmax, s[kt][i]);
                }
            }
            bmax = max_across_groups<16>(bmax);
            const float m_new = fmaxf(m_run, bmax);
            const float alpha = exp2f(m_run - m_new);
            m_run = m_new;
            uint32_t pb[8][2];
            float lsum = 0.f;
#pragma unroll
            for (int kt = 0; kt < 8; ++kt) {
                float pr[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t bits = f32_to_bf16_rne(exp2f(s[kt][i] - m_new));
                    pr[i] = __uint_as_float(bits << 16);
                    lsum += pr[i];
                }
                pb[kt][0] = pack_bf16x2(pr[0], pr[1]);
                pb[kt][1] = pack_bf16x2(pr[2], pr[3]);
            }
            l_run = l_run * alpha + lsum;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                // B operand of O^T = V^T P^T: keys of chunk c in PV k-order
                const uint4 bp = make_uint4(pb[2 * c][0], pb[2 * c][1], pb[2 * c + 1][0], pb[2 * c + 1][1]);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const int d = dt * 16 + (lane & 15);
                    const uint4 a = *(const uint4 *)&vbuf[buf][v_off(d, 4 * c + (lane >> 4))];
                    o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, bp), o[dt], 0, 0, 0);
                }
            }
        }
        buf ^= 1;
    }

    if (!tok_active) return;
    // sum the four lane groups (lane/16) that hold keys of the same head
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    const int64_t row = ((int64_t)q.s * (p.R * p.T) + n) * p.Hq + h0 + (lane & 15);
    if (lane < 16) {
        p.part_m[row] = any ? m_run : -INFINITY;
        p.part_l[row] = any ? l_tot : 0.f;
    }
    if (any) {
        // o[dt][i] = O^T[d = 16*dt + 4*(lane/16) + i][head lane%16]
        float *dst = p.part_acc + row * D + 4 * (lane >> 4);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) *(f32x4 *)(dst + dt * 16) = o[dt];
    }
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
hipError_t launch_mfma(const AttnParams &p, int64_t grid, hipStream_t s) {
    hipLaunchKernelGGL((attn_mfma_kernel<D>), dim3((unsigned)grid), dim3(256), 0, s, p);
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

int attn_splits(int32_t R, int32_t T, int32_t Hkv, int32_t k) {
    const int64_t TG = (T + kTokGroup - 1) / kTokGroup;
    const int64_t groups = (int64_t)R * Hkv * TG;
    const int64_t maxU = (int64_t)min(T, kTokGroup) * k;
    int64_t S = groups > 0 ? (kSplitTargetWGs + groups - 1) / groups : 1;
    S = S < 1 ? 1 : S;
    S = S > maxU ? maxU : S;
    return (int)(S < 1 ? 1 : S);
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t attn_workspace_bytes(int32_t R, int32_t T, int32_t Hq, int32_t Hkv, int32_t D, int32_t k) {
    const int S = attn_splits(R, T, Hkv, k);
    const size_t rows = (size_t)S * R * T * Hq;
    return align256(rows * 4) * 2 + align256(rows * D * 4);
}

void attn_carve_workspace(void *ws, int32_t S, int32_t N, int32_t Hq, int32_t D, float **m,
                          float **l, float **acc) {
    const size_t rows = (size_t)S * N * Hq;
    char *b = (char *)ws;
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
    if (G == 16 && q_type == E_BF16 && kv_type == E_FP8)
        return D == 64 ? launch_mfma<64>(p, grid, s) : launch_mfma<128>(p, grid, s);
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
