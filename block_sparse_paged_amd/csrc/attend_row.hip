// Row-level sparse attention: one workgroup per (request row, KV head, split
// of the row's list of selected blocks), for selections that a row's tokens
// largely share -- one selection per request, or per-token selections wide
// enough that the tokens' union is close to each token's own (top-k near all
// blocks).  The per-token unit (attn_unit.h) streams every page once per
// token that selected it; here each page is loaded from HBM into LDS once per
// row and every token that selected it runs its own 16-column MFMA tiles on
// it.
//
// Cacheon "Kernel ABI", "Attention block slots": attention.decode (attend
// exactly the supplied block ids; -1 entries and keys at or past a query's
// visibility excluded) and attention.msa_block_score (a per-request sheet,
// whose selection the request's tokens share).
//
// The workgroup (8 waves) first builds the row's list: per logical block, the
// bit mask of the row's tokens (2 to 4) that selected it and see a key of it
// (from topk_idx, or -- with SEL -- from each token's score row, wave t
// selecting for token t), and the ascending list of blocks with a nonzero
// mask.  Split s takes list entries s*U/S .. (s+1)*U/S - 1, every wave every
// page: wave group tg = wave / 4 the tokens tg*TPW .. (tg+1)*TPW - 1, the
// wave the keys 32*(wave % 4) .. +31 of each page.  Group 0 loads the
// quarter's K rows and group 1 its V rows straight into LDS (direct-to-LDS
// 16-byte non-temporal loads, three pages ahead in four buffers), one
// fence-free barrier per page making them visible to all; each wave decodes
// its quarter's K and V fragments FP8 -> bf16 and runs, per token, S^T = K
// Q^T, the online softmax update (lazily moved reference) and O^T += V^T P^T
// on bf16 MFMA, with P carried as two bf16 parts (queries read from LDS).
// The four quarter-waves of each token are merged in LDS in one round and
// each (token, split) partial goes to the workspace; the split merge kernel
// (attend.hip) combines them in a fixed order.
#include "attn_unit.h"
#include "device_util.h"
#include "msa_internal.h"
#include "select_unit.h"

namespace msa {

namespace {

constexpr int kRowTok = 4;          // tokens of a row this unit serves
constexpr double kRowMinPages = 64;  // expected pages per row below which the per-token unit serves
constexpr int kRowBufs = 4;          // pages in flight (LDS page buffers)

// softmax_weights for raw products: p = 2^(scale2 * s - m) (one fma before the
// exponent; scale2 > 0 keeps -inf at -inf), and `sum` the fp32 weights
// themselves (hi + lo equals p to 2^-17 relative).
__device__ __forceinline__ PWeights softmax_weights_scaled(const f32x4 (&sacc)[2], float scale2, float m) {
    uint32_t h[4], l[4];
    float sum = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const float a = exp2_fast(__builtin_fmaf(sacc[u][2 * hh], scale2, -m));
            const float b = exp2_fast(__builtin_fmaf(sacc[u][2 * hh + 1], scale2, -m));
            const uint32_t w = cvt_pk_bf16(a, b);
            const uint32_t wl = cvt_pk_bf16(a - bf16lo_to_f32(w), b - bf16hi_to_f32(w));
            h[2 * u + hh] = w;
            l[2 * u + hh] = wl;
            sum += a + b;
        }
    return PWeights{make_uint4(h[0], h[1], h[2], h[3]), make_uint4(l[0], l[1], l[2], l[3]), sum};
}

struct RowSlot {
    int r, g, s;
    bool live;
};

// Workgroup -> (row, KV head, split); with 8 or more rows a row's workgroups
// run on XCD r % 8 (workgroup id b on XCD b % 8).
__device__ __forceinline__ RowSlot decode_row_slot(const AttnParams &p) {
    RowSlot q;
    const int x = blockIdx.x & 7, local = blockIdx.x >> 3;
    q.s = local % p.splits;
    const int unit_local = local / p.splits;
    if (p.R >= 8) {
        q.g = unit_local % p.Hkv;
        q.r = x + 8 * (unit_local / p.Hkv);
    } else {
        const int u = x + 8 * unit_local;    // unit r*Hkv + g on XCD u % 8
        q.r = u / p.Hkv;
        q.g = u % p.Hkv;
    }
    q.live = q.r < p.R;
    return q;
}

template <int D, bool SEL, int NT>
__global__ __launch_bounds__(kAttnWaves * 64, 1) void attn_row_kernel(AttnParams p) {
    constexpr int NW = kAttnWaves;
    constexpr int KS = D / 32;               // k-steps of the QK product
    constexpr int DT = D / 16;               // 16-row d tiles of the PV product
    constexpr int CPR = D / 16;              // 16-byte units per K (V) row
    constexpr int KPL = 64 / CPR;            // rows per 1 KiB direct-to-LDS load
    constexpr int LPC = kChunk / KPL;        // loads per 32-row chunk and tensor
    constexpr int CB = kChunk * D;           // bytes of a wave's 32 K (or V) rows
    constexpr int QP = D + 8;                // query row in LDS, padded (bf16 elements)
    constexpr int TPW = (NT + 1) / 2;        // tokens per wave (wave group 0: the first TPW)
    static_assert(KPL % 8 == 0 && LPC >= 1 && NT * 4 * DT * 1024 <= 2 * kRowBufs * 4 * CB, "layout");
    // [K, V][page buffer][quarter][32 rows]; the wave merge reuses all of it
    __shared__ __attribute__((aligned(16))) uint8_t kv[2][kRowBufs][4][CB];
    __shared__ __attribute__((aligned(16))) uint16_t sq[NT][16][QP];
    __shared__ int sbt[kSelSlots], smask[kSelSlots];
    __shared__ uint8_t ulist[kSelSlots];
    __shared__ int sU;
    __shared__ int sslots[SEL ? NT : 1][kSelSlots];
    __shared__ __attribute__((aligned(16))) int shist[SEL ? NT : 1][256];
    __shared__ float smm[NT][4][16], sml[NT][4][16];

    const RowSlot rs = decode_row_slot(p);
    if (!rs.live) return;                    // uniform over the workgroup
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = lane >> 4, li = lane & 15;
    constexpr int T = NT;                    // tokens of the row (p.T)
    const int r = rs.r, g = rs.g, s = rs.s, MB = p.MB;
    const int h0 = g * 16;
    const int64_t n0 = (int64_t)r * T;
    const int64_t N = (int64_t)p.R * T;

    // ---- one round trip: seq_len, the block table row, the selection (or
    // score) rows, the queries
    const int Lraw = p.seq_lens[(int64_t)r * p.sl_s];
    if (tid < kSelSlots) {
        sbt[tid] = tid < MB ? p.bt[(int64_t)r * p.bt_sr + (int64_t)tid * p.bt_sj] : -1;
        smask[tid] = 0;
    }
    // waves 0 .. nrow-1 read (or, with SEL, select from) the row's selection
    // rows: one per token, or one for the whole request
    const int nrow = p.sel_per_row ? 1 : T;
    const int64_t srow_n = p.sel_per_row ? (int64_t)r : n0 + wave;
    float srow[2] = {0.f, 0.f};
    int tsel[2] = {-1, -1};
    if (wave < nrow) {
        if constexpr (SEL) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int jj = lane + 64 * c;
                srow[c] = jj < MB ? p.scores[srow_n * p.sc_sn + (int64_t)jj * p.sc_sj] : 0.f;
            }
        } else {
            const int64_t trow = (int64_t)g * p.tk_sg + srow_n * p.tk_sn;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int i = lane + 64 * c;
                tsel[c] = i < p.k ? p.topk[trow + (int64_t)i * p.tk_si] : -1;
            }
        }
    }
    for (int c = tid; c < T * 16 * (D / 8); c += NW * 64) {
        const int t = c / (16 * (D / 8)), rem = c % (16 * (D / 8));
        const int h = rem / (D / 8), d8 = rem % (D / 8);
        *(uint4 *)&sq[t][h][d8 * 8] =
            *(const uint4 *)((const uint16_t *)p.q + (n0 + t) * p.q_sn + (int64_t)(h0 + h) * p.q_sh + d8 * 8);
    }
    const int L = clamp_len(Lraw, MB);
    // keys visible to token t: the row's first L - (T - 1 - t)
    auto visible = [&](int t) { return max(0, L - (T - 1 - t)); };
    if constexpr (SEL) {
        if (wave < nrow) select_from_values<2>(srow, MB, p.k, sslots[wave], shist[wave]);
    }
    __syncthreads();                         // block table, cleared masks, slots, queries
    // ---- token bits per block: wave w sets, for each block of its selection
    // row that maps to a page, the bits of the tokens it belongs to and that
    // see a key of it
    if (wave < nrow) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int i = lane + 64 * c;
            int j = -1;
            if constexpr (SEL) j = i < p.k ? sslots[wave][i] : -1;
            else j = tsel[c];
            if (j >= 0 && j < MB) {
                const int pid = sbt[j];
                int bits = 0;
                for (int t = 0; t < T; ++t)
                    if ((p.sel_per_row || t == wave) && j * kBlock < visible(t)) bits |= 1 << t;
                if (bits && pid >= 0 && pid < p.P) atomicOr(&smask[j], bits);
            }
        }
        if constexpr (SEL) {
            if (s == 0 && g == 0)
                for (int i = lane; i < p.k; i += 64)
                    p.topk_out[srow_n * p.tk_sn + (int64_t)i * p.tk_si] = sslots[wave][i];
        }
    }
    __syncthreads();
    if (wave == 0) {
        // ascending list of blocks with a nonzero mask (lane l: blocks l, l + 64)
        const bool a = lane < MB && smask[lane] != 0, b = lane + 64 < MB && smask[lane + 64] != 0;
        const uint64_t ma = __ballot(a), mb = __ballot(b);
        const int na = __popcll(ma);
        if (a) ulist[lanes_below(ma)] = (uint8_t)lane;
        if (b) ulist[na + lanes_below(mb)] = (uint8_t)(lane + 64);
        if (lane == 0) sU = na + __popcll(mb);
    }
    __syncthreads();
    const int U = sU;
    const int b0 = (int)((int64_t)U * s / p.splits), b1 = (int)((int64_t)U * (s + 1) / p.splits);
    // nothing but the page loads below may be in the wave's load queue
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

    // ---- pages: every wave takes every page of the split; wave group
    // tg = wave / 4 its tokens tg*TPW .. (tg+1)*TPW - 1, the wave the keys
    // 32*quarter .. 32*quarter + 31 of each page.  Group 0 loads the
    // quarter's K rows, group 1 its V rows; a workgroup barrier per page makes
    // every wave's rows visible to the others.
    const int tg = wave >> 2, quarter = wave & 3;
    const int key0 = lane / CPR, unit = lane % CPR;
    const int64_t ksb = p.k_sb, vsb = p.v_sb;
    auto issue = [&](int b, int buf) {
        const int j = ulist[b];
        const int pid = sbt[j];
        if (tg == 0) {
            const uint8_t *kp = (const uint8_t *)p.k_cache + (int64_t)pid * p.k_sp + (int64_t)g * p.k_sh +
                                (int64_t)(kChunk * quarter) * ksb;
            // K units swizzled by kswz(key), V units by vswz(key) (as in attn_unit.h)
#pragma unroll
            for (int l = 0; l < LPC; ++l) {
                const int key = l * KPL + key0;
                dma16_nt(kp + (int64_t)key * ksb + ((unit ^ kswz<CPR>(key)) << 4), kv[0][buf][quarter] + l * 1024);
            }
        } else {
            const uint8_t *vp = (const uint8_t *)p.v_cache + (int64_t)pid * p.v_sp + (int64_t)g * p.v_sh +
                                (int64_t)(kChunk * quarter) * vsb;
#pragma unroll
            for (int l = 0; l < LPC; ++l) {
                const int key = l * KPL + key0;
                dma16_nt(vp + (int64_t)key * vsb + ((unit ^ (vswz(key) & (CPR - 1))) << 4),
                         kv[1][buf][quarter] + l * 1024);
            }
        }
    };

    const float scale2 = p.sm_scale * p.k_scale * kLog2e;
    float m_run[TPW], l_run[TPW];
    f32x4 o[TPW][DT];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
        m_run[j] = -INFINITY;
        l_run[j] = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[j][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // the wave's tokens (a token index past the row's stands in for nothing:
    // its queries are those of the last token and every key is masked for it)
    int tok[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) tok[j] = tg * TPW + j;
    const int n_pages = b1 - b0;
#pragma unroll
    for (int i = 0; i < kRowBufs - 1; ++i)
        if (i < n_pages) issue(b0 + i, i);
    for (int i = 0; i < n_pages; ++i) {
        const int buf = i % kRowBufs;
        // this page's loads landed (those of the up to kRowBufs - 2 later
        // pages issued may still fly), then every wave's
        const int later = min(n_pages - 1 - i, kRowBufs - 2);
        if (later >= 2) wait_vmcnt<2 * LPC>();
        else if (later == 1) wait_vmcnt<LPC>();
        else wait_vmcnt<0>();
        // a barrier without a memory fence (which would wait for every load
        // in flight): the wave's own LDS reads are done, then the workgroup
        // meets; the asm keeps the compiler from moving LDS accesses across it
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        // every wave is past page i - 1: its buffer takes page i + kRowBufs - 1
        if (i + kRowBufs - 1 < n_pages) issue(b0 + i + kRowBufs - 1, (i + kRowBufs - 1) % kRowBufs);
        const int j = ulist[b0 + i];
        const int tokmask = smask[j];
        const int kbase = j * kBlock + kChunk * quarter;
        if (kbase >= L) continue;            // no key of this quarter page is visible (uniform)
        // key kbase + i counts for token t when below lim (0 for a token that
        // did not select the block)
        int lim[TPW], lmin = L;
#pragma unroll
        for (int jj = 0; jj < TPW; ++jj) {
            const int t = tok[jj];
            lim[jj] = (t < NT && ((tokmask >> t) & 1)) ? L - (NT - 1 - t) : 0;
            lmin = min(lmin, lim[jj]);
        }
        const uint8_t *kq = kv[0][buf][quarter];
        const uint8_t *vq = kv[1][buf][quarter];
        // S^T = K Q^T for the wave's tokens: sacc[jj][u][e] = q . k for key
        // kbase + 16*u + 4*grp + e and head h0 + li.  A operand: key 16*u + li,
        // d = (D/4)*grp + 8*ks .. +8 (one 16-byte K unit holds two k-steps).
        f32x4 sacc[TPW][2];
#pragma unroll
        for (int jj = 0; jj < TPW; ++jj) sacc[jj][0] = sacc[jj][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kp2 = 0; kp2 < KS / 2; ++kp2) {
            bf16x8 ka[2][2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int key = 16 * u + li;
                const int ku = (((D / 4) * grp) / 16 + kp2) ^ kswz<CPR>(key);
                const uint4 raw = *(const uint4 *)(kq + key * D + (ku << 4));
                ka[u][0] = __builtin_bit_cast(bf16x8, fp8x8_to_bf16x8(raw.x, raw.y));
                ka[u][1] = __builtin_bit_cast(bf16x8, fp8x8_to_bf16x8(raw.z, raw.w));
            }
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int jj = 0; jj < TPW; ++jj) {
                    const int tq = min(tok[jj], NT - 1);
                    const bf16x8 qf = *(const bf16x8 *)&sq[tq][li][(D / 4) * grp + 16 * kp2 + 8 * hf];
#pragma unroll
                    for (int u = 0; u < 2; ++u)
                        sacc[jj][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[u][hf], qf, sacc[jj][u], 0, 0, 0);
                }
        }
        // V^T fragments, rows past seq_len dropped (their bytes may be NaN)
        const int vvalid = L - kbase;
        const int vkey = pv_key(grp, li >> 1);
        const uint8_t *vrow = vq + vkey * D + 8 * (li & 1);
        const int vsw = vswz(vkey) & (CPR - 1);
        uint32_t kill_lo = 0u, kill_hi = 0u;
        if (vvalid < kChunk) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const bool dead = pv_key(grp, e) >= vvalid;
                if (e < 4) kill_lo |= dead ? (0xffu << (8 * e)) : 0u;
                else kill_hi |= dead ? (0xffu << (8 * (e - 4))) : 0u;
            }
        }
        bf16x8 va[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const v2i raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (__attribute__((address_space(3))) v2i *)(vrow + ((dt ^ vsw) << 4)));
            va[dt] = __builtin_bit_cast(bf16x8, fp8x8_to_bf16x8((uint32_t)raw.x & ~kill_lo, (uint32_t)raw.y & ~kill_hi));
        }
        if (kbase + kChunk > lmin) {
#pragma unroll
            for (int jj = 0; jj < TPW; ++jj)
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        sacc[jj][u][e] = (kbase + u * 16 + 4 * grp + e < lim[jj]) ? sacc[jj][u][e] : -INFINITY;
        }
        // online softmax on the raw products (scale2 > 0 is applied inside
        // the exponent).  Each head keeps a reference m that moves only when a
        // chunk's max exceeds it by more than kSlack, so that the accumulators
        // are rescaled rarely (in a branch of its own); the weights 2^(s - m)
        // stay below 2^kSlack.  P as two bf16 parts.
        float cm[TPW];
        bool any_up = false;
#pragma unroll
        for (int jj = 0; jj < TPW; ++jj) {
            const f32x4 &s0 = sacc[jj][0], &s1 = sacc[jj][1];
            const float cmax = max3f(max3f(s0[0], s0[1], s0[2]), max3f(s0[3], s1[0], s1[1]), fmaxf(s1[2], s1[3]));
            cm[jj] = max_over_lane_groups(cmax) * scale2;
            any_up |= cm[jj] > m_run[jj] + kSlack;           // also a first visible key (m = -inf)
        }
        if (__ballot(any_up)) {
#pragma unroll
            for (int jj = 0; jj < TPW; ++jj) {
                const bool up = cm[jj] > m_run[jj] + kSlack;
                const float alpha = up ? exp2_fast(m_run[jj] - cm[jj]) : 1.f;
                m_run[jj] = up ? cm[jj] : m_run[jj];
                l_run[jj] *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) o[jj][dt] *= alpha;
            }
        }
#pragma unroll
        for (int jj = 0; jj < TPW; ++jj) {
            // a head that has seen no key keeps m = -inf: weights 2^(-inf - 0) = 0
            const PWeights pw = softmax_weights_scaled(sacc[jj], scale2, m_run[jj] == -INFINITY ? 0.f : m_run[jj]);
            l_run[jj] += pw.sum;
            // O^T += V^T P_hi^T + V^T P_lo^T
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                o[jj][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[dt], __builtin_bit_cast(bf16x8, pw.hi), o[jj][dt],
                                                                    0, 0, 0);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                o[jj][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[dt], __builtin_bit_cast(bf16x8, pw.lo), o[jj][dt],
                                                                    0, 0, 0);
        }
    }

    // ---- merge the four quarter-waves of each token in LDS, one round:
    // wave (tg, quarter) stores tile dt of token t's O^T at
    // [(t*4 + quarter)*DT + dt] (1 KiB each, 16 bytes a lane), then wave w
    // merges (token, tile) pairs w, w + 8, ... over the four quarters and
    // stores the (token, split) partial.
    __syncthreads();                         // every wave's page reads are done
    uint8_t *const region = &kv[0][0][0][0];
#pragma unroll
    for (int jj = 0; jj < TPW; ++jj) {
        const int t = tok[jj];
        if (t >= NT) break;
        const float l_tot = sum_over_lane_groups(l_run[jj]);
        uint8_t *const ow = region + (t * 4 + quarter) * DT * 1024 + lane * 16;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) *(f32x4 *)(ow + dt * 1024) = o[jj][dt];
        if (lane < 16) {
            smm[t][quarter][lane] = m_run[jj];
            sml[t][quarter][lane] = l_tot;
        }
    }
    __syncthreads();
    for (int pi = wave; pi < NT * DT; pi += NW) {
        const int t = pi / DT, dt = pi % DT;
        float mq[4], mx = -INFINITY;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            mq[qq] = smm[t][qq][li];
            mx = fmaxf(mx, mq[qq]);
        }
        f32x4 acc4 = {0.f, 0.f, 0.f, 0.f};
        float lm = 0.f;
        if (mx != -INFINITY) {
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const float wgt = exp2_fast(mq[qq] - mx);     // -inf -> 0
                lm += wgt * sml[t][qq][li];
                acc4 += wgt * *(const f32x4 *)(region + ((t * 4 + qq) * DT + dt) * 1024 + lane * 16);
            }
        }
        const int64_t n = n0 + t;
        const int h = h0 + li;
        *(f32x4 *)(p.part_acc + part_acc_index(s, n, h, 16 * dt + 4 * grp, N, p.Hq, D)) = acc4;
        if (dt == 0 && grp == 0) *(f32x2 *)(p.part_ml + part_ml_index(s, n, h, N, p.Hq)) = f32x2{mx, lm};
    }
}

template <int D, bool SEL, int NT>
hipError_t launch_nt(const AttnParams &p, int64_t grid, hipStream_t s) {
    hipLaunchKernelGGL((attn_row_kernel<D, SEL, NT>), dim3((unsigned)grid), dim3(kAttnWaves * 64), 0, s, p);
    return hipGetLastError();
}

template <int D, bool SEL>
hipError_t launch(const AttnParams &p, hipStream_t s) {
    const int64_t units_per_xcd = (p.R >= 8) ? (int64_t)((p.R + 7) / 8) * p.Hkv : ((int64_t)p.R * p.Hkv + 7) / 8;
    const int64_t grid = 8 * units_per_xcd * p.splits;
    if (grid == 0) return hipSuccess;
    switch (p.T) {
    case 2: return launch_nt<D, SEL, 2>(p, grid, s);
    case 3: return launch_nt<D, SEL, 3>(p, grid, s);
    case 4: return launch_nt<D, SEL, 4>(p, grid, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool attention_row_eligible(int q_type, int kv_type, int D, int G, int T, int MB, int k, bool sel_per_row,
                            float score_scale) {
    if (!(q_type == E_BF16 && kv_type == E_FP8 && G == 16 && (D == 64 || D == 128))) return false;
    if (!(score_scale > 0.f)) return false;      // the lazy softmax reference needs an order-keeping scale
    if (T < 2 || T > kRowTok || MB > kSelSlots || k > MB) return false;
    // the row's expected list: the shared selection, or the union of T
    // random per-token selections
    double U = k;
    if (!sel_per_row) {
        double miss = 1.0;
        for (int t = 0; t < T; ++t) miss *= 1.0 - (double)k / MB;
        U = MB * (1.0 - miss);
    }
    // worth its split partials and merge launch when the per-token unit would
    // stream at least twice the row's pages and the row has enough of them
    // (measured: a shared selection of 16 pages per row runs faster per token)
    return (double)T * k >= 2.0 * U && U >= kRowMinPages;
}

int32_t row_splits(int32_t R, int32_t Hkv) {
    const int64_t units = (int64_t)R * Hkv;
    int64_t S = units > 0 ? (kSplitTargetWGs + units - 1) / units : 1;
    S = S > kRowMaxSplits ? kRowMaxSplits : S;
    return (int32_t)(S < 1 ? 1 : S);
}

hipError_t launch_attention_row(const AttnParams &p, int D, bool select, hipStream_t s) {
    if (D == 128) return select ? launch<128, true>(p, s) : launch<128, false>(p, s);
    return select ? launch<64, true>(p, s) : launch<64, false>(p, s);
}

}  // namespace msa
