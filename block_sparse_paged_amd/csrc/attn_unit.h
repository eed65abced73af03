// The per-token MFMA attention unit behind msa_sparse_decode and the attention
// launch of msa_select_sparse_decode / msa_decode_step (attend.hip holds the
// kernels and the work split).
#pragma once

#include "device_util.h"
#include "msa_internal.h"
#include "select_unit.h"

namespace msa {

__device__ __forceinline__ int clamp_len(int L, int MB) { return max(0, min(L, MB * kBlock)); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kSelSlots = 128;             // selection slots (k <= MB <= 128)
constexpr int kChunk = 32;                 // keys per LDS sub-chunk
constexpr int kAttnWaves = 8;              // waves per attention workgroup
constexpr int kWaveKeys = 64;              // keys of a page one wave takes
constexpr int kWaveChunks = kWaveKeys / kChunk;   // 2
constexpr int kPipeKeys = 32;              // keys per pipeline chunk (one softmax update)

//
// One workgroup of 8 waves per (query token n, KV head g, split s of n's
// selection list).  The workgroup takes selection entries s*epw .. +epw
// (epw <= 4*bpw: small batches use fewer entries per split, leaving slots
// idle, to spread over more CUs); waves 2q and 2q+1 share page slot q
// (entries s*epw + q*bpw .. +bpw) and
// take its first and second 64 keys.  For each of its pages a wave
//   issues its 64 K and 64 V rows straight from HBM into its LDS slots with
//           direct-to-LDS 16-byte non-temporal loads (16-byte units
//           XOR-swizzled by key): the first page's all at once, each later
//           page's chunk by chunk as the previous page's chunk in the same
//           slots has been multiplied;
//   then, per pipeline chunk of kPipeKeys keys, as soon as its K rows have
//           landed: S^T = K Q^T on MFMA (K rows decoded FP8 -> bf16 as A
//           operands, the 16 heads of the token as the 16 columns) and the
//           online-softmax update (lazily moved reference), and as soon as
//           its V rows have landed O^T += V^T P^T with P as two bf16 parts
//           (two MFMAs), V read back by ds_read_b64_tr_b8, which hands each
//           lane 8 keys at one d (the A operand).
// The waits are explicit vmcnt counts over the wave's in-order load queue.
// Two waves per SIMD (128 KiB of K/V slots per workgroup, one workgroup per
// CU) let one wave's math overlap the other's.
// The 8 waves merge their softmax partials in LDS.  The splits of a token are
// then merged in this launch through a per-(token, KV head) arrival counter in
// the workspace: every workgroup leaves its partial, and the last one to
// arrive combines the S partials in a fixed order, writes the output and
// resets the counter to zero (so the counters are zero again after every
// call).  Workgroups are placed so that
// all those of a row (at least 8 rows) or of a token run on one XCD and share
// its L2: a page chosen by several of a row's tokens is then fetched from HBM
// once.  Correctness does not depend on the placement.

typedef int v2i __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));

// 16 bytes per lane from global memory straight into LDS (the 64 lanes' data
// land contiguously from lds, which must be wave-uniform), non-temporal.
// Written as inline assembly so that the compiler does not see a pending LDS
// write: it would otherwise wait for every such load before the first LDS
// read.  Every read of the data is preceded by an explicit wait_vmcnt.  M0
// (the LDS address operand) is restored afterwards.
__device__ __forceinline__ void dma16_nt(const void *g, void *lds) {
    const uint32_t l = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)lds;
    uint32_t save;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "global_load_lds_dwordx4 %1, off nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(save)
        : "v"(g), "s"(l)
        : "memory");
}

// s_waitcnt immediate for vmcnt(0) alone (expcnt and lgkmcnt at their maxima)
constexpr int kWaitVmcnt0 = (0x7 << 4) | (0xF << 8);

// wait until at most N vector memory operations of this wave are outstanding
// (also a compiler barrier for memory accesses)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Device-coherent accesses (agent scope: sc1 loads and stores, no
// cache-maintenance fences) for the in-launch split hand-off.  The 12-byte
// forms are inline assembly: a load's result may only be used after an
// explicit vmcnt wait that names the result register.
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
__device__ __forceinline__ void st_coherent12(uint32_t *p, u32x3 v) {
    asm volatile("global_store_dwordx3 %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ u32x3 ld_coherent12_nowait(const uint32_t *p) {
    u32x3 v;
    asm volatile("global_load_dwordx3 %0, %1, off sc1" : "=v"(v) : "v"(p) : "memory");
    return v;
}

// Four fp32 values as four 24-bit floats (sign, 8-bit exponent, 15-bit
// mantissa: fp32 rounded to nearest even on its low 8 bits, 2^-16 relative)
// packed into three words, and back.  Finite inputs only.
__device__ __forceinline__ uint32_t f32_to_f24(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7fu + ((u >> 8) & 1u)) >> 8;
}
__device__ __forceinline__ u32x3 pack_f24x4(f32x4 v) {
    const uint32_t a = f32_to_f24(v[0]), b = f32_to_f24(v[1]), c = f32_to_f24(v[2]), d = f32_to_f24(v[3]);
    return u32x3{a | (b << 24), (b >> 8) | (c << 16), (c >> 16) | (d << 8)};
}
__device__ __forceinline__ f32x4 unpack_f24x4(u32x3 w) {
    return f32x4{__uint_as_float(w.x << 8), __uint_as_float((w.x >> 24 | w.y << 8) << 8),
                 __uint_as_float((w.y >> 16 | w.z << 16) << 8), __uint_as_float(w.z & 0xffffff00u)};
}
__device__ __forceinline__ void st_coherent2(float *p, float a, float b) {
    const uint64_t v = (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
    __hip_atomic_store((uint64_t *)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x2 ld_coherent2(const float *p) {
    const uint64_t v = __hip_atomic_load((const uint64_t *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return f32x2{__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32))};
}

// FP8 K rows in LDS (CPR 16-byte units a row): unit c of key k stored at unit
// c ^ kswz<CPR>(k).  A ds_read_b128 serves 16 lanes a cycle from the 64 banks
// (256 bytes); the 16 keys k0 .. k0 + 15 at one unit fall on rows whose bank
// offset repeats every 16 / CPR keys, and kswz spreads the CPR keys of each
// offset over distinct units, so that the 16 reads hit 16 distinct 16-byte
// bank groups.
template <int CPR>
__device__ __forceinline__ int kswz(int key) {
    return ((key * CPR) >> 4) & (CPR - 1);
}

// V rows in LDS: 16-byte unit c of key k stored at unit c ^ vswz(k).  A
// ds_read_b64_tr_b8 of 64 lanes is served 32 lanes (256 bytes, the 64 banks) a
// cycle: two 16-lane groups, which read the 16-byte units of keys 4a..4a+3,
// 16+4a..16+4a+3 and 4a+4..4a+7, 20+4a..20+4a+3 of a 32-key chunk (a even).
// With 128-byte rows, key bit 0 already separates rows by half the banks;
// vswz spreads the keys of each parity by their bits 1, 2 and 4 over the 8
// unit positions, so that the 16 keys hit 16 distinct bank groups (keyed by
// bits 0 and 1 and bit 4 alone, the two groups collided pairwise: rocprofv3
// counted 64 bank-conflict cycles per wave of the attention launch, 32 with
// this form, at the same launch time).
__device__ __forceinline__ int vswz(int key) { return ((key >> 1) & 3) | (((key >> 4) & 1) << 2); }

// PV k-order inside a 32-key chunk: MFMA k index 8*grp + e holds key
//   e < 4 : 4*grp + e            (QK accumulator tile 0, row 4*grp + e)
//   e >= 4: 16 + 4*grp + (e - 4) (QK accumulator tile 1, row 4*grp + e - 4)
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

// Lazily moved softmax reference: a head's reference m moves only when a
// chunk's max exceeds it by more than kSlack (log2 units), so that the
// accumulators are rescaled rarely; the weights 2^(s - m) stay below 2^kSlack.
constexpr float kSlack = 8.f;

// max of a lane's 8 products of a 32-key chunk
__device__ __forceinline__ float chunk_max(const f32x4 (&sacc)[2]) {
    return max3f(max3f(sacc[0][0], sacc[0][1], sacc[0][2]), max3f(sacc[0][3], sacc[1][0], sacc[1][1]),
                 fmaxf(sacc[1][2], sacc[1][3]));
}

// Softmax weights p = 2^(s - m) of a 32-key chunk (sacc[u][e]: key
// 16*u + 4*grp + e of the lane's group) as MFMA B operands in two bf16 parts,
// hi = bf16(p) and lo = bf16(p - hi) (p - hi is exact in fp32), so that
// V^T P_hi^T + V^T P_lo^T carries p to about 2^-17 relative: bf16 alone
// (2^-9) passes straight into the output of a token that sees only a few keys
// (two keys of values -4 and 4 at equal weight: up to 4 * 2^-9 ~ 0.008).
// `sum` is the lane's fp32 weights (hi + lo equals each to 2^-17 relative).
struct PWeights {
    uint4 hi, lo;
    float sum;
};
__device__ __forceinline__ PWeights softmax_weights(const f32x4 (&sacc)[2], float m) {
    uint32_t h[4], l[4];
    float sum = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const float a = exp2_fast(sacc[u][2 * hh] - m), b = exp2_fast(sacc[u][2 * hh + 1] - m);
            const uint32_t w = cvt_pk_bf16(a, b);
            const float ah = bf16lo_to_f32(w), bh = bf16hi_to_f32(w);
            const uint32_t wl = cvt_pk_bf16(a - ah, b - bh);
            h[2 * u + hh] = w;
            l[2 * u + hh] = wl;
            sum += a + b;
        }
    return PWeights{make_uint4(h[0], h[1], h[2], h[3]), make_uint4(l[0], l[1], l[2], l[3]), sum};
}

// BF16 caches (attention.decode's dense cache): rows of 2*D bytes, so a wave
// takes 32 keys of a page (four waves per page, two page slots, twice the
// pages per wave: the same selection entries per workgroup) in 16-key LDS
// sub-chunks of the same size as the FP8 ones.  K fragments are read as they
// are; V^T fragments come from two ds_read_b64_tr_b16, each handing a lane 4
// keys at one d (lane i of a 16-lane group gets element i%4 of the 8-byte
// reads of lanes i/4, 4 + i/4, 8 + i/4, 12 + i/4).  16-byte units of both are
// XOR-swizzled by key & (units per row - 1).
__device__ __forceinline__ uint4 bf16x4x2(v2i a, v2i b) {
    return make_uint4((uint32_t)a.x, (uint32_t)a.y, (uint32_t)b.x, (uint32_t)b.y);
}

// SEL: the token's selection is computed here from its score row (MB <= 128;
// by wave 0, into LDS slots) instead of read from topk_idx, and the workgroup
// of split 0, KV head 0 writes it to topk_idx.  KV: E_FP8 or E_BF16 caches.
template <int D, bool SEL, int KV = E_FP8>
__device__ __forceinline__ void attn_unit(const AttnParams &p, const int n, const int g, const int qs) {
    constexpr bool BF = KV == E_BF16;
    constexpr int NW = kAttnWaves;
    constexpr int KS = D / 32;          // k-steps of the QK product
    constexpr int DT = D / 16;          // 16-row d tiles of the PV product
    constexpr int RB = BF ? 2 * D : D;  // bytes per K (V) row
    constexpr int CPR = RB / 16;        // 16-byte units per key row
    constexpr int KPL = 64 / CPR;       // keys per 1 KiB direct-to-LDS load
    constexpr int CHK = BF ? 16 : kChunk;   // keys per sub-chunk
    constexpr int WK = BF ? 32 : kWaveKeys; // keys of a page per wave
    constexpr int WPP = kBlock / WK;    // waves per page
    constexpr int SLOTS = NW / WPP;     // page slots per workgroup
    constexpr int LPC = CHK / KPL;      // loads per sub-chunk, for K and for V
    constexpr int CB = CHK * RB;        // bytes of one sub-chunk's K (or V) rows
    static_assert(CB % 1024 == 0 && LPC >= 1 && (BF || KPL % 8 == 0), "sub-chunk layout");
    static_assert(WK / CHK == kWaveChunks, "two sub-chunks per wave");
    constexpr int CK = BF ? 32 : kPipeKeys;  // keys per pipeline chunk (softmax update)
    constexpr int NS = CK / CHK;        // sub-chunks per pipeline chunk
    constexpr int NC = WK / CK;         // pipeline chunks per wave and page
    constexpr int TPS = CHK / 16;       // 16-key QK tiles per sub-chunk
    static_assert(NS >= 1 && NC >= 1 && NS * NC == kWaveChunks && CK == 32, "pipeline chunk");
    // per sub-chunk, [8 waves][32 keys][D bytes]; the wave merge reuses lk0, lk1
    __shared__ __attribute__((aligned(16))) uint8_t lk0[NW * CB], lk1[NW * CB];
    __shared__ __attribute__((aligned(16))) uint8_t lv0[NW * CB], lv1[NW * CB];
    __shared__ float smm[NW * 16], sml[NW * 16];
    __shared__ int sslots[SEL ? kSelSlots : 1];
    __shared__ __attribute__((aligned(16))) int shist[SEL ? 256 : 4];
    __shared__ int slast;
    // selection rows of more than 256 entries and block tables of more than
    // 128 blocks (caller-made selections only): the row's entries, its block
    // table and each block id's first entry, copied once into LDS so that
    // resolving a page never waits on a global load while page loads fly.
    // Dynamic LDS, given by the launch only for such sizes (token_xtab_bytes).
    extern __shared__ int xtab[];
    int *const lsel = xtab, *const lbt = xtab + kMaxMB, *const lfirst = xtab + 2 * kMaxMB;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pslot = wave / WPP, half = wave % WPP;
    const int bpw = p.bpw * 4 / SLOTS;          // pages per wave (the same entries per workgroup)
    const int r = n / p.T, t = n % p.T;
    const int e0 = qs * p.epw;                  // entries of this split (epw <= SLOTS * bpw)
    const int e1 = min(p.k, e0 + p.epw);
    const int h0 = g * 16;

    // One round trip for the small inputs: seq_len, the selection row up to e1
    // (lane l holds entries l + 64c) or the score row, the row's block table
    // (lane l holds logical blocks l and l + 64) and the query fragments.
    const int64_t srow_n = p.sel_per_row ? r : n;   // the selection / score row
    const int64_t trow = (int64_t)g * p.tk_sg + srow_n * p.tk_sn;
    int tkv[4];
    float srow[2];
    if constexpr (SEL) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int jj = lane + 64 * c;
            srow[c] = jj < p.MB ? p.scores[srow_n * p.sc_sn + (int64_t)jj * p.sc_sj] : 0.f;
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
    const int Lraw = p.seq_lens[(int64_t)r * p.sl_s];
    // B operand of S^T = K Q^T for k-step ks: lane holds q[n][h0 + lane%16][d],
    // d = (D/4)*(lane/16) + 8*ks + e   (the same d order as the K operand below)
    uint4 qf[KS];
    {
        const uint16_t *qp = (const uint16_t *)p.q + (int64_t)n * p.q_sn + (int64_t)(h0 + (lane & 15)) * p.q_sh;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = *(const uint4 *)(qp + (D / 4) * (lane >> 4) + 8 * ks);
    }
    const int L = clamp_len(Lraw, p.MB);
    const int vis = max(0, L - (p.T - 1 - t));
    const int MBt = min(p.MB, kMaxMB);                // blocks the LDS table holds
    if constexpr (!SEL) {
        if (e1 > 256 || p.MB > 128) {                  // uniform
            for (int i = tid; i < MBt; i += NW * 64) {
                lbt[i] = p.bt[(int64_t)r * p.bt_sr + (int64_t)i * p.bt_sj];
                lfirst[i] = 0x7fffffff;
            }
            __syncthreads();
            for (int i = tid; i < e1; i += NW * 64) {
                const int j = p.topk[trow + (int64_t)i * p.tk_si];
                lsel[i] = j;
                if (j >= 0 && j < MBt) atomicMin(&lfirst[j], i);
            }
            __syncthreads();
        }
    }
    if constexpr (SEL) {
        // wave 0 selects; the others read its slots
        if (wave == 0) select_from_values<2>(srow, p.MB, p.k, sslots, shist);
        __syncthreads();
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int idx = lane + 64 * c;
            tkv[c] = idx < e1 ? sslots[idx] : -1;
        }
    }
    // nothing but the page loads below may be in the wave's load queue: their
    // waits count positions in it.  (The builtin form, so that the compiler
    // knows the query fragments have landed and adds no waits of its own.)
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

    const float scale2 = p.sm_scale * p.k_scale * kLog2e;
    float m_run = -INFINITY, l_run = 0.f;
    f32x4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint8_t *const kc[kWaveChunks] = {lk0 + wave * CB, lk1 + wave * CB};
    uint8_t *const vc[kWaveChunks] = {lv0 + wave * CB, lv1 + wave * CB};
    const int grp = lane >> 4, li = lane & 15;
    const int64_t ksb = p.k_sb * (BF ? 2 : 1), vsb = p.v_sb * (BF ? 2 : 1);   // row strides in bytes

    // The wave's pages, resolved one ahead: entry b of its slot -> K and V row
    // addresses of its keys kbase .. kbase + WK - 1 (kbase visible).  Entries
    // that are padding, repeats of an earlier entry, past the row's blocks,
    // invisible to the token or mapped to no page are skipped.
    struct PageRef {
        const uint8_t *kp, *vp;
        int kbase;
    };
    auto next_page = [&](int &b, PageRef &pr) -> bool {
        for (; b < bpw; ++b) {
            const int i = e0 + pslot * bpw + b;
            if (i >= e1) break;
            // entry i and duplicate check against entries [0, i)  (wave-uniform;
            // with SEL, i < k <= 128)
            int j = -1;
            bool dup = false;
            if (i < 256) {
                const int c = i >> 6;
                const int src = c == 0 ? tkv[0] : c == 1 ? tkv[1] : c == 2 ? tkv[2] : tkv[3];
                j = __builtin_amdgcn_readlane(src, i & 63);
                // a selection made here is a set of distinct ids
                if constexpr (!SEL) {
#pragma unroll
                    for (int c2 = 0; c2 < 4; ++c2) dup |= __ballot(lane + 64 * c2 < i && tkv[c2] == j) != 0;
                }
            } else if constexpr (!SEL) {
                j = lsel[i];
                if (j >= 0 && j < MBt) {
                    dup = lfirst[j] != i;
                } else if (j >= MBt && j < p.MB) {
                    // block ids past the first-entry table (tables of more than
                    // kMaxMB blocks): compared with the earlier entries
                    for (int c2 = 0; c2 * 64 < i; ++c2) {
                        const int idx = c2 * 64 + lane;
                        const int v = (idx < i) ? lsel[idx] : -1;
                        dup |= __ballot(idx < i && v == j) != 0;
                    }
                }
            }
            const int kbase = j * kBlock + half * WK;
            if (dup || j < 0 || j >= p.MB || kbase >= vis) continue;
            int pid;
            if (j < 128) {
                pid = __builtin_amdgcn_readlane(j < 64 ? btv[0] : btv[1], j & 63);
            } else if (j < MBt) {
                pid = lbt[j];                          // !SEL (MB <= 128 with SEL)
            } else {
                pid = p.bt[(int64_t)r * p.bt_sr + (int64_t)j * p.bt_sj];
                __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            }
            if (pid < 0 || pid >= p.P) continue;
            // element strides: bytes for FP8, 2 bytes per element for bf16
            pr.kp = (const uint8_t *)p.k_cache + ((int64_t)pid * p.k_sp + (int64_t)g * p.k_sh +
                                                  (int64_t)(half * WK) * p.k_sb) * (BF ? 2 : 1);
            pr.vp = (const uint8_t *)p.v_cache + ((int64_t)pid * p.v_sp + (int64_t)g * p.v_sh +
                                                  (int64_t)(half * WK) * p.v_sb) * (BF ? 2 : 1);
            pr.kbase = kbase;
            ++b;
            return true;
        }
        b = bpw;
        return false;
    };
    // Issue pipeline chunk c of a page: its K sub-chunks, then its V
    // sub-chunks.  Load l of a sub-chunk covers its keys KPL*l .. +KPL; lane ->
    // (key KPL*l + key0 of the sub-chunk, 16-byte unit slot).  FP8 K units
    // are swizzled by kswz(key), V units by vswz(key); both depend on l but
    // not on the sub-chunk.  The slots' earlier LDS reads have all returned
    // first (the compiler does not see these writes).
    const int key0 = lane / CPR, slot = lane % CPR;
    auto issue_chunk = [&](const PageRef &pr, int c) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int u = 0; u < NS; ++u) {
            const int sc = c * NS + u;
#pragma unroll
            for (int l = 0; l < LPC; ++l) {
                if constexpr (BF) {
                    const int key = l * KPL + key0;
                    dma16_nt(pr.kp + (int64_t)(sc * CHK + key) * ksb + ((slot ^ (key & (CPR - 1))) << 4),
                             kc[sc] + l * 1024);
                } else {
                    const int key = l * KPL + key0;
                    dma16_nt(pr.kp + (int64_t)(sc * kChunk + key) * ksb + ((slot ^ kswz<CPR>(key)) << 4),
                             kc[sc] + l * 1024);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < NS; ++u) {
            const int sc = c * NS + u;
#pragma unroll
            for (int l = 0; l < LPC; ++l) {
                const int key = l * KPL + key0;
                const int sw = BF ? (key & (CPR - 1)) : (vswz(key) & (CPR - 1));
                dma16_nt(pr.vp + (int64_t)(sc * CHK + key) * vsb + ((slot ^ sw) << 4), vc[sc] + l * 1024);
            }
        }
    };
    // With two or more pipeline chunks per page the chunk buffers roll over
    // pages: once chunk c of a page has been multiplied, its slots take chunk
    // c of the wave's next page, so a wave with several pages keeps about a
    // page of loads in flight instead of draining the queue at each page.
    constexpr bool kRoll = NC >= 2;
    int b = 0;
    PageRef cur;
    bool have = next_page(b, cur);
    if (have) {
#pragma unroll
        for (int c = 0; c < NC; ++c) issue_chunk(cur, c);
    }
    while (have) {
        PageRef nxt{nullptr, nullptr, 0};
        const bool have_n = next_page(b, nxt);
        const bool roll = kRoll && have_n;             // next page's chunks issued in the loop
        const int kbase = cur.kbase;
        const bool full = kbase + WK <= vis;           // every key visible to this token
        // V rows past seq_len hold arbitrary bytes (NaN poison in the tests);
        // their P is 0, but 0 * NaN would poison the sum, so such keys are
        // dropped from the operand (only on the page holding seq_len)
        const int vvalid = L - kbase;
        const bool vfull = vvalid >= WK;
        static_for<0, NC>([&](auto C) {
            constexpr int c = decltype(C)::value;
            // loads issued after the last K (V) load of chunk c: the page's
            // later loads, plus chunks 0 .. c-1 of the next page when they roll
            constexpr int CL = NS * LPC;               // loads per chunk per tensor
            constexpr int after_k = CL + 2 * CL * (NC - 1 - c);
            constexpr int after_v = 2 * CL * (NC - 1 - c);
            constexpr int ahead = 2 * CL * c;
            // ---- K rows of chunk c landed
            if (roll) wait_vmcnt<after_k + ahead>();
            else wait_vmcnt<after_k>();
            // S^T tiles: sacc[u][e] = q . k for key c*CK + 16*u + 4*grp + e and
            // head h0 + lane%16.  A operand: key 16*(u%2) + lane%16 of sub-chunk
            // c*NS + u/2, d = (D/4)*grp + 8*ks .. +8
            f32x4 sacc[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int key = (u % TPS) * 16 + li;
                const uint8_t *krow = kc[c * NS + u / TPS] + key * RB;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                if constexpr (BF) {
                    // k-step ks, lane group grp: d = (D/4)*grp + 8*ks .. +8, one 16-byte unit
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const int unit = (D / 32) * grp + ks;
                        const uint4 a = *(const uint4 *)(krow + ((unit ^ (key & (CPR - 1))) << 4));
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, qf[ks]), acc, 0, 0, 0);
                    }
                } else {
                    const int ksw = kswz<CPR>(key);
#pragma unroll
                    for (int kp2 = 0; kp2 < KS / 2; ++kp2) {
                        const int unit = ((D / 4) * grp) / 16 + kp2;
                        const uint4 raw = *(const uint4 *)(krow + ((unit ^ ksw) << 4));
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, fp8x8_to_bf16x8(raw.x, raw.y)),
                            __builtin_bit_cast(bf16x8, qf[2 * kp2]), acc, 0, 0, 0);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, fp8x8_to_bf16x8(raw.z, raw.w)),
                            __builtin_bit_cast(bf16x8, qf[2 * kp2 + 1]), acc, 0, 0, 0);
                    }
                }
                sacc[u] = acc * scale2;
            }
            if (!full) {
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        sacc[u][e] = (kbase + c * CK + u * 16 + 4 * grp + e < vis) ? sacc[u][e] : -INFINITY;
            }
            const float cmax = max_over_lane_groups(chunk_max(sacc));
            // lazily moved reference (a rare rescale).  Chunk 0 holds the
            // wave's first key of the page, which is visible: m is finite from
            // the first chunk of the first page on.
            const bool up = cmax > m_run + kSlack;
            if (__ballot(up)) {
                const float alpha = up ? exp2_fast(m_run - cmax) : 1.f;
                m_run = up ? cmax : m_run;
                l_run *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
            }
            // P as two bf16 parts
            const PWeights pw = softmax_weights(sacc, m_run);
            l_run += pw.sum;
            // ---- V rows of chunk c landed
            if (roll) wait_vmcnt<after_v + ahead>();
            else wait_vmcnt<after_v>();
            if constexpr (BF) {
                // V^T A operand of the 32-key chunk: k index 8*grp + e holds key
                // pv_key(grp, e) = sub-chunk e/4, key 4*grp + e%4; lane li of the
                // group reads 4 d of key 4*grp + li/4 (d 16*dt + 4*(li%4) ..)
                const int vk = 4 * grp + (li >> 2);
                const int vq = li & 3;
                uint32_t kill[2][2] = {{0u, 0u}, {0u, 0u}};
                if (!vfull) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const bool dead = c * CK + pv_key(grp, e) >= vvalid;
                        const uint32_t m = dead ? (0xffffu << (16 * (e & 1))) : 0u;
                        kill[e >> 2][(e >> 1) & 1] |= m;
                    }
                }
                const uint8_t *v0 = vc[c * NS] + vk * RB + 8 * (vq & 1);
                const uint8_t *v1 = vc[c * NS + 1] + vk * RB + 8 * (vq & 1);
                const int vsw = vk & (CPR - 1);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const int unit = 2 * dt + (vq >> 1);
                    v2i r0 = __builtin_bit_cast(v2i, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) v4i16 *)(v0 + ((unit ^ vsw) << 4))));
                    v2i r1 = __builtin_bit_cast(v2i, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) v4i16 *)(v1 + ((unit ^ vsw) << 4))));
                    r0.x &= ~kill[0][0]; r0.y &= ~kill[0][1];
                    r1.x &= ~kill[1][0]; r1.y &= ~kill[1][1];
                    const bf16x8 a = __builtin_bit_cast(bf16x8, bf16x4x2(r0, r1));
                    o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, pw.hi), o[dt], 0, 0, 0);
                    o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, pw.lo), o[dt], 0, 0, 0);
                }
            } else {
                // lanes 2b, 2b+1 of a 16-lane group read the two 8-byte halves of
                // key pv_key(grp, b)'s 16-byte unit dt
                const int key = pv_key(grp, li >> 1);
                const int vsw = vswz(key) & (CPR - 1);
                const int sc = c * NS;
                const uint8_t *vrow = vc[sc] + key * D + 8 * (li & 1);
                uint32_t kill_lo = 0u, kill_hi = 0u;
                if (!vfull) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const bool dead = sc * kChunk + pv_key(grp, e) >= vvalid;
                        if (e < 4) kill_lo |= dead ? (0xffu << (8 * e)) : 0u;
                        else kill_hi |= dead ? (0xffu << (8 * (e - 4))) : 0u;
                    }
                }
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const v2i raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (__attribute__((address_space(3))) v2i *)(vrow + ((dt ^ vsw) << 4)));
                    const bf16x8 a = __builtin_bit_cast(
                        bf16x8, fp8x8_to_bf16x8((uint32_t)raw.x & ~kill_lo, (uint32_t)raw.y & ~kill_hi));
                    o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, pw.hi), o[dt], 0, 0, 0);
                    o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, pw.lo), o[dt], 0, 0, 0);
                }
            }
            if (roll) issue_chunk(nxt, c);
        });
        if (!kRoll && have_n) {
#pragma unroll
            for (int c = 0; c < NC; ++c) issue_chunk(nxt, c);
        }
        cur = nxt;
        have = have_n;
    }
    // full per-head sum over the wave's four lane groups
    const float l_tot = sum_over_lane_groups(l_run);

    // ---- merge the 8 waves in LDS.  Wave w stores tile dt of its O^T
    // accumulator at [w][dt][lane] (16 bytes per lane: conflict-free vector
    // accesses), waves 0-3 in lk0 and 4-7 in lk1.  Thread (wm, lane) then
    // merges tile dt = wm of that lane over the 8 waves: head h0 + lane%16,
    // d = 16*wm + 4*(lane/16) + 0..3.
    __syncthreads();                                   // every wave's K/V reads done
    static_assert(4 * DT * 1024 <= NW * CB, "merge space");
    {
        uint8_t *const ow = (wave < 4 ? lk0 : lk1) + (wave & 3) * DT * 1024 + lane * 16;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) *(f32x4 *)(ow + dt * 1024) = o[dt];
    }
    if (lane < 16) {
        smm[wave * 16 + lane] = m_run;
        sml[wave * 16 + lane] = l_tot;
    }
    __syncthreads();
    const int wm = wave;                               // the tile this thread merges
    const bool active = wm < DT;
    // every LDS read first (one wait), then the weighted sums
    float mw[NW], lw[NW], mx = -INFINITY;
    f32x4 ow[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        mw[w] = smm[w * 16 + li];
        lw[w] = sml[w * 16 + li];
        ow[w] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (active) ow[w] = *(const f32x4 *)((w < 4 ? lk0 : lk1) + (w & 3) * DT * 1024 + lane * 16 + wm * 1024);
    }
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, mw[w]);
    f32x4 acc4 = {0.f, 0.f, 0.f, 0.f};
    float lm = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float wgt = exp2_fast(mw[w] - mx);       // -inf -> 0
            lm += wgt * lw[w];
            acc4 += wgt * ow[w];
        }
    }
    const int h = h0 + li;
    const int d0 = 16 * wm + 4 * grp;                  // this thread's 4 d
    const int64_t N = (int64_t)p.R * p.T;
    auto write_out = [&](f32x4 a, float lsum) {
        const float inv = (lsum > 0.f) ? p.v_scale / lsum : 0.f;
        const f32x4 v = lsum > 0.f ? a * inv : f32x4{0.f, 0.f, 0.f, 0.f};
        const int64_t base = n * p.o_sn + (int64_t)h * p.o_sh + (int64_t)d0 * p.o_sd;
        if (p.out_bf16) {
            uint16_t *op = (uint16_t *)p.out;
            if (p.o_sd == 1) {
                *(uint2 *)(op + base) = make_uint2(cvt_pk_bf16(v[0], v[1]), cvt_pk_bf16(v[2], v[3]));
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) op[base + e * p.o_sd] = (uint16_t)cvt_pk_bf16(v[e], 0.f);
            }
        } else {
            float *op = (float *)p.out;
#pragma unroll
            for (int e = 0; e < 4; ++e) op[base + e * p.o_sd] = v[e];
        }
    };
    auto store_topk = [&]() {
        if constexpr (SEL) {
            if (qs == 0 && g == 0 && wave == 0 && (!p.sel_per_row || t == 0))
                for (int i = lane; i < p.k; i += 64) p.topk_out[trow + (int64_t)i * p.tk_si] = sslots[i];
        }
    };
    if (p.splits == 1) {
        if (active) write_out(acc4, lm);
        store_topk();
        return;
    }
    float *const ml_dst = p.part_ml + part_ml_index(qs, n, h, N, p.Hq);
    // A split's partial: (m, l) in fp32 and its accumulator as 24-bit floats
    // (fp32 rounded to 15 mantissa bits, 2^-16 relative: the merged output is
    // off by at most 2^-16 of the largest V, far inside its own bf16
    // rounding), four per thread in three words at 3/4 of the fp32 layout's
    // offsets: a quarter fewer bytes written and read back.  (fp16 averages,
    // half the bytes, were measured 0.3 us faster per step but leave up to
    // 2^-11 of the largest V where splits cancel; 16-bit fixed point over
    // the E4M3 range missed near-zero outputs by up to 2^-7 codes.)
    const int64_t acc_i = part_acc_index(qs, n, h, d0, N, p.Hq, D);
    // Split hand-off.  Partials are written and read with device-coherent
    // (sc1) accesses and the arrival counter is a device-scope atomic, so the
    // workgroups of one token may sit on different XCDs; no fence (which would
    // write back and invalidate the whole L2) is needed: each writer waits for
    // its stores to complete before the workgroup's single counter increment.
    store_topk();
    if (active) st_coherent12((uint32_t *)p.part_acc + acc_i / 4 * 3, pack_f24x4(acc4));
    if (wave == 0 && grp == 0) st_coherent2(ml_dst, mx, lm);
    wait_vmcnt<0>();
    __syncthreads();
    int *ctr = p.counters + ((int64_t)n * p.Hkv + g) * kCounterStride;
    if (tid == 0) {
        const int old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        slast = (old == p.splits - 1);
    }
    __syncthreads();
    if (!slast) return;
    if (active) {
        // every split wrote (m, l, acc) (m = -inf, l = 0, acc = 0 when empty):
        // all S <= kTokenMaxSplits of them are requested at once (one memory
        // round trip, not one per few splits), then weighted and summed in
        // split order
        static_assert(kTokenMaxSplits % 4 == 0, "partials named four at a time");
        const int S = p.splits;
        f32x2 ml[kTokenMaxSplits];
        u32x3 aw[kTokenMaxSplits];
#pragma unroll
        for (int u = 0; u < kTokenMaxSplits; ++u) {
            if (u < S) {
                aw[u] = ld_coherent12_nowait((const uint32_t *)p.part_acc +
                                             part_acc_index(u, n, h, d0, N, p.Hq, D) / 4 * 3);
                ml[u] = ld_coherent2(p.part_ml + part_ml_index(u, n, h, N, p.Hq));
            } else {
                aw[u] = u32x3{0u, 0u, 0u};
                ml[u] = f32x2{-INFINITY, 0.f};
            }
        }
        // one wait for all of them; the empty statements after it (kept in
        // order) name the loaded registers, so that no use of them is
        // scheduled before the wait
        wait_vmcnt<0>();
#pragma unroll
        for (int u = 0; u < kTokenMaxSplits; u += 4)
            asm volatile("" : "+v"(aw[u]), "+v"(aw[u + 1]), "+v"(aw[u + 2]), "+v"(aw[u + 3])::"memory");
        float m2 = -INFINITY, l2 = 0.f;
        f32x4 a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < kTokenMaxSplits; ++u) {
            if (u < S) {
                const float mu = ml[u].x;
                const float mn = fmaxf(m2, mu);
                const float wo = (m2 == -INFINITY) ? 0.f : exp2_fast(m2 - mn);
                const float wn = (mu == -INFINITY) ? 0.f : exp2_fast(mu - mn);
                l2 = l2 * wo + ml[u].y * wn;
                a2 = a2 * wo + unpack_f24x4(aw[u]) * wn;
                m2 = mn;
            }
        }
        write_out(a2, l2);
    }
    if (tid == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace msa
