// Stage 1: block scores over the paged index cache.
//
// scores[n][j] = idx_scale * max over the keys s of block j visible to query
// token n of sum_d q_idx[n][d] * index_k[page(j)][s][d]   (-inf when none).
// Cacheon "Kernel ABI", "Attention block slots": attention.msa_block_score
// (decode score sheet) and attention.msa_prefill_block_score (prefill).
//
// Kernels:
//  * score_valu  -- decode rows (T < 16 query tokens per row).  One wave per
//    (row, group of <= 4 tokens, block).  The wave streams the 128-token page
//    with coalesced 16-byte loads (8 lanes per 128-byte index row for FP8
//    Di=128), decodes FP8 in registers to bf16 and accumulates with
//    v_dot2_f32_bf16; the partial dots of a row are summed across its lanes
//    with DPP, masked by visibility and max-reduced.
//  * score_mfma_decode -- decode rows of up to 16 tokens with bf16 queries
//    and an FP8 index: one page per wave on v_mfma_f32_16x16x32_bf16.
//  * score_prefill -- prefill rows (T > 16).  A workgroup owns 256 or 512
//    query tokens of one row and a run of at most 8 blocks; each page is
//    decoded FP8 -> bf16 once into LDS and every wave multiplies its queries
//    against it on MFMA (prefill_tile.h, shared with the ragged prefill
//    score-to-selection call).
#include "device_util.h"
#include "msa_internal.h"
#include "prefill_tile.h"
#include "score_unit.h"

namespace msa {

namespace {



// ------------------------------------------------------------------ VALU path

template <bool QBF16, bool KFP8, int DI>
__global__ __launch_bounds__(256) void score_valu_kernel(ScoreParams p) {
    constexpr int ESZ = KFP8 ? 1 : 4;
    constexpr int ROWB = DI * ESZ;           // bytes per index row
    constexpr int LPT = ROWB / 16;           // lanes per token row
    constexpr int TPL = 64 / LPT;            // tokens per wave-wide load
    constexpr int NLOAD = kBlock / TPL;      // loads per page per lane
    constexpr int EPL = 16 / ESZ;            // elements per lane per load
    constexpr int CH = NLOAD < 16 ? NLOAD : 16;
    constexpr int TQ = kTokGroup;
    static_assert(LPT >= 1 && LPT <= 64 && (64 % LPT) == 0, "row size");

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int TG = (p.T + TQ - 1) / TQ;
    const int JC = (p.MB + 3) >> 2;
    int bid = blockIdx.x;
    const int jc = bid % JC;
    bid /= JC;
    const int tg = bid % TG;
    const int r = bid / TG;
    const int j = jc * 4 + wave;
    if (j >= p.MB) return;                   // no barriers below: a wave may leave

    const int t0 = tg * TQ;
    const int nt = min(TQ, p.T - t0);
    const int L = clamp_len(p.seq_lens[(int64_t)r * p.sl_s], p.MB);
    int vis[TQ];
#pragma unroll
    for (int t = 0; t < TQ; ++t) vis[t] = (t < nt) ? max(0, L - (p.T - 1 - (t0 + t))) : 0;
    const int vmax = max(0, L - (p.T - t0 - nt));   // the group's last token sees most
    const int64_t n0 = (int64_t)r * p.T + t0;

    float best[TQ];
#pragma unroll
    for (int t = 0; t < TQ; ++t) best[t] = -INFINITY;
    bool bad_page = false;

    if (j * kBlock < vmax) {
        const int pid = p.bt[(int64_t)r * p.bt_sr + (int64_t)j * p.bt_sj];
        if (pid < 0 || pid >= p.P) {
            bad_page = true;
        } else {
            const int dchunk = lane % LPT;
            const int grp = lane / LPT;
            // query fragments: elements [dchunk*EPL, +EPL) of each token's q_idx row
            constexpr int QW = (QBF16 && KFP8) ? EPL / 2 : EPL;   // words per token
            uint32_t qf[TQ][QW];
#pragma unroll
            for (int t = 0; t < TQ; ++t) {
                if (t < nt) {
                    const char *qrow = (const char *)p.q_idx +
                                       (n0 + t) * p.q_sn * (QBF16 ? 2 : 4);
                    if constexpr (QBF16 && KFP8) {
                        const uint4 *src = (const uint4 *)(qrow + dchunk * EPL * 2);
#pragma unroll
                        for (int w = 0; w < QW / 4; ++w) {
                            uint4 v = src[w];
                            qf[t][4 * w + 0] = v.x; qf[t][4 * w + 1] = v.y;
                            qf[t][4 * w + 2] = v.z; qf[t][4 * w + 3] = v.w;
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < EPL; ++e) {
                            float f;
                            if constexpr (QBF16)
                                f = __uint_as_float((uint32_t)((const uint16_t *)qrow)[dchunk * EPL + e] << 16);
                            else
                                f = ((const float *)qrow)[dchunk * EPL + e];
                            qf[t][e] = __float_as_uint(f);
                        }
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < QW; ++e) qf[t][e] = 0u;
                }
            }

            const char *page = (const char *)p.index_k + (int64_t)pid * p.k_sp * ESZ;
            const int kbase = j * kBlock;
#pragma unroll
            for (int c0 = 0; c0 < NLOAD; c0 += CH) {
                uint4 buf[CH];
#pragma unroll
                for (int i = 0; i < CH; ++i) {
                    const int s = (c0 + i) * TPL + grp;
                    buf[i] = *(const uint4 *)(page + (int64_t)s * p.k_sb * ESZ + dchunk * 16);
                }
#pragma unroll
                for (int i = 0; i < CH; ++i) {
                    const int s = (c0 + i) * TPL + grp;
                    float dot[TQ];
#pragma unroll
                    for (int t = 0; t < TQ; ++t) dot[t] = 0.f;
                    const uint32_t w4[4] = {buf[i].x, buf[i].y, buf[i].z, buf[i].w};
                    if constexpr (KFP8 && QBF16) {
#pragma unroll
                        for (int w = 0; w < 4; ++w) {
                            const bf16x2 k01 = __builtin_bit_cast(bf16x2, fp8x2_to_bf16x2<false>(w4[w]));
                            const bf16x2 k23 = __builtin_bit_cast(bf16x2, fp8x2_to_bf16x2<true>(w4[w]));
#pragma unroll
                            for (int t = 0; t < TQ; ++t) {
                                dot[t] = __builtin_amdgcn_fdot2_f32_bf16(
                                    k01, __builtin_bit_cast(bf16x2, qf[t][2 * w]), dot[t], false);
                                dot[t] = __builtin_amdgcn_fdot2_f32_bf16(
                                    k23, __builtin_bit_cast(bf16x2, qf[t][2 * w + 1]), dot[t], false);
                            }
                        }
                    } else if constexpr (KFP8) {
#pragma unroll
                        for (int w = 0; w < 4; ++w) {
                            const f32x2 a = fp8x2_to_f32x2<false>(w4[w]);
                            const f32x2 b = fp8x2_to_f32x2<true>(w4[w]);
#pragma unroll
                            for (int t = 0; t < TQ; ++t) {
                                dot[t] = fmaf(a.x, __uint_as_float(qf[t][4 * w + 0]), dot[t]);
                                dot[t] = fmaf(a.y, __uint_as_float(qf[t][4 * w + 1]), dot[t]);
                                dot[t] = fmaf(b.x, __uint_as_float(qf[t][4 * w + 2]), dot[t]);
                                dot[t] = fmaf(b.y, __uint_as_float(qf[t][4 * w + 3]), dot[t]);
                            }
                        }
                    } else {
#pragma unroll
                        for (int w = 0; w < 4; ++w) {
#pragma unroll
                            for (int t = 0; t < TQ; ++t)
                                dot[t] = fmaf(__uint_as_float(w4[w]), __uint_as_float(qf[t][w]), dot[t]);
                        }
                    }
                    const int pos = kbase + s;
#pragma unroll
                    for (int t = 0; t < TQ; ++t) {
                        const float d = group_sum<LPT>(dot[t]);
                        best[t] = (pos < vis[t]) ? fmaxf(best[t], d) : best[t];
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < TQ; ++t) best[t] = max_across_groups<LPT>(best[t]);
        }
    }
    if (p.per_row) {
        // one row per request (T <= kTokGroup: this wave holds all its
        // tokens): the max over them (tokens past nt hold -inf)
        float v = best[0];
#pragma unroll
        for (int t = 1; t < TQ; ++t) v = fmaxf(v, best[t]);
        v = bad_page ? __builtin_nanf("") : v * p.idx_scale;
        if (lane == 0) p.scores[(int64_t)r * p.sc_sn + (int64_t)j * p.sc_sj] = v;
    } else if (lane < nt) {
        float v = best[0];
#pragma unroll
        for (int t = 1; t < TQ; ++t) v = (lane == t) ? best[t] : v;
        v = bad_page ? __builtin_nanf("") : v * p.idx_scale;
        p.scores[(n0 + lane) * p.sc_sn + (int64_t)j * p.sc_sj] = v;
    }
}

// ------------------------------------------------------------- MFMA decode path

// pages (one per wave) per workgroup: 4, or 1 when the batch has too few
// pages to give every CU a workgroup of 4
template <int DI, bool STAGE>
__global__ __launch_bounds__(256) void score_mfma_decode_kernel(ScoreParams p) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int WPG = blockDim.x >> 6;
    const int JC = (p.MB + WPG - 1) / WPG;
    int r, jc;
    if (p.R >= 8) {
        // workgroup b runs on XCD b % 8: the row's workgroups all go to XCD r % 8,
        // where the attention workgroups of its tokens run (block table and
        // score row stay in that XCD's L2)
        const int x = blockIdx.x & 7, i = blockIdx.x >> 3;
        r = x + 8 * (i / JC);
        jc = i % JC;
        if (r >= p.R) return;
    } else {
        r = blockIdx.x / JC;
        jc = blockIdx.x % JC;
    }
    const int j = jc * WPG + wave;
    if (j >= p.MB) return;                      // no barriers in this kernel
    // STAGE: 128 * DI bytes of LDS per wave (dynamic: WPG waves)
    extern __shared__ __attribute__((aligned(16))) uint8_t spages[];
    score_page<DI, STAGE>(p, r, j, spages + wave * (kBlock * DI));
}

// ------------------------------------------------------------------ MFMA path
//
// Prefill rows (T > 16): a GEMM per row, S = Q_r K_r^T over the row's visible
// keys, reduced to block maxima (prefill_tile.h).  A workgroup owns 128*QT
// query tokens of a row (16*QT per wave = QT MFMA column tiles of 16) and an
// even share of the blocks those tokens see (at most kPMaxPC consecutive
// ones); the tiles are laid out so that the workgroups of one query chunk run
// on one XCD.  The running block max per (query, block) is staged in LDS and
// written out coalesced at the end.

constexpr int kPTargetWGs = 256;  // workgroups aimed for (one per CU)

template <int DI, int QT>
__global__ __launch_bounds__(64 * kPWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void score_prefill_kernel(ScoreParams p, int WPC) {
    constexpr int NT = 64 * kPWaves;            // threads per workgroup
    constexpr int PQ = PrefillLds<DI, QT, kPMaxPC>::PQ;  // query tokens per workgroup
    __shared__ PrefillLds<DI, QT, kPMaxPC> lds;

    const int tid = threadIdx.x;
    const int QC = (p.T + PQ - 1) / PQ;
    // Query chunk c = r*QC + qc has WPC workgroups, tiles u = c*WPC + w.
    // Workgroups are dispatched round-robin over the 8 XCDs (XCD = blockIdx %
    // 8), each with its own L2; XCD x runs the contiguous tile range [x*U8,
    // (x+1)*U8), so the workgroups of one query chunk (and of one row's pages)
    // share an L2 instead of every XCD fetching every chunk.
    const int U = p.R * QC * WPC, U8 = (U + 7) / 8;
    const int u = (int)(blockIdx.x % 8) * U8 + (int)(blockIdx.x / 8);
    if (u >= U) return;                                    // whole workgroup, before any barrier
    const int c = u / WPC, qc = c % QC, r = c / QC, w = u % WPC;
    const int L = clamp_len(p.seq_lens[(int64_t)r * p.sl_s], p.MB);
    const int tq0 = qc * PQ, tq1 = min(p.T, tq0 + PQ);
    const int64_t nrow = (int64_t)r * p.T;
    PrefillPages pg;
    pg.index_k = (const uint8_t *)p.index_k; pg.k_sp = p.k_sp; pg.k_sb = p.k_sb; pg.P = p.P;
    pg.bt_row = p.bt + (int64_t)r * p.bt_sr; pg.bt_sj = p.bt_sj;
    pg.vmin = max(0, L - (p.T - 1 - tq0));               // keys seen by the WG's first token
    pg.vmax = max(0, L - (p.T - 1 - (tq1 - 1)));         // ... by its last
    pg.scale = p.idx_scale;
    // Blocks the chunk's last token sees: 0 .. lp-1.  They are split evenly
    // over the chunk's workgroups (at most kPMaxPC each, by the choice of
    // WPC); blocks from lp on are seen by no token of the chunk: -inf, written
    // by workgroup w for every WPC-th of them.
    const int lp = min(p.MB, (pg.vmax + kBlock - 1) / kBlock);
    pg.j0 = (int)((int64_t)w * lp / WPC);
    pg.npg = (int)((int64_t)(w + 1) * lp / WPC) - pg.j0;
    for (int jd = lp + w; jd < p.MB; jd += WPC)
        for (int qq = tid; qq < tq1 - tq0; qq += NT)
            p.scores[(nrow + tq0 + qq) * p.sc_sn + (int64_t)jd * p.sc_sj] = -INFINITY;

    // Columns past the row's last token read that token again; their scores
    // are never stored, and no reduction mixes columns.
    const uint16_t *q = (const uint16_t *)p.q_idx;
    auto qrow = [&](int col) { return q + (nrow + min(p.T - 1, tq0 + col)) * p.q_sn; };
    auto vis = [&](int col) {
        const int t = tq0 + col;
        return t < p.T ? max(0, L - (p.T - 1 - t)) : 0;
    };
    prefill_tile<DI, QT, kPMaxPC>(pg, qrow, vis, lds);

    const int npg = pg.npg, j0 = pg.j0;
    for (int idx = tid; idx < (tq1 - tq0) * npg; idx += NT) {
        const int qq = idx / npg, pi = idx % npg;
        p.scores[(nrow + tq0 + qq) * p.sc_sn + (int64_t)(j0 + pi) * p.sc_sj] = lds.sbuf[qq][pi];
    }
}

template <bool QB, bool KF, int DI>
hipError_t launch_valu(const ScoreParams &p, hipStream_t s) {
    const int TG = (p.T + kTokGroup - 1) / kTokGroup;
    const int JC = (p.MB + 3) / 4;
    const int64_t grid = (int64_t)p.R * TG * JC;
    hipLaunchKernelGGL((score_valu_kernel<QB, KF, DI>), dim3((unsigned)grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

template <int DI>
hipError_t launch_mfma_decode(const ScoreParams &p, hipStream_t s) {
    const int WPG = (int64_t)p.R * ((p.MB + 3) / 4) < kSplitTargetWGs ? 1 : 4;
    const int64_t JC = (p.MB + WPG - 1) / WPG;
    // R >= 8: 8 XCDs x ceil(R / 8) rows each x JC (see the kernel)
    const int64_t grid = p.R >= 8 ? 8 * ((p.R + 7) / 8) * JC : (int64_t)p.R * JC;
    // pages staged through LDS when the launch has at least two waves per CU
    if (grid * WPG >= 2 * kChipCUs)
        hipLaunchKernelGGL((score_mfma_decode_kernel<DI, true>), dim3((unsigned)grid), dim3(64 * WPG),
                           (size_t)WPG * kBlock * DI, s, p);
    else
        hipLaunchKernelGGL((score_mfma_decode_kernel<DI, false>), dim3((unsigned)grid), dim3(64 * WPG), 0, s, p);
    return hipGetLastError();
}

template <int DI, int QT>
hipError_t launch_prefill(const ScoreParams &p, hipStream_t s) {
    const int64_t QC = (p.T + 16 * QT * kPWaves - 1) / (16 * QT * kPWaves), chunks = (int64_t)p.R * QC;
    // workgroups per query chunk: enough for kPTargetWGs in all, and enough
    // that none holds more than kPMaxPC blocks; no more than there are blocks
    int64_t WPC = (kPTargetWGs + chunks - 1) / chunks;
    WPC = WPC < (p.MB + kPMaxPC - 1) / kPMaxPC ? (p.MB + kPMaxPC - 1) / kPMaxPC : WPC;
    WPC = WPC > p.MB ? p.MB : WPC;
    const int64_t U = chunks * WPC;
    const int64_t grid = 8 * ((U + 7) / 8);               // tile ranges per XCD (see the kernel)
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;   // the kernel indexes tiles in int
    hipLaunchKernelGGL((score_prefill_kernel<DI, QT>), dim3((unsigned)grid), dim3(64 * kPWaves), 0, s, p, (int)WPC);
    return hipGetLastError();
}

// 4 query tiles per wave (512 tokens per workgroup) once a row has more than
// 256 query tokens, else 2
template <int DI>
hipError_t launch_mfma(const ScoreParams &p, hipStream_t s) {
    return p.T > 256 ? launch_prefill<DI, 4>(p, s) : launch_prefill<DI, 2>(p, s);
}

template <bool QB, bool KF>
hipError_t launch_valu_di(const ScoreParams &p, int Di, hipStream_t s) {
    switch (Di) {
    case 32: return launch_valu<QB, KF, 32>(p, s);
    case 64: return launch_valu<QB, KF, 64>(p, s);
    case 128: return launch_valu<QB, KF, 128>(p, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool score_supported(int q_type, int k_type, int Di) {
    return (q_type == E_F32 || q_type == E_BF16) && (k_type == E_F32 || k_type == E_FP8) &&
           (Di == 32 || Di == 64 || Di == 128);
}

bool score_per_row_supported(int q_type, int k_type, int Di, int T) {
    // the MFMA decode kernel holds a row's T <= 16 tokens in one wave; the
    // vector kernel holds kTokGroup of them
    const bool mfma = q_type == E_BF16 && k_type == E_FP8 && (Di == 64 || Di == 128);
    return T <= (mfma ? 16 : kTokGroup);
}

hipError_t launch_score(const ScoreParams &p, int q_type, int k_type, int Di, hipStream_t s) {
    const bool qb = q_type == E_BF16, kf = k_type == E_FP8;
    if (p.R == 0 || p.T == 0) return hipSuccess;
    if (qb && kf && p.T > 16 && (Di == 64 || Di == 128))
        return Di == 64 ? launch_mfma<64>(p, s) : launch_mfma<128>(p, s);
    if (qb && kf && (Di == 64 || Di == 128))
        return Di == 64 ? launch_mfma_decode<64>(p, s) : launch_mfma_decode<128>(p, s);
    if (qb && kf) return launch_valu_di<true, true>(p, Di, s);
    if (qb) return launch_valu_di<true, false>(p, Di, s);
    if (kf) return launch_valu_di<false, true>(p, Di, s);
    return launch_valu_di<false, false>(p, Di, s);
}

}  // namespace msa
