// Stage 1: block scores over the paged index cache.
//
// scores[n][j] = idx_scale * max over the keys s of block j visible to query
// token n of sum_d q_idx[n][d] * index_k[page(j)][s][d]   (-inf when none).
// Cacheon "Kernel ABI", "Attention block slots": attention.msa_block_score
// (decode score sheet) and attention.msa_prefill_block_score (prefill).
//
// Two kernels:
//  * score_valu  -- decode rows (T < 16 query tokens per row).  One wave per
//    (row, group of <= 4 tokens, block).  The wave streams the 128-token page
//    with coalesced 16-byte loads (8 lanes per 128-byte index row for FP8
//    Di=128), decodes FP8 in registers to bf16 and accumulates with
//    v_dot2_f32_bf16; the partial dots of a row are summed across its lanes
//    with DPP, masked by visibility and max-reduced.
//  * score_mfma  -- prefill rows (T >= 16).  A workgroup owns 128 query tokens
//    of one row and a run of blocks; each page is staged once in LDS (FP8,
//    XOR-swizzled) and every wave multiplies its 32 queries against it with
//    v_mfma_f32_16x16x32_bf16 after exact FP8 -> bf16 decoding.
#include "device_util.h"
#include "msa_internal.h"
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
    if (lane < nt) {
        float v = best[0];
#pragma unroll
        for (int t = 1; t < TQ; ++t) v = (lane == t) ? best[t] : v;
        v = bad_page ? __builtin_nanf("") : v * p.idx_scale;
        p.scores[(n0 + lane) * p.sc_sn + (int64_t)j * p.sc_sj] = v;
    }
}

// ------------------------------------------------------------- MFMA decode path

template <int DI>
__global__ __launch_bounds__(256) void score_mfma_decode_kernel(ScoreParams p) {
    const int wave = threadIdx.x >> 6;
    const int JC = (p.MB + 3) >> 2;
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
    const int j = jc * 4 + wave;
    if (j >= p.MB) return;                      // no barriers in this kernel
    score_page<DI>(p, r, j);
}

// ------------------------------------------------------------------ MFMA path

constexpr int kMQ = 128;      // query tokens per workgroup (4 waves x 2 tiles x 16)
constexpr int kMBlocks = 8;   // blocks per workgroup

// LDS page layout: [128 keys][DI bytes] FP8, 8-byte units XOR-swizzled by key so
// that the 16 lanes reading one MFMA fragment column hit distinct banks.
template <int DI>
__device__ __forceinline__ int page_off(int key, int unit) {
    constexpr int UNITS = DI / 8;
    return key * DI + ((unit ^ (key & (UNITS - 1))) << 3);
}

template <int DI>
__global__ __launch_bounds__(256) void score_mfma_kernel(ScoreParams p) {
    constexpr int KS = DI / 32;                 // MFMA k-steps per 16-key tile
    constexpr int PAGE = kBlock * DI;           // bytes per page
    constexpr int CHUNKS = PAGE / 16;           // 16-byte chunks per page
    constexpr int PER_T = CHUNKS / 256;         // chunks per thread
    static_assert(PER_T >= 1, "page too small");
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][PAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int QC = (p.T + kMQ - 1) / kMQ;
    const int BC = (p.MB + kMBlocks - 1) / kMBlocks;
    int bid = blockIdx.x;
    const int bc = bid % BC;
    bid /= BC;
    const int qc = bid % QC;
    const int r = bid / QC;
    const int L = clamp_len(p.seq_lens[(int64_t)r * p.sl_s], p.MB);
    const int tq0 = qc * kMQ;                          // first token of the WG (in row)
    const int tq1 = min(p.T, tq0 + kMQ);               // one past the last
    const int vmax_wg = max(0, L - (p.T - 1 - (tq1 - 1)));
    const int j0 = bc * kMBlocks;
    const int j1 = min(p.MB, j0 + kMBlocks);
    const int64_t nrow = (int64_t)r * p.T;

    // B-operand fragments of Q^T: for tile qt, k-step ks, lane holds
    // q_idx[token 16*qt + lane%16][d = 32*ks + 8*(lane/16) .. +8] (bf16).
    // vt[qt]: keys visible to that token.
    uint4 qf[2][KS];
    int vt[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        const int t = tq0 + wave * 32 + qt * 16 + (lane & 15);
        vt[qt] = (t < p.T) ? max(0, L - (p.T - 1 - t)) : 0;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (t < p.T) {
                const uint16_t *q = (const uint16_t *)p.q_idx + (nrow + t) * p.q_sn;
                qf[qt][ks] = *(const uint4 *)(q + 32 * ks + 8 * (lane >> 4));
            } else {
                qf[qt][ks] = make_uint4(0, 0, 0, 0);
            }
        }
    }

    auto page_ptr = [&](int j) -> const uint8_t * {
        const int pid = p.bt[(int64_t)r * p.bt_sr + (int64_t)j * p.bt_sj];
        return (const uint8_t *)p.index_k + (int64_t)pid * p.k_sp;
    };
    auto page_ok = [&](int j) -> int {
        if (j * kBlock >= vmax_wg) return 0;                 // nothing visible in the WG
        const int pid = p.bt[(int64_t)r * p.bt_sr + (int64_t)j * p.bt_sj];
        return (pid >= 0 && pid < p.P) ? 1 : 2;               // 2 = bad page id
    };

    uint4 stage[PER_T];
    auto load_page = [&](int j) {
        const uint8_t *pg = page_ptr(j);
#pragma unroll
        for (int c = 0; c < PER_T; ++c) {
            const int chunk = tid + 256 * c;
            const int key = chunk / (DI / 16);
            const int col = (chunk % (DI / 16)) * 16;
            stage[c] = *(const uint4 *)(pg + (int64_t)key * p.k_sb + col);
        }
    };
    auto store_page = [&](int buf) {
#pragma unroll
        for (int c = 0; c < PER_T; ++c) {
            const int chunk = tid + 256 * c;
            const int key = chunk / (DI / 16);
            const int unit = (chunk % (DI / 16)) * 2;
            *(uint2 *)&lds[buf][page_off<DI>(key, unit)] = make_uint2(stage[c].x, stage[c].y);
            *(uint2 *)&lds[buf][page_off<DI>(key, unit + 1)] = make_uint2(stage[c].z, stage[c].w);
        }
    };

    // find the next block (from j) whose page must be read
    int jn = j0;
    while (jn < j1 && page_ok(jn) != 1) ++jn;
    if (jn < j1) load_page(jn);
    int buf = 0;
    for (int j = j0; j < j1; ++j) {
        const int ok = page_ok(j);                             // uniform over the WG
        if (ok != 1) {
            const float v = ok == 0 ? -INFINITY : __builtin_nanf("");
            for (int t = tid; t < tq1 - tq0; t += 256)
                p.scores[(nrow + tq0 + t) * p.sc_sn + (int64_t)j * p.sc_sj] = v;
            continue;
        }
        store_page(buf);
        __syncthreads();
        jn = j + 1;
        while (jn < j1 && page_ok(jn) != 1) ++jn;
        if (jn < j1) load_page(jn);                            // overlaps the MFMAs below

        const int kbase = j * kBlock;
        float best[2] = {-INFINITY, -INFINITY};
#pragma unroll 2
        for (int kt = 0; kt < 8; ++kt) {
            // A operand: K rows (keys) 16*kt + lane%16, d = 32*ks + 8*(lane/16) .. +8
            f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
            const int key = kt * 16 + (lane & 15);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const uint2 raw = *(const uint2 *)&lds[buf][page_off<DI>(key, ks * 4 + (lane >> 4))];
                uint4 kb;
                kb.x = fp8x2_to_bf16x2<false>(raw.x);
                kb.y = fp8x2_to_bf16x2<true>(raw.x);
                kb.z = fp8x2_to_bf16x2<false>(raw.y);
                kb.w = fp8x2_to_bf16x2<true>(raw.y);
                const bf16x8 a = __builtin_bit_cast(bf16x8, kb);
#pragma unroll
                for (int qt = 0; qt < 2; ++qt)
                    acc[qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        a, __builtin_bit_cast(bf16x8, qf[qt][ks]), acc[qt], 0, 0, 0);
            }
            // acc[qt][i] = S^T[key 16*kt + 4*(lane/16) + i][token lane%16]
#pragma unroll
            for (int qt = 0; qt < 2; ++qt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int pos = kbase + kt * 16 + 4 * (lane >> 4) + i;
                    best[qt] = (pos < vt[qt]) ? fmaxf(best[qt], acc[qt][i]) : best[qt];
                }
        }
        // combine the four lane groups (lane/16) that hold keys of the same token
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            const float v = max_across_groups<16>(best[qt]);
            const int t = tq0 + wave * 32 + qt * 16 + (lane & 15);
            if (lane < 16 && t < p.T)
                p.scores[(nrow + t) * p.sc_sn + (int64_t)j * p.sc_sj] = v * p.idx_scale;
        }
        buf ^= 1;
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
    const int64_t JC = (p.MB + 3) / 4;
    // R >= 8: 8 XCDs x ceil(R / 8) rows each x JC (see the kernel)
    const int64_t grid = p.R >= 8 ? 8 * ((p.R + 7) / 8) * JC : (int64_t)p.R * JC;
    hipLaunchKernelGGL((score_mfma_decode_kernel<DI>), dim3((unsigned)grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

template <int DI>
hipError_t launch_mfma(const ScoreParams &p, hipStream_t s) {
    const int QC = (p.T + kMQ - 1) / kMQ;
    const int BC = (p.MB + kMBlocks - 1) / kMBlocks;
    const int64_t grid = (int64_t)p.R * QC * BC;
    hipLaunchKernelGGL((score_mfma_kernel<DI>), dim3((unsigned)grid), dim3(256), 0, s, p);
    return hipGetLastError();
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
