// Internal declarations shared by the gfx950 kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

constexpr int kBlock = 128;          // tokens per page (vLLM design note: block size 128)
constexpr int kMaxMB = 2048;         // logical blocks per row served by select/attention
constexpr int kTokGroup = 4;         // query tokens of one row handled together
constexpr int kChipCUs = 256;        // compute units of an MI355X (8 XCDs of 32)
constexpr int kSplitTargetWGs = kChipCUs;  // attention workgroups aimed for (one per CU)
constexpr int kTokenMaxSplits = 8;   // splits of one token's selection list (MFMA path)
constexpr int kCounterStride = 64;   // int32s between split-arrival counters (one per 256 B)
constexpr int kRowMaxSplits = 32;    // splits of one row's block list (row-level attention)

enum ElemType { E_F32 = 0, E_BF16 = 1, E_FP8 = 2, E_I32 = 3 };

struct ScoreParams {
    const void *q_idx;   int64_t q_sn;             // [N, Di], inner stride 1
    const void *index_k; int64_t k_sp, k_sb;       // [P, B, Di], inner stride 1
    const int32_t *bt;   int64_t bt_sr, bt_sj;     // [R, MB]
    const int32_t *seq_lens; int64_t sl_s;         // [R]
    float *scores;       int64_t sc_sn, sc_sj;     // [N, MB], or [R, MB] when per_row
    int32_t R, T, MB, P;
    float idx_scale;
    int32_t per_row;                               // one sheet row per request: max over its tokens
};

struct TopkParams {
    const float *scores; int64_t sc_sn, sc_sj;     // [N, MB]
    int32_t *topk;       int64_t tk_sn, tk_si;     // [N, k]
    int32_t N, MB, k;
};

struct AttnParams {
    const void *q;       int64_t q_sn, q_sh;       // [N, Hq, D], inner stride 1
    const void *k_cache; int64_t k_sp, k_sb, k_sh; // [P, B, Hkv, D], inner stride 1
    const void *v_cache; int64_t v_sp, v_sb, v_sh;
    const int32_t *bt;   int64_t bt_sr, bt_sj;
    const int32_t *seq_lens; int64_t sl_s;
    const int32_t *topk; int64_t tk_sg, tk_sn, tk_si;  // [Hkv, N, k]; tk_sg = 0: [N, k] shared
    int32_t sel_per_row;                           // selection (and score) rows per request: [.., R, k]
    // selection computed in the attention kernel: score sheet in, topk out
    const float *scores; int64_t sc_sn, sc_sj;     // [N, MB]
    int32_t *topk_out;                             // same strides as topk
    int32_t R, T, MB, P, Hq, Hkv, k;
    int32_t splits;                                // S
    int32_t bpw;                                   // selected pages per page slot (token path)
    int32_t epw;                                   // selection entries per split (token path)
    float sm_scale, k_scale, v_scale;
    // split-K partials (workspace), see part_ml_index / part_acc_index
    float *part_ml, *part_acc;
    int32_t *counters;                             // [N, Hkv] x kCounterStride, zero between calls
    void *out; int64_t o_sn, o_sh, o_sd;           // [N, Hq, D] (token path writes it)
    int32_t out_bf16;
};

struct ReduceParams {
    const float *part_ml, *part_acc;
    void *out; int64_t o_sn, o_sh, o_sd;           // [N, Hq, D]
    int32_t N, Hq, D, splits;
    int32_t out_bf16;
    float v_scale;
};

// Ragged prefill score-to-selection (msa_prefill_block_score).  Work is cut
// into chunks of one request: up to kPrefillCols (token, query head) columns
// covering whole query blocks of all heads (bsq*Hq <= kPrefillCols), whole
// query blocks of a group of heads (bsq <= kPrefillCols), or a part of one
// query block of one head; the scoring workgroups share the chunks' visible
// blocks ("pages") evenly, in tiles of at most kPMaxPC blocks of one chunk.
constexpr int kPrefillWaves = 8;             // waves per scoring workgroup (two per SIMD)
constexpr int kPrefillWGsPerCU = 1;          // scoring workgroups resident per CU
constexpr int kPrefillCols = 16 * 4 * kPrefillWaves;   // columns of a chunk: 4 MFMA column tiles per wave
constexpr int kPlanMaxBatch = 8192;          // requests one call takes

struct PrefillGeom {
    int32_t hc;     // query heads per chunk
    int32_t nqc;    // query blocks per chunk
    int32_t NP;     // parts per query block (1 unless bsq > kPrefillCols)
    int32_t HG;     // head groups: ceil(Hq / hc)
    int64_t Cmax;   // chunks at most
    int64_t Wmax;   // share weight at most: every chunk's pages plus its ramp weight
};

struct PrefillSelParams {
    const uint16_t *q; int64_t q_st, q_sh;             // [total_q, Hq, Di] bf16, inner stride 1
    const uint8_t *index_k; int64_t k_sp, k_sb;        // [P, B, Di] FP8
    const int32_t *bt; int64_t bt_sr, bt_sj;           // [nslots, MB]
    const int32_t *slot_ids, *cu_seqlens, *seq_lens, *prefix_lens, *cu_qb;
    int64_t s_slot, s_cu, s_sl, s_pl, s_cq;            // their strides
    int32_t *out; int64_t o_sh, o_sq, o_si;            // [Hq, all_qb, topk]
    int32_t total_q, Hq, P, nslots, MB, batch, bsq, topk, init_blocks, local_blocks, all_qb;
    float scale;
    PrefillGeom g;
    int32_t nwg;                                       // workgroups of the scoring launch (multiple of 8)
    int32_t fused;                                     // selection inside the scoring launch
    // workspace (msa_prefill_block_score_workspace_bytes)
    int32_t *counters;  // [Hq, all_qb] arrival counters (zero between calls)
    int32_t *rowinfo;   // [all_qb]: request owning the query-block row, or -1
    float *ws;          // [Hq, all_qb, NP, MB] query-block maxima
};

PrefillGeom prefill_geom(int64_t batch, int64_t Hq, int64_t all_qb, int64_t MB, int64_t bsq);
size_t prefill_workspace_bytes(int64_t batch, int64_t Hq, int64_t all_qb, int64_t MB, int64_t bsq);
void prefill_carve_workspace(void *ws, int64_t batch, int64_t Hq, int64_t all_qb, int64_t MB, int64_t bsq,
                             PrefillSelParams &p);
hipError_t launch_prefill_select(const PrefillSelParams &p, int Di, hipStream_t s);

// Split partials in the workspace.  Split s of query token n leaves, per query
// head h, its running max m (log2 units) and sum l as a pair, and its
// unnormalised accumulator with the 8 consecutive d of group d/8 of all heads
// side by side, so that the 16 heads x 8 d one thread group writes are
// contiguous:
//   (m, l)       at part_ml[part_ml_index(s, n, h)]     (2 floats)
//   acc[d]       at part_acc[part_acc_index(s, n, h, d)]
// (the per-token MFMA unit, which merges its splits itself, leaves acc as
// 24-bit floats, four of them (index i .. i+3, i a multiple of 4) packed in
// the three words at ((uint32_t *)part_acc)[i / 4 * 3])
__host__ __device__ __forceinline__ int64_t part_ml_index(int s, int64_t n, int h, int64_t N, int Hq) {
    return (((int64_t)s * N + n) * Hq + h) * 2;
}
__host__ __device__ __forceinline__ int64_t part_acc_index(int s, int64_t n, int h, int d, int64_t N, int Hq,
                                                           int D) {
    return ((((int64_t)s * N + n) * (D / 8) + d / 8) * Hq + h) * 8 + (d & 7);
}

// Attention that computes each token's selection from the score sheet first
// (the decode step's second launch); MB <= 128.  Like the MFMA path of
// launch_attention it merges its splits itself.
hipError_t launch_attention_select(const AttnParams &p, int D, int kv_type, hipStream_t s);
constexpr int kSelectInAttnMaxMB = 128;

// Row-level attention (attend_row.hip): one workgroup per (row, KV head,
// split of the row's ascending list of selected blocks), each page loaded and
// decoded once per row for all of the row's tokens that selected it; the
// splits are merged by the reduction kernel.  Served for bf16 queries, FP8
// K/V, 16 query heads per KV head, D 64 or 128, 2 to 4 tokens per row,
// MB <= 128, sm_scale * k_scale > 0, and selections the tokens share (one
// per request), or per-token selections whose expected union is at most half
// of the pages the per-token unit would stream.
bool attention_row_eligible(int q_type, int kv_type, int D, int G, int T, int MB, int k, bool sel_per_row,
                            float score_scale);
int32_t row_splits(int32_t R, int32_t Hkv);
hipError_t launch_attention_row(const AttnParams &p, int D, bool select, hipStream_t s);

// Split plan of msa_sparse_decode for the given sizes and element types.
struct AttnPlan {
    bool mfma;          // per-token MFMA kernel with in-launch split merge (else union VALU + reduce)
    bool row;           // row-level MFMA kernel + reduce
    int32_t splits;
    int32_t bpw;
    int32_t epw;
};
AttnPlan attn_plan(int32_t R, int32_t T, int32_t Hq, int32_t Hkv, int32_t D, int32_t MB, int32_t k,
                   bool sel_per_row, float score_scale, int q_type, int kv_type);
size_t attn_workspace_bytes(int32_t R, int32_t T, int32_t Hq, int32_t Hkv, int32_t D, int32_t k);
size_t attn_workspace_bytes_for_splits(int32_t S, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                                       int32_t counter_slots);
void attn_carve_workspace(void *ws, int32_t S, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                          int32_t counter_slots, float **ml, float **acc, int32_t **counters);

// Launchers return hipSuccess or the launch error; dispatch on element types.
hipError_t launch_score(const ScoreParams &p, int q_type, int k_type, int Di, hipStream_t s);
hipError_t launch_topk(const TopkParams &p, hipStream_t s);
hipError_t launch_attention(const AttnParams &p, int q_type, int kv_type, int D, hipStream_t s);
hipError_t launch_reduce(const ReduceParams &p, hipStream_t s);

bool score_supported(int q_type, int k_type, int Di);
// a sheet row per request (the max over its T tokens) is served for decode rows
bool score_per_row_supported(int q_type, int k_type, int Di, int T);
bool attention_supported(int q_type, int kv_type, int D, int G);
bool attention_uses_mfma(int q_type, int kv_type, int G);

}  // namespace msa
