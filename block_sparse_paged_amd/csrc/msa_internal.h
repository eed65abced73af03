// Internal declarations shared by the gfx950 kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

constexpr int kBlock = 128;          // tokens per page (vLLM design note: block size 128)
constexpr int kMaxMB = 2048;         // logical blocks per row served by select/attention
constexpr int kTokGroup = 4;         // query tokens of one row handled together
constexpr int kSplitTargetWGs = 256; // attention workgroups aimed for (one per CU)
constexpr int kCounterStride = 64;   // int32s between split-arrival counters (one per 256 B)

enum ElemType { E_F32 = 0, E_BF16 = 1, E_FP8 = 2, E_I32 = 3 };

struct ScoreParams {
    const void *q_idx;   int64_t q_sn;             // [N, Di], inner stride 1
    const void *index_k; int64_t k_sp, k_sb;       // [P, B, Di], inner stride 1
    const int32_t *bt;   int64_t bt_sr, bt_sj;     // [R, MB]
    const int32_t *seq_lens; int64_t sl_s;         // [R]
    float *scores;       int64_t sc_sn, sc_sj;     // [N, MB]
    int32_t R, T, MB, P;
    float idx_scale;
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
    const int32_t *topk; int64_t tk_sn, tk_si;     // [N, k]
    // selection computed in the attention kernel: score sheet in, topk out
    const float *scores; int64_t sc_sn, sc_sj;     // [N, MB]
    int32_t *topk_out;                             // same strides as topk
    int32_t R, T, MB, P, Hq, Hkv, k;
    int32_t splits;                                // S
    int32_t bpw;                                   // selected pages per wave (token path)
    float sm_scale, k_scale, v_scale;
    // split-K partials (workspace): m, l [S, N, Hq]; acc [S, N, Hq, D]
    float *part_m, *part_l, *part_acc;
    int32_t *counters;                             // [N, Hkv] x kCounterStride, zero between calls
    void *out; int64_t o_sn, o_sh, o_sd;           // [N, Hq, D] (token path writes it)
    int32_t out_bf16;
};

struct ReduceParams {
    const float *part_m, *part_l, *part_acc;
    void *out; int64_t o_sn, o_sh, o_sd;           // [N, Hq, D]
    int32_t N, Hq, D, splits;
    int32_t out_bf16;
    float v_scale;
};

// Attention that computes each token's selection from the score sheet first
// (the decode step's second launch); MB <= 128.  merge: the splits are merged
// in the same launch through the workspace counters (else the merge kernel
// must follow when splits > 1).
hipError_t launch_attention_select(const AttnParams &p, int D, bool merge, hipStream_t s);
constexpr int kSelectInAttnMaxMB = 128;

// Split plan of msa_sparse_decode for the given sizes and element types.
struct AttnPlan {
    bool mfma;          // per-token MFMA kernel with in-kernel merge (else union VALU + reduce)
    int32_t splits;
    int32_t bpw;
};
AttnPlan attn_plan(int32_t R, int32_t T, int32_t Hq, int32_t Hkv, int32_t k, int q_type, int kv_type);
size_t attn_workspace_bytes(int32_t R, int32_t T, int32_t Hq, int32_t Hkv, int32_t D, int32_t k);
void attn_carve_workspace(void *ws, int32_t S, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                          float **m, float **l, float **acc, int32_t **counters);

// Launchers return hipSuccess or the launch error; dispatch on element types.
hipError_t launch_score(const ScoreParams &p, int q_type, int k_type, int Di, hipStream_t s);
hipError_t launch_topk(const TopkParams &p, hipStream_t s);
hipError_t launch_attention(const AttnParams &p, int q_type, int kv_type, int D, hipStream_t s);
hipError_t launch_reduce(const ReduceParams &p, hipStream_t s);

bool score_supported(int q_type, int k_type, int Di);
bool attention_supported(int q_type, int kv_type, int D, int G);
bool attention_uses_mfma(int q_type, int kv_type, int G);

}  // namespace msa
