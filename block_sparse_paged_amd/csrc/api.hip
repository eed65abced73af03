// C ABI entry points (declared in include/msa.h): descriptor validation on the
// host, then kernel launches on the caller's stream.  Nothing here allocates,
// synchronises or keeps a pointer past the call.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "msa.h"
#include "msa_internal.h"

using namespace msa;

// Scratch of msa_decode_step_noalloc, for callers that cannot allocate: the
// step's split partials and arrival counters (16 MiB, one array per GPU, held
// until the process ends: room for every row-level plan of 16 query heads per
// KV head, whose partials come to about 8 MiB at any batch size).  Host code never passes `scratch` itself to a
// kernel: its device address comes from hipGetSymbolAddress (below).
constexpr size_t kScratchBytes = (size_t)16 << 20;
// arrival counters sit in a fixed region at its start (512 KiB, 2048 counters
// 256 bytes apart), so that a call never finds another call's partials where
// its counters are; every call leaves them at zero
constexpr int32_t kScratchCounters = 2048;
static __device__ __attribute__((aligned(256))) uint8_t scratch[kScratchBytes];

namespace {

thread_local int32_t g_last_error = MSA_OK;

void set_error(int32_t e) { g_last_error = e; }

struct Check {
    int32_t err = MSA_OK;
    bool ok() const { return err == MSA_OK; }
    void fail(int32_t e) {
        if (err == MSA_OK) err = e;
    }
};

int esize(int32_t dt) {
    switch (dt) {
    case MSA_F32: return 4;
    case MSA_BF16: return 2;
    case MSA_FP8_E4M3FN: return 1;
    case MSA_I32: return 4;
    }
    return 0;
}

// Basic descriptor sanity: non-null, ndim, non-negative sizes and strides.
void desc(Check &c, const msa_tensor *t, int ndim) {
    if (!t) { c.fail(MSA_ERR_NULL); return; }
    if (t->ndim != ndim) { c.fail(MSA_ERR_SHAPE); return; }
    int64_t numel = 1;
    for (int i = 0; i < ndim; ++i) {
        if (t->shape[i] < 0 || t->stride[i] < 0) { c.fail(MSA_ERR_SHAPE); return; }
        numel *= t->shape[i];
    }
    if (numel > 0 && !t->data) c.fail(MSA_ERR_NULL);
}

void dtype_in(Check &c, const msa_tensor *t, std::initializer_list<int32_t> ok) {
    if (!t) return;
    for (int32_t d : ok)
        if (t->dtype == d) return;
    c.fail(MSA_ERR_DTYPE);
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Innermost stride 1; the other strides and the base keep 16-byte rows aligned.
void rows16(Check &c, const msa_tensor *t) {
    if (!t || t->ndim < 1) return;
    const int es = esize(t->dtype);
    if (t->stride[t->ndim - 1] != 1 && t->shape[t->ndim - 1] > 1) { c.fail(MSA_ERR_LAYOUT); return; }
    if (!aligned16(t->data)) { c.fail(MSA_ERR_LAYOUT); return; }
    for (int i = 0; i < t->ndim - 1; ++i)
        if (t->shape[i] > 1 && ((t->stride[i] * es) & 15)) { c.fail(MSA_ERR_LAYOUT); return; }
}

bool fits_i32(int64_t x) { return x >= 0 && x <= 0x7fffffff; }

int etype(int32_t dt) {
    switch (dt) {
    case MSA_F32: return E_F32;
    case MSA_BF16: return E_BF16;
    case MSA_FP8_E4M3FN: return E_FP8;
    }
    return E_I32;
}

// Shared checks of block_table [R, MB] and seq_lens [R].
void paging(Check &c, const msa_tensor *bt, const msa_tensor *sl) {
    desc(c, bt, 2);
    desc(c, sl, 1);
    dtype_in(c, bt, {MSA_I32});
    dtype_in(c, sl, {MSA_I32});
    if (!c.ok()) return;
    if (sl->shape[0] != bt->shape[0]) c.fail(MSA_ERR_SHAPE);
    if (bt->shape[1] < 1 || bt->shape[1] > kMaxMB) c.fail(MSA_ERR_UNSUPPORTED);
}

}  // namespace

extern "C" {

int32_t msa_get_last_error(void) {
    const int32_t e = g_last_error;
    g_last_error = MSA_OK;
    return e;
}

const char *msa_error_string(int32_t code) {
    switch (code) {
    case MSA_OK: return "no error";
    case MSA_ERR_NULL: return "a required pointer is NULL";
    case MSA_ERR_DTYPE: return "dtype outside the supported set";
    case MSA_ERR_SHAPE: return "tensor rank or sizes disagree";
    case MSA_ERR_LAYOUT: return "innermost stride must be 1 with 16-byte aligned rows";
    case MSA_ERR_UNSUPPORTED: return "size outside the supported domain";
    case MSA_ERR_WORKSPACE: return "workspace missing or too small";
    case MSA_ERR_ARG: return "scalar argument out of range";
    case MSA_ERR_LAUNCH: return "kernel launch failed";
    case MSA_ERR_SCRATCH_LIMIT: return "sizes need more scratch than msa_decode_step_noalloc holds";
    case MSA_ERR_SCRATCH_SETUP: return "the scratch array's device address could not be obtained";
    }
    return "unknown error";
}

}  // extern "C"

namespace {

// ---- validation + parameter building shared by the entry points ------------

int32_t prep_score(const msa_tensor *q_idx, const msa_tensor *index_k, const msa_tensor *block_table,
                   const msa_tensor *seq_lens, int32_t tokens_per_row, int32_t block_size,
                   float idx_scale, msa_tensor *scores, ScoreParams &p, int &qt, int &kt, int &Di) {
    Check c;
    desc(c, q_idx, 2);
    desc(c, index_k, 3);
    desc(c, scores, 2);
    paging(c, block_table, seq_lens);
    dtype_in(c, q_idx, {MSA_BF16, MSA_F32});
    dtype_in(c, index_k, {MSA_FP8_E4M3FN, MSA_F32});
    dtype_in(c, scores, {MSA_F32});
    if (!c.ok()) return c.err;
    if (block_size != kBlock) c.fail(MSA_ERR_UNSUPPORTED);
    if (tokens_per_row < 1) c.fail(MSA_ERR_ARG);
    if (!(idx_scale > 0.f) || !isfinite(idx_scale)) c.fail(MSA_ERR_ARG);
    const int64_t R = block_table->shape[0], MB = block_table->shape[1];
    const int64_t N = R * (int64_t)tokens_per_row;
    Di = (int)q_idx->shape[1];
    // [N, MB]: one row per query token; [R, MB] with T > 1: one row per
    // request, the max over its tokens
    const bool per_row = tokens_per_row > 1 && scores->shape[0] == R;
    if (q_idx->shape[0] != N || (scores->shape[0] != N && !per_row) || scores->shape[1] != MB)
        c.fail(MSA_ERR_SHAPE);
    if (index_k->shape[1] != kBlock || index_k->shape[2] != Di) c.fail(MSA_ERR_SHAPE);
    qt = etype(q_idx->dtype);
    kt = etype(index_k->dtype);
    if (!score_supported(qt, kt, Di)) c.fail(MSA_ERR_UNSUPPORTED);
    if (per_row && !score_per_row_supported(qt, kt, Di, tokens_per_row)) c.fail(MSA_ERR_UNSUPPORTED);
    if (!fits_i32(N) || !fits_i32(index_k->shape[0])) c.fail(MSA_ERR_UNSUPPORTED);
    rows16(c, q_idx);
    rows16(c, index_k);
    if (!c.ok()) return c.err;
    p = ScoreParams{};
    p.q_idx = q_idx->data; p.q_sn = q_idx->stride[0];
    p.index_k = index_k->data; p.k_sp = index_k->stride[0]; p.k_sb = index_k->stride[1];
    p.bt = (const int32_t *)block_table->data;
    p.bt_sr = block_table->stride[0]; p.bt_sj = block_table->stride[1];
    p.seq_lens = (const int32_t *)seq_lens->data; p.sl_s = seq_lens->stride[0];
    p.scores = (float *)scores->data; p.sc_sn = scores->stride[0]; p.sc_sj = scores->stride[1];
    p.R = (int32_t)R; p.T = tokens_per_row; p.MB = (int32_t)MB;
    p.P = (int32_t)index_k->shape[0];
    p.idx_scale = idx_scale;
    p.per_row = per_row;
    return MSA_OK;
}

int32_t prep_topk(const msa_tensor *scores, int32_t k, msa_tensor *topk_idx, TopkParams &p) {
    Check c;
    desc(c, scores, 2);
    desc(c, topk_idx, 2);
    dtype_in(c, scores, {MSA_F32});
    dtype_in(c, topk_idx, {MSA_I32});
    if (!c.ok()) return c.err;
    const int64_t N = scores->shape[0], MB = scores->shape[1];
    if (MB < 1 || MB > kMaxMB) c.fail(MSA_ERR_UNSUPPORTED);
    if (k < 1 || k > MB) c.fail(MSA_ERR_ARG);
    if (topk_idx->shape[0] != N || topk_idx->shape[1] != k) c.fail(MSA_ERR_SHAPE);
    if (!fits_i32(N)) c.fail(MSA_ERR_UNSUPPORTED);
    if (!c.ok()) return c.err;
    p = TopkParams{};
    p.scores = (const float *)scores->data; p.sc_sn = scores->stride[0]; p.sc_sj = scores->stride[1];
    p.topk = (int32_t *)topk_idx->data; p.tk_sn = topk_idx->stride[0]; p.tk_si = topk_idx->stride[1];
    p.N = (int32_t)N; p.MB = (int32_t)MB; p.k = k;
    return MSA_OK;
}

// Validates the attention arguments and fills p except the workspace pointers.
int32_t prep_attn(const msa_tensor *q, const msa_tensor *k_cache, const msa_tensor *v_cache,
                  const msa_tensor *block_table, const msa_tensor *seq_lens, const msa_tensor *topk_idx,
                  int32_t tokens_per_row, msa_tensor *out, float sm_scale, float k_scale, float v_scale,
                  int32_t block_size, AttnParams &p, AttnPlan &plan, int &qt, int &kvt, int &D) {
    Check c;
    desc(c, q, 3);
    desc(c, k_cache, 4);
    desc(c, v_cache, 4);
    // [N, k] shared by the KV heads, or [Hkv, N, k] one selection per KV head
    const bool per_head = topk_idx && topk_idx->ndim == 3;
    desc(c, topk_idx, per_head ? 3 : 2);
    desc(c, out, 3);
    paging(c, block_table, seq_lens);
    dtype_in(c, q, {MSA_BF16, MSA_F32});
    dtype_in(c, k_cache, {MSA_FP8_E4M3FN, MSA_BF16, MSA_F32});
    dtype_in(c, topk_idx, {MSA_I32});
    dtype_in(c, out, {MSA_BF16, MSA_F32});
    if (!c.ok()) return c.err;
    if (v_cache->dtype != k_cache->dtype) c.fail(MSA_ERR_DTYPE);
    if (block_size != kBlock) c.fail(MSA_ERR_UNSUPPORTED);
    if (tokens_per_row < 1) c.fail(MSA_ERR_ARG);
    if (!isfinite(sm_scale) || !isfinite(k_scale) || !isfinite(v_scale)) c.fail(MSA_ERR_ARG);
    const int64_t R = block_table->shape[0], MB = block_table->shape[1];
    const int64_t N = R * (int64_t)tokens_per_row;
    const int64_t Hq = q->shape[1];
    D = (int)q->shape[2];
    const int64_t P = k_cache->shape[0], Hkv = k_cache->shape[2];
    const int64_t K = topk_idx->shape[per_head ? 2 : 1];
    // selection rows: one per query token, or (T > 1) one per request shared
    // by its tokens
    const int64_t trows = topk_idx->shape[per_head ? 1 : 0];
    const bool sel_per_row = tokens_per_row > 1 && trows == R;
    if (q->shape[0] != N || (trows != N && !sel_per_row)) c.fail(MSA_ERR_SHAPE);
    if (per_head && topk_idx->shape[0] != Hkv) c.fail(MSA_ERR_SHAPE);
    if (k_cache->shape[1] != kBlock || k_cache->shape[3] != D) c.fail(MSA_ERR_SHAPE);
    for (int i = 0; i < 4; ++i)
        if (v_cache->shape[i] != k_cache->shape[i]) c.fail(MSA_ERR_SHAPE);
    if (out->shape[0] != N || out->shape[1] != Hq || out->shape[2] != D) c.fail(MSA_ERR_SHAPE);
    if (Hkv < 1 || Hq < 1 || Hq % Hkv) c.fail(MSA_ERR_SHAPE);
    if (K < 1) c.fail(MSA_ERR_SHAPE);
    if (!c.ok()) return c.err;
    qt = etype(q->dtype);
    kvt = etype(k_cache->dtype);
    if (!attention_supported(qt, kvt, D, (int)(Hq / Hkv))) c.fail(MSA_ERR_UNSUPPORTED);
    if (!fits_i32(N) || !fits_i32(P) || K > kMaxMB) c.fail(MSA_ERR_UNSUPPORTED);
    rows16(c, q);
    rows16(c, k_cache);
    rows16(c, v_cache);
    if (!c.ok()) return c.err;
    p = AttnParams{};
    p.q = q->data; p.q_sn = q->stride[0]; p.q_sh = q->stride[1];
    p.k_cache = k_cache->data;
    p.k_sp = k_cache->stride[0]; p.k_sb = k_cache->stride[1]; p.k_sh = k_cache->stride[2];
    p.v_cache = v_cache->data;
    p.v_sp = v_cache->stride[0]; p.v_sb = v_cache->stride[1]; p.v_sh = v_cache->stride[2];
    p.bt = (const int32_t *)block_table->data;
    p.bt_sr = block_table->stride[0]; p.bt_sj = block_table->stride[1];
    p.seq_lens = (const int32_t *)seq_lens->data; p.sl_s = seq_lens->stride[0];
    p.topk = (const int32_t *)topk_idx->data;
    p.tk_sg = per_head ? topk_idx->stride[0] : 0;
    p.tk_sn = topk_idx->stride[per_head ? 1 : 0];
    p.tk_si = topk_idx->stride[per_head ? 2 : 1];
    p.sel_per_row = sel_per_row;
    p.R = (int32_t)R; p.T = tokens_per_row; p.MB = (int32_t)MB; p.P = (int32_t)P;
    p.Hq = (int32_t)Hq; p.Hkv = (int32_t)Hkv; p.k = (int32_t)K;
    plan = attn_plan((int32_t)R, tokens_per_row, (int32_t)Hq, (int32_t)Hkv, (int32_t)D, (int32_t)MB, (int32_t)K,
                     sel_per_row, sm_scale * k_scale, qt, kvt);
    p.splits = plan.splits;
    p.bpw = plan.bpw;
    p.epw = plan.epw;
    p.sm_scale = sm_scale; p.k_scale = k_scale; p.v_scale = v_scale;
    p.out = out->data; p.o_sn = out->stride[0]; p.o_sh = out->stride[1]; p.o_sd = out->stride[2];
    p.out_bf16 = out->dtype == MSA_BF16;
    return MSA_OK;
}

// the merge kernel over the split partials the VALU and row-level attention
// launches left (the per-token MFMA launch merges its splits itself)
int32_t run_merge(const AttnParams &p, const AttnPlan &plan, int D, hipStream_t stream) {
    if (plan.mfma && !plan.row) return MSA_OK;
    ReduceParams rp{};
    rp.part_ml = p.part_ml; rp.part_acc = p.part_acc;
    rp.out = p.out; rp.o_sn = p.o_sn; rp.o_sh = p.o_sh; rp.o_sd = p.o_sd;
    rp.N = p.R * p.T; rp.Hq = p.Hq; rp.D = D; rp.splits = p.splits;
    rp.out_bf16 = p.out_bf16;
    rp.v_scale = p.v_scale;
    return launch_reduce(rp, stream) == hipSuccess ? MSA_OK : MSA_ERR_LAUNCH;
}

// attention + merge with the workspace already carved
int32_t run_attn(AttnParams &p, const AttnPlan &plan, int qt, int kvt, int D, hipStream_t stream) {
    const hipError_t le = plan.row ? launch_attention_row(p, D, false, stream) : launch_attention(p, qt, kvt, D, stream);
    if (le != hipSuccess) return MSA_ERR_LAUNCH;
    return run_merge(p, plan, D, stream);
}

// selection + attention + merge.  On the MFMA path with MB <= 128 the
// selection runs inside the attention launch: each workgroup selects its
// token's blocks from the score row (the same wave-level select as the top-k
// kernel) and one of them stores topk_idx; otherwise the top-k kernel runs
// first.
int32_t run_select_attn(const TopkParams &tk, AttnParams &at, const AttnPlan &plan, int qt, int kvt,
                        int D, hipStream_t stream) {
    if (plan.mfma && tk.MB <= kSelectInAttnMaxMB) {
        at.scores = tk.scores; at.sc_sn = tk.sc_sn; at.sc_sj = tk.sc_sj;
        at.topk_out = tk.topk;
        if (plan.row) {
            if (launch_attention_row(at, D, true, stream) != hipSuccess) return MSA_ERR_LAUNCH;
            return run_merge(at, plan, D, stream);
        }
        return launch_attention_select(at, D, kvt, stream) == hipSuccess ? MSA_OK : MSA_ERR_LAUNCH;
    }
    if (launch_topk(tk, stream) != hipSuccess) return MSA_ERR_LAUNCH;
    return run_attn(at, plan, qt, kvt, D, stream);
}

// Validates the ragged prefill arguments and fills p except the workspace.
int32_t prep_prefill(const msa_tensor *q, const msa_tensor *index_k, const msa_tensor *block_table,
                     const msa_tensor *slot_ids, const msa_tensor *cu_seqlens, const msa_tensor *seq_lens,
                     const msa_tensor *prefix_lens, int32_t block_size_q, int32_t block_size_k, int32_t topk,
                     int32_t init_blocks, int32_t local_blocks, float scale,
                     const msa_tensor *cu_seqblocks_q, msa_tensor *out_topk, PrefillSelParams &p, int &Di) {
    Check c;
    desc(c, q, 3);
    desc(c, index_k, 3);
    desc(c, block_table, 2);
    desc(c, slot_ids, 1);
    desc(c, cu_seqlens, 1);
    desc(c, seq_lens, 1);
    desc(c, prefix_lens, 1);
    desc(c, cu_seqblocks_q, 1);
    desc(c, out_topk, 3);
    dtype_in(c, q, {MSA_BF16});
    dtype_in(c, index_k, {MSA_FP8_E4M3FN});
    for (const msa_tensor *t : {block_table, slot_ids, cu_seqlens, seq_lens, prefix_lens, cu_seqblocks_q,
                                (const msa_tensor *)out_topk})
        dtype_in(c, t, {MSA_I32});
    if (!c.ok()) return c.err;
    const int64_t total_q = q->shape[0], Hq = q->shape[1];
    Di = (int)q->shape[2];
    const int64_t P = index_k->shape[0], nslots = block_table->shape[0], MB = block_table->shape[1];
    const int64_t batch = slot_ids->shape[0], all_qb = out_topk->shape[1];
    if (seq_lens->shape[0] != batch || prefix_lens->shape[0] != batch || cu_seqlens->shape[0] != batch + 1 ||
        cu_seqblocks_q->shape[0] != batch + 1)
        c.fail(MSA_ERR_SHAPE);
    if (index_k->shape[1] != kBlock || index_k->shape[2] != Di) c.fail(MSA_ERR_SHAPE);
    if (out_topk->shape[0] != Hq || out_topk->shape[2] != topk) c.fail(MSA_ERR_SHAPE);
    if (Hq < 1) c.fail(MSA_ERR_SHAPE);
    if (!c.ok()) return c.err;
    if (Di != 64 && Di != 128) c.fail(MSA_ERR_UNSUPPORTED);
    if (block_size_k != kBlock) c.fail(MSA_ERR_UNSUPPORTED);
    if (MB < 1 || MB > kMaxMB) c.fail(MSA_ERR_UNSUPPORTED);
    if (batch > kPlanMaxBatch) c.fail(MSA_ERR_UNSUPPORTED);
    if (block_size_q < 1 || topk < 1 || init_blocks < 0 || local_blocks < 0) c.fail(MSA_ERR_ARG);
    if (!(scale > 0.f) || !isfinite(scale)) c.fail(MSA_ERR_ARG);
    if (!fits_i32(total_q) || !fits_i32(P) || !fits_i32(nslots) || !fits_i32(all_qb) ||
        !fits_i32(Hq * all_qb))
        c.fail(MSA_ERR_UNSUPPORTED);
    if (!c.ok()) return c.err;
    const PrefillGeom g = prefill_geom(batch, Hq, all_qb, MB, block_size_q);
    if (g.Wmax > 0x7fffffff) c.fail(MSA_ERR_UNSUPPORTED);   // share weights are counted in int
    rows16(c, q);
    rows16(c, index_k);
    if (!c.ok()) return c.err;
    p = PrefillSelParams{};
    p.q = (const uint16_t *)q->data; p.q_st = q->stride[0]; p.q_sh = q->stride[1];
    p.index_k = (const uint8_t *)index_k->data; p.k_sp = index_k->stride[0]; p.k_sb = index_k->stride[1];
    p.bt = (const int32_t *)block_table->data; p.bt_sr = block_table->stride[0]; p.bt_sj = block_table->stride[1];
    p.slot_ids = (const int32_t *)slot_ids->data; p.s_slot = slot_ids->stride[0];
    p.cu_seqlens = (const int32_t *)cu_seqlens->data; p.s_cu = cu_seqlens->stride[0];
    p.seq_lens = (const int32_t *)seq_lens->data; p.s_sl = seq_lens->stride[0];
    p.prefix_lens = (const int32_t *)prefix_lens->data; p.s_pl = prefix_lens->stride[0];
    p.cu_qb = (const int32_t *)cu_seqblocks_q->data; p.s_cq = cu_seqblocks_q->stride[0];
    p.out = (int32_t *)out_topk->data;
    p.o_sh = out_topk->stride[0]; p.o_sq = out_topk->stride[1]; p.o_si = out_topk->stride[2];
    p.total_q = (int32_t)total_q; p.Hq = (int32_t)Hq; p.P = (int32_t)P; p.nslots = (int32_t)nslots;
    p.MB = (int32_t)MB; p.batch = (int32_t)batch; p.bsq = block_size_q; p.topk = topk;
    p.init_blocks = init_blocks; p.local_blocks = local_blocks; p.all_qb = (int32_t)all_qb;
    p.scale = scale;
    return MSA_OK;
}

// workgroups of the persistent prefill scoring launch: kPrefillWGsPerCU per
// CU of the current device, a multiple of the 8 XCDs
int32_t prefill_workgroups() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256 * kPrefillWGsPerCU;
    if (!cache[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 8) n = 256;
        cache[dev] = n / 8 * 8 * kPrefillWGsPerCU;
    }
    return cache[dev];
}

// ---- scratch of msa_decode_step_noalloc ------------------------------------
//
// For callers that cannot allocate: the split partials and arrival counters
// live in this file-scope device array (each GPU the library runs on holds its
// own copy until the process ends).  In host code `scratch` names a host-side
// stand-in, not the array's device address: the address is looked up once per
// device with hipGetSymbolAddress and only that pointer is handed to kernels.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};
bool g_scratch_zeroed[kMaxDevices] = {};   // a zero fill has been enqueued outside graph capture

__global__ void scratch_zero_kernel(uint4 *p, size_t n16) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The current device's scratch address, looked up once per device (with the
// device current) by the first call on it.  Until a zero fill of the array has
// been enqueued outside graph capture, every call enqueues one on `stream`
// ahead of its kernels (a kernel, so that a call being captured records no
// memset node; a captured fill runs at each replay of that graph); after that
// the arrival counters are zero between calls because every call's kernels
// leave them at zero.
int32_t scratch_for_current_device(hipStream_t stream, void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MSA_ERR_SCRATCH_SETUP;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MSA_ERR_SCRATCH_SETUP;
        g_scratch_ptr[dev] = p;
    }
    if (!g_scratch_zeroed[dev]) {
        hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(stream, &st) != hipSuccess) return MSA_ERR_SCRATCH_SETUP;
        hipLaunchKernelGGL(scratch_zero_kernel, dim3(512), dim3(256), 0, stream, (uint4 *)g_scratch_ptr[dev],
                           kScratchBytes / 16);
        if (hipGetLastError() != hipSuccess) return MSA_ERR_LAUNCH;
        if (st == hipStreamCaptureStatusNone) g_scratch_zeroed[dev] = true;
    }
    *out = g_scratch_ptr[dev];
    return MSA_OK;
}

// The whole step (msa_decode_step and msa_decode_step_noalloc): validation,
// then the launches on `stream` with the split partials and arrival counters
// in the workspace, or with `scratch` set in the device's scratch array
// (sizes that need more than it holds are rejected before anything is
// enqueued).
int32_t decode_step(const msa_tensor *q_idx, const msa_tensor *index_k, const msa_tensor *q,
                    const msa_tensor *k_cache, const msa_tensor *v_cache, const msa_tensor *block_table,
                    const msa_tensor *seq_lens, int32_t tokens_per_row, int32_t k, int32_t block_size,
                    float idx_scale, float sm_scale, float k_scale, float v_scale, msa_tensor *scores,
                    msa_tensor *topk_idx, msa_tensor *out, void *workspace, size_t workspace_bytes, bool scratch,
                    hipStream_t stream) {
    ScoreParams sc;
    TopkParams tk;
    AttnParams at;
    AttnPlan plan;
    int qit, kit, Di, qt, kvt, D;
    int32_t e = prep_score(q_idx, index_k, block_table, seq_lens, tokens_per_row, block_size, idx_scale,
                           scores, sc, qit, kit, Di);
    if (e == MSA_OK) e = prep_topk(scores, k, topk_idx, tk);
    if (e == MSA_OK)
        e = prep_attn(q, k_cache, v_cache, block_table, seq_lens, topk_idx, tokens_per_row, out, sm_scale,
                      k_scale, v_scale, block_size, at, plan, qt, kvt, D);
    if (e == MSA_OK && k_cache->shape[0] != index_k->shape[0]) e = MSA_ERR_SHAPE;
    if (e == MSA_OK && (bool)sc.per_row != (bool)at.sel_per_row) e = MSA_ERR_SHAPE;
    if (e != MSA_OK) return e;
    const int32_t N = sc.R * sc.T;
    if (N == 0) return MSA_OK;
    size_t need = attn_workspace_bytes(sc.R, sc.T, at.Hq, at.Hkv, D, k);
    if (scratch) {
        // the scratch array holds what this call's plan touches
        need = attn_workspace_bytes_for_splits(at.splits, N, at.Hq, at.Hkv, D, kScratchCounters);
        if (need > kScratchBytes || (int64_t)N * at.Hkv > kScratchCounters) return MSA_ERR_SCRATCH_LIMIT;
        const int32_t se = scratch_for_current_device(stream, &workspace);
        if (se != MSA_OK) return se;
        workspace_bytes = kScratchBytes;
    }
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u)) return MSA_ERR_WORKSPACE;
    attn_carve_workspace(workspace, at.splits, N, at.Hq, at.Hkv, D, scratch ? kScratchCounters : 0, &at.part_ml,
                         &at.part_acc, &at.counters);
    if (launch_score(sc, qit, kit, Di, stream) != hipSuccess) return MSA_ERR_LAUNCH;
    return run_select_attn(tk, at, plan, qt, kvt, D, stream);
}

}  // namespace

extern "C" {

void msa_block_score(const msa_tensor *q_idx, const msa_tensor *index_k,
                     const msa_tensor *block_table, const msa_tensor *seq_lens,
                     int32_t tokens_per_row, int32_t block_size, float idx_scale,
                     msa_tensor *scores, hipStream_t stream) {
    ScoreParams p;
    int qt, kt, Di;
    const int32_t e = prep_score(q_idx, index_k, block_table, seq_lens, tokens_per_row, block_size,
                                 idx_scale, scores, p, qt, kt, Di);
    if (e != MSA_OK) { set_error(e); return; }
    if (p.R == 0) return;
    if (launch_score(p, qt, kt, Di, stream) != hipSuccess) set_error(MSA_ERR_LAUNCH);
}

void msa_select_topk(const msa_tensor *scores, int32_t k, msa_tensor *topk_idx,
                     hipStream_t stream) {
    TopkParams p;
    const int32_t e = prep_topk(scores, k, topk_idx, p);
    if (e != MSA_OK) { set_error(e); return; }
    if (p.N == 0) return;
    if (launch_topk(p, stream) != hipSuccess) set_error(MSA_ERR_LAUNCH);
}

size_t msa_sparse_decode_workspace_bytes(int32_t rows, int32_t tokens_per_row,
                                         int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t k) {
    if (rows < 0 || tokens_per_row < 1 || num_q_heads < 1 || num_kv_heads < 1 || head_dim < 1 || k < 1)
        return 0;
    return attn_workspace_bytes(rows, tokens_per_row, num_q_heads, num_kv_heads, head_dim, k);
}

void msa_sparse_decode(const msa_tensor *q, const msa_tensor *k_cache,
                       const msa_tensor *v_cache, const msa_tensor *block_table,
                       const msa_tensor *seq_lens, const msa_tensor *topk_idx,
                       int32_t tokens_per_row, msa_tensor *out,
                       float sm_scale, float k_scale, float v_scale, int32_t block_size,
                       void *workspace, size_t workspace_bytes, hipStream_t stream) {
    AttnParams p;
    AttnPlan plan;
    int qt, kvt, D;
    const int32_t e = prep_attn(q, k_cache, v_cache, block_table, seq_lens, topk_idx, tokens_per_row,
                                out, sm_scale, k_scale, v_scale, block_size, p, plan, qt, kvt, D);
    if (e != MSA_OK) { set_error(e); return; }
    const int32_t N = p.R * p.T;
    if (N == 0) return;
    const size_t need = attn_workspace_bytes(p.R, p.T, p.Hq, p.Hkv, D, p.k);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u)) {
        set_error(MSA_ERR_WORKSPACE);
        return;
    }
    attn_carve_workspace(workspace, p.splits, N, p.Hq, p.Hkv, D, 0, &p.part_ml, &p.part_acc,
                         &p.counters);
    const int32_t r = run_attn(p, plan, qt, kvt, D, stream);
    if (r != MSA_OK) set_error(r);
}

size_t msa_decode_step_workspace_bytes(int32_t rows, int32_t tokens_per_row, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t k) {
    return msa_sparse_decode_workspace_bytes(rows, tokens_per_row, num_q_heads, num_kv_heads, head_dim, k);
}

void msa_select_sparse_decode(const msa_tensor *scores, int32_t k, msa_tensor *topk_idx,
                              const msa_tensor *q, const msa_tensor *k_cache,
                              const msa_tensor *v_cache, const msa_tensor *block_table,
                              const msa_tensor *seq_lens, int32_t tokens_per_row, msa_tensor *out,
                              float sm_scale, float k_scale, float v_scale, int32_t block_size,
                              void *workspace, size_t workspace_bytes, hipStream_t stream) {
    TopkParams tk;
    AttnParams at;
    AttnPlan plan;
    int qt, kvt, D;
    int32_t e = prep_topk(scores, k, topk_idx, tk);
    if (e == MSA_OK)
        e = prep_attn(q, k_cache, v_cache, block_table, seq_lens, topk_idx, tokens_per_row, out, sm_scale,
                      k_scale, v_scale, block_size, at, plan, qt, kvt, D);
    if (e == MSA_OK && (scores->shape[0] != (at.sel_per_row ? (int64_t)at.R : (int64_t)at.R * at.T) ||
                        scores->shape[1] != at.MB))
        e = MSA_ERR_SHAPE;
    if (e != MSA_OK) { set_error(e); return; }
    const int32_t N = at.R * at.T;
    if (N == 0) return;
    const size_t need = attn_workspace_bytes(at.R, at.T, at.Hq, at.Hkv, D, k);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u)) {
        set_error(MSA_ERR_WORKSPACE);
        return;
    }
    attn_carve_workspace(workspace, at.splits, N, at.Hq, at.Hkv, D, 0, &at.part_ml,
                         &at.part_acc, &at.counters);
    const int32_t r = run_select_attn(tk, at, plan, qt, kvt, D, stream);
    if (r != MSA_OK) set_error(r);
}

void msa_decode_step(const msa_tensor *q_idx, const msa_tensor *index_k, const msa_tensor *q,
                     const msa_tensor *k_cache, const msa_tensor *v_cache,
                     const msa_tensor *block_table, const msa_tensor *seq_lens,
                     int32_t tokens_per_row, int32_t k, int32_t block_size,
                     float idx_scale, float sm_scale, float k_scale, float v_scale,
                     msa_tensor *scores, msa_tensor *topk_idx, msa_tensor *out,
                     void *workspace, size_t workspace_bytes, hipStream_t stream) {
    const int32_t e = decode_step(q_idx, index_k, q, k_cache, v_cache, block_table, seq_lens, tokens_per_row, k,
                                  block_size, idx_scale, sm_scale, k_scale, v_scale, scores, topk_idx, out,
                                  workspace, workspace_bytes, false, stream);
    if (e != MSA_OK) set_error(e);
}

void msa_decode_step_noalloc(const msa_tensor *q_idx, const msa_tensor *index_k, const msa_tensor *q,
                             const msa_tensor *k_cache, const msa_tensor *v_cache,
                             const msa_tensor *block_table, const msa_tensor *seq_lens,
                             int32_t tokens_per_row, int32_t k, int32_t block_size,
                             float idx_scale, float sm_scale, float k_scale, float v_scale,
                             msa_tensor *scores, msa_tensor *topk_idx, msa_tensor *out,
                             hipStream_t stream) {
    const int32_t e = decode_step(q_idx, index_k, q, k_cache, v_cache, block_table, seq_lens, tokens_per_row, k,
                                  block_size, idx_scale, sm_scale, k_scale, v_scale, scores, topk_idx, out,
                                  nullptr, 0, true, stream);
    if (e != MSA_OK) set_error(e);
}

size_t msa_prefill_block_score_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t all_seqblock_q,
                                               int32_t max_blocks, int32_t block_size_q) {
    if (batch < 0 || num_q_heads < 1 || all_seqblock_q < 0 || max_blocks < 1 || block_size_q < 1) return 0;
    return prefill_workspace_bytes(batch, num_q_heads, all_seqblock_q, max_blocks, block_size_q);
}

void msa_prefill_block_score(const msa_tensor *q, const msa_tensor *index_k, const msa_tensor *block_table,
                             const msa_tensor *slot_ids, const msa_tensor *cu_seqlens,
                             const msa_tensor *seq_lens, const msa_tensor *prefix_lens,
                             int32_t block_size_q, int32_t block_size_k, int32_t topk, int32_t init_blocks,
                             int32_t local_blocks, float scale, const msa_tensor *cu_seqblocks_q,
                             msa_tensor *out_topk, void *workspace, size_t workspace_bytes,
                             hipStream_t stream) {
    PrefillSelParams p;
    int Di;
    const int32_t e = prep_prefill(q, index_k, block_table, slot_ids, cu_seqlens, seq_lens, prefix_lens,
                                   block_size_q, block_size_k, topk, init_blocks, local_blocks, scale,
                                   cu_seqblocks_q, out_topk, p, Di);
    if (e != MSA_OK) { set_error(e); return; }
    if ((int64_t)p.Hq * p.all_qb == 0) return;
    const size_t need = prefill_workspace_bytes(p.batch, p.Hq, p.all_qb, p.MB, p.bsq);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u)) {
        set_error(MSA_ERR_WORKSPACE);
        return;
    }
    prefill_carve_workspace(workspace, p.batch, p.Hq, p.all_qb, p.MB, p.bsq, p);
    p.nwg = prefill_workgroups();
    if (launch_prefill_select(p, Di, stream) != hipSuccess) set_error(MSA_ERR_LAUNCH);
}

}  // extern "C"
