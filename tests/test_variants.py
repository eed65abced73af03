"""GPU parity of the attention-boundary variants of attention.decode (Cacheon
"Kernel ABI", "Attention block slots"): a selection per KV head in the
(Hkv, B, K) layout, and the dense bf16 K/V cache.  Each is compared with the
oracle on the same inputs to the attention bar (bf16-rounded outputs within
2e-3 max-abs)."""
import numpy as np
import pytest
import torch

import synth
from msa_harness import check_attention, check_scores, oracle_attention, poisoned, upload, workspace

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def msa():
    import block_sparse_paged_amd as m
    return m


def per_head_topk(case, seeds):
    """[Hkv, N, k] int32: an independent random selection per KV head."""
    tk = np.stack([synth.random_topk(case, seed=s).numpy() for s in seeds])
    for g in range(1, tk.shape[0]):
        assert not np.array_equal(tk[0], tk[g])
    return tk


def attend(msa, case, d, topk, out_dtype=torch.bfloat16):
    out = poisoned((case.N, case.Hq, case.D), out_dtype)
    msa.msa_sparse_decode(d.q, d.k_cache, d.v_cache, d.block_table, d.seq_lens, topk, case.T, out,
                          case.sm_scale, case.k_scale, case.v_scale, case.B,
                          workspace(msa, case, topk.shape[-1]))
    torch.cuda.synchronize()
    return out


PER_HEAD = [
    # MFMA path: bf16 queries, FP8 caches, 16 query heads per KV head
    dict(R=2, T=4, Hq=32, Hkv=2, D=128, Di=128, seq_lens=[900, 2100], P=30, k=5),
    # vector path: 4 query heads per KV head, D = 64
    dict(R=2, T=3, Hq=8, Hkv=2, D=64, Di=64, seq_lens=[700, 1300], P=20, k=4),
]


@pytest.mark.parametrize("spec", PER_HEAD, ids=["mfma_hkv2", "valu_g4"])
def test_selection_per_kv_head(msa, spec):
    c = synth.make_case("per_head", seed=61, **spec)
    print(f"case per_head {spec}", flush=True)
    d = upload(c)
    tk = per_head_topk(c, seeds=range(62, 62 + c.Hkv))
    out = attend(msa, c, d, torch.from_numpy(tk).cuda())
    check_attention(out, oracle_attention(c, tk))


def test_selection_per_kv_head_full_size_sampled(msa):
    """The launch configuration of the timed 2-KV-head variant: 16 rows x 4
    tokens at 16384 context, 32 query / 2 KV heads, one random selection of 16
    visible blocks per KV head (128 token-head units: 2 splits of 8 pages per
    token), checked against the oracle on 16 sampled tokens."""
    c = synth.make_case("per_head_full", R=16, T=4, Hq=32, Hkv=2, D=128, Di=128,
                        seq_lens=[16384] * 16, P=4096, k=16, seed=63)
    print("case per_head_full", flush=True)
    d = upload(c)
    tk = per_head_topk(c, seeds=range(64, 64 + c.Hkv))
    out = attend(msa, c, d, torch.from_numpy(tk).cuda())
    ref = oracle_attention(c, tk, n_range=(0, 8))
    ref[56:64] = oracle_attention(c, tk, n_range=(56, 64))[56:64]
    check_attention(out, ref, rows=list(range(8)) + list(range(56, 64)))


def test_selection_per_kv_head_identical_heads_equal_shared(msa):
    """[Hkv, N, k] holding the same selection for every KV head gives the
    shared-selection result bit for bit (also through non-contiguous views)."""
    c = synth.make_case("per_head_same", R=2, T=4, Hq=32, Hkv=2, D=128, Di=128,
                        seq_lens=[1000, 1800], P=30, k=6, seed=63)
    d = upload(c)
    tk = synth.random_topk(c, seed=64).cuda()
    shared = attend(msa, c, d, tk)
    stacked = tk.unsqueeze(0).expand(c.Hkv, -1, -1)          # KV-head stride 0
    per_head = attend(msa, c, d, stacked)
    copied = attend(msa, c, d, stacked.contiguous())
    assert torch.equal(shared.view(torch.int16), per_head.view(torch.int16))
    assert torch.equal(shared.view(torch.int16), copied.view(torch.int16))


BF16_KV = [
    # MFMA path (bf16 queries, 16 query heads per KV head)
    dict(R=2, T=4, Hq=16, Hkv=1, D=128, Di=128, seq_lens=[900, 1700], P=25, k=5, qbf16=True),
    dict(R=3, T=4, Hq=16, Hkv=1, D=64, Di=64, seq_lens=[129, 2000, 3333], P=50, k=9, qbf16=True),
    dict(R=2, T=4, Hq=32, Hkv=2, D=128, Di=128, seq_lens=[1000, 4000], P=45, k=16, qbf16=True),
    dict(R=1, T=4, Hq=16, Hkv=1, D=128, Di=128, seq_lens=[16000], P=130, k=40, qbf16=True),
    dict(R=1, T=4, Hq=16, Hkv=1, D=128, Di=128, seq_lens=[40000], P=318, k=300, qbf16=True),
    # vector path (f32 queries, 4 query heads per KV head)
    dict(R=2, T=3, Hq=8, Hkv=2, D=64, Di=64, seq_lens=[600, 1300], P=20, k=4, qbf16=False),
]


def bf16_case(spec, seed):
    spec = dict(spec)
    qbf16 = spec.pop("qbf16")
    c = synth.make_case("bf16kv", fp8=False, seed=seed, **spec)
    c.k_cache = c.k_cache.to(torch.bfloat16)
    c.v_cache = c.v_cache.to(torch.bfloat16)
    if qbf16:
        c.q = c.q.to(torch.bfloat16)
    return c


@pytest.mark.parametrize("spec", BF16_KV, ids=["d128", "d64_ragged", "hkv2_k16", "k40_16k", "k300_313blocks",
                                               "valu_f32q"])
def test_bf16_kv_cache(msa, spec):
    c = bf16_case(spec, seed=65)
    print(f"case bf16kv {spec}", flush=True)
    d = upload(c)
    tk = synth.random_topk(c, seed=66)
    out = attend(msa, c, d, tk.cuda(), out_dtype=torch.bfloat16)
    check_attention(out, oracle_attention(c, tk.numpy()))
    # per-KV-head selection on the bf16 cache as well
    if c.Hkv > 1:
        tk3 = per_head_topk(c, seeds=range(67, 67 + c.Hkv))
        out = attend(msa, c, d, torch.from_numpy(tk3).cuda(), out_dtype=torch.bfloat16)
        check_attention(out, oracle_attention(c, tk3))


def test_bf16_kv_cache_select_path(msa):
    """msa_select_sparse_decode on a bf16 cache (selection inside the attention
    launch): its selection is the oracle's on the same sheet and its output
    equals msa_sparse_decode's over that selection, bit for bit."""
    import oracle
    c = bf16_case(dict(R=2, T=4, Hq=16, Hkv=1, D=128, Di=128, seq_lens=[3000, 1500], P=40, k=8,
                       qbf16=True), seed=69)
    d = upload(c)
    sheet = np.random.default_rng(70).standard_normal((c.N, c.MB)).astype(np.float32)
    scores = torch.from_numpy(sheet).cuda()
    tk = poisoned((c.N, c.k), torch.int32)
    out = poisoned((c.N, c.Hq, c.D), torch.bfloat16)
    ws = workspace(msa, c, c.k)
    msa.msa_select_sparse_decode(scores, c.k, tk, d.q, d.k_cache, d.v_cache, d.block_table,
                                 d.seq_lens, c.T, out, c.sm_scale, c.k_scale, c.v_scale, c.B, ws)
    torch.cuda.synchronize()
    gt = tk.cpu().numpy()
    assert np.array_equal(gt, oracle.select_topk(sheet.astype(np.float64), c.k))
    out2 = attend(msa, c, d, tk)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    check_attention(out, oracle_attention(c, gt))


def test_per_head_selection_shape_is_checked(msa):
    c = synth.make_case("per_head_bad", R=1, T=2, Hq=32, Hkv=2, D=128, Di=128, seq_lens=[600],
                        P=10, k=3, seed=68)
    d = upload(c)
    bad = torch.zeros((3, c.N, c.k), dtype=torch.int32, device="cuda")     # 3 != Hkv
    out = poisoned((c.N, c.Hq, c.D), torch.bfloat16)
    with pytest.raises(msa.MsaError, match="sizes disagree"):
        msa.msa_sparse_decode(d.q, d.k_cache, d.v_cache, d.block_table, d.seq_lens, bad, c.T, out,
                              c.sm_scale, c.k_scale, c.v_scale, c.B, workspace(msa, c, c.k))
    # the selecting calls write one selection for every KV head: [N, k] only
    scores = torch.zeros((c.N, c.MB), dtype=torch.float32, device="cuda")
    tk3 = torch.zeros((c.Hkv, c.N, c.k), dtype=torch.int32, device="cuda")
    with pytest.raises(msa.MsaError):
        msa.msa_select_sparse_decode(scores, c.k, tk3, d.q, d.k_cache, d.v_cache, d.block_table,
                                     d.seq_lens, c.T, out, c.sm_scale, c.k_scale, c.v_scale, c.B,
                                     workspace(msa, c, c.k))


# ---- one selection per request, shared by its tokens (per-request sheet)

PER_ROW = [
    # MFMA decode score + MFMA attention (bf16 queries, FP8, 16 query heads per KV head)
    dict(R=3, T=4, Hq=16, Hkv=1, D=128, Di=128, seq_lens=[900, 3000, 129], P=40, k=6),
    # vector score (f32 index queries, 3 tokens) + vector attention, Di = D = 64
    dict(R=2, T=3, Hq=8, Hkv=2, D=64, Di=64, seq_lens=[700, 1500], P=25, k=4, fp8=False),
]


def per_row_case(spec, seed):
    return synth.make_case("per_row", seed=seed, **spec)


@pytest.mark.parametrize("spec", PER_ROW, ids=["mfma", "valu"])
def test_per_request_sheet_selection_attention(msa, spec):
    """msa_block_score into an [R, MB] sheet (one row per request: the max
    over its tokens), msa_select_topk over it, msa_sparse_decode with the
    [R, k] selection shared by each request's tokens (and as [Hkv, R, k])."""
    import oracle
    c = per_row_case(spec, seed=71)
    print(f"case per_row {spec}", flush=True)
    d = upload(c)
    scores = poisoned((c.R, c.MB), torch.float32)
    msa.msa_block_score(d.q_idx, d.index_k, d.block_table, d.seq_lens, c.T, c.B, c.idx_scale, scores)
    tk = poisoned((c.R, c.k), torch.int32)
    msa.msa_select_topk(scores, c.k, tk)
    torch.cuda.synchronize()
    gs, gt = scores.cpu().numpy(), tk.cpu().numpy()
    ref_s = oracle.block_score_per_row(c.q_idx, c.index_k, c.block_table, c.seq_lens, c.T,
                                       c.idx_scale, threads=8)
    check_scores(gs, ref_s)
    assert np.array_equal(gt, oracle.select_topk(gs.astype(np.float64), c.k))
    out = attend(msa, c, d, tk, out_dtype=torch.bfloat16 if c.fp8 else torch.float32)
    check_attention(out, oracle_attention(c, gt))
    if c.Hkv > 1:
        tk3 = np.stack([gt, gt[::-1].copy()])
        out = attend(msa, c, d, torch.from_numpy(tk3).cuda(),
                     out_dtype=torch.bfloat16 if c.fp8 else torch.float32)
        check_attention(out, oracle_attention(c, tk3))


def test_per_request_select_and_step_calls(msa):
    """msa_select_sparse_decode and msa_decode_step with a per-request sheet
    and selection: the selection is the oracle's on the GPU's own sheet, and
    the outputs equal the separate calls' bit for bit."""
    import oracle
    c = per_row_case(PER_ROW[0], seed=72)
    d = upload(c)
    ws = workspace(msa, c, c.k)
    scores = poisoned((c.R, c.MB), torch.float32)
    tk = poisoned((c.R, c.k), torch.int32)
    out = poisoned((c.N, c.Hq, c.D), torch.bfloat16)
    msa.msa_decode_step(d.q_idx, d.index_k, d.q, d.k_cache, d.v_cache, d.block_table, d.seq_lens,
                        c.T, c.k, c.B, c.idx_scale, c.sm_scale, c.k_scale, c.v_scale, scores, tk,
                        out, ws)
    torch.cuda.synchronize()
    gs, gt = scores.cpu().numpy(), tk.cpu().numpy()
    ref_s = oracle.block_score_per_row(c.q_idx, c.index_k, c.block_table, c.seq_lens, c.T,
                                       c.idx_scale, threads=8)
    check_scores(gs, ref_s)
    assert np.array_equal(gt, oracle.select_topk(gs.astype(np.float64), c.k))
    check_attention(out, oracle_attention(c, gt))
    # the two-stage call on the same sheet, and the attention alone
    tk2 = poisoned((c.R, c.k), torch.int32)
    out2 = poisoned((c.N, c.Hq, c.D), torch.bfloat16)
    msa.msa_select_sparse_decode(scores, c.k, tk2, d.q, d.k_cache, d.v_cache, d.block_table,
                                 d.seq_lens, c.T, out2, c.sm_scale, c.k_scale, c.v_scale, c.B, ws)
    out3 = attend(msa, c, d, tk)
    torch.cuda.synchronize()
    assert torch.equal(tk2, tk)
    assert torch.equal(out2.view(torch.int16), out.view(torch.int16))
    assert torch.equal(out3.view(torch.int16), out.view(torch.int16))


def test_per_request_shapes_checked(msa):
    c = per_row_case(PER_ROW[0], seed=73)
    d = upload(c)
    ws = workspace(msa, c, c.k)
    out = poisoned((c.N, c.Hq, c.D), torch.bfloat16)
    # a per-request sheet with a per-token selection (and the reverse) disagree
    with pytest.raises(msa.MsaError, match="sizes disagree"):
        msa.msa_decode_step(d.q_idx, d.index_k, d.q, d.k_cache, d.v_cache, d.block_table,
                            d.seq_lens, c.T, c.k, c.B, c.idx_scale, c.sm_scale, c.k_scale,
                            c.v_scale, poisoned((c.R, c.MB), torch.float32),
                            poisoned((c.N, c.k), torch.int32), out, ws)
    # per-request sheets are served for decode rows (T <= 16) only
    big = synth.make_case("per_row_prefill", R=1, T=40, Hq=16, Hkv=1, D=128, Di=128,
                          seq_lens=[600], P=8, k=2, seed=74)
    db = upload(big)
    with pytest.raises(msa.MsaError, match="size outside"):
        msa.msa_block_score(db.q_idx, db.index_k, db.block_table, db.seq_lens, big.T, big.B,
                            big.idx_scale, poisoned((big.R, big.MB), torch.float32))
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()


SAMPLED = list(range(8)) + list(range(56, 64))   # tokens of rows 0, 1, 14 and 15


def _sampled_ref(c, tk):
    ref = oracle_attention(c, tk, n_range=(0, 8))
    ref[56:64] = oracle_attention(c, tk, n_range=(56, 64))[56:64]
    return ref


def test_bf16_kv_cache_full_size_sampled(msa):
    """The timed dense-bf16 variant: the 16-row, 16384-context decode batch with
    its K/V caches widened exactly to bf16, a random selection of 16 visible
    blocks per token; the oracle of the FP8 batch (same values) on 16 tokens."""
    c = synth.hbm_decode(16)
    print("case bf16kv_full", flush=True)
    d = upload(c)
    kc, vc = d.k_cache.to(torch.bfloat16), d.v_cache.to(torch.bfloat16)
    tk = synth.random_topk(c, seed=81)
    out = poisoned((c.N, c.Hq, c.D), torch.bfloat16)
    msa.msa_sparse_decode(d.q, kc, vc, d.block_table, d.seq_lens, tk.cuda(), c.T, out, c.sm_scale,
                          c.k_scale, c.v_scale, c.B, workspace(msa, c, c.k))
    torch.cuda.synchronize()
    check_attention(out, _sampled_ref(c, tk.numpy()), rows=SAMPLED)


def test_per_request_full_size_sampled(msa):
    """The timed per-request variant: the 16-row, 16384-context decode batch,
    its [16, 128] per-request sheet, top-16 per request, attention with the
    selection shared by each request's 4 tokens; oracle on 16 tokens."""
    import oracle
    c = synth.hbm_decode(16)
    print("case per_request_full", flush=True)
    d = upload(c)
    scores = poisoned((c.R, c.MB), torch.float32)
    msa.msa_block_score(d.q_idx, d.index_k, d.block_table, d.seq_lens, c.T, c.B, c.idx_scale, scores)
    tk = poisoned((c.R, c.k), torch.int32)
    msa.msa_select_topk(scores, c.k, tk)
    out = poisoned((c.N, c.Hq, c.D), torch.bfloat16)
    msa.msa_sparse_decode(d.q, d.k_cache, d.v_cache, d.block_table, d.seq_lens, tk, c.T, out, c.sm_scale,
                          c.k_scale, c.v_scale, c.B, workspace(msa, c, c.k))
    torch.cuda.synchronize()
    gs, gt = scores.cpu().numpy(), tk.cpu().numpy()
    assert np.array_equal(gt, oracle.select_topk(gs.astype(np.float64), c.k))
    check_attention(out, _sampled_ref(c, gt), rows=SAMPLED)
