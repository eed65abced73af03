"""GPU parity: the HIP library against the CPU oracle on seeded workloads.

Covers the five workload families at full size (tiny fp32; 4-row decode
bucket at 16K; the 1/4/8/16-row bucket sweep with ragged lengths and padded
rows; the 4 x 2048-token prefill score -> select; the 16-row 16K HBM-bound
decode with k in {8, 16, 32, 128}) plus small cases that exercise ragged
tails, token groups, head dims, index dims, shared pages and the vector-ALU
paths.  The 16-row config runs in the same launch configuration as the bench.
"""
import sys

import numpy as np
import pytest
import torch

import synth
from msa_harness import (check_attention, check_scores, check_topk_end_to_end,
                         check_topk_isolated, full_step_parity, oracle_attention, oracle_scores,
                         run_attend, run_score, run_select, upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def msa():
    import block_sparse_paged_amd as m
    return m


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_tiny_fp32(msa):
    c = synth.tiny()
    _say(f"case {c.name}")
    res = full_step_parity(msa, c)
    _say(str(res))


def test_decode_bucket4(msa):
    c = synth.decode_bucket4()
    _say(f"case {c.name}")
    _say(str(full_step_parity(msa, c)))


@pytest.mark.parametrize("R", [1, 4, 8, 16])
def test_bucket_sweep(msa, R):
    c = synth.bucket_sweep(R)
    _say(f"case {c.name} lens={c.seq_lens.tolist()}")
    _say(str(full_step_parity(msa, c)))


def test_bucket_sweep_padded_rows(msa):
    c = synth.bucket_sweep(8, seed=3100, pad_rows=(2, 7))
    _say(f"case {c.name}+pad lens={c.seq_lens.tolist()}")
    d = upload(c)
    scores = run_score(msa, c, d)
    topk = run_select(msa, c, scores)
    out = run_attend(msa, c, d, topk)
    torch.cuda.synchronize()
    gs, gt, go = scores.cpu().numpy(), topk.cpu().numpy(), out.float().cpu().numpy()
    for r in (2, 7):
        rows = slice(r * c.T, (r + 1) * c.T)
        assert np.isneginf(gs[rows]).all()
        assert (gt[rows] == -1).all()
        assert (go[rows] == 0).all()
    ref = oracle_scores(c)
    check_scores(gs, ref)
    check_topk_isolated(gt, gs)
    check_topk_end_to_end(gt, ref)
    check_attention(out, oracle_attention(c, gt))


def test_prefill_score_select(msa):
    c = synth.prefill()
    _say(f"case {c.name}")
    d = upload(c)
    scores = run_score(msa, c, d)
    topk = run_select(msa, c, scores)
    torch.cuda.synchronize()
    gs, gt = scores.cpu().numpy(), topk.cpu().numpy()
    assert gt.shape == (8192, 16)
    check_topk_isolated(gt, gs)              # whole sheet, bit-exact
    # the oracle's whole [8192, 80] sheet (about 15 s on 16 host threads)
    ref = oracle_scores(c, threads=16)
    check_scores(gs, ref)
    check_topk_end_to_end(gt, ref)


def test_prefill_noncausal_reading(msa):
    """The other reading of the prefill key set: every query token sees exactly
    the 8192-token context, no causal mask.  It fits the same calls as one row
    per query token (R = 8192, T = 1, seq_len 8192), each row carrying its
    request's block table; scores and selection are checked on sampled rows."""
    import dataclasses
    base = synth.prefill()
    R0, T0 = base.R, base.T
    MB = 8192 // base.B
    bt = base.block_table[:, :MB].repeat_interleave(T0, dim=0).contiguous()      # [8192, 64]
    c = dataclasses.replace(base, name="prefill_noncausal", R=R0 * T0, T=1, MB=MB, block_table=bt,
                            seq_lens=torch.full((R0 * T0,), 8192, dtype=torch.int32))
    _say(f"case {c.name}")
    d = upload(c)
    scores = run_score(msa, c, d)
    topk = run_select(msa, c, scores)
    torch.cuda.synchronize()
    gs, gt = scores.cpu().numpy(), topk.cpu().numpy()
    check_topk_isolated(gt, gs)
    rows = sorted(set(list(range(0, 40)) + list(range(2040, 2060)) + list(range(8150, 8192))))
    ref = np.full_like(gs, np.nan, dtype=np.float64)
    for a, b in ((0, 40), (2040, 2060), (8150, 8192)):
        ref[a:b] = oracle_scores(c, n_range=(a, b), threads=16)[a:b]
    check_scores(gs, ref, rows=rows)
    check_topk_end_to_end(gt, np.where(np.isnan(ref), -np.inf, ref), rows=rows)


@pytest.mark.parametrize("k", [8, 16, 32, 128])
def test_hbm_decode(msa, k):
    c = synth.hbm_decode(k)
    _say(f"case {c.name}")
    _say(str(full_step_parity(msa, c, threads=16)))


def test_hbm_decode_all_blocks_is_dense(msa):
    import oracle
    c = synth.hbm_decode(128)
    _say(f"case {c.name} dense")
    d = upload(c)
    topk = torch.arange(128, dtype=torch.int32, device="cuda").repeat(c.N, 1)
    out = run_attend(msa, c, d, topk)
    torch.cuda.synchronize()
    rows = list(range(0, c.N, 7))
    dense = np.full((c.N, c.Hq, c.D), np.nan)
    for n in rows:
        dense[n:n + 1] = oracle.dense_attention(c.q, c.k_cache, c.v_cache, c.block_table,
                                                c.seq_lens, c.T, c.sm_scale, c.k_scale,
                                                c.v_scale, n_range=(n, n + 1))[n:n + 1]
    check_attention(out, dense, rows=rows)


SMALL = [
    dict(R=2, T=4, lens=(700, 1500), k=4),
    dict(R=3, T=1, lens=(129, 5000, 1), k=8),
    dict(R=2, T=5, lens=(1000, 2100), k=6),          # two token groups per row
    dict(R=1, T=8, lens=(3000,), k=3),
    dict(R=2, T=4, lens=(700, 1500), k=4, D=64, Di=64),
    dict(R=2, T=4, lens=(900, 300), k=4, Di=32),
    dict(R=2, T=2, lens=(2000, 2500), k=5, shared_pages=True, P=40),
    dict(R=2, T=40, lens=(300, 1700), k=4),          # MFMA score path, ragged
    dict(R=1, T=130, lens=(1200,), k=3, D=64, Di=64),
    dict(R=2, T=300, lens=(400, 2000), k=4, D=64, Di=64),   # 8 query tiles per wave
    dict(R=2, T=600, lens=(700, 1900), k=5),        # two 512-token query chunks, ragged
    dict(R=2, T=4, lens=(600, 900), k=4, Hq=32),     # 2 KV heads via Hkv below
    dict(R=4, T=64, lens=(2000, 6000, 600, 9000), k=24),   # 256 tokens: one split, 6 pages per slot
    dict(R=1, T=4, lens=(40000,), k=300),            # 313 blocks: ids past 127, entries past 255
]


@pytest.mark.parametrize("spec", SMALL, ids=[str(i) for i in range(len(SMALL))])
def test_small_fp8(msa, spec):
    spec = dict(spec)
    lens = spec.pop("lens")
    hq = spec.pop("Hq", 16)
    if hq == 32:
        c = synth.make_case("small_hkv2", R=spec["R"], T=spec["T"], Hq=32, Hkv=2, D=128,
                            Di=128, seq_lens=list(lens), P=30, k=spec["k"], seed=21)
    else:
        c = synth.small_fp8(lens=lens, **spec)
    _say(f"case {c.name} {spec} lens={lens}")
    _say(str(full_step_parity(msa, c)))


FP32 = [
    dict(R=2, T=3, Hq=4, Hkv=1, D=64, Di=32, lens=(500, 300), k=2),
    dict(R=1, T=4, Hq=16, Hkv=1, D=128, Di=128, lens=(1000,), k=3),
    dict(R=2, T=2, Hq=8, Hkv=2, D=64, Di=64, lens=(260, 900), k=4),
]


@pytest.mark.parametrize("spec", FP32, ids=[str(i) for i in range(len(FP32))])
def test_small_fp32(msa, spec):
    spec = dict(spec)
    lens = spec.pop("lens")
    nblk = sum((x + 127) // 128 for x in lens)
    c = synth.make_case("small_fp32", seq_lens=list(lens), P=nblk + 3, fp8=False, seed=31, **spec)
    _say(f"case {c.name} {spec}")
    _say(str(full_step_parity(msa, c)))


def test_mixed_precision_variants(msa):
    """bf16 queries with fp32 caches, fp32 queries with FP8 caches, fp32 output."""
    base = synth.small_fp8(R=2, T=4, lens=(700, 1300), k=4, seed=41)
    variants = {
        "f32q_fp8kv": dict(q=base.q.float(), q_idx=base.q_idx.float()),
        "bf16q_f32kv": dict(index_k=base.index_k.view(torch.float8_e4m3fn).float(),
                            k_cache=base.k_cache.view(torch.float8_e4m3fn).float(),
                            v_cache=base.v_cache.view(torch.float8_e4m3fn).float()),
    }
    for name, repl in variants.items():
        c = synth.Case(**{**base.__dict__, **repl})
        c.name = name
        _say(f"case {name}")
        _say(str(full_step_parity(msa, c)))
    c = base
    d = upload(c)
    scores = run_score(msa, c, d)
    topk = run_select(msa, c, scores)
    out = run_attend(msa, c, d, topk, out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_attention(out, oracle_attention(c, topk.cpu().numpy()))


def test_caller_topk_with_gaps(msa):
    """attention on a caller-made selection: -1 holes, out-of-range ids,
    duplicates, blocks past the visible range, and empty rows."""
    c = synth.small_fp8(R=2, T=4, lens=(1000, 600), k=6, seed=51)
    d = upload(c)
    tk = synth.random_topk(c, seed=52).numpy()
    tk[0, 1] = -1
    tk[1, 2] = c.MB + 3
    tk[2, 0] = tk[2, 3]                            # duplicate counts once
    tk[4, 5] = 7                                   # past row 1's visible blocks (0..4)
    tk[5, :] = -1                                  # empty selection
    out = run_attend(msa, c, d, torch.from_numpy(tk).cuda())
    torch.cuda.synchronize()
    clean = tk.copy()
    clean[clean >= c.MB] = -1
    clean[2, 0] = -1
    ref = oracle_attention(c, clean)
    check_attention(out, ref)
    assert (out[5].float().cpu() == 0).all()


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_tokens_that_see_few_keys(msa, kv):
    """Rows of 2, 3 and 5 tokens read by 4 query tokens each (tokens that see
    0 to 5 keys, whose outputs mix a few V rows: any rounding of the softmax
    weights shows in them directly), on the per-token MFMA kernel with FP8 and
    bf16 K/V caches.  Beyond the 2e-3 bound, every output must lie within one
    bf16 step of the oracle's rounded value plus 2^-14 (outputs near zero come
    from cancelling V rows, so their error is absolute): weights carried as a
    single bf16 leave up to |v| * 2^-9 (about 2e-3 here) in such outputs."""
    import oracle
    from msa_harness import bf16_ulp, poisoned, workspace
    c = synth.small_fp8(R=4, T=4, lens=(2, 3, 5, 3000), k=2, seed=6501)
    _say(f"case few keys, kv {kv}: lens {c.seq_lens.tolist()} k={c.k} MB={c.MB}")
    d = upload(c)
    kc, vc = d.k_cache, d.v_cache
    if kv == "bf16":
        kc, vc = kc.to(torch.bfloat16), vc.to(torch.bfloat16)
    tk = synth.random_topk(c, seed=6502)
    out = poisoned((c.N, c.Hq, c.D), torch.bfloat16)
    msa.msa_sparse_decode(d.q, kc, vc, d.block_table, d.seq_lens, tk.cuda(), c.T, out, c.sm_scale,
                          c.k_scale, c.v_scale, c.B, workspace(msa, c, c.k))
    torch.cuda.synchronize()
    ref = oracle_attention(c, tk.numpy())
    check_attention(out, ref)
    g = out.float().cpu().double().numpy()
    rb = oracle.round_bf16(ref)
    excess = np.abs(g - rb) - bf16_ulp(rb)
    worst = np.unravel_index(np.argmax(excess), excess.shape)
    assert (excess <= 2.0 ** -14).all(), (
        f"{int((excess > 2.0 ** -14).sum())} cells off; worst at {worst}: gpu {g[worst]!r} "
        f"oracle {ref[worst]!r} (visible keys {c.visible(worst[0])})")


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_splits_that_cancel(msa, kv):
    """Split partials that cancel.  Every K code is 0, so every logit is 0 and
    a token's output is the plain mean of the V rows of its 16 pages; the
    first 8 pages hold non-negative codes and page 8 + j the rows of page
    (j + 1) % 8 with the sign bit set (keys reversed), so the exact output is
    0 while each split's accumulator (the sum of its two pages' V rows) is
    large.  8 rows of one token each give every token 8 splits of 2 pages, and
    no split holds the negation of another: the partials pass through the
    workspace in their stored form and cancel in the merge, leaving only that
    form's rounding.  Through
    the per-token kernel and the one that selects in-launch, every output must
    be within 2^-14 of 0 (a stored form with an 11-bit mantissa leaves about
    1e-4 here, one with 16 bits about 1e-5)."""
    import dataclasses
    from msa_harness import poisoned, workspace
    c = synth.small_fp8(R=8, T=1, lens=(16 * 128,) * 8, k=16, seed=6701)
    assert c.MB == 16
    bt = c.block_table.numpy()
    kc, vc = c.k_cache.clone(), c.v_cache.clone()
    kc[torch.from_numpy(bt.reshape(-1).astype(np.int64))] = 0
    for r in range(c.R):
        for j in range(8):
            vc[int(bt[r, j])] &= 0x7F
        for j in range(8):
            vc[int(bt[r, j + 8])] = vc[int(bt[r, (j + 1) % 8])].flip(0) | 0x80
    c = dataclasses.replace(c, k_cache=kc, v_cache=vc)
    _say(f"case cancelling splits, kv {kv}: R={c.R} T={c.T} MB={c.MB} k={c.k}")
    tk = torch.arange(c.k, dtype=torch.int32).repeat(c.N, 1)
    ref = oracle_attention(c, tk.numpy())
    assert np.abs(ref).max() == 0.0, "the construction leaves a nonzero exact output"
    d = upload(c)
    kd, vd = d.k_cache, d.v_cache
    if kv == "bf16":
        kd, vd = kd.to(torch.bfloat16), vd.to(torch.bfloat16)
    ws = workspace(msa, c, c.k)
    out = poisoned((c.N, c.Hq, c.D), torch.bfloat16)
    msa.msa_sparse_decode(d.q, kd, vd, d.block_table, d.seq_lens, tk.cuda(), c.T, out, c.sm_scale,
                          c.k_scale, c.v_scale, c.B, ws)
    sheet = torch.from_numpy(np.random.default_rng(6702).standard_normal((c.N, c.MB)).astype(np.float32))
    t = poisoned((c.N, c.k), torch.int32)
    out2 = poisoned((c.N, c.Hq, c.D), torch.bfloat16)
    msa.msa_select_sparse_decode(sheet.cuda(), c.k, t, d.q, kd, vd, d.block_table, d.seq_lens, c.T,
                                 out2, c.sm_scale, c.k_scale, c.v_scale, c.B, ws)
    torch.cuda.synchronize()
    assert torch.equal(t.cpu(), tk), "with k = MB every block is selected, ascending"
    for name, o in (("sparse_decode", out), ("select_sparse_decode", out2)):
        check_attention(o, ref)
        g = o.float().cpu().double().numpy()
        worst = float(np.abs(g).max())
        _say(f"{name}: largest |out| {worst:.3g}")
        assert worst <= 2.0 ** -14, f"{name}: cancelling splits leave {worst:.3g}"


def test_caller_topk_long_selection_with_gaps(msa):
    """Selections of more than 256 entries over more than 128 blocks (the
    token kernel resolves them from tables in LDS): -1 holes, ids >= MB,
    duplicates of earlier entries and blocks past the visible range, all at
    entries past 256 as well."""
    c = synth.small_fp8(R=2, T=2, lens=(40000, 35000), k=300, seed=6601)
    _say(f"case long selection: MB={c.MB} k={c.k}")
    d = upload(c)
    tk = synth.random_topk(c, seed=6602).numpy()
    rng = np.random.default_rng(6603)
    clean = tk.copy()
    for n in range(c.N):
        pos = rng.choice(np.arange(200, c.k), size=12, replace=False)
        tk[n, pos[0]] = -1
        tk[n, pos[1]] = c.MB + 5
        tk[n, pos[2]] = tk[n, pos[3] - 150]                 # repeats an earlier entry
        tk[n, pos[4]] = tk[n, 3]
        tk[n, pos[5]] = c.MB - 1                             # may lie past the visible range
        row = tk[n].copy()
        row[(row >= c.MB) | (row < 0)] = -1
        seen = set()
        for i, j in enumerate(row):
            if j in seen:
                row[i] = -1
            elif j >= 0:
                seen.add(int(j))
        clean[n] = row
    out = run_attend(msa, c, d, torch.from_numpy(tk).cuda())
    torch.cuda.synchronize()
    check_attention(out, oracle_attention(c, clean))
