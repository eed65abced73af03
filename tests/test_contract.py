"""GPU contract of the write-into-output ABI (Cacheon "Kernel ABI", "Core
rules" and "Graph behavior"; "Slot contract", "CUDA graph contract"):
every logical output cell is written, strided outputs are honoured, inputs are
left unchanged, results replay correctly from a captured HIP graph after the
inputs are rewritten in place, and two runs give identical bits."""
import numpy as np
import pytest
import torch

import synth
from msa_harness import (check_attention, check_scores, check_topk_end_to_end,
                         check_topk_isolated, oracle_attention, oracle_scores, poisoned,
                         run_attend, run_score, run_select, upload, workspace)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def msa():
    import block_sparse_paged_amd as m
    return m


def _inputs(d):
    return [t for t in (d.q_idx, d.index_k, d.block_table, d.seq_lens, d.q, d.k_cache, d.v_cache)
            if t is not None]


def test_inputs_unchanged_and_all_cells_written(msa):
    c = synth.bucket_sweep(4, seed=3201, pad_rows=(1,))
    d = upload(c)
    before = [t.clone() for t in _inputs(d)]
    scores = run_score(msa, c, d)
    topk = run_select(msa, c, scores)
    out = run_attend(msa, c, d, topk)
    torch.cuda.synchronize()
    for a, b in zip(before, _inputs(d)):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), "an input was written"
    assert not torch.isnan(scores).any()
    assert (topk != -7777).all()
    assert not torch.isnan(out.float()).any()


def test_strided_outputs(msa):
    c = synth.small_fp8(R=2, T=4, lens=(900, 1700), k=5, seed=61)
    d = upload(c)
    # score sheet as a transposed view of a padded buffer
    sbuf = torch.full((c.MB + 3, c.N + 5), float("nan"), device="cuda")
    scores = sbuf[:c.MB, :c.N].t()
    run_score(msa, c, d, scores=scores)
    # topk as a column-major view
    tbuf = torch.full((c.k, c.N), -7777, dtype=torch.int32, device="cuda")
    topk = tbuf.t()
    run_select(msa, c, scores, topk=topk)
    # output with heads outermost and a padded d stride
    obuf = torch.full((c.Hq, c.N, c.D * 2), float("nan"), dtype=torch.bfloat16, device="cuda")
    out = obuf[:, :, ::2].permute(1, 0, 2)
    run_attend(msa, c, d, topk, out=out)
    torch.cuda.synchronize()
    assert torch.isnan(sbuf[c.MB:]).all() and torch.isnan(sbuf[:, c.N:]).all()
    assert torch.isnan(obuf[:, :, 1::2].float()).all(), "wrote outside the logical cells"
    gs = scores.cpu().numpy()
    ref = oracle_scores(c)
    check_scores(gs, ref)
    check_topk_isolated(topk.cpu().numpy(), gs)
    check_attention(out, oracle_attention(c, topk.cpu().numpy()))
    # contiguous run gives the same bits
    d2 = upload(c)
    s2 = run_score(msa, c, d2)
    t2 = run_select(msa, c, s2)
    o2 = run_attend(msa, c, d2, t2)
    torch.cuda.synchronize()
    assert torch.equal(s2, scores) and torch.equal(t2, topk)
    assert torch.equal(o2.view(torch.int16), out.contiguous().view(torch.int16))


def test_run_to_run_bitwise_identical(msa):
    c = synth.hbm_decode(16)
    d = upload(c)
    res = []
    for _ in range(2):
        s = run_score(msa, c, d)
        t = run_select(msa, c, s)
        o = run_attend(msa, c, d, t)
        torch.cuda.synchronize()
        res.append((s.clone(), t.clone(), o.clone()))
    assert torch.equal(res[0][0], res[1][0])
    assert torch.equal(res[0][1], res[1][1])
    assert torch.equal(res[0][2].view(torch.int16), res[1][2].view(torch.int16))


def test_graph_replay_with_rewritten_inputs(msa):
    """Capture the three calls once; rewrite every dynamic input in place with a
    new seed before each replay; every replay must match a fresh oracle."""
    shape = dict(R=2, T=4, lens=(1100, 1900), k=5)
    c0 = synth.small_fp8(seed=71, P=40, **shape)
    d = upload(c0)
    scores = poisoned((c0.N, c0.MB), torch.float32)
    topk = poisoned((c0.N, c0.k), torch.int32)
    out = poisoned((c0.N, c0.Hq, c0.D), torch.bfloat16)
    ws = workspace(msa, c0, c0.k)
    # scales are captured by value, so all seeds below share c0's scalars
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        msa.msa_block_score(d.q_idx, d.index_k, d.block_table, d.seq_lens, c0.T, c0.B,
                            c0.idx_scale, scores)
        msa.msa_select_topk(scores, c0.k, topk)
        msa.msa_sparse_decode(d.q, d.k_cache, d.v_cache, d.block_table, d.seq_lens, topk, c0.T,
                              out, c0.sm_scale, c0.k_scale, c0.v_scale, c0.B, ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        msa.msa_block_score(d.q_idx, d.index_k, d.block_table, d.seq_lens, c0.T, c0.B,
                            c0.idx_scale, scores)
        msa.msa_select_topk(scores, c0.k, topk)
        msa.msa_sparse_decode(d.q, d.k_cache, d.v_cache, d.block_table, d.seq_lens, topk, c0.T,
                              out, c0.sm_scale, c0.k_scale, c0.v_scale, c0.B, ws)
    torch.cuda.synchronize()
    for seed in (72, 73, 74):
        c = synth.small_fp8(seed=seed, P=40, **shape)
        for name in ("idx_scale", "k_scale", "v_scale", "sm_scale"):
            setattr(c, name, getattr(c0, name))
        nd = upload(c)
        for dst, src in zip(_inputs(d), _inputs(nd)):
            dst.copy_(src)
        scores.fill_(float("nan"))
        topk.fill_(-7777)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        gs, gt = scores.cpu().numpy(), topk.cpu().numpy()
        ref = oracle_scores(c)
        check_scores(gs, ref)
        check_topk_isolated(gt, gs)
        check_topk_end_to_end(gt, ref)
        check_attention(out, oracle_attention(c, gt))


def test_bad_page_ids_do_not_fault(msa):
    """Out-of-range physical page ids in the block table: the score sheet marks
    the block NaN (never selected) and attention skips it."""
    c = synth.small_fp8(R=2, T=4, lens=(900, 700), k=3, seed=81)
    bt = c.block_table.clone()
    bt[0, 2] = c.P + 1000
    bt[1, 1] = -5
    c.block_table = bt
    d = upload(c)
    scores = run_score(msa, c, d)
    topk = run_select(msa, c, scores)
    tk_all = torch.arange(c.MB, dtype=torch.int32, device="cuda").repeat(c.N, 1)
    out = run_attend(msa, c, d, tk_all[:, :c.MB])
    torch.cuda.synchronize()
    gs = scores.cpu().numpy()
    assert np.isnan(gs[0:4, 2]).all() and np.isnan(gs[4:8, 1]).all()
    gt = topk.cpu().numpy()
    assert not (gt[0:4] == 2).any() and not (gt[4:8] == 1).any()
    assert not torch.isnan(out.float()).any()


def test_rejected_call_leaves_poison(msa):
    c = synth.small_fp8(R=1, T=4, lens=(500,), k=2, seed=91)
    d = upload(c)
    scores = poisoned((c.N, c.MB), torch.float32)
    with pytest.raises(msa.MsaError):
        msa.msa_block_score(d.q_idx, d.index_k, d.block_table, d.seq_lens, c.T, 64, c.idx_scale,
                            scores)
    topk = poisoned((c.N, c.k), torch.int32)
    with pytest.raises(msa.MsaError):
        msa.msa_select_topk(scores, c.MB + 1, poisoned((c.N, c.MB + 1), torch.int32))
    out = poisoned((c.N, c.Hq, c.D), torch.bfloat16)
    small_ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(msa.MsaError):
        msa.msa_sparse_decode(d.q, d.k_cache, d.v_cache, d.block_table, d.seq_lens, topk, c.T,
                              out, c.sm_scale, c.k_scale, c.v_scale, c.B, small_ws)
    torch.cuda.synchronize()
    assert torch.isnan(scores).all() and torch.isnan(out.float()).all()


def test_workspace_counters_left_zero(msa):
    """The split-merge arrival counters (N*Hkv int32 256 bytes apart at the start
    of the workspace) are zero again after every call, so a workspace can be
    reused without clearing."""
    for k in (16, 5, 128):
        c = synth.small_fp8(R=2, T=4, lens=(3000, 16384), k=min(k, 24), seed=95, P=200)
        d = upload(c)
        tk = synth.random_topk(c, seed=96).cuda()
        ws = workspace(msa, c, tk.shape[1])
        for _ in range(3):
            run_attend(msa, c, d, tk, ws=ws)
        torch.cuda.synchronize()
        ctr = ws[: c.N * c.Hkv * 256].view(torch.int32)
        assert (ctr == 0).all()
