"""GPU tests of msa_decode_step (the whole step in one call) and
msa_select_sparse_decode (stages 2 + 3): their scores, topk_idx and out must be
bit-identical to msa_block_score -> msa_select_topk -> msa_sparse_decode
(selection inside the attention launch and the separate top-k launch alike),
match the oracle, leave the workspace counters zeroed, and replay from a graph
with rewritten inputs."""
import sys

import numpy as np
import pytest
import torch

import synth
from msa_harness import (check_attention, check_scores, check_topk_end_to_end, check_topk_isolated,
                         oracle_attention, oracle_scores, poisoned, run_attend, run_score,
                         run_select, upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def msa():
    import block_sparse_paged_amd as m
    return m


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def step_ws(msa, c):
    n = msa.msa_decode_step_workspace_bytes(c.R, c.T, c.Hq, c.Hkv, c.D, c.k)
    return torch.zeros(n, dtype=torch.uint8, device="cuda")


def control_zero(ws, c):
    """The part that must be zero between calls: the split-arrival counters at
    the start of the workspace (one int32 per token and KV head, 256 bytes apart); the split
    partials after them hold scratch data."""
    return bool((ws[:c.N * c.Hkv * 256] == 0).all())


def run_step(msa, c, d, ws=None, out_dtype=None):
    out_dtype = out_dtype or (torch.bfloat16 if c.fp8 else torch.float32)
    scores = poisoned((c.N, c.MB), torch.float32)
    topk = poisoned((c.N, c.k), torch.int32)
    out = poisoned((c.N, c.Hq, c.D), out_dtype)
    ws = step_ws(msa, c) if ws is None else ws
    msa.msa_decode_step(d.q_idx, d.index_k, d.q, d.k_cache, d.v_cache, d.block_table, d.seq_lens,
                        c.T, c.k, c.B, c.idx_scale, c.sm_scale, c.k_scale, c.v_scale, scores, topk,
                        out, ws)
    return scores, topk, out, ws


def three_calls(msa, c, d, out_dtype=None):
    s = run_score(msa, c, d)
    t = run_select(msa, c, s)
    o = run_attend(msa, c, d, t, out_dtype=out_dtype)
    return s, t, o


def same_bits(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a, b)


CASES = {
    "decode_r4_16k": lambda: synth.decode_bucket4(),
    "sweep_r16": lambda: synth.bucket_sweep(16),
    "sweep_r8_pad": lambda: synth.bucket_sweep(8, seed=3100, pad_rows=(2, 7)),
    "sweep_r1": lambda: synth.bucket_sweep(1),
    "hbm_k8": lambda: synth.hbm_decode(8),
    "hbm_k16": lambda: synth.hbm_decode(16),
    "hbm_k32": lambda: synth.hbm_decode(32),
    "hbm_k128": lambda: synth.hbm_decode(128),
    "small_t1": lambda: synth.small_fp8(R=3, T=1, lens=(129, 5000, 1), k=8),
    "small_t5": lambda: synth.small_fp8(R=2, T=5, lens=(1000, 2100), k=6),
    "small_d64": lambda: synth.small_fp8(R=2, T=4, lens=(700, 1500), k=4, D=64, Di=64),
    "fallback_tiny_fp32": lambda: synth.tiny(),
    "fallback_t40": lambda: synth.small_fp8(R=2, T=40, lens=(300, 1700), k=4),
    # 313 blocks (MB > 128): the step selects with the top-k launch before the attention
    "mb313_k300": lambda: synth.small_fp8(R=1, T=4, lens=(40000,), k=300),
    "mb160_k16": lambda: synth.small_fp8(R=3, T=4, lens=(20480, 700, 19000), k=16, seed=17),
}


@pytest.mark.parametrize("name", list(CASES))
def test_step_bit_identical_to_three_calls(msa, name):
    c = CASES[name]()
    _say(f"case {name}")
    d = upload(c)
    s1, t1, o1 = three_calls(msa, c, d)
    s2, t2, o2, ws = run_step(msa, c, d)
    torch.cuda.synchronize()
    assert same_bits(s1, s2), "scores differ"
    assert same_bits(t1, t2), "topk differs"
    assert same_bits(o1, o2), "attention output differs"
    assert control_zero(ws, c), "workspace counters not left zeroed"
    # stages 2 + 3 from the same score sheet
    t3 = poisoned((c.N, c.k), torch.int32)
    o3 = poisoned(tuple(o1.shape), o1.dtype)
    ws3 = step_ws(msa, c)
    msa.msa_select_sparse_decode(s1, c.k, t3, d.q, d.k_cache, d.v_cache, d.block_table, d.seq_lens,
                                 c.T, o3, c.sm_scale, c.k_scale, c.v_scale, c.B, ws3)
    torch.cuda.synchronize()
    assert same_bits(t1, t3), "select_sparse_decode topk differs"
    assert same_bits(o1, o3), "select_sparse_decode output differs"
    assert control_zero(ws3, c)


def test_step_matches_oracle(msa):
    c = synth.hbm_decode(16, seed=5901)
    _say("case hbm_k16 seed 5901 vs oracle")
    d = upload(c)
    s, t, o, ws = run_step(msa, c, d)
    torch.cuda.synchronize()
    gs, gt = s.cpu().numpy(), t.cpu().numpy()
    ref = oracle_scores(c, threads=16)
    check_scores(gs, ref)
    check_topk_isolated(gt, gs)
    check_topk_end_to_end(gt, ref)
    check_attention(o, oracle_attention(c, gt, threads=16))


GRAPH_SHAPES = {
    # the per-token attention kernel (selection and split merge in its launch)
    "token_k16": dict(R=4, T=4, lens=(3000, 16384, 9000, 128), k=16, P=300),
    # the row-level attention kernel and the split merge launch (k = all blocks)
    "row_k128": dict(R=4, T=4, lens=(9000, 16384, 8300, 128), k=128, P=300),
}


@pytest.mark.parametrize("name", list(GRAPH_SHAPES))
def test_step_repeated_and_graph_replay(msa, name):
    shape = GRAPH_SHAPES[name]
    _say(f"case graph replay {name}")
    c0 = synth.small_fp8(seed=111, **shape)
    d = upload(c0)
    scores = poisoned((c0.N, c0.MB), torch.float32)
    topk = poisoned((c0.N, c0.k), torch.int32)
    out = poisoned((c0.N, c0.Hq, c0.D), torch.bfloat16)
    ws = step_ws(msa, c0)

    def call():
        msa.msa_decode_step(d.q_idx, d.index_k, d.q, d.k_cache, d.v_cache, d.block_table,
                            d.seq_lens, c0.T, c0.k, c0.B, c0.idx_scale, c0.sm_scale, c0.k_scale,
                            c0.v_scale, scores, topk, out, ws)

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for _ in range(5):
            call()
    torch.cuda.synchronize()
    ref = [x.clone() for x in (scores, topk, out)]
    assert control_zero(ws, c0)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        call()
    torch.cuda.synchronize()
    for seed in (112, 113):
        c = synth.small_fp8(seed=seed, **shape)
        for name in ("idx_scale", "k_scale", "v_scale", "sm_scale"):
            setattr(c, name, getattr(c0, name))
        nd = upload(c)
        for dst, src in zip((d.q_idx, d.index_k, d.block_table, d.seq_lens, d.q, d.k_cache, d.v_cache),
                            (nd.q_idx, nd.index_k, nd.block_table, nd.seq_lens, nd.q, nd.k_cache, nd.v_cache)):
            dst.copy_(src)
        scores.fill_(float("nan"))
        topk.fill_(-7777)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert control_zero(ws, c0)
        s1, t1, o1 = three_calls(msa, c, nd)
        torch.cuda.synchronize()
        assert same_bits(s1, scores) and same_bits(t1, topk) and same_bits(o1, out)
        gs, gt = scores.cpu().numpy(), topk.cpu().numpy()
        check_scores(gs, oracle_scores(c))
        check_topk_isolated(gt, gs)
        check_attention(out, oracle_attention(c, gt))
    # the inputs of the first capture still give the first results
    for dst, src in zip((d.q_idx, d.index_k, d.block_table, d.seq_lens, d.q, d.k_cache, d.v_cache),
                        (upload(c0).q_idx, upload(c0).index_k, upload(c0).block_table,
                         upload(c0).seq_lens, upload(c0).q, upload(c0).k_cache, upload(c0).v_cache)):
        dst.copy_(src)
    g.replay()
    torch.cuda.synchronize()
    assert all(same_bits(a, b) for a, b in zip(ref, (scores, topk, out)))
