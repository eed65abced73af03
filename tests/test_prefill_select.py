"""GPU parity of msa_prefill_block_score (Cacheon "Kernel ABI", "Attention block
slots", attention.msa_prefill_block_score: the V2 ragged score-to-selection
call) against the oracle on the same seeded batches.

Grading (the selection bar of the decode path, applied per (head, query-block)
row): the forced blocks (first init_blocks, last local_blocks candidates) must
match exactly; rows whose last selected and first unselected oracle scores are
at least 1e-4 (relative) apart must match exactly; at near-tie rows every
differing id must score within 1e-4 (relative) of the last selected one; mean
overlap >= 0.99.  Every row must be ascending, unique, padded with -1 at the
end, and hold min(topk, candidates) ids; rows no request owns are all -1.
Small batches are checked on every row, the full-size workload on sampled rows
(the oracle computes only those)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from msa_harness import TIE_RTOL, poisoned

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def msa():
    import block_sparse_paged_amd as m
    return m


def upload(pb):
    d = dict(q=pb.q.cuda(), index_k=pb.index_k.view(torch.float8_e4m3fn).cuda(),
             block_table=pb.block_table.cuda())
    for name in ("slot_ids", "cu_seqlens", "seq_lens", "prefix_lens", "cu_seqblocks_q"):
        d[name] = getattr(pb, name).cuda()
    return d


def prefill_workspace(msa, pb):
    n = msa.msa_prefill_block_score_workspace_bytes(pb.batch, pb.Hq, pb.all_qb, pb.MB,
                                                    pb.block_size_q)
    assert n > 0 and n % 256 == 0
    return torch.zeros((n,), dtype=torch.uint8, device="cuda")    # zero-filled once


def run(msa, pb, d, ws=None, out=None):
    if out is None:
        out = poisoned((pb.Hq, pb.all_qb, pb.topk), torch.int32)
    ws = prefill_workspace(msa, pb) if ws is None else ws
    msa.msa_prefill_block_score(d["q"], d["index_k"], d["block_table"], d["slot_ids"],
                                d["cu_seqlens"], d["seq_lens"], d["prefix_lens"], pb.block_size_q,
                                pb.B, pb.topk, pb.init_blocks, pb.local_blocks, pb.scale,
                                d["cu_seqblocks_q"], out, ws)
    torch.cuda.synchronize()
    return out


def reference(pb, rows=None, threads=8):
    return oracle.prefill_select(pb.q, pb.index_k, pb.block_table, pb.slot_ids, pb.cu_seqlens,
                                 pb.seq_lens, pb.prefix_lens, pb.block_size_q, pb.topk,
                                 pb.init_blocks, pb.local_blocks, pb.scale, pb.cu_seqblocks_q,
                                 pb.all_qb, threads=threads, return_scores=True, rows=rows)


def row_owner(pb):
    """[all_qb] request owning each output row (-1: none) and its query block."""
    owner = np.full(pb.all_qb, -1)
    qbl = np.zeros(pb.all_qb, dtype=np.int64)
    cu = pb.cu_seqblocks_q.numpy()
    for b in range(pb.batch):
        owner[cu[b]:cu[b + 1]] = b
        qbl[cu[b]:cu[b + 1]] = np.arange(cu[b + 1] - cu[b])
    return owner, qbl


def check_prefill(pb, gpu, ref, sc, rows=None):
    """Grades the GPU's out_topk against the oracle's on the rows marked in
    ``rows`` (all rows when None).  Returns the number of exact rows."""
    gpu = gpu.cpu().numpy() if torch.is_tensor(gpu) else gpu
    owner, qbl = row_owner(pb)
    rows = np.ones((pb.Hq, pb.all_qb), dtype=bool) if rows is None else rows
    overlaps, exact = [], 0
    for h, g in zip(*np.nonzero(rows)):
        grow, rrow = gpu[h, g], ref[h, g]
        sel = grow[grow >= 0]
        n = len(sel)
        assert (grow[n:] == -1).all(), (h, g, grow)              # -1 only at the end
        assert (np.diff(sel) > 0).all(), (h, g, grow)            # ascending, unique
        if owner[g] < 0:
            assert n == 0, (h, g, grow)
            continue
        b = owner[g]
        V = min(int(pb.seq_lens[b]), int(pb.prefix_lens[b]) + int(qbl[g]) * pb.block_size_q)
        ncand = -(-V // pb.B)
        assert n == min(pb.topk, ncand), (h, g, n, ncand)
        assert sel.size == 0 or sel.max() < ncand
        G, R = set(sel.tolist()), set(rrow[rrow >= 0].tolist())
        if G == R:
            exact += 1
            overlaps.append(1.0)
            continue
        forced = {j for j in range(ncand) if j < pb.init_blocks or j >= ncand - pb.local_blocks}
        assert G & forced == R & forced, (h, g, sorted(G), sorted(R))
        s = sc[h, g]
        rn = [j for j in R if j not in forced]
        tau = min(s[j] for j in rn)
        # near ties relative to the scores involved, as for decode rows
        for j in G ^ R:
            assert abs(s[j] - tau) <= TIE_RTOL * max(abs(tau), abs(s[j])), (h, g, j, s[j], tau)
        overlaps.append(len(G & R) / len(R))
    if overlaps:
        assert np.mean(overlaps) >= 0.99
    return exact


SMALL = [
    # all heads x whole query blocks per chunk (bsq*Hq <= 512), partial last
    # query blocks, a request with no prefix (its first query block sees no key)
    dict(name="hq4_bsq64", new_tokens=[130, 64, 1, 700], prefix=[300, 0, 5000, 2047], Hq=4,
         Di=128, block_size_q=64, topk=4, init_blocks=1, local_blocks=2, extra_qb_rows=3),
    # head groups (bsq*Hq > 512 >= bsq), an odd head count
    dict(name="hq5_bsq256", new_tokens=[600, 300], prefix=[900, 2500], Hq=5, Di=128,
         block_size_q=256, topk=6, init_blocks=0, local_blocks=1),
    # query blocks longer than a chunk: parts, one of them empty
    dict(name="hq2_bsq1024", new_tokens=[1500, 300], prefix=[1000, 3333], Hq=2, Di=64,
         block_size_q=1024, topk=5, init_blocks=2, local_blocks=0),
    # one-token query blocks: 128 query blocks per chunk
    dict(name="hq4_bsq1", new_tokens=[150, 37], prefix=[1200, 130], Hq=4, Di=128,
         block_size_q=1, topk=3, init_blocks=0, local_blocks=0),
    # Di = 64, three heads, small query blocks
    dict(name="hq3_bsq16_d64", new_tokens=[90, 250, 17], prefix=[129, 640, 3000], Hq=3, Di=64,
         block_size_q=16, topk=7, init_blocks=1, local_blocks=1),
    # forced blocks outnumber topk; topk above the candidates of short rows
    dict(name="forced_gt_topk", new_tokens=[200, 70], prefix=[1500, 260], Hq=2, Di=128,
         block_size_q=32, topk=3, init_blocks=2, local_blocks=3),
    dict(name="topk_gt_cand", new_tokens=[100, 64], prefix=[200, 700], Hq=4, Di=128,
         block_size_q=64, topk=20, init_blocks=1, local_blocks=1),
    # a request without new tokens between two others
    dict(name="empty_request", new_tokens=[96, 0, 40], prefix=[400, 1000, 260], Hq=4, Di=128,
         block_size_q=32, topk=4, init_blocks=1, local_blocks=1, extra_qb_rows=1),
    # many requests (the plan's scans over several chunks per request)
    dict(name="batch40", new_tokens=[(37 * i) % 120 + 1 for i in range(40)],
         prefix=[(613 * i) % 1500 for i in range(40)], Hq=2, Di=128, block_size_q=64, topk=8,
         init_blocks=1, local_blocks=2),
    # more than 256 blocks: a wider selection row
    dict(name="mb320", new_tokens=[20, 70], prefix=[40700, 9000], Hq=2, Di=128,
         block_size_q=64, topk=16, init_blocks=1, local_blocks=2),
]


@pytest.mark.parametrize("i", range(len(SMALL)), ids=[s["name"] for s in SMALL])
def test_prefill_select_small(msa, i):
    spec = dict(SMALL[i])
    pb = synth.prefill_batch(spec.pop("name"), seed=4200 + i, **spec)
    print(f"case prefill {pb.name} MB={pb.MB} all_qb={pb.all_qb}", flush=True)
    d = upload(pb)
    out = run(msa, pb, d)
    ref, sc = reference(pb)
    check_prefill(pb, out, ref, sc)


def test_prefill_select_workspace_reuse_smaller_second_call(msa):
    """Two calls in a row on one workspace (left with the first call's
    contents), the second with a smaller batch: both graded in full."""
    big = synth.prefill_batch("reuse_big", new_tokens=[300, 200, 129], prefix=[2000, 0, 900],
                              Hq=4, Di=128, block_size_q=64, topk=6, init_blocks=1,
                              local_blocks=1, seed=4301)
    small = synth.prefill_batch("reuse_small", new_tokens=[65], prefix=[1000], Hq=4, Di=128,
                                block_size_q=64, topk=6, init_blocks=1, local_blocks=1,
                                seed=4302, MB=big.MB)
    ws = prefill_workspace(msa, big)
    assert ws.numel() >= msa.msa_prefill_block_score_workspace_bytes(
        small.batch, small.Hq, small.all_qb, small.MB, small.block_size_q)
    for pb in (big, small):
        out = run(msa, pb, upload(pb), ws=ws)
        ref, sc = reference(pb)
        check_prefill(pb, out, ref, sc)


def test_prefill_select_no_requests(msa):
    """batch 0 with output rows: every row is -1."""
    pb = synth.prefill_batch("none", new_tokens=[64], prefix=[128], Hq=2, Di=128, block_size_q=64,
                             topk=4, seed=4303)
    pb.slot_ids = pb.slot_ids[:0]
    pb.seq_lens = pb.seq_lens[:0]
    pb.prefix_lens = pb.prefix_lens[:0]
    pb.cu_seqlens = pb.cu_seqlens[:1]
    pb.cu_seqblocks_q = pb.cu_seqblocks_q[:1]
    out = run(msa, pb, upload(pb))
    assert (out.cpu() == -1).all()


def test_prefill_select_deterministic(msa):
    pb = synth.prefill_batch("det", new_tokens=[500, 260], prefix=[3000, 700], Hq=4, Di=128,
                             block_size_q=64, topk=8, init_blocks=1, local_blocks=2, seed=4304)
    d = upload(pb)
    a = run(msa, pb, d)
    ws = prefill_workspace(msa, pb)
    b = run(msa, pb, d, ws=ws)
    c = run(msa, pb, d, ws=ws)                            # the counters are back at zero
    assert torch.equal(a, b) and torch.equal(a, c)


def test_prefill_select_graph_replay(msa):
    """The call captured in a graph and replayed several times, with eager
    work and new input values between the replays: every replay matches the
    eager call on the same inputs (the arrival counters are left at zero)."""
    pb = synth.prefill_batch("graph", new_tokens=[300, 130], prefix=[2000, 500], Hq=4, Di=128,
                             block_size_q=64, topk=6, init_blocks=1, local_blocks=1, seed=4306)
    d = upload(pb)
    ws = prefill_workspace(msa, pb)
    out = poisoned((pb.Hq, pb.all_qb, pb.topk), torch.int32)
    stream = torch.cuda.Stream()

    def call():
        msa.msa_prefill_block_score(d["q"], d["index_k"], d["block_table"], d["slot_ids"],
                                    d["cu_seqlens"], d["seq_lens"], d["prefix_lens"],
                                    pb.block_size_q, pb.B, pb.topk, pb.init_blocks,
                                    pb.local_blocks, pb.scale, d["cu_seqblocks_q"], out, ws)
    with torch.cuda.stream(stream):
        call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        call()
    torch.cuda.synchronize()
    q0 = d["q"].clone()
    for rep in range(3):
        # new query values in place (same address), then the eager reference
        d["q"].copy_(q0 if rep == 0 else torch.roll(q0, shifts=rep, dims=0))
        out.fill_(-5)
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        replayed = out.clone()
        out.fill_(-5)
        call()
        torch.cuda.synchronize()
        assert torch.equal(replayed, out), rep
    pb.q = d["q"].cpu()
    ref, sc = reference(pb)
    check_prefill(pb, out, ref, sc)


def sample_rows(pb, per_request=6, seed=4400):
    """Rows to grade at full size: for each request and head, its first and
    last query blocks plus random ones."""
    rng = np.random.default_rng(seed)
    rows = np.zeros((pb.Hq, pb.all_qb), dtype=bool)
    cu = pb.cu_seqblocks_q.numpy()
    for b in range(pb.batch):
        n = cu[b + 1] - cu[b]
        if n == 0:
            continue
        pick = {0, n - 1} | set(rng.integers(0, n, size=per_request).tolist())
        h = rng.integers(0, pb.Hq, size=len(pick))
        for hh, qb in zip(h, sorted(pick)):
            rows[hh, cu[b] + qb] = True
    return rows


def test_prefill_select_ragged_full_size_sampled(msa):
    """The full ragged prefill workload (4 requests, 2048/1536/1024/512 new
    tokens over 8192/4096/12288/2048 cached, 4 heads, Di 128, 64-token query
    blocks, top-16 with 1 initial and 2 local blocks) in the launch
    configuration the bench times; graded on sampled rows."""
    pb = synth.prefill_ragged()
    d = upload(pb)
    out = run(msa, pb, d)
    rows = sample_rows(pb)
    ref, sc = reference(pb, rows=rows)
    check_prefill(pb, out, ref, sc, rows=rows)
    # every row, sampled or not, is well formed
    check_format(pb, out.cpu().numpy())


def check_format(pb, gpu):
    owner, qbl = row_owner(pb)
    for h in range(pb.Hq):
        for g in range(pb.all_qb):
            row = gpu[h, g]
            sel = row[row >= 0]
            assert (row[len(sel):] == -1).all() and (np.diff(sel) > 0).all()
            if owner[g] < 0:
                assert len(sel) == 0
                continue
            b = owner[g]
            V = min(int(pb.seq_lens[b]), int(pb.prefix_lens[b]) + int(qbl[g]) * pb.block_size_q)
            ncand = -(-V // pb.B)
            assert len(sel) == min(pb.topk, ncand)
            forced = [j for j in range(ncand) if j < pb.init_blocks or j >= ncand - pb.local_blocks]
            assert set(forced[:pb.topk]) <= set(sel.tolist())


def test_prefill_select_strided_views(msa):
    """Every tensor passed as a strided view (query heads sliced out of a wider
    tensor, padded index pages, a transposed block table, offsets with stride 2,
    a permuted out_topk): the same selection as the contiguous call, bit for
    bit."""
    pb = synth.prefill_batch("strided", new_tokens=[200, 77, 130], prefix=[1500, 300, 4000], Hq=4,
                             Di=128, block_size_q=64, topk=5, init_blocks=1, local_blocks=1,
                             seed=4307, extra_qb_rows=2)
    d = upload(pb)
    ref = run(msa, pb, d)
    qw = torch.zeros((pb.total_q, pb.Hq + 2, pb.Di), dtype=torch.bfloat16, device="cuda")
    qw[:, 1:pb.Hq + 1] = d["q"]
    kw = torch.zeros((pb.P, 130, pb.Di), dtype=torch.uint8, device="cuda")
    kw[:, :128] = d["index_k"].view(torch.uint8)
    btw = d["block_table"].t().contiguous().t()                   # column-major

    def stride2(x):
        return torch.stack([x, torch.full_like(x, -99)], dim=1)[:, 0]
    sv = {n: stride2(d[n]) for n in ("slot_ids", "cu_seqlens", "seq_lens", "prefix_lens",
                                     "cu_seqblocks_q")}
    assert all(v.stride(0) == 2 for v in sv.values())
    outw = poisoned((pb.topk, pb.all_qb, pb.Hq), torch.int32).permute(2, 1, 0)
    ws = prefill_workspace(msa, pb)
    msa.msa_prefill_block_score(qw[:, 1:pb.Hq + 1], kw[:, :128].view(torch.float8_e4m3fn), btw,
                                sv["slot_ids"], sv["cu_seqlens"], sv["seq_lens"], sv["prefix_lens"],
                                pb.block_size_q, pb.B, pb.topk, pb.init_blocks, pb.local_blocks,
                                pb.scale, sv["cu_seqblocks_q"], outw, ws)
    torch.cuda.synchronize()
    assert torch.equal(outw, ref)


def test_prefill_select_bad_page_and_slot_ids_stay_in_bounds(msa):
    """Inputs outside the contract: a visible block whose page id lies outside
    [0, P) in one request's table row, and a slot id past the table in
    another request.  The call reads nothing outside its tensors (the kernels
    check both before any load) and the other requests' rows are exact."""
    pb = synth.prefill_batch("bad_ids", new_tokens=[150, 100, 90, 70], prefix=[900, 1300, 600, 2000],
                             Hq=4, Di=128, block_size_q=64, topk=5, init_blocks=1, local_blocks=1,
                             seed=4308)
    cu = pb.cu_seqblocks_q.numpy()
    good_rows = np.zeros((pb.Hq, pb.all_qb), dtype=bool)
    for b in (0, 3):
        good_rows[:, cu[b]:cu[b + 1]] = True
    ref, sc = reference(pb, rows=good_rows)
    bt = pb.block_table.clone()
    s1 = int(pb.slot_ids[1])
    bt[s1, 2] = -1                          # visible blocks of request 1
    bt[s1, 5] = pb.P + 3
    d = upload(pb)
    d["block_table"] = bt.cuda()
    d["slot_ids"][2] = bt.shape[0] + 7      # request 2: a slot past the table
    out = run(msa, pb, d)
    check_prefill(pb, out, ref, sc, rows=good_rows)
    g = out.cpu().numpy()
    assert ((g >= -1) & (g < pb.MB)).all()  # every cell written, ids in range or -1
