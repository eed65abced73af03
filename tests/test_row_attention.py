"""GPU parity of the row-level attention kernel: the form msa_sparse_decode,
msa_select_sparse_decode and msa_decode_step take for bf16 queries, FP8 K/V,
16 query heads per KV head and 2 to 4 tokens per row when a row's tokens
share most of at least 64 selected blocks -- one selection per request, or
per-token selections close to all of a row's blocks (the vLLM design note
"MiniMax-M3 decode through the ATOM kernel library", "Cacheon kernel ABI",
attention.decode over the supplied block ids).

Every case compares the GPU output with the oracle element by element:
ragged lengths with partial last pages (NaN poison past seq_len), rows
shorter than their token count (tokens that see no key give zeros), an empty
row, D = 64 and 128, 2, 3 and 4 tokens per row, selections per KV head with
-1 holes, duplicates and ids past the visible range, and one selection per
request.  The selecting calls are checked bit for bit against the separate
calls."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from msa_harness import (bf16_ulp, check_attention, oracle_attention, poisoned, run_attend, run_score,
                         run_select, upload, workspace)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def msa():
    import block_sparse_paged_amd as m
    return m


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _all_visible(c):
    """[N, k]: every block visible to each token, ascending, -1 padded."""
    tk = np.full((c.N, c.k), -1, dtype=np.int32)
    for n in range(c.N):
        nvis = min(c.k, (c.visible(n) + c.B - 1) // c.B)
        tk[n, :nvis] = np.arange(nvis)
    return tk


def _with_gaps(tk, MB, seed):
    """A caller's selection with holes: -1 entries, ids >= MB, duplicates and
    blocks past the token's visible range; and the clean set the oracle
    reads."""
    g = np.random.default_rng(seed)
    tk = tk.copy()
    flat = tk.reshape(-1, tk.shape[-1])
    for row in range(flat.shape[0]):
        a, b, c2 = g.choice(flat.shape[1], size=3, replace=False)
        flat[row, a] = -1
        flat[row, b] = MB + int(g.integers(0, 5))
        flat[row, c2] = flat[row, (c2 + 1) % flat.shape[1]]    # duplicate
    clean = tk.copy()
    clean[(clean >= MB) | (clean < 0)] = -1
    for row in clean.reshape(-1, clean.shape[-1]):
        seen = set()
        for i, j in enumerate(row):
            if j in seen:
                row[i] = -1
            elif j >= 0:
                seen.add(int(j))
    return tk, clean


ROW = {
    # all visible blocks of each token: lengths 1 (three tokens see nothing),
    # 3 (tokens that see 0 to 3 keys), 130, 9000, 16384 (128 blocks)
    "t4_d128_all_blocks": dict(R=5, T=4, Hq=16, Hkv=1, D=128, Di=128,
                               seq_lens=[1, 3, 130, 9000, 16384], P=220, k=128, MB=128),
    # D = 64, three tokens per row, an empty row
    "t3_d64_all_blocks": dict(R=4, T=3, Hq=16, Hkv=1, D=64, Di=64,
                              seq_lens=[9000, 0, 129, 8500], P=150, k=71, MB=71),
    # two tokens per row, two KV heads (32 query heads)
    "t2_d128_hkv2": dict(R=3, T=2, Hq=32, Hkv=2, D=128, Di=128,
                         seq_lens=[9000, 257, 8300], P=150, k=71, MB=71),
}


def _near_exact(out, ref):
    """Within one bf16 step of the oracle's rounded value plus 2^-14 (the
    weights are carried to about 2^-17: see test_tokens_that_see_few_keys)."""
    g = out.float().cpu().double().numpy()
    rb = oracle.round_bf16(ref)
    excess = np.abs(g - rb) - bf16_ulp(rb)
    assert (excess <= 2.0 ** -14).all(), f"{int((excess > 2.0 ** -14).sum())} cells beyond the bound"


@pytest.mark.parametrize("name", list(ROW))
def test_row_attention_all_visible_blocks(msa, name):
    c = synth.make_case(name, seed=6100 + len(name), **ROW[name])
    _say(f"case {name}: R={c.R} T={c.T} D={c.D} Hkv={c.Hkv} k={c.k} MB={c.MB}")
    d = upload(c)
    tk = _all_visible(c)
    out = run_attend(msa, c, d, torch.from_numpy(tk).cuda())
    torch.cuda.synchronize()
    ref = oracle_attention(c, tk)
    check_attention(out, ref)
    _near_exact(out, ref)
    # tokens that see no key give zeros
    for n in range(c.N):
        if c.visible(n) == 0:
            assert (out[n].float().cpu() == 0).all(), f"token {n} sees no key"


def test_row_attention_per_head_selection_with_gaps(msa):
    spec = dict(R=3, T=3, Hq=32, Hkv=2, D=64, Di=64, seq_lens=[9000, 129, 8800], P=160, k=60)
    c = synth.make_case("row_gaps", seed=6201, **spec)
    _say(f"case row_gaps: R={c.R} T={c.T} D={c.D} Hkv={c.Hkv} k={c.k} MB={c.MB}")
    d = upload(c)
    g = np.random.default_rng(6202)
    sel = np.full((c.Hkv, c.N, c.k), -1, dtype=np.int32)
    for h in range(c.Hkv):
        for n in range(c.N):
            nvis = (c.visible(n) + c.B - 1) // c.B
            m = min(c.k - 3, nvis)
            # some entries past the visible range as well
            pool = np.arange(min(c.MB, nvis + 2))
            sel[h, n, :m] = np.sort(g.choice(pool, size=m, replace=False))
    tk, clean = _with_gaps(sel, c.MB, seed=6203)
    out = poisoned((c.N, c.Hq, c.D), torch.bfloat16)
    msa.msa_sparse_decode(d.q, d.k_cache, d.v_cache, d.block_table, d.seq_lens, torch.from_numpy(tk).cuda(),
                          c.T, out, c.sm_scale, c.k_scale, c.v_scale, c.B, workspace(msa, c, c.k))
    torch.cuda.synchronize()
    check_attention(out, oracle_attention(c, clean))


@pytest.mark.parametrize("T", [2, 4])
def test_row_attention_selection_per_request(msa, T):
    spec = dict(R=4, Hq=16, Hkv=1, D=128, Di=128, seq_lens=[9000, 128, 2, 8500], P=150, k=64)
    c = synth.make_case(f"row_per_request_t{T}", T=T, seed=6300 + T, **spec)
    _say(f"case row_per_request: R={c.R} T={c.T} k={c.k} MB={c.MB}")
    d = upload(c)
    g = np.random.default_rng(6310 + T)
    sel = np.full((c.R, c.k), -1, dtype=np.int32)
    for r in range(c.R):
        nblk = (int(c.seq_lens[r]) + c.B - 1) // c.B
        m = min(c.k, nblk)
        sel[r, :m] = np.sort(g.choice(nblk, size=m, replace=False))
    out = run_attend(msa, c, d, torch.from_numpy(sel).cuda())
    torch.cuda.synchronize()
    ref = oracle_attention(c, sel)
    check_attention(out, ref)
    _near_exact(out, ref)


@pytest.mark.parametrize("D", [64, 128])
def test_row_attention_step_selects_in_launch(msa, D):
    """msa_decode_step with k = all of a row's blocks (the selection made
    inside the row-level launch) equals the three separate calls bit for bit
    and the oracle on its own selection."""
    c = synth.small_fp8(R=3, T=4, lens=(9000, 130, 8300), k=71, D=D, Di=D, seed=6400 + D)
    _say(f"case row_step: D={D} k={c.k} MB={c.MB}")
    d = upload(c)
    s1 = run_score(msa, c, d)
    t1 = run_select(msa, c, s1)
    o1 = run_attend(msa, c, d, t1)
    scores = poisoned((c.N, c.MB), torch.float32)
    topk = poisoned((c.N, c.k), torch.int32)
    out = poisoned((c.N, c.Hq, c.D), torch.bfloat16)
    ws = torch.zeros(msa.msa_decode_step_workspace_bytes(c.R, c.T, c.Hq, c.Hkv, c.D, c.k),
                     dtype=torch.uint8, device="cuda")
    msa.msa_decode_step(d.q_idx, d.index_k, d.q, d.k_cache, d.v_cache, d.block_table, d.seq_lens,
                        c.T, c.k, c.B, c.idx_scale, c.sm_scale, c.k_scale, c.v_scale, scores, topk, out, ws)
    torch.cuda.synchronize()
    assert torch.equal(scores.view(torch.int32), s1.view(torch.int32))
    assert torch.equal(topk, t1)
    assert torch.equal(out.view(torch.int16), o1.view(torch.int16))
    check_attention(out, oracle_attention(c, topk.cpu().numpy()))


def test_row_attention_step_per_request_sheet(msa):
    """msa_decode_step with one sheet row and one selection per request (64 of
    each row's blocks, the selection made inside the row-level launch by one
    wave for the whole row) equals msa_block_score -> msa_select_topk ->
    msa_sparse_decode on the per-request sheet bit for bit, and the oracle."""
    c = synth.make_case("row_step_per_request", R=3, T=4, Hq=16, Hkv=1, D=128, Di=128,
                        seq_lens=[9000, 8300, 130], P=150, k=64, seed=6501)
    _say(f"case row_step_per_request: R={c.R} T={c.T} k={c.k} MB={c.MB}")
    d = upload(c)
    s1 = poisoned((c.R, c.MB), torch.float32)
    msa.msa_block_score(d.q_idx, d.index_k, d.block_table, d.seq_lens, c.T, c.B, c.idx_scale, s1)
    t1 = poisoned((c.R, c.k), torch.int32)
    msa.msa_select_topk(s1, c.k, t1)
    o1 = run_attend(msa, c, d, t1)
    scores = poisoned((c.R, c.MB), torch.float32)
    topk = poisoned((c.R, c.k), torch.int32)
    out = poisoned((c.N, c.Hq, c.D), torch.bfloat16)
    ws = torch.zeros(msa.msa_decode_step_workspace_bytes(c.R, c.T, c.Hq, c.Hkv, c.D, c.k),
                     dtype=torch.uint8, device="cuda")
    msa.msa_decode_step(d.q_idx, d.index_k, d.q, d.k_cache, d.v_cache, d.block_table, d.seq_lens,
                        c.T, c.k, c.B, c.idx_scale, c.sm_scale, c.k_scale, c.v_scale, scores, topk, out, ws)
    torch.cuda.synchronize()
    assert torch.equal(scores.view(torch.int32), s1.view(torch.int32))
    assert torch.equal(topk, t1)
    assert torch.equal(out.view(torch.int16), o1.view(torch.int16))
    gt = topk.cpu().numpy()
    assert np.array_equal(gt, oracle.select_topk(scores.cpu().numpy().astype(np.float64), c.k))
    ref = oracle_attention(c, gt)
    check_attention(out, ref)
    _near_exact(out, ref)
