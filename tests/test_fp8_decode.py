"""Bit-exact GPU pins of the kernels' E4M3FN decode (OCP FP8 with |x|max 448,
the FP8 index and K/V caches of the vLLM design note "MiniMax-M3 decode
through the ATOM kernel library", "Supported experiment").

Every finite code is placed where the result is that code's value alone, so
the GPU must equal the oracle exactly (fp32 holds every product involved):
  * block scores over pages of constant codes with one-hot queries: the MFMA
    decode score kernel (pages loaded straight into registers, and staged
    through LDS), the vector score kernel (bf16 and fp32 queries), the prefill
    score sheet, with idx_scale 1 and a scale that rounds;
  * the ragged prefill score-to-selection call over the same pages, whose
    selections order every prefix of the codes from the top and the bottom;
  * attention with one visible key (out = v_scale * value(V code)) on the MFMA
    and the vector attention paths, and with two keys whose logits are equal
    exactly when the K codes decode right (out = v_scale / 2).
NaN codes sit only past seq_len, where they must not be read into a result.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from msa_harness import poisoned, run_attend, run_score, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def msa():
    import block_sparse_paged_amd as m
    return m


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


SCORE_CASES = {
    "mfma_decode_di128": dict(Di=128, T=4),
    "mfma_decode_di64_t16": dict(Di=64, T=16),
    # 8 rows: 1024 waves, pages staged through LDS (fewer rows load straight
    # into registers)
    "mfma_decode_di128_staged": dict(Di=128, T=4, R=8),
    "mfma_decode_di64_t16_staged": dict(Di=64, T=16, R=8),
    "vector_bf16q_di32": dict(Di=32, T=4),
    "vector_f32q_di128": dict(Di=128, T=3, q_f32=True),
    "prefill_sheet_t40": dict(Di=128, T=40),
    "mfma_decode_scale": dict(Di=128, T=4, idx_scale=0.3),
    "prefill_sheet_scale": dict(Di=64, T=24, idx_scale=0.3),
}


@pytest.mark.parametrize("name", list(SCORE_CASES))
def test_scores_every_code_exact(msa, name):
    c = synth.fp8_code_score_case(**SCORE_CASES[name])
    _say(f"case {name}: R={c.R} T={c.T} Di={c.Di} MB={c.MB}")
    d = upload(c)
    g = run_score(msa, c, d)
    torch.cuda.synchronize()
    gs = g.cpu().numpy()
    ref = oracle.block_score(c.q_idx, c.index_k, c.block_table, c.seq_lens, c.T, c.idx_scale)
    # the fp32 result of value * idx_scale is the correctly rounded product
    ref32 = ref.astype(np.float32)
    assert not np.isnan(gs).any()
    assert np.array_equal(gs, ref32), np.argwhere(gs != ref32)[:8]
    # every finite code appears as some block's score
    seen = {float(v) for v in ref32[:, :].ravel() if np.isfinite(v)}
    assert len(seen) >= 253 if c.idx_scale == 1.0 else True


def test_prefill_selection_orders_every_code(msa):
    pb = synth.fp8_code_prefill_batch()
    _say(f"case fp8 codes prefill: batch {pb.batch} Hq {pb.Hq} MB {pb.MB}")
    d = dict(q=pb.q.cuda(), index_k=pb.index_k.view(torch.float8_e4m3fn).cuda(),
             block_table=pb.block_table.cuda())
    for n in ("slot_ids", "cu_seqlens", "seq_lens", "prefix_lens", "cu_seqblocks_q"):
        d[n] = getattr(pb, n).cuda()
    nbytes = msa.msa_prefill_block_score_workspace_bytes(pb.batch, pb.Hq, pb.all_qb, pb.MB,
                                                         pb.block_size_q)
    ws = torch.zeros((nbytes,), dtype=torch.uint8, device="cuda")
    out = poisoned((pb.Hq, pb.all_qb, pb.topk), torch.int32)
    msa.msa_prefill_block_score(d["q"], d["index_k"], d["block_table"], d["slot_ids"],
                                d["cu_seqlens"], d["seq_lens"], d["prefix_lens"], pb.block_size_q,
                                pb.B, pb.topk, pb.init_blocks, pb.local_blocks, pb.scale,
                                d["cu_seqblocks_q"], out, ws)
    torch.cuda.synchronize()
    ref = oracle.prefill_select(pb.q, pb.index_k, pb.block_table, pb.slot_ids, pb.cu_seqlens,
                                pb.seq_lens, pb.prefix_lens, pb.block_size_q, pb.topk,
                                pb.init_blocks, pb.local_blocks, pb.scale, pb.cu_seqblocks_q,
                                pb.all_qb, threads=8)
    g = out.cpu().numpy()
    bad = np.argwhere((g != ref).any(axis=2))
    assert bad.size == 0, f"selections differ at (head, row) {bad[:8].tolist()}"


def _attend(msa, c):
    d = upload(c)
    tk = torch.zeros((c.N, 1), dtype=torch.int32)
    out = run_attend(msa, c, d, tk.cuda())
    torch.cuda.synchronize()
    ref = oracle.sparse_decode(c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens, tk.numpy(),
                               c.T, c.sm_scale, c.k_scale, c.v_scale)
    return out.float().cpu().double().numpy(), oracle.round_bf16(ref)


@pytest.mark.parametrize("Hq", [16, 4], ids=["mfma", "vector"])
def test_attention_one_key_every_v_code(msa, Hq):
    c = synth.fp8_one_key_v_case(Hq=Hq)
    _say(f"case one visible key, Hq={Hq}")
    g, rb = _attend(msa, c)
    assert np.array_equal(g, rb), np.argwhere(g != rb)[:8]
    # the expected values are the code values themselves, scaled
    codes = c.v_cache[:c.R, 0, 0].view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(rb, np.broadcast_to(codes[:, None, :] * c.v_scale, rb.shape))


@pytest.mark.parametrize("Hq", [16, 4], ids=["mfma", "vector"])
def test_attention_k_codes_equal_logits(msa, Hq):
    c = synth.fp8_k_pair_case(Hq=Hq)
    _say(f"case K code pairs, Hq={Hq}, {c.R} tokens")
    g, rb = _attend(msa, c)
    assert np.array_equal(rb, np.full(rb.shape, c.v_scale / 2))
    assert np.array_equal(g, rb), np.argwhere(g != rb)[:8]
