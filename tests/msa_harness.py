"""Shared GPU-test helpers: upload a synthetic workload, run the three library
stages through the C ABI, and grade the results against the CPU oracle.

Grading (tolerances of the parity bar):
  * scores: |gpu - ref| <= 1e-3 * max(|ref|, 1); -inf exactly where the oracle
    has -inf; no NaN.
  * topk on the GPU's own score sheet: bit-exact with the oracle's selection on
    that same fp32 sheet (integer work: no tolerance).
  * topk end to end: rows whose k-th and (k+1)-th oracle scores are at least
    1e-4 (relative) apart must match exactly; at near-tie rows every differing
    id must score within 1e-4 (relative) of the k-th; mean overlap >= 0.99.
  * attention: the oracle runs on the GPU's own topk_idx; both outputs are
    rounded to bf16 and must agree within 2e-3 (max abs), or within one bf16
    ulp of the reference where that ulp is larger (|out| >= 0.25).
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np
import torch

import oracle
import synth

SCORE_RTOL = 1e-3
TIE_RTOL = 1e-4
ATTN_ATOL = 2e-3


def dev(t: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    return None if t is None else t.to("cuda")


def fp8(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.float8_e4m3fn) if t.dtype == torch.uint8 else t


@dataclasses.dataclass
class Dev:
    q_idx: Optional[torch.Tensor]
    index_k: Optional[torch.Tensor]
    block_table: torch.Tensor
    seq_lens: torch.Tensor
    q: Optional[torch.Tensor]
    k_cache: Optional[torch.Tensor]
    v_cache: Optional[torch.Tensor]


def upload(case: synth.Case) -> Dev:
    return Dev(q_idx=dev(case.q_idx), index_k=dev(None if case.index_k is None else fp8(case.index_k)),
               block_table=dev(case.block_table), seq_lens=dev(case.seq_lens),
               q=dev(case.q), k_cache=dev(None if case.k_cache is None else fp8(case.k_cache)),
               v_cache=dev(None if case.v_cache is None else fp8(case.v_cache)))


def poisoned(shape, dtype) -> torch.Tensor:
    if dtype == torch.int32:
        return torch.full(shape, -7777, dtype=dtype, device="cuda")
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


def run_score(msa, case, d: Dev, scores: Optional[torch.Tensor] = None) -> torch.Tensor:
    if scores is None:
        scores = poisoned((case.N, case.MB), torch.float32)
    msa.msa_block_score(d.q_idx, d.index_k, d.block_table, d.seq_lens, case.T, case.B,
                        case.idx_scale, scores)
    return scores


def run_select(msa, case, scores, topk: Optional[torch.Tensor] = None, k: Optional[int] = None):
    k = case.k if k is None else k
    if topk is None:
        topk = poisoned((scores.shape[0], k), torch.int32)
    msa.msa_select_topk(scores, k, topk)
    return topk


def workspace(msa, case, k: int) -> torch.Tensor:
    nbytes = msa.msa_sparse_decode_workspace_bytes(case.R, case.T, case.Hq, case.Hkv, case.D, k)
    return torch.zeros(max(nbytes, 1), dtype=torch.uint8, device="cuda")


def run_attend(msa, case, d: Dev, topk, out: Optional[torch.Tensor] = None,
               ws: Optional[torch.Tensor] = None, out_dtype=None) -> torch.Tensor:
    if out is None:
        out_dtype = out_dtype or (torch.bfloat16 if case.fp8 else torch.float32)
        out = poisoned((case.N, case.Hq, case.D), out_dtype)
    if ws is None:
        ws = workspace(msa, case, topk.shape[1])
    msa.msa_sparse_decode(d.q, d.k_cache, d.v_cache, d.block_table, d.seq_lens, topk, case.T,
                          out, case.sm_scale, case.k_scale, case.v_scale, case.B, ws)
    return out


# ------------------------------------------------------------------ grading

def check_scores(gpu: np.ndarray, ref: np.ndarray, rows: Optional[Sequence[int]] = None):
    if rows is not None:
        gpu, ref = gpu[rows], ref[rows]
    assert not np.isnan(gpu).any(), "NaN left in the score sheet"
    ninf_ref = np.isneginf(ref)
    assert np.array_equal(np.isneginf(gpu), ninf_ref), "-inf pattern differs"
    fin = ~ninf_ref
    err = np.abs(gpu[fin] - ref[fin]) / np.maximum(np.abs(ref[fin]), 1.0)
    worst = float(err.max()) if err.size else 0.0
    assert worst <= SCORE_RTOL, f"score rel err {worst:.3g} > {SCORE_RTOL}"
    return worst


def check_topk_isolated(gpu_topk: np.ndarray, gpu_scores: np.ndarray):
    ref = oracle.select_topk(gpu_scores.astype(np.float64), gpu_topk.shape[1])
    bad = np.nonzero((ref != gpu_topk).any(axis=1))[0]
    assert bad.size == 0, f"topk differs from the oracle on the GPU's own sheet at rows {bad[:8]}"


def check_topk_end_to_end(gpu_topk: np.ndarray, ref_scores: np.ndarray,
                          rows: Optional[Sequence[int]] = None) -> float:
    k = gpu_topk.shape[1]
    ref_topk = oracle.select_topk(ref_scores, k)
    rows = range(gpu_topk.shape[0]) if rows is None else rows
    overlaps = []
    for n in rows:
        a, b = set(gpu_topk[n][gpu_topk[n] >= 0]), set(ref_topk[n][ref_topk[n] >= 0])
        s = ref_scores[n]
        cand = np.sort(s[np.isfinite(s) | (s == np.inf)])[::-1]
        overlaps.append(1.0 if a == b else len(a & b) / max(len(a), len(b)))
        if a == b:
            continue
        assert len(cand) > k, f"row {n}: fewer candidates than k but sets differ"
        sk, sk1 = cand[k - 1], cand[k]
        near = abs(sk - sk1) < TIE_RTOL * max(abs(sk), abs(sk1))
        assert near, f"row {n}: selections differ away from a near tie"
        for j in a ^ b:
            assert abs(s[j] - sk) <= TIE_RTOL * max(abs(sk), abs(sk1)), f"row {n}: id {j} is not a near-tie"
    mean = float(np.mean(overlaps)) if overlaps else 1.0
    assert mean >= 0.99, f"mean topk overlap {mean:.4f} < 0.99"
    return mean


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |x| (8 significant bits)."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, np.ldexp(1.0, (e - 7).astype(int)), 0.0)


def check_attention(gpu_out: torch.Tensor, ref: np.ndarray,
                    rows: Optional[Sequence[int]] = None) -> float:
    g = gpu_out.float().cpu().double().numpy()
    if rows is not None:
        g, ref = g[rows], ref[rows]
    assert not np.isnan(g).any(), "NaN in the attention output"
    gb = oracle.round_bf16(g)
    rb = oracle.round_bf16(ref)
    diff = np.abs(gb - rb)
    # Both sides rounding to bf16 may land on adjacent values; where one bf16
    # ulp exceeds 2e-3 (|out| >= 0.25, never in the named workloads) one ulp of
    # the reference is allowed instead.
    tol = np.maximum(ATTN_ATOL, bf16_ulp(rb))
    bad = diff > tol
    assert not bad.any(), (f"attention err {diff[bad].max():.3g} > tol at {int(bad.sum())} cells"
                           f" (max-abs err {diff.max():.3g})")
    err = float(diff.max()) if g.size else 0.0
    return err


def oracle_scores(case, n_range=None, threads: int = 8) -> np.ndarray:
    return oracle.block_score(case.q_idx, case.index_k, case.block_table, case.seq_lens, case.T,
                              case.idx_scale, n_range=n_range, threads=threads)


def oracle_attention(case, topk: np.ndarray, n_range=None, threads: int = 8) -> np.ndarray:
    return oracle.sparse_decode(case.q, case.k_cache, case.v_cache, case.block_table,
                                case.seq_lens, topk, case.T, case.sm_scale, case.k_scale,
                                case.v_scale, n_range=n_range, threads=threads)


def full_step_parity(msa, case, threads: int = 8, check_e2e: bool = True):
    """Run score -> select -> attend on the GPU and grade every stage."""
    d = upload(case)
    scores = run_score(msa, case, d)
    topk = run_select(msa, case, scores)
    out = run_attend(msa, case, d, topk) if case.q is not None else None
    torch.cuda.synchronize()
    gs = scores.cpu().numpy()
    gt = topk.cpu().numpy()
    ref_s = oracle_scores(case, threads=threads)
    res = {"score_err": check_scores(gs, ref_s)}
    check_topk_isolated(gt, gs)
    if check_e2e:
        res["overlap"] = check_topk_end_to_end(gt, ref_s)
    if out is not None:
        ref_o = oracle_attention(case, gt, threads=threads)
        res["attn_err"] = check_attention(out, ref_o)
    return res
