"""Seeded synthetic inputs for MSA sparse-layer decode attention.

This module only draws values and lays them out in the storage formats the
pages describe (paged FP8 E4M3FN index and K/V caches with 128-token blocks,
bf16 queries, int32 block tables and sequence lengths).  It holds none of the
method's arithmetic: no score, selection or attention is computed here.  Both
the CPU oracle and the HIP library consume the buffers it returns unchanged.

Workload shapes follow the vLLM design note "MiniMax-M3 decode through the
ATOM kernel library", section "Supported experiment": FP8 main and index
caches, block size 128, maximum model length 16384, decode/verification rows of
1 + 3 speculative tokens, buckets of 1/4/8/16 rows, and a 1024-block pool.

Value recipe: N(0,1) draws (numpy PCG64, one independent stream per tensor,
seeded by ``[seed, tensor_id]``).  FP8 tensors are quantised with a per-tensor
scale ``amax / 448`` so that the largest magnitude maps to the E4M3FN maximum,
rounded to nearest-even and saturated to +-448 (torch's float8_e4m3fn cast
turns overflow into NaN, so the clamp is explicit).  Pool pages that no row
maps, tail tokens past a row's length, and block-table entries past a row's
last block are poisoned so that any read of them shows up as NaN.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np
import torch

BLOCK = 128
E4M3_MAX = 448.0
E4M3_NAN_CODE = 0x7F

_TENSOR_IDS = {
    "q_idx": 1, "index": 2, "q": 3, "k": 4, "v": 5, "perm": 6, "lens": 7, "topk": 8,
    "slots": 9,
}


def _rng(seed: int, name: str) -> np.random.Generator:
    return np.random.default_rng([int(seed), _TENSOR_IDS[name]])


def quantize_e4m3(x: np.ndarray) -> tuple[torch.Tensor, float]:
    """Per-tensor E4M3FN quantisation: returns (uint8 codes, fp32 scale)."""
    amax = float(np.max(np.abs(x))) if x.size else 1.0
    scale = float(np.float32(amax / E4M3_MAX)) if amax > 0 else 1.0
    y = np.clip(x.astype(np.float32) / np.float32(scale), -E4M3_MAX, E4M3_MAX)
    codes = torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn)
    return codes.view(torch.uint8), scale


def to_bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x.astype(np.float32))).to(torch.bfloat16)


@dataclasses.dataclass
class Case:
    """One synthetic workload.  Tensors live on the CPU; shapes:

    q_idx [N, Di], index_k [P, B, Di], block_table [R, MB], seq_lens [R],
    q [N, Hq, D], k_cache / v_cache [P, B, Hkv, D].  FP8 tensors are uint8
    code tensors (``fp8=True``); otherwise float32.  Queries are bf16 when
    ``fp8`` else float32.
    """
    name: str
    R: int
    T: int
    Hq: int
    Hkv: int
    D: int
    Di: int
    P: int
    MB: int
    k: int
    B: int
    fp8: bool
    seq_lens: torch.Tensor
    block_table: torch.Tensor
    q_idx: torch.Tensor
    index_k: torch.Tensor
    q: Optional[torch.Tensor]
    k_cache: Optional[torch.Tensor]
    v_cache: Optional[torch.Tensor]
    idx_scale: float
    k_scale: float
    v_scale: float
    sm_scale: float

    @property
    def N(self) -> int:
        return self.R * self.T

    def visible(self, n: int) -> int:
        """Key positions visible to query token n (row-causal, new tokens in cache)."""
        r, t = divmod(n, self.T)
        return max(0, int(self.seq_lens[r]) - (self.T - 1 - t))


def make_case(name: str, *, R: int, T: int, Hq: int, Hkv: int, D: int, Di: int,
              seq_lens: Sequence[int], P: int, k: int, MB: Optional[int] = None,
              fp8: bool = True, seed: int = 0, attention: bool = True,
              shared_pages: bool = False, nan_q_rows: Sequence[int] = (),
              B: int = BLOCK) -> Case:
    """Build a paged workload.

    Each row r owns ceil(seq_lens[r] / B) logical blocks mapped to physical pages
    through a random block table.  With ``shared_pages=False`` rows take disjoint
    random page sets; with ``True`` every row draws its pages independently from
    the whole pool (pages may be shared between rows).  Unused pool pages, tail
    tokens past seq_len and block-table entries past the last block are poisoned.
    Rows listed in ``nan_q_rows`` get NaN queries (padded rows of a bucket).
    """
    lens = np.asarray(seq_lens, dtype=np.int64)
    assert lens.shape == (R,)
    nblk = (lens + B - 1) // B
    if MB is None:
        MB = int(max(1, nblk.max()))
    assert nblk.max() <= MB
    N = R * T
    prng = _rng(seed, "perm")
    used = int(nblk.sum())
    bt = np.zeros((R, MB), dtype=np.int32)
    if shared_pages:
        assert P > 1
        poison_page = P - 1
        for r in range(R):
            bt[r, : nblk[r]] = prng.choice(P - 1, size=nblk[r], replace=False)
        used_pages = np.unique(bt[nblk[:, None] > np.arange(MB)[None, :]])
    else:
        assert used < P, "need at least one spare page to serve as the poisoned page"
        perm = prng.permutation(P).astype(np.int32)
        off = 0
        for r in range(R):
            bt[r, : nblk[r]] = perm[off: off + nblk[r]]
            off += nblk[r]
        used_pages = perm[:used]
        poison_page = int(perm[used])
    for r in range(R):
        bt[r, nblk[r]:] = poison_page

    # which (page, token) slots hold real data
    slot_valid = np.zeros((P, B), dtype=bool)
    for r in range(R):
        for j in range(nblk[r]):
            ntok = min(B, int(lens[r]) - j * B)
            slot_valid[bt[r, j], :ntok] = True
    if shared_pages:
        slot_valid[used_pages] = True  # shared pages are fully written

    def pool(name_: str, shape_tail: tuple) -> tuple[torch.Tensor, float]:
        g = _rng(seed, name_)
        vals = g.standard_normal((len(used_pages), B) + shape_tail, dtype=np.float32)
        if fp8:
            codes, scale = quantize_e4m3(vals)
            out = torch.full((P, B) + shape_tail, E4M3_NAN_CODE, dtype=torch.uint8)
            out[torch.from_numpy(used_pages.astype(np.int64))] = codes
            mask = torch.from_numpy(~slot_valid)
            out[mask] = E4M3_NAN_CODE
            return out, scale
        out = torch.full((P, B) + shape_tail, float("nan"), dtype=torch.float32)
        out[torch.from_numpy(used_pages.astype(np.int64))] = torch.from_numpy(vals)
        out[torch.from_numpy(~slot_valid)] = float("nan")
        return out, 1.0

    index_k, idx_scale = pool("index", (Di,))
    qi = _rng(seed, "q_idx").standard_normal((N, Di), dtype=np.float32)
    q_idx = to_bf16(qi) if fp8 else torch.from_numpy(qi)
    q = k_cache = v_cache = None
    k_scale = v_scale = 1.0
    if attention:
        k_cache, k_scale = pool("k", (Hkv, D))
        v_cache, v_scale = pool("v", (Hkv, D))
        qq = _rng(seed, "q").standard_normal((N, Hq, D), dtype=np.float32)
        q = to_bf16(qq) if fp8 else torch.from_numpy(qq)
    for r in nan_q_rows:
        q_idx[r * T:(r + 1) * T] = float("nan")
        if q is not None:
            q[r * T:(r + 1) * T] = float("nan")
    sm_scale = float(np.float32(1.0 / math.sqrt(D)))
    return Case(name=name, R=R, T=T, Hq=Hq, Hkv=Hkv, D=D, Di=Di, P=P, MB=MB, k=k, B=B,
                fp8=fp8, seq_lens=torch.from_numpy(lens.astype(np.int32)),
                block_table=torch.from_numpy(bt), q_idx=q_idx, index_k=index_k,
                q=q, k_cache=k_cache, v_cache=v_cache, idx_scale=idx_scale,
                k_scale=k_scale, v_scale=v_scale, sm_scale=sm_scale)


# ---------------------------------------------------------------- named workloads

def tiny(seed: int = 1000) -> Case:
    """fp32, 1 row x 1 token, 4 q heads / 1 KV head, D=64, Di=32, 1024 tokens
    (8 blocks) mapped into a 16-page pool, top-k 4, all scales 1.0."""
    c = make_case("tiny_fp32", R=1, T=1, Hq=4, Hkv=1, D=64, Di=32, seq_lens=[1024],
                  P=16, k=4, fp8=False, seed=seed)
    c.sm_scale = 0.125
    return c


def decode_bucket4(seed: int = 2000) -> Case:
    """4 rows x 4 tokens, 16 q heads / 1 KV head, D=Di=128, FP8 caches, 16384
    context (128 blocks), top-k 16, 1024-page pool with a random block table."""
    return make_case("decode_r4_16k", R=4, T=4, Hq=16, Hkv=1, D=128, Di=128,
                     seq_lens=[16384] * 4, P=1024, k=16, seed=seed)


def bucket_sweep(R: int, seed: Optional[int] = None, pad_rows: Sequence[int] = ()) -> Case:
    """R rows x 4 tokens, per-row lengths uniform in [2048, 16384], top-k 16,
    4096-page pool, MB=128.  ``pad_rows`` get seq_len 0 and NaN queries."""
    seed = 3000 + R if seed is None else seed
    g = _rng(seed, "lens")
    lens = g.integers(2048, 16384, size=R, endpoint=True)
    for r in pad_rows:
        lens[r] = 0
    return make_case(f"sweep_r{R}", R=R, T=4, Hq=16, Hkv=1, D=128, Di=128,
                     seq_lens=lens.tolist(), P=4096, k=16, MB=128, seed=seed,
                     nan_q_rows=pad_rows)


def prefill(seed: int = 4000) -> Case:
    """4 requests x 2048 new tokens over an 8192-token prefix (seq_len 10240,
    80 blocks), FP8 index dim 128, per-token top-k 16 -> topk [8192, 16]."""
    return make_case("prefill_4x2048", R=4, T=2048, Hq=16, Hkv=1, D=128, Di=128,
                     seq_lens=[10240] * 4, P=1024, k=16, seed=seed, attention=False)


def hbm_decode(k: int = 16, seed: Optional[int] = None) -> Case:
    """16 rows x 4 tokens at 16384 context, 16 q / 1 KV heads, D=Di=128, FP8
    caches, 4096-page pool with non-overlapping tables, top-k ``k``."""
    seed = 5000 + k if seed is None else seed
    return make_case(f"hbm_r16_16k_k{k}", R=16, T=4, Hq=16, Hkv=1, D=128, Di=128,
                     seq_lens=[16384] * 16, P=4096, k=k, seed=seed)


def small_fp8(R: int = 2, T: int = 4, lens: Sequence[int] = (700, 1500), k: int = 4,
              P: Optional[int] = None, Hq: int = 16, D: int = 128, Di: int = 128,
              seed: int = 7, **kw) -> Case:
    """A small FP8 case spanning several blocks with ragged tails."""
    nblk = sum((int(x) + BLOCK - 1) // BLOCK for x in lens)
    P = P if P is not None else nblk + 5
    return make_case(f"small_fp8_r{R}", R=R, T=T, Hq=Hq, Hkv=1, D=D, Di=Di,
                     seq_lens=list(lens), P=P, k=k, seed=seed, **kw)


def random_topk(case: Case, seed: int = 11) -> torch.Tensor:
    """Caller-style topk_idx [N, k]: each token draws k distinct visible blocks
    (ascending, -1 padded) -- for testing attention on its own."""
    g = _rng(seed, "topk")
    out = np.full((case.N, case.k), -1, dtype=np.int32)
    for n in range(case.N):
        nvis = (case.visible(n) + case.B - 1) // case.B
        m = min(case.k, nvis)
        if m:
            out[n, :m] = np.sort(g.choice(nvis, size=m, replace=False))
    return torch.from_numpy(out)


# ------------------------------------------------- ragged prefill (score + select)

@dataclasses.dataclass
class PrefillBatch:
    """A ragged prefill batch for the fused score-to-selection call
    (attention.msa_prefill_block_score in Cacheon "Kernel ABI").  Request b
    (block-table row slot_ids[b]) has new tokens q[cu_seqlens[b] ..
    cu_seqlens[b+1]) after prefix_lens[b] cached keys; seq_lens[b] =
    prefix_lens[b] + its new tokens.

    q [total_q, Hq, Di] (bf16 or f32), index_k [P, B, Di] (E4M3 codes or f32),
    block_table [slots, MB] i32, the int32 vectors, and the selection policy."""
    name: str
    Hq: int
    Di: int
    B: int
    P: int
    MB: int
    block_size_q: int
    topk: int
    init_blocks: int
    local_blocks: int
    scale: float
    q: torch.Tensor
    index_k: torch.Tensor
    block_table: torch.Tensor
    slot_ids: torch.Tensor
    cu_seqlens: torch.Tensor
    seq_lens: torch.Tensor
    prefix_lens: torch.Tensor
    cu_seqblocks_q: torch.Tensor
    all_qb: int
    fp8: bool = True

    @property
    def batch(self) -> int:
        return int(self.slot_ids.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.q.shape[0])


def prefill_batch(name: str, *, new_tokens: Sequence[int], prefix: Sequence[int], Hq: int, Di: int,
                  block_size_q: int, topk: int, init_blocks: int = 0, local_blocks: int = 0,
                  slots: Optional[int] = None, P: Optional[int] = None, MB: Optional[int] = None,
                  extra_qb_rows: int = 0, fp8: bool = True, seed: int = 0,
                  B: int = BLOCK) -> PrefillBatch:
    """Random ragged prefill batch.  Requests take disjoint random pages of the
    pool and random block-table rows (slot ids); unused pages, tail slots and
    table entries past a request's last block are poisoned.  ``extra_qb_rows``
    output rows past the last request's query blocks belong to no request."""
    nq = np.asarray(new_tokens, dtype=np.int64)
    pre = np.asarray(prefix, dtype=np.int64)
    lens = nq + pre
    batch = len(nq)
    nblk = (lens + B - 1) // B
    MB = int(max(1, nblk.max())) if MB is None else MB
    assert nblk.max() <= MB
    slots = batch + 2 if slots is None else slots
    P = int(nblk.sum()) + 3 if P is None else P
    assert int(nblk.sum()) < P
    g = _rng(seed, "perm")
    perm = g.permutation(P).astype(np.int32)
    poison_page = int(perm[int(nblk.sum())])
    slot_ids = _rng(seed, "slots").permutation(slots)[:batch].astype(np.int32)
    bt = np.full((slots, MB), poison_page, dtype=np.int32)
    slot_valid = np.zeros((P, B), dtype=bool)
    off = 0
    for b in range(batch):
        pages = perm[off: off + nblk[b]]
        off += nblk[b]
        bt[slot_ids[b], : nblk[b]] = pages
        for j, pg in enumerate(pages):
            slot_valid[pg, : min(B, int(lens[b]) - j * B)] = True
    vals = _rng(seed, "index").standard_normal((P, B, Di), dtype=np.float32)
    if fp8:
        codes, scale = quantize_e4m3(vals[slot_valid])
        index_k = torch.full((P, B, Di), E4M3_NAN_CODE, dtype=torch.uint8)
        index_k[torch.from_numpy(slot_valid)] = codes
    else:
        scale = 1.0
        index_k = torch.from_numpy(vals)
        index_k[torch.from_numpy(~slot_valid)] = float("nan")
    total_q = int(nq.sum())
    qv = _rng(seed, "q_idx").standard_normal((total_q, Hq, Di), dtype=np.float32)
    q = to_bf16(qv) if fp8 else torch.from_numpy(qv)
    cu = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    nqb = (nq + block_size_q - 1) // block_size_q
    cuqb = np.concatenate([[0], np.cumsum(nqb)]).astype(np.int32)
    return PrefillBatch(name=name, Hq=Hq, Di=Di, B=B, P=P, MB=MB, block_size_q=block_size_q,
                        topk=topk, init_blocks=init_blocks, local_blocks=local_blocks,
                        scale=scale, q=q, index_k=index_k, block_table=torch.from_numpy(bt),
                        slot_ids=torch.from_numpy(slot_ids), cu_seqlens=torch.from_numpy(cu),
                        seq_lens=torch.from_numpy(lens.astype(np.int32)),
                        prefix_lens=torch.from_numpy(pre.astype(np.int32)),
                        cu_seqblocks_q=torch.from_numpy(cuqb), all_qb=int(cuqb[-1]) + extra_qb_rows,
                        fp8=fp8)


def prefill_ragged(seed: int = 4100) -> PrefillBatch:
    """The fused prefill score-to-selection workload: 4 requests with 2048,
    1536, 1024 and 512 new tokens over prefixes of 8192, 4096, 12288 and 2048
    tokens (up to 13824 keys, 108 blocks), 4 index query heads, Di = 128,
    query blocks of 64 tokens, top-k 16 with 1 initial and 2 local blocks."""
    return prefill_batch("prefill_ragged_4req", new_tokens=[2048, 1536, 1024, 512],
                         prefix=[8192, 4096, 12288, 2048], Hq=4, Di=128, block_size_q=64, topk=16,
                         init_blocks=1, local_blocks=2, P=512, seed=seed)


# ------------------------------------------- FP8 decode pins (every E4M3FN code)
#
# Inputs whose exact results follow from the E4M3FN value table alone: pages
# holding one code each, one-hot queries, a single visible key.  The values the
# codes stand for are never computed here; the tests take them from the oracle.

E4M3_FINITE_CODES = [c for c in range(256) if c not in (0x7F, 0xFF)]


def _code_pages(n_pages: int, Di: int, first: int = 0) -> torch.Tensor:
    """[n_pages, B, Di] uint8: page i holds code E4M3_FINITE_CODES[(first + i) % 254]
    in every key and dimension."""
    codes = torch.tensor([E4M3_FINITE_CODES[(first + i) % len(E4M3_FINITE_CODES)]
                          for i in range(n_pages)], dtype=torch.uint8)
    return codes.view(n_pages, 1, 1).expand(n_pages, BLOCK, Di).contiguous()


def fp8_code_score_case(Di: int = 128, T: int = 4, q_f32: bool = False, idx_scale: float = 1.0,
                        seed: int = 6100, R: int = 2) -> Case:
    """Block scores over pages of constant codes: R >= 2 rows x 128 blocks,
    page (r, j) holding finite code number 128 r + j (mod 254), so every finite
    code is some page; row 1 ends 5 keys into its last block, whose remaining
    keys hold the two NaN codes, the other rows are whole.  Token n's query is
    one-hot (1.0) at dimension (7 n + 3) mod Di, so its score for block j is
    the value of page j's code times idx_scale."""
    MB = 128
    P = R * MB + 1
    perm = _rng(seed, "perm").permutation(P).astype(np.int32)
    bt = perm[:R * MB].reshape(R, MB).copy()
    index_k = torch.full((P, BLOCK, Di), E4M3_NAN_CODE, dtype=torch.uint8)
    index_k[torch.from_numpy(bt.reshape(-1).astype(np.int64))] = _code_pages(R * MB, Di)
    lens = [MB * BLOCK, (MB - 1) * BLOCK + 5] + [MB * BLOCK] * (R - 2)
    last = int(bt[1, MB - 1])
    index_k[last, 5::2] = 0x7F
    index_k[last, 6::2] = 0xFF
    N = R * T
    qi = np.zeros((N, Di), dtype=np.float32)
    for n in range(N):
        qi[n, (7 * n + 3) % Di] = 1.0
    q_idx = torch.from_numpy(qi) if q_f32 else to_bf16(qi)
    return Case(name=f"fp8_codes_score_di{Di}_t{T}_r{R}", R=R, T=T, Hq=16, Hkv=1, D=128, Di=Di, P=P,
                MB=MB, k=16, B=BLOCK, fp8=True, seq_lens=torch.tensor(lens, dtype=torch.int32),
                block_table=torch.from_numpy(bt), q_idx=q_idx, index_k=index_k, q=None,
                k_cache=None, v_cache=None, idx_scale=float(np.float32(idx_scale)), k_scale=1.0,
                v_scale=1.0, sm_scale=float(np.float32(1.0 / math.sqrt(128))))


def fp8_code_prefill_batch(Hq: int = 2, topk: int = 16) -> PrefillBatch:
    """Ragged prefill batch over 254 shared pages of constant codes (every
    finite E4M3FN code once, in a seeded random block order).  Request b has
    prefix 128 (17 + b) keys and one new token (query blocks of one token), so
    its only query block selects among the first 17 + b blocks; head 0's query
    is +1 and head 1's -1 at one dimension, so the selections order the codes
    by value from the top and from the bottom."""
    Di, nb = 128, len(E4M3_FINITE_CODES)
    g = _rng(6200, "perm")
    order = g.permutation(nb)
    P = nb + 1
    index_k = torch.full((P, BLOCK, Di), 0x00, dtype=torch.uint8)
    index_k[:nb] = _code_pages(nb, Di)[torch.from_numpy(order.astype(np.int64))]
    batch = nb - 17
    prefix = np.array([BLOCK * (17 + b) for b in range(batch)], dtype=np.int64)
    MB = nb + 1
    bt = np.full((batch, MB), nb, dtype=np.int32)       # entry nb: the spare page (new tokens)
    bt[:, :nb] = np.arange(nb, dtype=np.int32)
    qv = np.zeros((batch, Hq, Di), dtype=np.float32)
    for b in range(batch):
        for h in range(Hq):
            qv[b, h, (5 * b + 11 * h) % Di] = 1.0 if h % 2 == 0 else -1.0
    cu = np.arange(batch + 1, dtype=np.int32)
    return PrefillBatch(name="fp8_codes_prefill", Hq=Hq, Di=Di, B=BLOCK, P=P, MB=MB, block_size_q=1,
                        topk=topk, init_blocks=0, local_blocks=0, scale=1.0, q=to_bf16(qv),
                        index_k=index_k, block_table=torch.from_numpy(bt),
                        slot_ids=torch.arange(batch, dtype=torch.int32), cu_seqlens=torch.from_numpy(cu),
                        seq_lens=torch.from_numpy((prefix + 1).astype(np.int32)),
                        prefix_lens=torch.from_numpy(prefix.astype(np.int32)),
                        cu_seqblocks_q=torch.from_numpy(cu.copy()), all_qb=batch)


def fp8_one_key_v_case(Hq: int = 16, v_scale: float = 0.125) -> Case:
    """Attention with one visible key per token (T = 1, seq_len 1): token r's
    key-0 V row holds finite codes 128 r .. 128 r + 127 (mod 254) over its 128
    dimensions, so out = v_scale * value(code) in every head.  K rows hold
    finite codes; every other slot of the page holds the NaN code."""
    R, D = 2, 128
    P = R + 1
    k_cache = torch.full((P, BLOCK, 1, D), E4M3_NAN_CODE, dtype=torch.uint8)
    v_cache = torch.full((P, BLOCK, 1, D), E4M3_NAN_CODE, dtype=torch.uint8)
    for r in range(R):
        row = torch.tensor([E4M3_FINITE_CODES[(128 * r + d) % len(E4M3_FINITE_CODES)]
                            for d in range(D)], dtype=torch.uint8)
        v_cache[r, 0, 0] = row
        k_cache[r, 0, 0] = row.flip(0)
    q = to_bf16(_rng(6300, "q").standard_normal((R, Hq, D), dtype=np.float32))
    return Case(name=f"fp8_one_key_v_h{Hq}", R=R, T=1, Hq=Hq, Hkv=1, D=D, Di=128, P=P, MB=1, k=1,
                B=BLOCK, fp8=True, seq_lens=torch.ones(R, dtype=torch.int32),
                block_table=torch.arange(R, dtype=torch.int32).view(R, 1), q_idx=None,
                index_k=None, q=q, k_cache=k_cache, v_cache=v_cache, idx_scale=1.0, k_scale=1.0,
                v_scale=float(np.float32(v_scale)), sm_scale=float(np.float32(1.0 / math.sqrt(D))))


def fp8_k_pair_case(Hq: int = 16, v_scale: float = 0.125) -> Case:
    """Attention with two visible keys per token (T = 1, seq_len 2) whose
    logits are equal exactly when the K codes decode right: head h's query is
    1.0 at dimensions 2h and 2h + 1; key 0 holds code c at both, key 1 the code
    of 2 value(c) at 2h and +0 at 2h + 1.  V is 1.0 for key 0 and 0 for key 1,
    so every output equals v_scale / 2.  Codes c run over every finite code
    whose double is a finite E4M3FN value, Hq of them per token."""
    D = 128
    assert 2 * Hq <= D
    vals = torch.tensor(E4M3_FINITE_CODES, dtype=torch.uint8).view(torch.float8_e4m3fn).float()
    dbl = (2 * vals).to(torch.float8_e4m3fn)
    ok = [i for i in range(len(vals))
          if torch.isfinite(dbl[i].float()) and dbl[i].float() == 2 * vals[i] and abs(float(vals[i])) <= 224]
    pairs = [(E4M3_FINITE_CODES[i], int(dbl[i].view(torch.uint8))) for i in ok]
    R = -(-len(pairs) // Hq)
    P = R + 1
    k_cache = torch.full((P, BLOCK, 1, D), E4M3_NAN_CODE, dtype=torch.uint8)
    v_cache = torch.full((P, BLOCK, 1, D), E4M3_NAN_CODE, dtype=torch.uint8)
    qv = np.zeros((R, Hq, D), dtype=np.float32)
    for r in range(R):
        k_cache[r, 0:2, 0] = 0x00
        v_cache[r, 0, 0] = 0x38                   # 1.0
        v_cache[r, 1, 0] = 0x00
        for h in range(Hq):
            c, c2 = pairs[(r * Hq + h) % len(pairs)]
            k_cache[r, 0, 0, 2 * h] = c
            k_cache[r, 0, 0, 2 * h + 1] = c
            k_cache[r, 1, 0, 2 * h] = c2
            qv[r, h, 2 * h] = qv[r, h, 2 * h + 1] = 1.0
    return Case(name=f"fp8_k_pairs_h{Hq}", R=R, T=1, Hq=Hq, Hkv=1, D=D, Di=128, P=P, MB=1, k=1,
                B=BLOCK, fp8=True, seq_lens=torch.full((R,), 2, dtype=torch.int32),
                block_table=torch.arange(R, dtype=torch.int32).view(R, 1), q_idx=None,
                index_k=None, q=to_bf16(qv), k_cache=k_cache, v_cache=v_cache, idx_scale=1.0,
                k_scale=1.0, v_scale=float(np.float32(v_scale)),
                sm_scale=float(np.float32(1.0 / math.sqrt(D))))
