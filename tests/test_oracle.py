"""Pins for the CPU oracle (no GPU).

The oracle is checked against things other than itself:
  * library routines: torch's float8_e4m3fn / bfloat16 casts for the decoders;
  * hand-worked examples under tests/golden/ (each with its citation);
  * closed forms: one-hot and constant inputs, single visible key, equal keys,
    sm_scale = 0, value scaling;
  * brute force on tiny inputs by a structurally different route (a dense
    masked [N, L] matrix built with numpy matmul, reshaped per block);
  * invariants: top-k with every block selected equals dense attention,
    permuting physical pages together with the block table changes nothing,
    selections are the k best with ties to the lower id.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f(x):
    if x is None:
        return float("nan")
    if isinstance(x, str):
        return float(x)
    return float(x)


def _arr(nested):
    return np.vectorize(_f, otypes=[np.float64])(np.array(nested, dtype=object))


# ------------------------------------------------------------------ decoding

def test_e4m3fn_all_codes_match_torch(orc):
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).double().numpy()
    got = np.array([orc.e4m3fn_value(c) for c in range(256)])
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))


def test_e4m3fn_spec_codes(orc):
    g = json.load(open(os.path.join(GOLDEN, "e4m3fn_codes.json")))
    for k, v in g["codes"].items():
        got = orc.e4m3fn_value(int(k, 16))
        if v == "nan":
            assert math.isnan(got), k
        else:
            assert got == v and math.copysign(1, got) == math.copysign(1, v), k


def test_bf16_all_patterns_match_torch(orc):
    bits = torch.arange(-32768, 32768, dtype=torch.int32).to(torch.int16)
    ref = bits.view(torch.bfloat16).to(torch.float32).double().numpy()
    sample = np.arange(0, 65536, 7)   # every 7th pattern through the C entry point
    got = np.array([orc.bf16_value(int(bits[i]) & 0xFFFF) for i in sample])
    r = ref[sample]
    assert np.array_equal(np.isnan(r), np.isnan(got))
    ok = ~np.isnan(r)
    assert np.array_equal(r[ok], got[ok])


# ------------------------------------------------------------ brute force

def _decode(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.uint8:
        return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return t.to(torch.float64).numpy()


def _dense_keys(case, pool, r):
    """All key positions of row r in order, gathered through the block table."""
    arr = _decode(pool)
    L = int(case.seq_lens[r])
    pages = case.block_table[r].numpy()
    idx = np.arange(L)
    return arr[pages[idx // case.B], idx % case.B]


def brute_scores(case):
    """score[n, j] via a dense masked dot matrix per row, reshaped into blocks."""
    qi = _decode(case.q_idx)
    N, MB, B = case.N, case.MB, case.B
    out = np.full((N, MB), -np.inf)
    for r in range(case.R):
        L = int(case.seq_lens[r])
        if L == 0:
            continue
        K = _dense_keys(case, case.index_k, r)                 # [L, Di]
        rows = slice(r * case.T, (r + 1) * case.T)
        dots = qi[rows] @ K.T                                  # [T, L]
        vis = np.array([case.visible(n) for n in range(r * case.T, (r + 1) * case.T)])
        dots = np.where(np.arange(L)[None, :] < vis[:, None], dots, -np.inf)
        pad = MB * B - L
        dots = np.concatenate([dots, np.full((case.T, pad), -np.inf)], axis=1)
        out[rows] = dots.reshape(case.T, MB, B).max(axis=2) * case.idx_scale
    return out


def brute_attention(case, topk):
    """Masked dense softmax over [N, Hq, L] built from numpy matmuls.  topk is
    [N, K] (shared by the KV heads) or [Hkv, N, K] (one selection per KV head)."""
    q = _decode(case.q)
    N, Hq, D = q.shape
    G = case.Hq // case.Hkv
    per_head = np.ndim(topk) == 3
    out = np.zeros((N, Hq, D))
    for r in range(case.R):
        L = int(case.seq_lens[r])
        if L == 0:
            continue
        Kf = _dense_keys(case, case.k_cache, r) * case.k_scale   # [L, Hkv, D]
        Vf = _dense_keys(case, case.v_cache, r) * case.v_scale
        for t in range(case.T):
            n = r * case.T + t
            for h in range(Hq):
                g = h // G
                sel = np.zeros(L, dtype=bool)
                for j in (topk[g][n] if per_head else topk[n]):
                    if 0 <= j < case.MB:
                        sel[j * case.B:(j + 1) * case.B] = True
                sel &= np.arange(L) < case.visible(n)
                if not sel.any():
                    continue
                logits = case.sm_scale * (Kf[sel, g] @ q[n, h])
                w = np.exp(logits - logits.max())
                out[n, h] = (w / w.sum()) @ Vf[sel, g]
    return out


def small_cases():
    return [
        synth.make_case("b4_fp32", R=2, T=3, Hq=4, Hkv=2, D=8, Di=4, seq_lens=[13, 7], P=12,
                        k=2, fp8=False, seed=1, B=4),
        synth.make_case("b4_fp8", R=3, T=4, Hq=4, Hkv=1, D=16, Di=8, seq_lens=[17, 3, 0],
                        P=14, k=3, fp8=True, seed=2, B=4),
        synth.make_case("b8_fp8_shared", R=2, T=2, Hq=2, Hkv=1, D=8, Di=8, seq_lens=[30, 25],
                        P=9, k=2, fp8=True, seed=3, B=8, shared_pages=True),
        synth.make_case("b128_fp8", R=1, T=4, Hq=16, Hkv=1, D=32, Di=32, seq_lens=[300],
                        P=6, k=2, fp8=True, seed=4),
    ]


@pytest.mark.parametrize("case", small_cases(), ids=lambda c: c.name)
def test_score_matches_brute_force(orc, case):
    got = orc.block_score(case.q_idx, case.index_k, case.block_table, case.seq_lens, case.T,
                          case.idx_scale)
    ref = brute_scores(case)
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    fin = np.isfinite(ref)
    np.testing.assert_allclose(got[fin], ref[fin], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("case", small_cases(), ids=lambda c: c.name)
def test_attention_matches_brute_force(orc, case):
    topk = synth.random_topk(case, seed=5).numpy()
    got = orc.sparse_decode(case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens,
                            topk, case.T, case.sm_scale, case.k_scale, case.v_scale)
    ref = brute_attention(case, topk)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


def test_attention_per_kv_head_selection(orc):
    """attention.decode's (Hkv, B, K) selection: KV head g's query heads attend
    topk[g] only.  Different random selections per head against brute force,
    and a head that selects every block against dense attention."""
    case = synth.make_case("b4_fp32_hkv2", R=2, T=3, Hq=4, Hkv=2, D=8, Di=4, seq_lens=[13, 7],
                           P=12, k=2, fp8=False, seed=1, B=4)
    tk = np.stack([synth.random_topk(case, seed=5).numpy(), synth.random_topk(case, seed=6).numpy()])
    assert not np.array_equal(tk[0], tk[1])
    got = orc.sparse_decode(case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens,
                            tk, case.T, case.sm_scale, case.k_scale, case.v_scale)
    np.testing.assert_allclose(got, brute_attention(case, tk), rtol=1e-11, atol=1e-12)
    every = np.tile(np.arange(case.MB, dtype=np.int32), (case.N, 1))
    first = np.full_like(every, -1)
    first[:, :tk.shape[2]] = tk[0]
    mixed = np.stack([first, every])
    got = orc.sparse_decode(case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens,
                            mixed, case.T, case.sm_scale, case.k_scale, case.v_scale)
    dense = orc.dense_attention(case.q, case.k_cache, case.v_cache, case.block_table,
                                case.seq_lens, case.T, case.sm_scale, case.k_scale, case.v_scale)
    np.testing.assert_allclose(got[:, 2:], dense[:, 2:], rtol=1e-11, atol=1e-12)   # KV head 1
    np.testing.assert_allclose(got[:, :2], brute_attention(case, tk[0])[:, :2], rtol=1e-11, atol=1e-12)


def test_attention_bf16_cache_matches_brute_force(orc):
    """A dense bf16 K/V cache (attention.decode's commissioned cache): the
    oracle reads the bf16 values exactly."""
    case = synth.make_case("b4_bf16kv", R=2, T=3, Hq=4, Hkv=2, D=8, Di=4, seq_lens=[13, 7], P=12,
                           k=2, fp8=False, seed=7, B=4)
    case.k_cache = case.k_cache.to(torch.bfloat16)
    case.v_cache = case.v_cache.to(torch.bfloat16)
    topk = synth.random_topk(case, seed=8).numpy()
    got = orc.sparse_decode(case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens,
                            topk, case.T, case.sm_scale, case.k_scale, case.v_scale)
    np.testing.assert_allclose(got, brute_attention(case, topk), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("case", small_cases(), ids=lambda c: c.name)
def test_all_blocks_selected_equals_dense(orc, case):
    topk = np.tile(np.arange(case.MB, dtype=np.int32), (case.N, 1))
    sparse = orc.sparse_decode(case.q, case.k_cache, case.v_cache, case.block_table,
                               case.seq_lens, topk, case.T, case.sm_scale, case.k_scale,
                               case.v_scale)
    dense = orc.dense_attention(case.q, case.k_cache, case.v_cache, case.block_table,
                                case.seq_lens, case.T, case.sm_scale, case.k_scale, case.v_scale)
    np.testing.assert_allclose(sparse, dense, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dense, brute_attention(case, topk), rtol=1e-11, atol=1e-12)


def test_select_matches_brute_force(orc):
    g = np.random.default_rng(9)
    for trial in range(200):
        MB = int(g.integers(1, 40))
        k = int(g.integers(1, 45))
        vals = g.choice([-1.0, 0.0, -0.0, 1.0, 2.5, np.inf, -np.inf, np.nan, 3.0], size=MB)
        vals = np.where(g.random(MB) < 0.5, g.normal(size=MB).round(1), vals)
        got = orc.select_topk(vals[None, :], k)[0]
        cand = [(0.0 if v == 0 else v, j) for j, v in enumerate(vals)
                if not (np.isnan(v) or v == -np.inf)]
        best = sorted(cand, key=lambda x: (-x[0], x[1]))[:k]
        want = sorted(j for _, j in best)
        want = want + [-1] * (k - len(want))
        assert got.tolist() == want, (vals, k)


def test_select_invariants(orc):
    MB = 32
    eq = orc.select_topk(np.full((1, MB), 1.5), 5)[0]
    assert eq.tolist() == [0, 1, 2, 3, 4]                       # ties -> lower ids
    inc = orc.select_topk(np.arange(MB, dtype=np.float64)[None], 4)[0]
    assert inc.tolist() == [28, 29, 30, 31]
    few = np.full((1, MB), -np.inf)
    few[0, [3, 17]] = [2.0, -5.0]
    assert orc.select_topk(few, 4)[0].tolist() == [3, 17, -1, -1]
    z = np.array([[-0.0, 0.0, -0.0]])
    assert orc.select_topk(z, 1)[0].tolist() == [0]            # -0 equals +0
    g = np.random.default_rng(3)
    s = g.normal(size=(50, MB))
    tk = orc.select_topk(s, 7)
    for n in range(50):
        sel = s[n, tk[n]]
        rest = np.delete(s[n], tk[n])
        assert sel.min() >= rest.max()
        assert np.all(np.diff(tk[n]) > 0)


# ------------------------------------------------------------ closed forms

def test_score_one_hot_query(orc):
    case = small_cases()[1]
    for d in range(case.Di):
        qi = torch.zeros_like(case.q_idx, dtype=torch.float32)
        qi[:, d] = 1.0
        got = orc.block_score(qi, case.index_k, case.block_table, case.seq_lens, case.T,
                              case.idx_scale)
        codes = _decode(case.index_k)
        for n in range(case.N):
            r = n // case.T
            vis = case.visible(n)
            for j in range(case.MB):
                lo, hi = j * case.B, min((j + 1) * case.B, vis)
                if lo >= hi:
                    assert got[n, j] == -np.inf
                    continue
                col = codes[int(case.block_table[r, j]), : hi - lo, d]
                assert got[n, j] == col.max() * case.idx_scale


def test_score_constant_codes(orc):
    case = small_cases()[1]
    idx = torch.full_like(case.index_k, 0x40)           # every code = 2.0
    got = orc.block_score(case.q_idx, idx, case.block_table, case.seq_lens, case.T,
                          case.idx_scale)
    qsum = _decode(case.q_idx).sum(axis=1)
    for n in range(case.N):
        for j in range(case.MB):
            if j * case.B < case.visible(n):
                assert got[n, j] == pytest.approx(2.0 * qsum[n] * case.idx_scale, rel=1e-13)
            else:
                assert got[n, j] == -np.inf


def test_score_causal_offset(orc):
    """Token t of a row sees exactly seq_len - (T-1-t) keys."""
    case = synth.make_case("causal", R=1, T=4, Hq=2, Hkv=1, D=4, Di=4, seq_lens=[10], P=4, k=1,
                           fp8=False, seed=1, B=4)
    idx = case.index_k.clone()
    qi = torch.zeros(4, 4)
    qi[:, 0] = 1.0
    for s in range(10):                                 # key s has value s in dim 0
        idx[int(case.block_table[0, s // 4]), s % 4, 0] = float(s)
    got = orc.block_score(qi, idx, case.block_table, case.seq_lens, 4, 1.0)
    # visible counts 7, 8, 9, 10 -> last visible key 6, 7, 8, 9 (block 1 or 2)
    assert got[0].tolist() == [3.0, 6.0, -np.inf]
    assert got[1].tolist() == [3.0, 7.0, -np.inf]
    assert got[2].tolist() == [3.0, 7.0, 8.0]
    assert got[3].tolist() == [3.0, 7.0, 9.0]


def test_golden_score_select(orc):
    g = json.load(open(os.path.join(GOLDEN, "score_select_hand.json")))
    idx = torch.tensor(_arr(g["index_k"]), dtype=torch.float32)
    qi = torch.tensor(g["q_idx"], dtype=torch.float32)
    bt = torch.tensor(g["block_table"], dtype=torch.int32)
    sl = torch.tensor(g["seq_lens"], dtype=torch.int32)
    got = orc.block_score(qi, idx, bt, sl, g["T"], g["idx_scale"])
    want = _arr(g["scores"])
    assert np.array_equal(got, want)
    assert orc.select_topk(got, 1).tolist() == g["topk1"]
    assert orc.select_topk(got, 2).tolist() == g["topk2"]


def test_golden_attention(orc):
    g = json.load(open(os.path.join(GOLDEN, "attention_hand.json")))
    kc = torch.tensor(_arr(g["k_cache"]), dtype=torch.float32)
    vc = torch.tensor(_arr(g["v_cache"]), dtype=torch.float32)
    q = torch.tensor(g["q"], dtype=torch.float32)
    bt = torch.tensor(g["block_table"], dtype=torch.int32)
    sl = torch.tensor(g["seq_lens"], dtype=torch.int32)
    for c in g["cases"]:
        got = orc.sparse_decode(q, kc, vc, bt, sl, np.array(c["topk"], dtype=np.int32), g["T"],
                                math.log(2.0), 1.0, 1.0)
        np.testing.assert_allclose(got, np.array(c["out"]), rtol=1e-14, atol=1e-14)


def _attn(orc, case, topk, **kw):
    a = dict(sm_scale=case.sm_scale, k_scale=case.k_scale, v_scale=case.v_scale)
    a.update(kw)
    return orc.sparse_decode(kw.pop("q", case.q), kw.pop("k_cache", case.k_cache),
                             kw.pop("v_cache", case.v_cache), case.block_table, case.seq_lens,
                             topk, case.T, a["sm_scale"], a["k_scale"], a["v_scale"])


def test_attention_closed_forms(orc):
    case = synth.make_case("cf", R=1, T=1, Hq=4, Hkv=1, D=8, Di=4, seq_lens=[9], P=5, k=3,
                           fp8=True, seed=8, B=4)
    topk = np.array([[0, 2, -1]], dtype=np.int32)          # keys 0..3 and 8
    v = _decode(case.v_cache)
    kc = _decode(case.k_cache)
    pg = case.block_table[0].numpy()
    keys = [(pg[0], s) for s in range(4)] + [(pg[2], 0)]
    base = _attn(orc, case, topk)
    # v_scale doubles -> output doubles exactly
    twice = _attn(orc, case, topk, v_scale=2 * case.v_scale)
    assert np.array_equal(twice, 2 * base)
    # sm_scale = 0 -> plain mean of the selected visible values
    uni = _attn(orc, case, topk, sm_scale=0.0)
    mean = np.mean([v[p, s, 0] for p, s in keys], axis=0) * case.v_scale
    for h in range(4):
        np.testing.assert_allclose(uni[0, h], mean, rtol=1e-13)
    # one visible key (block 2 holds only key 8) -> exactly that value
    one = _attn(orc, case, np.array([[2, -1, -1]], dtype=np.int32))
    for h in range(4):
        assert np.array_equal(one[0, h], v[pg[2], 0, 0] * case.v_scale)
    # identical keys -> weights equal -> mean of the values
    kk = case.k_cache.clone()
    for p, s in keys:
        kk[p, s] = case.k_cache[pg[0], 0]
    same = orc.sparse_decode(case.q, kk, case.v_cache, case.block_table, case.seq_lens, topk,
                             case.T, case.sm_scale, case.k_scale, case.v_scale)
    for h in range(4):
        np.testing.assert_allclose(same[0, h], mean, rtol=1e-13)
    # constant values -> that constant whatever the weights
    vv = case.v_cache.clone()
    vv[:] = 0x38                                          # code 1.0
    const = orc.sparse_decode(case.q, case.k_cache, vv, case.block_table, case.seq_lens, topk,
                              case.T, case.sm_scale, case.k_scale, case.v_scale)
    np.testing.assert_allclose(const, case.v_scale, rtol=1e-14)
    assert np.isfinite(kc[pg[0]]).all()


def test_attention_empty_and_invalid_ids(orc):
    case = small_cases()[1]                              # row 2 has seq_len 0
    topk = np.full((case.N, case.k), -1, dtype=np.int32)
    out = _attn(orc, case, topk)
    assert np.array_equal(out, np.zeros_like(out))
    tk = synth.random_topk(case, seed=3).numpy()
    base = _attn(orc, case, tk)
    odd = tk.copy()
    odd[odd == -1] = case.MB + 7                          # out-of-range ids count as none
    assert np.array_equal(_attn(orc, case, odd), base)
    dup = tk.copy()
    dup[0, 1] = dup[0, 0]
    with pytest.raises(Exception):
        _attn(orc, case, dup)


def test_page_permutation_invariance(orc):
    case = small_cases()[1]
    g = np.random.default_rng(12)
    perm = g.permutation(case.P)                          # new page of old page p = perm[p]
    inv = np.argsort(perm)

    def move(pool):
        return pool[torch.from_numpy(inv)]

    bt2 = torch.from_numpy(perm[case.block_table.numpy()].astype(np.int32))
    s1 = orc.block_score(case.q_idx, case.index_k, case.block_table, case.seq_lens, case.T,
                         case.idx_scale)
    s2 = orc.block_score(case.q_idx, move(case.index_k), bt2, case.seq_lens, case.T,
                         case.idx_scale)
    assert np.array_equal(s1, s2)
    tk = orc.select_topk(s1, case.k)
    o1 = orc.sparse_decode(case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens,
                           tk, case.T, case.sm_scale, case.k_scale, case.v_scale)
    o2 = orc.sparse_decode(case.q, move(case.k_cache), move(case.v_cache), bt2, case.seq_lens,
                           tk, case.T, case.sm_scale, case.k_scale, case.v_scale)
    assert np.array_equal(o1, o2)


def test_round_bf16_matches_torch(orc):
    g = np.random.default_rng(1)
    x = np.concatenate([g.normal(size=5000) * 0.05, g.normal(size=5000) * 30])
    x32 = x.astype(np.float32).astype(np.float64)      # exactly representable in f32
    ref = torch.from_numpy(x32).to(torch.float32).to(torch.bfloat16).double().numpy()
    assert np.array_equal(orc.round_bf16(x32), ref)
    m = x32[:6000].reshape(60, 100)
    assert np.array_equal(orc.round_bf16(m.T), ref[:6000].reshape(60, 100).T)   # strided input


# ------------------------------------------- ragged prefill score + select

def _pb_dense_keys(pb, b):
    """Request b's keys in position order, decoded, [L, Di]."""
    arr = _decode(pb.index_k)
    L = int(pb.seq_lens[b])
    pages = pb.block_table[int(pb.slot_ids[b])].numpy()
    idx = np.arange(L)
    return arr[pages[idx // pb.B], idx % pb.B]


def brute_prefill_select(pb):
    """Dense numpy route: per (head, query block) a masked [block tokens x keys]
    dot matrix, block maxima by reshaping, then the forced-then-by-score rule."""
    q = _decode(pb.q)
    out = np.full((pb.Hq, pb.all_qb, pb.topk), -1, dtype=np.int32)
    for b in range(pb.batch):
        q0, q1 = int(pb.cu_seqlens[b]), int(pb.cu_seqlens[b + 1])
        nq = q1 - q0
        K = _pb_dense_keys(pb, b)
        for qb in range((nq + pb.block_size_q - 1) // pb.block_size_q):
            V = min(int(pb.seq_lens[b]), int(pb.prefix_lens[b]) + qb * pb.block_size_q)
            ncand = -(-V // pb.B)
            t0, t1 = q0 + qb * pb.block_size_q, min(q1, q0 + (qb + 1) * pb.block_size_q)
            for h in range(pb.Hq):
                dots = q[t0:t1, h] @ K[:V].T                                  # [tokens, V]
                pad = ncand * pb.B - V
                dots = np.concatenate([dots, np.full((t1 - t0, pad), -np.inf)], axis=1)
                sc = pb.scale * dots.reshape(t1 - t0, ncand, pb.B).max(axis=(0, 2))
                forced = [j for j in range(ncand) if j < pb.init_blocks or j >= ncand - pb.local_blocks]
                chosen = forced[:pb.topk]
                rest = sorted((j for j in range(ncand) if j not in forced), key=lambda j: (-sc[j], j))
                chosen += rest[:pb.topk - len(chosen)]
                chosen = sorted(chosen)
                out[h, int(pb.cu_seqblocks_q[b]) + qb, :len(chosen)] = chosen
    return out


def _tiny_batches():
    return [
        synth.prefill_batch("pb_fp8", new_tokens=[5, 3, 8], prefix=[6, 0, 11], Hq=2, Di=4,
                            block_size_q=3, topk=3, init_blocks=1, local_blocks=1, B=4, seed=11,
                            extra_qb_rows=2),
        synth.prefill_batch("pb_f32", new_tokens=[9, 1], prefix=[30, 2], Hq=3, Di=8,
                            block_size_q=4, topk=4, init_blocks=0, local_blocks=2, B=4, seed=12,
                            fp8=False),
        synth.prefill_batch("pb_bsq1", new_tokens=[6, 4], prefix=[17, 9], Hq=1, Di=4,
                            block_size_q=1, topk=2, B=4, seed=13),
    ]


@pytest.mark.parametrize("pb", _tiny_batches(), ids=lambda p: p.name)
def test_prefill_select_matches_brute_force(orc, pb):
    got, sc = orc.prefill_select(pb.q, pb.index_k, pb.block_table, pb.slot_ids, pb.cu_seqlens,
                                 pb.seq_lens, pb.prefix_lens, pb.block_size_q, pb.topk,
                                 pb.init_blocks, pb.local_blocks, pb.scale, pb.cu_seqblocks_q,
                                 pb.all_qb, return_scores=True)
    assert np.array_equal(got, brute_prefill_select(pb))
    assert (got[:, int(pb.cu_seqblocks_q[-1]):] == -1).all()      # rows no query block owns


def test_prefill_select_one_token_blocks_equal_per_token_path(orc):
    """1-token query blocks, one head, no forced blocks: the per-token score and
    select of the decode rows whose visibility is the same key range (a decode
    token sees its own key, a query block only the keys before it: seq_len =
    prefix + T - 1), through the independent per-token oracle functions."""
    T, R = 6, 3
    pb = synth.prefill_batch("pb_eq", new_tokens=[T] * R, prefix=[40, 3, 77], Hq=1, Di=8,
                             block_size_q=1, topk=4, B=8, seed=14)
    got = orc.prefill_select(pb.q, pb.index_k, pb.block_table, pb.slot_ids, pb.cu_seqlens,
                             pb.seq_lens, pb.prefix_lens, 1, pb.topk, 0, 0, pb.scale,
                             pb.cu_seqblocks_q, pb.all_qb)[0]
    bt = pb.block_table[pb.slot_ids.long()].contiguous()
    lens = (pb.prefix_lens + T - 1).to(torch.int32)
    scores = orc.block_score(pb.q[:, 0, :].contiguous(), pb.index_k, bt, lens, T, pb.scale)
    ref = orc.select_topk(scores, pb.topk)
    assert np.array_equal(got, ref)


def test_prefill_select_forced_blocks(orc):
    """topk <= forced blocks: exactly the forced blocks, lower ids first;
    topk >= candidates: every candidate."""
    base = dict(new_tokens=[8, 5], prefix=[33, 21], Hq=2, Di=4, block_size_q=2, B=4, seed=15)
    pb = synth.prefill_batch("pb_forced", topk=3, init_blocks=2, local_blocks=3, **base)
    got = orc.prefill_select(pb.q, pb.index_k, pb.block_table, pb.slot_ids, pb.cu_seqlens,
                             pb.seq_lens, pb.prefix_lens, pb.block_size_q, pb.topk, pb.init_blocks,
                             pb.local_blocks, pb.scale, pb.cu_seqblocks_q, pb.all_qb)
    for b in range(pb.batch):
        for qb in range(int(pb.cu_seqblocks_q[b + 1] - pb.cu_seqblocks_q[b])):
            V = min(int(pb.seq_lens[b]), int(pb.prefix_lens[b]) + qb * pb.block_size_q)
            ncand = -(-V // pb.B)
            forced = sorted({j for j in range(ncand) if j < 2 or j >= ncand - 3})[:3]
            for h in range(pb.Hq):
                row = got[h, int(pb.cu_seqblocks_q[b]) + qb]
                assert list(row[row >= 0]) == forced
    pb = synth.prefill_batch("pb_all", topk=40, init_blocks=1, local_blocks=1, **base)
    got = orc.prefill_select(pb.q, pb.index_k, pb.block_table, pb.slot_ids, pb.cu_seqlens,
                             pb.seq_lens, pb.prefix_lens, pb.block_size_q, pb.topk, pb.init_blocks,
                             pb.local_blocks, pb.scale, pb.cu_seqblocks_q, pb.all_qb)
    for b in range(pb.batch):
        for qb in range(int(pb.cu_seqblocks_q[b + 1] - pb.cu_seqblocks_q[b])):
            V = min(int(pb.seq_lens[b]), int(pb.prefix_lens[b]) + qb * pb.block_size_q)
            row = got[0, int(pb.cu_seqblocks_q[b]) + qb]
            assert list(row[row >= 0]) == list(range(-(-V // pb.B)))


def test_prefill_select_row_mask_computes_only_marked_rows(orc):
    """The row mask (used to sample large batches) changes no computed row:
    marked rows equal the unmasked call's, unmarked rows stay -1 / -inf."""
    pb = _tiny_batches()[0]
    args = (pb.q, pb.index_k, pb.block_table, pb.slot_ids, pb.cu_seqlens, pb.seq_lens,
            pb.prefix_lens, pb.block_size_q, pb.topk, pb.init_blocks, pb.local_blocks, pb.scale,
            pb.cu_seqblocks_q, pb.all_qb)
    full, fsc = orc.prefill_select(*args, return_scores=True)
    mask = np.random.default_rng(16).random((pb.Hq, pb.all_qb)) < 0.5
    got, sc = orc.prefill_select(*args, return_scores=True, rows=mask, threads=2)
    assert np.array_equal(got[mask], full[mask]) and np.array_equal(sc[mask], fsc[mask])
    assert (got[~mask] == -1).all() and np.isneginf(sc[~mask]).all()


@pytest.mark.parametrize("case", small_cases(), ids=lambda c: c.name)
def test_per_request_score_matches_brute_force(orc, case):
    """One sheet row per request (the max over the request's tokens), against a
    dense route that takes the max over the tokens first and over each block's
    keys second."""
    got = orc.block_score_per_row(case.q_idx, case.index_k, case.block_table, case.seq_lens, case.T,
                                  case.idx_scale)
    qi = _decode(case.q_idx)
    ref = np.full((case.R, case.MB), -np.inf)
    for r in range(case.R):
        L = int(case.seq_lens[r])
        if L == 0:
            continue
        K = _dense_keys(case, case.index_k, r)
        rows = range(r * case.T, (r + 1) * case.T)
        dots = qi[list(rows)] @ K.T
        vis = np.array([case.visible(n) for n in rows])
        dots = np.where(np.arange(L)[None, :] < vis[:, None], dots, -np.inf).max(axis=0)   # [L]
        dots = np.concatenate([dots, np.full(case.MB * case.B - L, -np.inf)])
        ref[r] = dots.reshape(case.MB, case.B).max(axis=1) * case.idx_scale
    assert got.shape == (case.R, case.MB)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref))
    fin = np.isfinite(ref)
    assert np.allclose(got[fin], ref[fin], rtol=1e-12, atol=1e-12)


def test_attention_per_request_selection(orc):
    """A selection per request ([R, K], and [Hkv, R, K]) is attended by every
    token of the request, each with its own visibility: the brute-force route
    with the rows repeated per token."""
    case = synth.make_case("per_row", R=3, T=3, Hq=4, Hkv=2, D=8, Di=4, seq_lens=[21, 9, 14], P=16,
                           k=3, fp8=True, seed=17, B=4)
    rng = np.random.default_rng(18)
    rows = np.stack([rng.choice(case.MB, size=case.k, replace=False) for _ in range(case.R)]).astype(np.int32)
    got = _attn(orc, case, rows)
    ref = brute_attention(case, np.repeat(rows, case.T, axis=0))
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)
    per_head = np.stack([rows, rows[::-1].copy()])
    got = _attn(orc, case, per_head)
    ref = brute_attention(case, np.repeat(per_head, case.T, axis=1))
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)
