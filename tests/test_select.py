"""GPU tests of the top-k block selection on crafted score sheets.

Both selection paths -- the top-k kernel (msa_select_topk) and the selection
the attention launch makes itself (msa_select_sparse_decode, MB <= 128) -- must
equal the oracle's selection bit for bit: the k largest scores, ties to the
lower block id, NaN and -inf never selected, -0 equal to +0, ids ascending,
-1 after the candidates run out.  The sheets stress the byte-wise radix select:
ties inside and across its bins, keys differing only in the low byte,
negative and infinite scores, subnormals, k = 1 and k = MB.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from msa_harness import poisoned, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def msa():
    import block_sparse_paged_amd as m
    return m


def sheets(N: int, MB: int, seed: int):
    """Named float32 score sheets [N, MB]."""
    rng = np.random.default_rng([seed, MB])
    out = {"normal": rng.standard_normal((N, MB)).astype(np.float32)}
    out["few_values"] = rng.integers(0, 3, (N, MB)).astype(np.float32)       # ties everywhere
    out["all_equal"] = np.full((N, MB), 0.75, dtype=np.float32)
    base = np.float32(1.0)
    ulps = rng.permutation(np.arange(N * MB)).reshape(N, MB) % 200           # low-byte keys
    out["low_byte"] = (base.view(np.int32) + ulps.astype(np.int32)).view(np.float32)
    mixed = rng.standard_normal((N, MB)).astype(np.float32)
    mask = rng.random((N, MB))
    mixed[mask < 0.15] = np.nan
    mixed[(mask >= 0.15) & (mask < 0.3)] = -np.inf
    mixed[(mask >= 0.3) & (mask < 0.35)] = np.inf
    mixed[(mask >= 0.35) & (mask < 0.45)] = 0.0
    mixed[(mask >= 0.45) & (mask < 0.55)] = -0.0
    mixed[(mask >= 0.55) & (mask < 0.6)] = np.float32(1e-42)                 # subnormal
    out["special"] = mixed
    sparse = np.full((N, MB), -np.inf, dtype=np.float32)                     # < k candidates
    for n in range(N):
        cols = rng.choice(MB, size=min(MB, 1 + n % 5), replace=False)
        sparse[n, cols] = rng.standard_normal(cols.size)
    out["few_candidates"] = sparse
    out["negative"] = -np.abs(rng.standard_normal((N, MB))).astype(np.float32) - 1.0
    return out


def oracle_topk(sheet: np.ndarray, k: int) -> np.ndarray:
    return oracle.select_topk(sheet.astype(np.float64), k)


@pytest.mark.parametrize("MB", [1, 7, 64, 65, 128, 129, 300, 1024, 2048])
def test_topk_kernel_on_crafted_sheets(msa, MB):
    N = 12
    for name, sheet in sheets(N, MB, seed=41).items():
        for k in sorted({1, min(MB, 16), min(MB, 37), MB}):
            print(f"MB {MB} sheet {name} k {k}", flush=True)
            s = torch.from_numpy(sheet).cuda()
            t = poisoned((N, k), torch.int32)
            msa.msa_select_topk(s, k, t)
            torch.cuda.synchronize()
            got = t.cpu().numpy()
            ref = oracle_topk(sheet, k)
            bad = np.nonzero((got != ref).any(axis=1))[0]
            assert bad.size == 0, f"{name} k={k}: rows {bad[:6]} got {got[bad[0]]} want {ref[bad[0]]}"


@pytest.mark.parametrize("MB", [5, 64, 128])
def test_selection_inside_attention_on_crafted_sheets(msa, MB):
    """msa_select_sparse_decode's own selection equals the oracle's, and its
    output equals msa_sparse_decode's over that selection."""
    R, T = 3, 4
    lens = (MB * 128, max(1, MB * 128 - 77), max(1, MB * 64))
    c = synth.small_fp8(R=R, T=T, lens=lens, k=min(16, MB), seed=43)
    assert c.MB == MB
    d = upload(c)
    ws = torch.zeros(msa.msa_sparse_decode_workspace_bytes(c.R, c.T, c.Hq, c.Hkv, c.D, c.k),
                     dtype=torch.uint8, device="cuda")
    for name, sheet in sheets(c.N, MB, seed=44).items():
        print(f"MB {MB} sheet {name}", flush=True)
        s = torch.from_numpy(sheet).cuda()
        t = poisoned((c.N, c.k), torch.int32)
        out = poisoned((c.N, c.Hq, c.D), torch.bfloat16)
        msa.msa_select_sparse_decode(s, c.k, t, d.q, d.k_cache, d.v_cache, d.block_table,
                                     d.seq_lens, c.T, out, c.sm_scale, c.k_scale, c.v_scale, c.B, ws)
        torch.cuda.synchronize()
        got = t.cpu().numpy()
        ref = oracle_topk(sheet, c.k)
        assert np.array_equal(got, ref), f"{name}: selection differs from the oracle"
        out2 = poisoned((c.N, c.Hq, c.D), torch.bfloat16)
        msa.msa_sparse_decode(d.q, d.k_cache, d.v_cache, d.block_table, d.seq_lens, t, c.T, out2,
                              c.sm_scale, c.k_scale, c.v_scale, c.B, ws)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), f"{name}: outputs differ"
