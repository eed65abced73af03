"""msa_decode_step_noalloc (the step for callers that cannot allocate: its
scratch is a device array inside the library) against msa_decode_step with a
caller workspace: bit-identical scores, topk_idx and out on two calls in a
row, the second on a smaller batch (the array keeps the first call's data),
and sizes beyond the array are rejected before anything is enqueued."""
import sys

import pytest
import torch

import synth
from msa_harness import poisoned, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def msa():
    import block_sparse_paged_amd as m
    return m


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _outputs(c):
    return (poisoned((c.N, c.MB), torch.float32), poisoned((c.N, c.k), torch.int32),
            poisoned((c.N, c.Hq, c.D), torch.bfloat16))


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a, b)


def _with_workspace(msa, c, d):
    s, t, o = _outputs(c)
    ws = torch.zeros(msa.msa_decode_step_workspace_bytes(c.R, c.T, c.Hq, c.Hkv, c.D, c.k),
                     dtype=torch.uint8, device="cuda")
    msa.msa_decode_step(d.q_idx, d.index_k, d.q, d.k_cache, d.v_cache, d.block_table, d.seq_lens,
                        c.T, c.k, c.B, c.idx_scale, c.sm_scale, c.k_scale, c.v_scale, s, t, o, ws)
    return s, t, o


def _noalloc(msa, c, d):
    s, t, o = _outputs(c)
    msa.msa_decode_step_noalloc(d.q_idx, d.index_k, d.q, d.k_cache, d.v_cache, d.block_table,
                                d.seq_lens, c.T, c.k, c.B, c.idx_scale, c.sm_scale, c.k_scale,
                                c.v_scale, s, t, o)
    return s, t, o


def test_noalloc_matches_workspace_step_twice(msa):
    cases = [synth.hbm_decode(128, seed=5991),                      # row-level plan, ~8 MiB of partials
             synth.hbm_decode(16, seed=5990),                       # 16 rows, the bench shape
             synth.small_fp8(R=3, T=4, lens=(900, 5000, 130), k=6, seed=77)]   # then smaller
    for c in cases:
        _say(f"case {c.name}: R={c.R} T={c.T} k={c.k} MB={c.MB}")
        d = upload(c)
        ref = _with_workspace(msa, c, d)
        got = _noalloc(msa, c, d)
        torch.cuda.synchronize()
        for name, a, b in zip(("scores", "topk_idx", "out"), ref, got):
            assert _same(a, b), f"{c.name}: {name} differs from msa_decode_step"
    # a third call at the first size again: the counters the second call left are zero
    c = cases[0]
    d = upload(c)
    ref = _with_workspace(msa, c, d)
    got = _noalloc(msa, c, d)
    torch.cuda.synchronize()
    assert all(_same(a, b) for a, b in zip(ref, got))


def test_noalloc_rejects_sizes_beyond_its_scratch(msa):
    # 1024 rows x 4 tokens x 16 heads x 128 dims of split partials: > 16 MiB
    R, T, MB, P, k = 1024, 4, 1, 4, 1
    assert msa.msa_decode_step_workspace_bytes(R, T, 16, 1, 128, k) > (16 << 20)
    f8 = torch.float8_e4m3fn
    q_idx = torch.zeros((R * T, 128), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros((P, 128, 128), dtype=torch.uint8, device="cuda").view(f8)
    q = torch.zeros((R * T, 16, 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((P, 128, 1, 128), dtype=torch.uint8, device="cuda").view(f8)
    bt = torch.zeros((R, MB), dtype=torch.int32, device="cuda")
    sl = torch.ones((R,), dtype=torch.int32, device="cuda")
    s = poisoned((R * T, MB), torch.float32)
    t = poisoned((R * T, k), torch.int32)
    o = poisoned((R * T, 16, 128), torch.bfloat16)
    with pytest.raises(msa.MsaError) as e:
        msa.msa_decode_step_noalloc(q_idx, idx, q, kc, kc, bt, sl, T, k, 128, 1.0, 0.088, 1.0, 1.0,
                                    s, t, o)
    assert e.value.code == 9
    torch.cuda.synchronize()
    assert torch.isnan(s).all() and (t == -7777).all() and torch.isnan(o.float()).all()
