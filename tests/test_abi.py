"""The C-ABI library on the host (no GPU needed): it loads, exports every entry
point ``include/msa.h`` declares, sizes its workspace from the sizes alone, and
rejects out-of-domain descriptors before launching anything -- the outputs keep
their poison and the error code says why.  No compute call is made here."""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def msa():
    import block_sparse_paged_amd as m
    return m


def header_functions():
    text = open(os.path.join(ROOT, "include", "msa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(msa):
    names = header_functions()
    assert set(names) == set(msa.EXPORTS)
    for name in names:
        assert hasattr(msa.lib, name), name
    nm = os.popen(f"nm -D --defined-only {msa.LIB_PATH}").read()
    for name in names:
        assert re.search(rf"\bT {name}\b", nm), f"{name} not exported"


def test_error_strings(msa):
    for code in range(0, 11):
        s = msa.lib.msa_error_string(code)
        assert s and isinstance(s, bytes)
    assert msa.lib.msa_get_last_error() == 0


def test_workspace_bytes_depends_on_sizes_only(msa):
    a = msa.msa_sparse_decode_workspace_bytes(16, 4, 16, 1, 128, 16)
    b = msa.msa_sparse_decode_workspace_bytes(16, 4, 16, 1, 128, 16)
    assert a == b and a > 0 and a % 256 == 0
    # 16 splits x 64 tokens x 16 heads x (128 + 2) floats, each section 256-aligned
    assert a >= 16 * 64 * 16 * 130 * 4
    assert msa.msa_sparse_decode_workspace_bytes(0, 0, 16, 1, 128, 16) == 0


def _cpu_case():
    R, T, MB, P, Di, Hq, D, k = 2, 4, 8, 20, 128, 16, 128, 4
    N = R * T
    t = dict(
        q_idx=torch.zeros(N, Di, dtype=torch.bfloat16),
        index_k=torch.zeros(P, 128, Di, dtype=torch.uint8),
        block_table=torch.zeros(R, MB, dtype=torch.int32),
        seq_lens=torch.full((R,), 700, dtype=torch.int32),
        scores=torch.full((N, MB), float("nan")),
        topk=torch.full((N, k), -7, dtype=torch.int32),
        q=torch.zeros(N, Hq, D, dtype=torch.bfloat16),
        k_cache=torch.zeros(P, 128, 1, D, dtype=torch.uint8),
        v_cache=torch.zeros(P, 128, 1, D, dtype=torch.uint8),
        out=torch.full((N, Hq, D), float("nan"), dtype=torch.bfloat16),
        ws=torch.zeros(1 << 20, dtype=torch.uint8),
    )
    return t


def _expect(msa, code, fn, *args):
    with pytest.raises(msa.MsaError) as e:
        fn(*args, stream=0)
    assert e.value.code == code, (e.value, code)
    assert msa.lib.msa_get_last_error() == 0


def test_block_score_rejects(msa):
    c = _cpu_case()
    f = msa.msa_block_score
    base = [c["q_idx"], c["index_k"], c["block_table"], c["seq_lens"], 4, 128, 0.01, c["scores"]]

    def with_(i, v):
        a = list(base)
        a[i] = v
        return a

    _expect(msa, 2, f, *with_(0, c["q_idx"].to(torch.float16)))          # dtype
    _expect(msa, 3, f, *with_(0, c["q_idx"][:, None]))                   # ndim
    _expect(msa, 3, f, *with_(4, 3))                                      # N mismatch
    _expect(msa, 5, f, *with_(5, 64))                                     # block size
    _expect(msa, 7, f, *with_(6, 0.0))                                    # idx_scale
    _expect(msa, 7, f, *with_(6, float("inf")))
    a = with_(1, torch.zeros(20, 128, 96, dtype=torch.uint8))             # Di = 96
    a[0] = torch.zeros(8, 96, dtype=torch.bfloat16)
    _expect(msa, 5, f, *a)
    _expect(msa, 4, f, *with_(1, c["index_k"].transpose(1, 2).contiguous().transpose(1, 2)))
    _expect(msa, 2, f, *with_(7, c["scores"].double()))
    assert torch.isnan(c["scores"]).all()


def test_select_rejects(msa):
    c = _cpu_case()
    _expect(msa, 7, msa.msa_select_topk, c["scores"], 0, c["topk"])
    _expect(msa, 7, msa.msa_select_topk, c["scores"], 9, torch.zeros(8, 9, dtype=torch.int32))
    _expect(msa, 3, msa.msa_select_topk, c["scores"], 3, c["topk"])
    _expect(msa, 2, msa.msa_select_topk, c["scores"].to(torch.bfloat16), 4, c["topk"])
    _expect(msa, 5, msa.msa_select_topk, torch.zeros(2, 4096), 4, torch.zeros(2, 4, dtype=torch.int32))
    assert (c["topk"] == -7).all()


def test_sparse_decode_rejects(msa):
    c = _cpu_case()
    f = msa.msa_sparse_decode
    base = [c["q"], c["k_cache"], c["v_cache"], c["block_table"], c["seq_lens"], c["topk"], 4,
            c["out"], 0.088, 0.01, 0.01, 128, c["ws"]]

    def with_(i, v):
        a = list(base)
        a[i] = v
        return a

    _expect(msa, 6, f, *with_(12, None))                                  # no workspace
    _expect(msa, 6, f, *with_(12, c["ws"][:1024]))                        # too small
    _expect(msa, 6, f, *with_(12, c["ws"][1:]))                           # misaligned
    _expect(msa, 2, f, *with_(2, c["v_cache"].view(torch.int8).float()))  # K/V dtypes differ
    _expect(msa, 3, f, *with_(0, c["q"][:, :15]))                         # Hq mismatch vs out
    a = with_(0, torch.zeros(8, 16, 96, dtype=torch.bfloat16))            # head dim 96
    a[1] = a[2] = torch.zeros(20, 128, 1, 96, dtype=torch.uint8)
    a[7] = torch.zeros(8, 16, 96, dtype=torch.bfloat16)
    _expect(msa, 5, f, *a)
    _expect(msa, 5, f, *with_(11, 256))                                   # block size
    _expect(msa, 7, f, *with_(8, float("nan")))                           # sm_scale
    _expect(msa, 4, f, *with_(1, torch.zeros(20, 128, 1, 256, dtype=torch.uint8)[..., ::2]))
    _expect(msa, 3, f, *with_(3, None))                                   # empty descriptor
    # a NULL descriptor pointer through the raw C entry point
    dt = msa.tensor_desc(c["topk"])
    msa.lib.msa_select_topk(None, 4, ctypes.byref(dt), None)
    assert msa.lib.msa_get_last_error() == 1
    assert torch.isnan(c["out"].float()).all()


def test_select_sparse_decode_rejects(msa):
    c = _cpu_case()
    f = msa.msa_select_sparse_decode
    base = [c["scores"], 4, c["topk"], c["q"], c["k_cache"], c["v_cache"], c["block_table"],
            c["seq_lens"], 4, c["out"], 0.088, 0.01, 0.01, 128, c["ws"]]

    def with_(i, v):
        a = list(base)
        a[i] = v
        return a

    _expect(msa, 7, f, *with_(1, 0))                                      # k < 1
    _expect(msa, 3, f, *with_(2, torch.zeros(8, 3, dtype=torch.int32)))   # topk width != k
    _expect(msa, 3, f, *with_(0, torch.zeros(8, 9)))                      # scores width != MB
    _expect(msa, 3, f, *with_(0, torch.zeros(6, 8)))                      # scores rows != N
    _expect(msa, 6, f, *with_(14, c["ws"][:1024]))                        # workspace too small
    _expect(msa, 2, f, *with_(0, c["scores"].double()))
    assert (c["topk"] == -7).all() and torch.isnan(c["out"].float()).all()


def test_decode_step_rejects(msa):
    c = _cpu_case()
    f = msa.msa_decode_step
    base = [c["q_idx"], c["index_k"], c["q"], c["k_cache"], c["v_cache"], c["block_table"],
            c["seq_lens"], 4, 4, 128, 0.01, 0.088, 0.01, 0.01, c["scores"], c["topk"], c["out"],
            c["ws"]]

    def with_(i, v):
        a = list(base)
        a[i] = v
        return a

    _expect(msa, 3, f, *with_(3, torch.zeros(21, 128, 1, 128, dtype=torch.uint8)))  # pool sizes differ
    _expect(msa, 7, f, *with_(8, 9))                                      # k > MB
    _expect(msa, 6, f, *with_(17, c["ws"][:1024]))
    _expect(msa, 5, f, *with_(9, 64))                                     # block size
    assert torch.isnan(c["scores"]).all() and (c["topk"] == -7).all()
    assert torch.isnan(c["out"].float()).all()


def test_prefill_workspace_bytes(msa):
    f = msa.msa_prefill_block_score_workspace_bytes
    a = f(4, 4, 80, 104, 64)
    assert a == f(4, 4, 80, 104, 64) and a > 0 and a % 256 == 0
    assert a >= 4 * 80 * 104 * 4                      # the query-block score sheet
    # query blocks longer than a chunk keep one sheet per 512-token part
    assert f(1, 2, 3, 10, 2048) >= 2 * 3 * 4 * 10 * 4
    assert f(4, 0, 80, 104, 64) == 0 and f(4, 4, 80, 0, 64) == 0 and f(4, 4, 80, 104, 0) == 0


def test_prefill_block_score_rejects(msa):
    batch, total_q, Hq, Di, P, MB, all_qb, k = 2, 100, 4, 128, 20, 8, 3, 4
    i32 = lambda *s: torch.zeros(*s, dtype=torch.int32)
    out = torch.full((Hq, all_qb, k), -7, dtype=torch.int32)
    ws = torch.zeros(1 << 20, dtype=torch.uint8)
    base = [torch.zeros(total_q, Hq, Di, dtype=torch.bfloat16),
            torch.zeros(P, 128, Di, dtype=torch.uint8), i32(3, MB), i32(batch), i32(batch + 1),
            i32(batch), i32(batch), 64, 128, k, 1, 2, 0.05, i32(batch + 1), out, ws]
    f = msa.msa_prefill_block_score

    def with_(i, v):
        a = list(base)
        a[i] = v
        return a

    _expect(msa, 2, f, *with_(0, base[0].float()))                        # q must be bf16
    _expect(msa, 2, f, *with_(1, base[1].float()))                        # index must be FP8
    _expect(msa, 2, f, *with_(3, torch.zeros(batch, dtype=torch.int64)))  # int32 offsets
    _expect(msa, 3, f, *with_(4, i32(batch)))                             # cu_seqlens [batch+1]
    _expect(msa, 3, f, *with_(13, i32(batch + 2)))                        # cu_seqblocks_q
    _expect(msa, 3, f, *with_(9, k + 1))                                  # topk vs out width
    _expect(msa, 3, f, *with_(14, torch.zeros(Hq + 1, all_qb, k, dtype=torch.int32)))
    a = with_(0, torch.zeros(total_q, Hq, 32, dtype=torch.bfloat16))     # Di = 32
    a[1] = torch.zeros(P, 128, 32, dtype=torch.uint8)
    _expect(msa, 5, f, *a)
    _expect(msa, 5, f, *with_(8, 64))                                     # block_size_k
    _expect(msa, 5, f, *with_(2, i32(3, 4096)))                           # MB > 2048
    _expect(msa, 7, f, *with_(7, 0))                                      # block_size_q
    _expect(msa, 7, f, *with_(10, -1))                                    # init_blocks
    _expect(msa, 7, f, *with_(11, -1))                                    # local_blocks
    _expect(msa, 7, f, *with_(12, 0.0))                                   # scale
    _expect(msa, 7, f, *with_(12, float("nan")))
    _expect(msa, 4, f, *with_(0, torch.zeros(total_q, Hq, 2 * Di, dtype=torch.bfloat16)[..., ::2]))
    _expect(msa, 6, f, *with_(15, None))                                  # no workspace
    _expect(msa, 6, f, *with_(15, ws[:256]))                              # too small
    _expect(msa, 6, f, *with_(15, ws[1:]))                                # misaligned
    assert (out == -7).all()


def test_build_refuses_scratch_memory():
    """The build reads the compiler's resource remarks and names every kernel
    given scratch memory (the attention kernels count their own loads in the
    wave's queue, which scratch accesses would join)."""
    from block_sparse_paged_amd.build import scratch_users
    remarks = "\n".join([
        "a.hip:1:1: remark: Function Name: kern_a [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark: Function Name: kern_b [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark:     VGPRs: 256 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark:     ScratchSize [bytes/lane]: 560 [-Rpass-analysis=kernel-resource-usage]",
    ])
    assert scratch_users(remarks) == [("kern_b", 560)]
