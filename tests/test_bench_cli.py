"""CPU tests of bench.py's host logic: the one-GPU guard and the byte model
the roofline figures divide by (worked by hand on a two-block case)."""
import os
import subprocess
import sys

import numpy as np

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout


def test_algorithmic_bytes_by_hand():
    import bench
    # one row, two tokens, 200 cached tokens = blocks 0 (128 tokens) and 1 (72)
    c = synth.small_fp8(R=1, T=2, lens=(200,), k=2, D=128, Di=128, Hq=16)
    assert (c.MB, c.N, c.Hkv) == (2, 2, 1)
    topk = np.array([[0, 1], [1, -1]], dtype=np.int32)     # union {0, 1}: 200 tokens
    ab = bench.algorithmic_bytes(c, topk)
    index = 200 * 128                    # every cached token's index row, 1 byte per dim
    kv = 200 * 128 * 2                   # K and V rows of the union's tokens
    q_idx = 2 * 128 * 2                  # bf16 index queries
    qo = 2 * 16 * 128 * 2 * 2            # bf16 queries in, bf16 output out
    sheet = 2 * 2 * 4                    # [N, MB] fp32 scores
    sel = 2 * 2 * 4                      # [N, k] int32 ids
    paging = 2 * 4 + 4                   # block table row + seq_len
    assert ab["index"] == index and ab["kv"] == kv
    assert ab["score"] == index + q_idx + sheet + paging
    assert ab["select"] == sheet + sel
    assert ab["decode"] == kv + qo + sel + paging
    assert ab["select_decode"] == kv + qo + sheet + sel + paging
    assert ab["step"] == ab["score"] + ab["select_decode"]


def test_copies_time_the_requested_steps():
    import bench
    # 20 timed steps after 5 warmup steps are run exactly
    assert bench.plan_copies(20, 5) == (5, 20, 5)
    assert bench.plan_copies(400, 40) == (8, 400, 40)
    for steps, warm in [(20, 5), (24, 6), (7, 0), (2000, 200), (17, 3), (1, 1)]:
        m, s, w = bench.plan_copies(steps, warm)
        assert m >= 5 and s % m == 0 and w % m == 0      # >= 5 cold copies, whole replays
        assert s >= steps and w >= warm                   # never fewer than asked
        if any(steps % c == 0 and warm % c == 0 for c in range(5, 17)):
            assert (s, w) == (steps, warm)


def test_short_kernel_names():
    """The trace summary keys kernels by name without return type, namespaces
    and argument list, whichever form rocprofv3 prints."""
    import bench
    full = "void msa::(anonymous namespace)::attn_token_select_kernel<128, 2>(msa::AttnParams)"
    assert bench.short_kernel_name(full) == "attn_token_select_kernel<128, 2>"
    assert bench.short_kernel_name("attn_token_select_kernel<128, 2>(msa::AttnParams)") == \
        "attn_token_select_kernel<128, 2>"
    assert bench.short_kernel_name("(anonymous namespace)::stream_read_kernel(unsigned int __vector(4) "
                                   "const*, long, unsigned int*)") == "stream_read_kernel"
    assert bench.short_kernel_name("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"
