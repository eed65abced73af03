"""Planted mistakes in the oracle must each fail the oracle's pins.

Each mutant is a copy of ``oracle/msa_oracle.c`` with one plausible mistake
(a dropped term, a wrong sign or index, a wrong constant), compiled to a
temporary library and run under ``tests/test_oracle.py`` in a child process.
A mutant that survives means the pins would not have caught that mistake.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "msa_oracle.c")

# (name, exact text, replacement, which occurrence (0-based))
MUTANTS = [
    ("visibility_off_by_one", "(T - 1 - t)", "(T - t)", 0),
    ("dot_drops_first_dim", "for (int64_t d = 0; d < Di; d++)", "for (int64_t d = 1; d < Di; d++)", 0),
    ("score_drops_idx_scale", "best *= idx_scale;", "best *= 1.0;", 0),
    ("score_uses_row_query", "elem(q_idx, q_dtype, n * Di + d)", "elem(q_idx, q_dtype, (n / T) * T * Di + d)", 0),
    ("select_ties_to_higher_id", "return (x->j > y->j) - (x->j < y->j);", "return (x->j < y->j) - (x->j > y->j);", 0),
    ("select_keeps_neg_inf", "if (isnan(s) || s == -INFINITY)", "if (isnan(s))", 0),
    ("select_takes_k_minus_1", "int64_t take = nc < k ? nc : k;", "int64_t take = nc < k ? nc : k - 1;", 0),
    ("attn_drops_k_scale", "logit[e] = sm_scale * k_scale * dot;", "logit[e] = sm_scale * dot;", 0),
    ("attn_drops_v_scale", "out[qoff + d] = nkeys ? v_scale * acc[d] / denom : 0.0;", "out[qoff + d] = nkeys ? acc[d] / denom : 0.0;", 0),
    ("attn_wrong_gqa_head", "int64_t g = h / G;", "int64_t g = h % Hkv;", 0),
    ("attn_ignores_visibility", "int64_t lo = j * B, hi = (j + 1) * B < vis ? (j + 1) * B : vis;", "int64_t lo = j * B, hi = (j + 1) * B;", 1),
    ("attn_transposed_value_index", "acc[d] += p * elem(v_cache, kv_dtype, voff + d);", "acc[d] += p * elem(v_cache, kv_dtype, voff + (D - 1 - d));", 0),
    ("e4m3_wrong_bias", "v = ldexp(1.0 + m / 8.0, e - 7);", "v = ldexp(1.0 + m / 8.0, e - 8);", 0),
    ("e4m3_wrong_subnormal", "v = ldexp((double)m, -9);", "v = ldexp((double)m, -10);", 0),
    ("bf16_wrong_half", "uint32_t u = (uint32_t)bits << 16;", "uint32_t u = (uint32_t)bits << 15;", 0),
    ("prefill_sees_own_block", "int64_t V = (int64_t)prefix_lens[b] + qb * bsq;", "int64_t V = (int64_t)prefix_lens[b] + (qb + 1) * bsq;", 0),
    ("prefill_block_max_first_token", "for (int64_t t = qb * bsq; t < t1; t++)", "for (int64_t t = qb * bsq; t < qb * bsq + 1; t++)", 0),
    ("prefill_wrong_head", "elem(q, q_dtype, ((q0 + t) * Hq + h) * Di + d)", "elem(q, q_dtype, ((q0 + t) * Hq) * Di + d)", 0),
    ("prefill_local_off_by_one", "forced[j] = (j < init_blocks) || (j >= ncand - local_blocks);", "forced[j] = (j < init_blocks) || (j > ncand - local_blocks);", 0),
    ("prefill_drops_init", "forced[j] = (j < init_blocks) || (j >= ncand - local_blocks);", "forced[j] = (j >= ncand - local_blocks);", 0),
    ("prefill_ignores_slot", "const int64_t page = block_table[slot * MB + j];", "const int64_t page = block_table[b * MB + j];", 0),
]


def _mutate(text, old, new, occ):
    pos = -1
    for _ in range(occ + 1):
        pos = text.find(old, pos + 1)
        assert pos >= 0, f"mutation anchor not found: {old!r}"
    return text[:pos] + new + text[pos + len(old):]


@pytest.mark.parametrize("name,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_killed(tmp_path, name, old, new, occ):
    src = open(SRC).read()
    mutated = _mutate(src, old, new, occ)
    assert mutated != src
    c = tmp_path / "mut.c"
    c.write_text(mutated)
    so = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", str(so), str(c), "-lm"],
                   check=True)
    env = dict(os.environ, MSA_ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the oracle pins:\n{r.stdout[-2000:]}"
