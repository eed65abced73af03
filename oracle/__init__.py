"""CPU oracle for MSA sparse-layer decode attention -- TEST INFRASTRUCTURE ONLY.

A ctypes wrapper around ``msa_oracle.c`` (plain C, double precision).  Only the
tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package; the library under ``block_sparse_paged_amd`` never does.

Every function takes CPU torch tensors holding the exact bytes the GPU sees
(uint8 E4M3FN codes, bf16, float32, int32) and returns float64 numpy arrays.
``build()`` compiles the shared object with gcc.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msa_oracle.c")
_LIB = os.environ.get("MSA_ORACLE_LIB") or os.path.join(_HERE, "libmsa_oracle.so")

F32, BF16, E4M3FN = 0, 1, 2
_ERRORS = {1: "bad argument", 2: "physical page out of range", 3: "seq_len out of range",
           4: "duplicate block id in a selection", 5: "NaN in a visible position"}

_lib = None
_lock = threading.Lock()


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math: IEEE double throughout)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"],
                       check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build(force=True)
            lib = ctypes.CDLL(_LIB)
            i64, dbl, vp = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
            lib.orc_e4m3fn_value.restype = dbl
            lib.orc_e4m3fn_value.argtypes = [ctypes.c_uint8]
            lib.orc_bf16_value.restype = dbl
            lib.orc_bf16_value.argtypes = [ctypes.c_uint16]
            lib.orc_block_score.restype = ctypes.c_int
            lib.orc_block_score.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, vp, vp,
                                            i64, i64, i64, i64, i64, i64, dbl, i64, i64, vp]
            lib.orc_select_topk.restype = ctypes.c_int
            lib.orc_select_topk.argtypes = [vp, i64, i64, i64, vp]
            lib.orc_sparse_decode.restype = ctypes.c_int
            lib.orc_sparse_decode.argtypes = [vp, ctypes.c_int, vp, vp, ctypes.c_int, vp, vp, vp,
                                              i64, i64, i64, i64, i64, i64, i64, i64, i64,
                                              dbl, dbl, dbl, i64, i64, vp]
            lib.orc_prefill_select.restype = ctypes.c_int
            lib.orc_prefill_select.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, ctypes.c_int, i64,
                                               i64, vp, i64, i64, vp, vp, vp, vp, i64, i64, i64, i64,
                                               i64, dbl, vp, i64, i64, i64, vp, vp, vp]
            lib.orc_dense_attention.restype = ctypes.c_int
            lib.orc_dense_attention.argtypes = [vp, ctypes.c_int, vp, vp, ctypes.c_int, vp, vp,
                                                i64, i64, i64, i64, i64, i64, i64, i64,
                                                dbl, dbl, dbl, i64, i64, vp]
            _lib = lib
    return _lib


class OracleError(RuntimeError):
    pass


def _check(rc: int):
    if rc != 0:
        raise OracleError(f"oracle precondition failed: {_ERRORS.get(rc, rc)}")


def _raw(t: torch.Tensor) -> tuple[np.ndarray, int]:
    """Contiguous host bytes of a tensor and its oracle dtype code."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return t.view(torch.uint8).numpy(), E4M3FN
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy(), BF16
    if t.dtype == torch.float32:
        return t.numpy(), F32
    if t.dtype == torch.int32:
        return t.numpy(), -1
    raise TypeError(f"oracle: unsupported dtype {t.dtype}")


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _ranges(n0: int, n1: int, threads: int):
    threads = max(1, min(threads, n1 - n0))
    step = (n1 - n0 + threads - 1) // threads
    return [(a, min(a + step, n1)) for a in range(n0, n1, step)]


def e4m3fn_value(code: int) -> float:
    return _load().orc_e4m3fn_value(code)


def bf16_value(bits: int) -> float:
    return _load().orc_bf16_value(bits & 0xFFFF)


def block_score(q_idx, index_k, block_table, seq_lens, T: int, idx_scale: float,
                n_range: Optional[tuple[int, int]] = None, threads: int = 1) -> np.ndarray:
    """scores [N, MB] float64; rows outside ``n_range`` are NaN."""
    lib = _load()
    q, qd = _raw(q_idx)
    k, kd = _raw(index_k)
    bt, _ = _raw(block_table)
    sl, _ = _raw(seq_lens)
    R, MB = bt.shape
    P, B, Di = k.shape
    N = R * T
    n0, n1 = n_range if n_range is not None else (0, N)
    out = np.full((N, MB), np.nan, dtype=np.float64)

    def run(a, b):
        return lib.orc_block_score(_ptr(q), qd, _ptr(k), kd, _ptr(bt), _ptr(sl), R, T, MB, P, B,
                                   Di, float(idx_scale), a, b, _ptr(out))

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        for rc in ex.map(lambda ab: run(*ab), _ranges(n0, n1, threads)):
            _check(rc)
    return out


def block_score_per_row(q_idx, index_k, block_table, seq_lens, T: int, idx_scale: float,
                        threads: int = 1) -> np.ndarray:
    """scores [R, MB] float64: one sheet row per request (attention.msa_block_score's
    per-request block-max sheet in Cacheon "Kernel ABI", "Attention block slots"),
    the block max taken over the request's T tokens as well: row r, block j holds
    the max over the row's tokens of their block-j scores (-inf where no token sees
    a key of block j; NaN propagates)."""
    per_token = block_score(q_idx, index_k, block_table, seq_lens, T, idx_scale, threads=threads)
    R = per_token.shape[0] // T
    return per_token.reshape(R, T, -1).max(axis=1)


def select_topk(scores, k: int) -> np.ndarray:
    """topk_idx [N, k] int32 from a score sheet (float64 or float32 values)."""
    lib = _load()
    s = np.ascontiguousarray(np.asarray(scores, dtype=np.float64))
    N, MB = s.shape
    out = np.empty((N, k), dtype=np.int32)
    _check(lib.orc_select_topk(_ptr(s), N, MB, k, _ptr(out)))
    return out


def sparse_decode(q, k_cache, v_cache, block_table, seq_lens, topk_idx, T: int,
                  sm_scale: float, k_scale: float, v_scale: float,
                  n_range: Optional[tuple[int, int]] = None, threads: int = 1) -> np.ndarray:
    """out [N, Hq, D] float64 (rows outside ``n_range`` are NaN).

    ``topk_idx`` rows are per query token (N = R*T of them) or, with T > 1, per
    request (R rows, shared by the request's tokens).  It is [N, K] (one
    selection shared by every KV head) or [Hkv, N, K]
    (one selection per KV head, the (Hkv, B, K) layout of attention.decode in
    Cacheon "Kernel ABI", "Attention block slots"): query head h attends the
    blocks of topk_idx[h // (Hq // Hkv)].  The per-head form is the shared form
    evaluated once per KV head, keeping that head's query heads."""
    tk_all = np.asarray(torch.as_tensor(topk_idx, dtype=torch.int32).cpu())
    N = int(q.shape[0])
    if T > 1 and tk_all.shape[-2] == N // T and N // T != N:
        # one selection per request, shared by its T tokens (each token keeps
        # its own visibility): token r*T + t uses row r
        tk_all = np.repeat(tk_all, T, axis=-2)
    if tk_all.ndim == 3:
        Hkv, Hq = k_cache.shape[2], q.shape[1]
        assert tk_all.shape[0] == Hkv and Hq % Hkv == 0
        G = Hq // Hkv
        out = None
        for g in range(Hkv):
            o = sparse_decode(q, k_cache, v_cache, block_table, seq_lens, tk_all[g], T, sm_scale,
                              k_scale, v_scale, n_range=n_range, threads=threads)
            if out is None:
                out = o.copy()
            out[:, g * G:(g + 1) * G] = o[:, g * G:(g + 1) * G]
        return out
    lib = _load()
    qa, qd = _raw(q)
    ka, kvd = _raw(k_cache)
    va, _ = _raw(v_cache)
    bt, _ = _raw(block_table)
    sl, _ = _raw(seq_lens)
    tk, _ = _raw(torch.as_tensor(tk_all, dtype=torch.int32))
    R, MB = bt.shape
    P, B, Hkv, D = ka.shape
    N, Hq, _ = qa.shape
    K = tk.shape[1]
    n0, n1 = n_range if n_range is not None else (0, N)
    out = np.full((N, Hq, D), np.nan, dtype=np.float64)

    def run(a, b):
        return lib.orc_sparse_decode(_ptr(qa), qd, _ptr(ka), _ptr(va), kvd, _ptr(bt), _ptr(sl),
                                     _ptr(tk), R, T, MB, P, B, Hq, Hkv, D, K, float(sm_scale),
                                     float(k_scale), float(v_scale), a, b, _ptr(out))

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        for rc in ex.map(lambda ab: run(*ab), _ranges(n0, n1, threads)):
            _check(rc)
    return out


def prefill_select(q, index_k, block_table, slot_ids, cu_seqlens, seq_lens, prefix_lens,
                   block_size_q: int, topk: int, init_blocks: int, local_blocks: int, scale: float,
                   cu_seqblocks_q, all_qb: int, threads: int = 1, return_scores: bool = False,
                   rows=None):
    """Prefill score-to-selection over a ragged batch (attention.msa_prefill_block_score):
    out_topk [Hq, all_qb, topk] int32, and with ``return_scores`` also the
    scores [Hq, all_qb, MB] float64 (-inf where a block is no candidate).
    q [total_q, Hq, Di]; index_k [P, B, Di]; block_table [slots, MB].  ``rows``
    (bool [Hq, all_qb]) restricts the work to the marked rows; the others stay
    -1 (and -inf)."""
    lib = _load()
    qa, qd = _raw(q)
    ka, kd = _raw(index_k)
    bt, _ = _raw(block_table)
    arrs = [_raw(torch.as_tensor(x, dtype=torch.int32))[0]
            for x in (slot_ids, cu_seqlens, seq_lens, prefix_lens, cu_seqblocks_q)]
    total_q, Hq, Di = qa.shape
    P, B, _ = ka.shape
    nslots, MB = bt.shape
    batch = arrs[0].shape[0]
    out = np.full((Hq, all_qb, topk), -1, dtype=np.int32)
    sc = np.full((Hq, all_qb, MB), -np.inf) if return_scores else None
    mask = None
    if rows is not None:
        mask = np.ascontiguousarray(np.asarray(rows, dtype=bool).reshape(Hq, all_qb), dtype=np.uint8)

    def run(h0, h1):
        return lib.orc_prefill_select(_ptr(qa), qd, total_q, Hq, Di, _ptr(ka), kd, P, B, _ptr(bt),
                                      nslots, MB, _ptr(arrs[0]), _ptr(arrs[1]), _ptr(arrs[2]),
                                      _ptr(arrs[3]), batch, block_size_q, topk, init_blocks,
                                      local_blocks, float(scale), _ptr(arrs[4]), all_qb, h0, h1,
                                      _ptr(mask) if mask is not None else None, _ptr(out),
                                      _ptr(sc) if sc is not None else None)

    with ThreadPoolExecutor(max_workers=max(1, min(threads, Hq))) as ex:
        for rc in ex.map(lambda ab: run(*ab), _ranges(0, Hq, threads)):
            _check(rc)
    return (out, sc) if return_scores else out


def dense_attention(q, k_cache, v_cache, block_table, seq_lens, T: int, sm_scale: float,
                    k_scale: float, v_scale: float,
                    n_range: Optional[tuple[int, int]] = None, threads: int = 1) -> np.ndarray:
    lib = _load()
    qa, qd = _raw(q)
    ka, kvd = _raw(k_cache)
    va, _ = _raw(v_cache)
    bt, _ = _raw(block_table)
    sl, _ = _raw(seq_lens)
    R, MB = bt.shape
    P, B, Hkv, D = ka.shape
    N, Hq, _ = qa.shape
    n0, n1 = n_range if n_range is not None else (0, N)
    out = np.full((N, Hq, D), np.nan, dtype=np.float64)

    def run(a, b):
        return lib.orc_dense_attention(_ptr(qa), qd, _ptr(ka), _ptr(va), kvd, _ptr(bt), _ptr(sl),
                                       R, T, MB, P, B, Hq, Hkv, D, float(sm_scale),
                                       float(k_scale), float(v_scale), a, b, _ptr(out))

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        for rc in ex.map(lambda ab: run(*ab), _ranges(n0, n1, threads)):
            _check(rc)
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (nearest-even) and return them as float64.

    Goes through float32 first only when that step is exact for the comparison
    at hand; to avoid double rounding it rounds from float64 directly here.
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    flat = x.reshape(-1)
    res = out.reshape(-1)
    m, e = np.frexp(flat)                     # flat = m * 2^e, 0.5 <= |m| < 1
    # bf16 keeps 8 significant bits: round m * 2^8 to nearest even integer
    scaled = m * 256.0
    rounded = np.round(scaled)                # numpy rounds half to even
    res[:] = np.ldexp(rounded / 256.0, e)
    # subnormal / huge values are not produced by these workloads
    res[~np.isfinite(flat)] = flat[~np.isfinite(flat)]
    return out
