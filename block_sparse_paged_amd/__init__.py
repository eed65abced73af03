"""MI355X (gfx950) MSA sparse-layer decode attention.

Thin ctypes binding over the C ABI in ``include/msa.h`` (``libmsa.so``, built
in-tree by ``block_sparse_paged_amd.build``).  The functions take torch CUDA
tensors only for their device pointers, sizes and strides, and the current
torch stream for the HIP stream; every step runs in the library's kernels.
There is no CPU fallback: importing fails when the library is missing.

    msa_block_score(q_idx, index_k, block_table, seq_lens, tokens_per_row,
                    block_size, idx_scale, scores)
    msa_select_topk(scores, k, topk_idx)
    msa_sparse_decode(q, k_cache, v_cache, block_table, seq_lens, topk_idx,
                      tokens_per_row, out, sm_scale, k_scale, v_scale,
                      block_size, workspace)
    msa_select_sparse_decode(scores, k, topk_idx, q, k_cache, v_cache, block_table,
                             seq_lens, tokens_per_row, out, sm_scale, k_scale, v_scale,
                             block_size, workspace)
    msa_decode_step(q_idx, index_k, q, k_cache, v_cache, block_table, seq_lens,
                    tokens_per_row, k, block_size, idx_scale, sm_scale, k_scale,
                    v_scale, scores, topk_idx, out, workspace)
    msa_decode_step_noalloc(q_idx, index_k, q, k_cache, v_cache, block_table, seq_lens,
                            tokens_per_row, k, block_size, idx_scale, sm_scale, k_scale,
                            v_scale, scores, topk_idx, out)
    msa_prefill_block_score(q, index_k, block_table, slot_ids, cu_seqlens, seq_lens,
                            prefix_lens, block_size_q, block_size_k, topk, init_blocks,
                            local_blocks, scale, cu_seqblocks_q, out_topk, workspace)

Each call writes into the outputs given (same argument order as the C ABI)
and returns None; a rejected call raises MsaError and leaves the outputs as
they were.  FP8 tensors may be passed as torch.float8_e4m3fn or uint8 codes.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmsa.so")

MSA_F32, MSA_BF16, MSA_FP8_E4M3FN, MSA_I32 = 0, 1, 2, 3
_DTYPES = {
    torch.float32: MSA_F32,
    torch.bfloat16: MSA_BF16,
    torch.float8_e4m3fn: MSA_FP8_E4M3FN,
    torch.uint8: MSA_FP8_E4M3FN,
    torch.int32: MSA_I32,
}
EXPORTS = ("msa_block_score", "msa_select_topk", "msa_sparse_decode_workspace_bytes",
           "msa_sparse_decode", "msa_select_sparse_decode", "msa_decode_step_workspace_bytes",
           "msa_decode_step", "msa_decode_step_noalloc", "msa_prefill_block_score_workspace_bytes",
           "msa_prefill_block_score",
           "msa_get_last_error", "msa_error_string")


class msa_tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class MsaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"msa error {code}: {msg}")
        self.code = code


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing; build it with "
                          "`python block_sparse_paged_amd/build.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(msa_tensor)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.msa_block_score.restype = None
    lib.msa_block_score.argtypes = [P, P, P, P, i32, i32, f32, P, vp]
    lib.msa_select_topk.restype = None
    lib.msa_select_topk.argtypes = [P, i32, P, vp]
    lib.msa_sparse_decode_workspace_bytes.restype = sz
    lib.msa_sparse_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.msa_sparse_decode.restype = None
    lib.msa_sparse_decode.argtypes = [P, P, P, P, P, P, i32, P, f32, f32, f32, i32, vp, sz, vp]
    lib.msa_select_sparse_decode.restype = None
    lib.msa_select_sparse_decode.argtypes = [P, i32, P, P, P, P, P, P, i32, P, f32, f32, f32, i32,
                                             vp, sz, vp]
    lib.msa_decode_step_workspace_bytes.restype = sz
    lib.msa_decode_step_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.msa_decode_step.restype = None
    lib.msa_decode_step.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, f32, f32, f32, f32, P, P, P,
                                    vp, sz, vp]
    lib.msa_decode_step_noalloc.restype = None
    lib.msa_decode_step_noalloc.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, f32, f32, f32, f32, P, P,
                                            P, vp]
    lib.msa_prefill_block_score_workspace_bytes.restype = sz
    lib.msa_prefill_block_score_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.msa_prefill_block_score.restype = None
    lib.msa_prefill_block_score.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, i32, f32, P, P,
                                            vp, sz, vp]
    lib.msa_get_last_error.restype = i32
    lib.msa_get_last_error.argtypes = []
    lib.msa_error_string.restype = ctypes.c_char_p
    lib.msa_error_string.argtypes = [i32]
    return lib


lib = _load()


def tensor_desc(t: Optional[torch.Tensor], ndim: Optional[int] = None) -> msa_tensor:
    """msa_tensor describing a torch tensor (pointer, dtype, sizes, strides)."""
    d = msa_tensor()
    if t is None:
        return d
    if t.dim() > 4:
        raise ValueError("at most 4 dimensions")
    d.data = t.data_ptr() if t.numel() else None
    d.dtype = _DTYPES.get(t.dtype, -1)
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check():
    code = lib.msa_get_last_error()
    if code:
        raise MsaError(code, lib.msa_error_string(code).decode())


def msa_block_score(q_idx, index_k, block_table, seq_lens, tokens_per_row: int,
                    block_size: int, idx_scale: float, scores, stream=None) -> None:
    d = [tensor_desc(t) for t in (q_idx, index_k, block_table, seq_lens, scores)]
    lib.msa_block_score(ctypes.byref(d[0]), ctypes.byref(d[1]), ctypes.byref(d[2]),
                        ctypes.byref(d[3]), int(tokens_per_row), int(block_size),
                        float(idx_scale), ctypes.byref(d[4]), _stream(stream))
    _check()


def msa_select_topk(scores, k: int, topk_idx, stream=None) -> None:
    ds, dt = tensor_desc(scores), tensor_desc(topk_idx)
    lib.msa_select_topk(ctypes.byref(ds), int(k), ctypes.byref(dt), _stream(stream))
    _check()


def msa_sparse_decode_workspace_bytes(rows: int, tokens_per_row: int, num_q_heads: int,
                                      num_kv_heads: int, head_dim: int, k: int) -> int:
    return int(lib.msa_sparse_decode_workspace_bytes(rows, tokens_per_row, num_q_heads,
                                                     num_kv_heads, head_dim, k))


def msa_sparse_decode(q, k_cache, v_cache, block_table, seq_lens, topk_idx,
                      tokens_per_row: int, out, sm_scale: float, k_scale: float,
                      v_scale: float, block_size: int, workspace, stream=None) -> None:
    d = [tensor_desc(t) for t in (q, k_cache, v_cache, block_table, seq_lens, topk_idx, out)]
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    lib.msa_sparse_decode(*(ctypes.byref(x) for x in d[:6]), int(tokens_per_row),
                          ctypes.byref(d[6]), float(sm_scale), float(k_scale), float(v_scale),
                          int(block_size), ws_ptr, ws_bytes, _stream(stream))
    _check()


def msa_select_sparse_decode(scores, k: int, topk_idx, q, k_cache, v_cache, block_table,
                             seq_lens, tokens_per_row: int, out, sm_scale: float, k_scale: float,
                             v_scale: float, block_size: int, workspace, stream=None) -> None:
    d = [tensor_desc(t) for t in (scores, topk_idx, q, k_cache, v_cache, block_table, seq_lens, out)]
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    lib.msa_select_sparse_decode(ctypes.byref(d[0]), int(k), *(ctypes.byref(x) for x in d[1:7]),
                                 int(tokens_per_row), ctypes.byref(d[7]), float(sm_scale),
                                 float(k_scale), float(v_scale), int(block_size), ws_ptr, ws_bytes,
                                 _stream(stream))
    _check()


def msa_decode_step_workspace_bytes(rows: int, tokens_per_row: int, num_q_heads: int,
                                    num_kv_heads: int, head_dim: int, k: int) -> int:
    return int(lib.msa_decode_step_workspace_bytes(rows, tokens_per_row, num_q_heads,
                                                   num_kv_heads, head_dim, k))


def msa_decode_step(q_idx, index_k, q, k_cache, v_cache, block_table, seq_lens,
                    tokens_per_row: int, k: int, block_size: int, idx_scale: float,
                    sm_scale: float, k_scale: float, v_scale: float, scores, topk_idx, out,
                    workspace, stream=None) -> None:
    d = [tensor_desc(t) for t in (q_idx, index_k, q, k_cache, v_cache, block_table, seq_lens,
                                  scores, topk_idx, out)]
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    lib.msa_decode_step(*(ctypes.byref(x) for x in d[:7]), int(tokens_per_row), int(k),
                        int(block_size), float(idx_scale), float(sm_scale), float(k_scale),
                        float(v_scale), *(ctypes.byref(x) for x in d[7:]), ws_ptr, ws_bytes,
                        _stream(stream))
    _check()


def msa_decode_step_noalloc(q_idx, index_k, q, k_cache, v_cache, block_table, seq_lens,
                            tokens_per_row: int, k: int, block_size: int, idx_scale: float,
                            sm_scale: float, k_scale: float, v_scale: float, scores, topk_idx, out,
                            stream=None) -> None:
    d = [tensor_desc(t) for t in (q_idx, index_k, q, k_cache, v_cache, block_table, seq_lens,
                                  scores, topk_idx, out)]
    lib.msa_decode_step_noalloc(*(ctypes.byref(x) for x in d[:7]), int(tokens_per_row), int(k),
                                int(block_size), float(idx_scale), float(sm_scale), float(k_scale),
                                float(v_scale), *(ctypes.byref(x) for x in d[7:]), _stream(stream))
    _check()


def msa_prefill_block_score_workspace_bytes(batch: int, num_q_heads: int, all_seqblock_q: int,
                                            max_blocks: int, block_size_q: int) -> int:
    return int(lib.msa_prefill_block_score_workspace_bytes(batch, num_q_heads, all_seqblock_q,
                                                           max_blocks, block_size_q))


def msa_prefill_block_score(q, index_k, block_table, slot_ids, cu_seqlens, seq_lens, prefix_lens,
                            block_size_q: int, block_size_k: int, topk: int, init_blocks: int,
                            local_blocks: int, scale: float, cu_seqblocks_q, out_topk, workspace,
                            stream=None) -> None:
    d = [tensor_desc(t) for t in (q, index_k, block_table, slot_ids, cu_seqlens, seq_lens,
                                  prefix_lens, cu_seqblocks_q, out_topk)]
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    lib.msa_prefill_block_score(*(ctypes.byref(x) for x in d[:7]), int(block_size_q),
                                int(block_size_k), int(topk), int(init_blocks), int(local_blocks),
                                float(scale), ctypes.byref(d[7]), ctypes.byref(d[8]), ws_ptr,
                                ws_bytes, _stream(stream))
    _check()
