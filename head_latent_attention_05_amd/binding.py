"""Thin ctypes binding over libmla.so (see include/mla.h for the contract).

Only argument marshalling happens here: torch tensors supply device pointers
and the current HIP stream; every step of the computation runs in libmla's HIP
kernels.  There is no fallback: if the library is missing or a call fails, an
exception is raised.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla.so")

MLA_F32 = 0
MLA_BF16 = 1

STATUS = {0: "MLA_OK", 1: "MLA_ERR_INVALID_ARG", 2: "MLA_ERR_UNSUPPORTED",
          3: "MLA_ERR_WORKSPACE", 4: "MLA_ERR_HIP"}

DEVERR_POSITION, DEVERR_SEQ, DEVERR_BLOCK, DEVERR_LENGTH = 1, 2, 4, 8

EXPORTS = ["mla_status_string", "mla_rope_table", "mla_absorb_q", "mla_append_cache",
           "mla_decode_workspace_size", "mla_decode", "mla_out_proj", "mla_decode_noalloc",
           "mla_kv_down_workspace_size", "mla_kv_down_append", "mla_absorb_q_fused",
           "mla_out_proj_fused_workspace_size", "mla_out_proj_fused",
           "mla_prefill_workspace_size", "mla_prefill_decompressed", "mla_append_cache_fp8",
           "mla_decode_fp8"]


class MlaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")
        self.status = status


class MlaConfig(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("d_latent", ctypes.c_int32),
                ("d_rope", ctypes.c_int32), ("d_nope", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("dtype", ctypes.c_int32)]

    @classmethod
    def from_dims(cls, dims, block_size: int = 64) -> "MlaConfig":
        return cls(dims.num_heads, dims.d_latent, dims.d_rope, dims.d_nope, dims.d_v,
                   block_size, 1.0 / math.sqrt(dims.d_nope + dims.d_rope),
                   MLA_BF16 if dims.dtype == "bf16" else MLA_F32)


def declare(lib: ctypes.CDLL) -> ctypes.CDLL:
    """Set the ctypes signatures of the C ABI (include/mla.h) on a loaded library."""
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    C = ctypes.POINTER(MlaConfig)
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_status_string.argtypes = [I32]
    lib.mla_rope_table.restype = I32
    lib.mla_rope_table.argtypes = [P, P, I32, I32, ctypes.c_double]
    lib.mla_absorb_q.restype = I32
    lib.mla_absorb_q.argtypes = [C, I32, P, P, P, P]
    lib.mla_append_cache.restype = I32
    lib.mla_append_cache.argtypes = [C, I32, P, P, P, P, P, P, I32, I32, I64, P, P, I32, P, P, P, P]
    lib.mla_decode_workspace_size.restype = I32
    lib.mla_decode_workspace_size.argtypes = [C, I32, P, P, I32, I32, ctypes.POINTER(SZ)]
    lib.mla_decode.restype = I32
    lib.mla_decode.argtypes = [C, I32, P, P, P, P, P, I32, I64, P, P, I32, I32, P, SZ, P, P, P]
    lib.mla_out_proj.restype = I32
    lib.mla_out_proj.argtypes = [C, I32, P, P, P, P]
    lib.mla_decode_noalloc.restype = I32
    lib.mla_decode_noalloc.argtypes = [C, I32, P, P, P, P, P, I32, I64, P, P, I32, I32, P, P, P]
    lib.mla_absorb_q_fused.restype = I32
    lib.mla_absorb_q_fused.argtypes = [C, I32, I32, P, P, P, P]
    lib.mla_out_proj_fused_workspace_size.restype = I32
    lib.mla_out_proj_fused_workspace_size.argtypes = [C, I32, I32, ctypes.POINTER(SZ)]
    lib.mla_out_proj_fused.restype = I32
    lib.mla_out_proj_fused.argtypes = [C, I32, I32, P, P, P, P, SZ, P]
    lib.mla_prefill_workspace_size.restype = I32
    lib.mla_prefill_workspace_size.argtypes = [C, I32, P, P, ctypes.POINTER(SZ)]
    lib.mla_prefill_decompressed.restype = I32
    lib.mla_prefill_decompressed.argtypes = [C, I32, P, P, P, P, P, I32, I64, P, P, P, P, P, I32,
                                             P, SZ, P, P, P]
    lib.mla_kv_down_workspace_size.restype = I32
    lib.mla_kv_down_workspace_size.argtypes = [C, I32, I32, ctypes.POINTER(SZ)]
    lib.mla_kv_down_append.restype = I32
    lib.mla_kv_down_append.argtypes = [C, I32, I32, P, P, P, P, ctypes.c_float, P, P, P, P, I32,
                                       I32, I64, P, P, I32, P, SZ, P, P, P, P]
    lib.mla_append_cache_fp8.restype = I32
    lib.mla_append_cache_fp8.argtypes = [C, I32, P, P, P, P, P, P, I32, I32, I64, P, P, I32,
                                         ctypes.c_float, P, P, P, P]
    lib.mla_decode_fp8.restype = I32
    lib.mla_decode_fp8.argtypes = [C, I32, P, P, P, P, P, I32, I64, P, P, ctypes.c_float, I32,
                                   I32, P, SZ, P, P, P]
    return lib


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmla.so (built by head_latent_attention_05_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: run `python -m head_latent_attention_05_amd.build`")
    lib = ctypes.CDLL(path)
    declare(lib)
    _lib = lib
    return lib


def _check(fn: str, st: int) -> None:
    if st != 0:
        raise MlaError(fn, st)


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def rope_table(max_pos: int, d_rope: int, theta: float = 10000.0):
    """Host RoPE tables (cos, sin) as float32 numpy arrays [max_pos, d_rope/2]."""
    lib = load()
    cos = np.empty((max_pos, d_rope // 2), np.float32)
    sin = np.empty((max_pos, d_rope // 2), np.float32)
    _check("mla_rope_table", lib.mla_rope_table(cos.ctypes.data, sin.ctypes.data, max_pos,
                                                d_rope, theta))
    return cos, sin


def absorb_q(cfg: MlaConfig, q_nope, w_uk, q_lat, stream=None) -> None:
    lib = load()
    T = q_nope.shape[0]
    _check("mla_absorb_q", lib.mla_absorb_q(ctypes.byref(cfg), T, _ptr(q_nope), _ptr(w_uk),
                                            _ptr(q_lat), _stream(stream)))


def append_cache(cfg: MlaConfig, c_kv, k_pe, q_pe, token_seq, positions, block_table,
                 num_pool_blocks: int, rope_cos, rope_sin, kv_pool, q_lat=None,
                 dev_error=None, stream=None) -> None:
    lib = load()
    T = c_kv.shape[0]
    _check("mla_append_cache", lib.mla_append_cache(
        ctypes.byref(cfg), T, _ptr(c_kv), _ptr(k_pe), _ptr(q_pe), _ptr(token_seq),
        _ptr(positions), _ptr(block_table), block_table.shape[0], block_table.shape[1],
        num_pool_blocks, _ptr(rope_cos), _ptr(rope_sin), rope_cos.shape[0], _ptr(kv_pool),
        _ptr(q_lat), _ptr(dev_error), _stream(stream)))


def append_cache_fp8(cfg: MlaConfig, c_kv, k_pe, q_pe, token_seq, positions, block_table,
                     num_pool_blocks: int, rope_cos, rope_sin, kv_scale: float, kv_pool,
                     q_lat=None, dev_error=None, stream=None) -> None:
    lib = load()
    T = c_kv.shape[0]
    _check("mla_append_cache_fp8", lib.mla_append_cache_fp8(
        ctypes.byref(cfg), T, _ptr(c_kv), _ptr(k_pe), _ptr(q_pe), _ptr(token_seq),
        _ptr(positions), _ptr(block_table), block_table.shape[0], block_table.shape[1],
        num_pool_blocks, _ptr(rope_cos), _ptr(rope_sin), rope_cos.shape[0], kv_scale,
        _ptr(kv_pool), _ptr(q_lat), _ptr(dev_error), _stream(stream)))


def decode_workspace_size(cfg: MlaConfig, q_start_host: np.ndarray, kv_lens_host: np.ndarray,
                          causal: bool, num_workgroups: int = 0) -> int:
    lib = load()
    qs = np.ascontiguousarray(q_start_host, np.int32)
    kl = np.ascontiguousarray(kv_lens_host, np.int32)
    out = ctypes.c_size_t(0)
    _check("mla_decode_workspace_size", lib.mla_decode_workspace_size(
        ctypes.byref(cfg), len(kl), qs.ctypes.data, kl.ctypes.data, int(causal),
        num_workgroups, ctypes.byref(out)))
    return out.value


def decode(cfg: MlaConfig, q_start, kv_lens, q_start_host: np.ndarray, kv_lens_host: np.ndarray,
           block_table, num_pool_blocks: int, q_lat, kv_pool, causal: bool, o_lat,
           workspace=None, num_workgroups: int = 0, dev_error=None, stream=None) -> None:
    lib = load()
    qs = np.ascontiguousarray(q_start_host, np.int32)
    kl = np.ascontiguousarray(kv_lens_host, np.int32)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("mla_decode", lib.mla_decode(
        ctypes.byref(cfg), len(kl), _ptr(q_start), _ptr(kv_lens), qs.ctypes.data,
        kl.ctypes.data, _ptr(block_table), block_table.shape[1], num_pool_blocks,
        _ptr(q_lat), _ptr(kv_pool), int(causal), num_workgroups, _ptr(workspace), ws_bytes,
        _ptr(o_lat), _ptr(dev_error), _stream(stream)))


def decode_fp8(cfg: MlaConfig, q_start, kv_lens, q_start_host: np.ndarray,
               kv_lens_host: np.ndarray, block_table, num_pool_blocks: int, q_lat, kv_pool,
               kv_scale: float, causal: bool, o_lat, workspace=None, num_workgroups: int = 0,
               dev_error=None, stream=None) -> None:
    lib = load()
    qs = np.ascontiguousarray(q_start_host, np.int32)
    kl = np.ascontiguousarray(kv_lens_host, np.int32)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("mla_decode_fp8", lib.mla_decode_fp8(
        ctypes.byref(cfg), len(kl), _ptr(q_start), _ptr(kv_lens), qs.ctypes.data,
        kl.ctypes.data, _ptr(block_table), block_table.shape[1], num_pool_blocks,
        _ptr(q_lat), _ptr(kv_pool), kv_scale, int(causal), num_workgroups, _ptr(workspace),
        ws_bytes, _ptr(o_lat), _ptr(dev_error), _stream(stream)))


def decode_noalloc(cfg: MlaConfig, q_start, kv_lens, q_start_host: np.ndarray,
                   kv_lens_host: np.ndarray, block_table, num_pool_blocks: int, q_lat, kv_pool,
                   causal: bool, o_lat, num_workgroups: int = 0, dev_error=None,
                   stream=None) -> None:
    lib = load()
    qs = np.ascontiguousarray(q_start_host, np.int32)
    kl = np.ascontiguousarray(kv_lens_host, np.int32)
    _check("mla_decode_noalloc", lib.mla_decode_noalloc(
        ctypes.byref(cfg), len(kl), _ptr(q_start), _ptr(kv_lens), qs.ctypes.data,
        kl.ctypes.data, _ptr(block_table), block_table.shape[1], num_pool_blocks,
        _ptr(q_lat), _ptr(kv_pool), int(causal), num_workgroups, _ptr(o_lat), _ptr(dev_error),
        _stream(stream)))


def out_proj(cfg: MlaConfig, o_lat, w_uv, out, stream=None) -> None:
    lib = load()
    T = o_lat.shape[0]
    _check("mla_out_proj", lib.mla_out_proj(ctypes.byref(cfg), T, _ptr(o_lat), _ptr(w_uv),
                                            _ptr(out), _stream(stream)))


def kv_down_workspace_size(cfg: MlaConfig, T: int, d_model: int) -> int:
    lib = load()
    out = ctypes.c_size_t(0)
    _check("mla_kv_down_workspace_size",
           lib.mla_kv_down_workspace_size(ctypes.byref(cfg), T, d_model, ctypes.byref(out)))
    return out.value


def kv_down_append(cfg: MlaConfig, x, w_dkv, b_dkv, rms_gamma, rms_eps: float, q_pe,
                   token_seq, positions, block_table, num_pool_blocks: int, rope_cos, rope_sin,
                   workspace, kv_pool, q_lat=None, dev_error=None, stream=None) -> None:
    lib = load()
    T, d_model = x.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("mla_kv_down_append", lib.mla_kv_down_append(
        ctypes.byref(cfg), T, d_model, _ptr(x), _ptr(w_dkv), _ptr(b_dkv), _ptr(rms_gamma),
        float(rms_eps), _ptr(q_pe), _ptr(token_seq), _ptr(positions), _ptr(block_table),
        block_table.shape[0], block_table.shape[1], num_pool_blocks, _ptr(rope_cos),
        _ptr(rope_sin), rope_cos.shape[0], _ptr(workspace), ws_bytes, _ptr(kv_pool), _ptr(q_lat),
        _ptr(dev_error), _stream(stream)))


def absorb_q_fused(cfg: MlaConfig, c_q, w_kq, q_lat, stream=None) -> None:
    lib = load()
    T, d_cq = c_q.shape
    _check("mla_absorb_q_fused", lib.mla_absorb_q_fused(
        ctypes.byref(cfg), T, d_cq, _ptr(c_q), _ptr(w_kq), _ptr(q_lat), _stream(stream)))


def out_proj_fused_workspace_size(cfg: MlaConfig, T: int, d_model: int) -> int:
    lib = load()
    out = ctypes.c_size_t(0)
    _check("mla_out_proj_fused_workspace_size", lib.mla_out_proj_fused_workspace_size(
        ctypes.byref(cfg), T, d_model, ctypes.byref(out)))
    return out.value


def out_proj_fused(cfg: MlaConfig, o_lat, w_ov, out, workspace, stream=None) -> None:
    lib = load()
    T = o_lat.shape[0]
    d_model = out.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("mla_out_proj_fused", lib.mla_out_proj_fused(
        ctypes.byref(cfg), T, d_model, _ptr(o_lat), _ptr(w_ov), _ptr(out), _ptr(workspace),
        ws_bytes, _stream(stream)))


def prefill_workspace_size(cfg: MlaConfig, q_start_host: np.ndarray,
                           kv_lens_host: np.ndarray) -> int:
    lib = load()
    qs = np.ascontiguousarray(q_start_host, np.int32)
    kl = np.ascontiguousarray(kv_lens_host, np.int32)
    out = ctypes.c_size_t(0)
    _check("mla_prefill_workspace_size", lib.mla_prefill_workspace_size(
        ctypes.byref(cfg), len(kl), qs.ctypes.data, kl.ctypes.data, ctypes.byref(out)))
    return out.value


def prefill_decompressed(cfg: MlaConfig, q_start, kv_lens, q_start_host: np.ndarray,
                         kv_lens_host: np.ndarray, block_table, num_pool_blocks: int, q_nope,
                         q_lat, kv_pool, w_uk, w_uv, causal: bool, workspace, out,
                         dev_error=None, stream=None) -> None:
    lib = load()
    qs = np.ascontiguousarray(q_start_host, np.int32)
    kl = np.ascontiguousarray(kv_lens_host, np.int32)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("mla_prefill_decompressed", lib.mla_prefill_decompressed(
        ctypes.byref(cfg), len(kl), _ptr(q_start), _ptr(kv_lens), qs.ctypes.data,
        kl.ctypes.data, _ptr(block_table), block_table.shape[1], num_pool_blocks, _ptr(q_nope),
        _ptr(q_lat), _ptr(kv_pool), _ptr(w_uk), _ptr(w_uv), int(causal), _ptr(workspace),
        ws_bytes, _ptr(out), _ptr(dev_error), _stream(stream)))
