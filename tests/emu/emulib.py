"""Runs the library's C ABI with every kernel executed by the host emulator
(tests/emu/_build/libmla_emu.so, built from the same HIP sources).  Test
infrastructure: buffers are host memory whose end touches an inaccessible page,
so a kernel reading or writing past the end of a buffer faults.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import numpy as np

from head_latent_attention_05_amd import binding as B
from head_latent_attention_05_amd.synth import BLOCK_SIZE, Inputs
from tests.emu import build_emu

SENTINEL_BF16 = 0x7FC1
SENTINEL_F32 = 0x7FC00001


class Emu:
    def __init__(self, cus: int = 8, seed: int = 1, lib_path: Optional[str] = None):
        lib = ctypes.CDLL(lib_path or build_emu.build())
        B.declare(lib)
        lib.emu_alloc.restype = ctypes.c_void_p
        lib.emu_alloc.argtypes = [ctypes.c_size_t]
        lib.emu_free.argtypes = [ctypes.c_void_p]
        lib.emu_set_cus.argtypes = [ctypes.c_int]
        lib.emu_set_seed.argtypes = [ctypes.c_ulonglong]
        lib.emu_counters.argtypes = [ctypes.c_void_p]
        self.lib = lib
        self._held = []
        lib.emu_set_cus(cus)
        lib.emu_set_seed(seed)

    def set_seed(self, seed: int) -> None:
        self.lib.emu_set_seed(seed)

    def counters(self):
        out = np.zeros(3, np.uint64)
        self.lib.emu_counters(out.ctypes.data)
        return {"blocks": int(out[0]), "wave_ops": int(out[1]), "barriers": int(out[2])}

    def empty(self, shape, dtype) -> np.ndarray:
        """Guarded, zero-filled host buffer."""
        dtype = np.dtype(dtype)
        n = int(np.prod(shape)) * dtype.itemsize
        p = self.lib.emu_alloc(max(n, 16))
        if not p:
            raise MemoryError(n)
        self._held.append(p)
        raw = (ctypes.c_uint8 * max(n, 16)).from_address(p)
        return np.frombuffer(raw, np.uint8, count=n).view(dtype).reshape(shape)

    def put(self, arr: np.ndarray) -> np.ndarray:
        out = self.empty(arr.shape, arr.dtype)
        out[...] = arr
        return out

    def close(self) -> None:
        for p in self._held:
            self.lib.emu_free(p)
        self._held = []

    # -- the C ABI on host buffers (stream argument: none) ----------------------
    def check(self, fn: str, st: int) -> None:
        if st != 0:
            raise B.MlaError(fn, st)

    def absorb_q(self, cfg, q_nope, w_uk, q_lat) -> None:
        self.check("mla_absorb_q", self.lib.mla_absorb_q(
            ctypes.byref(cfg), q_nope.shape[0], q_nope.ctypes.data, w_uk.ctypes.data,
            q_lat.ctypes.data, None))

    def out_proj(self, cfg, o_lat, w_uv, out) -> None:
        self.check("mla_out_proj", self.lib.mla_out_proj(
            ctypes.byref(cfg), o_lat.shape[0], o_lat.ctypes.data, w_uv.ctypes.data,
            out.ctypes.data, None))

    def append(self, cfg, c_kv, k_pe, q_pe, seq, pos, block_table, num_blocks, cos, sin, pool,
               q_lat=None, dev_error=None) -> None:
        p = lambda a: None if a is None else a.ctypes.data
        self.check("mla_append_cache", self.lib.mla_append_cache(
            ctypes.byref(cfg), c_kv.shape[0], p(c_kv), p(k_pe), p(q_pe), p(seq), p(pos),
            p(block_table), block_table.shape[0], block_table.shape[1], num_blocks, p(cos),
            p(sin), cos.shape[0], p(pool), p(q_lat), p(dev_error), None))

    def append_fp8(self, cfg, c_kv, k_pe, q_pe, seq, pos, block_table, num_blocks, cos, sin,
                   kv_scale, pool, q_lat=None, dev_error=None) -> None:
        p = lambda a: None if a is None else a.ctypes.data
        self.check("mla_append_cache_fp8", self.lib.mla_append_cache_fp8(
            ctypes.byref(cfg), c_kv.shape[0], p(c_kv), p(k_pe), p(q_pe), p(seq), p(pos),
            p(block_table), block_table.shape[0], block_table.shape[1], num_blocks, p(cos),
            p(sin), cos.shape[0], kv_scale, p(pool), p(q_lat), p(dev_error), None))

    def decode_fp8(self, cfg, q_start, kv_lens, block_table, num_blocks, q_lat, pool, kv_scale,
                   causal, o_lat, workspace=None, num_workgroups=0, dev_error=None) -> None:
        p = lambda a: None if a is None else a.ctypes.data
        ws_bytes = 0 if workspace is None else workspace.nbytes
        self.check("mla_decode_fp8", self.lib.mla_decode_fp8(
            ctypes.byref(cfg), len(kv_lens), p(q_start), p(kv_lens), p(q_start), p(kv_lens),
            p(block_table), block_table.shape[1], num_blocks, p(q_lat), p(pool), kv_scale,
            int(causal), num_workgroups, p(workspace), ws_bytes, p(o_lat), p(dev_error), None))

    def workspace_size(self, cfg, q_start_host, kv_lens_host, causal, num_workgroups=0) -> int:
        qs = np.ascontiguousarray(q_start_host, np.int32)
        kl = np.ascontiguousarray(kv_lens_host, np.int32)
        out = ctypes.c_size_t(0)
        self.check("mla_decode_workspace_size", self.lib.mla_decode_workspace_size(
            ctypes.byref(cfg), len(kl), qs.ctypes.data, kl.ctypes.data, int(causal),
            num_workgroups, ctypes.byref(out)))
        return out.value

    def decode(self, cfg, q_start, kv_lens, block_table, num_blocks, q_lat, pool, causal, o_lat,
               workspace=None, num_workgroups=0, dev_error=None) -> None:
        p = lambda a: None if a is None else a.ctypes.data
        ws_bytes = 0 if workspace is None else workspace.nbytes
        self.check("mla_decode", self.lib.mla_decode(
            ctypes.byref(cfg), len(kv_lens), p(q_start), p(kv_lens), p(q_start), p(kv_lens),
            p(block_table), block_table.shape[1], num_blocks, p(q_lat), p(pool), int(causal),
            num_workgroups, p(workspace), ws_bytes, p(o_lat), p(dev_error), None))

    def decode_noalloc(self, cfg, q_start, kv_lens, block_table, num_blocks, q_lat, pool, causal,
                       o_lat, num_workgroups=0, dev_error=None) -> None:
        p = lambda a: None if a is None else a.ctypes.data
        self.check("mla_decode_noalloc", self.lib.mla_decode_noalloc(
            ctypes.byref(cfg), len(kv_lens), p(q_start), p(kv_lens), p(q_start), p(kv_lens),
            p(block_table), block_table.shape[1], num_blocks, p(q_lat), p(pool), int(causal),
            num_workgroups, p(o_lat), p(dev_error), None))

    def absorb_q_fused(self, cfg, c_q, w_kq, q_lat) -> None:
        self.check("mla_absorb_q_fused", self.lib.mla_absorb_q_fused(
            ctypes.byref(cfg), c_q.shape[0], c_q.shape[1], c_q.ctypes.data, w_kq.ctypes.data,
            q_lat.ctypes.data, None))

    def out_proj_fused(self, cfg, o_lat, w_ov, out) -> None:
        T, d_model = out.shape
        n = ctypes.c_size_t(0)
        self.check("mla_out_proj_fused_workspace_size", self.lib.mla_out_proj_fused_workspace_size(
            ctypes.byref(cfg), T, d_model, ctypes.byref(n)))
        ws = self.empty((n.value,), np.uint8)
        self.check("mla_out_proj_fused", self.lib.mla_out_proj_fused(
            ctypes.byref(cfg), T, d_model, o_lat.ctypes.data, w_ov.ctypes.data, out.ctypes.data,
            ws.ctypes.data, ws.nbytes, None))

    def prefill_decompressed(self, cfg, q_start, kv_lens, block_table, num_blocks, q_nope, q_lat,
                             pool, w_uk, w_uv, causal, out, dev_error=None) -> None:
        p = lambda a: None if a is None else a.ctypes.data
        n = ctypes.c_size_t(0)
        self.check("mla_prefill_workspace_size", self.lib.mla_prefill_workspace_size(
            ctypes.byref(cfg), len(kv_lens), p(q_start), p(kv_lens), ctypes.byref(n)))
        ws = self.empty((n.value,), np.uint8)
        self.check("mla_prefill_decompressed", self.lib.mla_prefill_decompressed(
            ctypes.byref(cfg), len(kv_lens), p(q_start), p(kv_lens), p(q_start), p(kv_lens),
            p(block_table), block_table.shape[1], num_blocks, p(q_nope), p(q_lat), p(pool),
            p(w_uk), p(w_uv), int(causal), p(ws), ws.nbytes, p(out), p(dev_error), None))

    def kv_down_workspace_size(self, cfg, T, d_model) -> int:
        out = ctypes.c_size_t(0)
        self.check("mla_kv_down_workspace_size", self.lib.mla_kv_down_workspace_size(
            ctypes.byref(cfg), T, d_model, ctypes.byref(out)))
        return out.value

    def kv_down_append(self, cfg, x, w_dkv, b_dkv, gamma, eps, q_pe, seq, pos, block_table,
                       num_blocks, cos, sin, workspace, pool, q_lat=None, dev_error=None) -> None:
        p = lambda a: None if a is None else a.ctypes.data
        self.check("mla_kv_down_append", self.lib.mla_kv_down_append(
            ctypes.byref(cfg), x.shape[0], x.shape[1], p(x), p(w_dkv), p(b_dkv), p(gamma),
            float(eps), p(q_pe), p(seq), p(pos), p(block_table), block_table.shape[0],
            block_table.shape[1], num_blocks, p(cos), p(sin), cos.shape[0], p(workspace),
            0 if workspace is None else workspace.nbytes, p(pool), p(q_lat), p(dev_error), None))

    def rope_table(self, max_pos: int, d_rope: int):
        cos = self.empty((max_pos, d_rope // 2), np.float32)
        sin = self.empty((max_pos, d_rope // 2), np.float32)
        self.check("mla_rope_table", self.lib.mla_rope_table(cos.ctypes.data, sin.ctypes.data,
                                                             max_pos, d_rope, 10000.0))
        return cos, sin


class EmuStep:
    """One decode / prefill step of a synthetic workload through the emulated
    library, mirroring the device step: history appended first (untimed set-up),
    then absorb -> append (new tokens, with q_pe) -> decode -> out_proj.  With
    ``kv_scale`` set, the cache is e4m3 under that scale (the fp8 calls)."""

    def __init__(self, emu: Emu, inp: Inputs, num_workgroups: int = 0,
                 kv_scale: Optional[float] = None):
        self.emu, self.inp = emu, inp
        self.kv_scale = kv_scale
        self.d = d = inp.dims
        self.cfg = B.MlaConfig.from_dims(d, BLOCK_SIZE)
        self.num_workgroups = num_workgroups
        st = np.uint16 if d.dtype == "bf16" else np.float32
        H, dc, dr, dv = d.num_heads, d.d_latent, d.d_rope, d.d_v
        T = inp.T
        put = emu.put
        self.w_uk, self.w_uv = put(inp.w_uk), put(inp.w_uv)
        self.q_nope, self.q_pe = put(inp.q_nope), put(inp.q_pe)
        seqs, pos, ck, kp = inp.new_tokens()
        self.new = (put(ck), put(kp), put(seqs.astype(np.int32)), put(pos.astype(np.int32)))
        self.block_table = put(inp.block_table.astype(np.int32))
        self.q_start = put(inp.q_start.astype(np.int32))
        self.kv_lens = put(inp.kv_lens.astype(np.int32))
        self.cos, self.sin = emu.rope_table(max(inp.max_pos(), 1), dr)
        self.num_blocks = inp.num_blocks
        rows = inp.num_blocks * BLOCK_SIZE
        self.pool = emu.empty((rows, d.row), np.uint8 if kv_scale else st)
        if kv_scale:
            self.pool[...] = 0x7F
        elif d.dtype == "bf16":
            self.pool.view(np.uint16)[...] = SENTINEL_BF16
        else:
            self.pool.view(np.uint32)[...] = SENTINEL_F32
        self.q_lat = emu.empty((T, H, dc + dr), st)
        self.o_lat = emu.empty((T, H, dc), st)
        self.out = emu.empty((T, H, dv), np.float32)
        self.dev_error = emu.empty((1,), np.uint32)
        nbytes = emu.workspace_size(self.cfg, inp.q_start, inp.kv_lens, inp.workload.causal,
                                    num_workgroups)
        self.workspace = emu.empty((nbytes,), np.uint8) if nbytes else None
        hs, hp, hck, hkp = inp.history()
        if len(hs) and kv_scale:
            emu.append_fp8(self.cfg, put(hck), put(hkp), None, put(hs.astype(np.int32)),
                           put(hp.astype(np.int32)), self.block_table, self.num_blocks,
                           self.cos, self.sin, kv_scale, self.pool, dev_error=self.dev_error)
        elif len(hs):
            emu.append(self.cfg, put(hck), put(hkp), None, put(hs.astype(np.int32)),
                       put(hp.astype(np.int32)), self.block_table, self.num_blocks, self.cos,
                       self.sin, self.pool, dev_error=self.dev_error)

    def absorb(self):
        self.emu.absorb_q(self.cfg, self.q_nope, self.w_uk, self.q_lat)

    def append(self):
        ck, kp, seq, pos = self.new
        if self.kv_scale:
            self.emu.append_fp8(self.cfg, ck, kp, self.q_pe, seq, pos, self.block_table,
                                self.num_blocks, self.cos, self.sin, self.kv_scale, self.pool,
                                self.q_lat, self.dev_error)
            return
        self.emu.append(self.cfg, ck, kp, self.q_pe, seq, pos, self.block_table,
                        self.num_blocks, self.cos, self.sin, self.pool, self.q_lat,
                        self.dev_error)

    def decode(self, num_workgroups: Optional[int] = None):
        ws = self.workspace
        nwg = self.num_workgroups if num_workgroups is None else num_workgroups
        if nwg != self.num_workgroups:
            nbytes = self.emu.workspace_size(self.cfg, self.inp.q_start, self.inp.kv_lens,
                                             self.inp.workload.causal, nwg)
            ws = self.emu.empty((nbytes,), np.uint8) if nbytes else None
        if self.kv_scale:
            self.emu.decode_fp8(self.cfg, self.q_start, self.kv_lens, self.block_table,
                                self.num_blocks, self.q_lat, self.pool, self.kv_scale,
                                self.inp.workload.causal, self.o_lat, ws, nwg, self.dev_error)
            return
        self.emu.decode(self.cfg, self.q_start, self.kv_lens, self.block_table,
                        self.num_blocks, self.q_lat, self.pool, self.inp.workload.causal,
                        self.o_lat, ws, nwg, self.dev_error)

    def project(self):
        self.emu.out_proj(self.cfg, self.o_lat, self.w_uv, self.out)

    def run(self):
        self.absorb()
        self.append()
        self.decode()
        self.project()
