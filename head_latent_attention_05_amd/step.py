"""Device-resident decode/prefill step over libmla (torch supplies memory and streams).

``DeviceStep(inputs)`` uploads one step's synthetic inputs, fills the paged
latent cache with the history tokens, and ``run()`` enqueues the four library
calls of the step:

    mla_absorb_q -> mla_append_cache (new tokens, with q_pe) -> mla_decode -> mla_out_proj

With ``kv_scale`` set the cache is e4m3 (576 bytes per token) under that
power-of-two scale, and the append and decode calls are their fp8 forms.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import binding as B
from .synth import BLOCK_SIZE, Inputs

SENTINEL_BF16 = 0x7FC1
SENTINEL_F32 = 0x7FC00001
SENTINEL_FP8 = 0x7F


def to_device(arr: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Upload a storage array (uint16 bf16 bits or float32) as a torch tensor."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16))
        return t.to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr, np.float32)).to(device)


def to_host(t: torch.Tensor, dtype: str) -> np.ndarray:
    """Download a storage tensor as uint16 bf16 bits or float32."""
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


class DeviceStep:
    def __init__(self, inp: Inputs, device: str = "cuda:0", num_workgroups: int = 0,
                 pool_copies: int = 1, history_chunk: int = 32768,
                 kv_scale: Optional[float] = None):
        self.inp = inp
        self.kv_scale = kv_scale
        self.d = d = inp.dims
        self.dev = torch.device(device)
        self.cfg = B.MlaConfig.from_dims(d, BLOCK_SIZE)
        self.num_workgroups = num_workgroups
        dt = d.dtype
        self.tdt = torch.bfloat16 if dt == "bf16" else torch.float32
        H, dc, dr, dv = d.num_heads, d.d_latent, d.d_rope, d.d_v
        T = inp.T
        self.T = T
        self.causal = inp.workload.causal
        up = lambda a: to_device(a, dt, self.dev)
        self.w_uk, self.w_uv = up(inp.w_uk), up(inp.w_uv)
        self.q_nope, self.q_pe = up(inp.q_nope), up(inp.q_pe)
        seqs, pos, ck, kp = inp.new_tokens()
        self.new_seq = torch.from_numpy(seqs).to(self.dev)
        self.new_pos = torch.from_numpy(pos).to(self.dev)
        self.new_ckv, self.new_kpe = up(ck), up(kp)
        self.block_table = torch.from_numpy(inp.block_table).to(self.dev)
        self.q_start_host = inp.q_start.astype(np.int32)
        self.kv_lens_host = inp.kv_lens.astype(np.int32)
        self.q_start = torch.from_numpy(self.q_start_host).to(self.dev)
        self.kv_lens = torch.from_numpy(self.kv_lens_host).to(self.dev)
        self.max_pos = max(inp.max_pos(), 1)
        cos, sin = B.rope_table(self.max_pos, dr)
        self.rope_cos = torch.from_numpy(cos).to(self.dev)
        self.rope_sin = torch.from_numpy(sin).to(self.dev)
        self.num_blocks = inp.num_blocks
        rows = inp.num_blocks * BLOCK_SIZE
        self.pools = [self._new_pool(rows) for _ in range(pool_copies)]
        self.pool = self.pools[0]
        self.q_lat = torch.zeros((T, H, dc + dr), dtype=self.tdt, device=self.dev)
        self.o_lat = torch.zeros((T, H, dc), dtype=self.tdt, device=self.dev)
        self.out = torch.zeros((T, H, dv), dtype=torch.float32, device=self.dev)
        self.dev_error = torch.zeros(1, dtype=torch.int32, device=self.dev)
        nbytes = B.decode_workspace_size(self.cfg, self.q_start_host, self.kv_lens_host,
                                         self.causal, num_workgroups)
        self.workspace = (torch.empty(max(nbytes, 16), dtype=torch.uint8, device=self.dev)
                          if nbytes else None)
        self.history_chunk = history_chunk
        for p in self.pools:
            self.fill_history(p)

    def _new_pool(self, rows: int) -> torch.Tensor:
        d = self.d
        if self.kv_scale:
            return torch.full((rows, d.row), SENTINEL_FP8, dtype=torch.uint8, device=self.dev)
        if d.dtype == "bf16":
            t = torch.full((rows, d.row), SENTINEL_BF16, dtype=torch.int16, device=self.dev)
            return t.view(torch.bfloat16)
        t = torch.full((rows, d.row), SENTINEL_F32, dtype=torch.int32, device=self.dev)
        return t.view(torch.float32)

    def fill_history(self, pool: torch.Tensor) -> None:
        """Append every history token (untimed set-up), in chunks."""
        seqs, pos, ck, kp = self.inp.history()
        n = len(seqs)
        for a in range(0, n, self.history_chunk):
            b = min(n, a + self.history_chunk)
            if self.kv_scale:
                B.append_cache_fp8(self.cfg, to_device(ck[a:b], self.d.dtype, self.dev),
                                   to_device(kp[a:b], self.d.dtype, self.dev), None,
                                   torch.from_numpy(seqs[a:b]).to(self.dev),
                                   torch.from_numpy(pos[a:b]).to(self.dev), self.block_table,
                                   self.num_blocks, self.rope_cos, self.rope_sin, self.kv_scale,
                                   pool, dev_error=self.dev_error)
                continue
            B.append_cache(self.cfg, to_device(ck[a:b], self.d.dtype, self.dev),
                           to_device(kp[a:b], self.d.dtype, self.dev), None,
                           torch.from_numpy(seqs[a:b]).to(self.dev),
                           torch.from_numpy(pos[a:b]).to(self.dev), self.block_table,
                           self.num_blocks, self.rope_cos, self.rope_sin, pool,
                           dev_error=self.dev_error)
        torch.cuda.synchronize(self.dev)

    # -- the four calls -------------------------------------------------------
    def absorb(self) -> None:
        B.absorb_q(self.cfg, self.q_nope, self.w_uk, self.q_lat)

    def append(self, pool: Optional[torch.Tensor] = None) -> None:
        if self.kv_scale:
            B.append_cache_fp8(self.cfg, self.new_ckv, self.new_kpe, self.q_pe, self.new_seq,
                               self.new_pos, self.block_table, self.num_blocks, self.rope_cos,
                               self.rope_sin, self.kv_scale, self.pool if pool is None else pool,
                               self.q_lat, dev_error=self.dev_error)
            return
        B.append_cache(self.cfg, self.new_ckv, self.new_kpe, self.q_pe, self.new_seq,
                       self.new_pos, self.block_table, self.num_blocks, self.rope_cos,
                       self.rope_sin, self.pool if pool is None else pool, self.q_lat,
                       dev_error=self.dev_error)

    def decode(self, pool: Optional[torch.Tensor] = None, q_lat=None, o_lat=None) -> None:
        if self.kv_scale:
            B.decode_fp8(self.cfg, self.q_start, self.kv_lens, self.q_start_host,
                         self.kv_lens_host, self.block_table, self.num_blocks,
                         self.q_lat if q_lat is None else q_lat,
                         self.pool if pool is None else pool, self.kv_scale, self.causal,
                         self.o_lat if o_lat is None else o_lat, workspace=self.workspace,
                         num_workgroups=self.num_workgroups, dev_error=self.dev_error)
            return
        B.decode(self.cfg, self.q_start, self.kv_lens, self.q_start_host, self.kv_lens_host,
                 self.block_table, self.num_blocks, self.q_lat if q_lat is None else q_lat,
                 self.pool if pool is None else pool, self.causal,
                 self.o_lat if o_lat is None else o_lat, workspace=self.workspace,
                 num_workgroups=self.num_workgroups, dev_error=self.dev_error)

    def project(self) -> None:
        B.out_proj(self.cfg, self.o_lat, self.w_uv, self.out)

    def run(self, pool: Optional[torch.Tensor] = None) -> None:
        """One full step on the current stream."""
        self.absorb()
        self.append(pool)
        self.decode(pool)
        self.project()
