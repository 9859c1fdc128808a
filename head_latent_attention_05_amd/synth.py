"""Seeded synthetic inputs for MLA decode / chunked prefill.

This module only *draws* inputs: random weights, latent rows, queries, sequence
lengths and a shuffled paged-cache block table.  It contains none of the
method's arithmetic (no RoPE, no attention, no absorption); both the HIP path
and the CPU oracle receive exactly the arrays produced here.

Workloads (DeepSeek-V3 decode shapes: 128 heads, 512-d latent ``c_kv``, 64-d
decoupled-RoPE key, 128-d no-RoPE query part and 128-d value heads):

* ``tiny``      fp32, 4 heads, d_c=64, d_r=16, d_n=32, d_v=32, one sequence of
                128 tokens, one decode query.
* ``single``    V3 shapes, bf16 cache, one sequence of 4096 tokens.
* ``batch64``   V3 shapes, 64 sequences, lengths uniform in [1024, 8192].
* ``long``      V3 shapes, 4 sequences of 32768 tokens.
* ``prefill``   V3 shapes, 2 sequences, 15872 cached + 512 new causal queries.

Distributions: weights ~ N(0, std=1/sqrt(d_c)); c_kv ~ N(0,1) then
RMS-normalised per token (unit weight, eps 1e-6, in fp64); k_pe, q_nope,
q_pe ~ N(0,1).  Values are drawn in fp64, cast to fp32 and, for bf16
workloads, rounded to bf16 (round-to-nearest-even).  bf16 arrays are carried
as uint16 bit patterns.

Sequence b attends ``kv_lens[b]`` rows; its last ``q_lens[b]`` tokens are the
*new* tokens of the step (appended by the step itself, then attended as
queries).  The first ``kv_lens[b] - q_lens[b]`` tokens are history, written
to the cache before the step.  Positions are 0-based token indices.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

BLOCK_SIZE = 64


@dataclasses.dataclass(frozen=True)
class Dims:
    num_heads: int
    d_latent: int
    d_rope: int
    d_nope: int
    d_v: int
    dtype: str  # "bf16" or "f32": storage dtype of cache/queries/weights

    @property
    def row(self) -> int:
        return self.d_latent + self.d_rope


V3 = Dims(num_heads=128, d_latent=512, d_rope=64, d_nope=128, d_v=128, dtype="bf16")
TINY = Dims(num_heads=4, d_latent=64, d_rope=16, d_nope=32, d_v=32, dtype="f32")


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    dims: Dims
    batch: int
    kv_len: Optional[int]  # fixed attended length, or None for the uniform range
    kv_len_range: Optional[tuple]  # inclusive (lo, hi) for random lengths
    q_len: int
    causal: bool
    description: str


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 1, TINY, 1, 128, None, 1, False,
                     "tiny MLA decode, fp32: 1 sequence x 128 tokens, 4 heads, d_c=64"),
    "single": Workload("single", 2, V3, 1, 4096, None, 1, False,
                       "V3 shapes, 1 sequence x 4096 tokens, bf16 cache, 1 decode query"),
    "batch64": Workload("batch64", 3, V3, 64, None, (1024, 8192), 1, False,
                        "V3 shapes, 64 sequences, lengths U[1024,8192], paged bf16 cache"),
    "long": Workload("long", 4, V3, 4, 32768, None, 1, False,
                     "V3 shapes, 4 sequences x 32768 tokens, paged bf16 cache"),
    "prefill": Workload("prefill", 5, V3, 2, 16384, None, 512, True,
                        "V3 shapes, 2 sequences: 15872 cached + 512 new causal queries"),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits.
    Inputs here are finite, so no NaN handling is needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    return f32_to_bf16_bits(x32) if dtype == "bf16" else x32


def _rms_normalise(c: np.ndarray) -> np.ndarray:
    return c / np.sqrt(np.mean(c * c, axis=-1, keepdims=True) + 1e-6)


@dataclasses.dataclass
class Inputs:
    """One step's inputs.  Storage arrays are uint16 (bf16 bits) or float32."""
    workload: Workload
    dims: Dims
    kv_lens: np.ndarray        # int32 [B]  attended length per sequence
    q_lens: np.ndarray         # int32 [B]  new (query) tokens per sequence
    q_start: np.ndarray        # int32 [B+1] prefix sums of q_lens
    w_uk: np.ndarray           # [H, d_n, d_c]
    w_uv: np.ndarray           # [H, d_v, d_c]
    c_kv: List[np.ndarray]     # per sequence [L_b, d_c]
    k_pe: List[np.ndarray]     # per sequence [L_b, d_r] (before RoPE)
    q_nope: np.ndarray         # [T, H, d_n]
    q_pe: np.ndarray           # [T, H, d_r] (before RoPE)
    block_table: np.ndarray    # int32 [B, max_blocks]; unused = -1
    num_blocks: int            # physical blocks in the pool (includes spares)

    @property
    def T(self) -> int:
        return int(self.q_start[-1])

    def token_seq(self) -> np.ndarray:
        return np.repeat(np.arange(len(self.q_lens), dtype=np.int32), self.q_lens)

    def token_pos(self) -> np.ndarray:
        """Position of every new token (0-based), in query order."""
        out = []
        for b in range(len(self.q_lens)):
            L, q = int(self.kv_lens[b]), int(self.q_lens[b])
            out.append(np.arange(L - q, L, dtype=np.int32))
        return np.concatenate(out) if out else np.zeros(0, np.int32)

    def history(self):
        """(seq ids, positions, c_kv rows, k_pe rows) of the history tokens."""
        seqs, pos, ck, kp = [], [], [], []
        for b in range(len(self.q_lens)):
            h = int(self.kv_lens[b] - self.q_lens[b])
            seqs.append(np.full(h, b, np.int32))
            pos.append(np.arange(h, dtype=np.int32))
            ck.append(self.c_kv[b][:h])
            kp.append(self.k_pe[b][:h])
        return (np.concatenate(seqs), np.concatenate(pos),
                np.concatenate(ck), np.concatenate(kp))

    def new_tokens(self):
        """(seq ids, positions, c_kv rows, k_pe rows) of the step's new tokens."""
        ck, kp = [], []
        for b in range(len(self.q_lens)):
            L, q = int(self.kv_lens[b]), int(self.q_lens[b])
            ck.append(self.c_kv[b][L - q:L])
            kp.append(self.k_pe[b][L - q:L])
        return self.token_seq(), self.token_pos(), np.concatenate(ck), np.concatenate(kp)

    def max_pos(self) -> int:
        return int(self.kv_lens.max())


def make_inputs(workload: Workload | str, *, batch: Optional[int] = None,
                kv_lens: Optional[List[int]] = None, q_len: Optional[int] = None,
                seed: Optional[int] = None, spare_blocks: int = 2,
                dims: Optional[Dims] = None) -> Inputs:
    """Draw one step's inputs.  Overrides shrink a workload for fast tests while
    keeping its distributions; draw order is lengths, W_UK, W_UV, per-sequence
    (c_kv, k_pe), q_nope, q_pe, block permutation."""
    wl = WORKLOADS[workload] if isinstance(workload, str) else workload
    d = dims or wl.dims
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    B = batch if batch is not None else wl.batch
    ql = wl.q_len if q_len is None else q_len
    if kv_lens is not None:
        lens = np.asarray(kv_lens, dtype=np.int64)
        B = len(lens)
    elif wl.kv_len_range is not None:
        lo, hi = wl.kv_len_range
        lens = rng.integers(lo, hi + 1, size=B)
    else:
        lens = np.full(B, wl.kv_len, dtype=np.int64)
    lens = lens.astype(np.int32)
    q_lens = np.minimum(np.full(B, ql, np.int32), lens)
    q_start = np.zeros(B + 1, np.int32)
    q_start[1:] = np.cumsum(q_lens)
    H, dc, dr, dn, dv = d.num_heads, d.d_latent, d.d_rope, d.d_nope, d.d_v
    wstd = 1.0 / np.sqrt(dc)
    w_uk = _store(rng.standard_normal((H, dn, dc)) * wstd, d.dtype)
    w_uv = _store(rng.standard_normal((H, dv, dc)) * wstd, d.dtype)
    c_kv, k_pe = [], []
    for b in range(B):
        L = int(lens[b])
        c_kv.append(_store(_rms_normalise(rng.standard_normal((L, dc))), d.dtype))
        k_pe.append(_store(rng.standard_normal((L, dr)), d.dtype))
    T = int(q_start[-1])
    q_nope = _store(rng.standard_normal((T, H, dn)), d.dtype)
    q_pe = _store(rng.standard_normal((T, H, dr)), d.dtype)
    nblk = (lens.astype(np.int64) + BLOCK_SIZE - 1) // BLOCK_SIZE
    total = int(nblk.sum()) + spare_blocks
    perm = rng.permutation(total).astype(np.int32)
    maxb = int(nblk.max()) if B else 0
    bt = np.full((B, max(maxb, 1)), -1, np.int32)
    o = 0
    for b in range(B):
        n = int(nblk[b])
        bt[b, :n] = perm[o:o + n]
        o += n
    return Inputs(wl, d, lens, q_lens, q_start, w_uk, w_uv, c_kv, k_pe,
                  q_nope, q_pe, bt, total)


def random_latent_queries(dims: Dims, T: int, seed: int) -> np.ndarray:
    """Absorbed queries q_lat [T, H, d_c + d_r]: latent columns with the spread
    that W_UK^T q_nope has under the weight distribution above (std
    sqrt(d_n/d_c)), rope columns N(0,1).  Drives the decode call alone."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, dims.num_heads, dims.row))
    x[..., :dims.d_latent] *= np.sqrt(dims.d_nope / dims.d_latent)
    return _store(x, dims.dtype)


def random_latent_outputs(dims: Dims, T: int, seed: int) -> np.ndarray:
    """Latent attention outputs o_lat [T, H, d_c], used to drive the V
    up-projection call alone."""
    rng = np.random.default_rng(seed)
    return _store(rng.standard_normal((T, dims.num_heads, dims.d_latent)) * 0.05, dims.dtype)


@dataclasses.dataclass
class DownInputs:
    """Hidden states and weights of the joint KV down-projection (storage form)."""
    x: np.ndarray                 # [T, d_model]
    w_dkv: np.ndarray             # [d_c + d_r, d_model] (linear layer weight)
    b_dkv: Optional[np.ndarray]   # [d_c + d_r] or None
    gamma: np.ndarray             # [d_c] RMSNorm gain
    eps: float


def make_down_inputs(dims: Dims, T: int, d_model: int, seed: int, bias: bool = True,
                     eps: float = 1e-6) -> DownInputs:
    """x ~ N(0, 1); W_DKV ~ N(0, 1/d_model), so each projected value is about
    N(0, 1); bias ~ N(0, 0.1^2); gain ~ 1 + N(0, 0.1^2).  Draw order: x, W, b, gain."""
    rng = np.random.default_rng(seed)
    n = dims.d_latent + dims.d_rope
    x = _store(rng.standard_normal((T, d_model)), dims.dtype)
    w = _store(rng.standard_normal((n, d_model)) / np.sqrt(d_model), dims.dtype)
    b = _store(rng.standard_normal(n) * 0.1, dims.dtype)
    g = _store(1.0 + 0.1 * rng.standard_normal(dims.d_latent), dims.dtype)
    return DownInputs(x, w, b if bias else None, g, eps)


@dataclasses.dataclass
class FusedInputs:
    """Inputs of the weight-level absorbed calls (storage form)."""
    c_q: np.ndarray     # [T, d_cq] compressed queries
    w_kq: np.ndarray    # [H, d_cq, d_c] query-side fused weight
    o_lat: np.ndarray   # [T, H, d_c] attended latents
    w_ov: np.ndarray    # [H, d_c, d_model] output-side fused weight


def _normal_store(rng, shape, std: float, dtype: str) -> np.ndarray:
    """N(0, std^2) values in storage form, drawn in fp32 and converted in
    chunks (the fused weights run to hundreds of MB)."""
    n = int(np.prod(shape))
    out = np.empty(n, np.uint16 if dtype == "bf16" else np.float32)
    step = 1 << 24
    for a in range(0, n, step):
        x = rng.standard_normal(min(step, n - a), dtype=np.float32) * np.float32(std)
        if dtype == "bf16":
            u = x.view(np.uint32)   # finite, so u + 0x8000 does not wrap
            x = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
                 >> np.uint32(16)).astype(np.uint16)
        out[a:a + len(x)] = x
    return out.reshape(shape)


def make_fused_inputs(dims: Dims, T: int, d_cq: int, d_model: int, seed: int) -> FusedInputs:
    """Synthetic fused weights with the spread of the products they stand for:
    W_UQ ~ N(0, 1/d_cq) and W_UK ~ N(0, 1/d_c) give W_KQ entries of variance
    d_n / (d_cq d_c); W_UV ~ N(0, 1/d_c) and W_O ~ N(0, 1/(H d_v)) give W_OV
    entries of variance 1 / (d_c H).  c_q ~ N(0, 1); o_lat as
    random_latent_outputs.  Draw order: c_q, W_KQ, o_lat, W_OV."""
    rng = np.random.default_rng(seed)
    H, dc, dn, dt = dims.num_heads, dims.d_latent, dims.d_nope, dims.dtype
    c_q = _normal_store(rng, (T, d_cq), 1.0, dt)
    w_kq = _normal_store(rng, (H, d_cq, dc), float(np.sqrt(dn / (d_cq * dc))), dt)
    o_lat = _normal_store(rng, (T, H, dc), 0.05, dt)
    w_ov = _normal_store(rng, (H, dc, d_model), float(1.0 / np.sqrt(dc * H)), dt)
    return FusedInputs(c_q, w_kq, o_lat, w_ov)
