"""CPU oracle for MLA decode with weight absorption -- TEST INFRASTRUCTURE ONLY.

Plain, slow and (meant to be) obviously correct numpy code, in float64 except
where the cache contract fixes a storage precision.  It shares no code with the
HIP library and must only be imported by the tests, by the smoke check and by
the benchmark's CPU-baseline leg; the product path never routes through it.

Sources (web pages; cited by page and section):

* [MLA explainer]  xxmr.cn/news/206254 -- sections "MLA的计算过程" (stage 2A:
  explicit decompression; stage 2B: absorption) and "MLA的实现" (``RoPE``
  module, ``forward_training``, ``forward_inference_absorbed``, self-test).
* [MLA architecture]  intelliparadigm.com, "MLA架构：低秩注意力机制优化LLM显存与计算效率"
  -- section 1 (128 heads, qk dim 192 = 128 no-RoPE + 64 RoPE, 576-value cache
  = 512 + 64), 2.2 (joint KV projection), 3.1 (absorption is associativity),
  3.2 (two cache parts: 512-d latent and shared 64-d RoPE key), 4.2
  (pre-allocated cache, fused RoPE + cache update).
* [MLA deep dive]  mlqm.cn/news/500296 -- 2.3 (weight absorption), 5.1 (paged
  cache in serving frameworks).

Readings where the pages are silent:
rotate-half RoPE pairing with theta 10000; 0-based positions; scale
1/sqrt(d_nope + d_rope); exact max-subtracted softmax; causal mask for new
tokens; cache rows hold [c_kv | RoPE(k_pe)] in storage precision; the RoPE of
a cached key is computed in fp32 as ``x*cos - x2*sin`` / ``x2*cos + x*sin``
with every product and sum rounded to fp32 (no fused multiply-add) and then
rounded to bf16 (nearest-even) for bf16 caches.

Every function here is pinned by tests/test_oracle_pins.py against something
other than itself: closed forms of the RoPE table and rotation, brute-force
scalar loops, torch's scaled-dot-product attention, special cases, the
absorption identity, and, for the cache rows written by append_cache, an exact
fp64 rotation at each token's true position read back through the paged pool
plus the relative-position property of the scores; the weight-level
absorption by brute-force loops and its associativity with the per-head
calls; kv_down by brute-force
scalar loops, one-hot inputs and closed forms of the normalisation, and the
one-step bf16 rounding by constructed ties; the e4m3 cache by torch's own
float8_e4m3fn conversions, the format's closed-form values, constructed ties,
and the rotated RoPE columns read back against an exact fp64 rotation at each
token's true position; none is "parity unpinned".
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

ROPE_THETA = 10000.0


# ----------------------------------------------------------------------------
# storage precision helpers (own implementation; not shared with anything)
# ----------------------------------------------------------------------------

def to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    return ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def storage_to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_to_f64(x) if dtype == "bf16" else np.asarray(x, np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# RoPE  ([MLA explainer] "MLA的实现", RoPE module: inverse frequencies
# theta^(-2i/d), angles p * inv_freq duplicated over both halves, output
# x*cos + rotate_half(x)*sin with rotate_half(x) = [-x2, x1])
# ----------------------------------------------------------------------------

def rope_inv_freq(d_rope: int, theta: float = ROPE_THETA) -> np.ndarray:
    """inv_freq[i] = 1 / theta**(2i/d_rope), i < d_rope/2, in fp64."""
    return np.array([1.0 / (theta ** (2.0 * i / d_rope)) for i in range(d_rope // 2)],
                    dtype=np.float64)


def rope_angles(pos, d_rope: int, theta: float = ROPE_THETA) -> np.ndarray:
    """angle[p, i] = p * inv_freq[i] in fp64, shape [len(pos), d_rope/2]."""
    return np.outer(np.asarray(pos, dtype=np.float64), rope_inv_freq(d_rope, theta))


def rope_table_f32(max_pos: int, d_rope: int, theta: float = ROPE_THETA):
    """cos/sin tables [max_pos, d_rope/2]: fp64 angle and fp64 cos/sin (libm via
    Python's math module), rounded once to fp32."""
    inv = [float(v) for v in rope_inv_freq(d_rope, theta)]
    ang = [float(p) * f for p in range(max_pos) for f in inv]
    shape = (max_pos, d_rope // 2)
    cos = np.array([math.cos(a) for a in ang], np.float64).astype(np.float32).reshape(shape)
    sin = np.array([math.sin(a) for a in ang], np.float64).astype(np.float32).reshape(shape)
    return cos, sin


def rope_f64(x: np.ndarray, pos, d_rope: int, theta: float = ROPE_THETA) -> np.ndarray:
    """Exact (fp64) rotate-half RoPE of x[..., d_rope] at positions ``pos``
    (pos broadcasts against x.shape[:-1] after a trailing axis is added)."""
    x = np.asarray(x, np.float64)
    h = d_rope // 2
    ang = np.asarray(pos, np.float64)[..., None] * rope_inv_freq(d_rope, theta)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rope_cache_f32(x32: np.ndarray, cos32: np.ndarray, sin32: np.ndarray) -> np.ndarray:
    """RoPE of a cached key in fp32 with the contract's op order:
    y1 = x1*c - x2*s, y2 = x2*c + x1*s, every product and every sum rounded to
    fp32 (numpy float32 arithmetic is IEEE, no fused multiply-add)."""
    x32 = np.asarray(x32, np.float32)
    h = x32.shape[-1] // 2
    x1, x2 = x32[..., :h], x32[..., h:]
    c, s = np.asarray(cos32, np.float32), np.asarray(sin32, np.float32)
    y1 = (x1 * c).astype(np.float32) - (x2 * s).astype(np.float32)
    y2 = (x2 * c).astype(np.float32) + (x1 * s).astype(np.float32)
    return np.concatenate([y1.astype(np.float32), y2.astype(np.float32)], axis=-1)


# ----------------------------------------------------------------------------
# Paged latent cache  ([MLA architecture] 3.2 / 4.2: two parts per token,
# 512-d latent and the shared 64-d RoPE key, pre-allocated and written in
# place; [MLA deep dive] 5.1: paged blocks via a block table)
# ----------------------------------------------------------------------------

def slot_of(block_table: np.ndarray, seq: int, pos: int, block_size: int) -> int:
    """Physical row of (sequence, position): block_table[seq][pos // bs]*bs + pos % bs."""
    blk = int(block_table[seq, pos // block_size])
    if blk < 0:
        raise ValueError("position maps to an unassigned block")
    return blk * block_size + pos % block_size


def new_pool(num_blocks: int, block_size: int, row: int, dtype: str) -> np.ndarray:
    """A pool filled with a sentinel so stray or missing writes are visible:
    bf16 NaN payload 0x7FC1, or the fp32 NaN 0x7FC00001."""
    if dtype == "bf16":
        return np.full((num_blocks * block_size, row), 0x7FC1, np.uint16)
    return np.full((num_blocks * block_size, row), 0x7FC00001, np.uint32).view(np.float32)


def append_cache(pool: np.ndarray, dims, block_size: int, seqs, positions,
                 c_kv: np.ndarray, k_pe: np.ndarray, block_table: np.ndarray,
                 cos32: np.ndarray, sin32: np.ndarray) -> None:
    """Write one row per token: [c_kv (as stored) | RoPE(k_pe) at the token's
    position, rounded to the storage dtype] ([MLA explainer] forward_inference_absorbed
    caches c_kv and the rotated k_r; [MLA architecture] 4.2 fuses the two)."""
    dc = dims.d_latent
    positions = np.asarray(positions)
    slots = np.array([slot_of(block_table, int(b), int(p), block_size)
                      for b, p in zip(seqs, positions)], dtype=np.int64)
    if len(slots) == 0:
        return
    if dims.dtype == "bf16":
        x32 = bf16_to_f64(k_pe).astype(np.float32)
        y = to_bf16_bits(rope_cache_f32(x32, cos32[positions], sin32[positions]))
    else:
        y = rope_cache_f32(np.asarray(k_pe, np.float32), cos32[positions], sin32[positions])
    pool[slots, :dc] = c_kv
    pool[slots, dc:] = y


def gather_rows(pool: np.ndarray, dims, block_size: int, block_table: np.ndarray,
                seq: int, length: int) -> np.ndarray:
    """Logical rows 0..length-1 of one sequence, upcast to fp64 [length, d_c+d_r]."""
    idx = [slot_of(block_table, seq, p, block_size) for p in range(length)]
    return storage_to_f64(pool[idx], dims.dtype)



# ----------------------------------------------------------------------------
# fp8 (e4m3) latent cache  ([MLA architecture] 4.2, "量化的影响": a quantised
# cache halves the bytes per cached token, at a cost in numerical stability).
# Reading (the pages leave the format open): rows are stored as OCP e4m3
# (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; subnormals down to
# 2^-9; largest finite 448; 0x7F / 0xFF are NaN).  One power-of-two scale per
# cache: code = e4m3(x / kv_scale), value = kv_scale * decode(code).  Encoding
# rounds to nearest, ties to even, and saturates finite values at +-448.
# ----------------------------------------------------------------------------

E4M3_MAX = 448.0
E4M3_SENTINEL = 0x7F  # NaN: marks pool slots that were never written


def e4m3_to_f64(bits: np.ndarray) -> np.ndarray:
    """Value of each e4m3 code (uint8) in fp64; NaN codes give NaN."""
    b = np.asarray(bits, np.uint8).astype(np.int64)
    sign = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 3) & 15
    m = (b & 7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m, -9), np.ldexp(8.0 + m, e - 10))
    mag = np.where((e == 15) & ((b & 7) == 7), np.nan, mag)
    return sign * mag


def f32_to_e4m3_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 -> e4m3 code: round to nearest, ties to even, |x| clamped to 448
    first (saturation); NaN -> 0x7F.  The quantum is 2^(e-3) for a value in
    [2^e, 2^(e+1)), e >= -6, and 2^-9 below 2^-6 (subnormals)."""
    x = np.asarray(x32, np.float32).astype(np.float64)
    nan = np.isnan(x)
    x = np.where(nan, 0.0, x)
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    _, ex = np.frexp(a)                      # a = f * 2^ex, 0.5 <= f < 1
    e = np.maximum(ex - 1, -6)               # a in [2^e, 2^(e+1)) for normals
    quantum = np.ldexp(1.0, e - 3)
    q = np.rint(a / quantum) * quantum       # rint: half to even; exact in fp64
    q = np.minimum(q, E4M3_MAX)
    # encode q exactly
    _, qx = np.frexp(q)
    qe = np.maximum(qx - 1, -6)
    normal = q >= 2.0 ** -6
    mant = np.where(normal, q / np.ldexp(1.0, qe - 3) - 8.0, q / 2.0 ** -9)
    code = np.where(normal, ((qe + 7) << 3) + mant.astype(np.int64), mant.astype(np.int64))
    code = code.astype(np.int64) | np.where(neg & (q > 0), 0x80, 0)
    code = np.where(neg & (q == 0), 0x80, code)   # keep the sign of zero
    return np.where(nan, 0x7F, code).astype(np.uint8)


def new_pool_fp8(num_blocks: int, block_size: int, row: int) -> np.ndarray:
    """An e4m3 pool filled with the NaN sentinel 0x7F."""
    return np.full((num_blocks * block_size, row), E4M3_SENTINEL, np.uint8)


def append_cache_fp8(pool: np.ndarray, dims, block_size: int, seqs, positions,
                     c_kv: np.ndarray, k_pe: np.ndarray, block_table: np.ndarray,
                     cos32: np.ndarray, sin32: np.ndarray, kv_scale: float) -> None:
    """The fp8 form of append_cache: the token's c_kv (bf16 input, exact in
    fp32) and its RoPE-rotated k_pe (fp32, the same op order as the bf16 cache,
    no intermediate bf16 rounding) are divided by the power-of-two kv_scale
    (exact) and rounded once to e4m3."""
    check_kv_scale(kv_scale)
    dc = dims.d_latent
    positions = np.asarray(positions)
    slots = np.array([slot_of(block_table, int(b), int(p), block_size)
                      for b, p in zip(seqs, positions)], dtype=np.int64)
    if len(slots) == 0:
        return
    inv = np.float32(1.0 / kv_scale)
    c32 = bf16_to_f64(c_kv).astype(np.float32)
    x32 = bf16_to_f64(k_pe).astype(np.float32)
    y32 = rope_cache_f32(x32, cos32[positions], sin32[positions])
    pool[slots, :dc] = f32_to_e4m3_bits((c32 * inv).astype(np.float32))
    pool[slots, dc:] = f32_to_e4m3_bits((y32 * inv).astype(np.float32))


def check_kv_scale(kv_scale: float) -> None:
    m, _ = math.frexp(float(kv_scale))
    if not (kv_scale > 0 and m == 0.5 and 2.0 ** -60 <= kv_scale <= 2.0 ** 60):
        raise ValueError("kv_scale must be a power of two in [2^-60, 2^60]")


def gather_rows_fp8(pool: np.ndarray, dims, block_size: int, block_table: np.ndarray,
                    seq: int, length: int, kv_scale: float) -> np.ndarray:
    """Logical rows 0..length-1 of one sequence of an e4m3 pool, dequantised
    to fp64: kv_scale * decode(code)."""
    idx = [slot_of(block_table, seq, p, block_size) for p in range(length)]
    return kv_scale * e4m3_to_f64(pool[idx])

# ----------------------------------------------------------------------------
# Attention
# ----------------------------------------------------------------------------

def softmax_f64(s: np.ndarray) -> np.ndarray:
    """Exact softmax along the last axis, max-subtracted; -inf entries get 0."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def scale_of(dims) -> float:
    """1/sqrt(d_nope + d_rope): [MLA explainer] "MLA的实现" sets the dot-product
    scale from the no-RoPE plus RoPE head width (192 for V3)."""
    return 1.0 / math.sqrt(dims.d_nope + dims.d_rope)


def naive_mla(dims, w_uk, w_uv, q_nope, q_pe, rows_of_seq, kv_lens, q_start,
              causal: bool, heads: Optional[list] = None) -> np.ndarray:
    """Naive MLA with explicit decompression ([MLA explainer] stage 2A and
    forward_training): per head, K_t = [W_UK[h] c_kv_t | k_pe_t] (the shared
    RoPE key broadcast to every head), V_t = W_UV[h] c_kv_t, q = [q_nope |
    RoPE(q_pe)], standard softmax attention with scale 1/sqrt(d_n + d_r).

    rows_of_seq(b) returns that sequence's cached rows [L_b, d_c+d_r] in fp64
    (c_kv then the already-rotated k_pe).  Query j of sequence b sits at
    position L_b - q_len_b + j; with ``causal`` it sees positions <= its own
    (decode queries are the last token, so they see every row either way).
    Returns out [T, H', d_v] in fp64 for the requested heads (default all)."""
    dt = dims.dtype
    dc, dn = dims.d_latent, dims.d_nope
    heads = list(range(dims.num_heads)) if heads is None else list(heads)
    Wk = storage_to_f64(w_uk, dt)
    Wv = storage_to_f64(w_uv, dt)
    qn = storage_to_f64(q_nope, dt)
    qp = storage_to_f64(q_pe, dt)
    T = int(q_start[-1])
    out = np.zeros((T, len(heads), dims.d_v))
    scale = scale_of(dims)
    for b in range(len(kv_lens)):
        L = int(kv_lens[b])
        t0, t1 = int(q_start[b]), int(q_start[b + 1])
        if t1 == t0:
            continue
        rows = rows_of_seq(b)
        ckv, kpe = rows[:L, :dc], rows[:L, dc:]
        qpos = np.arange(L - (t1 - t0), L)
        for hi, h in enumerate(heads):
            K = np.concatenate([ckv @ Wk[h].T, kpe], axis=1)           # [L, d_n+d_r]
            V = ckv @ Wv[h].T                                            # [L, d_v]
            q = np.concatenate([qn[t0:t1, h], rope_f64(qp[t0:t1, h], qpos, dims.d_rope)],
                               axis=1)                                   # [q, d_n+d_r]
            s = (q @ K.T) * scale                                        # [q, L]
            if causal:
                s = np.where(np.arange(L)[None, :] <= qpos[:, None], s, -np.inf)
            out[t0:t1, hi] = softmax_f64(s) @ V
    return out


# ----- absorbed form, one function per library call ([MLA explainer] stage 2B
# and forward_inference_absorbed; [MLA architecture] 3.1; [MLA deep dive] 2.3)

def absorb_q(dims, q_nope, w_uk) -> np.ndarray:
    """q_lat[t,h,c] = sum_d q_nope[t,h,d] * W_UK[h,d,c]  (fp64) [T, H, d_c]."""
    dt = dims.dtype
    return np.einsum("thd,hdc->thc", storage_to_f64(q_nope, dt), storage_to_f64(w_uk, dt))


def rope_queries(dims, q_pe, positions) -> np.ndarray:
    """RoPE(q_pe) per head at each query token's position (fp64) [T, H, d_r]."""
    qp = storage_to_f64(q_pe, dims.dtype)
    return rope_f64(qp, np.asarray(positions)[:, None], dims.d_rope)


def latent_decode(dims, q_lat, rows_of_seq, kv_lens, q_start, causal: bool,
                  heads: Optional[list] = None) -> np.ndarray:
    """Absorbed attention over latent rows: s_j = (q_lat . row_j) * scale over
    all d_c + d_r columns (latent score plus RoPE score), p = softmax(s),
    o_lat = sum_j p_j c_kv_j.  q_lat is fp64 [T, H, d_c+d_r]; returns fp64
    o_lat [T, H', d_c]."""
    dc = dims.d_latent
    heads = list(range(dims.num_heads)) if heads is None else list(heads)
    T = int(q_start[-1])
    out = np.zeros((T, len(heads), dc))
    scale = scale_of(dims)
    for b in range(len(kv_lens)):
        L = int(kv_lens[b])
        t0, t1 = int(q_start[b]), int(q_start[b + 1])
        if t1 == t0:
            continue
        rows = rows_of_seq(b)[:L]
        qpos = np.arange(L - (t1 - t0), L)
        for hi, h in enumerate(heads):
            s = (q_lat[t0:t1, h] @ rows.T) * scale
            if causal:
                s = np.where(np.arange(L)[None, :] <= qpos[:, None], s, -np.inf)
            out[t0:t1, hi] = softmax_f64(s) @ rows[:, :dc]
    return out


def out_proj(dims, o_lat_f64, w_uv, heads: Optional[list] = None) -> np.ndarray:
    """out[t,h,v] = sum_c W_UV[h,v,c] * o_lat[t,h,c]  (fp64) [T, H', d_v]."""
    W = storage_to_f64(w_uv, dims.dtype)
    if heads is not None:
        W = W[list(heads)]
    return np.einsum("thc,hvc->thv", o_lat_f64, W)


def absorbed_mla(dims, w_uk, w_uv, q_nope, q_pe, rows_of_seq, kv_lens, q_start,
                 causal: bool, heads: Optional[list] = None):
    """Composition absorb_q -> RoPE(q_pe) -> latent_decode -> out_proj, all fp64.
    Returns (out [T,H',d_v], o_lat [T,H',d_c])."""
    pos = []
    for b in range(len(kv_lens)):
        q = int(q_start[b + 1] - q_start[b])
        pos.extend(range(int(kv_lens[b]) - q, int(kv_lens[b])))
    pos = np.asarray(pos, np.int64)
    q_lat = np.concatenate([absorb_q(dims, q_nope, w_uk),
                            rope_queries(dims, q_pe, pos)], axis=-1)
    o_lat = latent_decode(dims, q_lat, rows_of_seq, kv_lens, q_start, causal, heads)
    return out_proj(dims, o_lat, w_uv, heads), o_lat


# ----------------------------------------------------------------------------
# Weight-level absorption ([MLA explainer] forward_inference_absorbed:
# w_q_absorbed = W_UQ^T W_UK per head, so the compressed query c_q maps straight
# into the latent space; w_o_absorbed = W_UV^T W_O per head, so the attended
# latent maps straight to the model width with the sum over heads;
# "MLA的常见问题" Q3; [MLA architecture] 3.1)
# ----------------------------------------------------------------------------

def fuse_q_weight(dims, w_uq, w_uk) -> np.ndarray:
    """W_KQ[h, j, c] = sum_d W_UQ[h, d, j] * W_UK[h, d, c]  (fp64) [H, d_cq, d_c].
    W_UQ [H, d_n, d_cq] maps c_q to the no-RoPE query: q_nope[t,h,d] =
    sum_j W_UQ[h,d,j] c_q[t,j]."""
    dt = dims.dtype
    return np.einsum("hdj,hdc->hjc", storage_to_f64(w_uq, dt), storage_to_f64(w_uk, dt))


def fuse_o_weight(dims, w_uv, w_o) -> np.ndarray:
    """W_OV[h, c, m] = sum_v W_UV[h, v, c] * W_O[m, h, v]  (fp64) [H, d_c, d_model].
    W_O [d_model, H, d_v] is the output projection over the concatenated heads."""
    dt = dims.dtype
    return np.einsum("hvc,mhv->hcm", storage_to_f64(w_uv, dt), storage_to_f64(w_o, dt))


def absorb_q_fused(dims, c_q, w_kq) -> np.ndarray:
    """q_lat[t, h, c] = sum_j c_q[t, j] * W_KQ[h, j, c]  (fp64) [T, H, d_c]."""
    dt = dims.dtype
    return np.einsum("tj,hjc->thc", storage_to_f64(c_q, dt), storage_to_f64(w_kq, dt))


def out_proj_fused(dims, o_lat_f64, w_ov, cols: Optional[list] = None) -> np.ndarray:
    """out[t, m] = sum_h sum_c o_lat[t, h, c] * W_OV[h, c, m]  (fp64) [T, d_model],
    or only the columns m in ``cols``."""
    w = np.asarray(w_ov)
    if cols is not None:
        w = w[:, :, list(cols)]
    return np.einsum("thc,hcm->tm", np.asarray(o_lat_f64, np.float64),
                     storage_to_f64(w, dims.dtype))


# ----------------------------------------------------------------------------
# Upstream of the cache: joint KV down-projection and latent RMSNorm
# ([MLA architecture] 2.2: kv_a_proj_with_mqa maps the hidden state to
# d_c + d_r = 576 values, the 512-d latent part goes through an RMSNorm,
# kv_a_layernorm; the remaining 64 are the shared RoPE key before rotation)
# ----------------------------------------------------------------------------

def f64_to_bf16_bits(y: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bits, round to nearest, ties to even, in one step (no
    intermediate fp32 rounding).  Finite normal inputs or zero."""
    y = np.asarray(y, np.float64)
    m, e = np.frexp(y)                      # y = m * 2^e, 0.5 <= |m| < 1
    q = np.rint(m * 256.0)                  # 8 significant bits, half to even
    v = np.ldexp(q, e - 8)                  # exactly representable in bf16
    return to_bf16_bits(v.astype(np.float32))


def round_storage(y: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 values rounded once to the storage dtype (bf16 bits or fp32)."""
    return f64_to_bf16_bits(y) if dtype == "bf16" else np.asarray(y, np.float64).astype(np.float32)


def rms_norm(c: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis in fp64: gamma * c / sqrt(mean(c^2) + eps)."""
    c = np.asarray(c, np.float64)
    return np.asarray(gamma, np.float64) * c / np.sqrt(np.mean(c * c, axis=-1, keepdims=True) + eps)


def kv_down(dims, x, w_dkv, b_dkv, gamma, eps: float):
    """The cache inputs of new tokens from their hidden states x [T, d_model]:
    y = x W_DKV^T (+ b), W_DKV [d_c + d_r, d_model] (a linear layer's weight);
    y is a tensor of the model, so it is rounded to the storage dtype; the
    latent part is RMS-normalised with gain gamma [d_c] and rounded again.
    Returns (c_kv [T, d_c], k_pe [T, d_r]) in storage form, ready for
    append_cache (which rotates k_pe)."""
    dt, dc = dims.dtype, dims.d_latent
    y = storage_to_f64(x, dt) @ storage_to_f64(w_dkv, dt).T
    if b_dkv is not None:
        y = y + storage_to_f64(b_dkv, dt)
    kv = round_storage(y, dt)
    c = storage_to_f64(kv, dt)[:, :dc]
    c_kv = round_storage(rms_norm(c, storage_to_f64(gamma, dt), eps), dt)
    return c_kv, kv[:, dc:]


# ----------------------------------------------------------------------------
# Whole step on synthetic inputs
# ----------------------------------------------------------------------------

def build_pool(inp, block_size: int = 64, cos32=None, sin32=None,
               which: str = "all") -> np.ndarray:
    """The oracle's own cache after history and (optionally) the step's new
    tokens were appended.  ``which`` is "all", "history" or "new" (new tokens
    on top of the history)."""
    d = inp.dims
    if cos32 is None:
        cos32, sin32 = rope_table_f32(inp.max_pos(), d.d_rope)
    pool = new_pool(inp.num_blocks, block_size, d.row, d.dtype)
    if which in ("all", "history"):
        s, p, ck, kp = inp.history()
        append_cache(pool, d, block_size, s, p, ck, kp, inp.block_table, cos32, sin32)
    if which == "all":
        s, p, ck, kp = inp.new_tokens()
        append_cache(pool, d, block_size, s, p, ck, kp, inp.block_table, cos32, sin32)
    return pool


def build_pool_fp8(inp, kv_scale: float, block_size: int = 64, cos32=None, sin32=None,
                   which: str = "all") -> np.ndarray:
    """build_pool for an e4m3 cache (bf16 inputs only)."""
    d = inp.dims
    if d.dtype != "bf16":
        raise ValueError("the fp8 cache is built from bf16 inputs")
    if cos32 is None:
        cos32, sin32 = rope_table_f32(inp.max_pos(), d.d_rope)
    pool = new_pool_fp8(inp.num_blocks, block_size, d.row)
    if which in ("all", "history"):
        s, p, ck, kp = inp.history()
        append_cache_fp8(pool, d, block_size, s, p, ck, kp, inp.block_table, cos32, sin32,
                         kv_scale)
    if which == "all":
        s, p, ck, kp = inp.new_tokens()
        append_cache_fp8(pool, d, block_size, s, p, ck, kp, inp.block_table, cos32, sin32,
                         kv_scale)
    return pool


def step_fp8(inp, kv_scale: float, heads: Optional[list] = None, block_size: int = 64):
    """Full step over an e4m3 cache: append every token, then naive attention
    over the dequantised rows.  Returns (out fp64 [T,H',d_v], pool)."""
    pool = build_pool_fp8(inp, kv_scale, block_size)
    rows = lambda b: gather_rows_fp8(pool, inp.dims, block_size, inp.block_table, b,
                                     int(inp.kv_lens[b]), kv_scale)
    out = naive_mla(inp.dims, inp.w_uk, inp.w_uv, inp.q_nope, inp.q_pe, rows,
                    inp.kv_lens, inp.q_start, inp.workload.causal, heads)
    return out, pool


def step(inp, heads: Optional[list] = None, block_size: int = 64):
    """Full step: append every token, then naive attention.  Returns
    (out fp64 [T,H',d_v], pool)."""
    pool = build_pool(inp, block_size)
    rows = lambda b: gather_rows(pool, inp.dims, block_size, inp.block_table, b,
                                 int(inp.kv_lens[b]))
    out = naive_mla(inp.dims, inp.w_uk, inp.w_uv, inp.q_nope, inp.q_pe, rows,
                    inp.kv_lens, inp.q_start, inp.workload.causal, heads)
    return out, pool
