"""Shared helpers for the GPU parity tests (runs the HIP path and the oracle on
the same seeded inputs)."""
from __future__ import annotations

import dataclasses
import math

import numpy as np

from head_latent_attention_05_amd import synth
from oracle import mla_oracle as O

# tolerances on the step output out[T, H, d_v]
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
F32_REL = 1e-5


def check_out(dims, got: np.ndarray, ref: np.ndarray, label: str = "") -> dict:
    err = np.abs(got.astype(np.float64) - ref)
    stats = {"max_abs": float(err.max()), "mean_abs": float(err.mean()),
             "ref_max": float(np.abs(ref).max()),
             "rel_l2": float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))}
    print(f"[parity] {label} {stats}", flush=True)
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    if dims.dtype == "bf16":
        assert stats["max_abs"] <= BF16_MAX_ABS, (label, stats)
        assert stats["mean_abs"] <= BF16_MEAN_ABS, (label, stats)
        # not a gate from the spec, but a real bug (a dropped split, a wrong row)
        # moves the relative L2 error far above the bf16 rounding level
        assert stats["rel_l2"] <= 2e-2, (label, stats)
    else:
        assert stats["max_abs"] <= F32_REL * stats["ref_max"], (label, stats)
    return stats


def oracle_pool(inp, which="all"):
    return O.build_pool(inp, 64, which=which)


def rows_fn(pool, inp):
    return lambda b: O.gather_rows(pool, inp.dims, 64, inp.block_table, b, int(inp.kv_lens[b]))


# e4m3 cache: one power-of-two scale per cache, chosen so the synthetic rows
# (RMS-normalised latents, N(0,1) RoPE keys; magnitudes below about 6) use the
# format's upper range (codes up to about 96 of 448) and rarely its subnormals.
FP8_KV_SCALE = 2.0 ** -4


def oracle_pool_fp8(inp, kv_scale=FP8_KV_SCALE, which="all"):
    return O.build_pool_fp8(inp, kv_scale, 64, which=which)


def rows_fn_fp8(pool, inp, kv_scale=FP8_KV_SCALE):
    return lambda b: O.gather_rows_fp8(pool, inp.dims, 64, inp.block_table, b,
                                       int(inp.kv_lens[b]), kv_scale)


def pool_bits(pool_np, dims):
    return pool_np.view(np.uint16) if dims.dtype == "bf16" else pool_np.view(np.uint32)


def sample_heads(H: int, n: int = 6):
    if H <= n:
        return list(range(H))
    hs = {0, H - 1, H // 2}
    rng = np.random.default_rng(H)
    while len(hs) < n:
        hs.add(int(rng.integers(0, H)))
    return sorted(hs)


def sub_inputs(inp, seqs):
    """The same step restricted to a subset of sequences (for sampled oracle runs);
    rows are read from the full pool through the original block table rows."""
    q_lens = inp.q_lens[seqs]
    q_start = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    tok = np.concatenate([np.arange(inp.q_start[b], inp.q_start[b + 1]) for b in seqs])
    return q_start, tok


def drop_queries(inp, zero):
    """The same step with no query tokens for the sequences in `zero` (their
    rows all become history); the other sequences' queries are unchanged."""
    q_lens = inp.q_lens.copy()
    keep = np.concatenate([np.full(int(q), b not in zero) for b, q in enumerate(inp.q_lens)])
    q_lens[list(zero)] = 0
    q_start = np.zeros(len(q_lens) + 1, np.int32)
    q_start[1:] = np.cumsum(q_lens)
    return dataclasses.replace(inp, q_lens=q_lens, q_start=q_start, q_nope=inp.q_nope[keep],
                               q_pe=inp.q_pe[keep])


def scale_rows(inp, f):
    """The same step with every cached row of sequence b (c_kv and k_pe) scaled
    by f(b, position): drives the logits over a wide range."""
    c_kv, k_pe = [], []
    for b in range(len(inp.kv_lens)):
        s = np.array([f(b, p) for p in range(int(inp.kv_lens[b]))], np.float64)[:, None]
        cf = synth.bf16_bits_to_f32(inp.c_kv[b]).astype(np.float64) * s
        kf = synth.bf16_bits_to_f32(inp.k_pe[b]).astype(np.float64) * s
        c_kv.append(synth.f32_to_bf16_bits(cf.astype(np.float32)))
        k_pe.append(synth.f32_to_bf16_bits(kf.astype(np.float32)))
    return dataclasses.replace(inp, c_kv=c_kv, k_pe=k_pe)


# Row scalings that drive the logits over a wide range.  "rising": the logit
# spread grows along the sequence to ~60x the unit spread, so the running maximum
# grows many times by far more than any rescale threshold and, without
# rescaling, 2^(s - m) would overflow fp32 long before the end; "falling": the
# maximum comes first; "sink": one dominant row in the middle.
LOGIT_PROFILES = {
    "rising": lambda L: (lambda b, p: 1.0 + 60.0 * p / L[b]),
    "falling": lambda L: (lambda b, p: 61.0 - 60.0 * p / L[b]),
    "sink": lambda L: (lambda b, p: 12.0 if p == L[b] // 2 else 1.0),
}


# ---------------------------------------------------------------- KV down-projection
# Rows written from a token's hidden state go through an fp32 product and an
# fp32 normalisation before their roundings to bf16, the oracle through fp64:
# a value may land one bf16 unit away at a rounding boundary.  A latent value
# then differs by at most two units, 2^-6 of itself; and the fp32 sum of d_model
# products (about unit size, as the generator scales them) carries an absolute
# error near sqrt(d_model) fp32 units, which a value close to zero cannot hide
# in its own size: 2^-13 absolute covers it at d_model = 7168, while a lost or
# repeated 512-deep slice moves a value by about 0.3.  A key value one unit off
# moves both values of its rotated pair by up to a unit of the pair's larger
# input, and a rotated value can be much smaller than its inputs (the two
# products cancel), so key values are held to 2^-6 of the row's largest key
# value.  Almost every value must still be identical.
KV_DOWN_REL = 2.0 ** -6
KV_DOWN_ABS = 2.0 ** -13
KV_DOWN_MAX_DIFF_FRACTION = 0.01


def oracle_kv_down_rows(dims, di, positions, cos32, sin32):
    """The oracle's cache rows [T, d_c + d_r] (bf16 bits) for new tokens at
    ``positions`` whose cache inputs come from the joint down-projection."""
    c_kv, k_pe = O.kv_down(dims, di.x, di.w_dkv, di.b_dkv, di.gamma, di.eps)
    T = len(positions)
    positions = np.asarray(positions, np.int64)
    bt = np.full((T, int(positions.max()) // 64 + 1), -1, np.int32)
    bt[np.arange(T), positions // 64] = np.arange(T)
    pool = O.new_pool(T, 64, dims.row, dims.dtype)
    O.append_cache(pool, dims, 64, np.arange(T), positions, c_kv, k_pe, bt, cos32, sin32)
    return pool[np.arange(T) * 64 + positions % 64]


def check_kv_down_rows(got_bits: np.ndarray, exp_bits: np.ndarray, d_latent: int,
                       label: str = "") -> None:
    g = O.bf16_to_f64(got_bits)
    e = O.bf16_to_f64(exp_bits)
    assert np.all(np.isfinite(g)), f"{label}: non-finite row values"
    scale = np.abs(e)
    scale[:, d_latent:] = np.abs(e[:, d_latent:]).max(axis=1, keepdims=True)
    diff = got_bits != exp_bits
    frac = float(diff.mean())
    bound = KV_DOWN_REL * scale + KV_DOWN_ABS
    rel = np.abs(g - e) / bound
    worst = float(rel[diff].max()) if diff.any() else 0.0
    cols = np.nonzero(diff)[1]
    print(f"[parity] {label} kv_down rows: {int(diff.sum())} of {diff.size} values differ "
          f"({int((cols < d_latent).sum())} latent, {int((cols >= d_latent).sum())} key), "
          f"worst {worst:.3g} of the bound", flush=True)
    assert np.all(np.abs(g - e) <= bound), (label, worst)
    assert frac <= KV_DOWN_MAX_DIFF_FRACTION, (label, frac)


def kv_down_slots(inp):
    """Physical rows of the step's new tokens."""
    seqs, pos, _, _ = inp.new_tokens()
    return np.array([O.slot_of(inp.block_table, int(s), int(p), 64) for s, p in zip(seqs, pos)],
                    np.int64), pos
