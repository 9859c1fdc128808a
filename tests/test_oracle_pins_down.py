"""Pins for the oracle's joint KV down-projection and latent RMSNorm
([MLA architecture] 2.2, kv_a_proj_with_mqa + kv_a_layernorm).  CPU only.

The pins are brute-force scalar loops on tiny inputs, one-hot hidden states
(the projection then picks one weight column), closed forms of the
normalisation (where eps enters, scale invariance, unit mean square) and
constructed rounding ties, so that a transposed weight, a dropped bias, a
normalisation over the wrong axis or with eps outside the root, or a
double rounding through fp32 each fail one of them.
"""
import math
import struct

import numpy as np
import pytest

from oracle import mla_oracle as O
from head_latent_attention_05_amd import synth


def _dims(dtype, dc=8, dr=4):
    return synth.Dims(num_heads=2, d_latent=dc, d_rope=dr, d_nope=4, d_v=4, dtype=dtype)


def _f32(v: float) -> float:
    return struct.unpack("<f", struct.pack("<f", v))[0]


def test_bf16_rounding_is_one_step_to_nearest_even():
    one = 1.0
    ulp = 2.0 ** -7                       # bf16 spacing in [1, 2)
    tie = one + ulp / 2                   # exactly halfway: to even (1.0)
    above = tie + 2.0 ** -30              # above the tie; fp32 would first round to the tie
    below = tie - 2.0 ** -30
    odd_tie = one + ulp + ulp / 2         # halfway between an odd and an even code: up
    got = O.bf16_to_f64(O.f64_to_bf16_bits(np.array([tie, above, below, odd_tie, -above, 0.0])))
    assert list(got) == [1.0, 1.0 + ulp, 1.0, 1.0 + 2 * ulp, -(1.0 + ulp), 0.0]
    # through fp32 the 'above' case lands on the tie and goes down: the oracle must not
    assert O.bf16_to_f64(O.to_bf16_bits(np.array([above], np.float32)))[0] == 1.0


def test_bf16_rounding_agrees_with_fp32_rounding_on_fp32_values():
    rng = np.random.default_rng(3)
    x32 = (rng.standard_normal(4096) * np.exp(rng.uniform(-20, 20, 4096))).astype(np.float32)
    np.testing.assert_array_equal(O.f64_to_bf16_bits(x32.astype(np.float64)), O.to_bf16_bits(x32))


def test_rms_norm_closed_forms():
    g = np.array([1.0, 2.0, -0.5, 4.0])
    # constant vector a: every entry becomes g * a / sqrt(a^2 + eps); a = 1, eps = 3 -> g / 2
    np.testing.assert_allclose(O.rms_norm(np.ones(4), g, 3.0), g / 2, rtol=0, atol=1e-15)
    a, eps = 0.25, 1e-2
    np.testing.assert_allclose(O.rms_norm(np.full(4, a), g, eps), g * a / math.sqrt(a * a + eps),
                               rtol=1e-15)
    rng = np.random.default_rng(5)
    c = rng.standard_normal((3, 16))
    one = np.ones(16)
    # unit mean square with gain 1 and eps 0, and invariance to a positive scale
    y = O.rms_norm(c, one, 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(O.rms_norm(7.5 * c, one, 0.0), y, rtol=1e-14)
    # each row is normalised on its own (the statistic is over the last axis)
    np.testing.assert_allclose(O.rms_norm(c[1:2], one, 0.0), y[1:2], rtol=1e-14)


def _brute_kv_down(d, x, w, b, gamma, eps):
    """Scalar loops over python floats: projection, rounding, RMSNorm, rounding."""
    T, K = x.shape
    N = w.shape[0]
    dt, dc = d.dtype, d.d_latent
    xf, wf = O.storage_to_f64(x, dt), O.storage_to_f64(w, dt)
    bf = O.storage_to_f64(b, dt) if b is not None else None
    gf = O.storage_to_f64(gamma, dt)

    def rnd(v):
        if dt == "bf16":
            return float(O.bf16_to_f64(O.f64_to_bf16_bits(np.array([v])))[0])
        return _f32(v)

    c_out, k_out = [], []
    for t in range(T):
        kv = []
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += float(xf[t, k]) * float(wf[n, k])
            if bf is not None:
                acc += float(bf[n])
            kv.append(rnd(acc))
        ms = sum(v * v for v in kv[:dc]) / dc
        r = 1.0 / math.sqrt(ms + eps)
        c_out.append([rnd(float(gf[i]) * kv[i] * r) for i in range(dc)])
        k_out.append(kv[dc:])
    return np.array(c_out), np.array(k_out)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("bias", [True, False])
def test_kv_down_matches_scalar_loops(dtype, bias):
    d = _dims(dtype)
    di = synth.make_down_inputs(d, T=3, d_model=24, seed=11, bias=bias, eps=1e-3)
    c_kv, k_pe = O.kv_down(d, di.x, di.w_dkv, di.b_dkv, di.gamma, di.eps)
    bc, bk = _brute_kv_down(d, di.x, di.w_dkv, di.b_dkv, di.gamma, di.eps)
    assert c_kv.shape == (3, d.d_latent) and k_pe.shape == (3, d.d_rope)
    # the two sums differ only in the order of fp64 additions: the rounded
    # results agree to the last stored bit except at astronomically rare ties
    np.testing.assert_allclose(O.storage_to_f64(c_kv, dtype), bc, rtol=2 ** -22, atol=0)
    np.testing.assert_allclose(O.storage_to_f64(k_pe, dtype), bk, rtol=2 ** -22, atol=0)


def test_kv_down_one_hot_picks_a_weight_column():
    d = _dims("bf16")
    di = synth.make_down_inputs(d, T=1, d_model=16, seed=2, bias=True, eps=1e-6)
    k = 5
    x = np.zeros((2, 16), np.float64)
    x[0, k] = 1.0
    x[1, k] = -2.0
    xb = O.f64_to_bf16_bits(x)
    c_kv, k_pe = O.kv_down(d, xb, di.w_dkv, di.b_dkv, di.gamma, di.eps)
    col = O.bf16_to_f64(di.w_dkv)[:, k]
    b = O.bf16_to_f64(di.b_dkv)
    for t, s in ((0, 1.0), (1, -2.0)):
        kv = O.bf16_to_f64(O.f64_to_bf16_bits(s * col + b))
        np.testing.assert_array_equal(O.bf16_to_f64(k_pe[t]), kv[d.d_latent:])
        c = kv[:d.d_latent]
        want = O.bf16_to_f64(di.gamma) * c / math.sqrt(float(np.mean(c * c)) + di.eps)
        np.testing.assert_array_equal(c_kv[t], O.f64_to_bf16_bits(want))


def test_kv_down_zero_hidden_state_gives_bias_and_eps_floor():
    """x = 0: the projection is the bias alone; with no bias the latent is 0 and
    the normalisation returns 0 (eps keeps the root away from zero)."""
    d = _dims("f32")
    di = synth.make_down_inputs(d, T=1, d_model=8, seed=4, bias=True, eps=1e-6)
    x = np.zeros((1, 8), np.float32)
    c_kv, k_pe = O.kv_down(d, x, di.w_dkv, di.b_dkv, di.gamma, di.eps)
    np.testing.assert_array_equal(k_pe[0], di.b_dkv[d.d_latent:])
    c0, _ = O.kv_down(d, x, di.w_dkv, None, di.gamma, di.eps)
    assert np.all(c0 == 0.0)


def test_kv_down_rounds_the_projection_once():
    """y = 1 + 2^-8 + 2^-30 exactly (three bf16 products): one rounding to bf16
    gives 1 + 2^-7; a detour through fp32 would land on the tie and give 1."""
    d = _dims("bf16", dc=4, dr=2)
    n = d.d_latent + d.d_rope
    x = O.f64_to_bf16_bits(np.ones((1, 3)))
    w = np.zeros((n, 3))
    w[d.d_latent] = [1.0, 2.0 ** -8, 2.0 ** -30]     # first RoPE-key value
    w[0] = [1.0, 2.0 ** -8, 2.0 ** -30]              # first latent value
    w[1:d.d_latent] = [1.0, 0.0, 0.0]
    _, k_pe = O.kv_down(d, x, O.f64_to_bf16_bits(w), None,
                        O.f64_to_bf16_bits(np.ones(d.d_latent)), 0.0)
    assert O.bf16_to_f64(k_pe)[0, 0] == 1.0 + 2.0 ** -7
