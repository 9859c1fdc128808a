"""The library's HIP kernels, compiled as host C++ and run by the CPU emulator
(tests/emu), checked against the oracle on the same seeded inputs.  CPU only.

This checks indexing, tiling, cross-lane operand layouts (MFMA, transposing LDS
reads), the split plan and the merge without a GPU; buffers end at an
inaccessible page, so an out-of-bounds access faults.  The emulator models
gfx950's cross-lane layouts; the decode kernel, whose results on MI355X match
the oracle, matching it here too is what ties that model to the hardware.
Timing and memory ordering are not emulated: waits and fences are checked on
the GPU only.
"""
import dataclasses
import os

import numpy as np
import pytest

from head_latent_attention_05_amd import binding as B
from head_latent_attention_05_amd import synth
from oracle import mla_oracle as O
from tests.emu import build_emu
from tests.emu.emulib import Emu, EmuStep
from tests.gpu_util import check_out, oracle_pool, pool_bits, rows_fn, sample_heads


@pytest.fixture(scope="module")
def emu():
    if not os.path.exists(build_emu.CXX):
        pytest.skip(f"host compiler {build_emu.CXX} not found")
    e = Emu(cus=8, seed=1)
    yield e
    e.close()


def _inputs(workload, causal=None, **kw):
    wl = synth.WORKLOADS[workload]
    if causal is not None and causal != wl.causal:
        wl = dataclasses.replace(wl, causal=causal)
    return synth.make_inputs(wl, **kw)


CASES = {
    "tiny": dict(workload="tiny"),
    "tiny_prefill": dict(workload="tiny", kv_lens=[150, 77], q_len=40, causal=True),
    "v3_batch_ragged": dict(workload="batch64", kv_lens=[70, 129, 1, 64, 200]),
    "v3_prefill_small": dict(workload="prefill", kv_lens=[150, 77], q_len=40),
    # long segments: tiles stream through the loads-in-flight pipeline for many
    # iterations, so the wait counts are exercised
    "v3_long_segments": dict(workload="batch64", kv_lens=[2000, 700]),
}


@pytest.mark.parametrize("name", list(CASES))
def test_emu_step(emu, name):
    inp = _inputs(**CASES[name])
    d = inp.dims
    st = EmuStep(emu, inp)
    st.run()
    assert int(st.dev_error[0]) == 0
    pool = oracle_pool(inp)
    np.testing.assert_array_equal(pool_bits(st.pool, d), pool_bits(pool, d))
    heads = sample_heads(d.num_heads, 8) + ([64] if d.num_heads > 64 else [])
    heads = sorted(set(heads))
    ref = O.naive_mla(d, inp.w_uk, inp.w_uv, inp.q_nope, inp.q_pe, rows_fn(pool, inp),
                      inp.kv_lens, inp.q_start, inp.workload.causal, heads)
    check_out(d, st.out[:, heads], ref, f"emu {name}")


@pytest.mark.parametrize("name", ["tiny_prefill", "v3_batch_ragged", "v3_prefill_small",
                                  "v3_long_segments"])
def test_emu_decode_splits(emu, name):
    """Every split plan (forced 1, 2, 7 and more workgroups than units) against
    the oracle's latent decode; the same plan twice, and under another
    interleaving of the emulated work-items, gives identical bits."""
    inp = _inputs(**CASES[name])
    d = inp.dims
    st = EmuStep(emu, inp)
    st.append()
    q = synth.random_latent_queries(d, inp.T, seed=5)
    st.q_lat[...] = q
    pool = oracle_pool(inp)
    heads = sample_heads(d.num_heads)
    ref = O.latent_decode(d, O.storage_to_f64(q, d.dtype), rows_fn(pool, inp), inp.kv_lens,
                          inp.q_start, inp.workload.causal, heads)
    tol = (2.0 ** -7 if d.dtype == "bf16" else 1e-5) * np.abs(ref).max()
    outs = {}
    for G in (1, 2, 7, 0, 100000):
        st.o_lat[...] = 0
        st.decode(G)
        got = O.storage_to_f64(st.o_lat, d.dtype)
        assert np.all(np.isfinite(got)), G
        assert np.abs(got[:, heads] - ref).max() <= tol, (G, np.abs(got[:, heads] - ref).max())
        outs[G] = st.o_lat.copy()
    for seed in (2, 3):
        emu.set_seed(seed)
        st.decode(7)
        np.testing.assert_array_equal(st.o_lat, outs[7])
    emu.set_seed(1)


@pytest.mark.parametrize("T", [1, 63, 64, 65, 130])
def test_emu_projections(emu, T):
    """MFMA absorb and up-projection kernels over one or several 64-token tiles
    with ragged tails, against the oracle's per-call definitions."""
    inp = _inputs("prefill", kv_lens=[T], q_len=T)
    d = inp.dims
    cfg = B.MlaConfig.from_dims(d)
    q_nope, w_uk, w_uv = emu.put(inp.q_nope), emu.put(inp.w_uk), emu.put(inp.w_uv)
    q_lat = emu.empty((T, d.num_heads, d.row), np.uint16)
    q_lat.view(np.uint16)[...] = 0x7FC1  # RoPE columns must stay untouched
    emu.absorb_q(cfg, q_nope, w_uk, q_lat)
    ref = O.absorb_q(d, inp.q_nope, inp.w_uk)
    got = O.storage_to_f64(q_lat[:, :, :d.d_latent], d.dtype)
    err = np.abs(got - ref)
    assert np.all(err <= np.abs(ref) * 2.0 ** -8 + 1e-6), err.max()
    assert np.all(q_lat[:, :, d.d_latent:] == 0x7FC1)

    o_np = synth.random_latent_outputs(d, T, seed=11)
    out = emu.empty((T, d.num_heads, d.d_v), np.float32)
    emu.out_proj(cfg, emu.put(o_np), w_uv, out)
    ref = O.out_proj(d, O.storage_to_f64(o_np, d.dtype), inp.w_uv)
    assert np.abs(out - ref).max() <= 1e-5 * np.abs(ref).max()


def test_emu_bad_entries_flagged(emu):
    """Out-of-range positions, sequence ids and block ids are skipped and flagged
    (append), and a bad block-table entry is flagged by the decode kernel."""
    inp = _inputs("batch64", kv_lens=[70, 129])
    st = EmuStep(emu, inp)
    before = st.pool.copy()
    seq = emu.put(np.array([0, 5, 0], np.int32))
    pos = emu.put(np.array([100000, 3, 127], np.int32))
    bt = emu.put(inp.block_table.astype(np.int32))
    bt[0, 1] = -1
    err = emu.empty((1,), np.uint32)
    ck = emu.put(np.zeros((3, inp.dims.d_latent), np.uint16))
    kp = emu.put(np.zeros((3, inp.dims.d_rope), np.uint16))
    emu.append(st.cfg, ck, kp, None, seq, pos, bt, st.num_blocks, st.cos, st.sin, st.pool,
               dev_error=err)
    e = int(err[0])
    assert e & B.DEVERR_POSITION and e & B.DEVERR_SEQ and e & B.DEVERR_BLOCK
    np.testing.assert_array_equal(st.pool, before)
    # decode over a table with an unassigned block: flagged, nothing outside the
    # given buffers touched (the guard pages would fault)
    st.block_table[1, 1] = -1
    st.decode()
    assert int(st.dev_error[0]) & B.DEVERR_BLOCK


def _drop_queries(inp, zero):
    """The same step with no query tokens for the sequences in `zero` (their
    rows all become history); the other sequences' queries are unchanged."""
    q_lens = inp.q_lens.copy()
    keep = np.concatenate([np.full(int(q), b not in zero) for b, q in enumerate(inp.q_lens)])
    q_lens[list(zero)] = 0
    q_start = np.zeros(len(q_lens) + 1, np.int32)
    q_start[1:] = np.cumsum(q_lens)
    return dataclasses.replace(inp, q_lens=q_lens, q_start=q_start, q_nope=inp.q_nope[keep],
                               q_pe=inp.q_pe[keep])


@pytest.mark.parametrize("workload,causal,q_len", [("batch64", False, 1), ("prefill", True, 5)])
def test_emu_sequences_without_queries(emu, workload, causal, q_len):
    """Sequences with no query tokens in the batch (empty q_start ranges) are
    skipped by the split plan, the merge and the projections."""
    inp = _inputs(workload, causal=causal, kv_lens=[100, 64, 300, 1, 129], q_len=q_len)
    inp = _drop_queries(inp, {1, 3})
    d = inp.dims
    for G in (0, 3, 100000):
        st = EmuStep(emu, inp, num_workgroups=G)
        st.run()
        assert int(st.dev_error[0]) == 0
        pool = oracle_pool(inp)
        np.testing.assert_array_equal(pool_bits(st.pool, d), pool_bits(pool, d))
        heads = [0, 63, 64, 127]
        ref = O.naive_mla(d, inp.w_uk, inp.w_uv, inp.q_nope, inp.q_pe, rows_fn(pool, inp),
                          inp.kv_lens, inp.q_start, causal, heads)
        check_out(d, st.out[:, heads], ref, f"emu no-query seqs {workload} G={G}")


def _random_case(rng, it):
    """A random small batch: V3 bf16 or tiny fp32, causal or not, lengths near
    tile and block edges or anywhere up to 400, some sequences without queries,
    and a random split plan."""
    v3 = rng.random() < 0.7
    causal = rng.random() < 0.4
    B = int(rng.integers(1, 7))
    edges = [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129]
    lens = [int(rng.choice(edges)) if rng.random() < 0.5 else int(rng.integers(1, 400))
            for _ in range(B)]
    q_len = int(rng.choice([1, 2, 3, 17, 40])) if causal else 1
    inp = _inputs("batch64" if v3 else "tiny", causal=causal, kv_lens=lens, q_len=q_len,
                  seed=5000 + it)
    zero = {b for b in range(B) if rng.random() < 0.2}
    if zero and len(zero) < B:
        inp = _drop_queries(inp, zero)
    G = int(rng.choice([0, 1, 2, 3, 5, 8, 13, 64, 100000]))
    return inp, G


@pytest.mark.parametrize("it", range(12))
def test_emu_decode_random_shapes(emu, it):
    rng = np.random.default_rng(it)
    inp, G = _random_case(rng, it)
    d = inp.dims
    emu.set_seed(int(rng.integers(1, 1 << 30)))
    st = EmuStep(emu, inp, num_workgroups=G)
    st.append()
    q = synth.random_latent_queries(d, inp.T, seed=it)
    st.q_lat[...] = q
    st.decode()
    emu.set_seed(1)
    assert int(st.dev_error[0]) == 0
    pool = oracle_pool(inp)
    heads = [0, 1, d.num_heads - 1] + ([63, 64] if d.num_heads == 128 else [])
    ref = O.latent_decode(d, O.storage_to_f64(q, d.dtype), rows_fn(pool, inp), inp.kv_lens,
                          inp.q_start, inp.workload.causal, heads)
    got = O.storage_to_f64(st.o_lat, d.dtype)[:, heads]
    tol = (2.0 ** -7 if d.dtype == "bf16" else 1e-5) * np.abs(ref).max()
    assert np.abs(got - ref).max() <= tol, (inp.kv_lens, inp.q_lens, G)


@pytest.mark.parametrize("causal,q_len", [(False, 1), (True, 3)])
def test_emu_more_than_64_sequences(emu, causal, q_len):
    """Batches wider than one wave: the plan walk and the merge scan the
    sequences 64 at a time."""
    lens = [int(x) for x in np.random.default_rng(7).integers(1, 100, size=90)]
    inp = _inputs("batch64", causal=causal, kv_lens=lens, q_len=q_len, seed=11)
    d = inp.dims
    st = EmuStep(emu, inp)
    st.append()
    q = synth.random_latent_queries(d, inp.T, seed=3)
    st.q_lat[...] = q
    pool = oracle_pool(inp)
    heads = [0, 64, 127]
    ref = O.latent_decode(d, O.storage_to_f64(q, d.dtype), rows_fn(pool, inp), inp.kv_lens,
                          inp.q_start, causal, heads)
    for G in (0, 7, 100000):
        st.decode(G)
        got = O.storage_to_f64(st.o_lat, d.dtype)[:, heads]
        assert np.abs(got - ref).max() <= 2.0 ** -7 * np.abs(ref).max(), G


def _scale_rows(inp, f):
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


@pytest.mark.parametrize("profile", ["rising", "falling", "sink"])
def test_emu_decode_wide_logit_range(emu, profile):
    """Logits that rise along the sequence (the running maximum grows by far
    more than the lazy-rescale threshold, many times, and by more than the fp32
    exponent range overall), fall (the maximum is found first), or have one
    dominant row in the middle."""
    inp = _inputs("batch64", kv_lens=[700, 333])
    L = inp.kv_lens
    # logit spread grows to ~60x the unit spread: without rescaling, 2^(s - m)
    # would overflow fp32 long before the end of the rising sequence
    f = {"rising": lambda b, p: 1.0 + 60.0 * p / L[b],
         "falling": lambda b, p: 61.0 - 60.0 * p / L[b],
         "sink": lambda b, p: 12.0 if p == L[b] // 2 else 1.0}[profile]
    inp = _scale_rows(inp, f)
    d = inp.dims
    st = EmuStep(emu, inp)
    st.append()
    q = synth.random_latent_queries(d, inp.T, seed=9)
    st.q_lat[...] = q
    pool = oracle_pool(inp)
    heads = [0, 17, 64, 127]
    ref = O.latent_decode(d, O.storage_to_f64(q, d.dtype), rows_fn(pool, inp), inp.kv_lens,
                          inp.q_start, False, heads)
    for G in (1, 0, 5):
        st.decode(G)
        got = O.storage_to_f64(st.o_lat, d.dtype)[:, heads]
        assert np.all(np.isfinite(got))
        assert np.abs(got - ref).max() <= 2.0 ** -7 * np.abs(ref).max(), (profile, G)


def test_emu_step_without_any_query(emu):
    """A batch with no query tokens at all: every call is a no-op that leaves
    its outputs untouched (only the history rows are in the cache)."""
    inp = _drop_queries(_inputs("batch64", kv_lens=[70, 129]), {0, 1})
    assert inp.T == 0
    st = EmuStep(emu, inp)
    st.run()
    pool = oracle_pool(inp)
    np.testing.assert_array_equal(pool_bits(st.pool, inp.dims), pool_bits(pool, inp.dims))
    assert int(st.dev_error[0]) == 0
