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
from tests.gpu_util import (FP8_KV_SCALE, LOGIT_PROFILES, check_kv_down_rows, check_out,
                            drop_queries, kv_down_slots, oracle_kv_down_rows, oracle_pool,
                            oracle_pool_fp8, pool_bits, rows_fn, rows_fn_fp8, sample_heads,
                            scale_rows)


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


@pytest.mark.parametrize("name", ["tiny", "v3_batch_ragged", "v3_prefill_small"])
def test_emu_append_bit_exact(emu, name):
    """Cache rows and the RoPE columns of q_lat written by the append kernel
    (the vectorised DeepSeek-V3 form and the generic one) match the oracle bit
    for bit, sentinel rows included."""
    inp = _inputs(**CASES[name])
    d = inp.dims
    st = EmuStep(emu, inp)
    st.append()
    assert int(st.dev_error[0]) == 0
    np.testing.assert_array_equal(pool_bits(st.pool, d), pool_bits(oracle_pool(inp), d))
    cos, sin = O.rope_table_f32(inp.max_pos(), d.d_rope)
    pos = inp.token_pos()
    qpe = O.storage_to_f64(inp.q_pe, d.dtype).astype(np.float32)
    exp = O.rope_cache_f32(qpe, cos[pos][:, None, :], sin[pos][:, None, :])
    exp = O.to_bf16_bits(exp) if d.dtype == "bf16" else exp
    np.testing.assert_array_equal(pool_bits(st.q_lat[:, :, d.d_latent:], d), pool_bits(exp, d))


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


@pytest.mark.parametrize("kv_lens", [
    [1000],                                   # one token over 16 ranges: 2 rounds of 8
    [200, 100],                               # at most 4 ranges per token: 1 round
    [1000] + [37 * k for k in range(1, 16)],  # 16 tokens of 1 to 16 ranges
    [2000, 1500, 1, 64],                      # 32 ranges: 4 rounds
])
def test_emu_merge_rounds(emu, kv_lens):
    """The V3 merge with each token split over one range per cache block: one
    round of eight ranges, several rounds combined online, and tokens of one
    block (finished in place) beside split ones."""
    inp = _inputs("batch64", kv_lens=kv_lens)
    d = inp.dims
    st = EmuStep(emu, inp)
    st.append()
    q = synth.random_latent_queries(d, inp.T, seed=6)
    st.q_lat[...] = q
    heads = sample_heads(d.num_heads)
    ref = O.latent_decode(d, O.storage_to_f64(q, d.dtype), rows_fn(oracle_pool(inp), inp),
                          inp.kv_lens, inp.q_start, inp.workload.causal, heads)
    st.o_lat[...] = 0
    st.decode(100000)
    got = O.storage_to_f64(st.o_lat, d.dtype)
    assert np.abs(got[:, heads] - ref).max() <= 2.0 ** -7 * np.abs(ref).max()


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


@pytest.mark.parametrize("workload,causal,q_len", [("batch64", False, 1), ("prefill", True, 5)])
def test_emu_sequences_without_queries(emu, workload, causal, q_len):
    """Sequences with no query tokens in the batch (empty q_start ranges) are
    skipped by the split plan, the merge and the projections."""
    inp = _inputs(workload, causal=causal, kv_lens=[100, 64, 300, 1, 129], q_len=q_len)
    inp = drop_queries(inp, {1, 3})
    d = inp.dims
    for G in (1, 2, 7, 0, 3, 100000):
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
        inp = drop_queries(inp, zero)
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
    lens = [int(x) for x in np.random.default_rng(7).integers(1, 100, size=70)]
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
    for G in (1, 7, 0, 100000):
        st.decode(G)
        got = O.storage_to_f64(st.o_lat, d.dtype)[:, heads]
        assert np.abs(got - ref).max() <= 2.0 ** -7 * np.abs(ref).max(), G


@pytest.mark.parametrize("profile", ["rising", "falling", "sink"])
def test_emu_decode_wide_logit_range(emu, profile):
    """Logits that rise along the sequence (the running maximum grows by far
    more than the lazy-rescale threshold, many times, and by more than the fp32
    exponent range overall), fall (the maximum is found first), or have one
    dominant row in the middle."""
    inp = _inputs("batch64", kv_lens=[700, 333, 2100])
    inp = scale_rows(inp, LOGIT_PROFILES[profile](inp.kv_lens))
    d = inp.dims
    st = EmuStep(emu, inp)
    st.append()
    q = synth.random_latent_queries(d, inp.T, seed=9)
    st.q_lat[...] = q
    pool = oracle_pool(inp)
    heads = [0, 17, 63, 64, 127]
    ref = O.latent_decode(d, O.storage_to_f64(q, d.dtype), rows_fn(pool, inp), inp.kv_lens,
                          inp.q_start, False, heads)
    for G in (1, 2, 7, 0):
        st.decode(G)
        got = O.storage_to_f64(st.o_lat, d.dtype)[:, heads]
        assert np.all(np.isfinite(got))
        assert np.abs(got - ref).max() <= 2.0 ** -7 * np.abs(ref).max(), (profile, G)


def test_emu_step_without_any_query(emu):
    """A batch with no query tokens at all: every call is a no-op that leaves
    its outputs untouched (only the history rows are in the cache)."""
    inp = drop_queries(_inputs("batch64", kv_lens=[70, 129]), {0, 1})
    assert inp.T == 0
    st = EmuStep(emu, inp)
    st.run()
    pool = oracle_pool(inp)
    np.testing.assert_array_equal(pool_bits(st.pool, inp.dims), pool_bits(pool, inp.dims))
    assert int(st.dev_error[0]) == 0


def test_emu_decode_noalloc_matches_decode(emu):
    """mla_decode_noalloc (library-owned scratch) gives the bits of mla_decode
    (caller workspace) for the same plan, on two calls in a row, the second on a
    smaller batch; a plan needing more scratch than the library holds is
    rejected before any launch."""
    for kv_lens, G in (([700, 129, 1, 2000], 0), ([70, 300], 3)):
        inp = _inputs("batch64", kv_lens=kv_lens)
        d = inp.dims
        st = EmuStep(emu, inp, num_workgroups=G)
        st.append()
        st.q_lat[...] = synth.random_latent_queries(d, inp.T, seed=4)
        st.decode()
        want = st.o_lat.copy()
        st.o_lat[...] = 0
        emu.decode_noalloc(st.cfg, st.q_start, st.kv_lens, st.block_table, st.num_blocks,
                           st.q_lat, st.pool, False, st.o_lat, G, st.dev_error)
        assert int(st.dev_error[0]) == 0
        np.testing.assert_array_equal(st.o_lat, want)
    inp = _inputs("batch64", kv_lens=[20000])
    st = EmuStep(emu, inp)
    with pytest.raises(B.MlaError) as e:
        emu.decode_noalloc(st.cfg, st.q_start, st.kv_lens, st.block_table, st.num_blocks,
                           st.q_lat, st.pool, False, st.o_lat, 300, st.dev_error)
    assert e.value.status == 3  # MLA_ERR_WORKSPACE


def _emu_kv_down(emu, st, inp, di, pos=None):
    ck, kp, seq, p = st.new
    if pos is not None:
        p = emu.put(pos.astype(np.int32))
    nbytes = emu.kv_down_workspace_size(st.cfg, inp.T, di.x.shape[1])
    ws = emu.empty((nbytes,), np.uint8)
    emu.kv_down_append(st.cfg, emu.put(di.x), emu.put(di.w_dkv),
                       None if di.b_dkv is None else emu.put(di.b_dkv), emu.put(di.gamma), di.eps,
                       st.q_pe, seq, p, st.block_table, st.num_blocks, st.cos, st.sin, ws,
                       st.pool, st.q_lat, st.dev_error)


@pytest.mark.parametrize("name,bias", [("v3_batch_ragged", True), ("v3_prefill_small", False)])
def test_emu_kv_down_append(emu, name, bias):
    """Joint KV down-projection + latent RMSNorm fused with the append: the new
    rows agree with the oracle within two bf16 units (almost all identical);
    history rows, sentinels and the q_lat RoPE columns bit for bit.  The
    prefill case has 80 new tokens: two token tiles, the second ragged."""
    inp = _inputs(**CASES[name])
    d = inp.dims
    st = EmuStep(emu, inp)
    di = synth.make_down_inputs(d, inp.T, d_model=1024, seed=21, bias=bias)
    _emu_kv_down(emu, st, inp, di)
    assert int(st.dev_error[0]) == 0
    slots, pos = kv_down_slots(inp)
    cos32, sin32 = O.rope_table_f32(inp.max_pos(), d.d_rope)
    got = st.pool.view(np.uint16)
    check_kv_down_rows(got[slots], oracle_kv_down_rows(d, di, pos, cos32, sin32), d.d_latent,
                       f"emu {name}")
    keep = np.ones(len(got), bool)
    keep[slots] = False
    np.testing.assert_array_equal(got[keep], oracle_pool(inp, "history").view(np.uint16)[keep])
    qpe = O.storage_to_f64(inp.q_pe, d.dtype).astype(np.float32)
    exp = O.to_bf16_bits(O.rope_cache_f32(qpe, cos32[pos][:, None, :], sin32[pos][:, None, :]))
    np.testing.assert_array_equal(st.q_lat[:, :, d.d_latent:].view(np.uint16), exp)


def test_emu_kv_down_bad_entry_is_skipped_and_flagged(emu):
    inp = _inputs(**CASES["v3_batch_ragged"])
    d = inp.dims
    st = EmuStep(emu, inp)
    di = synth.make_down_inputs(d, inp.T, d_model=512, seed=22)
    before = st.pool.copy()
    _, pos = kv_down_slots(inp)
    bad = pos.copy()
    bad[2] = st.cos.shape[0]          # one past the RoPE table
    _emu_kv_down(emu, st, inp, di, pos=bad)
    assert int(st.dev_error[0]) & B.DEVERR_POSITION
    slots, _ = kv_down_slots(inp)
    np.testing.assert_array_equal(st.pool[slots[2]], before[slots[2]])
    assert not np.array_equal(st.pool[slots[0]], before[slots[0]])


@pytest.mark.parametrize("T", [5, 70])
def test_emu_fused_weight_projections(emu, T):
    """Weight-level absorbed calls (fused W_KQ and W_OV streamed through LDS)
    over one and two token tiles, against the oracle's definitions."""
    d = synth.V3
    cfg = B.MlaConfig.from_dims(d)
    fi = synth.make_fused_inputs(d, T, d_cq=256, d_model=512, seed=9)
    q_lat = emu.empty((T, d.num_heads, d.row), np.uint16)
    q_lat[...] = 0x7FC1   # RoPE columns must stay untouched
    emu.absorb_q_fused(cfg, emu.put(fi.c_q), emu.put(fi.w_kq), q_lat)
    ref = O.absorb_q_fused(d, fi.c_q, fi.w_kq)
    got = O.storage_to_f64(q_lat[:, :, :d.d_latent], d.dtype)
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-5 * np.abs(ref).max())
    assert np.all(q_lat[:, :, d.d_latent:] == 0x7FC1)
    out = emu.empty((T, 512), np.float32)
    emu.out_proj_fused(cfg, emu.put(fi.o_lat), emu.put(fi.w_ov), out)
    ref = O.out_proj_fused(d, O.storage_to_f64(fi.o_lat, d.dtype), fi.w_ov)
    assert np.abs(out - ref).max() <= 5e-5 * np.abs(ref).max()


@pytest.mark.parametrize("name", ["v3_prefill_small"])
def test_emu_prefill_decompressed(emu, name):
    """Non-absorbed attention (decompressed K and V) against the oracle's
    explicit-decompression attention on a causal chunked prefill of two
    sequences (the GPU tests add decode batches and the full-size prefill)."""
    inp = _inputs(**CASES[name])
    d = inp.dims
    st = EmuStep(emu, inp)
    st.append()
    out = emu.empty((inp.T, d.num_heads, d.d_v), np.float32)
    emu.prefill_decompressed(st.cfg, st.q_start, st.kv_lens, st.block_table, st.num_blocks,
                             st.q_nope, st.q_lat, st.pool, st.w_uk, st.w_uv,
                             inp.workload.causal, out, st.dev_error)
    assert int(st.dev_error[0]) == 0
    pool = oracle_pool(inp)
    heads = sample_heads(d.num_heads, 6)
    ref = O.naive_mla(d, inp.w_uk, inp.w_uv, inp.q_nope, inp.q_pe, rows_fn(pool, inp),
                      inp.kv_lens, inp.q_start, inp.workload.causal, heads)
    check_out(d, out[:, heads], ref, f"emu prefill {name}")


@pytest.mark.parametrize("name", ["tiny_prefill", "v3_batch_ragged"])
def test_emu_device_lengths_disagreeing_with_host_are_flagged(emu, name):
    """The split plan comes from the host copies of the lengths; device copies
    that disagree are flagged (MLA_DEVERR_LENGTH) and nothing outside the given
    buffers is touched (every buffer ends at a guard page)."""
    import ctypes
    inp = _inputs(**CASES[name])
    st = EmuStep(emu, inp)
    st.append()
    bad = emu.put(np.asarray(inp.kv_lens, np.int32) + 100)
    qs = np.ascontiguousarray(inp.q_start, np.int32)
    kl = np.ascontiguousarray(inp.kv_lens, np.int32)
    st.dev_error[0] = 0
    p = lambda a: None if a is None else a.ctypes.data
    for G in (0, 7):
        nbytes = emu.workspace_size(st.cfg, qs, kl, inp.workload.causal, G)
        ws = emu.empty((max(nbytes, 16),), np.uint8)
        rc = emu.lib.mla_decode(
            ctypes.byref(st.cfg), len(kl), p(st.q_start), p(bad), qs.ctypes.data, kl.ctypes.data,
            p(st.block_table), st.block_table.shape[1], st.num_blocks, p(st.q_lat), p(st.pool),
            int(inp.workload.causal), G, p(ws), nbytes, p(st.o_lat), p(st.dev_error), None)
        assert rc == 0
        assert int(st.dev_error[0]) & B.DEVERR_LENGTH


def test_emu_prefill_device_lengths_disagreeing_with_host_are_flagged(emu):
    import ctypes
    inp = _inputs(**CASES["v3_prefill_small"])
    d = inp.dims
    st = EmuStep(emu, inp)
    st.append()
    bad = emu.put(np.asarray(inp.kv_lens, np.int32) + 100)
    qs = np.ascontiguousarray(inp.q_start, np.int32)
    kl = np.ascontiguousarray(inp.kv_lens, np.int32)
    p = lambda a: None if a is None else a.ctypes.data
    n = ctypes.c_size_t(0)
    assert emu.lib.mla_prefill_workspace_size(ctypes.byref(st.cfg), len(kl), qs.ctypes.data,
                                              kl.ctypes.data, ctypes.byref(n)) == 0
    ws = emu.empty((n.value,), np.uint8)
    out = emu.empty((inp.T, d.num_heads, d.d_v), np.float32)
    st.dev_error[0] = 0
    rc = emu.lib.mla_prefill_decompressed(
        ctypes.byref(st.cfg), len(kl), p(st.q_start), p(bad), qs.ctypes.data, kl.ctypes.data,
        p(st.block_table), st.block_table.shape[1], st.num_blocks, p(st.q_nope), p(st.q_lat),
        p(st.pool), p(st.w_uk), p(st.w_uv), 1, p(ws), ws.nbytes, p(out), p(st.dev_error), None)
    assert rc == 0
    assert int(st.dev_error[0]) & B.DEVERR_LENGTH


# ---------------------------------------------------------------- e4m3 cache
FP8_CASES = ["v3_batch_ragged", "v3_prefill_small"]


@pytest.mark.parametrize("name", FP8_CASES)
def test_emu_fp8_step(emu, name):
    """The step over an e4m3 cache: the pool matches the oracle's e4m3 pool bit
    for bit (sentinels included), q_lat's RoPE columns match the bf16 path, and
    the output matches naive attention over the dequantised rows at the bf16
    tolerances."""
    inp = _inputs(**CASES[name])
    d = inp.dims
    st = EmuStep(emu, inp, kv_scale=FP8_KV_SCALE)
    st.run()
    assert int(st.dev_error[0]) == 0
    pool = oracle_pool_fp8(inp)
    np.testing.assert_array_equal(st.pool, pool)
    cos, sin = O.rope_table_f32(inp.max_pos(), d.d_rope)
    pos = inp.token_pos()
    qpe = O.bf16_to_f64(inp.q_pe).astype(np.float32)
    exp = O.to_bf16_bits(O.rope_cache_f32(qpe, cos[pos][:, None, :], sin[pos][:, None, :]))
    np.testing.assert_array_equal(st.q_lat[:, :, d.d_latent:], exp)
    heads = sorted(set(sample_heads(d.num_heads, 8) + [64]))
    ref = O.naive_mla(d, inp.w_uk, inp.w_uv, inp.q_nope, inp.q_pe, rows_fn_fp8(pool, inp),
                      inp.kv_lens, inp.q_start, inp.workload.causal, heads)
    check_out(d, st.out[:, heads], ref, f"emu fp8 {name}")


@pytest.mark.parametrize("name", ["v3_batch_ragged"])
def test_emu_fp8_decode_splits(emu, name):
    """Every split plan against the oracle's latent decode over the dequantised
    rows; the same plan under another interleaving gives identical bits."""
    inp = _inputs(**CASES[name])
    d = inp.dims
    st = EmuStep(emu, inp, kv_scale=FP8_KV_SCALE)
    st.append()
    q = synth.random_latent_queries(d, inp.T, seed=5)
    st.q_lat[...] = q
    pool = oracle_pool_fp8(inp)
    heads = sample_heads(d.num_heads)
    ref = O.latent_decode(d, O.bf16_to_f64(q), rows_fn_fp8(pool, inp), inp.kv_lens,
                          inp.q_start, inp.workload.causal, heads)
    tol = 2.0 ** -7 * np.abs(ref).max()
    outs = {}
    for G in (1, 2, 7, 0, 100000):
        st.o_lat[...] = 0
        st.decode(G)
        got = O.bf16_to_f64(st.o_lat)
        assert np.all(np.isfinite(got)), G
        err = np.abs(got[:, heads] - ref).max()
        assert err <= tol, (G, err, tol)
        outs[G] = st.o_lat.copy()
    for seed in (2, 3):
        emu.set_seed(seed)
        st.decode(7)
        np.testing.assert_array_equal(st.o_lat, outs[7])
    emu.set_seed(1)


@pytest.mark.parametrize("profile", ["rising", "sink"])
def test_emu_fp8_decode_wide_logit_range(emu, profile):
    """Logits far beyond the unit spread over an e4m3 cache: the softmax weights
    reach the lazy-rescale bound 2^8 and the rescaling path runs."""
    base = _inputs("batch64", kv_lens=[300, 97])
    inp = scale_rows(base, LOGIT_PROFILES[profile]([int(L) for L in base.kv_lens]))
    d = inp.dims
    # the scaled rows must stay inside the e4m3 range under the cache scale
    kv_scale = 2.0 ** 2 if profile == "rising" else FP8_KV_SCALE
    st = EmuStep(emu, inp, kv_scale=kv_scale)
    st.run()
    pool = oracle_pool_fp8(inp, kv_scale)
    np.testing.assert_array_equal(st.pool, pool)
    heads = sample_heads(d.num_heads)
    ref = O.naive_mla(d, inp.w_uk, inp.w_uv, inp.q_nope, inp.q_pe,
                      rows_fn_fp8(pool, inp, kv_scale), inp.kv_lens, inp.q_start, False, heads)
    err = np.abs(st.out[:, heads] - ref)
    assert np.all(np.isfinite(st.out[:, heads]))
    # relative to the output's size (the scaled rows make it large)
    assert err.max() <= 2e-2 * max(1.0, np.abs(ref).max()), (err.max(), np.abs(ref).max())


def test_emu_fp8_bad_entries_and_lengths_flagged(emu):
    """The e4m3 calls skip and flag out-of-range positions, sequence ids and
    block ids (append) and an unassigned block (decode); device lengths that
    disagree with the host copies are flagged before any access.  Every buffer
    ends at a guard page, so no access outside them goes unnoticed."""
    import ctypes
    inp = _inputs("batch64", kv_lens=[70, 129])
    st = EmuStep(emu, inp, kv_scale=FP8_KV_SCALE)
    before = st.pool.copy()
    seq = emu.put(np.array([0, 5, 0], np.int32))
    pos = emu.put(np.array([100000, 3, 127], np.int32))
    bt = emu.put(inp.block_table.astype(np.int32))
    bt[0, 1] = -1
    err = emu.empty((1,), np.uint32)
    ck = emu.put(np.zeros((3, inp.dims.d_latent), np.uint16))
    kp = emu.put(np.zeros((3, inp.dims.d_rope), np.uint16))
    emu.append_fp8(st.cfg, ck, kp, None, seq, pos, bt, st.num_blocks, st.cos, st.sin,
                   FP8_KV_SCALE, st.pool, dev_error=err)
    e = int(err[0])
    assert e & B.DEVERR_POSITION and e & B.DEVERR_SEQ and e & B.DEVERR_BLOCK
    np.testing.assert_array_equal(st.pool, before)
    st.append()
    qs = np.ascontiguousarray(inp.q_start, np.int32)
    kl = np.ascontiguousarray(inp.kv_lens, np.int32)
    bad = emu.put(kl + 100)
    p = lambda a: None if a is None else a.ctypes.data
    st.dev_error[0] = 0
    for G in (0, 7):
        nbytes = emu.workspace_size(st.cfg, qs, kl, False, G)
        ws = emu.empty((max(nbytes, 16),), np.uint8)
        rc = emu.lib.mla_decode_fp8(
            ctypes.byref(st.cfg), len(kl), p(st.q_start), p(bad), qs.ctypes.data, kl.ctypes.data,
            p(st.block_table), st.block_table.shape[1], st.num_blocks, p(st.q_lat), p(st.pool),
            ctypes.c_float(FP8_KV_SCALE), 0, G, p(ws), nbytes, p(st.o_lat), p(st.dev_error),
            None)
        assert rc == 0
        assert int(st.dev_error[0]) & B.DEVERR_LENGTH
    st.dev_error[0] = 0
    st.block_table[1, 1] = -1
    st.decode()
    assert int(st.dev_error[0]) & B.DEVERR_BLOCK
