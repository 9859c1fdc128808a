"""GPU parity of the e4m3 (fp8) latent cache ([MLA architecture] 4.2, quantised
cache): the fp8 append against the oracle's e4m3 pool bit for bit (sentinels
included), and the fp8 decode against attention over the dequantised rows at
the bf16 path's tolerances, for every split plan, at small sizes and at the
full workload sizes in the benchmark's launch configuration."""
import dataclasses

import numpy as np
import pytest
import torch

from head_latent_attention_05_amd import synth
from head_latent_attention_05_amd.step import DeviceStep, to_device, to_host
from oracle import mla_oracle as O
from tests.gpu_util import (FP8_KV_SCALE, LOGIT_PROFILES, check_out, oracle_pool_fp8,
                            rows_fn_fp8, sample_heads, scale_rows)

pytestmark = pytest.mark.gpu

SMALL = {
    "v3_single_ragged": dict(workload="single", kv_lens=[1000]),
    "v3_batch_ragged": dict(workload="batch64", kv_lens=[1, 64, 65, 700, 1333]),
    "v3_prefill_small": dict(workload="prefill", kv_lens=[300, 170], q_len=130),
}


def make(name):
    spec = dict(SMALL[name])
    return synth.make_inputs(synth.WORKLOADS[spec.pop("workload")], **spec)


def announce(msg):
    print(f"\n[case] {msg}", flush=True)


@pytest.mark.parametrize("name", list(SMALL))
def test_fp8_append_bit_exact(name):
    announce(f"fp8 append {name}")
    inp = make(name)
    d = inp.dims
    st = DeviceStep(inp, kv_scale=FP8_KV_SCALE)
    st.append()
    torch.cuda.synchronize()
    assert int(st.dev_error.item()) == 0
    np.testing.assert_array_equal(st.pool.cpu().numpy(), oracle_pool_fp8(inp))
    cos, sin = O.rope_table_f32(inp.max_pos(), d.d_rope)
    pos = inp.token_pos()
    qpe = O.bf16_to_f64(inp.q_pe).astype(np.float32)
    exp = O.to_bf16_bits(O.rope_cache_f32(qpe, cos[pos][:, None, :], sin[pos][:, None, :]))
    np.testing.assert_array_equal(to_host(st.q_lat, "bf16")[:, :, d.d_latent:], exp)


def _decode_only(inp, st, q_np, num_workgroups):
    from head_latent_attention_05_amd import binding as B
    st.num_workgroups = num_workgroups
    nbytes = B.decode_workspace_size(st.cfg, st.q_start_host, st.kv_lens_host, st.causal,
                                     num_workgroups)
    st.workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=st.dev) if nbytes else None
    q = to_device(q_np, "bf16", st.dev)
    o = torch.full_like(st.o_lat, float("nan"))
    st.decode(q_lat=q, o_lat=o)
    torch.cuda.synchronize()
    return O.bf16_to_f64(to_host(o, "bf16"))


@pytest.mark.parametrize("name", list(SMALL))
def test_fp8_decode_latent_and_split_invariance(name):
    inp = make(name)
    d = inp.dims
    st = DeviceStep(inp, kv_scale=FP8_KV_SCALE)
    st.append()
    q_np = synth.random_latent_queries(d, inp.T, seed=5)
    pool = oracle_pool_fp8(inp)
    heads = sample_heads(d.num_heads)
    ref = O.latent_decode(d, O.bf16_to_f64(q_np), rows_fn_fp8(pool, inp), inp.kv_lens,
                          inp.q_start, inp.workload.causal, heads)
    tol = 2.0 ** -7 * np.abs(ref).max()
    outs = {}
    for G in (1, 2, 7, 0, 100000):
        announce(f"fp8 decode {name} G={G}")
        got = _decode_only(inp, st, q_np, G)
        assert np.all(np.isfinite(got)), f"G={G}"
        err = np.abs(got[:, heads] - ref).max()
        print(f"[parity] fp8 decode {name} G={G} max_abs={err:.3e} tol={tol:.3e}", flush=True)
        assert err <= tol, (G, err, tol)
        outs[G] = got
    again = _decode_only(inp, st, q_np, 7)
    np.testing.assert_array_equal(again, outs[7])


@pytest.mark.parametrize("name", list(SMALL))
def test_fp8_full_step(name):
    announce(f"fp8 step {name}")
    inp = make(name)
    d = inp.dims
    st = DeviceStep(inp, kv_scale=FP8_KV_SCALE)
    st.run()
    torch.cuda.synchronize()
    assert int(st.dev_error.item()) == 0
    heads = sample_heads(d.num_heads, 8)
    ref, _ = O.step_fp8(inp, FP8_KV_SCALE, heads)
    check_out(d, st.out.cpu().numpy()[:, heads], ref, f"fp8 {name}")


@pytest.mark.parametrize("profile", ["rising", "sink"])
def test_fp8_wide_logit_range(profile):
    """Logits far beyond the unit spread: the softmax weights reach the
    lazy-rescale bound and the rescaling runs (several split plans)."""
    base = synth.make_inputs("batch64", kv_lens=[700, 1333])
    inp = scale_rows(base, LOGIT_PROFILES[profile]([int(L) for L in base.kv_lens]))
    d = inp.dims
    kv_scale = 2.0 ** 2 if profile == "rising" else FP8_KV_SCALE
    heads = sample_heads(d.num_heads)
    pool = oracle_pool_fp8(inp, kv_scale)
    ref = O.naive_mla(d, inp.w_uk, inp.w_uv, inp.q_nope, inp.q_pe,
                      rows_fn_fp8(pool, inp, kv_scale), inp.kv_lens, inp.q_start, False, heads)
    for G in (1, 7, 0):
        announce(f"fp8 wide logits {profile} G={G}")
        st = DeviceStep(inp, num_workgroups=G, kv_scale=kv_scale)
        st.run()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(st.pool.cpu().numpy(), pool)
        got = st.out.cpu().numpy()[:, heads]
        assert np.all(np.isfinite(got))
        err = np.abs(got - ref).max()
        print(f"[parity] fp8 wide {profile} G={G} max_abs={err:.3e} "
              f"ref_max={np.abs(ref).max():.3e}", flush=True)
        assert err <= 2e-2 * max(1.0, np.abs(ref).max()), (G, err)


def test_fp8_more_than_64_sequences_and_empty_queries():
    """130 short sequences (the plan walks sequences 64 at a time), some of them
    with no query token."""
    announce("fp8 130 sequences")
    rng = np.random.default_rng(130)
    lens = [int(x) for x in rng.integers(1, 200, 130)]
    base = synth.make_inputs("batch64", kv_lens=lens)
    from tests.gpu_util import drop_queries
    inp = drop_queries(base, {3, 64, 65, 129})
    d = inp.dims
    st = DeviceStep(inp, kv_scale=FP8_KV_SCALE)
    st.run()
    torch.cuda.synchronize()
    assert int(st.dev_error.item()) == 0
    heads = sample_heads(d.num_heads, 4)
    ref, pool = O.step_fp8(inp, FP8_KV_SCALE, heads)
    np.testing.assert_array_equal(st.pool.cpu().numpy(), pool)
    check_out(d, st.out.cpu().numpy()[:, heads], ref, "fp8 130 sequences")


HEADS = [0, 63, 64, 127]


@pytest.mark.parametrize("name", ["single", "batch64", "long", "prefill"])
def test_fp8_fullsize_step_sampled(name):
    """Full workload sizes, default split plan (as benchmarked): the whole e4m3
    cache bit for bit, the output on sampled sequences and heads."""
    announce(f"fp8 full-size step {name}")
    inp = synth.make_inputs(name)
    d = inp.dims
    st = DeviceStep(inp, kv_scale=FP8_KV_SCALE)
    st.run()
    torch.cuda.synchronize()
    assert int(st.dev_error.item()) == 0
    pool = oracle_pool_fp8(inp)
    np.testing.assert_array_equal(st.pool.cpu().numpy(), pool)
    B = len(inp.kv_lens)
    seqs = []
    for b in [0, B - 1, int(np.argmax(inp.kv_lens)), int(np.argmin(inp.kv_lens))]:
        if b not in seqs:
            seqs.append(b)
    toks = np.concatenate([np.arange(inp.q_start[b], inp.q_start[b + 1]) for b in seqs])
    q_lens = np.array([inp.q_start[b + 1] - inp.q_start[b] for b in seqs])
    q_start = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int64)
    kv = inp.kv_lens[seqs]
    rows = lambda i: O.gather_rows_fp8(pool, d, 64, inp.block_table, seqs[i], int(kv[i]),
                                       FP8_KV_SCALE)
    ref = O.naive_mla(d, inp.w_uk, inp.w_uv, inp.q_nope[toks], inp.q_pe[toks], rows, kv,
                      q_start, inp.workload.causal, HEADS)
    check_out(d, st.out.cpu().numpy()[toks][:, HEADS], ref, f"fp8 full {name} seqs={seqs}")


@pytest.mark.parametrize("fp8", [False, True])
def test_error_flags_bad_entries_and_lengths(fp8):
    """Both caches: the append skips and flags out-of-range positions, sequence
    ids and block ids; the decode flags an unassigned block (and reads only
    inside the pool) and flags device lengths that disagree with the host
    copies before touching anything."""
    from head_latent_attention_05_amd import binding as B
    announce(f"error flags fp8={fp8}")
    inp = synth.make_inputs("batch64", kv_lens=[70, 129])
    st = DeviceStep(inp, kv_scale=FP8_KV_SCALE if fp8 else None)
    dev = st.dev
    before = st.pool.clone()
    seq = torch.tensor([0, 5, 0], dtype=torch.int32, device=dev)
    pos = torch.tensor([100000, 3, 127], dtype=torch.int32, device=dev)
    bt = st.block_table.clone()
    bt[0, 1] = -1
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    ck = torch.zeros((3, inp.dims.d_latent), dtype=torch.bfloat16, device=dev)
    kp = torch.zeros((3, inp.dims.d_rope), dtype=torch.bfloat16, device=dev)
    if fp8:
        B.append_cache_fp8(st.cfg, ck, kp, None, seq, pos, bt, st.num_blocks, st.rope_cos,
                           st.rope_sin, FP8_KV_SCALE, st.pool, dev_error=err)
    else:
        B.append_cache(st.cfg, ck, kp, None, seq, pos, bt, st.num_blocks, st.rope_cos,
                       st.rope_sin, st.pool, dev_error=err)
    torch.cuda.synchronize()
    e = int(err.item())
    assert e & B.DEVERR_POSITION and e & B.DEVERR_SEQ and e & B.DEVERR_BLOCK
    assert torch.equal(st.pool.view(torch.uint8), before.view(torch.uint8))
    st.append()
    torch.cuda.synchronize()
    # device lengths that disagree with the host plan
    st.dev_error.zero_()
    good = st.kv_lens
    st.kv_lens = good + 100
    st.decode()
    torch.cuda.synchronize()
    assert int(st.dev_error.item()) & B.DEVERR_LENGTH
    st.kv_lens = good
    # an unassigned block in the table
    st.dev_error.zero_()
    st.block_table[1, 1] = -1
    st.decode()
    torch.cuda.synchronize()
    assert int(st.dev_error.item()) & B.DEVERR_BLOCK
