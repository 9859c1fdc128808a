"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (default split plan): the whole cache is compared bit for bit
and the step output is compared with the naive oracle on sampled sequences and
heads (both head halves of the decode kernel)."""
import numpy as np
import pytest
import torch

from head_latent_attention_05_amd import synth
from head_latent_attention_05_amd.step import DeviceStep, to_host
from oracle import mla_oracle as O
from tests.gpu_util import check_out, oracle_pool, pool_bits

pytestmark = pytest.mark.gpu

HEADS = [0, 63, 64, 127]


def _sample_seqs(inp, k=8):
    """The first, last, longest and shortest sequences, then seeded random ones,
    up to k distinct."""
    B = len(inp.kv_lens)
    out = []
    for b in [0, B - 1, int(np.argmax(inp.kv_lens)), int(np.argmin(inp.kv_lens))]:
        if b not in out:
            out.append(b)
    rng = np.random.default_rng(B)
    while len(out) < min(k, B):
        b = int(rng.integers(0, B))
        if b not in out:
            out.append(b)
    return out


@pytest.mark.parametrize("name", ["single", "batch64", "long", "prefill"])
def test_fullsize_step_sampled(name):
    print(f"\n[case] full-size step {name}", flush=True)
    inp = synth.make_inputs(name)
    d = inp.dims
    st = DeviceStep(inp)
    st.run()
    torch.cuda.synchronize()
    assert int(st.dev_error.item()) == 0
    # the whole paged cache, bit for bit (sentinels included)
    pool = oracle_pool(inp)
    np.testing.assert_array_equal(pool_bits(to_host(st.pool, d.dtype), d), pool_bits(pool, d))
    # sampled sequences x heads against the naive (explicit-decompression) oracle
    seqs = _sample_seqs(inp)
    toks = np.concatenate([np.arange(inp.q_start[b], inp.q_start[b + 1]) for b in seqs])
    q_lens = np.array([inp.q_start[b + 1] - inp.q_start[b] for b in seqs])
    q_start = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int64)
    kv = inp.kv_lens[seqs]
    rows = lambda i: O.gather_rows(pool, d, 64, inp.block_table, seqs[i], int(kv[i]))
    ref = O.naive_mla(d, inp.w_uk, inp.w_uv, inp.q_nope[toks], inp.q_pe[toks], rows, kv, q_start,
                      inp.workload.causal, HEADS)
    got = st.out.cpu().numpy()[toks][:, HEADS]
    check_out(d, got, ref, f"full {name} seqs={seqs}")
