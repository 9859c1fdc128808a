"""GPU parity of the weight-level absorbed calls (mla_absorb_q_fused,
mla_out_proj_fused) against the oracle, at DeepSeek-V3 widths (d_cq 1536,
d_model 7168) and token counts spanning one and two 64-token tiles."""
import numpy as np
import pytest
import torch

from head_latent_attention_05_amd import binding as B
from head_latent_attention_05_amd import synth
from head_latent_attention_05_amd.step import to_device, to_host
from oracle import mla_oracle as O

pytestmark = pytest.mark.gpu

# fp32 sums of up to 65536 products: a few fp32 units per partial sum of about
# the output's size; 5e-5 of the largest output bounds that with a wide margin
# while a lost range or head (about 1/16 of a value) is far outside it
OUT_REL = 5e-5


@pytest.mark.parametrize("T", [1, 64, 70])
def test_absorb_q_fused(T):
    print(f"\n[case] absorb_q_fused T={T}", flush=True)
    d = synth.V3
    dev = torch.device("cuda:0")
    cfg = B.MlaConfig.from_dims(d)
    fi = synth.make_fused_inputs(d, T, d_cq=1536, d_model=256, seed=51)
    q_lat = torch.full((T, d.num_heads, d.row), 0x7FC1, dtype=torch.int16,
                       device=dev).view(torch.bfloat16)
    B.absorb_q_fused(cfg, to_device(fi.c_q, d.dtype, dev), to_device(fi.w_kq, d.dtype, dev), q_lat)
    torch.cuda.synchronize()
    got_bits = to_host(q_lat, d.dtype)
    ref = O.absorb_q_fused(d, fi.c_q, fi.w_kq)
    got = O.storage_to_f64(got_bits[:, :, :d.d_latent], d.dtype)
    # one bf16 rounding of an fp32 sum of 1536 products
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-5 * np.abs(ref).max())
    assert np.all(got_bits[:, :, d.d_latent:].view(np.uint16) == 0x7FC1)


@pytest.mark.parametrize("T", [1, 64, 70])
def test_out_proj_fused(T):
    print(f"\n[case] out_proj_fused T={T}", flush=True)
    d = synth.V3
    dev = torch.device("cuda:0")
    cfg = B.MlaConfig.from_dims(d)
    d_model = 7168
    fi = synth.make_fused_inputs(d, T, d_cq=128, d_model=d_model, seed=52)
    out = torch.full((T, d_model), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty(B.out_proj_fused_workspace_size(cfg, T, d_model), dtype=torch.uint8,
                     device=dev)
    o = to_device(fi.o_lat, d.dtype, dev)
    w = to_device(fi.w_ov, d.dtype, dev)
    B.out_proj_fused(cfg, o, w, out, ws)
    torch.cuda.synchronize()
    # 96 sampled columns (the first and last tile's edges among them) of all tokens
    rng = np.random.default_rng(T)
    cols = sorted(set([0, 255, 256, d_model - 1]) | set(rng.integers(0, d_model, 92).tolist()))
    got = out.cpu().numpy()[:, cols]
    assert np.all(np.isfinite(out.cpu().numpy()))
    ref = O.out_proj_fused(d, O.storage_to_f64(fi.o_lat, d.dtype), fi.w_ov, cols)
    err = np.abs(got - ref).max()
    print(f"[parity] out_proj_fused T={T} max err {err:.3g} of max |ref| "
          f"{np.abs(ref).max():.3g}", flush=True)
    assert err <= OUT_REL * np.abs(ref).max()
    # the fixed-order reduction: a second call gives the same bits
    out2 = torch.empty_like(out)
    B.out_proj_fused(cfg, o, w, out2, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
