"""Minimal driver for hardware-counter runs of the decode call.

Builds one synthetic workload on the GPU, fills two copies of its paged cache
and issues ``--calls`` decode calls alternating between them (so consecutive
calls do not hit a cache left warm by the previous one), then synchronises.
Nothing else is launched after the set-up, which keeps a counter profile's
dispatch list short:

    rocprofv3 --pmc FETCH_SIZE -- python -m head_latent_attention_05_amd.profile_decode
"""
from __future__ import annotations

import argparse


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="batch64")
    ap.add_argument("--calls", type=int, default=4)
    args = ap.parse_args()

    import torch

    from . import synth
    from .step import DeviceStep

    inp = synth.make_inputs(args.workload)
    st = DeviceStep(inp, pool_copies=2)
    for i in range(args.calls):
        st.decode(st.pools[i % 2])
    torch.cuda.synchronize()
    print(f"{args.calls} decode calls on '{args.workload}' done", flush=True)
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
