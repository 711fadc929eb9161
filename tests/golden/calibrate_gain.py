"""Bisect the generator gain g against the reference mask sparsity.

The synthetic Q/K generator is scaled by a gain g (larger g -> sharper
attention -> sparser CDF mask). This script finds, for a workload, the g at
which the CPU reference mask stage (pool -> reduced attention -> CDF select,
NABLA summary, Metodologia section 2) drops the target share of key blocks on
seed 0, over the heads given. It calls only the input generator and the
reference; the gains it prints are frozen in ``gen/configs.py``.

    python tests/golden/calibrate_gain.py wan480 0.875 --heads 0 1 2 3
"""

import argparse
import dataclasses
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))

from gen import WORKLOADS, generate_head  # noqa: E402
from gen.fourier import _features  # noqa: E402
from oracle import layout as ol, mask as om  # noqa: E402


def sparsity(w, heads, seed=0):
    st, ln = ol.raster_blocks(w.n_valid, w.block)
    phi = _features(w, seed)
    kept = total = 0
    for h in heads:
        q, k, _ = generate_head(w, 0, h, seed, phi)
        # bf16 rounding as the GPU path sees the inputs
        import torch
        q = torch.from_numpy(q).to(torch.bfloat16).double().numpy()
        k = torch.from_numpy(k).to(torch.bfloat16).double().numpy()
        keep, _ = om.block_mask(q, k, st, ln, st, ln, w.thr)
        kept += keep.sum()
        total += keep.size
    return 1.0 - kept / total


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("workload")
    ap.add_argument("target", type=float)
    ap.add_argument("--heads", type=int, nargs="+", default=[0, 1, 2, 3])
    ap.add_argument("--lo", type=float, default=4.0)
    ap.add_argument("--hi", type=float, default=16.0)
    ap.add_argument("--iters", type=int, default=8)
    a = ap.parse_args()
    base = WORKLOADS[a.workload]
    lo, hi = a.lo, a.hi
    for _ in range(a.iters):
        g = 0.5 * (lo + hi)
        s = sparsity(dataclasses.replace(base, gain=g), a.heads)
        print(f"g={g:.4f} sparsity={s:.4f}", flush=True)
        if s < a.target:
            lo = g
        else:
            hi = g
    print(f"gain ~ {0.5 * (lo + hi):.3f}")


if __name__ == "__main__":
    main()
