"""Workload table: shapes, method parameters and generator gains.

Each entry describes one synthetic attention layer of a video diffusion
transformer. Token counts are video-latent sizes T x H x W (frames x latent
rows x latent columns) flattened row-major (t slowest); the sequence is
padded with zero rows up to ``N``, a multiple of the 64-token block.

The method parameters come from the pages:
  * block size 64 and the CDF threshold ``thr`` -- NABLA summary
    (Metodologia, section 2 "Sottocampionamento" and "CDF Thresholding");
  * the sliding-tile window OR'd into the mask -- NABLA summary
    (Metodologia, section 3, M = M_nabla OR M_STA);
  * fractal flattening into P x P spatial patches -- NABLA summary
    (Metodologia, section 1);
  * k-means clusters C_q, C_k and the top-p budget -- Sparse VideoGen2
    summary (Metodologia A "Clustering" and B "Strategia Top-p");
  * per-head tile factorisations (p_t, p_h, p_w) of the 64-token tile --
    Veda summary, section 2.2 (the three factorisations of 64 into a
    frame x row x column box that fit a 480p latent; the pages choose one per
    head offline on a calibration set, which is not reproduced: heads take
    them in turn).

``gain`` is the scale g applied to the Fourier-feature Q/K generator so that
the content-adaptive mask drops the target share of key blocks. The values
were found by bisection of g against the block sparsity of the CPU reference
mask stage on seed 0 (``tests/golden/calibrate_gain.py``); the test suite
re-checks the achieved sparsity.
"""

from __future__ import annotations

import dataclasses
from typing import Optional, Tuple


@dataclasses.dataclass(frozen=True)
class Workload:
    key: str
    B: int
    H: int
    d: int
    T: int          # latent frames
    Hl: int         # latent rows
    Wl: int         # latent columns
    N: int          # padded sequence length (multiple of 64)
    thr: float      # CDF threshold (drop mass)
    gain: float     # generator gain g
    block: int = 64
    order: str = "raster"            # "raster" | "fractal" | "semantic"
    patch: int = 8                   # fractal patch edge P
    window: Optional[Tuple[int, int, int]] = None   # (rt, ry, rx) in block units
    Cq: int = 0                      # query clusters (semantic order)
    Ck: int = 0                      # key clusters (semantic order)
    kmeans_iters: int = 0
    top_p: float = 0.0
    target_sparsity: Optional[Tuple[float, float]] = None
    tilings: Optional[Tuple[Tuple[int, int, int], ...]] = None   # head h takes tilings[h % len]

    @property
    def n_valid(self) -> int:
        return self.T * self.Hl * self.Wl

    @property
    def nb(self) -> int:
        return self.N // self.block


def _pad64(n: int) -> int:
    return (n + 63) // 64 * 64


# Gains calibrated on the reference mask stage (see module docstring).
GAIN_WAN480 = 8.25
GAIN_HUNYUAN720 = 12.125

TINY = Workload(key="tiny", B=1, H=2, d=64, T=4, Hl=8, Wl=8, N=256,
                thr=0.1, gain=1.0)

WAN480 = Workload(key="wan480", B=1, H=12, d=128, T=21, Hl=30, Wl=52,
                  N=_pad64(21 * 30 * 52), thr=0.2, gain=GAIN_WAN480,
                  target_sparsity=(0.85, 0.90))

HUNYUAN720 = Workload(key="hunyuan720", B=1, H=24, d=128, T=33, Hl=45, Wl=80,
                      N=_pad64(33 * 45 * 80), thr=0.1, gain=GAIN_HUNYUAN720,
                      target_sparsity=(0.875, 0.925))

WAN480_FRACTAL_STA = dataclasses.replace(
    WAN480, key="wan480_fractal_sta", order="fractal", patch=8,
    window=(1, 2, 2), target_sparsity=None)

WAN480_SEMANTIC = dataclasses.replace(
    WAN480, key="wan480_semantic", order="semantic", Cq=64, Ck=256,
    kmeans_iters=10, top_p=0.9, thr=0.1, target_sparsity=None)

WAN480_HEAD_TILING = dataclasses.replace(
    WAN480, key="wan480_head_tiling", order="head_tiling",
    tilings=((1, 8, 8), (2, 4, 8), (4, 4, 4)), target_sparsity=None)

WORKLOADS = {w.key: w for w in (TINY, WAN480, HUNYUAN720,
                                WAN480_FRACTAL_STA, WAN480_SEMANTIC, WAN480_HEAD_TILING)}

# Configs in the order they are listed for this method (1-based index).
BY_INDEX = {1: TINY, 2: WAN480, 3: HUNYUAN720, 4: WAN480_FRACTAL_STA,
            5: WAN480_SEMANTIC}
