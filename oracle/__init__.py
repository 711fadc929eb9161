"""CPU reference for content-adaptive block-sparse attention (TEST INFRASTRUCTURE).

This package is the oracle the GPU path is checked against. It is plain,
slow, float64 numpy, written step by step from the method descriptions:

  * NABLA summary ("Riepilogo Tecnico: NABLA - Neighborhood Adaptive
    Block-Level Attention ..."), Metodologia sections 1-3: fractal
    flattening, block average pooling, reduced attention, CDF thresholding,
    expansion to token resolution, union with a sliding-tile window;
  * Sparse VideoGen2 summary, Metodologia A-C: k-means clustering of Q and K,
    semantic permutation and its inverse, centroid-based top-p selection,
    attention over variable-size blocks.

It shares no code with the HIP library and never imports it. Only the test
suite, the smoke check and the benchmark's CPU-baseline leg may use it; the
product path must never route through it.

Parity status of each function (what pins it against something other than
itself) is listed in each module's docstring.
"""

from . import attention, kmeans, layout, mask  # noqa: F401
