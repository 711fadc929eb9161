"""Block-sparse attention by its definition (CPU reference, test infrastructure).

NABLA summary, Metodologia section 2 ("Espansione"): the binary block mask is
expanded back to token resolution and decides which query x key tiles are
computed. Attention restricted to those tiles is exactly softmax attention
with every score outside a kept tile set to -inf, which is what this module
computes, explicitly, one query block at a time, in float64.

Sparse VideoGen2 summary, Metodologia A ("Equivalenza Matematica"): after a
token permutation the output, permuted back, equals attention in the original
order; ``permuted_attention`` follows those steps literally.

Pins (tests/test_oracle_attention.py): with every block kept the result equals
dense attention from ``torch.nn.functional.scaled_dot_product_attention`` in
float64; a window-only mask equals that library routine under an explicit
token-level mask built from coordinates; two-key closed form; every output row
lies in the per-column range of V; permutation equivariance.
"""

from __future__ import annotations

import numpy as np


def masked_attention(q, k, v, qstart, qlen, kstart, klen, keep,
                     scale: float | None = None, blocks=None, n_rows=None):
    """Attention where query block I sees key block J only if keep[I, J].

    q, k, v: [N, d] (any float dtype; converted to float64).
    Returns float64 [N, d]; rows outside every listed query block are zero.
    ``blocks`` restricts the computation to a subset of query blocks (rows of
    other blocks stay zero), used to sample large problems.
    A query block with no kept key block yields zero rows.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, d = q.shape
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    out = np.zeros((N if n_rows is None else n_rows, v.shape[1]), dtype=np.float64)
    keep = np.asarray(keep, dtype=bool)
    rng = range(len(qstart)) if blocks is None else blocks
    for I in rng:
        s0, n = int(qstart[I]), int(qlen[I])
        if n == 0:
            continue
        s = np.full((n, N), -np.inf)
        for J in np.nonzero(keep[I])[0]:
            a, m = int(kstart[J]), int(klen[J])
            s[:, a:a + m] = scale * (q[s0:s0 + n] @ k[a:a + m].T)
        if not np.isfinite(s).any():
            continue
        mx = s.max(axis=1, keepdims=True)
        e = np.exp(s - mx)
        p = e / e.sum(axis=1, keepdims=True)
        out[s0:s0 + n] = p @ v
    return out


def permuted_attention(q, k, v, perm_q, perm_k, qstart, qlen, kstart, klen, keep,
                       scale: float | None = None, blocks=None):
    """Reorder tokens, attend block-sparsely, inverse-reorder the output.

    perm_q[i] / perm_k[i] give the original index of the token placed at
    position i. Q is reordered by perm_q, K and V by perm_k; blocks are in the
    reordered positions. Returns the output in the original token order.
    """
    q = np.asarray(q, dtype=np.float64)[perm_q]
    k = np.asarray(k, dtype=np.float64)[perm_k]
    v = np.asarray(v, dtype=np.float64)[perm_k]
    o = masked_attention(q, k, v, qstart, qlen, kstart, klen, keep, scale, blocks)
    out = np.zeros_like(o)
    out[perm_q] = o
    return out


def effective_flops(qlen, klen, keep, d: int) -> float:
    """4 * d * sum over kept (I, J) of len_I * len_J (QK^T and PV products)."""
    keep = np.asarray(keep, dtype=bool)
    ql = np.asarray(qlen, dtype=np.float64)
    kl = np.asarray(klen, dtype=np.float64)
    return float(4.0 * d * (ql[:, None] * kl[None, :] * keep).sum())
