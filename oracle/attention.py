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
lies in the per-column range of V; permutation equivariance. The backward and
the row normaliser are pinned against torch autograd / logsumexp of the dense
masked softmax in float64, central finite differences, and the one-key
closed form (dq = dk = 0, dv = the summed upstream gradient).
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


def masked_attention_lse(q, k, qstart, qlen, kstart, klen, keep, scale: float | None = None):
    """Natural-log row normaliser of the block-sparse softmax, float64 [N].

    lse_i = log sum_j exp(scale * q_i . k_j) over the key tokens j of the key
    blocks kept for row i's query block (the same restriction as
    ``masked_attention``); -inf for rows with no kept key block and for rows
    outside every query block. It is what a training forward keeps for the
    backward pass.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    N, d = q.shape
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    out = np.full(N, -np.inf)
    keep = np.asarray(keep, dtype=bool)
    for I in range(len(qstart)):
        s0, n = int(qstart[I]), int(qlen[I])
        cols = [np.arange(int(kstart[J]), int(kstart[J]) + int(klen[J])) for J in np.nonzero(keep[I])[0]]
        cols = np.concatenate(cols) if cols else np.zeros(0, dtype=np.int64)
        if n == 0 or cols.size == 0:
            continue
        s = scale * (q[s0:s0 + n] @ k[cols].T)
        mx = s.max(axis=1, keepdims=True)
        out[s0:s0 + n] = (mx + np.log(np.exp(s - mx).sum(axis=1, keepdims=True)))[:, 0]
    return out


def masked_attention_bwd(q, k, v, do, qstart, qlen, kstart, klen, keep,
                         scale: float | None = None):
    """Gradients (dq, dk, dv) of the block-sparse attention, float64 [N, d] each.

    The NABLA summary (Contributi Chiave, "Accelerazione a Due Fasi"; Risultati
    Sperimentali, 2, pre-training) applies the sparse attention in training as
    well, so its backward is the derivative of ``masked_attention`` with
    respect to q, k and v for an upstream gradient do. Per query block I,
    over the key tokens of its kept blocks:
        S = scale * Q_I K^T,  P = softmax_rows(S),  O_I = P V
        dV += P^T dO_I,  dP = dO_I V^T,  Dr_i = sum_j P_ij dP_ij
        dS = P * (dP - Dr),  dQ_I = scale * dS K,  dK += scale * dS^T Q_I
    Query blocks with no kept key block contribute nothing.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    N, d = q.shape
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    keep = np.asarray(keep, dtype=bool)
    for I in range(len(qstart)):
        s0, n = int(qstart[I]), int(qlen[I])
        cols = [np.arange(int(kstart[J]), int(kstart[J]) + int(klen[J])) for J in np.nonzero(keep[I])[0]]
        cols = np.concatenate(cols) if cols else np.zeros(0, dtype=np.int64)
        if n == 0 or cols.size == 0:
            continue
        qi, gi = q[s0:s0 + n], do[s0:s0 + n]
        kc, vc = k[cols], v[cols]
        s = scale * (qi @ kc.T)
        e = np.exp(s - s.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        dv[cols] += p.T @ gi
        dp = gi @ vc.T
        dr = (p * dp).sum(axis=1, keepdims=True)
        ds = p * (dp - dr)
        dq[s0:s0 + n] = scale * (ds @ kc)
        dk[cols] += scale * (ds.T @ qi)
    return dq, dk, dv


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
