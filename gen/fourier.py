"""Seeded synthetic Q/K/V with spatio-temporal structure.

The pages measure on attention layers of real video models; none of those
weights or videos is available, so every input here is synthetic. Queries and
keys are smooth functions of the token's (t, y, x) latent position plus noise,
which gives the attention maps the local, content-dependent structure that
block pooling exploits:

    phi_k(pos) = cos(omega_k . pos + b_k),   k = 1..nfeat (random Fourier
                                             features, omega_k ~ N(0, s^2 I3),
                                             b_k ~ U[0, 2 pi))
    q_i = g * (W_q phi(pos_i) + 0.3 eps_i),  W_q ~ N(0, 1/nfeat), eps ~ N(0, 1)
    k_i = g * (W_k phi(pos_i) + 0.3 eps'_i)  (own W_k and noise)
    v_i ~ N(0, 1)

Values are drawn in float32 and rounded to bfloat16 (round-to-nearest-even,
torch's conversion). Rows past the last real token are zero.

Random streams: one numpy ``SeedSequence(seed)`` is split into independent
children so that any head can be generated on its own:
  child 0            -> omega, b (shared by Q, K and all heads)
  child 1 + h        -> W_q^h, W_k^h
  child 1 + H + b*H + h -> eps_q, eps_k, V of (batch b, head h)

This module holds no step of the attention method; it only makes inputs.
"""

from __future__ import annotations

from typing import Iterable, Optional

import numpy as np
import torch

from .configs import Workload

NFEAT = 32
OMEGA_STD = 0.5
NOISE = 0.3


def token_coords(T: int, Hl: int, Wl: int) -> np.ndarray:
    """Integer (t, y, x) of every latent token in row-major order, [T*Hl*Wl, 3]."""
    t, y, x = np.meshgrid(np.arange(T), np.arange(Hl), np.arange(Wl), indexing="ij")
    return np.stack([t.ravel(), y.ravel(), x.ravel()], axis=1).astype(np.int64)


def _children(seed: int, count: int):
    return np.random.SeedSequence(seed).spawn(count)


def _features(w: Workload, seed: int) -> np.ndarray:
    ch = _children(seed, 1)[0]
    rng = np.random.default_rng(ch)
    omega = rng.normal(0.0, OMEGA_STD, size=(NFEAT, 3))
    phase = rng.uniform(0.0, 2.0 * np.pi, size=NFEAT)
    pos = token_coords(w.T, w.Hl, w.Wl).astype(np.float64)
    return np.cos(pos @ omega.T + phase).astype(np.float32)  # [n_valid, NFEAT]


def generate_head(w: Workload, b: int, h: int, seed: int = 0,
                  phi: Optional[np.ndarray] = None):
    """float32 numpy (q, k, v) for one (batch, head), each [N, d], pads zero."""
    if phi is None:
        phi = _features(w, seed)
    kids = _children(seed, 1 + w.H + w.B * w.H)
    rw = np.random.default_rng(kids[1 + h])
    sd = np.sqrt(1.0 / NFEAT)
    wq = rw.normal(0.0, sd, size=(w.d, NFEAT)).astype(np.float32)
    wk = rw.normal(0.0, sd, size=(w.d, NFEAT)).astype(np.float32)
    rn = np.random.default_rng(kids[1 + w.H + b * w.H + h])
    n = w.n_valid
    eq = rn.standard_normal((n, w.d), dtype=np.float32)
    ek = rn.standard_normal((n, w.d), dtype=np.float32)
    ev = rn.standard_normal((n, w.d), dtype=np.float32)
    out = []
    for base, noise in ((phi @ wq.T, eq), (phi @ wk.T, ek)):
        x = np.zeros((w.N, w.d), dtype=np.float32)
        x[:n] = w.gain * (base + NOISE * noise)
        out.append(x)
    v = np.zeros((w.N, w.d), dtype=np.float32)
    v[:n] = ev
    out.append(v)
    return tuple(out)


def generate(w: Workload, seed: int = 0, heads: Optional[Iterable[int]] = None):
    """bf16 torch tensors (q, k, v), each [B, Hsel, N, d] on the CPU.

    ``heads`` selects a subset of heads (default: all); each head's values do
    not depend on which other heads are generated.
    """
    heads = list(range(w.H)) if heads is None else list(heads)
    phi = _features(w, seed)
    shape = (w.B, len(heads), w.N, w.d)
    q = torch.empty(shape, dtype=torch.bfloat16)
    k = torch.empty(shape, dtype=torch.bfloat16)
    v = torch.empty(shape, dtype=torch.bfloat16)
    for b in range(w.B):
        for i, h in enumerate(heads):
            qh, kh, vh = generate_head(w, b, h, seed, phi)
            q[b, i] = torch.from_numpy(qh).to(torch.bfloat16)
            k[b, i] = torch.from_numpy(kh).to(torch.bfloat16)
            v[b, i] = torch.from_numpy(vh).to(torch.bfloat16)
    return q, k, v


def kmeans_uniforms(B: int, H: int, C: int, seed: int = 0, stream: int = 0) -> np.ndarray:
    """Uniform draws in [0, 1) for k-means++ seeding, float32 [B, H, C].

    The seeding step of k-means++ draws one uniform per chosen centre; both
    implementations receive the same draws as an input array. ``stream``
    separates the query and key clusterings.
    """
    ss = np.random.SeedSequence([seed, 0x6B6D, stream])
    u = np.random.default_rng(ss).random((B, H, C), dtype=np.float32)
    return u


def next_step(x: torch.Tensor, step: int, drift: float = 0.05, seed: int = 0, stream: int = 0) -> torch.Tensor:
    """Stand-in for the same activation ``step`` denoising steps later.

    Activations of a video DiT change slowly from one denoising step to the
    next; this adds independent Gaussian noise of standard deviation
    ``drift`` times the tensor's RMS to every element (bf16 [B, H, N, d] in,
    same out), seeded by (seed, step, stream). All-zero rows (padding) stay
    zero.
    """
    xf = x.float()
    rms = float(xf.pow(2).mean().sqrt())
    ss = np.random.SeedSequence([seed, 0x5354, step, stream])
    eta = torch.from_numpy(np.random.default_rng(ss).standard_normal(tuple(x.shape), dtype=np.float32))
    live = (xf != 0).any(-1, keepdim=True)
    return torch.where(live, xf + drift * rms * eta, xf).to(x.dtype)
