"""Token layouts and the static window (CPU reference, test infrastructure).

Pins: ``fractal_order`` -- bijection, per-block coordinate consistency and the
closed-form patch-length histogram (tests/test_oracle_layout.py);
``tile_order`` -- equals ``fractal_order`` for (1, P, P), one box over the
whole latent is the identity, bijection, every block is one box at its grid
position, closed-form box lengths;
``window_blocks`` -- closed-form per-row counts (product of clipped ranges) and
a brute-force token-level check; ``raster_blocks`` -- closed form.
"""

from __future__ import annotations

import numpy as np


def raster_blocks(n_valid: int, block: int = 64):
    """Consecutive blocks of ``block`` tokens over the valid prefix.

    NABLA summary, Metodologia section 2 ("Sottocampionamento"): Q and K are
    reshaped into blocks of N tokens. The last block holds the remainder.
    Returns (start, length) int64 arrays.
    """
    nb = -(-n_valid // block)
    start = np.arange(nb, dtype=np.int64) * block
    length = np.minimum(block, n_valid - start)
    return start, length


def fractal_order(T: int, Hl: int, Wl: int, P: int, N: int | None = None):
    """Fractal flattening: every P x P spatial patch becomes contiguous.

    NABLA summary, Metodologia section 1 ("Riordinamento dei Token (Fractal
    Flattening)"): tokens inside each P x P spatial patch are grouped into a
    contiguous run and the time dimension stays ordered.

    Reading for latent sizes that P does not divide: patches tile each frame
    row-major on a ceil(Hl/P) x ceil(Wl/P) grid and edge patches are smaller;
    inside a patch tokens stay row-major; no padding tokens are inserted, so
    blocks (= patches) have variable length.

    Returns
      perm    int64 [N]: perm[new_position] = original raster index
              (positions >= T*Hl*Wl map to themselves),
      start, length  int64 [nblocks]: the block of each patch in the new order,
      coords  int64 [nblocks, 3]: (t, patch_row, patch_col) of each block.
    """
    n_valid = T * Hl * Wl
    N = n_valid if N is None else N
    perm = []
    start, length, coords = [], [], []
    npy, npx = -(-Hl // P), -(-Wl // P)
    for t in range(T):
        for py in range(npy):
            for px in range(npx):
                s = len(perm)
                for y in range(py * P, min(Hl, (py + 1) * P)):
                    for x in range(px * P, min(Wl, (px + 1) * P)):
                        perm.append((t * Hl + y) * Wl + x)
                start.append(s)
                length.append(len(perm) - s)
                coords.append((t, py, px))
    perm.extend(range(n_valid, N))
    return (np.asarray(perm, dtype=np.int64), np.asarray(start, dtype=np.int64),
            np.asarray(length, dtype=np.int64), np.asarray(coords, dtype=np.int64))


def tile_order(T: int, Hl: int, Wl: int, pt: int, ph: int, pw: int, N: int | None = None):
    """Head-aware tiling layout: every pt x ph x pw box of the latent becomes
    one contiguous block.

    Veda summary, section 2.2 ("Tiling Consapevole delle Teste"): each layer and
    head gets its own tiling configuration pi = (p_t, p_h, p_w), a
    factorisation of the hardware tile, so the tokens of one tile are a
    p_t x p_h x p_w box of the video instead of a fixed spatial patch.

    Reading (as for the fractal order): boxes are numbered row-major over the
    ceil(T/pt) x ceil(Hl/ph) x ceil(Wl/pw) grid, frame boxes slowest; inside a
    box tokens keep raster order (t, y, x); edge boxes are smaller and no
    padding tokens are inserted, so blocks have variable length. Positions
    >= T*Hl*Wl map to themselves.

    Computed as a stable sort of the raster tokens by box number. Returns
    (perm, start, length, coords) like ``fractal_order``, with coords the box
    grid position (bt, by, bx).
    """
    n_valid = T * Hl * Wl
    N = n_valid if N is None else N
    t, y, x = np.meshgrid(np.arange(T), np.arange(Hl), np.arange(Wl), indexing="ij")
    nby, nbx = -(-Hl // ph), -(-Wl // pw)
    nbt = -(-T // pt)
    box = ((t // pt) * nby + y // ph) * nbx + x // pw
    box = box.reshape(-1)
    order = np.argsort(box, kind="stable")
    counts = np.bincount(box, minlength=nbt * nby * nbx)
    start = np.concatenate([[0], np.cumsum(counts)[:-1]])
    g = np.arange(nbt * nby * nbx)
    coords = np.stack([g // (nby * nbx), (g // nbx) % nby, g % nbx], axis=1)
    perm = np.concatenate([order, np.arange(n_valid, N)]).astype(np.int64)
    return perm, start.astype(np.int64), counts.astype(np.int64), coords.astype(np.int64)


def block_coords_from_tokens(token_xyz: np.ndarray, perm: np.ndarray,
                             start: np.ndarray, length: np.ndarray, P: int):
    """Block (t, y//P, x//P) derived from the coordinates of its tokens.

    ``token_xyz`` holds the raster (t, y, x) of every original token. Raises
    if the tokens of one block disagree (the block is then not a patch).
    """
    out = np.zeros((len(start), 3), dtype=np.int64)
    for i, (s, n) in enumerate(zip(start, length)):
        c = token_xyz[perm[s:s + n]]
        c = np.stack([c[:, 0], c[:, 1] // P, c[:, 2] // P], axis=1)
        if not (c == c[0]).all():
            raise ValueError(f"block {i} spans several patches")
        out[i] = c[0]
    return out


def window_blocks(coords_q: np.ndarray, coords_k: np.ndarray, rt: int, ry: int, rx: int):
    """Static sliding-tile window between blocks, bool [nq, nk].

    NABLA summary, Metodologia section 3: the final mask is the union of the
    content-adaptive mask and a static Sliding Tile Attention window.
    Reading: a key tile is inside the window of a query tile when their tile
    coordinates differ by at most rt frames, ry tile rows and rx tile columns
    (a box clipped at the video edges, no wrap-around).
    """
    d = np.abs(coords_q[:, None, :] - coords_k[None, :, :])
    return (d[..., 0] <= rt) & (d[..., 1] <= ry) & (d[..., 2] <= rx)
