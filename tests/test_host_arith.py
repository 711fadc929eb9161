"""Host checks of arithmetic facts the kernels rely on (no GPU).

The k-means assignment forms x.c from a three-way bf16 split of each fp32
centroid, c = c1 + c2 + c3 with c1 = bf16(c), c2 = bf16(c - c1),
c3 = bf16(c - c1 - c2), all rounded to nearest even. Each remainder is exact
in fp32 and the last one fits bf16, so the split loses nothing: the products
with bf16 tokens are then exact and only the fp32 accumulation rounds.
"""

import numpy as np
import torch


def _split3(c: torch.Tensor):
    c1 = c.to(torch.bfloat16).float()
    r1 = c - c1
    c2 = r1.to(torch.bfloat16).float()
    r2 = r1 - c2
    c3 = r2.to(torch.bfloat16).float()
    return c1, c2, c3, r1, r2


def test_three_way_bf16_split_is_exact():
    g = torch.Generator().manual_seed(7)
    # centroid-like values over a wide range of magnitudes, plus edge patterns
    mant = torch.rand(200000, generator=g, dtype=torch.float64) * 2 - 1
    expo = torch.randint(-30, 30, (200000,), generator=g).double()
    c = (mant * torch.pow(2.0, expo)).float()
    edge = torch.tensor([1.0, -1.0, 1.0 + 2 ** -23, 1.0 - 2 ** -24, 3.0 * 2 ** -10, 65504.0, 1e-20, -7.75e7,
                         np.float32(0.1), np.float32(1 / 3)], dtype=torch.float32)
    c = torch.cat([c, edge])
    c1, c2, c3, r1, r2 = _split3(c)
    # the remainders are exact in fp32 (computed in fp64 they agree)
    assert torch.equal(r1.double(), c.double() - c1.double())
    assert torch.equal(r2.double(), r1.double() - c2.double())
    # the last remainder fits bf16, so the three parts sum back to c exactly
    assert torch.equal(c3, r2)
    assert torch.equal(c1.double() + c2.double() + c3.double(), c.double())


def test_split_products_with_bf16_tokens_are_exact():
    """A bf16 token times a bf16 part is exact in fp32 (8 + 8 significant bits)."""
    g = torch.Generator().manual_seed(8)
    x = torch.randn(5000, generator=g).to(torch.bfloat16).float()
    c = torch.randn(5000, generator=g) * 3
    for part in _split3(c)[:3]:
        assert torch.equal((x * part).double(), x.double() * part.double())
