"""The synthetic workloads reach the sparsity their gains were calibrated for
(reference mask stage on the CPU; no GPU)."""

import numpy as np
import pytest
import torch

from gen import BY_INDEX, WORKLOADS, generate, generate_head
from oracle import layout as ol, mask as om


def _sparsity(w, heads):
    st, ln = ol.raster_blocks(w.n_valid, w.block)
    kept = total = 0
    for h in heads:
        q, k, _ = generate_head(w, 0, h)
        q = torch.from_numpy(q).to(torch.bfloat16).double().numpy()
        k = torch.from_numpy(k).to(torch.bfloat16).double().numpy()
        keep, _ = om.block_mask(q, k, st, ln, st, ln, w.thr)
        kept += keep.sum()
        total += keep.size
    return 1.0 - kept / total


def test_wan480_sparsity_in_band():
    w = WORKLOADS["wan480"]
    s = _sparsity(w, range(w.H))
    lo, hi = w.target_sparsity
    assert lo <= s <= hi, s


@pytest.mark.slow
def test_hunyuan720_sparsity_in_band():
    w = WORKLOADS["hunyuan720"]
    s = _sparsity(w, [0, 7, 15, 23])
    lo, hi = w.target_sparsity
    assert lo <= s <= hi, s


def test_generator_shapes_padding_and_head_independence():
    w = BY_INDEX[1]
    q, k, v = generate(w)
    assert q.shape == (1, 2, 256, 64) and q.dtype == torch.bfloat16
    q1, _, v1 = generate(w, heads=[1])
    assert torch.equal(q1[0, 0], q[0, 1]) and torch.equal(v1[0, 0], v[0, 1])
    w2 = WORKLOADS["wan480"]
    qh, kh, vh = generate_head(w2, 0, 3)
    assert (qh[w2.n_valid:] == 0).all() and (vh[w2.n_valid:] == 0).all()
    assert np.abs(qh[:w2.n_valid]).max() > 0
