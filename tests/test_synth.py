"""The seeded input generators (test infrastructure): the structure the parity cases rely on."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
from synth import make_inputs, make_inputs_on_device  # noqa: E402


def _check_structure(inp, T, H, K):
    assert inp.rows.shape == (T * K, H) and inp.idx.shape == (T, K)
    assert inp.idx.dtype == torch.int32
    idx = inp.idx.cpu().numpy().ravel()
    valid = idx[idx >= 0]
    # exactly floor(T*K/4) absent routes; the present ones use distinct rows in range
    assert (idx < 0).sum() == (T * K) // 4
    assert len(np.unique(valid)) == valid.size and valid.max(initial=0) < T * K
    sc = inp.scales.cpu().double().numpy()
    assert (sc > 0).all() and np.allclose(sc.sum(axis=1), 1.0, atol=1e-6)
    for t in (inp.shared, inp.residual):
        assert t.shape == (T, H) and t.dtype == inp.rows.dtype
    assert inp.gamma.shape == (H,)


def test_host_generator_structure_and_determinism():
    a = make_inputs(13, 64, 6, seed=11)
    b = make_inputs(13, 64, 6, seed=11)
    _check_structure(a, 13, 64, 6)
    assert torch.equal(a.rows, b.rows) and torch.equal(a.idx, b.idx)


def test_device_generator_structure_and_determinism():
    """The device generator draws the same distributions (checked on the CPU device)."""
    a = make_inputs_on_device(37, 96, 8, seed=5, device="cpu")
    b = make_inputs_on_device(37, 96, 8, seed=5, device="cpu")
    _check_structure(a, 37, 96, 8)
    assert torch.equal(a.rows, b.rows) and torch.equal(a.idx, b.idx)
    assert torch.equal(a.scales, b.scales) and torch.equal(a.gamma, b.gamma)
    r = a.rows.double()
    assert abs(float(r.mean())) < 0.05 and abs(float(r.std()) - 1.0) < 0.05
