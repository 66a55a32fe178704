"""The admissible-window rule separates float32 accumulation from per-step rounding (CPU only).

[FI6631] test changes: the updated reference models float32 accumulation, the "Cake" reference
keeps per-step rounding, and the kernel without the change fails the updated check, so the check
pins the new numerics. Here a numpy float32 model of the finalize (any route order) must pass the
window on every element, and the per-step-rounding model kept in the oracle must fail it.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
from synth import make_inputs
from tests.comparators import admissible_bounds, outside, ulp_distance, values_to_bits


def _fp32_model(rows, idx, sc, sh, rsf, act, reverse=False):
    """float32 accumulation in a fixed route order, one rounding at the end (test model only)."""
    T, K = idx.shape
    acc = np.zeros((T, rows.shape[1]), dtype=np.float32)
    order = range(K - 1, -1, -1) if reverse else range(K)
    for k in order:
        for t in range(T):
            p = idx[t, k]
            if 0 <= p < rows.shape[0]:
                acc[t] = acc[t] + np.float32(sc[t, k]) * rows[p].astype(np.float32)
    s32 = np.float32(rsf) * acc + sh.astype(np.float32)
    dt = torch.bfloat16 if act == "bf16" else torch.float16
    return torch.from_numpy(s32).to(dt).double().numpy()


@pytest.mark.parametrize("case", [(4, 1024, 8, "bf16"), (32, 7168, 8, "bf16"),
                                  (32, 7168, 8, "fp16"), (16, 2048, 22, "bf16")])
def test_window_accepts_fp32_and_rejects_per_step(case):
    T, H, K, act = case
    inp = make_inputs(T, H, K, seed=500 + T + K, act_dtype=act)
    rows = inp.rows.double().numpy()
    idx = inp.idx.numpy()
    sc = inp.scales.double().numpy()
    sh = inp.shared.double().numpy()
    S = O.finalize_unrounded(rows, idx, sc, sh, 2.5)
    mag = O.finalize_magnitude(rows, idx, sc, sh, 2.5)
    lo, hi = admissible_bounds(S, mag, K, act)
    for rev in (False, True):
        f32 = _fp32_model(rows, idx, sc, sh, 2.5, act, reverse=rev)
        assert not outside(f32, lo, hi).any()
    old = O.finalize_per_step_rounding(rows, idx, sc, sh, 2.5, act)
    bad = outside(old, lo, hi)
    assert bad.mean() > 0.05, bad.mean()
    # and the exact single rounding is of course inside
    assert not outside(O.finalize(rows, idx, sc, sh, 2.5, act), lo, hi).any()


def test_ulp_distance():
    a = np.array([0x3F80, 0x3F80, 0x0000, 0x8000, 0x8001, 0x7F7F], dtype=np.uint16)
    b = np.array([0x3F81, 0x3F7F, 0x8000, 0x0001, 0x0001, 0x7F7E], dtype=np.uint16)
    assert list(ulp_distance(a, b)) == [1, 1, 0, 1, 2, 1]
    v = np.array([1.0, -2.0])
    assert list(values_to_bits(v, "bf16")) == [0x3F80, 0xC000]
