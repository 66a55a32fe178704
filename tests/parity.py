"""Shared machinery of the GPU parity tests: run the HIP path through the C ABI and compare it
with the FP64 oracle on the same seeded inputs (test infrastructure)."""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

import oracle as O
from tests.comparators import admissible_bounds, outside, spacing, ulp_distance


def np64(t):
    return None if t is None else t.double().cpu().numpy()


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().contiguous().view(torch.int16).numpy().astype(np.int64) & 0xFFFF


@dataclass
class Ref:
    S: np.ndarray       # unrounded S*
    mag: np.ndarray     # sum of magnitudes (float32 window)
    s: np.ndarray       # RNE_T(S*)
    R: np.ndarray       # residual_out
    N: np.ndarray       # norm_out
    lo: np.ndarray
    hi: np.ndarray


def oracle_ref(inp, rsf=None, eps=None, with_norm=True) -> Ref:
    rsf = inp.rsf if rsf is None else rsf
    eps = inp.eps if eps is None else eps
    rows, idx = np64(inp.rows), inp.idx.numpy()
    sc, sh = np64(inp.scales), np64(inp.shared)
    S = O.finalize_unrounded(rows, idx, sc, sh, rsf)
    mag = O.finalize_magnitude(rows, idx, sc, sh, rsf)
    s = O.round_to_format(S, O.FORMATS[inp.act_dtype])
    R = N = None
    if with_norm:
        R, N = O.residual_rmsnorm(s, np64(inp.residual), np64(inp.gamma), eps, inp.act_dtype)
    lo, hi = admissible_bounds(S, mag, inp.K, inp.act_dtype)
    return Ref(S, mag, s, R, N, lo, hi)


def to_dev(inp, dev="cuda"):
    d = {}
    for k in ("rows", "idx", "scales", "shared", "residual", "gamma"):
        v = getattr(inp, k)
        d[k] = None if v is None else v.to(dev).contiguous()
    return d


def report(name, got, ref_vals, act):
    fmt = O.FORMATS[act]
    ud = ulp_distance(O.encode_bits(got, fmt), O.encode_bits(ref_vals, fmt))
    return {"name": name, "max_ulp": int(ud.max()) if ud.size else 0,
            "n_gt1ulp": int((ud > 1).sum()), "n_diff": int((ud > 0).sum()),
            "n": int(ud.size)}


def check_finalize(got_s: np.ndarray, ref: Ref, act: str):
    """Finalize values: every element inside the float32 admissible window."""
    bad = outside(got_s, ref.lo, ref.hi)
    assert not bad.any(), f"{int(bad.sum())} finalize elements outside the float32 window; " \
                          f"first at {np.argwhere(bad)[0]}"
    rep = report("s", got_s, ref.s, act)
    assert rep["n_gt1ulp"] <= max(2, rep["n"] // 10000), rep
    return rep


def check_residual(got_R: np.ndarray, ref: Ref, residual: np.ndarray, act: str):
    """residual_out = RNE_T(a + residual) for some a in the admissible window of s; RNE_T is
    monotone, so it lies between the images of the window's ends."""
    fmt = O.FORMATS[act]
    rlo = O.round_to_format(ref.lo + residual, fmt)
    rhi = O.round_to_format(ref.hi + residual, fmt)
    bad = outside(got_R, rlo, rhi)
    assert not bad.any(), f"{int(bad.sum())} residual_out elements outside the window; " \
                          f"first at {np.argwhere(bad)[0]}"
    return report("residual_out", got_R, ref.R, act)


def check_norm(got_N: np.ndarray, got_R: np.ndarray, ref: Ref, gamma: np.ndarray, eps, act: str):
    """norm_out within 1 ulp of the oracle's wherever residual_out matched the oracle; where an
    element of residual_out took another value of its window, the norm may move by that
    difference times gamma / rms (plus 1 ulp)."""
    fmt = O.FORMATS[act]
    ud = ulp_distance(O.encode_bits(got_N, fmt), O.encode_bits(ref.N, fmt))
    same_R = got_R == ref.R
    ok = ud <= 1
    rms = np.sqrt(np.mean(ref.R * ref.R, axis=-1, keepdims=True) + float(np.float32(eps)))
    slack = np.abs(got_R - ref.R) * np.abs(gamma) / rms
    ulp = spacing(np.maximum(np.abs(got_N), np.abs(ref.N)), act)
    ok_moved = np.abs(got_N - ref.N) <= slack + ulp
    bad = ~(ok | (~same_R & ok_moved))
    assert not bad.any(), f"{int(bad.sum())} norm_out elements off; first at {np.argwhere(bad)[0]}"
    return report("norm_out", got_N, ref.N, act)
