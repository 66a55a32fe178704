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


def _ulps(a, b, act):
    fmt = O.FORMATS[act]
    return ulp_distance(O.encode_bits(a, fmt), O.encode_bits(b, fmt))


def report(name, got, ref_vals, act):
    ud = _ulps(got, ref_vals, act)
    return {"name": name, "max_ulp": int(ud.max()) if ud.size else 0,
            "n_gt1ulp": int((ud > 1).sum()), "n_diff": int((ud > 0).sum()),
            "n": int(ud.size)}


def _one_ulp_rule(name, got, want, lo, hi, act):
    """Within 1 ulp of the oracle's value everywhere except where the float32 window [lo, hi]
    itself reaches farther than 1 ulp from it (certified cancellation: there a correct float32
    evaluation may land farther away). Returns the report with the count of such elements."""
    ud = _ulps(got, want, act)
    wide = (_ulps(lo, want, act) > 1) | (_ulps(hi, want, act) > 1)
    narrow_bad = (ud > 1) & ~wide
    assert not narrow_bad.any(), f"{int(narrow_bad.sum())} {name} elements > 1 ulp where the " \
                                 f"float32 window is within 1 ulp; first at " \
                                 f"{np.argwhere(narrow_bad)[0]}"
    rep = report(name, got, want, act)
    rep["n_window_wider_than_1ulp"] = int(wide.sum())
    return rep


def check_finalize(got_s: np.ndarray, ref: Ref, act: str):
    """Finalize values: every element inside the float32 admissible window, and within 1 ulp of
    the oracle's wherever that window is."""
    bad = outside(got_s, ref.lo, ref.hi)
    assert not bad.any(), f"{int(bad.sum())} finalize elements outside the float32 window; " \
                          f"first at {np.argwhere(bad)[0]}"
    return _one_ulp_rule("s", got_s, ref.s, ref.lo, ref.hi, act)


def check_residual(got_R: np.ndarray, ref: Ref, residual: np.ndarray, act: str):
    """residual_out = RNE_T(a + residual) for some a in the admissible window of s; RNE_T is
    monotone, so it lies between the images of the window's ends. Within 1 ulp of the oracle's
    wherever that image is."""
    fmt = O.FORMATS[act]
    rlo = O.round_to_format(ref.lo + residual, fmt)
    rhi = O.round_to_format(ref.hi + residual, fmt)
    bad = outside(got_R, rlo, rhi)
    assert not bad.any(), f"{int(bad.sum())} residual_out elements outside the window; " \
                          f"first at {np.argwhere(bad)[0]}"
    return _one_ulp_rule("residual_out", got_R, ref.R, rlo, rhi, act)


def oracle_norm_of(got_R: np.ndarray, gamma: np.ndarray, eps, act: str) -> np.ndarray:
    """The oracle's RMSNorm of a given residual_out (R + 0 rounds to R exactly)."""
    return O.residual_rmsnorm(got_R, np.zeros_like(got_R), gamma, eps, act)[1]


def check_norm(got_N: np.ndarray, got_R: np.ndarray, ref: Ref, gamma: np.ndarray, eps, act: str):
    """norm_out within 1 ulp, everywhere, of the oracle's RMSNorm of the kernel's own
    residual_out; reported against the primary oracle's norm_out as well."""
    own = oracle_norm_of(got_R, gamma, eps, act)
    ud = _ulps(got_N, own, act)
    assert ud.max(initial=0) <= 1, f"{int((ud > 1).sum())} norm_out elements > 1 ulp from the " \
                                   f"oracle's norm of the kernel's residual_out; first at " \
                                   f"{np.argwhere(ud > 1)[0]}"
    rep = report("norm_out", got_N, ref.N, act)
    rep["max_ulp_vs_norm_of_own_residual"] = int(ud.max(initial=0))
    return rep


# ---- accuracy records (written to $MFIN_ACCURACY_JSON at the end of a pytest session) ---------
ACCURACY = []


def record_accuracy(config: str, inp, entry: str, rows: str, reps, R=None, N=None, extra=None):
    """One record per configuration sub-case: the comparison reports (max ulp and counts against
    the oracle) and, when residual_out / norm_out are given, their mean absolute error against the
    unrounded FP64 reference beside the rounding floor (the mean error of rounding that exact
    result to the activation dtype once) and the oracle's own error ([FI6631] Description and
    benchmark script: mean |err| of residual_out and norm_out against FP64)."""
    rec = {"config": config, "T": inp.T, "H": inp.H, "K": inp.K, "act": inp.act_dtype,
           "scales": inp.scale_dtype, "shared": inp.shared is not None, "seed": inp.seed,
           "entry": entry, "rows": rows, "checks": reps}
    if R is not None:
        res_ref, norm_ref = O.reference_unrounded(np64(inp.rows), inp.idx.numpy(),
                                                  np64(inp.scales), np64(inp.shared), inp.rsf,
                                                  np64(inp.residual), np64(inp.gamma), inp.eps)
        fmt = O.FORMATS[inp.act_dtype]
        ref = oracle_ref(inp)
        for name, got, exact, orc in (("residual_out", R, res_ref, ref.R),
                                      ("norm_out", N, norm_ref, ref.N)):
            if got is None:
                continue
            rec[name] = {"mean_abs_err": float(np.abs(got - exact).mean()),
                         "oracle_mean_abs_err": float(np.abs(orc - exact).mean()),
                         "floor_mean_abs_err": float(np.abs(O.round_to_format(exact, fmt)
                                                            - exact).mean()),
                         "max_abs_err": float(np.abs(got - exact).max())}
    if extra:
        rec.update(extra)
    ACCURACY.append(rec)
    return rec


def write_accuracy(path: str, command: str) -> None:
    import json
    with open(path, "w") as fh:
        json.dump({"command": command, "records": ACCURACY}, fh, indent=1)
