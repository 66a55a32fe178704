"""Pins of the FP64 oracle against facts that do not come from the oracle itself.

Each test states what pins it: a library routine, exact rational brute force, a closed form, an
invariant the pages fix, or a number the pages print. Runs on the CPU (no GPU marker).
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from synth import make_inputs
from tests.exact_ref import frac, grid, rne_exact

RNG = np.random.Generator(np.random.PCG64(20261202))


def _wide_doubles(n):
    """Random doubles across many binades, both signs, plus exact midpoints of narrow grids."""
    mant = RNG.uniform(0.5, 1.0, n)
    ex = RNG.integers(-30, 20, n)
    return np.ldexp(mant, ex) * RNG.choice([-1.0, 1.0], n)


def _midpoints(fmt: str, n: int):
    vals, _ = grid(fmt)
    vals = [float(v) for v in vals]
    i = RNG.integers(0, len(vals) - 1, n)
    lo = np.array([vals[j] for j in i])
    hi = np.array([vals[j + 1] for j in i])
    mid = (lo + hi) / 2  # exact in FP64 for these narrow formats
    return np.concatenate([mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf)])


# ------------------------------------------------------------------------------------------------
# Rounding: pinned by exact rational brute force and by library conversions.
# ------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("fmt", ["bf16", "fp16", "e4m3", "e2m1"])
def test_round_matches_exact_bruteforce(fmt):
    f = O.FORMATS[fmt]
    scale = {"bf16": 1.0, "fp16": 1.0, "e4m3": 2.0 ** 4, "e2m1": 2.0}[fmt]
    xs = np.concatenate([_wide_doubles(400) * scale, _midpoints(fmt, 300), [0.0, -0.0]])
    got = O.round_to_format(xs, f)
    for x, g in zip(xs, got):
        want = rne_exact(Fraction(float(x)), fmt)
        if want is None:
            assert math.isinf(g) and np.sign(g) == np.sign(x)
        else:
            assert Fraction(float(g)) == want, (fmt, x, g, want)


def test_round_fp16_matches_numpy_direct_conversion():
    # numpy converts float64 -> float16 in one correctly rounded step (library pin).
    xs = np.concatenate([_wide_doubles(20000) * 0.01, _midpoints("fp16", 5000),
                         np.array([7e4, -7e4, 65520.0, 65519.99, 1e-9, 3e-8])])
    got = O.round_to_format(xs, O.FP16)
    with np.errstate(over="ignore"):             # values past 65520 overflow to inf, as intended
        want = xs.astype(np.float16).astype(np.float64)
    np.testing.assert_array_equal(got, want)


def test_round_bf16_matches_torch_on_float32_inputs():
    # torch's float32 -> bfloat16 is a single round-to-nearest-even (library pin).
    x32 = (RNG.standard_normal(50000) * np.exp(RNG.uniform(-20, 20, 50000))).astype(np.float32)
    got = O.round_to_format(x32.astype(np.float64), O.BF16)
    want = torch.from_numpy(x32).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(got, want)


def test_round_e4m3_matches_torch_in_range():
    # torch.float8_e4m3fn is OCP E4M3 with round-to-nearest-even; it does not saturate, so only
    # magnitudes that round to at most 448 are compared (library pin).
    x32 = (RNG.uniform(-460, 460, 50000) * np.exp(RNG.uniform(-14, 0, 50000))).astype(np.float32)
    got = O.round_to_format(x32.astype(np.float64), O.E4M3)
    want = torch.from_numpy(x32).to(torch.float8_e4m3fn).float().double().numpy()
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("fmt", ["bf16", "fp16", "e4m3", "e2m1"])
def test_codec_round_trip_exhaustive(fmt):
    f = O.FORMATS[fmt]
    nbits = {"bf16": 16, "fp16": 16, "e4m3": 8, "e2m1": 4}[fmt]
    codes = np.arange(1 << nbits)
    dt = np.uint16 if nbits == 16 else np.uint8
    vals = O.decode_bits(codes.astype(dt), f)
    finite = np.isfinite(vals)
    re = O.encode_bits(vals[finite], f)
    np.testing.assert_array_equal(re.astype(np.int64), codes[finite])
    # every finite value is a fixed point of the rounding
    np.testing.assert_array_equal(O.round_to_format(vals[finite], f), vals[finite])


def test_e4m3_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.decode_bits(codes, O.E4M3)
    theirs = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().double().numpy()
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(theirs))
    ok = ~np.isnan(ours)
    np.testing.assert_array_equal(ours[ok], theirs[ok])


def test_e2m1_magnitudes():
    # The E2M1 value set (0, 0.5, 1, 1.5, 2, 3, 4, 6) and saturation above 6.
    mags = O.decode_bits(np.arange(8, dtype=np.uint8), O.E2M1)
    assert list(mags) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 100.0])
    assert list(O.round_to_format(ties, O.E2M1)) == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, 6.0]


# ------------------------------------------------------------------------------------------------
# Finalize: invariants the pages fix, and exact brute force.
# ------------------------------------------------------------------------------------------------
def _np(inp):
    rows = inp.rows.double().numpy()
    idx = inp.idx.numpy()
    sc = None if inp.scales is None else inp.scales.double().numpy()
    sh = None if inp.shared is None else inp.shared.double().numpy()
    return rows, idx, sc, sh


@pytest.mark.parametrize("act", ["bf16", "fp16"])
def test_k1_is_exact_gather(act):
    # K=1, weight 1, RSF 1, no shared term: the finalized row is the gathered row, bit for bit;
    # an absent route gives zeros.
    inp = make_inputs(9, 64, 1, seed=11, act_dtype=act, scale_dtype=None, with_shared=False,
                      mask_frac=0.25, n_rows=20)
    rows, idx, _, _ = _np(inp)
    s = O.finalize(rows, idx, None, None, 1.0, act)
    for t in range(9):
        p = idx[t, 0]
        want = rows[p] if p >= 0 else np.zeros(64)
        np.testing.assert_array_equal(s[t], want)


def test_route_order_invariance():
    inp = make_inputs(6, 96, 8, seed=12)
    rows, idx, sc, sh = _np(inp)
    base = O.finalize(rows, idx, sc, sh, 2.5, "bf16")
    for trial in range(3):
        perm = np.stack([RNG.permutation(8) for _ in range(6)])
        s2 = O.finalize(rows, np.take_along_axis(idx, perm, 1), np.take_along_axis(sc, perm, 1),
                        sh, 2.5, "bf16")
        np.testing.assert_array_equal(s2, base)


def test_absent_routes_contribute_nothing_and_are_never_read():
    inp = make_inputs(8, 64, 10, seed=13, n_rows=200)
    rows, idx, sc, sh = _np(inp)
    base = O.finalize(rows, idx, sc, sh, 2.5, "bf16")
    # Poison every row no route references and the scale of every absent route.
    poisoned = rows.copy()
    used = set(int(p) for p in idx.ravel() if p >= 0)
    for r in range(rows.shape[0]):
        if r not in used:
            poisoned[r] = np.nan
    sc_p = np.where(idx < 0, np.nan, sc)
    np.testing.assert_array_equal(O.finalize(poisoned, idx, sc_p, sh, 2.5, "bf16"), base)
    # Out-of-range indices on either side are absent routes too.
    idx_oob = np.where(idx < 0, 10_000, idx)
    np.testing.assert_array_equal(O.finalize(rows, idx_oob, sc, sh, 2.5, "bf16"), base)
    # Same result with the absent routes deleted from each token's list.
    for t in range(8):
        keep = idx[t] >= 0
        s_t = O.finalize(rows, idx[t:t + 1, keep], sc[t:t + 1, keep], sh[t:t + 1], 2.5, "bf16")
        np.testing.assert_array_equal(s_t[0], base[t])


def test_optional_terms():
    inp = make_inputs(4, 32, 6, seed=14)
    rows, idx, sc, sh = _np(inp)
    np.testing.assert_array_equal(O.finalize(rows, idx, None, sh, 2.5, "bf16"),
                                  O.finalize(rows, idx, np.ones_like(sc), sh, 2.5, "bf16"))
    np.testing.assert_array_equal(O.finalize(rows, idx, sc, None, 2.5, "bf16"),
                                  O.finalize(rows, idx, sc, np.zeros_like(sh), 2.5, "bf16"))
    # A token with no valid route finalizes to its shared-expert row (or zero).
    idx0 = np.full_like(idx, -1)
    np.testing.assert_array_equal(O.finalize(rows, idx0, sc, sh, 2.5, "bf16"), sh)
    assert not np.any(O.finalize(rows, idx0, sc, None, 2.5, "bf16"))


@pytest.mark.parametrize("act", ["bf16", "fp16"])
@pytest.mark.parametrize("K", [1, 3, 6])
def test_finalize_exact_bruteforce(act, K):
    # Exact rational sum and exact round-to-nearest-even must agree with the oracle bit for bit.
    inp = make_inputs(2, 16, K, seed=100 + K, act_dtype=act, n_rows=2 * K + 3,
                      mask_frac=0.25 if K > 1 else 0.0)
    rows, idx, sc, sh = _np(inp)
    rsf = 2.5
    s = O.finalize(rows, idx, sc, sh, rsf, act)
    for t in range(2):
        for h in range(16):
            acc = Fraction(0)
            for k in range(K):
                p = int(idx[t, k])
                if 0 <= p < rows.shape[0]:
                    acc += frac(sc[t, k]) * frac(rows[p, h])
            exact = Fraction(rsf) * acc + frac(sh[t, h])
            assert Fraction(float(s[t, h])) == rne_exact(exact, act)


def test_dyadic_fixture_closed_form():
    # Integer rows, power-of-two weights, RSF 2 and an integer shared term: every value is exact,
    # so S* is a closed-form integer combination.
    T, H, K = 3, 8, 4
    rows = np.arange(40 * H, dtype=np.float64).reshape(40, H) % 17 - 8
    idx = np.array([[3, -1, 7, 20], [0, 1, 2, 39], [-1, -1, -1, 5]])
    sc = np.array([[0.5, 0.25, 0.125, 1.0], [1.0, 0.5, 0.25, 0.25], [4.0, 4.0, 4.0, 0.0625]])
    sh = np.full((T, H), 3.0)
    s = O.finalize(rows, idx, sc, sh, 2.0, "bf16")
    want0 = 2 * (0.5 * rows[3] + 0.125 * rows[7] + 1.0 * rows[20]) + 3
    want1 = 2 * (rows[0] + 0.5 * rows[1] + 0.25 * rows[2] + 0.25 * rows[39]) + 3
    want2 = 2 * (0.0625 * rows[5]) + 3
    np.testing.assert_array_equal(s, np.stack([want0, want1, want2]))


# ------------------------------------------------------------------------------------------------
# Residual add + RMSNorm.
# ------------------------------------------------------------------------------------------------
def _assert_correctly_rounded_norm(R, gamma, eps, N, act):
    """Check N[h] = RNE(R[h] * g[h] / sqrt(ms + eps)) exactly: the real value y lies between the
    midpoints around N[h] (squared comparisons of rationals; ties are not reachable because y
    is irrational or the comparison is strict)."""
    H = len(R)
    ms = sum(frac(r) * frac(r) for r in R) / H + frac(np.float32(eps))
    vals, codes = grid(act)
    for h in range(H):
        a = frac(R[h]) * frac(gamma[h])          # y = a / sqrt(ms)
        n = frac(N[h])
        if a == 0:
            assert n == 0
            continue
        assert (n > 0) == (a > 0) or n == 0
        mag = abs(n)
        i = vals.index(mag)
        lo_mid = (vals[i - 1] + mag) / 2 if i > 0 else Fraction(0)
        hi_mid = (vals[i + 1] + mag) / 2
        # lo_mid <= |y| <= hi_mid  <=>  lo_mid^2 * ms <= a^2 <= hi_mid^2 * ms
        assert lo_mid * lo_mid * ms <= a * a <= hi_mid * hi_mid * ms, (h, float(N[h]))


@pytest.mark.parametrize("act", ["bf16", "fp16"])
def test_rmsnorm_correctly_rounded_bruteforce(act):
    inp = make_inputs(3, 24, 4, seed=21, act_dtype=act)
    rows, idx, sc, sh = _np(inp)
    res = inp.residual.double().numpy()
    gam = inp.gamma.double().numpy()
    s, R, N = O.finalize_rmsnorm(rows, idx, sc, sh, 2.5, res, gam, 1e-6, act)
    for t in range(3):
        # residual_out is the single rounding of the exact sum of two act-dtype values
        for h in range(24):
            assert frac(R[t, h]) == rne_exact(frac(s[t, h]) + frac(res[t, h]), act)
        _assert_correctly_rounded_norm(R[t], gam, 1e-6, N[t], act)


def test_rmsnorm_constant_row_closed_form():
    # A constant row c gives N = RNE(c * g / sqrt(c^2 + eps)) for every element.
    for c, g, eps in [(1.5, 1.0, 1e-6), (-0.375, 1.25, 1e-5), (3.0, 0.5, 0.0), (1.5 * 2.0 ** -10, 1.0, 1e-6)]:
        H = 64
        R, N = O.residual_rmsnorm(np.full((1, H), c), np.zeros((1, H)), np.full(H, g), eps, "bf16")
        assert np.all(R == c)
        y2_num = Fraction(c) ** 2 * Fraction(g) ** 2
        y2_den = Fraction(c) ** 2 + frac(np.float32(eps))
        n = frac(N[0, 0])
        vals, _ = grid("bf16")
        i = vals.index(abs(n))
        lo, hi = (vals[i - 1] + abs(n)) / 2, (vals[i + 1] + abs(n)) / 2
        assert lo * lo * y2_den <= y2_num <= hi * hi * y2_den
        assert np.all(N == N[0, 0]) and np.sign(N[0, 0]) == np.sign(c * g)


def test_rmsnorm_scale_invariance_eps0():
    # With eps = 0, RMSNorm(2^j * r) == RMSNorm(r) exactly.
    inp = make_inputs(4, 128, 2, seed=22)
    r = inp.residual.double().numpy()
    gam = inp.gamma.double().numpy()
    _, N0 = O.residual_rmsnorm(r, np.zeros_like(r), gam, 0.0, "bf16")
    for j in (-3, 1, 5):
        _, Nj = O.residual_rmsnorm(r * 2.0 ** j, np.zeros_like(r), gam, 0.0, "bf16")
        np.testing.assert_array_equal(Nj, N0)


# ------------------------------------------------------------------------------------------------
# The pages' printed accuracy numbers (worked example): TP4, BF16, top-8, RSF 2.5, eps 1e-5, bench
# distributions. Mean |error| of residual_out vs the FP64 reference: BF16 rounding floor ~4.8e-3
# (4.85e-3), FP32 accumulation rounded once 6.0e-3, per-step rounding 7.6e-3 to 8.0e-3.
# ------------------------------------------------------------------------------------------------
def tp4_errors(H, T, W=4, seed0=0):
    parts_new, parts_old, exact = [], [], 0.0
    for r in range(W):
        inp = make_inputs(T, H, 8, seed=seed0 + 1000 * r + T, scale_dtype="bf16",
                          n_rows=2 * T * 8 + 8, mask_frac=0.0, row_scale=0.5, shared_scale=0.5)
        rows, idx, sc, sh = _np(inp)
        exact = exact + O.finalize_unrounded(rows, idx, sc, sh, 2.5)
        parts_new.append(O.finalize(rows, idx, sc, sh, 2.5, "bf16"))
        parts_old.append(O.finalize_per_step_rounding(rows, idx, sc, sh, 2.5, "bf16"))
    g = torch.Generator().manual_seed(7 + T)
    residual = (torch.randn(T, H, generator=g) * 4).bfloat16().double().numpy()
    ref_res = exact + residual
    new = O.round_to_format(O.rank_sum_rounded(parts_new, "bf16") + residual, O.BF16)
    acc = np.zeros_like(residual)
    for p in parts_old:
        acc = O.round_to_format(acc + p, O.BF16)
    old = O.round_to_format(acc + residual, O.BF16)
    floor = np.abs(O.round_to_format(ref_res, O.BF16) - ref_res).mean()
    return floor, np.abs(new - ref_res).mean(), np.abs(old - ref_res).mean()


def _golden_ranges(name):
    """quantity -> (low, high) from a fixture under tests/golden/ (whitespace columns, # comments)."""
    out = {}
    with open(os.path.join(os.path.dirname(__file__), "golden", name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].split()
            if line:
                out[line[0]] = (float(line[1]), float(line[2]))
    return out


def test_pages_tp4_accuracy_figures():
    want = _golden_ranges("tp4_accuracy.txt")
    floor, new, old = tp4_errors(6144, 32)
    for name, got in (("bf16_rounding_floor", floor), ("fp32_accumulation_rounded_once", new),
                      ("per_step_rounding", old)):
        lo, hi = want[name]
        assert lo <= got <= hi, (name, got)


# ------------------------------------------------------------------------------------------------
# The unrounded reference (the accuracy reports' baseline) and the magnitude behind the float32
# window: pinned by exact rational brute force on tiny inputs.
@pytest.mark.parametrize("act,seed", [("bf16", 61), ("fp16", 62), ("bf16", 63)])
def test_reference_unrounded_and_magnitude_bruteforce(act, seed):
    """residual = RSF * sum of w * x over present routes + shared + residual, norm = residual *
    gamma / sqrt(mean(residual^2) + eps) with no rounding anywhere, and the magnitude |RSF| * sum
    |w * x| + |shared|, against Fractions (the square root taken last, in float64 of the exact
    radicand)."""
    T, H, K = 3, 16, 5
    inp = make_inputs(T, H, K, seed=seed, act_dtype=act, n_rows=T * K + 2)
    inp.idx[1, 2] = -1
    inp.idx[2, :] = -1                       # a token with no present route
    f = lambda t: t.double().numpy()  # noqa: E731
    rows, idx, sc, sh = f(inp.rows), inp.idx.numpy(), f(inp.scales), f(inp.shared)
    res, gam = f(inp.residual), f(inp.gamma)
    eps = float(np.float32(inp.eps))
    rsf = Fraction(inp.rsf)
    ref_res, ref_norm = O.reference_unrounded(rows, idx, sc, sh, inp.rsf, res, gam, inp.eps)
    mag = O.finalize_magnitude(rows, idx, sc, sh, inp.rsf)
    for t in range(T):
        acc = [Fraction(0)] * H
        mg = [Fraction(0)] * H
        for k in range(K):
            p = int(idx[t, k])
            if 0 <= p < rows.shape[0]:
                w = Fraction(float(sc[t, k]))
                for h in range(H):
                    term = w * Fraction(float(rows[p, h]))
                    acc[h] += term
                    mg[h] += abs(term)
        R = [rsf * acc[h] + Fraction(float(sh[t, h])) + Fraction(float(res[t, h])) for h in range(H)]
        M = [abs(rsf) * mg[h] + abs(Fraction(float(sh[t, h]))) for h in range(H)]
        ms = sum(r * r for r in R) / H
        root = math.sqrt(float(ms + Fraction(eps)))
        for h in range(H):
            assert ref_res[t, h] == pytest.approx(float(R[h]), rel=1e-13, abs=1e-300)
            want = float(R[h] * Fraction(float(gam[h]))) / root
            assert ref_norm[t, h] == pytest.approx(want, rel=1e-12, abs=1e-300)
            assert mag[t, h] == pytest.approx(float(M[h]), rel=1e-13, abs=1e-300)
    # the window's magnitude bounds the sum, with equality when every term is non-negative
    S = O.finalize_unrounded(rows, idx, sc, sh, inp.rsf)
    assert np.all(mag >= np.abs(S) * (1 - 1e-15))
    pos = make_inputs(2, 16, 4, seed=seed + 100, act_dtype=act)
    pr, ps, psh = np.abs(f(pos.rows)), np.abs(f(pos.scales)), np.abs(f(pos.shared))
    assert np.allclose(O.finalize_magnitude(pr, pos.idx.numpy(), ps, psh, 2.5),
                       O.finalize_unrounded(pr, pos.idx.numpy(), ps, psh, 2.5), rtol=1e-15, atol=0)
