"""CPU check of the arithmetic behind the device's narrow-format encoders (no GPU, no HIP).

The kernels quantize with the gfx950 conversion instructions (v_cvt_scalef32_pk_fp4_f32,
v_cvt_pk_fp8_f32), which round their float32 input to nearest even. The exact result the pages
define rounds the exact real product or quotient instead, so the kernels add steps that make the
two agree: a bracket of two conversions, an exact FMA sign against the midpoint between them and
a nudged third conversion (E2M1 codes, E4M3 block scales), and a round-to-odd float32 product
(FP8 codes). Here those steps are replayed in numpy float32 arithmetic, with the conversions
modelled as probed on the device (round to nearest even on the float32 value, saturation at 6
for E2M1, NaN from 464 up for E4M3), and compared with exact rounding over every bf16 / fp16
value of the ranges that matter, for many scales. The negative controls show the sweeps reach
the cases the extra steps exist for: without them, codes differ.

Only the kernels' arithmetic is emulated here; the GPU parity tests check the kernels' outputs.
"""
from __future__ import annotations

import numpy as np
import pytest

f32, f64 = np.float32, np.float64

E2M1_GRID = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
E2M1_MIDS = (E2M1_GRID[:-1] + E2M1_GRID[1:]) / 2
E4M3_GRID = np.array([m * 2.0 ** -9 if e == 0 else (8 + m) * 2.0 ** (e - 10)
                      for e in range(16) for m in range(8)][:127])
E4M3_MIDS = (E4M3_GRID[:-1] + E4M3_GRID[1:]) / 2


# ---- exact references: decisions on exact float64 products against exact midpoints ----------
def _count_above(p, mids_scaled):
    """Round-to-nearest-even code of p on a grid whose scaled midpoints are mids_scaled (codes
    of even index are the even ones: a tie at midpoint i goes up when i is odd)."""
    c = np.zeros(np.shape(p), np.int64)
    for i, t in enumerate(mids_scaled):
        c += (p > t) | ((p == t) & (i % 2 == 1))
    return c


def exact_e2m1(a, gs, sf):
    """E2M1 magnitude code of a*gs/sf: a*gs and m*sf are exact in float64."""
    return _count_above(a.astype(f64) * f64(gs), E2M1_MIDS * f64(sf))


def exact_e4m3_scale(amax, gs):
    """E4M3 code of amax*gs/6, saturating at 448: compare amax*gs with 6*midpoint."""
    return _count_above(amax.astype(f64) * f64(gs), 6.0 * E4M3_MIDS)


def exact_e4m3(a, s8):
    return _count_above(a.astype(f64) * f64(s8), E4M3_MIDS)


# ---- the device conversions and FMA, as float32 operations ------------------------------------
def hw_e2m1(y):
    """v_cvt_scalef32_pk_fp4_f32 with scale 1: nearest even on the float32 value, saturating."""
    return _count_above(np.abs(np.asarray(y, f64)), E2M1_MIDS)


def hw_e4m3(y):
    """v_cvt_pk_fp8_f32 on a nonnegative float32 value: nearest even; NaN code from 464 up."""
    y = np.asarray(y, f64)
    return np.where(y >= 464.0, 0x7F, np.minimum(_count_above(y, E4M3_MIDS), 0x7E))


def fma32(a, b, c):
    """a*b + c rounded once to float32. The products here (at most 24 x 24 significant bits)
    are exact in float64; the float64 sum is exact wherever the result decides a code (the
    operands are then close), so the one float32 rounding is the FMA's."""
    return (np.asarray(a, f64) * np.asarray(b, f64) + np.asarray(c, f64)).astype(f32)


def rcp32(x, ulp_err):
    """v_rcp_f32: within one ulp of 1/x (both extremes are tried)."""
    r = (f32(1) / x).astype(f32)
    if ulp_err:
        r = np.nextafter(r, f32(np.inf) if ulp_err > 0 else f32(0)).astype(f32)
    return r


# ---- the three encoders' steps ------------------------------------------------------------------
def dev_e2m1(a, gs, sf, ulp_err=0, nudge=True):
    """e2m1_pack_exact on magnitudes a (returns codes and which elements were bracketed)."""
    a = a.astype(f32)
    gs, sf = f32(gs), f32(sf)
    r = rcp32(np.array([sf], f32), ulp_err)[0]
    q = f32(gs * r)
    c_lo = hw_e2m1(a * f32(q * f32(1 - 2 ** -19)))
    c_hi = hw_e2m1(a * f32(q * f32(1 + 2 ** -19)))
    if not nudge:
        return c_hi, c_lo != c_hi
    s2 = (E2M1_GRID[c_lo].astype(f32) + E2M1_GRID[c_hi].astype(f32)).astype(f32)
    d = fma32(a, np.full_like(a, gs), -(s2 * f32(f32(0.5) * sf)).astype(f32))
    bd = f32(f32(2.0 ** -22) * sf)
    dc = np.clip(d, -bd, bd).astype(f32)
    y2 = fma32(dc, np.full_like(dc, f32(f32(2.0 ** 17) * r)), s2)
    return hw_e2m1((y2 / f32(2)).astype(f32)), c_lo != c_hi


def dev_e4m3_scale(amax, gs, nudge=True):
    """e4m3_block_scale_exact."""
    amax = amax.astype(f32)
    gs = f32(gs)
    v = (amax * f32(gs * f32(1 / 6))).astype(f32)
    c_lo = hw_e4m3(np.minimum(v * f32(1 - 2 ** -19), f32(448)))
    c_hi = hw_e4m3(np.minimum(v * f32(1 + 2 ** -19), f32(448)))
    if not nudge:
        return c_hi, c_lo != c_hi
    s2 = (E4M3_GRID[c_lo].astype(f32) + E4M3_GRID[c_hi].astype(f32)).astype(f32)
    d = fma32(amax, np.full_like(amax, gs), (f32(-3) * s2).astype(f32))
    bd = (f32(2.0 ** -22) * s2).astype(f32)
    dc = np.clip(d, -bd, bd).astype(f32)
    y = (f32(0.5) * fma32(dc, np.full_like(dc, f32(2.0 ** 16)), s2)).astype(f32)
    return hw_e4m3(y), c_lo != c_hi


def dev_e4m3(a, s8, round_to_odd=True):
    """e4m3_pack8_exact on magnitudes a."""
    a = a.astype(f32)
    s8 = f32(s8)
    with np.errstate(over="ignore", invalid="ignore"):
        p = (a * s8).astype(f32)
        r = (a.astype(f64) * f64(s8) - p.astype(f64)).astype(f32)   # the exact FMA residual
    t = p
    if round_to_odd:
        rb = r.view(np.uint32).astype(np.int64)
        t = ((p.view(np.uint32).astype(np.int64) - (rb >> 31)) | np.minimum(rb, 1))
        t = t.astype(np.uint32).view(f32)
    return hw_e4m3(np.where(p > 448, f32(448), t))


# ---- sweeps ------------------------------------------------------------------------------------
def _bf16_between(lo, hi):
    a, b = (int(np.array([v], f32).view(np.uint32)[0] >> 16) for v in (lo, hi))
    return (np.arange(a, b + 1, dtype=np.uint32) << 16).view(f32)


def _fp16_between(lo, hi):
    a, b = (int(np.array([v], np.float16).view(np.uint16)[0]) for v in (lo, min(hi, 65504.0)))
    return np.arange(a, b + 1, dtype=np.uint16).view(np.float16).astype(f32)


def _act_between(lo, hi, act):
    return _bf16_between(lo, hi) if act == "bf16" else _fp16_between(lo, hi)


def _global_scales(rng, n):
    """Small integers, float32 quotients 2688 / amax (a tensor-wide maximum's global scale),
    and random float32 values."""
    out = []
    for i in range(n):
        kind = i % 3
        if kind == 0:
            out.append(f32(rng.choice([1.0, 3.0, 6.0, 100.0, 448.0, 0.75])))
        elif kind == 1:
            amax = (np.array([rng.uniform(0.1, 40)], f32).view(np.uint32) & 0xFFFF0000).view(f32)[0]
            out.append(f32(2688.0 / float(amax)))
        else:
            out.append(f32(rng.uniform(0.01, 5000)))
    return out


@pytest.mark.parametrize("act", ["bf16", "fp16"])
def test_e2m1_codes_match_exact_rounding(act):
    rng = np.random.default_rng(11 if act == "bf16" else 12)
    sfs = E4M3_GRID[1:]
    n = bad = bracketed = bad_without_nudge = 0
    for gs in _global_scales(rng, 30):
        for sf in rng.choice(sfs, 8, replace=False):
            top = 7.0 * float(sf) / float(gs)
            a = _act_between(top * 2 ** -6, top, act)
            want = exact_e2m1(a, gs, sf)
            for err in (-1, 0, 1):
                got, br = dev_e2m1(a, gs, sf, err)
                bad += int((got != want).sum())
            bracketed += int(br.sum())
            bad_without_nudge += int((dev_e2m1(a, gs, sf, nudge=False)[0] != want).sum())
            n += len(a)
    assert n > 100_000 and bracketed > 20
    assert bad == 0
    assert bad_without_nudge > 0        # the sweep reaches ties and near ties


@pytest.mark.parametrize("act", ["bf16", "fp16"])
def test_e4m3_block_scale_matches_exact_rounding(act):
    rng = np.random.default_rng(21 if act == "bf16" else 22)
    n = bracketed = bad_without_nudge = 0
    for gs in _global_scales(rng, 45):
        amax = _act_between(2.0 ** -12 * 6 / float(gs), 470 * 6 / float(gs), act)
        want = exact_e4m3_scale(amax, gs)
        got, br = dev_e4m3_scale(amax, gs)
        assert np.array_equal(got, want), gs
        bracketed += int(br.sum())
        bad_without_nudge += int((dev_e4m3_scale(amax, gs, nudge=False)[0] != want).sum())
        n += len(amax)
    inf = dev_e4m3_scale(np.array([np.inf], f32), f32(100.0))[0]
    assert list(inf) == [0x7E]                 # an infinite block maximum saturates
    assert n > 100_000 and bracketed > 20 and bad_without_nudge > 0


@pytest.mark.parametrize("act", ["bf16", "fp16"])
def test_fp8_codes_match_exact_rounding(act):
    rng = np.random.default_rng(31 if act == "bf16" else 32)
    n = bad_plain = 0
    for s8 in _global_scales(rng, 30):
        a = _act_between(2.0 ** -12 / float(s8), 500 / float(s8), act)
        assert np.array_equal(dev_e4m3(a, s8), exact_e4m3(a, s8)), s8
        n += len(a)
    # scales built so that x * s8 lies within a float32 rounding of an E4M3 midpoint
    for _ in range(400):
        x0 = _act_between(rng.uniform(1, 1.9), 2, act)[0]
        s8 = f32(float(E4M3_MIDS[rng.integers(16, 100)]) / float(x0))
        a = np.concatenate([np.array([x0 * 2.0 ** k for k in range(-6, 6)], f32),
                            _act_between(1, 2, act)[:400] * f32(2.0 ** rng.integers(-4, 4))])
        want = exact_e4m3(a, s8)
        assert np.array_equal(dev_e4m3(a, s8), want), s8
        bad_plain += int((dev_e4m3(a, s8, round_to_odd=False) != want).sum())
        n += len(a)
    big = dev_e4m3(np.array([np.inf, 3e38, 1e4], f32), f32(448.0))
    assert list(big) == [0x7E] * 3             # infinities and overflow saturate
    assert n > 100_000 and bad_plain > 0
