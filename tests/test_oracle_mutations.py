"""Planted mistakes in the oracle must each fail at least one pin (CPU only).

Each mutant replaces one oracle function with a plausible wrong version (a dropped term, a wrong
sign, an off-by-one route, a double rounding, a swapped nibble, a transposed layout ...) and runs
the pins that should catch it. The oracle itself is restored after every case.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import oracle.moe_finalize_ref as R
from tests import test_oracle_pins as P
from tests import test_oracle_quant_pins as Q

_orig = {name: getattr(R, name) for name in
         ("finalize_unrounded", "round_to_format", "residual_rmsnorm", "quant_nvfp4",
          "quant_fp8", "sf_offset", "reference_unrounded", "finalize_magnitude")}


def _fin_no_rsf(rows, idx, scales, shared, rsf):
    return _orig["finalize_unrounded"](rows, idx, scales, shared, 1.0)


def _fin_shared_sign(rows, idx, scales, shared, rsf):
    neg = None if shared is None else -np.asarray(shared, dtype=np.float64)
    return _orig["finalize_unrounded"](rows, idx, scales, neg, rsf)


def _fin_scale_shift(rows, idx, scales, shared, rsf):
    sc = None if scales is None else np.roll(np.asarray(scales, dtype=np.float64), 1, axis=1)
    return _orig["finalize_unrounded"](rows, idx, sc, shared, rsf)


def _fin_rsf_on_shared(rows, idx, scales, shared, rsf):
    out = _orig["finalize_unrounded"](rows, idx, scales, shared, rsf)
    return out if shared is None else out + (rsf - 1.0) * np.asarray(shared, dtype=np.float64)


def _round_via_f32(x, fmt):
    x = np.asarray(x, dtype=np.float64)
    if fmt.name in ("bf16", "fp16"):
        x = x.astype(np.float32).astype(np.float64)   # rounds twice
    return _orig["round_to_format"](x, fmt)


def _round_ties_away(x, fmt):
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, E = np.frexp(a)
    e = np.maximum(E - 1, fmt.emin)
    q = np.ldexp(1.0, e - fmt.frac_bits)
    r = np.floor(a / q + 0.5) * q
    r = np.where(r > fmt.max_finite, np.inf if fmt.overflow == "inf" else fmt.max_finite, r)
    return np.copysign(r, x)


def _rms_eps_outside(s, residual, gamma, eps, act):
    fmt = R.FORMATS[act]
    Rr = _orig["round_to_format"](np.asarray(s, np.float64) + np.asarray(residual, np.float64),
                                  fmt)
    ms = np.mean(Rr * Rr, axis=-1, keepdims=True)
    N = _orig["round_to_format"](Rr * np.asarray(gamma, np.float64) / (np.sqrt(ms) + eps), fmt)
    return Rr, N


def _rms_unrounded_input(s, residual, gamma, eps, act):
    fmt = R.FORMATS[act]
    raw = np.asarray(s, np.float64) + np.asarray(residual, np.float64)
    Rr = _orig["round_to_format"](raw, fmt)
    ms = np.sum(raw * raw, axis=-1, keepdims=True) / raw.shape[-1]
    N = _orig["round_to_format"](raw * np.asarray(gamma, np.float64) /
                                 np.sqrt(ms + float(np.float32(eps))), fmt)
    return Rr, N


def _nvfp4_nibbles_swapped(N, gs, layout=1):
    packed, sf = _orig["quant_nvfp4"](N, gs, layout)
    return ((packed >> 4) | (packed << 4)).astype(np.uint8), sf


def _nvfp4_with_scale(N, gs, layout, scale_of, code_divisor):
    """NVFP4 built from a (possibly wrong) block-scale rule: scale_of(gs * amax / 6) gives the
    stored E4M3 scale, code_divisor(stored, exact) the divisor of the codes."""
    N = np.asarray(N, dtype=np.float64)
    T, H = N.shape
    gs = float(np.float32(gs))
    blocks = N.reshape(T, H // 16, 16)
    exact = gs * np.max(np.abs(blocks), axis=-1) / 6.0
    sf = scale_of(exact)
    div = code_divisor(sf, exact)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = _orig["round_to_format"](blocks * gs / div[..., None], R.E2M1)
    q = np.where((sf == 0.0)[..., None], np.copysign(np.zeros_like(blocks), blocks), q)
    c = R.encode_bits(q, R.E2M1).reshape(T, H)
    packed = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    t_i, b_i = np.meshgrid(np.arange(T), np.arange(H // 16), indexing="ij")
    sfb = np.zeros(R.sf_size(T, H, layout), dtype=np.uint8)
    sfb[R.sf_offset(t_i, b_i, H, layout)] = R.encode_bits(sf, R.E4M3)
    return packed, sfb


def _nvfp4_codes_from_unrounded_scale(N, gs, layout=1):
    return _nvfp4_with_scale(N, gs, layout, lambda v: _orig["round_to_format"](v, R.E4M3),
                             lambda sf, v: v)


def _nvfp4_scale_truncated(N, gs, layout=1):
    def rz(v):                      # the largest E4M3 value not above v (round toward zero)
        g = R.decode_bits(np.arange(0x7F, dtype=np.uint8), R.E4M3)
        return g[np.searchsorted(g, np.minimum(v, 448.0), side="right") - 1]
    return _nvfp4_with_scale(N, gs, layout, rz, lambda sf, v: sf)


def _nvfp4_zero_scale_unsigned(N, gs, layout=1):
    packed, sfb = _orig["quant_nvfp4"](N, gs, layout)
    T, H = np.asarray(N).shape
    t_i, b_i = np.meshgrid(np.arange(T), np.arange(H // 16), indexing="ij")
    zero = (sfb[R.sf_offset(t_i, b_i, H, layout)] == 0)            # [T, nb]
    mask = np.repeat(zero, 8, axis=1)                                # 8 bytes per block
    return np.where(mask, packed & 0x77, packed).astype(np.uint8), sfb


def _fp8_without_saturation(N, s8):
    codes = _orig["quant_fp8"](N, s8)
    over = np.abs(np.asarray(N, np.float64) * float(np.float32(s8))) >= 464.0
    return np.where(over, 0x7F, codes).astype(np.uint8)


def _fp8_float32_product(N, s8):
    p = (np.asarray(N, np.float64).astype(np.float32) * np.float32(s8)).astype(np.float64)
    return _orig["quant_fp8"](p, 1.0)


def _sf_offset_transposed(t, b, H, layout):
    if layout == R.SF_LINEAR:
        return _orig["sf_offset"](t, b, H, layout)
    nb = H // 16
    n_col_tiles = (nb + 3) // 4
    r = t % 128
    tile = (t // 128) * n_col_tiles + b // 4
    return tile * 512 + (r // 32) * 16 + (r % 32) * 4 + (b % 4) if r < 32 else \
        tile * 512 + (r % 32) * 16 + (r // 32) * 4 + (b % 4)


def _sf_offset_rows_in_order(t, b, H, layout):
    # rows of a 128-row tile in plain order (4 bytes each) instead of the 32 x 4 interleave
    if layout == R.SF_LINEAR:
        return _orig["sf_offset"](t, b, H, layout)
    nb = H // 16
    n_col_tiles = (nb + 3) // 4
    tile = (t // 128) * n_col_tiles + b // 4
    return tile * 512 + (t % 128) * 4 + (b % 4)


def _ref_eps_outside(rows, idx, scales, shared, rsf, residual, gamma, eps):
    res, _ = _orig["reference_unrounded"](rows, idx, scales, shared, rsf, residual, gamma, eps)
    ms = np.mean(res * res, axis=-1, keepdims=True)
    return res, res / (np.sqrt(ms) + float(np.float32(eps))) * np.asarray(gamma, np.float64)


def _ref_sum_not_mean(rows, idx, scales, shared, rsf, residual, gamma, eps):
    res, _ = _orig["reference_unrounded"](rows, idx, scales, shared, rsf, residual, gamma, eps)
    ms = np.sum(res * res, axis=-1, keepdims=True)
    return res, res / np.sqrt(ms + float(np.float32(eps))) * np.asarray(gamma, np.float64)


def _ref_no_residual(rows, idx, scales, shared, rsf, residual, gamma, eps):
    return _orig["reference_unrounded"](rows, idx, scales, shared, rsf, np.zeros_like(residual),
                                        gamma, eps)


def _mag_signed_shared(rows, idx, scales, shared, rsf):
    out = _orig["finalize_magnitude"](rows, idx, scales, None, rsf)
    return out if shared is None else out + np.asarray(shared, dtype=np.float64)


MUTANTS = [
    ("finalize_unrounded", _fin_no_rsf, [P.test_finalize_exact_bruteforce,
                                         P.test_dyadic_fixture_closed_form]),
    ("finalize_unrounded", _fin_shared_sign, [P.test_finalize_exact_bruteforce]),
    ("finalize_unrounded", _fin_scale_shift, [P.test_finalize_exact_bruteforce,
                                              P.test_route_order_invariance]),
    ("finalize_unrounded", _fin_rsf_on_shared, [P.test_dyadic_fixture_closed_form]),
    ("round_to_format", _round_via_f32, [P.test_round_matches_exact_bruteforce]),
    ("round_to_format", _round_ties_away, [P.test_round_matches_exact_bruteforce]),
    ("residual_rmsnorm", _rms_eps_outside, [P.test_rmsnorm_correctly_rounded_bruteforce,
                                             P.test_rmsnorm_constant_row_closed_form]),
    ("residual_rmsnorm", _rms_unrounded_input, [P.test_rmsnorm_correctly_rounded_bruteforce]),
    ("quant_nvfp4", _nvfp4_nibbles_swapped, [Q.test_nvfp4_exact_bruteforce]),
    ("quant_nvfp4", _nvfp4_codes_from_unrounded_scale, [Q.test_nvfp4_exact_bruteforce,
                                                        Q.test_nvfp4_exact_on_float32_near_ties]),
    ("quant_nvfp4", _nvfp4_scale_truncated, [Q.test_nvfp4_exact_bruteforce]),
    ("quant_nvfp4", _nvfp4_zero_scale_unsigned, [Q.test_nvfp4_zero_block_scale_gives_signed_zeros]),
    ("quant_fp8", _fp8_without_saturation, [Q.test_fp8_exact_bruteforce_and_saturation]),
    ("quant_fp8", _fp8_float32_product, [Q.test_fp8_exact_on_float32_near_ties]),
    ("sf_offset", _sf_offset_transposed, [Q.test_sf_layout_tile_structure]),
    ("sf_offset", _sf_offset_rows_in_order, [Q.test_sf_swizzled_map_matches_torch_to_blocked]),
    ("reference_unrounded", _ref_eps_outside, [P.test_reference_unrounded_and_magnitude_bruteforce]),
    ("reference_unrounded", _ref_sum_not_mean, [P.test_reference_unrounded_and_magnitude_bruteforce]),
    ("reference_unrounded", _ref_no_residual, [P.test_reference_unrounded_and_magnitude_bruteforce]),
    ("finalize_magnitude", _mag_signed_shared, [P.test_reference_unrounded_and_magnitude_bruteforce]),
]

_ARGS = {
    P.test_finalize_exact_bruteforce: [("bf16", 6), ("fp16", 3)],
    P.test_round_matches_exact_bruteforce: [("bf16",), ("fp16",)],
    P.test_rmsnorm_correctly_rounded_bruteforce: [("bf16",)],
    Q.test_nvfp4_exact_bruteforce: [(R.SF_SWIZZLED_128x4,)],
    Q.test_sf_swizzled_map_matches_torch_to_blocked: [((130, 96),), ((300, 2064),)],
    P.test_reference_unrounded_and_magnitude_bruteforce: [("bf16", 61), ("fp16", 62)],
}


@pytest.mark.parametrize("target,mutant,pins", MUTANTS,
                         ids=[m[1].__name__ for m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, target, mutant, pins):
    monkeypatch.setattr(R, target, mutant)
    monkeypatch.setattr(oracle, target, mutant)
    caught = False
    for pin in pins:
        for args in _ARGS.get(pin, [()]):
            try:
                pin(*args)
            except AssertionError:
                caught = True
    assert caught, f"no pin caught the mutant {mutant.__name__}"
