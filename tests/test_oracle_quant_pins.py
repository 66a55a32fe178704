"""Pins of the oracle's NVFP4 / FP8 quantization and scale-factor layout (CPU only)."""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from synth import make_inputs
from tests.exact_ref import frac, rne_exact


def _norm_out(T, H, seed, act="bf16"):
    inp = make_inputs(T, H, 8, seed=seed, act_dtype=act)
    rows = inp.rows.double().numpy()
    _, _, N = O.finalize_rmsnorm(rows, inp.idx.numpy(), inp.scales.double().numpy(),
                                 inp.shared.double().numpy(), 2.5, inp.residual.double().numpy(),
                                 inp.gamma.double().numpy(), 1e-6, act)
    return N


def _unpack(packed):
    lo = packed & 0xF
    hi = packed >> 4
    out = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2], out[:, 1::2] = lo, hi
    return out


@pytest.mark.parametrize("layout", [O.SF_SWIZZLED_128x4, O.SF_LINEAR])
def test_nvfp4_exact_bruteforce(layout):
    # Exact rationals: sf = RNE_e4m3(gs * amax / 6), q = RNE_e2m1(x * gs / sf), saturating.
    T, H = 3, 48
    N = _norm_out(T, H, seed=31)
    N[1, 5] = -N[1, 5]  # make sure both signs occur in a block
    gs = O.nvfp4_global_scale(N)
    packed, sfb = O.quant_nvfp4(N, gs, layout)
    codes = _unpack(packed)
    G = Fraction(float(np.float32(gs)))
    for t in range(T):
        for b in range(H // 16):
            blk = [frac(v) for v in N[t, 16 * b:16 * b + 16]]
            amax = max(abs(v) for v in blk)
            sf = rne_exact(G * amax / 6, "e4m3")
            got_sf = O.decode_bits(np.uint8(sfb[O.sf_offset(t, b, H, layout)]), O.E4M3)
            assert frac(got_sf) == sf
            for i, v in enumerate(blk):
                want = Fraction(0) if sf == 0 else rne_exact(v * G / sf, "e2m1")
                c = codes[t, 16 * b + i]
                assert frac(O.decode_bits(np.uint8(c), O.E2M1)) == want
                if want == 0:
                    assert (c >> 3) == (1 if v < 0 or (v == 0 and np.signbit(float(v))) else 0)


def test_nvfp4_tensor_amax_block_gets_scale_448_and_code_6():
    N = _norm_out(4, 256, seed=32)
    gs = O.nvfp4_global_scale(N)
    packed, sfb = O.quant_nvfp4(N, gs)
    t, h = np.unravel_index(np.argmax(np.abs(N)), N.shape)
    b = h // 16
    sf = O.decode_bits(np.uint8(sfb[O.sf_offset(t, b, 256, O.SF_SWIZZLED_128x4)]), O.E4M3)
    assert sf == 448.0
    q = O.decode_bits(_unpack(packed)[t, h], O.E2M1)
    assert abs(q) == 6.0 and np.sign(q) == np.sign(N[t, h])


E2M1_VALUES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_nvfp4_dequant_error_bound():
    # x * gs / sf lies between the midpoints around its code q (above 6 it saturates to 6).
    N = _norm_out(5, 512, seed=33)
    gs = O.nvfp4_global_scale(N)
    packed, sfb = O.quant_nvfp4(N, gs)
    codes = _unpack(packed)
    q = O.decode_bits(codes, O.E2M1)
    for t in range(5):
        for b in range(512 // 16):
            sf = float(O.decode_bits(np.uint8(sfb[O.sf_offset(t, b, 512, 1)]), O.E4M3))
            for i in range(16):
                x = N[t, 16 * b + i] * float(np.float32(gs)) / sf if sf else 0.0
                qq = abs(q[t, 16 * b + i])
                j = E2M1_VALUES.index(qq)
                lo = (E2M1_VALUES[j - 1] + qq) / 2 if j else 0.0
                hi = (E2M1_VALUES[j + 1] + qq) / 2 if qq < 6.0 else np.inf
                assert lo <= abs(x) <= hi


def test_sf_layout_size_bijection_padding():
    for T, H in [(1, 64), (5, 48), (130, 96), (64, 6144), (128, 7168)]:
        nb = H // 16
        size = O.sf_size(T, H, O.SF_SWIZZLED_128x4)
        assert size == ((T + 127) // 128 * 128) * ((nb + 3) // 4 * 4)
        offs = {O.sf_offset(t, b, H, O.SF_SWIZZLED_128x4) for t in range(T) for b in range(nb)}
        assert len(offs) == T * nb and min(offs) >= 0 and max(offs) < size
        if T % 128:
            # The lesson of the pages: a buffer of T*H/16 bytes is too small for this layout.
            assert size > T * H // 16
        lin = {O.sf_offset(t, b, H, O.SF_LINEAR) for t in range(T) for b in range(nb)}
        assert lin == set(range(O.sf_size(T, H, O.SF_LINEAR)))
    # Padding bytes of the swizzled buffer are zero.
    N = _norm_out(5, 48, seed=34)
    _, sfb = O.quant_nvfp4(N, O.nvfp4_global_scale(N))
    used = {O.sf_offset(t, b, 48, 1) for t in range(5) for b in range(3)}
    pad = [i for i in range(len(sfb)) if i not in used]
    assert len(pad) == len(sfb) - 15 and not np.any(sfb[pad])
    assert np.all(sfb[sorted(used)] != 0)


def test_sf_layout_tile_structure():
    # Within one 128-row x 4-block tile of 512 bytes, 4 consecutive blocks of a row are 4
    # consecutive bytes, and rows r, r+32, r+64, r+96 share one 16-byte line. Tiles of the same
    # row band follow each other along the blocks. (The pages name the layout but never print
    # it; test_sf_swizzled_map_matches_torch_to_blocked checks the map against PyTorch's.)
    H = 16 * 12
    for t in range(128):
        base = O.sf_offset(t, 0, H, 1)
        assert [O.sf_offset(t, b, H, 1) - base for b in range(4)] == [0, 1, 2, 3]
        assert O.sf_offset(t, 4, H, 1) == base + 512
        assert base // 16 == O.sf_offset(t % 32, 0, H, 1) // 16
    assert O.sf_offset(128, 0, H, 1) == 3 * 512


def test_fp8_exact_bruteforce_and_saturation():
    N = _norm_out(2, 64, seed=35)
    s8 = O.fp8_scale(N)
    codes = O.quant_fp8(N, s8)
    S = Fraction(float(np.float32(s8)))
    for t in range(2):
        for h in range(64):
            want = rne_exact(frac(N[t, h]) * S, "e4m3")
            assert frac(O.decode_bits(codes[t, h], O.E4M3)) == want
    # saturation, signed zero
    c = O.quant_fp8(np.array([[1000.0, -1000.0, -1e-30, 0.0]]), 1.0)
    assert list(c[0]) == [0x7E, 0xFE, 0x80, 0x00]
    # the tensor amax maps to 448
    assert np.max(np.abs(O.decode_bits(codes, O.E4M3))) == 448.0


def _bf16_values(lo, hi):
    """Every positive bf16 value in [lo, hi]."""
    a, b = (int(np.array([v], np.float32).view(np.uint32)[0] >> 16) for v in (lo, hi))
    return (np.arange(a, b + 1, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def test_fp8_exact_on_float32_near_ties():
    """Scales s8 = fl32(m / x0) put x0 * s8 within one float32 rounding of an E4M3 midpoint m
    without equalling it (and x0 * 2^k on m * 2^k): the codes must follow the exact product,
    which a rounding of the float32 product would get wrong on some of them."""
    mids = [(a + b) / 2 for a, b in zip(*(lambda g: (g[:-1], g[1:]))(O.decode_bits(
        np.arange(0x7F, dtype=np.uint8), O.E4M3)))]
    x0s = _bf16_values(1.0, 1.96875)
    n = 0
    for i, x0 in enumerate(x0s):
        m = mids[16 + (i * 13) % 80]
        s8 = float(np.float32(m / x0))
        xs = np.array([[x0 * 2.0 ** k for k in range(-5, 5)] + [-x0]])
        codes = O.quant_fp8(xs, s8)
        S = Fraction(s8)
        for j, v in enumerate(xs[0]):
            assert frac(O.decode_bits(codes[0, j], O.E4M3)) == rne_exact(frac(v) * S, "e4m3")
            n += 1
    assert n > 1000


def test_nvfp4_exact_on_float32_near_ties():
    """Global scales gs = fl32(m / x0) (block scale 1: block maximum 6 / gs) put x0 * gs / sf
    within one float32 rounding of each E2M1 midpoint m; codes and scales against exact
    rationals."""
    n = 0
    for i, x0 in enumerate(_bf16_values(1.0, 1.96875)[::2]):
        m = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0][i % 7]
        gs = float(np.float32(m / x0))
        amax = float(O.round_to_format(np.array([6.0 / gs]), O.BF16)[0])
        blk = np.zeros(16)
        blk[0], blk[1], blk[2], blk[3] = amax, x0, -x0, x0 / 2
        N = blk[None, :]
        packed, sfb = O.quant_nvfp4(N, gs, O.SF_LINEAR)
        codes = _unpack(packed)
        G = Fraction(float(np.float32(gs)))
        sf = rne_exact(G * frac(amax) / 6, "e4m3")
        assert frac(O.decode_bits(np.uint8(sfb[0]), O.E4M3)) == sf
        for j in range(16):
            want = Fraction(0) if sf == 0 else rne_exact(frac(N[0, j]) * G / sf, "e2m1")
            assert frac(O.decode_bits(np.uint8(codes[0, j]), O.E2M1)) == want
            n += 1
    assert n > 1000


def test_nvfp4_zero_block_scale_gives_signed_zeros():
    """A block whose gs * amax / 6 rounds to the E4M3 zero (below 2^-10) has scale byte 0 and,
    by the reading of the pages' formula, zero codes that keep each element's sign (-0 too)."""
    gs = 1.0
    blk = np.array([3e-3, -3e-3, 1e-3, -1e-3, 0.0, -0.0, 5e-4, -5e-4] * 2)
    assert float(np.max(np.abs(blk))) * gs / 6 < 2.0 ** -10
    N = np.stack([blk, -blk])
    packed, sfb = O.quant_nvfp4(N, gs, O.SF_LINEAR)
    assert not sfb.any()
    codes = _unpack(packed)
    want = np.signbit(N).astype(np.uint8) << 3
    assert np.array_equal(codes, want)


def test_nonfinite_inputs_follow_the_stated_reading():
    """Non-finite values (the pages are silent): infinities saturate like any value above the
    largest finite code; a NaN gives the E4M3 NaN code S.1111.111 with S = 0 whatever its sign;
    an NVFP4 block holding a NaN has a NaN amax, hence a NaN block scale (code 0x7F) and NaN
    ratios, which encode as E2M1 code 0 without sign. Finite blocks beside them are unaffected."""
    inf, nan = np.inf, np.nan
    fin = np.array([0.5, -1.5, 3.0, -0.25, 1.0, 2.0, -4.0, 0.75, 1.25, -0.5, 6.0, -3.0, 0.0, 1.75,
                    -2.5, 0.125])
    N = np.zeros((1, 64))
    N[0, :16] = fin
    N[0, 16:32] = fin
    N[0, 16] = inf
    N[0, 32:48] = fin
    N[0, 33] = -nan
    N[0, 48:64] = fin
    N[0, 63] = -inf
    gs = 1.0
    codes, sf = O.quant_nvfp4(N, gs, O.SF_LINEAR)
    c4 = _unpack(codes)[0]
    ref_codes, ref_sf = O.quant_nvfp4(fin[None, :], gs, O.SF_LINEAR)
    assert np.array_equal(c4[:16], _unpack(ref_codes)[0]) and sf[0] == ref_sf[0]
    assert sf[1] == 0x7E and c4[16] == 0x7              # +inf: scale 448, code +6
    assert sf[2] == 0x7F and not c4[32:48].any()        # NaN block: scale NaN, codes 0, no sign
    assert sf[3] == 0x7E and c4[63] == 0xF              # -inf: code -6
    q8 = O.quant_fp8(np.array([[inf, -inf, nan, -nan, 1.0, -0.0, 500.0, -500.0]]), 1.0)[0]
    assert list(q8) == [0x7E, 0xFE, 0x7F, 0x7F, 0x38, 0x80, 0x7E, 0xFE]


def _torch_to_blocked():
    """PyTorch's own producer of the 128x4 block-scaling-factor layout (`to_blocked` in
    torch/testing/_internal/common_quantized.py, with its `ceil_div`), an implementation
    independent of the oracle's. That module imports test utilities that are not installed
    here, so only these two functions are compiled from its source file."""
    import ast
    import os

    import torch
    path = os.path.join(os.path.dirname(torch.__file__), "testing", "_internal",
                        "common_quantized.py")
    if not os.path.exists(path):
        pytest.skip("torch's common_quantized.py is not in this torch build")
    tree = ast.parse(open(path).read())
    funcs = [n for n in tree.body if isinstance(n, ast.FunctionDef)
             and n.name in ("ceil_div", "to_blocked")]
    if len(funcs) != 2:
        pytest.skip("this torch build has no to_blocked")
    ns = {"torch": torch}
    exec(compile(ast.Module(body=funcs, type_ignores=[]), path, "exec"), ns)
    return ns["to_blocked"]


@pytest.mark.parametrize("TH", [(1, 64), (5, 48), (130, 96), (64, 6144), (128, 7168), (300, 2064),
                                (257, 16)])
def test_sf_swizzled_map_matches_torch_to_blocked(TH):
    """The oracle's SWIZZLED_128x4 byte map against an outside producer of the layout: scale
    (t, b) of a [T, H/16] scale matrix lands at the byte torch's to_blocked puts it, and every
    other byte of the padded buffer is padding (zero)."""
    import torch
    to_blocked = _torch_to_blocked()
    T, H = TH
    nb = H // 16
    ids = torch.arange(1, T * nb + 1, dtype=torch.int64).view(T, nb)   # a unique id per scale
    flat = to_blocked(ids).numpy()
    assert flat.size == O.sf_size(T, H, O.SF_SWIZZLED_128x4)
    offs = np.array([[O.sf_offset(t, b, H, O.SF_SWIZZLED_128x4) for b in range(nb)]
                     for t in range(T)])
    assert np.array_equal(flat[offs], ids.numpy())
    pad = np.ones(flat.size, bool)
    pad[offs.ravel()] = False
    assert not flat[pad].any()
