"""Plain, slow FP64 CPU oracle of the MoE finalize path.

TEST INFRASTRUCTURE. Only `tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg of
`bench.py` may import or call this module. The HIP library never uses it and shares no code,
table or constant with it; the two meet only in the seeded input generators of `synth/`.

Sources (cited by key):
  [FI6631]  flashinfer PR #6631, "perf(comm): gather MoE-finalize routes together and accumulate
            in FP32": Description, test changes, benchmark script, review walkthrough.
  [TR16778] TensorRT-LLM PR #16778, "MoE: fp32 accumulation in deferred MoEAllReduce finalize":
            Description / Fix.
  [FI6546]  flashinfer PR #6546, small-batch trtllm-gen MoE finalize: Description, Performance.
  [FI3385]  flashinfer PR #3385, "feat: MNNVL Allreduce quant fusion and performance optimization":
            walkthrough (FP8/NVFP4 outputs, SF layouts), review comments.

What the path computes, for token t and hidden element h ([FI6631] Description and the FP64
reference of its benchmark script; [TR16778] Fix):
  p_k = expanded_idx_to_permuted_idx[t, k]; a route is valid iff 0 <= p_k < n_rows
  S*  = RSF * sum_{valid k} w[t,k] * X[p_k, h] + shared[t, h]          (real arithmetic)
  s   = RNE_T(S*)                       -- the one rounding of the finalized row
  R   = RNE_T(s + residual[t, h])       -- residual_out
  N   = RNE_T(R * gamma[h] / sqrt(mean_h(R^2) + eps))   -- norm_out
followed optionally by an NVFP4 or FP8 quantization of N ([FI3385] walkthrough; [FI6631] test
changes for the SWIZZLED_128x4 scale buffer).

Why FP64 gives the exact rounding decisions here:
  * every product w*x has at most 24 + 11 = 35 significant bits, so it is exact in FP64;
  * the sum of <= 66 such terms errs by at most ~66 * 2^-53 of the sum of magnitudes, far below
    the ~2^-9 relative half-ulp of bf16/fp16, so RNE_T of the FP64 value equals RNE_T of the real
    value except within ~2^-46 (relative) of a midpoint, which the tests' windows absorb;
  * every rounding to a narrow format goes straight from FP64 (never through float32, which would
    round twice);
  * quantization decisions compare x*gs (<= 35 bits, exact in FP64) with multiples of narrow
    values; an FP64 quotient then lands on the same side of every midpoint as the real quotient,
    because a real quotient that is not exactly a midpoint sits at least ~2^-35 (relative) away
    from it, while the FP64 division errs by at most 2^-53.

Readings of points the pages leave open:
  R1  route validity: any index outside [0, n_rows) is an absent route; neither its row nor its
      scale is read ([FI6631] test changes: -1 routes; walkthrough: one bound check per route).
  R2  missing scales mean weight 1.0, missing shared output means 0, RSF 1.0 means "off"
      ([FI6631] review summary: missing expert scales; commit notes: the factor is 1.0 when off).
  R3  RMSNorm reads the rounded residual_out; eps is the float32 value widened to FP64.
  R4  NVFP4: 16-element blocks, block scale sf = E4M3(gs * amax / 6), codes q = E2M1(x * gs / sf),
      all with round-to-nearest-even and saturation; even element in the low nibble; scale bytes
      in the SWIZZLED_128x4 layout with zero padding. FP8: q = E4M3(x * s8), saturating.
  R5  signed zero: values compare +0 == -0; quantized codes keep the sign bit of the input.
  R7  non-finite values: an infinity saturates like any value above the largest finite code; a
      NaN encodes as the E4M3 NaN code 0x7F (sign clear); a NaN in an NVFP4 block makes its
      amax NaN, so the block scale byte is 0x7F and its codes are 0 (E2M1 has no NaN).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

__all__ = [
    "Fmt", "BF16", "FP16", "E4M3", "E2M1", "FORMATS",
    "round_to_format", "encode_bits", "decode_bits",
    "finalize", "finalize_unrounded", "finalize_magnitude", "residual_rmsnorm",
    "finalize_rmsnorm", "reference_unrounded", "finalize_per_step_rounding",
    "rank_sum_rounded",
    "SF_LINEAR", "SF_SWIZZLED_128x4", "sf_size", "sf_offset",
    "quant_nvfp4", "quant_fp8", "nvfp4_global_scale", "fp8_scale",
    "dequant_nvfp4", "dequant_fp8",
]


# ----------------------------------------------------------------------------------------------
# Number formats and round-to-nearest-even straight from FP64.
# ----------------------------------------------------------------------------------------------
@dataclass(frozen=True)
class Fmt:
    """A binary floating-point format: `frac_bits` stored fraction bits, smallest normal exponent
    `emin`, largest finite magnitude `max_finite`; on overflow either IEEE infinity ('inf') or
    saturation to +-max_finite ('sat')."""
    name: str
    frac_bits: int
    emin: int
    max_finite: float
    overflow: str
    exp_bits: int
    bias: int


BF16 = Fmt("bf16", 7, -126, float((2 - 2.0 ** -7) * 2.0 ** 127), "inf", 8, 127)
FP16 = Fmt("fp16", 10, -14, 65504.0, "inf", 5, 15)
# OCP FP8 E4M3 ("fn": no infinities, only S.1111.111 is NaN, max 448), saturating conversion.
E4M3 = Fmt("e4m3", 3, -6, 448.0, "sat", 4, 7)
# OCP FP4 E2M1: magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}, no NaN/inf, saturating conversion.
E2M1 = Fmt("e2m1", 1, 0, 6.0, "sat", 2, 1)
FORMATS = {f.name: f for f in (BF16, FP16, E4M3, E2M1)}


def round_to_format(x, fmt: Fmt) -> np.ndarray:
    """Round FP64 values to the nearest value of `fmt`, ties to even, in one step.

    For |x| with leading-bit exponent e (clamped below at emin, which gives subnormals), the
    spacing of `fmt` is q = 2^(e - frac_bits); x/q is exact in FP64 (a power-of-two scale) and
    numpy's rint rounds it half-to-even exactly. Overflow follows `fmt.overflow`. NaN stays NaN;
    the sign of zero is kept."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, E = np.frexp(a)                      # a = m * 2^E, m in [0.5, 1)
    e = np.maximum(E - 1, fmt.emin)
    q = np.ldexp(1.0, e - fmt.frac_bits)
    with np.errstate(invalid="ignore"):
        r = np.rint(a / q) * q
    if fmt.overflow == "inf":
        r = np.where(r > fmt.max_finite, np.inf, r)
    else:
        r = np.where(r > fmt.max_finite, fmt.max_finite, r)
    r = np.where(np.isnan(x), np.nan, r)
    return np.copysign(r, x)


def _code_table(fmt: Fmt) -> np.ndarray:
    """Value of every non-negative code of a narrow format (NaN where the code is NaN)."""
    n_codes = 1 << (fmt.exp_bits + fmt.frac_bits)
    vals = np.empty(n_codes, dtype=np.float64)
    for c in range(n_codes):
        ex = c >> fmt.frac_bits
        man = c & ((1 << fmt.frac_bits) - 1)
        if ex == 0:
            v = man * 2.0 ** (1 - fmt.bias - fmt.frac_bits)
        else:
            v = (1.0 + man / 2.0 ** fmt.frac_bits) * 2.0 ** (ex - fmt.bias)
        vals[c] = v
    if fmt is E4M3:
        vals[n_codes - 1] = np.nan          # S.1111.111 is the only NaN of E4M3 "fn"
    return vals


_TABLES = {f.name: _code_table(f) for f in (E4M3, E2M1)}


def encode_bits(v, fmt: Fmt) -> np.ndarray:
    """Bit pattern of values that are already exactly representable in `fmt` (ValueError
    otherwise). A narrow format's non-NaN codes 0, 1, 2, ... have strictly increasing values, so
    the code of |v| is its position in that table; the sign adds the top bit. NaN encodes as the
    E4M3 NaN S.1111.111 without a sign (E2M1 has no NaN; 0 is returned)."""
    v = np.asarray(v, dtype=np.float64)
    if fmt is BF16:
        return (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    if fmt is FP16:
        return v.astype(np.float16).view(np.uint16)
    table = _TABLES[fmt.name]
    finite = table[~np.isnan(table)]
    sign_bit = 1 << (fmt.exp_bits + fmt.frac_bits)
    nan = np.isnan(v)
    a = np.where(nan, 0.0, np.abs(v))
    c = np.minimum(np.searchsorted(finite, a), finite.size - 1)
    if not np.array_equal(finite[c], a):
        raise ValueError(f"value not representable in {fmt.name}")
    out = c | np.where(np.signbit(v), sign_bit, 0)
    out = np.where(nan, sign_bit - 1 if fmt is E4M3 else 0, out)
    return out.astype(np.uint8)


def decode_bits(bits, fmt: Fmt) -> np.ndarray:
    """Values of bit patterns of `fmt` (float64)."""
    bits = np.asarray(bits)
    if fmt is BF16:
        with np.errstate(invalid="ignore"):      # signalling-NaN patterns widen to NaN
            return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if fmt is FP16:
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    table = _TABLES[fmt.name]
    nbits = fmt.exp_bits + fmt.frac_bits
    mag = table[bits.astype(np.int64) & ((1 << nbits) - 1)]
    neg = (bits.astype(np.int64) >> nbits) & 1
    return np.where(neg == 1, -mag, mag)


def _act(act_dtype: str) -> Fmt:
    return {"bf16": BF16, "fp16": FP16}[act_dtype]


# ----------------------------------------------------------------------------------------------
# Finalize: gather, weighted sum, routed scaling, shared add, one rounding.
# ----------------------------------------------------------------------------------------------
def _valid_routes(idx: np.ndarray, n_rows: int) -> np.ndarray:
    """Reading R1: a route is present iff its permuted index lies in [0, n_rows)."""
    idx = np.asarray(idx, dtype=np.int64)
    return (idx >= 0) & (idx < n_rows)


def finalize_unrounded(rows, idx, scales, shared, rsf) -> np.ndarray:
    """S*[t,h] = RSF * sum over valid k of w[t,k] * X[p[t,k], h] + shared[t,h], in FP64.

    [FI6631] Description (routed sum, routed_scaling_factor and shared add kept wide, rounded
    once) and its benchmark script's FP64 reference (gather by index, times weight, sum over k,
    times RSF, plus shared); [TR16778] Fix (top-k sum and shared add in a wide accumulator).
    `rows` [n_rows, H], `idx` [T, K], `scales` [T, K] or None (reading R2: weight 1.0),
    `shared` [T, H] or None (reading R2: 0). Absent routes are skipped entirely (reading R1), so
    NaN in an unreferenced row or in an absent route's scale never reaches the result."""
    rows = np.asarray(rows, dtype=np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    T, K = idx.shape
    n_rows, H = rows.shape
    valid = _valid_routes(idx, n_rows)
    acc = np.zeros((T, H), dtype=np.float64)
    for t in range(T):
        for k in range(K):
            if not valid[t, k]:
                continue
            w = 1.0 if scales is None else float(scales[t, k])
            acc[t] += w * rows[idx[t, k]]
    out = float(rsf) * acc
    if shared is not None:
        out = out + np.asarray(shared, dtype=np.float64)
    return out


def finalize(rows, idx, scales, shared, rsf, act_dtype: str) -> np.ndarray:
    """moe_finalize_run's result: s = RNE_T(S*), the one rounding of the finalized row
    ([FI6631] Description; [TR16778] Fix: rounded to the activation dtype once)."""
    return round_to_format(finalize_unrounded(rows, idx, scales, shared, rsf), _act(act_dtype))


def finalize_magnitude(rows, idx, scales, shared, rsf) -> np.ndarray:
    """|RSF| * sum over valid k of |w * x| + |shared|: the magnitude that bounds the rounding
    error of any float32 evaluation order of S* (used by the tests' admissible windows)."""
    rows = np.asarray(rows, dtype=np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    T, K = idx.shape
    valid = _valid_routes(idx, rows.shape[0])
    mag = np.zeros((T, rows.shape[1]), dtype=np.float64)
    for t in range(T):
        for k in range(K):
            if valid[t, k]:
                w = 1.0 if scales is None else float(scales[t, k])
                mag[t] += np.abs(w * rows[idx[t, k]])
    mag *= abs(float(rsf))
    if shared is not None:
        mag += np.abs(np.asarray(shared, dtype=np.float64))
    return mag


def residual_rmsnorm(s, residual, gamma, eps, act_dtype: str):
    """residual_out R = RNE_T(s + residual) and norm_out N = RNE_T(R * gamma / sqrt(ms + eps)),
    ms = mean over the row of R^2 ([FI6631] Description: the residual add and RMSNorm work on the
    rounded sum; its benchmark script: mean over hidden, eps inside the root, then times the norm
    weight). Reading R3: the norm reads the rounded R; eps is widened from float32."""
    fmt = _act(act_dtype)
    s = np.asarray(s, dtype=np.float64)
    R = round_to_format(s + np.asarray(residual, dtype=np.float64), fmt)
    H = R.shape[-1]
    ms = np.sum(R * R, axis=-1, keepdims=True) / H
    eps64 = float(np.float32(eps))
    N = round_to_format(R * np.asarray(gamma, dtype=np.float64) / np.sqrt(ms + eps64), fmt)
    return R, N


def finalize_rmsnorm(rows, idx, scales, shared, rsf, residual, gamma, eps, act_dtype: str):
    """moe_finalize_rmsnorm_run's results (s, residual_out, norm_out), each rounded once."""
    s = finalize(rows, idx, scales, shared, rsf, act_dtype)
    R, N = residual_rmsnorm(s, residual, gamma, eps, act_dtype)
    return s, R, N


def reference_unrounded(rows, idx, scales, shared, rsf, residual, gamma, eps):
    """The benchmark script's FP64 reference with no rounding at all ([FI6631] benchmark script):
    residual = S* + residual, norm = residual * rsqrt(mean(residual^2) + eps) * gamma. Used only to
    report mean absolute errors the way the pages do; never as a pass/fail target."""
    ref_res = finalize_unrounded(rows, idx, scales, shared, rsf) + np.asarray(residual, np.float64)
    ms = np.mean(ref_res * ref_res, axis=-1, keepdims=True)
    ref_norm = ref_res / np.sqrt(ms + float(np.float32(eps))) * np.asarray(gamma, np.float64)
    return ref_res, ref_norm


def finalize_per_step_rounding(rows, idx, scales, shared, rsf, act_dtype: str) -> np.ndarray:
    """The numerics the pages replace, kept as a negative control: every multiply and add of the
    routed sum, the routed scaling and the shared add rounds to the activation dtype
    ([FI6631] Description: the old loop rounded after every step; test changes: the "Cake"
    reference keeps per-step rounding). Weights are first rounded to the activation dtype."""
    fmt = _act(act_dtype)
    rows = np.asarray(rows, dtype=np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    T, K = idx.shape
    valid = _valid_routes(idx, rows.shape[0])
    acc = np.zeros((T, rows.shape[1]), dtype=np.float64)
    for t in range(T):
        for k in range(K):
            if not valid[t, k]:
                continue
            w = 1.0 if scales is None else float(scales[t, k])
            w_t = float(round_to_format(w, fmt))
            term = round_to_format(w_t * rows[idx[t, k]], fmt)
            acc[t] = round_to_format(acc[t] + term, fmt)
    acc = round_to_format(acc * float(round_to_format(float(rsf), fmt)), fmt)
    if shared is not None:
        acc = round_to_format(acc + np.asarray(shared, np.float64), fmt)
    return acc


def rank_sum_rounded(partials, act_dtype: str) -> np.ndarray:
    """Sum of per-rank rounded partial rows, taken wide in rank order 0..W-1 and rounded once
    ([FI6631] Description: the rank sum stays in FP32 and is rounded once before the residual add;
    [FI3385] commit notes: ranks accumulate in 0..world_size-1 order). The HIP path is one GPU, so
    this serves only the oracle's pin against the pages' TP4 accuracy figures."""
    total = np.zeros_like(np.asarray(partials[0], dtype=np.float64))
    for p in partials:
        total = total + np.asarray(p, dtype=np.float64)
    return round_to_format(total, _act(act_dtype))


# ----------------------------------------------------------------------------------------------
# Quantized outputs: NVFP4 (16-element blocks, E4M3 block scales) and FP8 E4M3 per tensor.
# ----------------------------------------------------------------------------------------------
SF_LINEAR = 0
SF_SWIZZLED_128x4 = 1
NVFP4_BLOCK = 16


def _roundup(a: int, b: int) -> int:
    return (a + b - 1) // b * b


def sf_size(T: int, H: int, layout: int) -> int:
    """Bytes of the NVFP4 block-scale buffer. SWIZZLED_128x4 pads rows to a multiple of 128 and
    blocks per row to a multiple of 4 ([FI6631] test changes: the scale buffer must be sized for
    the swizzled layout, T*H/16 is too small); LINEAR is T*H/16 ([FI3385] review: LINEAR and
    SWIZZLED_128x4 are the accepted layouts)."""
    nb = H // NVFP4_BLOCK
    if layout == SF_SWIZZLED_128x4:
        return _roundup(T, 128) * _roundup(nb, 4)
    if layout == SF_LINEAR:
        return T * nb
    raise ValueError(f"unsupported scale layout {layout}")


def sf_offset(t: int, b: int, H: int, layout: int) -> int:
    """Byte offset of the scale of (row t, block b). SWIZZLED_128x4 tiles rows by 128 and blocks by
    4; a 512-byte tile holds row r = t % 128 at (r % 32) * 16 + (r // 32) * 4 and block b % 4 in
    the last position; tiles run along the blocks of a row tile first. This is the cuBLAS
    block-scaling-factor layout; the tests check it byte for byte against PyTorch's to_blocked."""
    nb = H // NVFP4_BLOCK
    if layout == SF_LINEAR:
        return t * nb + b
    n_col_tiles = _roundup(nb, 4) // 4
    r = t % 128
    tile = (t // 128) * n_col_tiles + b // 4
    return tile * 512 + (r % 32) * 16 + (r // 32) * 4 + (b % 4)


def nvfp4_global_scale(N) -> float:
    """Per-tensor global scale gs = 448 * 6 / amax(N) as float32 (so the largest block of the
    tensor gets block scale 448 and its largest element code 6)."""
    amax = float(np.max(np.abs(np.asarray(N, dtype=np.float64))))
    return float(np.float32(448.0 * 6.0 / amax))


def fp8_scale(N) -> float:
    """Per-tensor FP8 scale s8 = 448 / amax(N) as float32 (reading R4)."""
    amax = float(np.max(np.abs(np.asarray(N, dtype=np.float64))))
    return float(np.float32(448.0 / amax))


def quant_nvfp4(N, gs: float, layout: int = SF_SWIZZLED_128x4):
    """NVFP4 of N [T, H] with float32 global scale gs (reading R4).

    For each row t and 16-element block b: amax = max |N|, sf = E4M3(gs * amax / 6); codes
    q = E2M1(N * gs / sf), or signed zeros when sf == 0. Two codes per byte, even element in the
    low nibble. Returns (codes uint8 [T, H/2], scale bytes uint8 [sf_size]); padding bytes are 0."""
    N = np.asarray(N, dtype=np.float64)
    T, H = N.shape
    if H % NVFP4_BLOCK:
        raise ValueError("H must be a multiple of 16 for NVFP4")
    gs = float(np.float32(gs))
    nb = H // NVFP4_BLOCK
    blocks = N.reshape(T, nb, NVFP4_BLOCK)
    amax = np.max(np.abs(blocks), axis=-1)                     # [T, nb]; NaN if the block has one
    sf = round_to_format(gs * amax / 6.0, E4M3)
    t_i, b_i = np.meshgrid(np.arange(T), np.arange(nb), indexing="ij")
    sf_bytes = np.zeros(sf_size(T, H, layout), dtype=np.uint8)
    sf_bytes[sf_offset(t_i, b_i, H, layout)] = encode_bits(sf, E4M3)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = round_to_format(blocks * gs / sf[..., None], E2M1)
    # a zero block scale gives signed zero codes
    q = np.where((sf == 0.0)[..., None], np.copysign(np.zeros_like(blocks), blocks), q)
    codes4 = encode_bits(q, E2M1).reshape(T, H)
    packed = (codes4[:, 0::2] | (codes4[:, 1::2] << 4)).astype(np.uint8)
    return packed, sf_bytes


def dequant_nvfp4(packed, sf_bytes, gs: float, T: int, H: int, layout: int = SF_SWIZZLED_128x4):
    """Inverse map: x ~= q * sf / gs (used only to check error bounds)."""
    packed = np.asarray(packed, dtype=np.uint8)
    codes4 = np.empty((T, H), dtype=np.uint8)
    codes4[:, 0::2] = packed & 0xF
    codes4[:, 1::2] = packed >> 4
    q = decode_bits(codes4, E2M1)
    out = np.empty((T, H), dtype=np.float64)
    for t in range(T):
        for b in range(H // NVFP4_BLOCK):
            sf = float(decode_bits(np.uint8(sf_bytes[sf_offset(t, b, H, layout)]), E4M3))
            sl = slice(b * NVFP4_BLOCK, (b + 1) * NVFP4_BLOCK)
            out[t, sl] = q[t, sl] * sf / float(np.float32(gs))
    return out


def quant_fp8(N, s8: float) -> np.ndarray:
    """FP8 E4M3 codes of N [T, H]: E4M3(N * s8), saturating at 448 (reading R4)."""
    N = np.asarray(N, dtype=np.float64)
    return encode_bits(round_to_format(N * float(np.float32(s8)), E4M3), E4M3)


def dequant_fp8(codes, s8: float) -> np.ndarray:
    return decode_bits(codes, E4M3) / float(np.float32(s8))
