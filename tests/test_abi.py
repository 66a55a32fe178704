"""The C ABI on the CPU: the library loads, exports every symbol include/moe_finalize.h declares,
and rejects bad arguments with the documented codes before touching the GPU (no launches here;
every call below fails its host-side checks or is the T = 0 no-op)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import moe_expert_output_amd as M
import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_finalize.h")
LIB = M.LIB


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(moe_\w+)\s*\(", src, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert set(names) == set(M.EXPORTED), names
    for n in names:
        assert hasattr(LIB, n), n


def _header_consts():
    return {k: int(v) for k, v in re.findall(r"#define (MOE_\w+) \(?(-?\d+)\)?", open(HEADER).read())}


def test_binding_constants_match_header():
    c = _header_consts()
    assert c["MOE_DTYPE_BF16"] == M.MOE_DTYPE_BF16 and c["MOE_DTYPE_FP16"] == M.MOE_DTYPE_FP16
    assert c["MOE_QUANT_NVFP4"] == M.MOE_QUANT_NVFP4
    assert c["MOE_QUANT_FP8_E4M3"] == M.MOE_QUANT_FP8_E4M3
    assert c["MOE_SF_SWIZZLED_128x4"] == M.MOE_SF_SWIZZLED_128x4
    assert c["MOE_SF_LINEAR"] == M.MOE_SF_LINEAR
    assert c["MOE_FIN_LAUNCH_CONFIG_FIELDS"] == len(M.LAUNCH_CONFIG_FIELDS)
    assert (c["MOE_FIN_CACHE_AUTO"], c["MOE_FIN_CACHE_KEEP"], c["MOE_FIN_CACHE_STREAM"]) == (
        M.MOE_FIN_CACHE_AUTO, M.MOE_FIN_CACHE_KEEP, M.MOE_FIN_CACHE_STREAM)


def test_error_strings():
    for name, code in _header_consts().items():
        if name.startswith("MOE_FIN_ERR"):
            s = M.moe_finalize_error_string(code)
            assert s and s != "unknown error code", name
    assert M.moe_finalize_error_string(12345) == "unknown error code"


@pytest.mark.parametrize("T,H", [(1, 64), (5, 48), (64, 6144), (128, 7168), (130, 96), (0, 64)])
def test_sf_size_matches_oracle(T, H):
    for layout in (M.MOE_SF_LINEAR, M.MOE_SF_SWIZZLED_128x4):
        assert M.moe_finalize_sf_size(T, H, layout) == O.sf_size(T, H, layout)
    assert M.moe_finalize_sf_size(T, H, 7) == 0


# fake, never-dereferenced device addresses
A = 0x7F0000000000
B = 0x7F0010000000
C = 0x7F0020000000
D = 0x7F0030000000
E = 0x7F0040000000


def fin(rows=A, n_rows=64, idx=B, scales=C, sdt=2, shared=None, rsf=2.5, out=D, T=4, H=1024,
        K=8, act=0):
    return LIB.moe_finalize_run(rows, n_rows, idx, scales, sdt, shared, rsf, out, T, H, K, act,
                                None)


WS = 0x7F0050000000


def rms(rows=A, n_rows=64, idx=B, scales=C, sdt=2, shared=None, residual=E, gamma=E + 0x100000,
        eps=1e-6, res_out=E + 0x200000, norm_out=D, ws=None, ws_bytes=0, T=4, H=1024, K=8, act=0):
    return LIB.moe_finalize_rmsnorm_run(rows, n_rows, idx, scales, sdt, shared, 2.5, residual,
                                        gamma, eps, res_out, norm_out, ws, ws_bytes, T, H, K, act,
                                        None)


def quant(qt=1, qs=E + 0x300000, qo=E + 0x400000, so=E + 0x500000, layout=1, H=1024, T=4,
          norm_out=D, ws=None, ws_bytes=0):
    return LIB.moe_finalize_quant_run(A, 64, B, C, 2, None, 2.5, E, E + 0x100000, 1e-6, qt, qs,
                                      qo, so, layout, E + 0x200000, norm_out, ws, ws_bytes, T, H,
                                      8, 0, None)


def test_validation_codes():
    assert fin(K=0) == -3 and fin(K=65) == -3
    assert fin(act=5) == -6 and fin(sdt=9) == -6
    assert fin(H=1020) == -4 and fin(H=0) == -4
    assert fin(T=-1) == -2 and fin(n_rows=-1) == -2
    assert fin(T=0) == 0                       # no-op, nothing touched
    assert fin(T=0, idx=None, out=None) == 0
    assert fin(idx=None) == -1 and fin(out=None) == -1
    assert fin(rows=None) == -1
    assert fin(rows=A + 8) == -5 and fin(out=D + 2) == -5 and fin(idx=B + 2) == -5
    assert fin(scales=C + 2) == -5             # fp32 scales need 4-byte alignment
    assert fin(out=A + 4096) == -9             # output inside the permuted rows
    assert fin(out=B) == -9


def test_rmsnorm_validation_codes():
    assert rms(H=16392) == -4
    assert rms(residual=None) == -1 and rms(gamma=None) == -1 and rms(norm_out=None) == -1
    assert rms(res_out=E + 8) == -5
    assert rms(norm_out=E) == -9               # norm_out overlaps residual
    assert rms(res_out=D) == -9                # residual_out overlaps norm_out
    assert rms(T=0) == 0
    need = M.moe_finalize_workspace_size(4, 1024, 8)
    assert need == 256 + 4 * 128
    assert rms(ws=WS + 64, ws_bytes=need) == -5           # workspace must be 256-byte aligned
    assert rms(ws=WS, ws_bytes=need - 1) == -11           # too small
    assert rms(ws=E, ws_bytes=need) == -9                 # overlaps residual
    assert rms(ws=A + 256, ws_bytes=need) == -9           # overlaps the permuted rows
    assert quant(ws=WS, ws_bytes=16) == -11
    assert quant(ws=E + 0x400000, ws_bytes=need) == -9    # overlaps quant_out


def test_launch_floor_validation_codes():
    f = LIB.moe_finalize_launch_floor_run
    assert f(3, 4, 1024, 8, None) == -7 and f(-1, 4, 1024, 8, None) == -7
    assert f(1, 4, 1024, 0, None) == -3 and f(1, 4, 1020, 8, None) == -4
    assert f(1, 4, 16392, 8, None) == -4 and f(1, -1, 1024, 8, None) == -2
    assert f(1, 0, 1024, 8, None) == 0


def test_stream_floor_validation_codes():
    f = LIB.moe_finalize_stream_floor_run
    S, Dst = A, E
    assert f(S, 1000, Dst, 1024, None) == -2 and f(S, 1024, Dst, 24, None) == -2
    assert f(S, (1 << 31) + 16, Dst, 0, None) == -2
    assert f(None, 1024, Dst, 0, None) == -1 and f(S, 0, None, 1024, None) == -1
    assert f(S + 8, 1024, Dst, 1024, None) == -5 and f(S, 1024, Dst + 4, 1024, None) == -5
    assert f(S, 4096, S + 1024, 1024, None) == -9
    assert f(None, 0, None, 0, None) == 0


def test_quant_validation_codes():
    assert quant(qt=0) == -7 and quant(qt=3) == -7
    assert quant(layout=2) == -8               # SWIZZLED_8x4 is not accepted
    assert quant(H=1032) == -4                 # NVFP4 needs hidden % 16 == 0
    assert quant(qs=None) == -1 and quant(qo=None) == -1 and quant(so=None) == -1
    assert quant(qo=E + 0x400008) == -5
    assert quant(so=A) == -9
    assert quant(T=0) == 0


def test_quantize_validation_codes():
    q = LIB.moe_quantize_run
    X, QS, QO, SO = A, E + 0x300000, E + 0x400000, E + 0x500000
    assert q(X, 4, 1024, 0, 3, QS, QO, SO, 1, None) == -7
    assert q(X, 4, 1024, 0, 1, QS, QO, SO, 2, None) == -8
    assert q(X, 4, 1024, 9, 1, QS, QO, SO, 1, None) == -6
    assert q(X, 4, 1032, 0, 1, QS, QO, SO, 1, None) == -4      # NVFP4 needs hidden % 16 == 0
    assert q(X, 4, 1020, 0, 2, QS, QO, None, 0, None) == -4    # FP8 needs hidden % 8 == 0
    assert q(X, -1, 1024, 0, 1, QS, QO, SO, 1, None) == -2
    assert q(X, 0, 1024, 0, 1, None, None, None, 1, None) == 0
    assert q(None, 4, 1024, 0, 1, QS, QO, SO, 1, None) == -1
    assert q(X, 4, 1024, 0, 1, QS, QO, None, 1, None) == -1
    assert q(X + 8, 4, 1024, 0, 1, QS, QO, SO, 1, None) == -5
    assert q(X, 4, 1024, 0, 1, QS, X + 1024, SO, 1, None) == -9


def test_residual_rmsnorm_validation_codes():
    f = LIB.moe_residual_rmsnorm_run
    X, R, G, RO, NO = A, E, E + 0x100000, E + 0x200000, D

    def call(x=X, res=R, g=G, ro=RO, no=NO, ws=None, wb=0, T=4, H=1024, act=0):
        return f(x, res, g, 1e-6, ro, no, ws, wb, T, H, act, None)

    assert call(act=3) == -6
    assert call(H=1020) == -4 and call(H=16392) == -4 and call(H=0) == -4
    assert call(T=-1) == -2
    assert call(T=0) == 0 and call(T=0, x=None, res=None, g=None, no=None) == 0
    assert call(x=None) == -1 and call(res=None) == -1 and call(g=None) == -1
    assert call(no=None) == -1
    assert call(x=X + 8) == -5 and call(ro=RO + 8) == -5
    assert call(no=X) == -9 and call(ro=X + 4096) == -9      # outputs may not overlap x
    need = M.moe_finalize_workspace_size(4, 1024, 1)
    assert call(ws=WS + 64, wb=need) == -5
    assert call(ws=WS, wb=need - 1) == -11
    assert call(ws=X, wb=need) == -9


def test_rank_sum_validation_codes():
    f = LIB.moe_rank_sum_rmsnorm_run
    P_, R, G, RO, NO = A, E, E + 0x100000, E + 0x200000, D

    def call(p=P_, w=4, res=R, g=G, ro=RO, no=NO, ws=None, wb=0, T=4, H=1024, act=0):
        return f(p, w, res, g, 1e-6, ro, no, ws, wb, T, H, act, None)

    assert call(w=0) == -3 and call(w=65) == -3          # world size outside [1, 64]
    assert call(act=3) == -6
    assert call(H=1020) == -4 and call(H=16392) == -4
    assert call(T=-1) == -2 and call(T=1 << 26, w=64) == -2   # world_size * T > 2^31 - 1
    assert call(T=0) == 0 and call(T=0, p=None, res=None, g=None, no=None) == 0
    assert call(p=None) == -1 and call(no=None) == -1 and call(res=None) == -1
    assert call(p=P_ + 8) == -5 and call(ro=RO + 8) == -5
    assert call(no=P_ + 4 * 4 * 1024 * 2 - 64) == -9      # overlaps the last partial row
    need = M.moe_finalize_workspace_size(4, 1024, 4)
    assert call(ws=WS, wb=need - 1) == -11
    q = LIB.moe_rank_sum_quant_run
    QS, QO, SO = E + 0x300000, E + 0x400000, E + 0x500000

    def qcall(qt=1, layout=1, p=P_, w=4, so=SO, H=1024):
        return q(p, w, R, G, 1e-6, qt, QS, QO, so, layout, RO, None, None, 0, 4, H, 0, None)

    assert qcall(qt=0) == -7 and qcall(layout=2) == -8 and qcall(H=1032) == -4
    assert qcall(w=0) == -3 and qcall(p=None) == -1 and qcall(so=None) == -1


def test_launch_config_validation_codes():
    cfg = M.moe_finalize_launch_config
    for args, code in [((3, 4, 1024, 8), M.MoeFinalizeError), ((1, 4, 1024, 0), M.MoeFinalizeError),
                       ((1, 4, 1004, 8), M.MoeFinalizeError), ((1, 4, 16392, 8), M.MoeFinalizeError),
                       ((1, -1, 1024, 8), M.MoeFinalizeError)]:
        with pytest.raises(code):
            cfg(*args, num_cus=256)
    L = M.LIB
    out = (ctypes.c_int64 * 9)()
    assert L.moe_finalize_launch_config(1, 4, 1024, 8, 1, 256, None, 9) == -1
    assert L.moe_finalize_launch_config(1, 4, 1024, 8, 1, 256, out, 8) == -2
    assert L.moe_finalize_launch_config(3, 4, 1024, 8, 1, 256, out, 9) == -7
    assert L.moe_finalize_launch_config(1, 4, 1024, 65, 1, 256, out, 9) == -3
    assert L.moe_finalize_launch_config(1, 4, 16392, 8, 1, 256, out, 9) == -4
    assert L.moe_finalize_launch_config(0, 4, 16392, 8, 0, 256, out, 9) == 0   # finalize: any hidden
    assert cfg(1, 0, 7168, 8, num_cus=256)["workgroups"] == 0
    # the device's own count is only needed (and queried) for a split-row configuration
    assert L.moe_finalize_launch_config(0, 4, 1024, 8, 1, 0, out, 9) == 0
    assert L.moe_finalize_launch_config(1, 4, 1024, 8, 0, 0, out, 9) == 0


def test_slice_rule_follows_the_cu_count():
    """The slice rule scales with the device's compute units (injected here): at most one
    workgroup per CU up to top_k 8, about 7/8 of one above, within the hidden-size bounds."""
    cfg = M.moe_finalize_launch_config
    # hidden 7168, top_k 8, T = 64: min(896 / 128, CUs / 64) slices
    assert [cfg(1, 64, 7168, 8, num_cus=c)["slices"] for c in (64, 128, 256, 304, 512)] == \
        [1, 2, 4, 4, 7]
    # T = 128: two slices on 256 CUs, whole rows on 128
    assert cfg(1, 128, 7168, 8, num_cus=256)["slices"] == 2
    assert cfg(1, 128, 7168, 8, num_cus=128)["slices"] == 1
    # top_k 22, hidden 2048, T = 16: min(256 / 64, 7/8 CUs / 16)
    assert [cfg(1, 16, 2048, 22, num_cus=c)["slices"] for c in (32, 64, 256)] == [1, 3, 4]
    # the quantized entry splits by the same counts
    assert cfg(2, 64, 6144, 8, num_cus=128)["slices"] == 2


def test_launch_config_every_shape_has_a_kernel():
    """Host logic over a sweep of shapes (tokens 1..4096, hidden 8..16384, top_k 1..64, every
    entry kind, with and without a workspace): the chosen configuration has a compiled kernel, fits
    one workgroup (whole wavefronts, <= 1024 lanes, <= 64 KiB LDS), gives every route group work,
    covers each token's 8-element slots with non-empty slices, splits rows only within the slice
    rule's bounds for a device of C compute units (<= 16; up to top_k 8 <= hidden/1024 slices and
    <= C/T, above it <= hidden/512 and <= (7/8)C/T; whole rows for plain RMSNorm with top_k <= 4
    from T = 96 while a token's
    data stays within 128 KiB, and without a workspace), sizes whole-row
    workgroups by the slot rule (four-wavefront multiples from T = 1024 while a route group has at
    most 8 routes), and streams nontemporally exactly from 4 MiB of rows."""
    Ts = [1, 2, 3, 4, 7, 8, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 112, 127, 128, 129, 224, 225,
          256, 1000, 2048, 4096]
    Hs = [8, 16, 48, 512, 520, 1000, 1024, 1032, 2048, 3584, 4096, 4104, 6144, 7168, 8192, 8200,
          12288, 16376, 16384]
    Ks = [1, 2, 3, 4, 5, 6, 8, 10, 16, 17, 22, 31, 32, 33, 63, 64]
    n = 0
    for cus, entry, ws in [(256, e, w) for e in (0, 1, 2) for w in (False, True)] + \
            [(c, e, True) for c in (80, 304) for e in (1, 2)]:
        if True:
            for T in Ts:
                for H in Hs:
                    nv = H // 8
                    for K in Ks:
                        c = M.moe_finalize_launch_config(entry, T, H, K, ws, num_cus=cus)
                        n += 1
                        where = (entry, ws, T, H, K, c)
                        G, P, span = c["route_groups"], c["slots_per_lane"], c["slot_span"]
                        assert c["kernel_available"] == 1, where
                        assert c["lanes"] % 64 == 0 and 64 <= c["lanes"] <= 1024, where
                        assert G in (1, 2, 4) and c["lanes"] % (64 * G) == 0, where
                        assert G == 1 or G <= K, where               # every group has a route
                        lanes_per_group = c["lanes"] // G
                        assert P * lanes_per_group >= span, where
                        assert c["lds_bytes"] == (G - 1) * P * lanes_per_group * 32, where
                        assert c["lds_bytes"] <= 65536, where
                        assert c["nontemporal"] == int(T * K * H * 2 >= 4 << 20), where
                        if entry == 0:
                            assert span == 64 and P == 1, where
                            assert c["workgroups"] == T * -(-nv // 64), where
                            continue
                        S = c["slices"]
                        # split rows of cacheable calls: a token's slices share an XCD, tokens
                        # padded to a multiple of the 8 XCDs (idle workgroups)
                        xcd = S > 1 and not c["nontemporal"]
                        assert c["workgroups"] == (-(-T // 8) * 8 * S if xcd else T * S), where
                        bound = (min(nv // 64, cus * 7 // 8 // T, 16) if K > 8
                                 else min(nv // 128, cus // T))
                        if K <= 4 and T >= 96 and entry == 1 and (K + 2) * nv * 16 <= 128 << 10:
                            bound = 1
                        assert 1 <= S <= max(1, min(bound, 16)), where
                        if not ws:
                            assert S == 1, where
                        assert (S - 1) * span < nv <= S * span, where
                        assert S == 1 or span % 8 == 0, where
                        if S == 1:
                            # whole rows: one or two slots per lane, lanes rounded up to whole
                            # wavefronts, or from 1024 tokens to four wavefronts while a route
                            # group carries at most 8 routes
                            assert P == (1 if nv <= 1024 else 2), where
                            per_lane = -(-nv // P)
                            quad = T >= 1024 and -(-K // G) <= 8
                            r = 256 if quad else 64
                            assert lanes_per_group == -(-per_lane // r) * r, where
                            assert span == lanes_per_group * P, where
    assert n == (3 * 2 + 2 * 2) * len(Ts) * len(Hs) * len(Ks)


def test_cache_policy_setting():
    """The process-wide cache policy: returns the previous value, rejects unknown ones without
    changing anything, and decides the nontemporal choice every entry point reports."""
    L = M.LIB
    assert L.moe_finalize_set_cache_policy(M.MOE_FIN_CACHE_AUTO) == M.MOE_FIN_CACHE_AUTO
    try:
        big, small = (1, 128, 7168, 8), (1, 16, 6144, 8)
        assert M.moe_finalize_launch_config(*big, num_cus=256)["nontemporal"] == 1
        assert M.moe_finalize_launch_config(*small, num_cus=256)["nontemporal"] == 0
        assert M.moe_finalize_set_cache_policy(M.MOE_FIN_CACHE_KEEP) == M.MOE_FIN_CACHE_AUTO
        for e in (0, 1, 2):
            assert M.moe_finalize_launch_config(e, 128, 7168, 8, num_cus=256)["nontemporal"] == 0
        assert L.moe_finalize_set_cache_policy(3) == -12 and L.moe_finalize_set_cache_policy(-1) == -12
        with pytest.raises(M.MoeFinalizeError):
            M.moe_finalize_set_cache_policy(7)
        assert M.moe_finalize_set_cache_policy(M.MOE_FIN_CACHE_STREAM) == M.MOE_FIN_CACHE_KEEP
        for e in (0, 1, 2):
            assert M.moe_finalize_launch_config(e, 1, 1024, 1, num_cus=256)["nontemporal"] == 1
    finally:
        M.moe_finalize_set_cache_policy(M.MOE_FIN_CACHE_AUTO)
    assert M.moe_finalize_launch_config(*small, num_cus=256)["nontemporal"] == 0


def test_binding_rejects_mismatched_tensors():
    """The binding checks shapes and dtypes before any pointer reaches the C ABI (which sees no
    tensor extents): a tensor smaller than the call implies would be read or written past its
    end. CPU tensors of the right shapes get as far as the device check."""
    import torch
    T, H, K = 4, 64, 8
    bf = torch.bfloat16
    rows = torch.zeros(T * K, H, dtype=bf)
    idx = torch.zeros(T, K, dtype=torch.int32)
    sc = torch.zeros(T, K, dtype=torch.float32)
    res, gam = torch.zeros(T, H, dtype=bf), torch.zeros(H, dtype=bf)
    out = torch.zeros(T, H, dtype=bf)

    def fin(**kw):
        a = dict(rows=rows, idx=idx, sc=sc, sh=None, res=res, gam=gam, ro=None, no=out)
        a.update(kw)
        M.moe_finalize_rmsnorm_run(a["rows"], a["idx"], a["sc"], a["sh"], 2.5, a["res"], a["gam"],
                                   1e-6, a["ro"], a["no"])

    cases = [
        (dict(res=torch.zeros(T - 1, H, dtype=bf)), "residual must have shape"),
        (dict(gam=torch.zeros(H - 8, dtype=bf)), "gamma must have shape"),
        (dict(gam=torch.zeros(H, dtype=torch.float16)), "gamma must be"),
        (dict(idx=torch.zeros(T, K, dtype=torch.int64)), "must be torch.int32"),
        (dict(sc=torch.zeros(T, K - 1)), "expert_scales must have shape"),
        (dict(sc=torch.zeros(T, K, dtype=torch.float64)), "expert_scales must be"),
        (dict(sh=torch.zeros(T, H + 8, dtype=bf)), "shared_expert_output must have shape"),
        (dict(ro=torch.zeros(T, H, dtype=torch.float16)), "residual_out must be"),
        (dict(no=torch.zeros(T + 1, H, dtype=bf)), "norm_out must have shape"),
        (dict(rows=torch.zeros(T * K, H - 8, dtype=bf)), "permuted_rows must have shape"),
        (dict(rows=torch.zeros(T * K, H, dtype=torch.float32)), "is not bf16/fp16"),
        (dict(), "device (HIP) tensors"),            # shapes fine: stops at the device check
    ]
    for kw, msg in cases:
        with pytest.raises(ValueError, match=re.escape(msg)):
            fin(**kw)
    qs = torch.ones(1)
    for qo, so, msg in [(torch.zeros(T, H // 2 - 1, dtype=torch.uint8), torch.zeros(4096, dtype=torch.uint8),
                         "quant_out must hold exactly"),
                        (torch.zeros(T, H // 2, dtype=torch.uint8), torch.zeros(16, dtype=torch.uint8),
                         "scale_out must hold at least"),
                        (torch.zeros(T, H // 2, dtype=torch.uint8), None, "scale_out is required")]:
        with pytest.raises(ValueError, match=re.escape(msg)):
            M.moe_quantize_run(out, M.MOE_QUANT_NVFP4, qs, qo, so, M.MOE_SF_SWIZZLED_128x4)
    with pytest.raises(ValueError, match="quant_scale"):
        M.moe_quantize_run(out, M.MOE_QUANT_FP8_E4M3, torch.ones(1, dtype=torch.float64),
                           torch.zeros(T, H, dtype=torch.uint8), None, 0)
    with pytest.raises(ValueError, match=re.escape("rank_partials must be [world_size, T, H]")):
        M.moe_rank_sum_rmsnorm_run(torch.zeros(T, H, dtype=bf), res, gam, 1e-6, None, out)
    with pytest.raises(ValueError, match=re.escape("residual must have shape")):
        M.moe_rank_sum_rmsnorm_run(torch.zeros(2, T, H, dtype=bf), res[:2], gam, 1e-6, None, out)


def test_noalloc_entry_validation_codes():
    """The allocation-free entry point checks its shape (including the static scratch's limit of
    1024 tokens) before anything else; T = 0 is a no-op that needs no device."""
    f = LIB.moe_finalize_rmsnorm_noalloc_run

    def call(T=4, H=1024, K=8, rows=A, idx=B, no=D, act=0):
        return f(rows, T * K, idx, None, 2, None, 1.0, E, E + 0x200000, 1e-6, None, no, T, H, K, act,
                 None)

    assert call(T=1025) == -13 and call(T=1 << 20) == -13
    assert call(K=0) == -3 and call(H=1020) == -4 and call(H=16392) == -4 and call(act=5) == -6
    assert call(T=-1) == -2
    assert call(T=0) == 0
    assert M.moe_finalize_error_string(-13).startswith("num_tokens above")


def test_workspace_flag_validation_codes():
    """The flag query rejects a null result pointer and a misaligned workspace before touching the
    device."""
    import torch

    f = LIB.moe_finalize_workspace_flag
    v = ctypes.c_int(5)
    assert f(A, 0, None, None) == -1
    assert f(A + 4, 0, ctypes.byref(v), None) == -5 and v.value == 5
    with pytest.raises(ValueError):
        M.moe_finalize_workspace_flag(torch.zeros(0, dtype=torch.uint8))


def test_slice_reciprocal_is_exact_where_used():
    """The kernel divides a workgroup index q by the slice count S as (q * m) >> 32 with
    m = ceil(2^32 / S), and the host takes that form only where q * S < 2^32 for every index of
    the grid. Check the claim exhaustively for the indices a split-row grid can have (S up to 16,
    q below 2^20) and at the bound for every S a finalize-only grid can have (up to 2048)."""
    import numpy as np

    q = np.arange(1 << 20, dtype=np.uint64)
    for S in range(2, 17):
        m = np.uint64(((1 << 32) + S - 1) // S)
        assert np.array_equal((q * m) >> np.uint64(32), q // np.uint64(S)), S
    for S in range(2, 2049):
        m = ((1 << 32) + S - 1) // S
        top = ((1 << 32) - 1) // S                  # the largest q with q * S < 2^32
        edge = [top - i for i in range(min(top, 3 * S) + 1)] + list(range(0, 3 * S))
        # every residue class near the top, where the error term is largest
        assert all((v * m) >> 32 == v // S for v in edge), S


# Launch shapes the forced-slice and forced-group sweeps on MI355X (256 CUs) found fastest, with
# the measured margin over the runner-up (µs; warm / cold protocols as noted). The rules are
# tuned to these; a change that moves one of them needs a new measurement.
MEASURED_BEST = [
    # (entry, T, H, K, slices, route_groups, margin)
    (1, 1, 6144, 8, 6, 2, "6 slices 3.51 vs 8: 3.61; 2 groups beat 1 by 0.15 warm"),
    (1, 16, 6144, 8, 6, 2, "6 slices 3.80 vs 7: 3.85"),
    (1, 32, 7168, 8, 7, 2, "7 slices 4.76 cold vs 8: 4.82"),
    (1, 64, 7168, 8, 4, 1, "1 group 4.61 cold vs 2: 5.05"),
    (1, 48, 7168, 8, 5, 1, "1 group 4.60 cold vs 2: 5.00"),
    (1, 128, 7168, 8, 2, 1, "2 slices 5.92 vs whole rows 6.37"),
    (1, 1, 7680, 8, 7, 1, "1 group 3.65 cold vs 2: 3.91"),
    (1, 32, 7168, 16, 7, 2, "2 groups 4.91 cold vs 4: 5.11"),
    (1, 1, 2048, 22, 4, 4, "4 groups 3.88 vs 2: 4.36"),
    (1, 256, 2048, 8, 1, 1, "1 group 3.98 cold vs 2: 4.30"),
    (1, 1024, 2048, 22, 1, 1, "1 group 16.9 cold vs 2: 17.9, 4: 20.9"),
    (1, 512, 2048, 22, 1, 2, "2 groups 9.19 cold vs 1: 9.67, 4: 11.0"),
    (1, 1024, 1024, 10, 1, 1, "1 group 6.01 cold vs 2: 9.10"),
    (1, 4, 1024, 8, 1, 2, "2 groups 2.95 warm vs 1: 3.06"),
    (2, 64, 6144, 8, 4, 1, "NVFP4: 4 slices, 1 group 5.32 cold vs 2 groups 5.88"),
    (2, 1, 6144, 8, 6, 2, "NVFP4: 2 groups 4.15 warm vs 1: 4.35"),
    (0, 100, 7168, 17, 1, 4, "finalize: 4 groups 6.55 cold vs 1: 7.76"),
    (0, 100, 16384, 22, 1, 4, "finalize: 4 groups 12.28 cold vs 1: 13.45, 2: 12.68"),
    (0, 250, 7168, 22, 1, 4, "finalize: 4 groups 13.27 cold vs 1: 13.94"),
    (0, 250, 7168, 32, 1, 1, "finalize: 1 group 17.47 cold vs 4: 17.60"),
    (0, 1000, 7168, 33, 1, 1, "finalize: 1 group 68.3 cold vs 4: 71.5"),
]


@pytest.mark.parametrize("entry,T,H,K,slices,groups,margin", MEASURED_BEST)
def test_launch_rules_keep_the_measured_best(entry, T, H, K, slices, groups, margin):
    c = M.moe_finalize_launch_config(entry, T, H, K, num_cus=256)
    assert (c["slices"], c["route_groups"]) == (slices, groups), (c, margin)
