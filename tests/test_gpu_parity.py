"""GPU parity: the HIP path through the C ABI against the FP64 oracle on seeded inputs.

Comparison rules (see tests/comparators.py): finalize values inside the float32 admissible
window of the exact sum (and within 1 ulp except near cancellation); residual_out inside the
image of that window; norm_out within 1 ulp of the oracle where residual_out matched it;
indices / route selection bit-exact (dyadic fixtures, exact gathers, NaN poison); quantized codes
bit-exact where the kernel's norm_out equals the oracle's.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("needs a GPU", allow_module_level=True)

import moe_expert_output_amd as M  # noqa: E402
import oracle as O  # noqa: E402
from synth import MoeInputs, make_inputs, make_inputs_on_device, workload_seed  # noqa: E402
from tests.comparators import ulp_distance  # noqa: E402
from tests.parity import (bits16, check_finalize, check_norm, check_residual,  # noqa: E402
                          np64, oracle_ref, record_accuracy, to_dev)

ACT_T = {"bf16": torch.bfloat16, "fp16": torch.float16}


def _say(*a):
    print(*a, flush=True)


def run_finalize(inp, d=None, rsf=None):
    d = d or to_dev(inp)
    out = torch.empty(inp.T, inp.H, dtype=ACT_T[inp.act_dtype], device="cuda")
    M.moe_finalize_run(d["rows"], d["idx"], d["scales"], d["shared"],
                       inp.rsf if rsf is None else rsf, out)
    torch.cuda.synchronize()
    return out


_WS = {}


def workspace(T, H=0, K=0):
    """A zero-filled workspace shared by the tests (calls are serialized on one stream)."""
    need = M.moe_finalize_workspace_size(T, H, K)
    ws = _WS.get("ws")
    if ws is None or ws.numel() < need:
        ws = torch.zeros(max(need, 1 << 20), dtype=torch.uint8, device="cuda")
        _WS["ws"] = ws
    return ws


def ws_flag():
    ws = _WS.get("ws")
    return 0 if ws is None else int(ws[:4].view(torch.int32).item())


def run_rmsnorm(inp, d=None, residual_out=True, use_ws=True):
    d = d or to_dev(inp)
    dt = ACT_T[inp.act_dtype]
    ro = torch.empty(inp.T, inp.H, dtype=dt, device="cuda") if residual_out else None
    no = torch.empty(inp.T, inp.H, dtype=dt, device="cuda")
    ws = workspace(inp.T) if use_ws else None
    M.moe_finalize_rmsnorm_run(d["rows"], d["idx"], d["scales"], d["shared"], inp.rsf,
                               d["residual"], d["gamma"], inp.eps, ro, no, ws)
    torch.cuda.synchronize()
    assert ws_flag() == 0, "a split row timed out waiting for its slices"
    return ro, no


def full_check(inp, *, finalize=True, rmsnorm=True, config=None):
    """Finalize and RMSNorm (split and whole rows) against the oracle; with `config`, one
    accuracy record per entry point and row mode."""
    _say(f"case T={inp.T} H={inp.H} K={inp.K} act={inp.act_dtype} scales={inp.scale_dtype} "
         f"seed={inp.seed} shared={inp.shared is not None}")
    ref = oracle_ref(inp, with_norm=rmsnorm)
    reps = []
    d = to_dev(inp)
    if finalize:
        s = run_finalize(inp, d)
        r = check_finalize(np64(s), ref, inp.act_dtype)
        reps.append(r)
        if config:
            record_accuracy(config, inp, "moe_finalize_run", "-", [r])
    if rmsnorm:
        for use_ws in (True, False):      # split rows (workspace) and whole-row workgroups
            ro, no = run_rmsnorm(inp, d, use_ws=use_ws)
            R, N = np64(ro), np64(no)
            pair = [check_residual(R, ref, np64(inp.residual), inp.act_dtype),
                    check_norm(N, R, ref, np64(inp.gamma), inp.eps, inp.act_dtype)]
            reps += pair
            if config:
                rec = record_accuracy(config, inp, "moe_finalize_rmsnorm_run",
                                      "split" if use_ws else "whole", pair, R, N)
                _say(f"  mean|err| residual_out {rec['residual_out']['mean_abs_err']:.3e} "
                     f"(floor {rec['residual_out']['floor_mean_abs_err']:.3e}), norm_out "
                     f"{rec['norm_out']['mean_abs_err']:.3e} "
                     f"(floor {rec['norm_out']['floor_mean_abs_err']:.3e})")
    for r in reps:
        _say("  ", r)
    return reps


# ---- the workloads -------------------------------------------------------------------------------
def test_tiny_t4_h1024_k8():
    full_check(make_inputs(4, 1024, 8, seed=workload_seed("tiny", 4)), config="tiny")


@pytest.mark.parametrize("T", [1, 4, 16])
def test_decode_h6144_k8(T):
    full_check(make_inputs(T, 6144, 8, seed=workload_seed("decode", T)), config="decode")


@pytest.mark.parametrize("act", ["bf16", "fp16"])
@pytest.mark.parametrize("T", [32, 64, 128])
def test_larger_decode_h7168_k8(T, act):
    full_check(make_inputs(T, 7168, 8, act_dtype=act, seed=workload_seed("larger", T, act)),
               config="larger")


@pytest.mark.parametrize("HK", [(2048, 22), (3584, 16), (2048, 6), (2048, 10)])
@pytest.mark.parametrize("sdt", ["fp32", "bf16"])
@pytest.mark.parametrize("T", [1, 8, 16, 32])
def test_high_topk(T, sdt, HK):
    H, K = HK
    full_check(make_inputs(T, H, K, scale_dtype=sdt, with_shared=False,
                           seed=workload_seed("highk", T, "bf16", sdt, K)), config="high_topk")


@pytest.mark.parametrize("THKG", [(100, 7168, 17, 4), (300, 2048, 22, 4), (512, 4096, 24, 4),
                                  (250, 7168, 32, 1)])
def test_finalize_mid_batch_high_topk(THKG):
    """Finalize-only past the route-group wavefront cap: top_k 17..24 in four route groups,
    top_k 32 in one, against the oracle's admissible window."""
    T, H, K, G = THKG
    assert M.moe_finalize_launch_config(0, T, H, K, num_cus=256)["route_groups"] == G
    full_check(make_inputs(T, H, K, seed=workload_seed("highk", T, "bf16", "fp32", K) + H),
               rmsnorm=False)


# ---- exactness: indices, route selection, poison -------------------------------------------------
@pytest.mark.parametrize("act", ["bf16", "fp16"])
def test_k1_exact_gather(act):
    inp = make_inputs(37, 1032, 1, seed=71, act_dtype=act, scale_dtype=None, with_shared=False,
                      n_rows=80)
    s = run_finalize(inp, rsf=1.0)
    want = torch.zeros(37, 1032, dtype=ACT_T[act])
    for t in range(37):
        p = int(inp.idx[t, 0])
        if p >= 0:
            want[t] = inp.rows[p]
    assert np.array_equal(bits16(s), bits16(want))


def _dyadic_inputs(T, H, K, act, seed):
    """Small-integer rows, power-of-two weights, RSF 2, integer shared and residual: every float32
    operation is exact, so finalize and residual_out must match the oracle bit for bit."""
    rng = np.random.Generator(np.random.PCG64(seed))
    n_rows = T * K + 5
    inp = make_inputs(T, H, K, seed=seed, act_dtype=act, n_rows=n_rows)
    dt = ACT_T[act]
    inp.rows = torch.from_numpy(rng.integers(-8, 9, (n_rows, H)).astype(np.float32)).to(dt)
    inp.scales = torch.from_numpy(
        np.ldexp(1.0, rng.integers(-4, 2, (T, K))).astype(np.float32))
    inp.shared = torch.from_numpy(rng.integers(-16, 17, (T, H)).astype(np.float32)).to(dt)
    inp.residual = torch.from_numpy(rng.integers(-16, 17, (T, H)).astype(np.float32)).to(dt)
    inp.rsf = 2.0
    return inp


@pytest.mark.parametrize("act", ["bf16", "fp16"])
@pytest.mark.parametrize("TK", [(3, 8), (16, 22), (5, 64), (9, 6)])
def test_dyadic_bit_exact(act, TK):
    T, K = TK
    H = 2048 if act == "bf16" else 1024
    inp = _dyadic_inputs(T, H, K, act, seed=80 + K)
    ref = oracle_ref(inp)
    s = run_finalize(inp)
    assert np.array_equal(bits16(s), O.encode_bits(ref.s, O.FORMATS[act]).astype(np.int64))
    ro, no = run_rmsnorm(inp)
    assert np.array_equal(np64(ro), ref.R)
    check_norm(np64(no), np64(ro), ref, np64(inp.gamma), inp.eps, act)
    # routes reordered inside the top-k: bit-identical (every operation is exact)
    prng = np.random.Generator(np.random.PCG64(7 + K))
    perm = torch.from_numpy(np.stack([prng.permutation(K) for _ in range(T)]))
    inp2 = _dyadic_inputs(T, H, K, act, seed=80 + K)
    inp2.idx = torch.gather(inp.idx, 1, perm)
    inp2.scales = torch.gather(inp.scales, 1, perm)
    assert np.array_equal(bits16(run_finalize(inp2)), bits16(s))


def test_nan_poison_never_read():
    inp = make_inputs(24, 2048, 10, seed=90, n_rows=400)
    ref = oracle_ref(inp)
    used = set(int(p) for p in inp.idx.flatten().tolist() if p >= 0)
    rows = inp.rows.clone()
    for r in range(inp.n_rows):
        if r not in used:
            rows[r] = float("nan")
    sc = inp.scales.clone()
    sc[inp.idx < 0] = float("nan")
    inp.rows, inp.scales = rows, sc
    s = run_finalize(inp)
    ro, no = run_rmsnorm(inp)
    for t in (s, ro, no):
        assert torch.isfinite(t.float()).all()
    check_finalize(np64(s), ref, "bf16")
    # out-of-range indices on both sides are absent routes too
    inp.idx = torch.where(inp.idx < 0, torch.full_like(inp.idx, 1 << 30), inp.idx)
    assert np.array_equal(bits16(run_finalize(inp)), bits16(s))
    inp.idx = torch.where(inp.idx == (1 << 30), torch.full_like(inp.idx, -7), inp.idx)
    assert np.array_equal(bits16(run_finalize(inp)), bits16(s))


def test_no_valid_routes_and_no_rows():
    inp = make_inputs(6, 1024, 8, seed=91)
    inp.idx[2] = -1
    inp.idx[4] = -1
    full_check(inp)
    s = run_finalize(inp)
    assert np.array_equal(bits16(s[2]), bits16(inp.shared[2]))
    # zero permuted rows: every route absent
    inp0 = make_inputs(3, 512, 4, seed=92, with_shared=False)
    inp0.rows = inp0.rows[:0]
    inp0.n_rows = 0
    s0 = run_finalize(inp0)
    assert not s0.float().abs().sum().item()


# ---- edge shapes ------------------------------------------------------------------------------------
@pytest.mark.parametrize("H", [8, 1000, 1032, 4104, 8192, 12288, 16384])
def test_ragged_and_large_hidden(H):
    full_check(make_inputs(5, H, 8, seed=100 + H))


@pytest.mark.parametrize("K", [1, 2, 3, 5, 17, 33, 64])
def test_topk_range(K):
    full_check(make_inputs(7, 2048, K, seed=200 + K, mask_frac=0.25 if K > 1 else 0.0))


def test_zero_tokens_is_noop():
    inp = make_inputs(1, 1024, 8, seed=300)
    d = to_dev(inp)
    out = torch.full((1, 1024), 7.0, dtype=torch.bfloat16, device="cuda")
    M.moe_finalize_run(d["rows"], d["idx"][:0], d["scales"][:0], None, 2.5, out[:0])
    M.moe_finalize_rmsnorm_run(d["rows"], d["idx"][:0], d["scales"][:0], None, 2.5,
                               d["residual"][:0], d["gamma"], 1e-6, None, out[:0])
    torch.cuda.synchronize()
    assert (out.float() == 7.0).all()


def test_optional_terms_and_inplace_residual():
    inp = make_inputs(9, 3072, 8, seed=301)
    ref = oracle_ref(inp)
    d = to_dev(inp)
    # in-place: residual_out aliases residual
    res = d["residual"].clone()
    no = torch.empty_like(res)
    M.moe_finalize_rmsnorm_run(d["rows"], d["idx"], d["scales"], d["shared"], inp.rsf, res,
                               d["gamma"], inp.eps, res, no, workspace(inp.T))
    torch.cuda.synchronize()
    check_residual(np64(res), ref, np64(inp.residual), "bf16")
    # residual_out omitted: norm_out unchanged
    _, no2 = run_rmsnorm(inp, d, residual_out=False)
    assert np.array_equal(bits16(no2), bits16(no))
    # scales omitted == all-ones scales; shared omitted; RSF 1
    inp1 = make_inputs(9, 3072, 8, seed=302, with_shared=False)
    inp1.scales = None
    full_check(inp1)


def test_deterministic_and_graph_replay():
    inp = make_inputs(64, 7168, 8, seed=303)
    d = to_dev(inp)
    ro1, no1 = run_rmsnorm(inp, d)
    ro2, no2 = run_rmsnorm(inp, d)
    assert np.array_equal(bits16(ro1), bits16(ro2)) and np.array_equal(bits16(no1), bits16(no2))
    ro = torch.empty_like(ro1)
    no = torch.empty_like(no1)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    ws = workspace(inp.T)
    with torch.cuda.graph(g, stream=s):
        M.moe_finalize_rmsnorm_run(d["rows"], d["idx"], d["scales"], d["shared"], inp.rsf,
                                   d["residual"], d["gamma"], inp.eps, ro, no, ws)
    for _ in range(3):
        ro.zero_()
        no.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits16(ro), bits16(ro1)) and np.array_equal(bits16(no), bits16(no1))
    assert ws_flag() == 0


def test_workspace_shared_across_shapes():
    """One workspace, calls whose rows split into different slice counts, in any order."""
    cases = [(1, 6144), (128, 7168), (16, 6144), (4, 1024), (64, 7168), (1, 7168), (32, 3584)]
    for T, H in cases + cases[::-1]:
        inp = make_inputs(T, H, 8, seed=400 + T + H)
        ref = oracle_ref(inp)
        ro, no = run_rmsnorm(inp)
        check_residual(np64(ro), ref, np64(inp.residual), "bf16")
        check_norm(np64(no), np64(ro), ref, np64(inp.gamma), inp.eps, "bf16")
    assert ws_flag() == 0


def test_concurrent_streams_with_own_workspaces():
    """Split-row calls in flight on two streams at once, each stream with its own workspace (the
    way to overlap calls; one workspace shared by overlapping calls would race): every result
    equals the same call made alone, and neither workspace records a timeout."""
    cases = [(16, 6144, 601), (64, 7168, 602), (1, 6144, 603), (32, 7168, 604), (4, 1024, 605),
             (128, 7168, 606)]
    inps = [make_inputs(T, H, 8, seed=sd) for T, H, sd in cases]
    devs = [to_dev(i) for i in inps]
    alone = [run_rmsnorm(i, d) for i, d in zip(inps, devs)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [torch.zeros(M.moe_finalize_workspace_size(128, 7168, 8), dtype=torch.uint8,
                       device="cuda") for _ in streams]
    outs = [(torch.empty(i.T, i.H, dtype=torch.bfloat16, device="cuda"),
             torch.empty(i.T, i.H, dtype=torch.bfloat16, device="cuda")) for i in inps]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    for _ in range(10):
        for j, (i, d) in enumerate(zip(inps, devs)):
            k = j % 2
            with torch.cuda.stream(streams[k]):
                M.moe_finalize_rmsnorm_run(d["rows"], d["idx"], d["scales"], d["shared"], i.rsf,
                                           d["residual"], d["gamma"], i.eps, outs[j][0],
                                           outs[j][1], wss[k])
    torch.cuda.synchronize()
    for (ro, no), (ro1, no1) in zip(outs, alone):
        assert np.array_equal(bits16(ro), bits16(ro1)) and np.array_equal(bits16(no), bits16(no1))
    assert all(int(w[:4].view(torch.int32).item()) == 0 for w in wss)


@pytest.mark.parametrize("T,H", [(16, 6144), (64, 7168), (300, 3584)])
def test_cache_policy_changes_no_bits(T, H):
    """Every entry point gives bit-identical outputs under the three cache policies: cacheable or
    nontemporal accesses change where data is cached, never what is computed."""
    inp = make_inputs(T, H, 8, seed=700 + T)
    d = to_dev(inp)
    gs = O.nvfp4_global_scale(oracle_ref(inp).N)
    pols = (M.MOE_FIN_CACHE_AUTO, M.MOE_FIN_CACHE_KEEP, M.MOE_FIN_CACHE_STREAM)
    got = {}
    prev = M.moe_finalize_set_cache_policy(M.MOE_FIN_CACHE_AUTO)
    try:
        for pol in pols:
            M.moe_finalize_set_cache_policy(pol)
            outs = [run_finalize(inp, d)]
            outs += list(run_rmsnorm(inp, d)) + list(run_rmsnorm(inp, d, use_ws=False))
            ro, no, qo, so = run_quant(inp, M.MOE_QUANT_NVFP4, gs)
            got[pol] = [bits16(x) for x in outs + [ro, no]] + [np.asarray(qo), np.asarray(so)]
    finally:
        M.moe_finalize_set_cache_policy(prev)
    for pol in pols[1:]:
        for a, b in zip(got[pol], got[pols[0]]):
            assert np.array_equal(a, b), pol
    assert ws_flag() == 0


# ---- validation through the ABI on a device ---------------------------------------------------------
def test_validation_errors():
    inp = make_inputs(4, 1024, 8, seed=304)
    d = to_dev(inp)
    out = torch.empty(4, 1024, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(M.MoeFinalizeError) as e:
        M.moe_finalize_run(d["rows"], d["idx"], d["scales"], d["shared"], 2.5, d["rows"][:4])
    assert e.value.code == -9  # output overlaps an input
    buf = torch.empty(4 * 1024 + 8, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(M.MoeFinalizeError) as e:
        M.moe_finalize_run(d["rows"], d["idx"], d["scales"], d["shared"], 2.5,
                           buf[1:1 + 4096].view(4, 1024))
    assert e.value.code == -5  # misaligned output
    out.fill_(3.0)
    torch.cuda.synchronize()
    assert (out.float() == 3.0).all()


# ---- quantized outputs -------------------------------------------------------------------------------
def _sf_offsets(T, H, layout):
    return np.array([[O.sf_offset(t, b, H, layout) for b in range(H // 16)] for t in range(T)])


def run_quant(inp, qtype, qscale, layout=M.MOE_SF_SWIZZLED_128x4, with_norm=True, use_ws=True):
    d = to_dev(inp)
    dt = ACT_T[inp.act_dtype]
    T, H = inp.T, inp.H
    ro = torch.empty(T, H, dtype=dt, device="cuda")
    no = torch.empty(T, H, dtype=dt, device="cuda") if with_norm else None
    nv = qtype == M.MOE_QUANT_NVFP4
    qo = torch.full((T, H // 2 if nv else H), 0xAB, dtype=torch.uint8, device="cuda")
    so = None
    if nv:
        so = torch.full((M.moe_finalize_sf_size(T, H, layout),), 0xCD, dtype=torch.uint8,
                        device="cuda")
    qs = torch.tensor([qscale], dtype=torch.float32, device="cuda")
    M.moe_finalize_quant_run(d["rows"], d["idx"], d["scales"], d["shared"], inp.rsf,
                             d["residual"], d["gamma"], inp.eps, qtype, qs, qo, so, layout, ro,
                             no, workspace(T) if use_ws else None)
    torch.cuda.synchronize()
    assert ws_flag() == 0
    return ro, no, qo.cpu().numpy(), (None if so is None else so.cpu().numpy())


@pytest.mark.parametrize("layout", [1, 0])
@pytest.mark.parametrize("TH", [(64, 6144), (5, 1024), (130, 2048), (1, 48), (1030, 7168)])
def test_nvfp4(TH, layout):
    T, H = TH
    inp = make_inputs(T, H, 8, seed=workload_seed("quant", T) + H)
    _say(f"nvfp4 T={T} H={H} layout={layout}")
    ref = oracle_ref(inp)
    gs = O.nvfp4_global_scale(ref.N)            # 448 * 6 / amax(norm_out), as float32
    codes_or, sf_or = O.quant_nvfp4(ref.N, gs, layout)
    offs = _sf_offsets(T, H, layout)
    for use_ws in (True, False):
        ro, no, qo, so = run_quant(inp, M.MOE_QUANT_NVFP4, gs, layout, use_ws=use_ws)
        R, N = np64(ro), np64(no)
        pair = [check_residual(R, ref, np64(inp.residual), "bf16"),
                check_norm(N, R, ref, np64(inp.gamma), inp.eps, "bf16")]
        nb = H // 16
        same_blk = (N == ref.N).reshape(T, nb, 16).all(-1)
        c_g = qo.reshape(T, nb, 8)
        c_o = codes_or.reshape(T, nb, 8)
        sf_g, sf_o = so[offs], sf_or[offs]
        # codes and scales (padding included) are the NVFP4 quantization of the kernel's own
        # rounded norm_out, bit for bit
        own_c, own_s = O.quant_nvfp4(N, gs, layout)
        assert np.array_equal(qo, own_c) and np.array_equal(so, own_s)
        # blocks whose norm_out equals the primary oracle's: codes and scales bit-exact
        assert np.array_equal(c_g[same_blk], c_o[same_blk])
        assert np.array_equal(sf_g[same_blk], sf_o[same_blk])
        assert same_blk.mean() > 0.98, same_blk.mean()
        if (T, H) == (64, 6144):
            record_accuracy("quant", inp, f"moe_finalize_quant_run NVFP4 layout={layout}",
                            "split" if use_ws else "whole", pair, R, N,
                            {"codes_and_scales_bit_exact_vs_quant_of_own_norm_out": True,
                             "blocks_equal_to_oracle_norm_out": float(same_blk.mean())})
        # blocks within one ulp of it: scale within one E4M3 step
        near_blk = ~same_blk & (ulp_distance(O.encode_bits(N, O.FORMATS["bf16"]),
                                             O.encode_bits(ref.N, O.FORMATS["bf16"]))
                                <= 1).reshape(T, nb, 16).all(-1)
        diff_sf = np.abs(sf_g.astype(int) - sf_o.astype(int))
        assert diff_sf[near_blk].max(initial=0) <= 1
        # every byte outside the valid (t, b) scale positions is zero padding
        if layout == 1:
            pad = np.ones(so.size, bool)
            pad[offs.ravel()] = False
            assert not so[pad].any()
        else:
            assert so.size == T * nb
        _say(f"  exact blocks {same_blk.mean():.5f} of {same_blk.size}")
    # norm_out may be omitted: same codes
    _, _, qo2, so2 = run_quant(inp, M.MOE_QUANT_NVFP4, gs, layout, with_norm=False)
    assert np.array_equal(qo2, qo) and np.array_equal(so2, so)


@pytest.mark.parametrize("THK", [(1024, 2048, 22), (512, 2048, 22)])
@pytest.mark.parametrize("qt", ["nvfp4", "fp8"])
def test_quant_high_topk_whole_rows(THK, qt):
    """Quantized outputs of whole rows with many routes per group (one group of 22 routes in two
    chunks of loads from 1024 tokens, two groups of 11 below): codes and scales are the
    quantization of the kernel's own rounded norm_out, bit for bit."""
    T, H, K = THK
    inp = make_inputs(T, H, K, seed=workload_seed("quant", T) + K)
    _say(f"quant high top_k whole rows {qt} T={T} H={H} K={K}")
    ref = oracle_ref(inp)
    if qt == "nvfp4":
        scale = O.nvfp4_global_scale(ref.N)
        ro, no, qo, so = run_quant(inp, M.MOE_QUANT_NVFP4, scale, 1)
    else:
        scale = O.fp8_scale(ref.N)
        ro, no, qo, so = run_quant(inp, M.MOE_QUANT_FP8_E4M3, scale, 1)
    R, N = np64(ro), np64(no)
    check_residual(R, ref, np64(inp.residual), "bf16")
    check_norm(N, R, ref, np64(inp.gamma), inp.eps, "bf16")
    if qt == "nvfp4":
        own_c, own_s = O.quant_nvfp4(N, scale, 1)
        assert np.array_equal(qo, own_c) and np.array_equal(so, own_s)
    else:
        assert np.array_equal(qo, O.quant_fp8(N, scale))


@pytest.mark.parametrize("use_ws", [True, False])
@pytest.mark.parametrize("TH", [(3, 16384), (260, 12288)])
@pytest.mark.parametrize("qt", ["nvfp4", "fp8"])
def test_quant_wide_rows(TH, qt, use_ws):
    """Rows wider than 8192: whole-row workgroups hold two slots per lane, and split rows many
    slices; codes and scales are the quantization of the kernel's own rounded norm_out, bit for
    bit, in both row modes."""
    T, H = TH
    inp = make_inputs(T, H, 8, seed=workload_seed("quant", T) + H + 3)
    _say(f"quant wide rows {qt} T={T} H={H} use_ws={use_ws}")
    ref = oracle_ref(inp)
    if qt == "nvfp4":
        scale = O.nvfp4_global_scale(ref.N)
        ro, no, qo, so = run_quant(inp, M.MOE_QUANT_NVFP4, scale, 1, use_ws=use_ws)
    else:
        scale = O.fp8_scale(ref.N)
        ro, no, qo, so = run_quant(inp, M.MOE_QUANT_FP8_E4M3, scale, 1, use_ws=use_ws)
    R, N = np64(ro), np64(no)
    check_residual(R, ref, np64(inp.residual), "bf16")
    check_norm(N, R, ref, np64(inp.gamma), inp.eps, "bf16")
    if qt == "nvfp4":
        own_c, own_s = O.quant_nvfp4(N, scale, 1)
        assert np.array_equal(qo, own_c) and np.array_equal(so, own_s)
    else:
        assert np.array_equal(qo, O.quant_fp8(N, scale))


@pytest.mark.parametrize("T,H", [(64, 6144), (3, 6144), (1030, 5120)])
def test_fp8(T, H):
    inp = make_inputs(T, H, 8, seed=workload_seed("quant", T) + 7)
    ref = oracle_ref(inp)
    s8 = O.fp8_scale(ref.N)
    codes_or = O.quant_fp8(ref.N, s8)
    for use_ws in (True, False):
        ro, no, qo, _ = run_quant(inp, M.MOE_QUANT_FP8_E4M3, s8, use_ws=use_ws)
        R, N = np64(ro), np64(no)
        pair = [check_residual(R, ref, np64(inp.residual), "bf16"),
                check_norm(N, R, ref, np64(inp.gamma), inp.eps, "bf16")]
        # the codes are the FP8 quantization of the kernel's own rounded norm_out, bit for bit
        assert np.array_equal(qo, O.quant_fp8(N, s8))
        same = N == ref.N
        assert np.array_equal(qo[same], codes_or[same])
        # where norm_out is one ulp from the primary oracle's, the code moves by at most one E4M3
        # step (farther only near cancellation, where residual_out may sit several ulps away)
        near = ~same & (ulp_distance(O.encode_bits(N, O.FORMATS["bf16"]),
                                     O.encode_bits(ref.N, O.FORMATS["bf16"])) <= 1)
        d = np.abs((qo[near] & 0x7F).astype(int) - (codes_or[near] & 0x7F).astype(int))
        assert d.max(initial=0) <= 1
        assert same.mean() > 0.99
        if (T, H) == (64, 6144):
            record_accuracy("quant", inp, "moe_finalize_quant_run FP8",
                            "split" if use_ws else "whole", pair, R, N,
                            {"codes_bit_exact_vs_quant_of_own_norm_out": True,
                             "elements_equal_to_oracle_norm_out": float(same.mean())})


def test_quant_codec_edges():
    """Saturation, tiny blocks (zero block scale) and signed zeros through the kernel: a row whose
    values hit every E2M1 / E4M3 rounding midpoint exactly, built with dyadic inputs."""
    T, H = 2, 1024
    inp = _dyadic_inputs(T, H, 4, "bf16", seed=501)
    ref = oracle_ref(inp)
    for gs in (O.nvfp4_global_scale(ref.N), 1e-8, 3e4):
        codes_or, sf_or = O.quant_nvfp4(ref.N, gs, 1)
        ro, no, qo, so = run_quant(inp, M.MOE_QUANT_NVFP4, gs)
        N = np64(no)
        offs = _sf_offsets(T, H, 1)
        same_blk = (N == ref.N).reshape(T, H // 16, 16).all(-1)
        assert np.array_equal(qo.reshape(T, -1, 8)[same_blk], codes_or.reshape(T, -1, 8)[same_blk])
        assert np.array_equal(so[offs][same_blk], sf_or[offs][same_blk])
    for s8 in (O.fp8_scale(ref.N), 1e-6, 1e4):
        codes_or = O.quant_fp8(ref.N, s8)
        _, no, qo, _ = run_quant(inp, M.MOE_QUANT_FP8_E4M3, s8)
        same = np64(no) == ref.N
        assert np.array_equal(qo[same], codes_or[same])


# ---- quantizing the oracle's rounded values: bit-exact everywhere ------------------------------
def _quantize_dev_x(x, qtype, qscale, layout):
    """moe_quantize_run of the device tensor x; returns (codes, scale bytes or None)."""
    T, H = x.shape
    nv = qtype == M.MOE_QUANT_NVFP4
    qo = torch.full((T, H // 2 if nv else H), 0xAB, dtype=torch.uint8, device="cuda")
    so = None
    if nv:
        so = torch.full((M.moe_finalize_sf_size(T, H, layout),), 0xCD, dtype=torch.uint8,
                        device="cuda")
    qs = torch.tensor([qscale], dtype=torch.float32, device="cuda")
    M.moe_quantize_run(x, qtype, qs, qo, so, layout)
    torch.cuda.synchronize()
    return qo.cpu().numpy(), (None if so is None else so.cpu().numpy())


def _quantize_dev(N_vals, act, qtype, qscale, layout):
    x = torch.from_numpy(N_vals.astype(np.float32)).to(ACT_T[act]).cuda()   # exact: N is act-valued
    return _quantize_dev_x(x, qtype, qscale, layout)


@pytest.mark.parametrize("act", ["bf16", "fp16"])
@pytest.mark.parametrize("TH", [(64, 6144), (130, 2048), (3, 48), (1, 7168)])
def test_quantize_oracle_values_bit_exact(TH, act):
    T, H = TH
    inp = make_inputs(T, H, 8, act_dtype=act, seed=workload_seed("quant", T, act) + H + 1)
    N = oracle_ref(inp).N
    N[0, :16] = 0.0                         # an all-zero block (scale 0)
    N[-1, 16:32] = -N[-1, 16:32]
    for layout in (M.MOE_SF_SWIZZLED_128x4, M.MOE_SF_LINEAR):
        for gs in (O.nvfp4_global_scale(N), 1e-6, 5e3):
            want_c, want_s = O.quant_nvfp4(N, gs, layout)
            got_c, got_s = _quantize_dev(N, act, M.MOE_QUANT_NVFP4, gs, layout)
            assert np.array_equal(got_c, want_c), (layout, gs)
            assert np.array_equal(got_s, want_s), (layout, gs)
    for s8 in (O.fp8_scale(N), 1e-3, 1e3):
        want = O.quant_fp8(N, s8)
        got, _ = _quantize_dev(N, act, M.MOE_QUANT_FP8_E4M3, s8, 0)
        assert np.array_equal(got, want), s8


def test_quantize_rounding_midpoints_bit_exact():
    """Values placed exactly on E2M1 / E4M3 rounding midpoints (and one bf16 step either side),
    so every tie-to-even decision of the encoders is exercised."""
    gs = 1.0
    # block scale 1.0 needs amax = 6: put 6.0 first in every block, then midpoints
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    vals = []
    for m in mids:
        b = O.round_to_format(np.array([m]), O.BF16)[0]
        up = float(np.nextafter(np.float32(b), np.float32(10)).astype(np.float32))
        vals += [b, O.round_to_format(np.array([b * (1 + 2 ** -7)]), O.BF16)[0],
                 O.round_to_format(np.array([b * (1 - 2 ** -8)]), O.BF16)[0], -b]
    vals = np.array(vals)
    n_blocks = (len(vals) + 14) // 15
    row = np.zeros(n_blocks * 16)
    for i in range(n_blocks):
        row[16 * i] = 6.0
        chunk = vals[15 * i:15 * i + 15]
        row[16 * i + 1:16 * i + 1 + len(chunk)] = chunk
    H = ((len(row) + 63) // 64) * 64
    N = np.zeros((2, H))
    N[0, :len(row)] = row
    N[1, :len(row)] = row * 2.0 ** -5        # scale 6*2^-5/6: an E4M3 value
    want_c, want_s = O.quant_nvfp4(N, gs, 1)
    got_c, got_s = _quantize_dev(N, "bf16", M.MOE_QUANT_NVFP4, gs, 1)
    assert np.array_equal(got_c, want_c) and np.array_equal(got_s, want_s)
    # FP8: E4M3 midpoints in every binade
    e4 = O.decode_bits(np.arange(0x7E, dtype=np.uint8), O.E4M3)
    m8 = (e4[:-1] + e4[1:]) / 2
    x = O.round_to_format(np.concatenate([m8, -m8, e4]), O.BF16)
    H8 = ((len(x) + 7) // 8) * 8
    N8 = np.zeros((1, H8))
    N8[0, :len(x)] = x
    assert np.array_equal(_quantize_dev(N8, "bf16", M.MOE_QUANT_FP8_E4M3, 1.0, 0)[0],
                          O.quant_fp8(N8, 1.0))


def _act_vals(x, act):
    return O.round_to_format(np.asarray(x, dtype=np.float64), O.BF16 if act == "bf16" else O.FP16)


@pytest.mark.parametrize("act", ["bf16", "fp16"])
def test_quantize_near_midpoints_bit_exact(act):
    """Scales chosen so that x * scale lands within a float32 rounding of a rounding midpoint
    without being equal to it (the float32 product rounds onto the midpoint, the exact product
    is just above or below): FP8 codes, NVFP4 block scales and E2M1 codes must still follow the
    exact product, as the oracle does."""
    rng = np.random.default_rng(77 if act == "bf16" else 78)
    e4 = O.decode_bits(np.arange(0x7F, dtype=np.uint8), O.E4M3)
    m4 = (e4[:-1] + e4[1:]) / 2                       # E4M3 rounding midpoints
    m2 = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    ks = np.arange(-6, 6)
    for draw in range(16):
        x0 = float(_act_vals(rng.uniform(1, 2), act))
        # FP8: s8 = fl32(mid / x0); elements x0 * 2^k hit the midpoints mid * 2^k (normal range)
        mid = float(m4[rng.integers(16, 100)])
        s8 = float(np.float32(mid / x0))
        vals = np.concatenate([x0 * 2.0 ** ks, -x0 * 2.0 ** ks, _act_vals(rng.normal(size=40), act)])
        N = np.zeros((1, 64))
        N[0, :len(vals)] = vals
        got, _ = _quantize_dev(N, act, M.MOE_QUANT_FP8_E4M3, s8, 0)
        assert np.array_equal(got, O.quant_fp8(N, s8)), ("fp8", draw, s8)
        # NVFP4 E2M1 codes: gs = fl32(mid2 / x0) with block scale 1 (block amax a ~ 6 / gs), and
        # the same at block scales 2^k
        mid2 = float(m2[rng.integers(0, 7)])
        gs = float(np.float32(mid2 / x0))
        a = float(_act_vals(6.0 / gs, act))
        rows = []
        for k in range(-4, 4):
            blk = np.zeros(16)
            blk[0] = a * 2.0 ** k
            blk[1:4] = np.array([x0, -x0, x0]) * 2.0 ** k
            blk[4:] = _act_vals(rng.uniform(-1, 1, 12) * a * 2.0 ** k, act)
            rows.append(blk)
        # NVFP4 block scales: gs2 = fl32(6 * mid4 / a0), blocks with amax a0 * 2^k
        a0 = x0
        mid4 = float(m4[rng.integers(40, 100)])
        gs2 = float(np.float32(6.0 * mid4 / a0))
        N2 = np.concatenate(rows).reshape(2, 64)
        want_c, want_s = O.quant_nvfp4(N2, gs, 1)
        got_c, got_s = _quantize_dev(N2, act, M.MOE_QUANT_NVFP4, gs, 1)
        assert np.array_equal(got_c, want_c) and np.array_equal(got_s, want_s), ("e2m1", draw)
        rows = []
        for k in range(-3, 5):
            blk = _act_vals(rng.uniform(-1, 1, 16) * a0 * 2.0 ** k, act)
            blk[rng.integers(0, 16)] = -a0 * 2.0 ** k if k % 2 else a0 * 2.0 ** k
            rows.append(blk)
        N3 = np.concatenate(rows).reshape(2, 64)
        want_c, want_s = O.quant_nvfp4(N3, gs2, 1)
        got_c, got_s = _quantize_dev(N3, act, M.MOE_QUANT_NVFP4, gs2, 1)
        assert np.array_equal(got_c, want_c) and np.array_equal(got_s, want_s), ("scale", draw)


def _format_values_between(lo, hi, act):
    """Every positive bf16 / fp16 value in [lo, hi] (bit patterns of positive values are ordered)."""
    fmt = O.BF16 if act == "bf16" else O.FP16
    a, b = (int(O.encode_bits(_act_vals([v], act), fmt)[0]) for v in (lo, hi))
    return O.decode_bits(np.arange(a, b + 1, dtype=np.uint16), fmt)


@pytest.mark.parametrize("act", ["bf16", "fp16"])
def test_quantize_nvfp4_value_sweep_bit_exact(act):
    """Every bf16 / fp16 value from 1/64 of a block's maximum up to it, in blocks whose scales
    take every E4M3 significand, under global scales of three kinds: small integers, float32
    quotients 2688 / amax as a tensor-wide maximum gives them, and random float32 values. This
    puts elements on and next to all seven E2M1 rounding midpoints (exact ties and float32 near
    ties), where the encoder's bracketing conversion hands over to its exact midpoint test."""
    rng = np.random.default_rng(4242 if act == "bf16" else 4243)
    gss = [100.0, 6.0, float(np.float32(2688.0 / float(_act_vals([3.40625], act)[0]))),
           float(np.float32(2688.0 / float(_act_vals([0.71875], act)[0]))),
           float(np.float32(rng.uniform(10, 1000)))]
    H = 2048
    for gs in gss:
        blocks = []
        for sig in range(8, 16):
            sf_target = sig / 8.0 * 2.0 ** int(rng.integers(-3, 4))
            amax = float(_act_vals([6.0 * sf_target / gs], act)[0])
            vals = _format_values_between(amax / 64, amax, act)
            vals = vals[vals < amax]
            vals = vals * rng.choice([-1.0, 1.0], size=len(vals))
            for i in range(0, len(vals), 15):
                blk = np.zeros(16)
                blk[0] = amax if i % 2 else -amax
                chunk = vals[i:i + 15]
                blk[1:1 + len(chunk)] = chunk
                blocks.append(blk)
        nb = H // 16
        n_rows = -(-len(blocks) // nb)
        N = np.zeros((n_rows * nb, 16))
        N[:len(blocks)] = np.array(blocks)
        N = N.reshape(n_rows, H)
        for layout in (M.MOE_SF_SWIZZLED_128x4, M.MOE_SF_LINEAR):
            want_c, want_s = O.quant_nvfp4(N, gs, layout)
            got_c, got_s = _quantize_dev(N, act, M.MOE_QUANT_NVFP4, gs, layout)
            assert np.array_equal(got_s, want_s), (gs, layout)
            assert np.array_equal(got_c, want_c), (gs, layout)


@pytest.mark.parametrize("k", [-110, 0, 110])
def test_quantize_nvfp4_extreme_global_scales(k):
    """The E2M1 midpoint row of test_quantize_rounding_midpoints_bit_exact scaled by 2^k with the
    global scale 2^-k: the same codes and block scales. Global scales outside [2^-100, 2^100]
    take the encoder's per-midpoint tests instead of its bracketing conversion."""
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    vals = []
    for m in mids:
        b = O.round_to_format(np.array([m]), O.BF16)[0]
        vals += [b, O.round_to_format(np.array([b * (1 + 2 ** -7)]), O.BF16)[0],
                 O.round_to_format(np.array([b * (1 - 2 ** -8)]), O.BF16)[0], -b]
    row = np.zeros(64)
    for i in range(4):
        row[16 * i] = 6.0
        chunk = vals[7 * i:7 * i + 7]
        row[16 * i + 1:16 * i + 1 + len(chunk)] = chunk
    N0 = np.stack([row, row * 2.0 ** -5])
    want_c, want_s = O.quant_nvfp4(N0, 1.0, 1)
    N = N0 * 2.0 ** k                        # exact: powers of two within bf16's range
    gs = 2.0 ** -k
    got_c, got_s = _quantize_dev(N, "bf16", M.MOE_QUANT_NVFP4, gs, 1)
    assert np.array_equal(O.quant_nvfp4(N, gs, 1)[0], want_c)
    assert np.array_equal(got_c, want_c) and np.array_equal(got_s, want_s)


@pytest.mark.parametrize("act", ["bf16", "fp16"])
def test_quantize_nonfinite_bit_exact(act):
    """Infinities saturate (E4M3 448, E2M1 6); a NaN of either sign gives FP8 code 0x7F, and a
    NaN anywhere in a 16-element block gives that block scale code 0x7F and all-zero codes, as
    the oracle defines them. The tensor is built from bit patterns so NaN signs are exact."""
    fmt = O.BF16 if act == "bf16" else O.FP16
    rng = np.random.default_rng(91)
    T, H = 3, 128
    bits = O.encode_bits(_act_vals(rng.normal(size=(T, H)), act), fmt).astype(np.uint16)
    inf_b, nan_b = (0x7F80, 0x7FC0) if act == "bf16" else (0x7C00, 0x7E00)
    neg = 0x8000
    bits[0, 20] = inf_b                      # block 1: +inf
    bits[0, 40] = inf_b | neg                # block 2: -inf
    bits[0, 60] = nan_b                      # block 3: +NaN
    bits[1, 3] = nan_b | neg                 # block 0: -NaN next to an infinity
    bits[1, 5] = inf_b
    bits[1, 16:32] = 0                       # block 1: zeros, one of them -0
    bits[1, 17] = neg
    bits[2, 100] = nan_b | neg               # block 6: both NaN signs
    bits[2, 101] = nan_b
    N = O.decode_bits(bits, fmt)             # the values the kernel reads
    x = torch.from_numpy(bits.view(np.int16)).view(ACT_T[act]).cuda()
    finite_amax = float(np.max(np.abs(N[np.isfinite(N)])))
    for layout in (M.MOE_SF_SWIZZLED_128x4, M.MOE_SF_LINEAR):
        gs = float(np.float32(2688.0 / finite_amax))
        want_c, want_s = O.quant_nvfp4(N, gs, layout)
        got_c, got_s = _quantize_dev_x(x, M.MOE_QUANT_NVFP4, gs, layout)
        assert np.array_equal(got_c, want_c), layout
        assert np.array_equal(got_s, want_s), layout
        assert want_s[O.sf_offset(0, 3, H, layout)] == 0x7F
        assert want_s[O.sf_offset(0, 1, H, layout)] == 0x7E
    s8 = float(np.float32(448.0 / finite_amax))
    want = O.quant_fp8(N, s8)
    got, _ = _quantize_dev_x(x, M.MOE_QUANT_FP8_E4M3, s8, 0)
    assert np.array_equal(got, want)
    assert want[1, 3] == 0x7F and want[2, 100] == 0x7F and want[0, 40] == 0xFE


# ---- large batches (prefill-sized calls: whole rows, nontemporal streaming) ---------------------
@pytest.mark.parametrize("THK", [(256, 7168, 8), (512, 7168, 8), (2048, 2048, 8), (300, 3584, 16),
                                 (1024, 7168, 8), (1030, 5120, 8), (1024, 3584, 16),
                                 (1024, 7168, 4), (1024, 7168, 16), (100, 16384, 4),
                                 (1024, 1024, 10), (1024, 1024, 22), (1030, 1536, 33),
                                 (512, 2048, 22)])
def test_large_batch(THK):
    """From 1024 tokens whole-row workgroups are rounded up to four wavefronts (hidden 7168: 1024
    lanes for 896 slots; 5120: 768 for 640), so their last lanes hold no slot. From 1024 tokens
    a whole row also takes a single route group up to top_k 48, so top_k 22 and 33 load their
    routes in two and four chunks of 16; below that, top_k 22 runs as two groups of 11 routes."""
    T, H, K = THK
    full_check(make_inputs(T, H, K, seed=5000 + T + K))


@pytest.mark.parametrize("THK", [(1024, 1024, 22), (512, 2048, 22), (1024, 7168, 8)])
def test_large_batch_fp16_and_bf16_scales(THK):
    """The same whole-row shapes with fp16 activations, and with bf16 routing weights."""
    T, H, K = THK
    full_check(make_inputs(T, H, K, seed=5100 + T + K, act_dtype="fp16"))
    full_check(make_inputs(T, H, K, seed=5200 + T + K, scale_dtype="bf16"))


def test_rows_beyond_4gib_sampled_tokens():
    """Maximum-size addressing: 17000 tokens at hidden 16384 and top_k 8 give 4.46 GB of permuted
    rows, so routes reach rows past the 4 GiB mark. The whole batch runs through the finalize and
    the RMSNorm entry points; the oracle checks a seeded sample of tokens plus tokens routed to
    rows beyond 4 GiB (tokens are independent, so a sub-batch of the oracle is exact)."""
    T, H, K = 17000, 16384, 8
    inp = make_inputs_on_device(T, H, K, seed=7000 + T, device="cuda")
    _say(f"case rows beyond 4 GiB: T={T} H={H} K={K} seed={inp.seed} "
         f"rows {inp.rows.numel() * 2 / 1e9:.2f} GB")
    assert inp.rows.numel() * 2 > (1 << 32)
    d = to_dev(inp)
    s = run_finalize(inp, d)
    ro, no = run_rmsnorm(inp, d, use_ws=True)
    idx = inp.idx.cpu().numpy()
    far_row = (1 << 32) // (2 * H)
    far = np.flatnonzero((idx >= far_row).any(axis=1))
    rng = np.random.default_rng(inp.seed)
    pick = np.unique(np.concatenate([rng.choice(T, 48, replace=False), far[:16], [0, T - 1]]))
    assert (idx[pick] >= far_row).any()
    sub_idx = idx[pick]
    used = np.unique(sub_idx[sub_idx >= 0])
    remap = np.where(sub_idx >= 0, np.searchsorted(used, np.maximum(sub_idx, 0)), -1)
    rows_used = torch.as_tensor(used, device="cuda")
    sub = MoeInputs(T=len(pick), H=H, K=K, n_rows=len(used), act_dtype="bf16", scale_dtype="fp32",
                    seed=inp.seed, rows=inp.rows[rows_used].cpu(),
                    idx=torch.from_numpy(remap.astype(np.int32)),
                    scales=inp.scales.cpu()[pick], shared=inp.shared.cpu()[pick],
                    residual=inp.residual.cpu()[pick], gamma=inp.gamma.cpu(), rsf=inp.rsf,
                    eps=inp.eps)
    ref = oracle_ref(sub)
    sel = torch.as_tensor(pick, device="cuda")
    _say("  ", check_finalize(np64(s[sel]), ref, "bf16"))
    R, N = np64(ro[sel]), np64(no[sel])
    _say("  ", check_residual(R, ref, np64(sub.residual), "bf16"))
    _say("  ", check_norm(N, R, ref, np64(sub.gamma), inp.eps, "bf16"))


# ---- residual + RMSNorm of a given activation (moe_residual_rmsnorm_run) -------------------------
def run_residual_rmsnorm(x, residual, gamma, eps, use_ws=True, inplace=False):
    T, H = x.shape
    no = torch.empty_like(x)
    ro = residual if inplace else torch.empty_like(x)
    ws = workspace(T) if use_ws else None
    M.moe_residual_rmsnorm_run(x, residual, gamma, eps, ro, no, ws)
    torch.cuda.synchronize()
    assert ws_flag() == 0, "a split row timed out waiting for its slices"
    return ro, no


def _norm_within_1ulp(got_N, want_N, act):
    fmt = O.FORMATS[act]
    ud = ulp_distance(O.encode_bits(got_N, fmt), O.encode_bits(want_N, fmt))
    assert ud.max() <= 1, (int(ud.max()), np.argwhere(ud > 1)[0])


@pytest.mark.parametrize("act", ["bf16", "fp16"])
@pytest.mark.parametrize("TH", [(1, 6144), (4, 1024), (37, 1032), (128, 7168), (300, 3584),
                                (2, 16384), (5, 8), (1030, 7168)])
def test_residual_rmsnorm(TH, act):
    """r = RNE(x + residual) exactly (one float32 add of two activation values, rounded once,
    equals the single rounding of the exact sum); norm within 1 ulp of the oracle's."""
    T, H = TH
    inp = make_inputs(T, H, 1, act_dtype=act, seed=5000 + T + (100 if act == "fp16" else 0))
    _say(f"case residual_rmsnorm T={T} H={H} act={act} seed={inp.seed}")
    x, res, gam = (inp.shared.cuda(), inp.residual.cuda(), inp.gamma.cuda())
    R, N = O.residual_rmsnorm(np64(inp.shared), np64(inp.residual), np64(inp.gamma), inp.eps, act)
    outs = []
    for use_ws in (True, False):
        ro, no = run_residual_rmsnorm(x, res, gam, inp.eps, use_ws=use_ws)
        assert np.array_equal(np64(ro), R)
        _norm_within_1ulp(np64(no), N, act)
        outs.append((bits16(ro), bits16(no)))
    # deterministic, and the in-place residual update gives the same results
    ro2, no2 = run_residual_rmsnorm(x, res, gam, inp.eps)
    assert np.array_equal(bits16(ro2), outs[0][0]) and np.array_equal(bits16(no2), outs[0][1])
    res_io = res.clone()
    ro3, no3 = run_residual_rmsnorm(x, res_io, gam, inp.eps, inplace=True)
    assert ro3.data_ptr() == res_io.data_ptr()
    assert np.array_equal(bits16(res_io), outs[0][0]) and np.array_equal(bits16(no3), outs[0][1])


@pytest.mark.parametrize("THK", [(4, 1024, 8), (128, 7168, 8), (16, 2048, 22)])
def test_two_kernel_path_matches_oracle(THK):
    """moe_finalize_run followed by moe_residual_rmsnorm_run meets the same bars as the fused
    moe_finalize_rmsnorm_run against the oracle."""
    T, H, K = THK
    inp = make_inputs(T, H, K, seed=workload_seed("larger", T) + 7 * K)
    _say(f"case two-kernel T={T} H={H} K={K} seed={inp.seed}")
    ref = oracle_ref(inp)
    d = to_dev(inp)
    s = run_finalize(inp, d)
    check_finalize(np64(s), ref, "bf16")
    ro, no = run_residual_rmsnorm(s, d["residual"], d["gamma"], inp.eps)
    R, N = np64(ro), np64(no)
    check_residual(R, ref, np64(inp.residual), "bf16")
    check_norm(N, R, ref, np64(inp.gamma), inp.eps, "bf16")
    # on this finalize's own rounded output the second kernel is exact in residual_out
    R2, N2 = O.residual_rmsnorm(np64(s), np64(inp.residual), np64(inp.gamma), inp.eps, "bf16")
    assert np.array_equal(R, R2)
    _norm_within_1ulp(N, N2, "bf16")


@pytest.mark.parametrize("act", ["bf16", "fp16"])
def test_two_kernel_path_equals_fused_when_exact(act):
    """Dyadic inputs (every float32 operation exact): the fused kernel and the two-kernel path
    write the same residual_out bit for bit, and norms within 1 ulp of each other."""
    inp = _dyadic_inputs(16, 2048 if act == "bf16" else 1024, 22, act, seed=95)
    d = to_dev(inp)
    ro_f, no_f = run_rmsnorm(inp, d)
    s = run_finalize(inp, d)
    ro_2, no_2 = run_residual_rmsnorm(s, d["residual"], d["gamma"], inp.eps)
    assert np.array_equal(bits16(ro_f), bits16(ro_2))
    _norm_within_1ulp(np64(no_2), np64(no_f), act)


def _stream_fold(src, rb, wb, lanes):
    """Documented content of the stream kernels: chunk j of dst is the XOR of the source chunks c
    with c % lanes == j % lanes."""
    chunks = src.numpy().view(np.uint32).reshape(-1, 4)[: rb // 16]
    fold = np.zeros((lanes, 4), dtype=np.uint32)
    for start in range(0, len(chunks), lanes):
        part = chunks[start:start + lanes]
        fold[: len(part)] ^= part
    return fold[np.arange(wb // 16) % lanes]


@pytest.mark.parametrize("rb,wb", [(16 * 1000, 16 * 300), (14_680_064, 3_670_016),
                                   (16 * 5 * 262144 + 48, 16 * 70000), (0, 4096), (4096, 0)])
def test_stream_floor_writes_documented_fold(rb, wb):
    """The streaming-ceiling kernel (a measurement aid) writes exactly its documented content and
    nothing past write_bytes."""
    _say(f"stream floor read {rb} write {wb}")
    g = torch.Generator().manual_seed(rb + wb)
    src = torch.randint(0, 2 ** 31, (max(rb, 16) // 4,), generator=g, dtype=torch.int32)
    dst = torch.full(((wb + 4096) // 4,), -7, dtype=torch.int32)
    sd, dd = src.cuda(), dst.cuda()
    M.moe_finalize_stream_floor_run(sd, rb, dd, wb)
    torch.cuda.synchronize()
    got = dd.cpu().numpy()
    n_wr = wb // 16
    want = _stream_fold(src, rb, wb, 1024 * 512)
    assert np.array_equal(got[: n_wr * 4].view(np.uint32).reshape(-1, 4), want)
    assert np.all(got[n_wr * 4:] == -7)


@pytest.mark.parametrize("loads,lanes,grid,nt", [(1, 64, 3, 0), (16, 1024, 5, 1), (4, 256, 1000, 1),
                                                 (8, 512, 7, 0), (2, 128, 256, 1)])
def test_stream_probe_writes_documented_fold(loads, lanes, grid, nt):
    """The stream probe at other launch shapes (several rounds per lane, partial rounds, more
    lanes than chunks): documented content, nothing past write_bytes; bad shapes are refused."""
    rb, wb = 16 * 70001, 16 * 5003
    _say(f"stream probe loads {loads} lanes {lanes} grid {grid} nt {nt}")
    g = torch.Generator().manual_seed(loads * 1000 + grid)
    src = torch.randint(0, 2 ** 31, (rb // 4,), generator=g, dtype=torch.int32)
    dst = torch.full(((wb + 4096) // 4,), -7, dtype=torch.int32)
    sd, dd = src.cuda(), dst.cuda()
    M.moe_finalize_stream_probe_run(sd, rb, dd, wb, loads, lanes, grid, bool(nt))
    torch.cuda.synchronize()
    got = dd.cpu().numpy()
    want = _stream_fold(src, rb, wb, lanes * grid)
    assert np.array_equal(got[: wb // 4].view(np.uint32).reshape(-1, 4), want)
    assert np.all(got[wb // 4:] == -7)
    for bad in ((3, lanes, grid), (loads, 96, grid), (loads, lanes, 0), (16, 1024, 65536)):
        with pytest.raises(M.MoeFinalizeError):
            M.moe_finalize_stream_probe_run(sd, rb, dd, wb, *bad)


# ---- cancellation / high dynamic range (float32 accumulation, rounded once) -----------------------
def _cancelling_inputs(T, H, act, seed):
    """Per token: three pairs of large routed terms (+x, -x, equal weights) that cancel exactly,
    one small route, one absent route, in a random route order (partners may land in different
    route groups). Large terms are m * 2^5 (|m| <= 127, up to 2^12), small ones m * 2^-4 with
    weight 1/2, shared m * 2^-3, RSF 2: every partial sum of any float32 order spans at most 21
    significant bits, so the kernel's float32 value before its one rounding is exactly S*; per-step
    rounding to the activation dtype loses the small terms next to the large ones."""
    K = 8
    rng = np.random.Generator(np.random.PCG64(seed))
    n_rows = T * K
    inp = make_inputs(T, H, K, seed=seed, act_dtype=act, n_rows=n_rows)
    dt = ACT_T[act]
    rows = np.zeros((n_rows, H), dtype=np.float32)
    idx = np.full((T, K), -1, dtype=np.int32)
    sc = np.zeros((T, K), dtype=np.float32)
    nxt = 0
    for t in range(T):
        slots = rng.permutation(K)
        for p in range(3):
            big = rng.integers(-127, 128, H).astype(np.float32) * 32.0
            w = float(np.ldexp(1.0, int(rng.integers(-1, 1))))
            for sign, k in ((1.0, slots[2 * p]), (-1.0, slots[2 * p + 1])):
                rows[nxt] = sign * big
                idx[t, k] = nxt
                sc[t, k] = w
                nxt += 1
        rows[nxt] = rng.integers(-127, 128, H).astype(np.float32) / 16.0
        idx[t, slots[6]] = nxt
        sc[t, slots[6]] = 0.5
        nxt += 1
        sc[t, slots[7]] = 0.25               # absent route: its weight must not matter
    inp.rows = torch.from_numpy(rows).to(dt)
    inp.idx = torch.from_numpy(idx)
    inp.scales = torch.from_numpy(sc)
    inp.shared = torch.from_numpy(rng.integers(-64, 65, (T, H)).astype(np.float32) / 8.0).to(dt)
    inp.rsf = 2.0
    return inp


@pytest.mark.parametrize("act", ["bf16", "fp16"])
@pytest.mark.parametrize("TH", [(5, 1032), (64, 7168)])
def test_cancellation_high_dynamic_range_bit_exact(TH, act):
    T, H = TH
    inp = _cancelling_inputs(T, H, act, seed=600 + T)
    ref = oracle_ref(inp)
    fmt = O.FORMATS[act]
    # the fixture separates the two numerics: per-step rounding misses the small terms
    old = O.finalize_per_step_rounding(np64(inp.rows), inp.idx.numpy(), np64(inp.scales),
                                       np64(inp.shared), inp.rsf, act)
    assert np.mean(old != ref.s) > 0.3
    s = run_finalize(inp)
    assert np.array_equal(bits16(s), O.encode_bits(ref.s, fmt).astype(np.int64))
    for use_ws in (True, False):
        ro, no = run_rmsnorm(inp, use_ws=use_ws)
        assert np.array_equal(bits16(ro), O.encode_bits(ref.R, fmt).astype(np.int64))
        check_norm(np64(no), np64(ro), ref, np64(inp.gamma), inp.eps, act)


# ---- every output stays inside its buffer; inputs are never written -----------------------------
GUARD = 4096


def _guarded(nbytes, dtype, shape):
    """A view of `shape` inside a buffer with GUARD bytes of 0x5A before and after it."""
    full = torch.full((GUARD + nbytes + GUARD,), 0x5A, dtype=torch.uint8, device="cuda")
    return full, full[GUARD:GUARD + nbytes].view(dtype).view(shape)


def _guards_intact(full):
    g = full.cpu().numpy()
    return bool((g[:GUARD] == 0x5A).all() and (g[-GUARD:] == 0x5A).all())


@pytest.mark.parametrize("THK", [(5, 1032, 8), (37, 7168, 8), (130, 2048, 22), (3, 48, 6), (5, 4096, 8),
                                 (1, 6144, 8)])
def test_outputs_stay_in_bounds_and_inputs_untouched(THK):
    T, H, K = THK
    _say(f"guards T={T} H={H} K={K}")
    inp = make_inputs(T, H, K, seed=700 + T)
    d = to_dev(inp)
    before = {k: v.clone() for k, v in d.items() if v is not None}
    tb = T * H * 2
    ws_full, ws = _guarded(M.moe_finalize_workspace_size(T, H, K), torch.uint8, (-1,))
    ws.zero_()
    outs = []

    def new(nbytes, dtype, shape):
        full, view = _guarded(nbytes, dtype, shape)
        outs.append(full)
        return view

    M.moe_finalize_run(d["rows"], d["idx"], d["scales"], d["shared"], inp.rsf,
                       new(tb, torch.bfloat16, (T, H)))
    for w in (ws, None):
        M.moe_finalize_rmsnorm_run(d["rows"], d["idx"], d["scales"], d["shared"], inp.rsf,
                                   d["residual"], d["gamma"], inp.eps,
                                   new(tb, torch.bfloat16, (T, H)),
                                   new(tb, torch.bfloat16, (T, H)), w)
    qs = torch.tensor([3.0], dtype=torch.float32, device="cuda")
    x = torch.randn(T, H, device="cuda").to(torch.bfloat16)
    for layout in ((M.MOE_SF_SWIZZLED_128x4, M.MOE_SF_LINEAR) if H % 16 == 0 else ()):
        sfb = M.moe_finalize_sf_size(T, H, layout)
        M.moe_finalize_quant_run(d["rows"], d["idx"], d["scales"], d["shared"], inp.rsf,
                                 d["residual"], d["gamma"], inp.eps, M.MOE_QUANT_NVFP4, qs,
                                 new(tb // 4, torch.uint8, (T, H // 2)),
                                 new(sfb, torch.uint8, (-1,)), layout,
                                 new(tb, torch.bfloat16, (T, H)), new(tb, torch.bfloat16, (T, H)),
                                 ws)
        M.moe_quantize_run(x, M.MOE_QUANT_NVFP4, qs, new(tb // 4, torch.uint8, (T, H // 2)),
                           new(sfb, torch.uint8, (-1,)), layout)
    M.moe_finalize_quant_run(d["rows"], d["idx"], d["scales"], d["shared"], inp.rsf,
                             d["residual"], d["gamma"], inp.eps, M.MOE_QUANT_FP8_E4M3, qs,
                             new(tb // 2, torch.uint8, (T, H)), None, 0,
                             new(tb, torch.bfloat16, (T, H)), None, ws)
    M.moe_quantize_run(x, M.MOE_QUANT_FP8_E4M3, qs, new(tb // 2, torch.uint8, (T, H)), None, 0)
    M.moe_residual_rmsnorm_run(x, d["residual"], d["gamma"], inp.eps,
                               new(tb, torch.bfloat16, (T, H)), new(tb, torch.bfloat16, (T, H)),
                               ws)
    torch.cuda.synchronize()
    assert all(_guards_intact(f) for f in outs)
    assert _guards_intact(ws_full) and int(ws[:4].view(torch.int32).item()) == 0
    for k, v in before.items():
        assert torch.equal(d[k], v), k


def test_split_row_timeout_is_flagged_poisoned_and_bounded():
    """Failure detection of the split-row exchange, forced from the host: with a wait limit of 0
    polls every slice of a split row gives up at once, without waiting. Each sets the sticky flag
    in the workspace header and counts the partials it did not see as NaN, so norm_out and the
    quantized outputs come out NaN (FP8 code 0x7F; NVFP4 block scale 0x7F, codes 0) while
    residual_out is still exact; every call completes. The workspace needs no reset: with the
    default limit the next call on the same workspace is correct again (the flag stays set until
    the caller clears it)."""
    inp = make_inputs(1, 2048, 8, seed=800)          # T=1, hidden 2048: two slices per row
    assert M.moe_finalize_launch_config(1, 1, 2048, 8)["slices"] == 2
    assert M.moe_finalize_launch_config(2, 1, 2048, 8)["slices"] == 2
    d = to_dev(inp)
    ref = oracle_ref(inp)
    ws = torch.zeros(M.moe_finalize_workspace_size(1, 2048, 8), dtype=torch.uint8, device="cuda")
    ro = torch.empty(1, 2048, dtype=torch.bfloat16, device="cuda")
    no = torch.empty_like(ro)
    q8 = torch.zeros(1, 2048, dtype=torch.uint8, device="cuda")
    q4 = torch.full((1, 1024), 0xAB, dtype=torch.uint8, device="cuda")
    lay = M.MOE_SF_SWIZZLED_128x4
    sf = torch.full((M.moe_finalize_sf_size(1, 2048, lay),), 0xCD, dtype=torch.uint8,
                    device="cuda")
    qs = torch.tensor([100.0], dtype=torch.float32, device="cuda")
    _say("forcing split-row timeouts with a wait limit of 0 polls")
    prev = M.moe_finalize_set_wait_limit(0)
    try:
        assert prev == 1 << 22
        M.moe_finalize_rmsnorm_run(d["rows"], d["idx"], d["scales"], d["shared"], inp.rsf,
                                   d["residual"], d["gamma"], inp.eps, ro, no, ws)
        torch.cuda.synchronize()
        assert int(ws[:4].view(torch.int32).item()) == 1
        assert M.moe_finalize_workspace_flag(ws) == 1
        check_residual(np64(ro), ref, np64(inp.residual), "bf16")
        assert torch.isnan(no.float()).all()
        ro2 = torch.empty_like(ro)
        M.moe_finalize_quant_run(d["rows"], d["idx"], d["scales"], d["shared"], inp.rsf,
                                 d["residual"], d["gamma"], inp.eps, M.MOE_QUANT_FP8_E4M3, qs,
                                 q8, None, 0, ro2, None, ws)
        M.moe_finalize_quant_run(d["rows"], d["idx"], d["scales"], d["shared"], inp.rsf,
                                 d["residual"], d["gamma"], inp.eps, M.MOE_QUANT_NVFP4, qs, q4,
                                 sf, lay, None, None, ws)
        torch.cuda.synchronize()
        assert torch.equal(ro2, ro)
        assert (q8 == 0x7F).all()
        assert (q4 == 0).all()
        offs = _sf_offsets(1, 2048, lay).ravel()
        sfh = sf.cpu().numpy()
        assert (sfh[offs] == 0x7F).all()
        pad = np.ones(sfh.size, bool)
        pad[offs] = False
        assert not sfh[pad].any()
    finally:
        assert M.moe_finalize_set_wait_limit(-1) == 0
    assert M.moe_finalize_set_wait_limit(-1) == 1 << 22
    # every slot of the token advanced once per call
    slot_epochs = (ws[256:256 + 128].view(torch.int64).cpu() >> 32).numpy()
    assert (slot_epochs == 3).all(), slot_epochs
    for clear_flag in (False, True):
        if clear_flag:
            assert M.moe_finalize_workspace_flag(ws, clear=True) == 1
            assert M.moe_finalize_workspace_flag(ws) == 0
        M.moe_finalize_rmsnorm_run(d["rows"], d["idx"], d["scales"], d["shared"], inp.rsf,
                                   d["residual"], d["gamma"], inp.eps, ro, no, ws)
        torch.cuda.synchronize()
        assert int(ws[:4].view(torch.int32).item()) == (0 if clear_flag else 1)
        check_residual(np64(ro), ref, np64(inp.residual), "bf16")
        check_norm(np64(no), np64(ro), ref, np64(inp.gamma), inp.eps, "bf16")


def test_split_row_epochs_are_per_token():
    """The exchange words of a split row: after calls with different slice counts on one
    workspace, all 16 slots of each token carry one epoch, the number of split calls that touched
    the token, and slot j < S of the last call holds slice j's partial."""
    ws = workspace(64)
    ws.zero_()
    seq = [(1, 2048, 8), (4, 7168, 8), (1, 6144, 8), (64, 7168, 8), (1, 2048, 8)]
    count = {}
    for T, H, K in seq:
        inp = make_inputs(T, H, K, seed=810 + T + H)
        S = M.moe_finalize_launch_config(1, T, H, K)["slices"]
        assert S > 1
        ro, no = run_rmsnorm(inp)
        ref = oracle_ref(inp)
        check_norm(np64(no), np64(ro), ref, np64(inp.gamma), inp.eps, "bf16")
        for t in range(T):
            count[t] = count.get(t, 0) + 1
    blocks = ws[256:256 + 64 * 128].view(64, 16, 8).cpu()
    words = blocks.view(torch.int64).view(64, 16).numpy()
    for t, n in count.items():
        assert ((words[t] >> 32) == n).all(), (t, words[t] >> 32, n)
    # the last call (T=1, hidden 2048: two slices): the slices' partials sum to the row's sum of
    # squares of residual_out, and slots 2..15 carry no partial
    parts = (words[0] & 0xFFFFFFFF).astype(np.uint32).view(np.float32)
    R = np64(ro)
    assert abs(float(parts[0]) + float(parts[1]) - float((R * R).sum())) <= 1e-4 * float((R * R).sum())
    assert not parts[2:].any()


# ---- one GPU's share of the cross-rank reduction (moe_rank_sum_*_run) -----------------------------
def _rank_sum_inputs(T, H, W, act, seed):
    """W ranks' rounded finalize partials [W, T, H] (N(0,1) -> act), residual, gamma; expressed
    as a finalize problem whose routes are the ranks (row r*T + t, weight 1, RSF 1, no shared),
    which is how the oracle states the float32 rank sum rounded once."""
    inp = make_inputs(T, H, W, act_dtype=act, seed=seed, mask_frac=0.0, scale_dtype=None,
                      with_shared=False)
    inp.idx = torch.arange(W, dtype=torch.int32).view(1, W) * T + \
        torch.arange(T, dtype=torch.int32).view(T, 1)
    inp.rsf = 1.0
    return inp


@pytest.mark.parametrize("act", ["bf16", "fp16"])
@pytest.mark.parametrize("TWH", [(1, 4, 6144), (16, 4, 6144), (64, 4, 7168), (128, 4, 7168),
                                 (128, 8, 7168), (5, 2, 1032), (3, 1, 48), (300, 8, 2048),
                                 (1030, 4, 5120)])
def test_rank_sum_rmsnorm(TWH, act):
    T, W, H = TWH
    inp = _rank_sum_inputs(T, H, W, act, seed=6000 + T + 10 * W)
    _say(f"case rank_sum T={T} W={W} H={H} act={act} seed={inp.seed}")
    ref = oracle_ref(inp)
    parts = np64(inp.rows).reshape(W, T, H)
    assert np.array_equal(O.rank_sum_rounded(list(parts), act), ref.s)   # the two oracle forms agree
    P_ = inp.rows.view(W, T, H).cuda()
    res, gam = inp.residual.cuda(), inp.gamma.cuda()
    outs = []
    for use_ws in (True, False):
        ro = torch.empty(T, H, dtype=ACT_T[act], device="cuda")
        no = torch.empty_like(ro)
        M.moe_rank_sum_rmsnorm_run(P_, res, gam, inp.eps, ro, no, workspace(T) if use_ws else None)
        torch.cuda.synchronize()
        assert ws_flag() == 0
        R, N = np64(ro), np64(no)
        _say("  ", check_residual(R, ref, np64(inp.residual), act))
        _say("  ", check_norm(N, R, ref, np64(inp.gamma), inp.eps, act))
        outs.append(bits16(ro))
    assert np.array_equal(outs[0], outs[1])          # residual_out does not depend on the split


@pytest.mark.parametrize("act", ["bf16", "fp16"])
def test_rank_sum_dyadic_bit_exact(act):
    """Integer partials: the float32 rank sum is exact, so residual_out matches bit for bit."""
    T, W, H = 33, 8, 2048
    rng = np.random.Generator(np.random.PCG64(6100))
    inp = _rank_sum_inputs(T, H, W, act, seed=6101)
    inp.rows = torch.from_numpy(rng.integers(-64, 65, (W * T, H)).astype(np.float32)).to(ACT_T[act])
    inp.residual = torch.from_numpy(rng.integers(-64, 65, (T, H)).astype(np.float32)).to(ACT_T[act])
    ref = oracle_ref(inp)
    ro = torch.empty(T, H, dtype=ACT_T[act], device="cuda")
    no = torch.empty_like(ro)
    M.moe_rank_sum_rmsnorm_run(inp.rows.view(W, T, H).cuda(), inp.residual.cuda(),
                               inp.gamma.cuda(), inp.eps, ro, no, workspace(T))
    torch.cuda.synchronize()
    assert np.array_equal(np64(ro), ref.R)
    check_norm(np64(no), np64(ro), ref, np64(inp.gamma), inp.eps, act)


@pytest.mark.parametrize("TH", [(64, 6144), (100, 7168)])
@pytest.mark.parametrize("qt", [M.MOE_QUANT_NVFP4, M.MOE_QUANT_FP8_E4M3])
def test_rank_sum_quant(qt, TH):
    """Rank sum + residual + RMSNorm + quantization: codes and scales bit-exact against the
    oracle's quantization of the kernel's own norm_out (which meets the norm_out bar). At 100
    tokens and four partials the quantized call splits rows where plain RMSNorm takes whole rows,
    and the swizzled scales have padding rows."""
    T, H = TH
    W = 4
    inp = _rank_sum_inputs(T, H, W, "bf16", seed=6200 + T)
    ref = oracle_ref(inp)
    P_ = inp.rows.view(W, T, H).cuda()
    nv = qt == M.MOE_QUANT_NVFP4
    scale = O.nvfp4_global_scale(ref.N) if nv else O.fp8_scale(ref.N)
    qs = torch.tensor([scale], dtype=torch.float32, device="cuda")
    ro = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    no = torch.empty_like(ro)
    qo = torch.empty(T, H // 2 if nv else H, dtype=torch.uint8, device="cuda")
    so = torch.empty(M.moe_finalize_sf_size(T, H, M.MOE_SF_SWIZZLED_128x4), dtype=torch.uint8,
                     device="cuda") if nv else None
    M.moe_rank_sum_quant_run(P_, inp.residual.cuda(), inp.gamma.cuda(), inp.eps, qt, qs, qo, so,
                             M.MOE_SF_SWIZZLED_128x4, ro, no, workspace(T))
    torch.cuda.synchronize()
    R, N = np64(ro), np64(no)
    check_residual(R, ref, np64(inp.residual), "bf16")
    check_norm(N, R, ref, np64(inp.gamma), inp.eps, "bf16")
    if nv:
        want_c, want_s = O.quant_nvfp4(N, scale, M.MOE_SF_SWIZZLED_128x4)
        assert np.array_equal(qo.cpu().numpy(), want_c)
        assert np.array_equal(so.cpu().numpy(), want_s)
    else:
        assert np.array_equal(qo.cpu().numpy(), O.quant_fp8(N, scale))


def test_every_entry_point_replays_in_a_graph():
    """Each entry point captured in a HIP graph (with the shared workspace where it takes one),
    replayed three times with eager work and synchronizations between the replays: every replay
    equals the eager call bit for bit (the workspace needs no reset between replays)."""
    T, H, K = 48, 2048, 8
    inp = make_inputs(T, H, K, seed=900)
    d = to_dev(inp)
    ws = torch.zeros(M.moe_finalize_workspace_size(T, H, K), dtype=torch.uint8, device="cuda")
    qs_nv = torch.tensor([20.0], dtype=torch.float32, device="cuda")
    qs_f8 = torch.tensor([30.0], dtype=torch.float32, device="cuda")
    parts = torch.randn(4, T, H, device="cuda").to(torch.bfloat16)
    x = torch.randn(T, H, device="cuda").to(torch.bfloat16)
    bf = lambda: torch.empty(T, H, dtype=torch.bfloat16, device="cuda")  # noqa: E731
    u8 = lambda n: torch.empty(n, dtype=torch.uint8, device="cuda")      # noqa: E731
    sfb = M.moe_finalize_sf_size(T, H, M.MOE_SF_SWIZZLED_128x4)
    o = {k: bf() for k in ("fin", "ro", "no", "qro", "rsro", "rsno", "rrro", "rrno")}
    o.update(qnv=u8(T * H // 2).view(T, H // 2), sfnv=u8(sfb), qf8=u8(T * H).view(T, H),
             qz=u8(T * H // 2).view(T, H // 2), sfz=u8(sfb))
    calls = [
        lambda s: M.moe_finalize_run(d["rows"], d["idx"], d["scales"], d["shared"], inp.rsf,
                                     o["fin"], stream=s),
        lambda s: M.moe_finalize_rmsnorm_run(d["rows"], d["idx"], d["scales"], d["shared"],
                                             inp.rsf, d["residual"], d["gamma"], inp.eps, o["ro"],
                                             o["no"], ws, stream=s),
        lambda s: M.moe_finalize_quant_run(d["rows"], d["idx"], d["scales"], d["shared"], inp.rsf,
                                           d["residual"], d["gamma"], inp.eps, M.MOE_QUANT_NVFP4,
                                           qs_nv, o["qnv"], o["sfnv"], M.MOE_SF_SWIZZLED_128x4,
                                           o["qro"], None, ws, stream=s),
        lambda s: M.moe_finalize_quant_run(d["rows"], d["idx"], d["scales"], d["shared"], inp.rsf,
                                           d["residual"], d["gamma"], inp.eps,
                                           M.MOE_QUANT_FP8_E4M3, qs_f8, o["qf8"], None, 0, None,
                                           None, ws, stream=s),
        lambda s: M.moe_rank_sum_rmsnorm_run(parts, d["residual"], d["gamma"], inp.eps, o["rsro"],
                                             o["rsno"], ws, stream=s),
        lambda s: M.moe_residual_rmsnorm_run(x, d["residual"], d["gamma"], inp.eps, o["rrro"],
                                             o["rrno"], ws, stream=s),
        lambda s: M.moe_quantize_run(x, M.MOE_QUANT_NVFP4, qs_nv, o["qz"], o["sfz"],
                                     M.MOE_SF_SWIZZLED_128x4, stream=s),
    ]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for c in calls:
            c(s)
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in o.items()}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for c in calls:
            c(s)
    for rep in range(3):
        for v in o.values():
            v.zero_()
        torch.randn(1 << 20, device="cuda").sum().item()      # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in o.items():
            assert torch.equal(v, eager[k]), (rep, k)
    assert int(ws[:4].view(torch.int32).item()) == 0
