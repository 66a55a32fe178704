"""The allocation-free entry point (moe_finalize_rmsnorm_noalloc_run): through the C ABI, two
calls in a row (the second on a smaller input) give the same bits as moe_finalize_rmsnorm_run with
a zero-filled workspace, and meet the oracle's bars; num_tokens above its static scratch's limit is
rejected before anything is enqueued; a forced split-row timeout sets the static scratch's flag,
which the host reads and clears through moe_finalize_workspace_flag."""
from __future__ import annotations

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("needs a GPU", allow_module_level=True)

import moe_expert_output_amd as M  # noqa: E402
from synth import make_inputs, workload_seed  # noqa: E402
from tests.parity import bits16, check_norm, check_residual, np64, oracle_ref, to_dev  # noqa: E402


def _both(inp):
    """(residual_out, norm_out) of the allocation-free call and of the workspace call."""
    d = to_dev(inp)
    outs = []
    for noalloc in (True, False):
        ro = torch.full((inp.T, inp.H), 7.0, dtype=torch.bfloat16, device="cuda")
        no = torch.full_like(ro, 7.0)
        args = (d["rows"], d["idx"], d["scales"], d["shared"], inp.rsf, d["residual"], d["gamma"],
                inp.eps, ro, no)
        if noalloc:
            M.moe_finalize_rmsnorm_noalloc_run(*args)
        else:
            ws = torch.zeros(M.moe_finalize_workspace_size(inp.T, inp.H, inp.K),
                             dtype=torch.uint8, device="cuda")
            M.moe_finalize_rmsnorm_run(*args, ws)
        torch.cuda.synchronize()
        outs.append((ro, no))
    return outs


def test_noalloc_matches_workspace_entry_on_two_calls():
    cases = [make_inputs(128, 7168, 8, seed=workload_seed("larger", 128)),   # 2 slices per row
             make_inputs(16, 6144, 8, seed=workload_seed("decode", 16))]     # smaller, 6 slices
    for inp in cases:
        print(f"noalloc case T={inp.T} H={inp.H} K={inp.K} seed={inp.seed} slices="
              f"{M.moe_finalize_launch_config(1, inp.T, inp.H, inp.K)['slices']}", flush=True)
        (ro_a, no_a), (ro_w, no_w) = _both(inp)
        assert np.array_equal(bits16(ro_a), bits16(ro_w))
        assert np.array_equal(bits16(no_a), bits16(no_w))
        ref = oracle_ref(inp)
        R, N = np64(ro_a), np64(no_a)
        check_residual(R, ref, np64(inp.residual), "bf16")
        check_norm(N, R, ref, np64(inp.gamma), inp.eps, "bf16")


def test_noalloc_whole_rows_and_limit():
    inp = make_inputs(300, 2048, 8, seed=909)                                 # whole rows
    (ro_a, no_a), (ro_w, no_w) = _both(inp)
    assert np.array_equal(bits16(ro_a), bits16(ro_w))
    assert np.array_equal(bits16(no_a), bits16(no_w))
    big = make_inputs(1025, 64, 1, seed=910)
    d = to_dev(big)
    ro = torch.full((1025, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    no = torch.full_like(ro, 7.0)
    with pytest.raises(M.MoeFinalizeError) as e:
        M.moe_finalize_rmsnorm_noalloc_run(d["rows"], d["idx"], d["scales"], d["shared"], big.rsf,
                                           d["residual"], d["gamma"], big.eps, ro, no)
    assert e.value.code == -13
    torch.cuda.synchronize()
    assert (ro.float() == 7.0).all() and (no.float() == 7.0).all()


def test_noalloc_scratch_flag_reads_and_clears():
    """Failure detection on the static scratch, forced from the host with a wait limit of 0 polls:
    norm_out comes out NaN, residual_out stays exact, the flag reads 1 and clears; the next call
    with the default limit is correct again without any reset of the scratch."""
    inp = make_inputs(1, 2048, 8, seed=911)                                  # 2 slices per row
    assert M.moe_finalize_launch_config(1, 1, 2048, 8)["slices"] == 2
    d = to_dev(inp)
    ref = oracle_ref(inp)
    ro = torch.empty(1, 2048, dtype=torch.bfloat16, device="cuda")
    no = torch.empty_like(ro)
    args = (d["rows"], d["idx"], d["scales"], d["shared"], inp.rsf, d["residual"], d["gamma"],
            inp.eps, ro, no)
    M.moe_finalize_rmsnorm_noalloc_run(*args)
    assert M.moe_finalize_workspace_flag() == 0
    print("noalloc: forcing split-row timeouts with a wait limit of 0 polls", flush=True)
    prev = M.moe_finalize_set_wait_limit(0)
    try:
        M.moe_finalize_rmsnorm_noalloc_run(*args)
        torch.cuda.synchronize()
    finally:
        assert M.moe_finalize_set_wait_limit(-1) == 0
    assert prev == 1 << 22
    check_residual(np64(ro), ref, np64(inp.residual), "bf16")
    assert torch.isnan(no.float()).all()
    assert M.moe_finalize_workspace_flag(clear=True) == 1
    assert M.moe_finalize_workspace_flag() == 0
    M.moe_finalize_rmsnorm_noalloc_run(*args)
    torch.cuda.synchronize()
    assert M.moe_finalize_workspace_flag() == 0
    check_residual(np64(ro), ref, np64(inp.residual), "bf16")
    check_norm(np64(no), np64(ro), ref, np64(inp.gamma), inp.eps, "bf16")
