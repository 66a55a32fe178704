"""Seeded synthetic inputs shaped like the decode workloads of the MoE finalize pages.

Sources (the pages this repository follows; cited by key everywhere in the code):
  [FI6631]  flashinfer PR #6631, "perf(comm): gather MoE-finalize routes together and accumulate in
            FP32" (the fused finalize + all-reduce + residual + RMSNorm kernel, its tests and bench).
  [TR16778] TensorRT-LLM PR #16778, "MoE: fp32 accumulation in deferred MoEAllReduce finalize".
  [FI6546]  flashinfer PR #6546, the small-batch trtllm-gen MoE finalize (finalizeKernelSmallBatch).
  [FI3385]  flashinfer PR #3385, "feat: MNNVL Allreduce quant fusion and performance optimization".

What is drawn, and why (no finalize arithmetic lives here):
  * permuted expert-GEMM output rows X[n_rows, H] ~ N(0,1) (times `row_scale`), rounded to the
    activation dtype by torch's float32 -> bf16/fp16 conversion. [FI6631, benchmark script] draws
    its GEMM2 rows the same way (there with a 0.5 factor and n_rows = 2*T*K + 8).
  * expanded_idx_to_permuted_idx [T, K] int32: a seeded random choice of distinct permuted rows,
    with exactly floor(mask_frac * T * K) seeded positions set to -1. [FI6631, Description / test
    changes] masks a quarter of the routes with -1; "a quarter" is read as that exact count.
  * expert scales [T, K]: softmax over K of N(0,1) logits, evaluated in float64, delivered as
    float32 or bfloat16 ([FI6546, Performance] sweeps bf16 and fp32 expert weights). The softmax
    covers masked routes too, so the weights of the valid routes sum to less than one.
  * shared-expert output and residual [T, H] ~ N(0,1) (times their scales); gamma = 1 + 0.1*N(0,1).

Random numbers come from numpy's PCG64 generator seeded with an explicit integer, so the same
seed gives the same inputs on every machine. Problems too large to draw on the host (gigabytes of
rows) come from make_inputs_on_device: the same distributions from torch's seeded generator on
the device.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

ACT_DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16}
SCALE_DTYPES = {"fp32": torch.float32, "bf16": torch.bfloat16}

# Seed bases per workload group. A case's seed is base + T (+ offsets for dtype / K variants), so
# every case of every group has its own stream.
_GROUP_BASE = {"tiny": 0, "decode": 1000, "larger": 2000, "highk": 3000, "quant": 4000,
               "batch": 5000, "ranksum": 6000}


def workload_seed(group: str, T: int, act_dtype: str = "bf16", scale_dtype: str = "fp32",
                  K: Optional[int] = None) -> int:
    """Deterministic seed of one synthetic case: group base + T, +100 for fp16 activations,
    +200 for bf16 scales, +10000*K when a K variant of a group is drawn."""
    s = _GROUP_BASE[group] + int(T)
    if act_dtype == "fp16":
        s += 100
    if scale_dtype == "bf16":
        s += 200
    if K is not None:
        s += 10000 * int(K)
    return s


@dataclass
class MoeInputs:
    """One synthetic finalize problem. Tensors live on the CPU; callers move them."""
    T: int
    H: int
    K: int
    n_rows: int
    act_dtype: str
    scale_dtype: Optional[str]
    seed: int
    rows: torch.Tensor                 # [n_rows, H] act dtype
    idx: torch.Tensor                  # [T, K] int32, -1 = no route
    scales: Optional[torch.Tensor]     # [T, K] fp32 / bf16, or None
    shared: Optional[torch.Tensor]     # [T, H] act dtype, or None
    residual: torch.Tensor             # [T, H] act dtype
    gamma: torch.Tensor                # [H] act dtype
    rsf: float = 2.5
    eps: float = 1e-6
    meta: dict = field(default_factory=dict)


def _to_act(a32: np.ndarray, act_dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32)).to(ACT_DTYPES[act_dtype])


def make_inputs(T: int, H: int, K: int, *, seed: int, act_dtype: str = "bf16",
                scale_dtype: Optional[str] = "fp32", n_rows: Optional[int] = None,
                mask_frac: float = 0.25, with_shared: bool = True, rsf: float = 2.5,
                eps: float = 1e-6, row_scale: float = 1.0, shared_scale: float = 1.0,
                residual_scale: float = 1.0) -> MoeInputs:
    """Draw one seeded problem. `n_rows` defaults to T*K (the routes then use a permutation of
    every permuted row); a larger value leaves rows that no route references."""
    if act_dtype not in ACT_DTYPES:
        raise ValueError(f"act_dtype {act_dtype!r}")
    if scale_dtype is not None and scale_dtype not in SCALE_DTYPES:
        raise ValueError(f"scale_dtype {scale_dtype!r}")
    n_rows = T * K if n_rows is None else int(n_rows)
    if n_rows < T * K:
        raise ValueError("n_rows must be >= T*K so every route can get a distinct row")
    rng = np.random.Generator(np.random.PCG64(seed))

    rows = _to_act(rng.standard_normal((n_rows, H), dtype=np.float32) * np.float32(row_scale),
                   act_dtype)
    perm = rng.permutation(n_rows)[: T * K].astype(np.int64)
    n_masked = int(np.floor(mask_frac * T * K))
    if n_masked:
        masked = rng.choice(T * K, size=n_masked, replace=False)
        perm[masked] = -1
    idx = torch.from_numpy(perm.reshape(T, K).astype(np.int32))

    scales = None
    if scale_dtype is not None:
        logits = rng.standard_normal((T, K))
        e = np.exp(logits - logits.max(axis=1, keepdims=True))
        sm = e / e.sum(axis=1, keepdims=True)
        scales = torch.from_numpy(sm.astype(np.float32)).to(SCALE_DTYPES[scale_dtype])

    shared = None
    if with_shared:
        shared = _to_act(rng.standard_normal((T, H), dtype=np.float32) * np.float32(shared_scale),
                         act_dtype)
    residual = _to_act(rng.standard_normal((T, H), dtype=np.float32) * np.float32(residual_scale),
                       act_dtype)
    gamma = _to_act(1.0 + 0.1 * rng.standard_normal(H, dtype=np.float32), act_dtype)
    return MoeInputs(T=T, H=H, K=K, n_rows=n_rows, act_dtype=act_dtype, scale_dtype=scale_dtype,
                     seed=seed, rows=rows, idx=idx, scales=scales, shared=shared,
                     residual=residual, gamma=gamma, rsf=float(rsf), eps=float(eps),
                     meta={"mask_frac": mask_frac, "n_masked": n_masked})


def make_inputs_on_device(T: int, H: int, K: int, *, seed: int, device, act_dtype: str = "bf16",
                          mask_frac: float = 0.25, rsf: float = 2.5,
                          eps: float = 1e-6) -> MoeInputs:
    """The distributions of make_inputs (fp32 scales, shared expert present, n_rows = T*K), drawn
    on `device` by torch's generator seeded with `seed`, for problems too large to draw on the
    host. The tensors stay on `device`; the draws differ from make_inputs' for the same seed."""
    if act_dtype not in ACT_DTYPES:
        raise ValueError(f"act_dtype {act_dtype!r}")
    dt = ACT_DTYPES[act_dtype]
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    n_rows = T * K
    rows = torch.empty(n_rows, H, dtype=dt, device=device)
    chunk = max(1, (1 << 27) // H)                 # 512 MB of float32 draws at a time
    for r0 in range(0, n_rows, chunk):
        r1 = min(n_rows, r0 + chunk)
        rows[r0:r1] = torch.randn(r1 - r0, H, generator=g, device=device).to(dt)
    perm = torch.randperm(n_rows, generator=g, device=device)
    n_masked = int(np.floor(mask_frac * T * K))
    if n_masked:
        perm[torch.randperm(T * K, generator=g, device=device)[:n_masked]] = -1
    idx = perm.reshape(T, K).to(torch.int32)
    logits = torch.randn(T, K, generator=g, device=device, dtype=torch.float64)
    scales = torch.softmax(logits, dim=1).to(torch.float32)
    shared = torch.randn(T, H, generator=g, device=device).to(dt)
    residual = torch.randn(T, H, generator=g, device=device).to(dt)
    gamma = (1.0 + 0.1 * torch.randn(H, generator=g, device=device)).to(dt)
    return MoeInputs(T=T, H=H, K=K, n_rows=n_rows, act_dtype=act_dtype, scale_dtype="fp32",
                     seed=seed, rows=rows, idx=idx, scales=scales, shared=shared,
                     residual=residual, gamma=gamma, rsf=float(rsf), eps=float(eps),
                     meta={"mask_frac": mask_frac, "n_masked": n_masked, "device": str(device)})
