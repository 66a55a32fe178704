"""Thin ctypes binding of libmoe_finalize.so (argument marshalling only).

Every function here has the name of the C entry point it calls and does nothing but pass
pointers, sizes, dtype codes and the current HIP stream of the tensors' device. All arithmetic
runs in the library's HIP kernels. If the library is not built, importing this module fails
loudly; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

from .build_lib import LIB_PATH

MOE_DTYPE_BF16, MOE_DTYPE_FP16, MOE_DTYPE_FP32 = 0, 1, 2
MOE_QUANT_NVFP4, MOE_QUANT_FP8_E4M3 = 1, 2
MOE_SF_LINEAR, MOE_SF_SWIZZLED_128x4 = 0, 1
MOE_FIN_CACHE_AUTO, MOE_FIN_CACHE_KEEP, MOE_FIN_CACHE_STREAM = 0, 1, 2

# Every symbol include/moe_finalize.h declares.
EXPORTED = ("moe_finalize_run", "moe_finalize_rmsnorm_run", "moe_finalize_quant_run",
            "moe_finalize_sf_size", "moe_finalize_error_string", "moe_finalize_version",
            "moe_finalize_launch_floor_run", "moe_finalize_workspace_size", "moe_quantize_run",
            "moe_residual_rmsnorm_run", "moe_finalize_stream_floor_run",
            "moe_rank_sum_rmsnorm_run", "moe_rank_sum_quant_run", "moe_finalize_launch_config",
            "moe_finalize_set_cache_policy", "moe_finalize_set_wait_limit",
            "moe_finalize_rmsnorm_noalloc_run", "moe_finalize_stream_probe_run",
            "moe_finalize_workspace_flag")

_ACT = {torch.bfloat16: MOE_DTYPE_BF16, torch.float16: MOE_DTYPE_FP16}
_SCALE = {torch.float32: MOE_DTYPE_FP32, torch.bfloat16: MOE_DTYPE_BF16}


class MoeFinalizeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{msg} (code {code})")
        self.code = code


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python moe_expert_output_amd/build_lib.py` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    lib.moe_finalize_run.argtypes = [vp, i64, vp, vp, i32, vp, f32, vp, i64, i64, i32, i32, vp]
    sz = ctypes.c_size_t
    lib.moe_finalize_rmsnorm_run.argtypes = [vp, i64, vp, vp, i32, vp, f32, vp, vp, f32, vp, vp,
                                             vp, sz, i64, i64, i32, i32, vp]
    lib.moe_finalize_rmsnorm_noalloc_run.argtypes = [vp, i64, vp, vp, i32, vp, f32, vp, vp, f32,
                                                     vp, vp, i64, i64, i32, i32, vp]
    lib.moe_finalize_rmsnorm_noalloc_run.restype = ctypes.c_int
    lib.moe_finalize_quant_run.argtypes = [vp, i64, vp, vp, i32, vp, f32, vp, vp, f32, i32, vp,
                                           vp, vp, i32, vp, vp, vp, sz, i64, i64, i32, i32, vp]
    lib.moe_quantize_run.argtypes = [vp, i64, i64, i32, i32, vp, vp, vp, i32, vp]
    lib.moe_quantize_run.restype = ctypes.c_int
    lib.moe_residual_rmsnorm_run.argtypes = [vp, vp, vp, f32, vp, vp, vp, sz, i64, i64, i32, vp]
    lib.moe_residual_rmsnorm_run.restype = ctypes.c_int
    lib.moe_finalize_workspace_size.argtypes = [i64, i64, i32]
    lib.moe_finalize_workspace_size.restype = sz
    for f in ("moe_finalize_run", "moe_finalize_rmsnorm_run", "moe_finalize_quant_run"):
        getattr(lib, f).restype = ctypes.c_int
    lib.moe_finalize_sf_size.argtypes = [i64, i64, i32]
    lib.moe_finalize_sf_size.restype = ctypes.c_size_t
    lib.moe_finalize_error_string.argtypes = [i32]
    lib.moe_finalize_error_string.restype = ctypes.c_char_p
    lib.moe_finalize_version.restype = ctypes.c_int
    lib.moe_finalize_launch_floor_run.argtypes = [i32, i64, i64, i32, vp]
    lib.moe_finalize_launch_floor_run.restype = ctypes.c_int
    lib.moe_finalize_launch_config.argtypes = [i32, i64, i64, i32, i32, i32,
                                               ctypes.POINTER(ctypes.c_int64), i32]
    lib.moe_finalize_launch_config.restype = ctypes.c_int
    lib.moe_finalize_set_cache_policy.argtypes = [i32]
    lib.moe_finalize_set_cache_policy.restype = ctypes.c_int
    lib.moe_finalize_set_wait_limit.argtypes = [i64]
    lib.moe_finalize_set_wait_limit.restype = i64
    lib.moe_finalize_stream_floor_run.argtypes = [vp, sz, vp, sz, vp]
    lib.moe_finalize_stream_floor_run.restype = ctypes.c_int
    lib.moe_finalize_stream_probe_run.argtypes = [vp, sz, vp, sz, i32, i32, i64, i32, vp]
    lib.moe_finalize_stream_probe_run.restype = ctypes.c_int
    lib.moe_finalize_workspace_flag.argtypes = [vp, i32, ctypes.POINTER(i32), vp]
    lib.moe_finalize_workspace_flag.restype = ctypes.c_int
    lib.moe_rank_sum_rmsnorm_run.argtypes = [vp, i32, vp, vp, f32, vp, vp, vp, sz, i64, i64, i32,
                                             vp]
    lib.moe_rank_sum_rmsnorm_run.restype = ctypes.c_int
    lib.moe_rank_sum_quant_run.argtypes = [vp, i32, vp, vp, f32, i32, vp, vp, vp, i32, vp, vp, vp,
                                           sz, i64, i64, i32, vp]
    lib.moe_rank_sum_quant_run.restype = ctypes.c_int
    return lib


LIB = _load()


def moe_finalize_error_string(code: int) -> str:
    return LIB.moe_finalize_error_string(int(code)).decode()


def moe_finalize_sf_size(num_tokens: int, hidden: int, sf_layout: int) -> int:
    return int(LIB.moe_finalize_sf_size(int(num_tokens), int(hidden), int(sf_layout)))


def moe_finalize_workspace_size(num_tokens: int, hidden: int, top_k: int) -> int:
    return int(LIB.moe_finalize_workspace_size(int(num_tokens), int(hidden), int(top_k)))


def _ws(workspace: Optional[torch.Tensor]):
    if workspace is None:
        return None, 0
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def moe_finalize_version() -> int:
    return int(LIB.moe_finalize_version())


def moe_finalize_launch_floor_run(entry: int, num_tokens: int, hidden: int, top_k: int,
                                  device=None, stream=None) -> None:
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    s = int(stream.cuda_stream if hasattr(stream, "cuda_stream") else stream) if stream is not None \
        else torch.cuda.current_stream(dev).cuda_stream
    _check(LIB.moe_finalize_launch_floor_run(int(entry), int(num_tokens), int(hidden), int(top_k),
                                             s))


LAUNCH_CONFIG_FIELDS = ("workgroups", "lanes", "slices", "route_groups", "slots_per_lane",
                        "slot_span", "lds_bytes", "nontemporal", "kernel_available")


def moe_finalize_launch_config(entry: int, num_tokens: int, hidden: int, top_k: int,
                               with_workspace: bool = True, num_cus: int = 0) -> dict:
    """The launch configuration entry point `entry` (0 finalize, 1 RMSNorm, 2 quantized) uses
    for a shape on a device of `num_cus` compute units (0: the current device's; host only;
    raises MoeFinalizeError with the entry point's code for a bad shape)."""
    out = (ctypes.c_int64 * len(LAUNCH_CONFIG_FIELDS))()
    _check(LIB.moe_finalize_launch_config(int(entry), int(num_tokens), int(hidden), int(top_k),
                                          1 if with_workspace else 0, int(num_cus), out,
                                          len(LAUNCH_CONFIG_FIELDS)))
    return dict(zip(LAUNCH_CONFIG_FIELDS, (int(v) for v in out)))


def moe_finalize_set_cache_policy(policy: int) -> int:
    """Set the process-wide cache policy for streamed tensors (MOE_FIN_CACHE_AUTO / _KEEP /
    _STREAM); returns the previous one."""
    prev = int(LIB.moe_finalize_set_cache_policy(int(policy)))
    if prev < 0:
        raise MoeFinalizeError(prev, moe_finalize_error_string(prev))
    return prev


def moe_finalize_set_wait_limit(polls: int) -> int:
    """Set the process-wide poll limit of split-row waits (< 0: the default); returns the
    previous limit."""
    return int(LIB.moe_finalize_set_wait_limit(int(polls)))


def moe_finalize_workspace_flag(workspace: Optional[torch.Tensor] = None, clear: bool = False,
                                stream=None) -> int:
    """The timeout flag of a workspace, or with workspace None of the current device's static
    scratch of moe_finalize_rmsnorm_noalloc_run (waits for the stream); clear resets it."""
    flag = ctypes.c_int(0)
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < 256:
            raise ValueError("workspace must hold at least its 256-byte header")
        s = _stream(workspace, stream)
    elif stream is not None:
        s = int(stream.cuda_stream if hasattr(stream, "cuda_stream") else stream)
    else:
        s = torch.cuda.current_stream().cuda_stream
    _check(LIB.moe_finalize_workspace_flag(_ptr(workspace), 1 if clear else 0, ctypes.byref(flag),
                                           s))
    return int(flag.value)


def moe_finalize_stream_floor_run(src: torch.Tensor, read_bytes: int, dst: torch.Tensor,
                                  write_bytes: int, stream=None) -> None:
    for t, n in ((src, read_bytes), (dst, write_bytes)):
        if n > t.numel() * t.element_size():
            raise ValueError("byte count exceeds the tensor")
    _check(LIB.moe_finalize_stream_floor_run(_ptr(src), int(read_bytes), _ptr(dst),
                                             int(write_bytes), _stream(dst, stream)))


def moe_finalize_stream_probe_run(src: torch.Tensor, read_bytes: int, dst: torch.Tensor,
                                  write_bytes: int, loads_per_round: int, workgroup_lanes: int,
                                  workgroups: int, nontemporal: bool = True, stream=None) -> None:
    for t, n in ((src, read_bytes), (dst, write_bytes)):
        if n > t.numel() * t.element_size():
            raise ValueError("byte count exceeds the tensor")
    _check(LIB.moe_finalize_stream_probe_run(_ptr(src), int(read_bytes), _ptr(dst),
                                             int(write_bytes), int(loads_per_round),
                                             int(workgroup_lanes), int(workgroups),
                                             1 if nontemporal else 0, _stream(dst, stream)))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be device (HIP) tensors")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr() or None


def _check(code: int) -> None:
    if code != 0:
        raise MoeFinalizeError(code, moe_finalize_error_string(code))


def _stream(ref: torch.Tensor, stream) -> int:
    if stream is not None:
        return int(stream.cuda_stream if hasattr(stream, "cuda_stream") else stream)
    return torch.cuda.current_stream(ref.device).cuda_stream


def _need(t: Optional[torch.Tensor], name: str, shape, dtype, optional: bool = False) -> None:
    """Shape and dtype guard. The C ABI sees only pointers and the sizes passed beside them, so a
    tensor smaller than the shape a call implies would be read or written past its end."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _need_bytes(t: Optional[torch.Tensor], name: str, nbytes: int, exact: bool) -> None:
    if t is None:
        return
    have = t.numel() * t.element_size()
    if (have != nbytes) if exact else (have < nbytes):
        raise ValueError(f"{name} must hold {'exactly' if exact else 'at least'} {nbytes} bytes, "
                         f"got {have}")


def _act_dtype(t: torch.Tensor, name: str):
    if t.dtype not in _ACT:
        raise ValueError(f"{name}: activation dtype {t.dtype} is not bf16/fp16")
    return t.dtype


def _common(rows, idx, scales, shared, H):
    """Route inputs of the finalize entry points: rows [N_rows, H], idx [T, K] int32, scales
    [T, K] fp32 or bf16 (or None), shared [T, H] (or None), all activations of rows' dtype."""
    dt = _act_dtype(rows, "permuted_rows")
    if rows.dim() != 2 or idx.dim() != 2:
        raise ValueError("permuted_rows must be [N_rows, H] and the index map [T, K]")
    T, K = idx.shape
    _need(rows, "permuted_rows", (rows.shape[0], H), dt)
    _need(idx, "expanded_idx_to_permuted_idx", (T, K), torch.int32)
    if scales is not None:
        if scales.dtype not in _SCALE:
            raise ValueError(f"expert_scales must be float32 or bfloat16, got {scales.dtype}")
        _need(scales, "expert_scales", (T, K), scales.dtype)
    _need(shared, "shared_expert_output", (T, H), dt, optional=True)
    sdt = _SCALE[scales.dtype] if scales is not None else MOE_DTYPE_FP32
    return _ACT[dt], sdt, T, K


def _rows_out(dt, T, H, residual, gamma, residual_out, norm_out, norm_optional=False):
    """The residual + RMSNorm tensors: residual, residual_out, norm_out [T, H]; gamma [H]."""
    _need(residual, "residual", (T, H), dt)
    _need(gamma, "gamma", (H,), dt)
    _need(residual_out, "residual_out", (T, H), dt, optional=True)
    _need(norm_out, "norm_out", (T, H), dt, optional=norm_optional)


def _quant_out(T, H, quant_type, quant_scale, quant_out, scale_out, sf_layout):
    """quant_scale: one float32; quant_out: T*H/2 (NVFP4) or T*H (FP8) bytes; scale_out (NVFP4):
    at least moe_finalize_sf_size(T, H, sf_layout) bytes."""
    if quant_scale is None or quant_scale.dtype != torch.float32 or quant_scale.numel() < 1:
        raise ValueError("quant_scale must be a device float32 tensor with one element")
    nv = int(quant_type) == MOE_QUANT_NVFP4
    if quant_out is None:
        raise ValueError("quant_out is required")
    if quant_out.element_size() != 1:
        raise ValueError(f"quant_out must be a byte tensor, got {quant_out.dtype}")
    _need_bytes(quant_out, "quant_out", T * H // 2 if nv else T * H, exact=True)
    if nv:
        if scale_out is None:
            raise ValueError("scale_out is required for NVFP4")
        _need_bytes(scale_out, "scale_out", int(LIB.moe_finalize_sf_size(T, H, int(sf_layout))),
                    exact=False)


def moe_finalize_run(permuted_rows: torch.Tensor, expanded_idx_to_permuted_idx: torch.Tensor,
                     expert_scales: Optional[torch.Tensor],
                     shared_expert_output: Optional[torch.Tensor],
                     routed_scaling_factor: float, out: torch.Tensor, stream=None) -> None:
    H = out.shape[-1]
    act, sdt, T, K = _common(permuted_rows, expanded_idx_to_permuted_idx, expert_scales,
                             shared_expert_output, H)
    _need(out, "out", (T, H), permuted_rows.dtype)
    _check(LIB.moe_finalize_run(
        _ptr(permuted_rows), permuted_rows.shape[0], _ptr(expanded_idx_to_permuted_idx),
        _ptr(expert_scales), sdt, _ptr(shared_expert_output), float(routed_scaling_factor),
        _ptr(out), T, H, K, act, _stream(out, stream)))


def moe_finalize_rmsnorm_run(permuted_rows: torch.Tensor,
                             expanded_idx_to_permuted_idx: torch.Tensor,
                             expert_scales: Optional[torch.Tensor],
                             shared_expert_output: Optional[torch.Tensor],
                             routed_scaling_factor: float, residual: torch.Tensor,
                             gamma: torch.Tensor, eps: float,
                             residual_out: Optional[torch.Tensor], norm_out: torch.Tensor,
                             workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    H = residual.shape[-1]
    act, sdt, T, K = _common(permuted_rows, expanded_idx_to_permuted_idx, expert_scales,
                             shared_expert_output, H)
    _rows_out(permuted_rows.dtype, T, H, residual, gamma, residual_out, norm_out)
    wp, wb = _ws(workspace)
    _check(LIB.moe_finalize_rmsnorm_run(
        _ptr(permuted_rows), permuted_rows.shape[0], _ptr(expanded_idx_to_permuted_idx),
        _ptr(expert_scales), sdt, _ptr(shared_expert_output), float(routed_scaling_factor),
        _ptr(residual), _ptr(gamma), float(eps), _ptr(residual_out), _ptr(norm_out), wp, wb,
        T, H, K, act, _stream(residual, stream)))


def moe_finalize_rmsnorm_noalloc_run(permuted_rows: torch.Tensor,
                                     expanded_idx_to_permuted_idx: torch.Tensor,
                                     expert_scales: Optional[torch.Tensor],
                                     shared_expert_output: Optional[torch.Tensor],
                                     routed_scaling_factor: float, residual: torch.Tensor,
                                     gamma: torch.Tensor, eps: float,
                                     residual_out: Optional[torch.Tensor], norm_out: torch.Tensor,
                                     stream=None) -> None:
    H = residual.shape[-1]
    act, sdt, T, K = _common(permuted_rows, expanded_idx_to_permuted_idx, expert_scales,
                             shared_expert_output, H)
    _rows_out(permuted_rows.dtype, T, H, residual, gamma, residual_out, norm_out)
    _check(LIB.moe_finalize_rmsnorm_noalloc_run(
        _ptr(permuted_rows), permuted_rows.shape[0], _ptr(expanded_idx_to_permuted_idx),
        _ptr(expert_scales), sdt, _ptr(shared_expert_output), float(routed_scaling_factor),
        _ptr(residual), _ptr(gamma), float(eps), _ptr(residual_out), _ptr(norm_out),
        T, H, K, act, _stream(residual, stream)))


def moe_finalize_quant_run(permuted_rows: torch.Tensor, expanded_idx_to_permuted_idx: torch.Tensor,
                           expert_scales: Optional[torch.Tensor],
                           shared_expert_output: Optional[torch.Tensor],
                           routed_scaling_factor: float, residual: torch.Tensor,
                           gamma: torch.Tensor, eps: float, quant_type: int,
                           quant_scale: torch.Tensor, quant_out: torch.Tensor,
                           scale_out: Optional[torch.Tensor], sf_layout: int,
                           residual_out: Optional[torch.Tensor], norm_out: Optional[torch.Tensor],
                           workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    H = residual.shape[-1]
    act, sdt, T, K = _common(permuted_rows, expanded_idx_to_permuted_idx, expert_scales,
                             shared_expert_output, H)
    _rows_out(permuted_rows.dtype, T, H, residual, gamma, residual_out, norm_out,
              norm_optional=True)
    _quant_out(T, H, quant_type, quant_scale, quant_out, scale_out, sf_layout)
    wp, wb = _ws(workspace)
    _check(LIB.moe_finalize_quant_run(
        _ptr(permuted_rows), permuted_rows.shape[0], _ptr(expanded_idx_to_permuted_idx),
        _ptr(expert_scales), sdt, _ptr(shared_expert_output), float(routed_scaling_factor),
        _ptr(residual), _ptr(gamma), float(eps), int(quant_type), _ptr(quant_scale),
        _ptr(quant_out), _ptr(scale_out), int(sf_layout), _ptr(residual_out), _ptr(norm_out),
        wp, wb, T, H, K, act, _stream(residual, stream)))


def moe_quantize_run(x: torch.Tensor, quant_type: int, quant_scale: torch.Tensor,
                     quant_out: torch.Tensor, scale_out: Optional[torch.Tensor], sf_layout: int,
                     stream=None) -> None:
    _act_dtype(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be [T, H]")
    T, H = x.shape
    _quant_out(T, H, quant_type, quant_scale, quant_out, scale_out, sf_layout)
    _check(LIB.moe_quantize_run(_ptr(x), T, H, _ACT[x.dtype], int(quant_type), _ptr(quant_scale),
                                _ptr(quant_out), _ptr(scale_out), int(sf_layout),
                                _stream(x, stream)))


def moe_residual_rmsnorm_run(x: torch.Tensor, residual: torch.Tensor, gamma: torch.Tensor,
                             eps: float, residual_out: Optional[torch.Tensor],
                             norm_out: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                             stream=None) -> None:
    _act_dtype(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be [T, H]")
    T, H = x.shape
    _rows_out(x.dtype, T, H, residual, gamma, residual_out, norm_out)
    wp, wb = _ws(workspace)
    _check(LIB.moe_residual_rmsnorm_run(_ptr(x), _ptr(residual), _ptr(gamma), float(eps),
                                        _ptr(residual_out), _ptr(norm_out), wp, wb, T, H,
                                        _ACT[x.dtype], _stream(x, stream)))


def moe_rank_sum_rmsnorm_run(rank_partials: torch.Tensor, residual: torch.Tensor,
                             gamma: torch.Tensor, eps: float, residual_out: Optional[torch.Tensor],
                             norm_out: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                             stream=None) -> None:
    """rank_partials: [world_size, T, H]."""
    _act_dtype(rank_partials, "rank_partials")
    if rank_partials.dim() != 3:
        raise ValueError("rank_partials must be [world_size, T, H]")
    W, T, H = rank_partials.shape
    _rows_out(rank_partials.dtype, T, H, residual, gamma, residual_out, norm_out)
    wp, wb = _ws(workspace)
    _check(LIB.moe_rank_sum_rmsnorm_run(_ptr(rank_partials), W, _ptr(residual), _ptr(gamma),
                                        float(eps), _ptr(residual_out), _ptr(norm_out), wp, wb, T,
                                        H, _ACT[rank_partials.dtype], _stream(residual, stream)))


def moe_rank_sum_quant_run(rank_partials: torch.Tensor, residual: torch.Tensor,
                           gamma: torch.Tensor, eps: float, quant_type: int,
                           quant_scale: torch.Tensor, quant_out: torch.Tensor,
                           scale_out: Optional[torch.Tensor], sf_layout: int,
                           residual_out: Optional[torch.Tensor], norm_out: Optional[torch.Tensor],
                           workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """rank_partials: [world_size, T, H]."""
    _act_dtype(rank_partials, "rank_partials")
    if rank_partials.dim() != 3:
        raise ValueError("rank_partials must be [world_size, T, H]")
    W, T, H = rank_partials.shape
    _rows_out(rank_partials.dtype, T, H, residual, gamma, residual_out, norm_out,
              norm_optional=True)
    _quant_out(T, H, quant_type, quant_scale, quant_out, scale_out, sf_layout)
    wp, wb = _ws(workspace)
    _check(LIB.moe_rank_sum_quant_run(_ptr(rank_partials), W, _ptr(residual), _ptr(gamma),
                                      float(eps), int(quant_type), _ptr(quant_scale),
                                      _ptr(quant_out), _ptr(scale_out), int(sf_layout),
                                      _ptr(residual_out), _ptr(norm_out), wp, wb, T, H,
                                      _ACT[rank_partials.dtype], _stream(residual, stream)))
