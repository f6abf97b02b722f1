"""torch-facing wrappers of the C ABI (device memory and streams come from torch).

    out, lse = mla_verify(q_nope, q_rope, kv_latent, k_rope, tree_parent, prefix_len, scale)

Inputs are bf16 CUDA (HIP) tensors, row-major and contiguous; tree_parent is
int32 on the same device. Outputs are fp32. The work runs on the current torch
stream; the call returns without synchronising.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from . import _lib

H = 64  # the head count of the benchmark workloads (any count 1..1024 is accepted)
DL = 512
DR = 64


def _check(t: torch.Tensor, name: str, dtype, shape, device) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _gpu_device(t: torch.Tensor, name: str, ndim: int, at_least: bool = False) -> torch.device:
    """The device of `t`, which must be a GPU tensor with `ndim` dimensions (or
    at least that many): the library dereferences every pointer on the GPU, where
    a host pointer would fault."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("inputs must be on a GPU (the library has no CPU path)")
    if t.dim() < ndim if at_least else t.dim() != ndim:
        raise ValueError(f"{name} must have {'at least ' if at_least else ''}{ndim} dimensions, got {t.dim()}")
    return t.device


def _workspace(workspace: Optional[torch.Tensor], need: int, device) -> Tuple[Optional[int], int, Optional[torch.Tensor]]:
    """(pointer, bytes, tensor) of the split workspace: the caller's, checked, or a new one."""
    if workspace is None:
        if need <= 0:
            return None, 0, None
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if not isinstance(workspace, torch.Tensor) or workspace.device != device or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size(), workspace


def _stream_ptr(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def mla_verify(q_nope: torch.Tensor, q_rope: torch.Tensor, kv_latent: torch.Tensor, k_rope: torch.Tensor,
               tree_parent: torch.Tensor, prefix_len: int, scale: float,
               out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None, nsplit: int = 0, pv_mode: int = 0,
               kernel: int = 0, partials: int = 0, phase: int = 0,
               merge: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """One sequence: q_nope [q,H,512], q_rope [q,H,64], kv_latent [P+q,512], k_rope [P+q,64]
    (bf16), tree_parent [q] int32 -> out [q,H,512] fp32, lse [q,H] fp32.
    partials: 0 = int16 split partials with per-row scales (default), 1 = fp32.
    phase: 0 = whole call, 1 = split kernel only, 2 = combine kernel only (same workspace).
    merge: 0 = the combine kernel merges the splits (default), 1 = plans of 2..4 splits
    merge in the split kernel (one launch)."""
    dev = _gpu_device(q_nope, "q_nope", 3)
    q, h = int(q_nope.shape[0]), int(q_nope.shape[1])
    n = int(prefix_len) + q
    _check(q_nope, "q_nope", torch.bfloat16, (q, h, DL), dev)
    _check(q_rope, "q_rope", torch.bfloat16, (q, h, DR), dev)
    _check(kv_latent, "kv_latent", torch.bfloat16, (n, DL), dev)
    _check(k_rope, "k_rope", torch.bfloat16, (n, DR), dev)
    _check(tree_parent, "tree_parent", torch.int32, (q,), dev)
    if out is None:
        out = torch.empty(q, h, DL, dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(q, h, dtype=torch.float32, device=dev)
    _check(out, "out", torch.float32, (q, h, DL), dev)
    _check(lse, "lse", torch.float32, (q, h), dev)
    lib = _lib.load()
    opt = _lib.options(nsplit, pv_mode, kernel, partials, phase, merge)
    with torch.cuda.device(dev):  # the library plans for, and launches on, the current device
        need = int(lib.mla_verify_workspace_size(q, h, 1, n, n, 0, ctypes.byref(opt)))
        ws_ptr, ws_bytes, workspace = _workspace(workspace, need, dev)
        rc = lib.mla_verify_ex(q_nope.data_ptr(), q_rope.data_ptr(), kv_latent.data_ptr(), k_rope.data_ptr(),
                               tree_parent.data_ptr(), int(prefix_len), float(scale), out.data_ptr(),
                               lse.data_ptr(), q, h, ws_ptr, ws_bytes, _stream_ptr(dev), ctypes.byref(opt))
    if rc != _lib.MLAV_OK:
        raise _lib.MLAVError(rc, "mla_verify")
    return out, lse


def mla_verify_batched(q_nope: torch.Tensor, q_rope: torch.Tensor, kv_latent: torch.Tensor,
                       k_rope: torch.Tensor, tree_parent: torch.Tensor, kv_offsets: torch.Tensor,
                       scale: float, max_kv: Optional[int] = None,
                       out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, nsplit: int = 0, pv_mode: int = 0,
                       kernel: int = 0, partials: int = 0, merge: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """B sequences: q_nope [B,q,H,512], kv rows of sequence b = [off[b], off[b+1]),
    tree_parent [B,q] int32, kv_offsets [B+1] int64 (CPU or device)."""
    dev = _gpu_device(q_nope, "q_nope", 4)
    bsz, q, h = int(q_nope.shape[0]), int(q_nope.shape[1]), int(q_nope.shape[2])
    total = int(kv_latent.shape[0])
    if not isinstance(kv_offsets, torch.Tensor) or kv_offsets.dtype != torch.int64 or \
            tuple(kv_offsets.shape) != (bsz + 1,):
        raise ValueError("kv_offsets must be int64 [B+1]")
    if max_kv is None or not kv_offsets.is_cuda:
        host = kv_offsets.detach().cpu()
        max_kv = int((host[1:] - host[:-1]).max().item()) if max_kv is None else int(max_kv)
    offs_dev = kv_offsets.to(dev) if not kv_offsets.is_cuda else kv_offsets
    _check(q_nope, "q_nope", torch.bfloat16, (bsz, q, h, DL), dev)
    _check(q_rope, "q_rope", torch.bfloat16, (bsz, q, h, DR), dev)
    _check(kv_latent, "kv_latent", torch.bfloat16, (total, DL), dev)
    _check(k_rope, "k_rope", torch.bfloat16, (total, DR), dev)
    _check(tree_parent, "tree_parent", torch.int32, (bsz, q), dev)
    if out is None:
        out = torch.empty(bsz, q, h, DL, dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(bsz, q, h, dtype=torch.float32, device=dev)
    _check(out, "out", torch.float32, (bsz, q, h, DL), dev)
    _check(lse, "lse", torch.float32, (bsz, q, h), dev)
    if not offs_dev.is_contiguous():
        offs_dev = offs_dev.contiguous()
    lib = _lib.load()
    opt = _lib.options(nsplit, pv_mode, kernel, partials, merge=merge)
    with torch.cuda.device(dev):  # the library plans for, and launches on, the current device
        need = int(lib.mla_verify_workspace_size(q, h, bsz, total, max_kv, 0, ctypes.byref(opt)))
        ws_ptr, ws_bytes, workspace = _workspace(workspace, need, dev)
        rc = lib.mla_verify_batched(q_nope.data_ptr(), q_rope.data_ptr(), kv_latent.data_ptr(),
                                    k_rope.data_ptr(), tree_parent.data_ptr(), offs_dev.data_ptr(), bsz, total,
                                    max_kv, float(scale), out.data_ptr(), lse.data_ptr(), q, h, ws_ptr, ws_bytes,
                                    _stream_ptr(dev), ctypes.byref(opt))
    if rc != _lib.MLAV_OK:
        raise _lib.MLAVError(rc, "mla_verify_batched")
    return out, lse


def mla_verify_paged(q_nope: torch.Tensor, q_rope: torch.Tensor, pool_latent: torch.Tensor,
                     pool_rope: torch.Tensor, kv_index: torch.Tensor, tree_parent: torch.Tensor, scale: float,
                     kv_offsets: Optional[torch.Tensor] = None, max_kv: Optional[int] = None,
                     out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, nsplit: int = 0, pv_mode: int = 0,
                     kernel: int = 0, partials: int = 0, merge: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """Paged KV (one token per page): pool_latent [R,512], pool_rope [R,64] bf16,
    kv_index [N] int32 (logical row -> pool row). One sequence: q_nope [q,H,512],
    tree_parent [q], kv_offsets None (its N logical rows are its prefix then its
    tree). Batch: q_nope [B,q,H,512], tree_parent [B,q], kv_offsets [B+1] int64."""
    batched = kv_offsets is not None
    dev = _gpu_device(q_nope, "q_nope", 4 if batched else 3)
    if batched:
        bsz, q, h = int(q_nope.shape[0]), int(q_nope.shape[1]), int(q_nope.shape[2])
    else:
        bsz, (q, h) = 1, (int(q_nope.shape[0]), int(q_nope.shape[1]))
    total = int(kv_index.shape[0])
    pool = int(pool_latent.shape[0])
    lead = (bsz,) if batched else ()
    _check(q_nope, "q_nope", torch.bfloat16, lead + (q, h, DL), dev)
    _check(q_rope, "q_rope", torch.bfloat16, lead + (q, h, DR), dev)
    _check(pool_latent, "pool_latent", torch.bfloat16, (pool, DL), dev)
    _check(pool_rope, "pool_rope", torch.bfloat16, (pool, DR), dev)
    _check(kv_index, "kv_index", torch.int32, (total,), dev)
    _check(tree_parent, "tree_parent", torch.int32, lead + (q,), dev)
    offs_ptr = None
    if batched:
        if not isinstance(kv_offsets, torch.Tensor) or kv_offsets.dtype != torch.int64 or \
                tuple(kv_offsets.shape) != (bsz + 1,):
            raise ValueError("kv_offsets must be int64 [B+1]")
        if max_kv is None:
            host = kv_offsets.detach().cpu()
            max_kv = int((host[1:] - host[:-1]).max().item())
        kv_offsets = kv_offsets.to(dev).contiguous()
        offs_ptr = kv_offsets.data_ptr()
    else:
        max_kv = total
    if out is None:
        out = torch.empty(lead + (q, h, DL), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(lead + (q, h), dtype=torch.float32, device=dev)
    _check(out, "out", torch.float32, lead + (q, h, DL), dev)
    _check(lse, "lse", torch.float32, lead + (q, h), dev)
    lib = _lib.load()
    opt = _lib.options(nsplit, pv_mode, kernel, partials, merge=merge)
    with torch.cuda.device(dev):  # the library plans for, and launches on, the current device
        need = int(lib.mla_verify_workspace_size(q, h, bsz, total, int(max_kv), 0, ctypes.byref(opt)))
        ws_ptr, ws_bytes, workspace = _workspace(workspace, need, dev)
        rc = lib.mla_verify_paged(q_nope.data_ptr(), q_rope.data_ptr(), pool_latent.data_ptr(),
                                  pool_rope.data_ptr(), kv_index.data_ptr(), pool, tree_parent.data_ptr(), offs_ptr,
                                  bsz, total, int(max_kv), float(scale), out.data_ptr(), lse.data_ptr(), q, h,
                                  ws_ptr, ws_bytes, _stream_ptr(dev), ctypes.byref(opt))
    if rc != _lib.MLAV_OK:
        raise _lib.MLAVError(rc, "mla_verify_paged")
    return out, lse


def mla_verify_partials(q_nope: torch.Tensor, q_rope: torch.Tensor, kv_latent: torch.Tensor,
                        k_rope: torch.Tensor, tree_parent: torch.Tensor, prefix_len: int, scale: float,
                        plan: _lib.Plan, part_out: Optional[torch.Tensor] = None,
                        part_lse: Optional[torch.Tensor] = None, pv_mode: int = 0, kernel: int = 0):
    """The split phase for `plan`: part_out [S, q, H, 512], part_lse [S, q, H] (fp32); when
    q * H is not a multiple of 64 the rows are padded: [S, R, 512] and [S, R] with R = q * H
    rounded up to a multiple of 64."""
    dev = _gpu_device(q_nope, "q_nope", 3)
    q, h = int(q_nope.shape[0]), int(q_nope.shape[1])
    n = int(prefix_len) + q
    _check(q_nope, "q_nope", torch.bfloat16, (q, h, DL), dev)
    _check(q_rope, "q_rope", torch.bfloat16, (q, h, DR), dev)
    _check(kv_latent, "kv_latent", torch.bfloat16, (n, DL), dev)
    _check(k_rope, "k_rope", torch.bfloat16, (n, DR), dev)
    _check(tree_parent, "tree_parent", torch.int32, (q,), dev)
    s = int(plan.nsplit)
    # rows are (token, head) pairs in blocks of 64: padded when q * h is not a multiple of 64
    rows = q * h
    lead = (s, q, h) if rows % 64 == 0 else (s, (rows + 63) // 64 * 64)
    if part_out is None:
        part_out = torch.empty(lead + (DL,), dtype=torch.float32, device=dev)
    if part_lse is None:
        part_lse = torch.empty(lead, dtype=torch.float32, device=dev)
    _check(part_out, "part_out", torch.float32, lead + (DL,), dev)
    _check(part_lse, "part_lse", torch.float32, lead, dev)
    opt = _lib.options(0, pv_mode, kernel)
    with torch.cuda.device(dev):
        rc = _lib.load().mla_verify_partials(q_nope.data_ptr(), q_rope.data_ptr(), kv_latent.data_ptr(),
                                             k_rope.data_ptr(), tree_parent.data_ptr(), int(prefix_len),
                                             float(scale), part_out.data_ptr(), part_lse.data_ptr(), q, h,
                                             ctypes.byref(plan), _stream_ptr(dev), ctypes.byref(opt))
    if rc != _lib.MLAV_OK:
        raise _lib.MLAVError(rc, "mla_verify_partials")
    return part_out, part_lse


def combine(part_out: torch.Tensor, part_lse: torch.Tensor,
            out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """LSE merge of caller-made partials: part_out [S, rows, 512], part_lse [S, rows]."""
    dev = _gpu_device(part_out, "part_out", 2, at_least=True)
    s = int(part_out.shape[0])
    part_out = part_out.reshape(s, -1, DL)
    part_lse = part_lse.reshape(s, -1)
    rows = int(part_out.shape[1])
    _check(part_out, "part_out", torch.float32, (s, rows, DL), dev)
    _check(part_lse, "part_lse", torch.float32, (s, rows), dev)
    if out is None:
        out = torch.empty(rows, DL, dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(rows, dtype=torch.float32, device=dev)
    _check(out, "out", torch.float32, (rows, DL), dev)
    _check(lse, "lse", torch.float32, (rows,), dev)
    with torch.cuda.device(dev):
        rc = _lib.load().mla_verify_combine(part_out.data_ptr(), part_lse.data_ptr(), s, rows, out.data_ptr(),
                                            lse.data_ptr(), _stream_ptr(dev))
    if rc != _lib.MLAV_OK:
        raise _lib.MLAVError(rc, "mla_verify_combine")
    return out, lse


def device_plan(q_len: int, batch: int, total_kv: int, max_kv: int, nsplit: int = 0, pv_mode: int = 0,
                kernel: int = 0, device=None, num_heads: int = H, partials: int = 0, merge: int = 0) -> _lib.Plan:
    """The plan a call on `device` would use (reads the device's CU count)."""
    props = torch.cuda.get_device_properties(device if device is not None else torch.cuda.current_device())
    return _lib.plan(q_len, num_heads, batch, total_kv, max_kv, props.multi_processor_count, nsplit, pv_mode,
                     kernel, partials, merge)
