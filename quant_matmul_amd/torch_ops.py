"""Allocation helpers around the kq C ABI for torch callers.

These only allocate device tensors of the right shapes and call the
same-named entry points of the binding; all arithmetic runs in libkq.so.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (kq_gemm, kq_gemm_grouped, kq_gemm_partials, kq_gemm_tiles, kq_gemm_tiles_partials,
               kq_gemm_tiles_workspace_bytes, kq_gemm_workspace_bytes, kq_gemv, kq_gemv_f32, kq_gemv_partials,
               kq_pack, kq_packed_bytes, kq_q8k_tiles_bytes, kq_quantize_q8k, kq_quantize_q8k_tiles,
               kq_quantize_q8k_tiles_gather, kq_record_bytes, kq_unpack)

QK = 256


def upload_records(recs: np.ndarray, device="cuda") -> torch.Tensor:
    """ggml records (n, k/256, bytes) uint8 -> a flat device tensor."""
    return torch.from_numpy(np.ascontiguousarray(recs).reshape(-1)).to(device)


def pack(fmt, recs_dev: torch.Tensor, n: int, k: int, stream=None) -> torch.Tensor:
    planes = torch.empty(kq_packed_bytes(fmt, n, k), dtype=torch.uint8, device=recs_dev.device)
    kq_pack(fmt, recs_dev, n, k, planes, stream)
    return planes


def unpack(fmt, planes: torch.Tensor, n: int, k: int, stream=None) -> torch.Tensor:
    out = torch.empty(n * (k // QK) * kq_record_bytes(fmt), dtype=torch.uint8, device=planes.device)
    kq_unpack(fmt, planes, n, k, out, stream)
    return out


def q8k_buffers(t: int, k: int, device="cuda"):
    return (torch.empty((t, k), dtype=torch.int8, device=device),
            torch.empty((t, k // QK), dtype=torch.float32, device=device),
            torch.empty((t, k // 16), dtype=torch.int16, device=device))


def quantize_q8k(x: torch.Tensor, stream=None):
    t, k = x.shape
    xq, xs, xbs = q8k_buffers(t, k, x.device)
    kq_quantize_q8k(x, t, k, xq, xs, xbs, stream)
    return xq, xs, xbs


def q8k_tile_buffers(t: int, k: int, device="cuda"):
    """(code tiles int8, xs float32 [t][k/256], bsum tiles float16)."""
    nb = kq_q8k_tiles_bytes(t, k)
    return (torch.empty(nb, dtype=torch.int8, device=device),
            torch.empty((t, k // QK), dtype=torch.float32, device=device),
            torch.empty(nb // 16, dtype=torch.float16, device=device))


def quantize_q8k_tiles(x: torch.Tensor, stream=None):
    """Q8_K image for the GEMM: (code tiles, xs, bsum tiles)."""
    t, k = x.shape
    xq, xs, xbs = q8k_tile_buffers(t, k, x.device)
    kq_quantize_q8k_tiles(x, t, k, xq, xs, xbs, stream)
    return xq, xs, xbs


def quantize_q8k_tiles_gather(x: torch.Tensor, rows: torch.Tensor, stream=None):
    """Tile image of the gathered rows x[rows[i]] (an index outside x's rows
    gives a zero row), as kq_quantize_q8k_tiles_gather."""
    t, k = x.shape
    m = rows.shape[0]
    xq, xs, xbs = q8k_tile_buffers(m, k, x.device)
    kq_quantize_q8k_tiles_gather(x, t, k, rows, m, xq, xs, xbs, stream)
    return xq, xs, xbs


def pack_experts(fmt, recs_list, n: int, k: int, device="cuda"):
    """Pack several n x k matrices into one buffer; returns (planes, stride)."""
    stride = kq_packed_bytes(fmt, n, k)
    buf = torch.empty(stride * len(recs_list), dtype=torch.uint8, device=device)
    for e, recs in enumerate(recs_list):
        kq_pack(fmt, upload_records(recs, device), n, k, buf[e * stride:(e + 1) * stride])
    return buf, stride


def gemm_grouped(fmt, planes, stride: int, experts: int, tile_expert: torch.Tensor, n: int, k: int, q8t,
                 y=None, stream=None) -> torch.Tensor:
    xq, xs, xbs = q8t
    m = xs.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=xq.device)
    kq_gemm_grouped(fmt, planes, stride, experts, tile_expert, n, k, xq, xs, xbs, m, y, stream)
    return y


def gemv(fmt, planes, n: int, k: int, q8, stream=None) -> torch.Tensor:
    xq, xs, xbs = q8
    t = xq.shape[0]
    y = torch.empty((t, n), dtype=torch.float32, device=xq.device)
    kq_gemv(fmt, planes, n, k, xq, xs, xbs, t, y, stream)
    return y


def gemv_f32(fmt, planes, n: int, k: int, x: torch.Tensor, keep_image: bool = False, stream=None):
    """Fused quantise + GEMV; returns y, or (y, (xq, xs, xbs)) with keep_image."""
    t = x.shape[0]
    y = torch.empty((t, n), dtype=torch.float32, device=x.device)
    q8 = q8k_buffers(t, k, x.device) if (keep_image or t > 2) else (None, None, None)
    kq_gemv_f32(fmt, planes, n, k, x, t, y, *q8, stream)
    return (y, q8) if keep_image else y


def gemm_workspace(fmt, n: int, k: int, m: int, device="cuda") -> torch.Tensor:
    """The workspace kq_gemm needs for this shape (row image re-laid as the
    tile image, plus the k-split space)."""
    return torch.empty(kq_gemm_workspace_bytes(fmt, n, k, m), dtype=torch.uint8, device=device)


def gemm(fmt, planes, n: int, k: int, q8, workspace=None, stream=None) -> torch.Tensor:
    """q8: the row image (xq, xs, xbs) of kq_quantize_q8k.  workspace: None
    allocates one of kq_gemm_workspace_bytes."""
    xq, xs, xbs = q8
    m = xq.shape[0]
    if workspace is None:
        workspace = gemm_workspace(fmt, n, k, m, xq.device)
    y = torch.empty((m, n), dtype=torch.float32, device=xq.device)
    kq_gemm(fmt, planes, n, k, xq, xs, xbs, m, y, workspace, stream=stream)
    return y


def gemm_tiles_workspace(fmt, n: int, k: int, m: int, device="cuda"):
    """A kq_gemm_tiles workspace for this shape: at least 256 bytes, since a
    non-NULL workspace also lets the 32-token tile split k inside its
    workgroups where no slices are needed."""
    nb = kq_gemm_tiles_workspace_bytes(fmt, n, k, m)
    return torch.empty(max(nb, 256), dtype=torch.uint8, device=device)


def gemm_tiles(fmt, planes, n: int, k: int, q8t, workspace="auto", stream=None) -> torch.Tensor:
    """q8t: the GEMM's tile image (code tiles, xs, bsum tiles), as from
    quantize_q8k_tiles.  workspace: "auto" allocates one, None runs unsplit."""
    xq, xs, xbs = q8t
    m = xs.shape[0]
    if isinstance(workspace, str):
        workspace = gemm_tiles_workspace(fmt, n, k, m, xq.device)
    y = torch.empty((m, n), dtype=torch.float32, device=xq.device)
    kq_gemm_tiles(fmt, planes, n, k, xq, xs, xbs, m, y, workspace, stream=stream)
    return y


def matmul_partials(kind: str, fmt, planes, n: int, k: int, q8, stream=None):
    """(y, P, M) from kq_gemv_partials (kind 'gemv', row image),
    kq_gemm_partials (kind 'gemm', row image) or kq_gemm_tiles_partials
    (kind 'gemm_tiles', tile image)."""
    xq, xs, xbs = q8
    t = xs.shape[0]
    dev = xq.device
    y = torch.empty((t, n), dtype=torch.float32, device=dev)
    P = torch.empty((t, n, k // QK), dtype=torch.int32, device=dev)
    M = torch.empty((t, n, k // QK), dtype=torch.int32, device=dev)
    if kind == "gemv":
        kq_gemv_partials(fmt, planes, n, k, xq, xs, xbs, t, y, P, M, stream)
    elif kind == "gemm":
        kq_gemm_partials(fmt, planes, n, k, xq, xs, xbs, t, y, P, M, gemm_workspace(fmt, n, k, t, dev),
                         stream=stream)
    elif kind == "gemm_tiles":
        kq_gemm_tiles_partials(fmt, planes, n, k, xq, xs, xbs, t, y, P, M, stream)
    else:
        raise ValueError(kind)
    return y, P, M
