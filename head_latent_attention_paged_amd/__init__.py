"""Python binding of libmla.so: paged and sparse MLA decode on MI355X (gfx950).

Argument marshalling only.  Every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/mla.h``; there is no CPU or
PyTorch fallback.  PyTorch provides device memory and the current stream.
Importing this package raises if the library has not been built.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmla.so")

D_QK, D_V, PAGE, SPARSE_REC, META_INTS = 576, 512, 64, 640, 8
MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE, MLA_ERR_HIP = 0, 1, 2, 3, 4

EXPORTS = (
    "mla_status_string", "mla_num_parts", "mla_get_metadata", "mla_get_metadata_host",
    "mla_workspace_size", "mla_decode_paged", "mla_decode_paged_fp8", "mla_decode_paged_latent512",
    "mla_decode_paged_fp4", "mla_sparse_splits",
    "mla_workspace_size_sparse", "mla_decode_sparse", "mla_sparse_prefill", "mla_decode_paged_noalloc",
    "mla_decode_fused",
)
NOALLOC_SCRATCH_BYTES = 32 << 20     # MLA_NOALLOC_SCRATCH_BYTES


class MLAError(RuntimeError):
    """A non-OK status returned by libmla.so."""

    def __init__(self, call: str, status: int, msg: str):
        super().__init__("%s failed: %s" % (call, msg))
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError("libmla.so is not built (%s); run __graft_entry__.build() or "
                          "python head_latent_attention_paged_amd/build.py" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.mla_status_string.argtypes = [i32]
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_num_parts.argtypes = [i32, i32, i32]
    lib.mla_num_parts.restype = i32
    lib.mla_get_metadata.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp]
    lib.mla_get_metadata.restype = i32
    lib.mla_get_metadata_host.argtypes = [vp, i32, i32, i32, i32, vp, vp]
    lib.mla_get_metadata_host.restype = i32
    lib.mla_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.mla_workspace_size.restype = sz
    lib.mla_decode_paged.argtypes = [vp, vp, i64, vp, i32, vp, i32, i32, i32, f32, i32,
                                     vp, vp, i32, vp, sz, vp, vp, vp]
    lib.mla_decode_paged.restype = i32
    lib.mla_decode_paged_noalloc.argtypes = [vp, vp, i64, vp, i32, vp, i32, i32, i32, f32, i32,
                                             vp, vp, i32, vp, vp, vp]
    lib.mla_decode_paged_noalloc.restype = i32
    lib.mla_decode_paged_fp8.argtypes = lib.mla_decode_paged.argtypes
    lib.mla_decode_paged_fp8.restype = i32
    lib.mla_decode_paged_latent512.argtypes = [vp, vp, i64, vp, i32, vp, i32, i32, i32, f32, i32, vp,
                                               vp, vp, i32, vp, sz, vp, vp, vp]
    lib.mla_decode_paged_latent512.restype = i32
    lib.mla_decode_paged_fp4.argtypes = [vp, vp, vp, i64, vp, i32, vp, i32, i32, i32, f32, i32, vp,
                                         vp, vp, i32, vp, sz, vp, vp, vp]
    lib.mla_decode_paged_fp4.restype = i32
    lib.mla_decode_fused.argtypes = [vp, vp, vp, i64, vp, i32, vp, i32, i32, i32, f32, i32, vp,
                                     vp, f32, vp, vp, vp, i32, vp, sz, vp, vp, vp, vp]
    lib.mla_decode_fused.restype = i32
    lib.mla_sparse_splits.argtypes = [i32, i32, i32, i32]
    lib.mla_sparse_splits.restype = i32
    lib.mla_workspace_size_sparse.argtypes = [i32, i32, i32, i32, i32]
    lib.mla_workspace_size_sparse.restype = sz
    lib.mla_decode_sparse.argtypes = [vp, vp, i64, vp, i32, i32, i32, i32, f32, i32, vp, sz, vp, vp, vp]
    lib.mla_decode_sparse.restype = i32
    lib.mla_sparse_prefill.argtypes = [vp, vp, i64, vp, i32, i32, i32, f32, i32, vp, sz, vp, vp, vp]
    lib.mla_sparse_prefill.restype = i32
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.mla_status_string(status).decode()


def _check(call: str, status: int) -> None:
    if status != MLA_OK:
        raise MLAError(call, status, status_string(status))


def _stream_ptr(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _require(t: torch.Tensor, name: str, dtype: torch.dtype, shape=None) -> None:
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


# --------------------------------------------------------------------------
# Metadata
# --------------------------------------------------------------------------
def num_parts(h_q: int, s_q: int, num_cus: int = 0) -> int:
    return int(lib.mla_num_parts(num_cus, h_q, s_q))


def get_metadata(cache_seqlens: torch.Tensor, h_q: int, s_q: int,
                 num_parts_: Optional[int] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Tile-scheduler metadata for one decode step: (tile_meta [P, 8], num_splits [batch+1]) int32."""
    _require(cache_seqlens, "cache_seqlens", torch.int32)
    batch = cache_seqlens.shape[0]
    P = num_parts(h_q, s_q) if num_parts_ is None else int(num_parts_)
    dev = cache_seqlens.device
    tile_meta = torch.empty((P, META_INTS), dtype=torch.int32, device=dev)
    num_splits = torch.empty((batch + 1,), dtype=torch.int32, device=dev)
    _check("mla_get_metadata", lib.mla_get_metadata(
        cache_seqlens.data_ptr(), batch, h_q, s_q, P, tile_meta.data_ptr(), num_splits.data_ptr(),
        _stream_ptr(dev)))
    return tile_meta, num_splits


def get_metadata_host(cache_seqlens, num_parts_: int, h_q: int = 16, s_q: int = 1):
    """Host twin of get_metadata on host int32 arrays (numpy); returns numpy arrays."""
    import numpy as np

    L = np.ascontiguousarray(cache_seqlens, dtype=np.int32)
    batch = L.shape[0]
    tile_meta = np.zeros((num_parts_, META_INTS), dtype=np.int32)
    num_splits = np.zeros((batch + 1,), dtype=np.int32)
    _check("mla_get_metadata_host", lib.mla_get_metadata_host(
        L.ctypes.data, batch, h_q, s_q, num_parts_, tile_meta.ctypes.data, num_splits.ctypes.data))
    return tile_meta, num_splits


# --------------------------------------------------------------------------
# Paged decode
# --------------------------------------------------------------------------
def workspace_size(batch: int, s_q: int, h_q: int, num_parts_: int) -> int:
    return int(lib.mla_workspace_size(batch, s_q, h_q, num_parts_))


def decode_paged(q: torch.Tensor, kcache: torch.Tensor, block_table: torch.Tensor,
                 cache_seqlens: torch.Tensor, metadata: Tuple[torch.Tensor, torch.Tensor],
                 softmax_scale: float = D_QK ** -0.5, causal: bool = False,
                 out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None,
                 sinks: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Paged MLA decode; returns (out bf16 [b, s_q, h_q, 512], lse fp32 [b, s_q, h_q]).

    kcache is bf16 [num_blocks, 64, 1, 576]; or uint8 [num_blocks, 64, 640] fp8 records (e4m3
    codes of the 576 dims, the token's fp32 scale at byte 576), which calls mla_decode_paged_fp8;
    or, with q of 512 dims, bf16 [num_blocks, 64, 512] latent rows that are K and V (the
    DeepSeek-V4 geometry), which calls mla_decode_paged_latent512 with the optional per-head
    ``sinks`` (fp32 [h_q]).
    """
    batch, s_q, h_q, d = q.shape
    if d not in (D_QK, D_V):
        raise ValueError("q must have 576 (or 512) dims per head")
    _require(q, "q", torch.bfloat16)
    if d == D_V:
        return _decode_paged_latent512(q, kcache, block_table, cache_seqlens, metadata, softmax_scale,
                                       causal, out, lse, workspace, sinks)
    if sinks is not None:
        raise ValueError("attention sinks come with the 512-wide latent rows")
    fp8 = kcache.dtype == torch.uint8
    if fp8:
        _require(kcache, "kcache", torch.uint8)
        if kcache.dim() != 3 or tuple(kcache.shape[1:]) != (PAGE, SPARSE_REC):
            raise ValueError("an fp8 kcache must be [num_blocks, 64, 640] uint8 records")
    else:
        _require(kcache, "kcache", torch.bfloat16)
        if kcache.dim() != 4 or tuple(kcache.shape[1:]) != (PAGE, 1, D_QK):
            raise ValueError("kcache must be [num_blocks, 64, 1, 576]")
    _require(block_table, "block_table", torch.int32)
    _require(cache_seqlens, "cache_seqlens", torch.int32, (batch,))
    tile_meta, num_splits = metadata
    P = tile_meta.shape[0]
    dev = q.device
    if out is None:
        out = torch.empty((batch, s_q, h_q, D_V), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((batch, s_q, h_q), dtype=torch.float32, device=dev)
    _require(out, "out", torch.bfloat16, (batch, s_q, h_q, D_V))
    _require(lse, "lse", torch.float32, (batch, s_q, h_q))
    need = workspace_size(batch, s_q, h_q, P)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=dev)
    name = "mla_decode_paged_fp8" if fp8 else "mla_decode_paged"
    _check(name, getattr(lib, name)(
        q.data_ptr(), kcache.data_ptr(), kcache.shape[0], block_table.data_ptr(), block_table.shape[1],
        cache_seqlens.data_ptr(), batch, s_q, h_q, float(softmax_scale), 1 if causal else 0,
        tile_meta.data_ptr(), num_splits.data_ptr(), P,
        workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        out.data_ptr(), lse.data_ptr(), _stream_ptr(dev)))
    return out, lse


def decode_paged_noalloc(q: torch.Tensor, kcache: torch.Tensor, block_table: torch.Tensor,
                         cache_seqlens: torch.Tensor, metadata: Tuple[torch.Tensor, torch.Tensor],
                         softmax_scale: float = D_QK ** -0.5, causal: bool = False,
                         out: Optional[torch.Tensor] = None,
                         lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """mla_decode_paged_noalloc: the bf16 paged decode with the split-KV partials in the
    library's own per-GPU array (no workspace argument).  Shapes as for decode_paged with a
    bf16 [num_blocks, 64, 1, 576] cache.  Pass ``out`` and ``lse`` to allocate nothing here
    either."""
    batch, s_q, h_q, d = q.shape
    if d != D_QK:
        raise ValueError("q must have 576 dims per head")
    _require(q, "q", torch.bfloat16)
    _require(kcache, "kcache", torch.bfloat16)
    if kcache.dim() != 4 or tuple(kcache.shape[1:]) != (PAGE, 1, D_QK):
        raise ValueError("kcache must be [num_blocks, 64, 1, 576]")
    _require(block_table, "block_table", torch.int32)
    _require(cache_seqlens, "cache_seqlens", torch.int32, (batch,))
    tile_meta, num_splits = metadata
    dev = q.device
    if out is None:
        out = torch.empty((batch, s_q, h_q, D_V), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((batch, s_q, h_q), dtype=torch.float32, device=dev)
    _require(out, "out", torch.bfloat16, (batch, s_q, h_q, D_V))
    _require(lse, "lse", torch.float32, (batch, s_q, h_q))
    _check("mla_decode_paged_noalloc", lib.mla_decode_paged_noalloc(
        q.data_ptr(), kcache.data_ptr(), kcache.shape[0], block_table.data_ptr(), block_table.shape[1],
        cache_seqlens.data_ptr(), batch, s_q, h_q, float(softmax_scale), 1 if causal else 0,
        tile_meta.data_ptr(), num_splits.data_ptr(), tile_meta.shape[0],
        out.data_ptr(), lse.data_ptr(), _stream_ptr(dev)))
    return out, lse


def _decode_paged_latent512(q, kcache, block_table, cache_seqlens, metadata, softmax_scale, causal,
                            out, lse, workspace, sinks):
    batch, s_q, h_q, _ = q.shape
    _require(kcache, "kcache", torch.bfloat16)
    if kcache.dim() != 3 or tuple(kcache.shape[1:]) != (PAGE, D_V):
        raise ValueError("kcache must be [num_blocks, 64, 512] for 512-wide latent rows")
    _require(block_table, "block_table", torch.int32)
    _require(cache_seqlens, "cache_seqlens", torch.int32, (batch,))
    if sinks is not None:
        _require(sinks, "sinks", torch.float32, (h_q,))
    tile_meta, num_splits = metadata
    P = tile_meta.shape[0]
    dev = q.device
    if out is None:
        out = torch.empty((batch, s_q, h_q, D_V), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((batch, s_q, h_q), dtype=torch.float32, device=dev)
    _require(out, "out", torch.bfloat16, (batch, s_q, h_q, D_V))
    _require(lse, "lse", torch.float32, (batch, s_q, h_q))
    need = workspace_size(batch, s_q, h_q, P)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=dev)
    _check("mla_decode_paged_latent512", lib.mla_decode_paged_latent512(
        q.data_ptr(), kcache.data_ptr(), kcache.shape[0], block_table.data_ptr(), block_table.shape[1],
        cache_seqlens.data_ptr(), batch, s_q, h_q, float(softmax_scale), 1 if causal else 0,
        None if sinks is None else sinks.data_ptr(),
        tile_meta.data_ptr(), num_splits.data_ptr(), P,
        workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        out.data_ptr(), lse.data_ptr(), _stream_ptr(dev)))
    return out, lse


def decode_paged_fp4(q: torch.Tensor, kv_codes: torch.Tensor, kv_scales: torch.Tensor,
                     block_table: torch.Tensor, cache_seqlens: torch.Tensor,
                     metadata: Tuple[torch.Tensor, torch.Tensor],
                     softmax_scale: float = D_V ** -0.5, causal: bool = False,
                     out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None,
                     sinks: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """DeepSeek-V4-geometry decode over an FP4 cache (mla_decode_paged_fp4).

    q bf16 [b, s_q, h_q, 512]; kv_codes uint8 [num_blocks, 64, 256] (E2M1, low nibble first);
    kv_scales uint8 [num_blocks, 64, 32] (UE4M3, one per 16 values); sinks fp32 [h_q] or None.
    Returns (out bf16 [b, s_q, h_q, 512], lse fp32 [b, s_q, h_q]).
    """
    batch, s_q, h_q, d = q.shape
    if d != D_V:
        raise ValueError("q must have 512 dims per head")
    _require(q, "q", torch.bfloat16)
    _require(kv_codes, "kv_codes", torch.uint8)
    _require(kv_scales, "kv_scales", torch.uint8)
    nb = kv_codes.shape[0]
    if kv_codes.dim() != 3 or tuple(kv_codes.shape[1:]) != (PAGE, 256):
        raise ValueError("kv_codes must be [num_blocks, 64, 256] uint8")
    if tuple(kv_scales.shape) != (nb, PAGE, 32):
        raise ValueError("kv_scales must be [num_blocks, 64, 32] uint8")
    _require(block_table, "block_table", torch.int32)
    _require(cache_seqlens, "cache_seqlens", torch.int32, (batch,))
    if sinks is not None:
        _require(sinks, "sinks", torch.float32, (h_q,))
    tile_meta, num_splits = metadata
    P = tile_meta.shape[0]
    dev = q.device
    if out is None:
        out = torch.empty((batch, s_q, h_q, D_V), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((batch, s_q, h_q), dtype=torch.float32, device=dev)
    _require(out, "out", torch.bfloat16, (batch, s_q, h_q, D_V))
    _require(lse, "lse", torch.float32, (batch, s_q, h_q))
    need = workspace_size(batch, s_q, h_q, P)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=dev)
    _check("mla_decode_paged_fp4", lib.mla_decode_paged_fp4(
        q.data_ptr(), kv_codes.data_ptr(), kv_scales.data_ptr(), nb, block_table.data_ptr(),
        block_table.shape[1], cache_seqlens.data_ptr(), batch, s_q, h_q, float(softmax_scale),
        1 if causal else 0, None if sinks is None else sinks.data_ptr(),
        tile_meta.data_ptr(), num_splits.data_ptr(), P,
        workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        out.data_ptr(), lse.data_ptr(), _stream_ptr(dev)))
    return out, lse


def decode_fused(q: torch.Tensor, kcache: torch.Tensor, block_table: torch.Tensor,
                 cache_seqlens: torch.Tensor, metadata: Tuple[torch.Tensor, torch.Tensor],
                 norm_weight: torch.Tensor, norm_eps: float, rope_cs: torch.Tensor,
                 softmax_scale: float = D_V ** -0.5, causal: bool = False,
                 sinks: Optional[torch.Tensor] = None, kv_scales: Optional[torch.Tensor] = None,
                 out: Optional[torch.Tensor] = None, out_scale: Optional[torch.Tensor] = None,
                 lse: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """The fused decode (mla_decode_fused): query RMS norm and RoPE, attention over 512-wide latent
    rows, conjugate RoPE of the output and its FP8 cast.

    q bf16 [b, s_q, h_q, 512]; kcache bf16 [num_blocks, 64, 512], or (with kv_scales uint8
    [num_blocks, 64, 32]) uint8 [num_blocks, 64, 256] FP4 codes; norm_weight fp32 [512];
    rope_cs fp32 [b, s_q, 64] (cos then sin of the 32 pair angles of each query token); sinks fp32
    [h_q] or None.  Returns (codes uint8 [b, s_q, h_q, 512] e4m3, scale fp32 [b, s_q, h_q],
    lse fp32 [b, s_q, h_q]).
    """
    batch, s_q, h_q, d = q.shape
    if d != D_V:
        raise ValueError("q must have 512 dims per head")
    _require(q, "q", torch.bfloat16)
    nb = kcache.shape[0]
    if kv_scales is None:
        _require(kcache, "kcache", torch.bfloat16)
        if kcache.dim() != 3 or tuple(kcache.shape[1:]) != (PAGE, D_V):
            raise ValueError("kcache must be [num_blocks, 64, 512] bf16")
    else:
        _require(kcache, "kv_codes", torch.uint8)
        _require(kv_scales, "kv_scales", torch.uint8, (nb, PAGE, 32))
        if kcache.dim() != 3 or tuple(kcache.shape[1:]) != (PAGE, 256):
            raise ValueError("FP4 codes must be [num_blocks, 64, 256] uint8")
    _require(block_table, "block_table", torch.int32)
    _require(cache_seqlens, "cache_seqlens", torch.int32, (batch,))
    _require(norm_weight, "norm_weight", torch.float32, (D_V,))
    _require(rope_cs, "rope_cs", torch.float32, (batch, s_q, 64))
    if sinks is not None:
        _require(sinks, "sinks", torch.float32, (h_q,))
    tile_meta, num_splits = metadata
    P = tile_meta.shape[0]
    dev = q.device
    if out is None:
        out = torch.empty((batch, s_q, h_q, D_V), dtype=torch.uint8, device=dev)
    if out_scale is None:
        out_scale = torch.empty((batch, s_q, h_q), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((batch, s_q, h_q), dtype=torch.float32, device=dev)
    _require(out, "out", torch.uint8, (batch, s_q, h_q, D_V))
    _require(out_scale, "out_scale", torch.float32, (batch, s_q, h_q))
    _require(lse, "lse", torch.float32, (batch, s_q, h_q))
    need = workspace_size(batch, s_q, h_q, P)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=dev)
    _check("mla_decode_fused", lib.mla_decode_fused(
        q.data_ptr(), kcache.data_ptr(), None if kv_scales is None else kv_scales.data_ptr(), nb,
        block_table.data_ptr(), block_table.shape[1], cache_seqlens.data_ptr(), batch, s_q, h_q,
        float(softmax_scale), 1 if causal else 0, None if sinks is None else sinks.data_ptr(),
        norm_weight.data_ptr(), float(norm_eps), rope_cs.data_ptr(),
        tile_meta.data_ptr(), num_splits.data_ptr(), P,
        workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        out.data_ptr(), out_scale.data_ptr(), lse.data_ptr(), _stream_ptr(dev)))
    return out, out_scale, lse


# --------------------------------------------------------------------------
# Sparse fp8 decode
# --------------------------------------------------------------------------
def sparse_splits(batch: int, s_q: int, h_q: int, topk: int) -> int:
    return int(lib.mla_sparse_splits(batch, s_q, h_q, topk))


def workspace_size_sparse(batch: int, s_q: int, h_q: int, topk: int, splits: int = 0) -> int:
    return int(lib.mla_workspace_size_sparse(batch, s_q, h_q, topk, splits))


def decode_sparse(q: torch.Tensor, kv: torch.Tensor, indices: torch.Tensor,
                  softmax_scale: float = D_QK ** -0.5, splits: int = 0,
                  out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Sparse fp8 MLA decode over 640-byte records; indices -1 = skip."""
    batch, s_q, h_q, d = q.shape
    if d != D_QK:
        raise ValueError("q must have 576 dims per head")
    _require(q, "q", torch.bfloat16)
    _require(kv, "kv", torch.uint8)
    if kv.dim() != 2 or kv.shape[1] != SPARSE_REC:
        raise ValueError("kv must be [num_tokens, 640] uint8 records")
    _require(indices, "indices", torch.int32)
    if indices.dim() != 3 or tuple(indices.shape[:2]) != (batch, s_q):
        raise ValueError("indices must be [batch, s_q, topk]")
    topk = indices.shape[2]
    dev = q.device
    if out is None:
        out = torch.empty((batch, s_q, h_q, D_V), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((batch, s_q, h_q), dtype=torch.float32, device=dev)
    _require(out, "out", torch.bfloat16, (batch, s_q, h_q, D_V))
    _require(lse, "lse", torch.float32, (batch, s_q, h_q))
    need = workspace_size_sparse(batch, s_q, h_q, topk, splits)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=dev)
    _check("mla_decode_sparse", lib.mla_decode_sparse(
        q.data_ptr(), kv.data_ptr(), kv.shape[0], indices.data_ptr(), topk, batch, s_q, h_q,
        float(softmax_scale), int(splits), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), out.data_ptr(), lse.data_ptr(), _stream_ptr(dev)))
    return out, lse


def sparse_prefill(q: torch.Tensor, kv: torch.Tensor, indices: torch.Tensor,
                   softmax_scale: float = D_QK ** -0.5, splits: int = 0,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Sparse prefill (mla_sparse_prefill): q bf16 [s_q, h_q, 576], kv uint8 [num_tokens, 640]
    records, indices int32 [s_q, topk] or [s_q, 1, topk] (-1 = skip).  Returns
    (out bf16 [s_q, h_q, 512], lse fp32 [s_q, h_q])."""
    s_q, h_q, d = q.shape
    if d != D_QK:
        raise ValueError("q must have 576 dims per head")
    _require(q, "q", torch.bfloat16)
    _require(kv, "kv", torch.uint8)
    if kv.dim() != 2 or kv.shape[1] != SPARSE_REC:
        raise ValueError("kv must be [num_tokens, 640] uint8 records")
    _require(indices, "indices", torch.int32)
    if indices.dim() == 3 and indices.shape[1] == 1:
        indices = indices[:, 0]
    if indices.dim() != 2 or indices.shape[0] != s_q or not indices.is_contiguous():
        raise ValueError("indices must be a contiguous [s_q, topk] (or [s_q, 1, topk]) tensor")
    topk = indices.shape[1]
    dev = q.device
    if out is None:
        out = torch.empty((s_q, h_q, D_V), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((s_q, h_q), dtype=torch.float32, device=dev)
    _require(out, "out", torch.bfloat16, (s_q, h_q, D_V))
    _require(lse, "lse", torch.float32, (s_q, h_q))
    need = workspace_size_sparse(1, s_q, h_q, topk, splits)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=dev)
    _check("mla_sparse_prefill", lib.mla_sparse_prefill(
        q.data_ptr(), kv.data_ptr(), kv.shape[0], indices.data_ptr(), topk, s_q, h_q,
        float(softmax_scale), int(splits), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), out.data_ptr(), lse.data_ptr(), _stream_ptr(dev)))
    return out, lse
