"""block_sparse_attention_amd — block-sparse FlashAttention forward for MI355X (gfx950).

Thin Python binding over the C ABI of ``libbsattn.so`` (``include/bsattn.h``).
Functions carry the C names; they take torch tensors that live on the GPU,
pass their device pointers and the current HIP stream, and return the output
tensors.  Torch is used for device memory and streams only: every step of
the computation runs in the library's HIP kernels.  There is no fallback —
if the library is not built, or a tensor is not on the GPU, the call raises.

Build the library with ``python -m block_sparse_attention_amd.build``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

__all__ = [
    "BLOCK", "BsattnError", "load_library", "bsattn_status_string", "bsattn_version",
    "bsattn_build_mask_topk", "bsattn_build_mask_threshold", "bsattn_mask_to_indices",
    "bsattn_fwd_workspace_bytes", "bsattn_fwd_max_key_blocks", "bsattn_fwd", "bsattn_fwd_indices",
    "bsattn_fwd_chunk", "bsattn_fwd_topk", "bsattn_fwd_threshold",
    "bsattn_decode_num_splits", "bsattn_decode_default_splits", "bsattn_decode_workspace_bytes",
    "bsattn_decode_gqa", "bsattn_decode_gqa_noalloc", "bsattn_decode_noalloc_scratch_bytes",
    "bsattn_decode_gqa_mask", "bsattn_decode_gqa_paged",
    "bsattn_xattn_workspace_bytes", "bsattn_xattn_block_sums", "bsattn_build_mask_cumulative",
    "bsattn_xattn_estimate", "EXPORTED_SYMBOLS",
]

BLOCK = 64
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbsattn.so")

EXPORTED_SYMBOLS = (
    "bsattn_status_string", "bsattn_version", "bsattn_build_mask_topk",
    "bsattn_build_mask_threshold", "bsattn_mask_to_indices", "bsattn_fwd_workspace_bytes",
    "bsattn_fwd", "bsattn_fwd_indices", "bsattn_decode_num_splits",
    "bsattn_decode_workspace_bytes", "bsattn_decode_gqa", "bsattn_decode_default_splits",
    "bsattn_decode_gqa_mask", "bsattn_decode_gqa_paged", "bsattn_fwd_chunk",
    "bsattn_fwd_topk", "bsattn_fwd_threshold", "bsattn_xattn_workspace_bytes",
    "bsattn_xattn_block_sums", "bsattn_build_mask_cumulative", "bsattn_xattn_estimate",
    "bsattn_decode_gqa_noalloc", "bsattn_decode_noalloc_scratch_bytes", "bsattn_fwd_max_key_blocks",
)

_STATUS = {0: "BSATTN_OK", 1: "BSATTN_ERR_NULL", 2: "BSATTN_ERR_SHAPE",
           3: "BSATTN_ERR_UNSUPPORTED", 4: "BSATTN_ERR_WORKSPACE", 5: "BSATTN_ERR_HIP"}


class BsattnError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {_STATUS.get(status, status)}: {msg}")
        self.status = status


_lib: Optional[ctypes.CDLL] = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_Z = ctypes.c_size_t

_SIGS = {
    "bsattn_status_string": (ctypes.c_char_p, [_I]),
    "bsattn_version": (ctypes.c_char_p, []),
    "bsattn_build_mask_topk": (_I, [_P, _I, _I, _I, _I, _I, _I, _P, _P]),
    "bsattn_build_mask_threshold": (_I, [_P, _I, _I, _I, _F, _I, _I, _P, _P]),
    "bsattn_mask_to_indices": (_I, [_P, _I, _I, _I, _I, _P, _P, _P]),
    "bsattn_fwd_workspace_bytes": (_Z, [_I, _I, _I, _I]),
    "bsattn_fwd_max_key_blocks": (_I, [_I]),
    "bsattn_fwd": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _Z, _P]),
    "bsattn_fwd_indices": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P]),
    "bsattn_fwd_chunk": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P]),
    "bsattn_fwd_topk": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _Z, _P]),
    "bsattn_fwd_threshold": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _I, _P, _P, _P, _Z,
                                  _P]),
    "bsattn_decode_num_splits": (_I, [_I, _I, _I, _I, _I, _I]),
    "bsattn_decode_default_splits": (_I, [_I, _I, _I, _I, _I]),
    "bsattn_decode_workspace_bytes": (_Z, [_I, _I, _I, _I]),
    "bsattn_decode_gqa": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _Z, _P]),
    "bsattn_decode_gqa_noalloc": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P]),
    "bsattn_decode_noalloc_scratch_bytes": (_Z, []),
    "bsattn_decode_gqa_mask": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _Z, _P]),
    "bsattn_decode_gqa_paged": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I,
                                     _P, _P, _Z, _P]),
    "bsattn_xattn_workspace_bytes": (_Z, [_I, _I, _I, _I, _I]),
    "bsattn_xattn_block_sums": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _Z, _P]),
    "bsattn_build_mask_cumulative": (_I, [_P, _I, _I, _I, _I, _F, _I, _I, _I, _P, _P]),
    "bsattn_xattn_estimate": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _F, _F, _I, _I, _I, _P, _P, _P,
                                   _Z, _P]),
}


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libbsattn.so (once) and declare the C signatures.  Raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m block_sparse_attention_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def bsattn_status_string(status: int) -> str:
    return load_library().bsattn_status_string(status).decode()


def bsattn_version() -> str:
    return load_library().bsattn_version().decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise BsattnError(fn, status, bsattn_status_string(status))


def _torch():
    import torch
    return torch


def _dev(t, name: str, dtype, ndim: Optional[int] = None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims (got {tuple(t.shape)})")
    return t


def _stream(stream) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _empty(shape, dtype, device, stream):
    """A new device tensor owned by the stream the call runs on.  The caching
    allocator then hands its memory to another stream only after the work
    queued on `stream` is done with it, so temporaries (workspaces) dropped
    on return stay intact while the kernels still read or write them."""
    torch = _torch()
    if stream is None:
        return torch.empty(shape, dtype=dtype, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


def _ptr(t) -> int:
    return int(t.data_ptr())


def bsattn_build_mask_topk(scores, topk: int, dense_last_two_rows: bool = False,
                           force_diagonal: bool = True, out=None, stream=None):
    """scores float32 [B,H,nb,nb] -> uint8 0/1 mask (TileLang block-sparse guide §3.1)."""
    torch = _torch()
    _dev(scores, "scores", torch.float32, 4)
    B, H, nb, nb2 = scores.shape
    if nb != nb2:
        raise ValueError("scores must be [B, H, nb, nb]")
    if out is None:
        out = _empty((B, H, nb, nb), torch.uint8, scores.device, stream)
    _dev(out, "out", torch.uint8, 4)
    _check("bsattn_build_mask_topk", load_library().bsattn_build_mask_topk(
        _ptr(scores), B, H, nb, int(topk), int(bool(dense_last_two_rows)),
        int(bool(force_diagonal)), _ptr(out), _stream(stream)))
    return out


def bsattn_build_mask_threshold(scores, threshold: float, dense_last_two_rows: bool = False,
                                force_diagonal: bool = True, out=None, stream=None):
    """scores float32 [B,H,nb,nb] -> uint8 0/1 mask, score > threshold (guide §3.2)."""
    torch = _torch()
    _dev(scores, "scores", torch.float32, 4)
    B, H, nb, nb2 = scores.shape
    if nb != nb2:
        raise ValueError("scores must be [B, H, nb, nb]")
    if out is None:
        out = _empty((B, H, nb, nb), torch.uint8, scores.device, stream)
    _dev(out, "out", torch.uint8, 4)
    _check("bsattn_build_mask_threshold", load_library().bsattn_build_mask_threshold(
        _ptr(scores), B, H, nb, float(threshold), int(bool(dense_last_two_rows)),
        int(bool(force_diagonal)), _ptr(out), _stream(stream)))
    return out


def bsattn_mask_to_indices(mask, is_causal: bool = True, idx=None, cnt=None,
                           stream=None) -> Tuple[object, object]:
    """uint8 mask [B,H,nb,nb] -> (idx int32 [B,H,nb,nb] ascending, -1 padded; cnt int32 [B,H,nb]).
    idx / cnt may be given (written in place)."""
    torch = _torch()
    _dev(mask, "mask", torch.uint8, 4)
    B, H, nb, _ = mask.shape
    if idx is None:
        idx = _empty((B, H, nb, nb), torch.int32, mask.device, stream)
    if cnt is None:
        cnt = _empty((B, H, nb), torch.int32, mask.device, stream)
    _dev(idx, "idx", torch.int32, 4)
    _dev(cnt, "cnt", torch.int32, 3)
    if tuple(idx.shape) != (B, H, nb, nb) or tuple(cnt.shape) != (B, H, nb):
        raise ValueError("idx must be [B,H,nb,nb] and cnt [B,H,nb]")
    _check("bsattn_mask_to_indices", load_library().bsattn_mask_to_indices(
        _ptr(mask), B, H, nb, int(bool(is_causal)), _ptr(idx), _ptr(cnt), _stream(stream)))
    return idx, cnt


def bsattn_fwd_workspace_bytes(B: int, H: int, S: int, D: int) -> int:
    return int(load_library().bsattn_fwd_workspace_bytes(B, H, S, D))


def bsattn_fwd_max_key_blocks(D: int) -> int:
    """Most key blocks ceil(Sk/64) a forward call takes at head dim D (0: D unsupported)."""
    return int(load_library().bsattn_fwd_max_key_blocks(D))


def _qkv(q, k, v):
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev(t, name, torch.bfloat16, 4)
    if q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one [B, H, S, D] shape")
    return q.shape


def bsattn_fwd(q, k, v, block_mask, is_causal: bool = True, out=None, workspace=None, stream=None):
    """Block-sparse attention forward (guide §4).  q,k,v bf16 [B,H,S,D]; mask uint8 [B,H,nb,nb].

    Causal calls with more than 128 key blocks split long rows in two and need
    a device workspace of bsattn_fwd_workspace_bytes(B, H, S, D) bytes; when
    `workspace` is None one is allocated for the call."""
    torch = _torch()
    B, H, S, D = _qkv(q, k, v)
    _dev(block_mask, "block_mask", torch.uint8, 4)
    nb = -(-S // BLOCK)
    if tuple(block_mask.shape) != (B, H, nb, nb):
        raise ValueError(f"block_mask must be [{B}, {H}, {nb}, {nb}]")
    if out is None:
        out = _empty(q.shape, q.dtype, q.device, stream)
    _dev(out, "out", torch.bfloat16, 4)
    ws_ptr, ws_bytes = _split_workspace(B, H, S, D, is_causal, workspace, q.device, stream)
    _check("bsattn_fwd", load_library().bsattn_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(block_mask), B, H, S, D, int(bool(is_causal)),
        _ptr(out), ws_ptr, ws_bytes, _stream(stream)))
    return out


def _split_workspace(B, H, S, D, is_causal, workspace, device, stream):
    """(pointer, bytes) of the long-row split workspace: the caller's, or one
    allocated for the call when the split needs one and none was given."""
    need = bsattn_fwd_workspace_bytes(B, H, S, D)
    if not need or not (is_causal or workspace is not None):
        return 0, 0
    if workspace is None:
        workspace = _empty(need, _torch().uint8, device, stream)
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def bsattn_fwd_indices(q, k, v, idx, cnt, is_causal: bool = True, out=None, stream=None):
    """Forward pass from precomputed lists (output of bsattn_mask_to_indices)."""
    torch = _torch()
    B, H, S, D = _qkv(q, k, v)
    nb = -(-S // BLOCK)
    _dev(idx, "idx", torch.int32, 4)
    _dev(cnt, "cnt", torch.int32, 3)
    if tuple(idx.shape) != (B, H, nb, nb) or tuple(cnt.shape) != (B, H, nb):
        raise ValueError("idx must be [B,H,nb,nb] and cnt [B,H,nb]")
    if out is None:
        out = _empty(q.shape, q.dtype, q.device, stream)
    _dev(out, "out", torch.bfloat16, 4)
    _check("bsattn_fwd_indices", load_library().bsattn_fwd_indices(
        _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(cnt), B, H, S, D, int(bool(is_causal)),
        _ptr(out), _stream(stream)))
    return out


FUSED_MAX_BLOCKS = 256   # the one-launch fused forms hold a row of up to 256 key blocks


def _fused_setup(q, k, v, scores, out, mask_out, write_mask, stream):
    torch = _torch()
    B, H, S, D = _qkv(q, k, v)
    nb = -(-S // BLOCK)
    _dev(scores, "scores", torch.float32, 4)
    if tuple(scores.shape) != (B, H, nb, nb):
        raise ValueError("block scores must be [B, H, nb, nb]")
    if out is None:
        out = _empty(q.shape, q.dtype, q.device, stream)
    _dev(out, "out", torch.bfloat16, 4)
    mask = mask_out
    if mask is None and (write_mask or nb > FUSED_MAX_BLOCKS):
        # past FUSED_MAX_BLOCKS key blocks the call runs as builder + forward
        # and needs a mask buffer between the two
        mask = _empty((B, H, nb, nb), torch.uint8, q.device, stream)
    if mask is not None:
        _dev(mask, "mask_out", torch.uint8, 4)
        if tuple(mask.shape) != (B, H, nb, nb):
            raise ValueError("mask_out must be [B, H, nb, nb]")
    return B, H, S, D, out, mask


def bsattn_fwd_topk(q, k, v, scores, topk: int, dense_last_two_rows: bool = False,
                    force_diagonal: bool = True, is_causal: bool = True, out=None,
                    mask_out=None, write_mask: bool = False, workspace=None, stream=None):
    """Top-k mask build + compaction + forward in one launch (guide §3.1, §4).
    The mask goes to mask_out when given (or to a new tensor with write_mask).
    Long causal rows split as in bsattn_fwd (workspace as there).
    Returns out, or (out, mask) with write_mask."""
    B, H, S, D, out, mask = _fused_setup(q, k, v, scores, out, mask_out, write_mask, stream)
    ws_ptr, ws_bytes = _split_workspace(B, H, S, D, is_causal, workspace, q.device, stream)
    _check("bsattn_fwd_topk", load_library().bsattn_fwd_topk(
        _ptr(q), _ptr(k), _ptr(v), _ptr(scores), B, H, S, D, int(topk),
        int(bool(dense_last_two_rows)), int(bool(force_diagonal)), int(bool(is_causal)),
        _ptr(mask) if mask is not None else None, _ptr(out), ws_ptr, ws_bytes, _stream(stream)))
    return (out, mask) if write_mask else out


def bsattn_fwd_threshold(q, k, v, scores, threshold: float, dense_last_two_rows: bool = False,
                         force_diagonal: bool = True, is_causal: bool = True, out=None,
                         mask_out=None, write_mask: bool = False, workspace=None, stream=None):
    """Threshold mask build + compaction + forward in one launch (guide §3.2, §4).
    Long causal rows split as in bsattn_fwd (workspace as there)."""
    B, H, S, D, out, mask = _fused_setup(q, k, v, scores, out, mask_out, write_mask, stream)
    ws_ptr, ws_bytes = _split_workspace(B, H, S, D, is_causal, workspace, q.device, stream)
    _check("bsattn_fwd_threshold", load_library().bsattn_fwd_threshold(
        _ptr(q), _ptr(k), _ptr(v), _ptr(scores), B, H, S, D, float(threshold),
        int(bool(dense_last_two_rows)), int(bool(force_diagonal)), int(bool(is_causal)),
        _ptr(mask) if mask is not None else None, _ptr(out), ws_ptr, ws_bytes, _stream(stream)))
    return (out, mask) if write_mask else out


def bsattn_fwd_chunk(q, k, v, block_mask, is_causal: bool = True, out=None, stream=None):
    """Forward pass for Sq queries at the end of an Sk-token context (Sq <= Sk):
    q bf16 [B,H,Sq,D]; k, v bf16 [B,H,Sk,D]; block_mask uint8/bool
    [B,H,ceil(Sq/64),ceil(Sk/64)].  Causal rows see keys t <= row + Sk - Sq."""
    torch = _torch()
    _dev(q, "q", torch.bfloat16, 4)
    _dev(k, "k", torch.bfloat16, 4)
    _dev(v, "v", torch.bfloat16, 4)
    B, H, Sq, D = q.shape
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != D or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [B, H, Sk, D] matching q")
    Sk = k.shape[2]
    if block_mask.dtype == torch.bool:
        block_mask = block_mask.view(torch.uint8)
    _dev(block_mask, "block_mask", torch.uint8, 4)
    if tuple(block_mask.shape) != (B, H, -(-Sq // BLOCK), -(-Sk // BLOCK)):
        raise ValueError("block_mask must be [B, H, ceil(Sq/64), ceil(Sk/64)]")
    if out is None:
        out = _empty(q.shape, q.dtype, q.device, stream)
    _dev(out, "out", torch.bfloat16, 4)
    _check("bsattn_fwd_chunk", load_library().bsattn_fwd_chunk(
        _ptr(q), _ptr(k), _ptr(v), _ptr(block_mask), B, H, Sq, Sk, D, int(bool(is_causal)),
        _ptr(out), _stream(stream)))
    return out


def bsattn_decode_num_splits(B: int, Hq: int, Hkv: int, max_selected_blocks: int, D: int,
                             num_cus: int) -> int:
    return int(load_library().bsattn_decode_num_splits(B, Hq, Hkv, max_selected_blocks, D, num_cus))


def bsattn_decode_default_splits(B: int, Hq: int, Hkv: int, max_selected_blocks: int, D: int) -> int:
    return int(load_library().bsattn_decode_default_splits(B, Hq, Hkv, max_selected_blocks, D))


def bsattn_decode_workspace_bytes(B: int, Hq: int, D: int, num_splits: int) -> int:
    return int(load_library().bsattn_decode_workspace_bytes(B, Hq, D, num_splits))


def _decode_common(q, Hkv, Dv, slots, num_splits, out, workspace, stream):
    torch = _torch()
    B, Hq, D = q.shape
    ns = int(num_splits)
    if ns <= 0:
        ns = bsattn_decode_default_splits(B, Hq, Hkv, slots, D)
        if ns <= 0:
            raise BsattnError("bsattn_decode_default_splits", 5, "could not query the device")
    if out is None:
        out = _empty((B, Hq, Dv), torch.bfloat16, q.device, stream)
    _dev(out, "out", torch.bfloat16, 3)
    if tuple(out.shape) != (B, Hq, Dv):
        raise ValueError(f"out must be [{B}, {Hq}, {Dv}]")
    need = bsattn_decode_workspace_bytes(B, Hq, Dv, ns)
    ws_ptr, ws_bytes = 0, 0
    if need:
        if workspace is None:
            workspace = _empty(need, torch.uint8, q.device, stream)
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    return ns, out, ws_ptr, ws_bytes


def _decode_packed_checks(q, k, v, cu_seqlens_k):
    torch = _torch()
    _dev(q, "q", torch.bfloat16, 3)
    _dev(k, "k", torch.bfloat16, 3)
    _dev(v, "v", torch.bfloat16, 3)
    _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1)
    B, Hq, D = q.shape
    total_k, Hkv, Dk = k.shape
    if Dk != D or v.shape[0] != total_k or v.shape[1] != Hkv:
        raise ValueError("k must be [total_k, Hkv, D] with the query's D and v [total_k, Hkv, Dv]")
    if cu_seqlens_k.numel() != B + 1:
        raise ValueError("cu_seqlens_k must be [B+1]")
    return B, Hq, Hkv, D, v.shape[2], total_k


def bsattn_decode_gqa(q, k, v, cu_seqlens_k, block_indices, num_splits: int = 0, out=None,
                      workspace=None, stream=None):
    """Split-KV sparse GQA decode (guide §6).  q bf16 [B,Hq,D]; k,v bf16 [total_k,Hkv,D];
    cu_seqlens_k int32 [B+1]; block_indices int32 [B,Hkv,max_sel] (-1 = empty)."""
    torch = _torch()
    B, Hq, Hkv, D, Dv, total_k = _decode_packed_checks(q, k, v, cu_seqlens_k)
    _dev(block_indices, "block_indices", torch.int32, 3)
    if block_indices.shape[0] != B or block_indices.shape[1] != Hkv:
        raise ValueError("block_indices must be [B, Hkv, max_sel]")
    max_sel = block_indices.shape[2]
    ns, out, ws_ptr, ws_bytes = _decode_common(q, Hkv, Dv, max_sel, num_splits, out, workspace, stream)
    _check("bsattn_decode_gqa", load_library().bsattn_decode_gqa(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_k), _ptr(block_indices), B, Hq, Hkv, D, Dv,
        max_sel, total_k, ns, _ptr(out), ws_ptr, ws_bytes, _stream(stream)))
    return out


def bsattn_decode_noalloc_scratch_bytes() -> int:
    return int(load_library().bsattn_decode_noalloc_scratch_bytes())


def bsattn_decode_gqa_noalloc(q, k, v, cu_seqlens_k, block_indices, num_splits: int = 0, out=None,
                              stream=None):
    """bsattn_decode_gqa whose split partials live in the library's static
    scratch array (no workspace; the C call allocates nothing).  Calls that
    overlap in time on one GPU share that array and must not overlap."""
    torch = _torch()
    B, Hq, Hkv, D, Dv, total_k = _decode_packed_checks(q, k, v, cu_seqlens_k)
    _dev(block_indices, "block_indices", torch.int32, 3)
    if block_indices.shape[0] != B or block_indices.shape[1] != Hkv:
        raise ValueError("block_indices must be [B, Hkv, max_sel]")
    max_sel = block_indices.shape[2]
    if out is None:
        out = _empty((B, Hq, Dv), torch.bfloat16, q.device, stream)
    _dev(out, "out", torch.bfloat16, 3)
    if tuple(out.shape) != (B, Hq, Dv):
        raise ValueError(f"out must be [{B}, {Hq}, {Dv}]")
    _check("bsattn_decode_gqa_noalloc", load_library().bsattn_decode_gqa_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_k), _ptr(block_indices), B, Hq, Hkv, D, Dv,
        max_sel, total_k, int(num_splits), _ptr(out), _stream(stream)))
    return out


def bsattn_decode_gqa_mask(q, k, v, cu_seqlens_k, block_mask, num_splits: int = 0, out=None,
                           workspace=None, stream=None):
    """Mask-form sparse GQA decode (guide §6).  As bsattn_decode_gqa, with
    block_mask uint8/bool [B,Hkv,num_blocks] (nonzero = block selected)."""
    torch = _torch()
    B, Hq, Hkv, D, Dv, total_k = _decode_packed_checks(q, k, v, cu_seqlens_k)
    if block_mask.dtype == torch.bool:
        block_mask = block_mask.view(torch.uint8)
    _dev(block_mask, "block_mask", torch.uint8, 3)
    if block_mask.shape[0] != B or block_mask.shape[1] != Hkv:
        raise ValueError("block_mask must be [B, Hkv, num_blocks]")
    nblocks = block_mask.shape[2]
    ns, out, ws_ptr, ws_bytes = _decode_common(q, Hkv, Dv, nblocks, num_splits, out, workspace, stream)
    _check("bsattn_decode_gqa_mask", load_library().bsattn_decode_gqa_mask(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_k), _ptr(block_mask), B, Hq, Hkv, D, Dv,
        nblocks, total_k, ns, _ptr(out), ws_ptr, ws_bytes, _stream(stream)))
    return out


def bsattn_decode_gqa_paged(q, k_cache, v_cache, cache_seqlens, block_table, block_indices,
                            num_splits: int = 0, out=None, workspace=None, stream=None):
    """Paged-KV sparse GQA decode (guide §7).  q bf16 [B,Hq,D]; k_cache, v_cache bf16
    [num_pages,page_size,Hkv,D]; cache_seqlens int32 [B]; block_table int32
    [B,max_blocks_per_seq]; block_indices int32 [B,Hkv,max_sel] (logical 64-token blocks)."""
    torch = _torch()
    _dev(q, "q", torch.bfloat16, 3)
    _dev(k_cache, "k_cache", torch.bfloat16, 4)
    _dev(v_cache, "v_cache", torch.bfloat16, 4)
    _dev(cache_seqlens, "cache_seqlens", torch.int32, 1)
    _dev(block_table, "block_table", torch.int32, 2)
    _dev(block_indices, "block_indices", torch.int32, 3)
    B, Hq, D = q.shape
    num_pages, page_size, Hkv, Dk = k_cache.shape
    if tuple(v_cache.shape[:3]) != tuple(k_cache.shape[:3]) or Dk != D:
        raise ValueError("k_cache must be [num_pages, page_size, Hkv, D] and v_cache "
                         "[num_pages, page_size, Hkv, Dv]")
    Dv = v_cache.shape[3]
    if cache_seqlens.numel() != B or block_table.shape[0] != B:
        raise ValueError("cache_seqlens must be [B] and block_table [B, max_blocks_per_seq]")
    if block_indices.shape[0] != B or block_indices.shape[1] != Hkv:
        raise ValueError("block_indices must be [B, Hkv, max_sel]")
    max_sel = block_indices.shape[2]
    ns, out, ws_ptr, ws_bytes = _decode_common(q, Hkv, Dv, max_sel, num_splits, out, workspace, stream)
    _check("bsattn_decode_gqa_paged", load_library().bsattn_decode_gqa_paged(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_seqlens), _ptr(block_table),
        _ptr(block_indices), B, Hq, Hkv, D, Dv, num_pages, page_size, block_table.shape[1], max_sel,
        ns, _ptr(out), ws_ptr, ws_bytes, _stream(stream)))
    return out


# ---- XAttention block-importance estimator ----

def bsattn_xattn_workspace_bytes(B: int, H: int, Sq: int, Sk: int, stride: int) -> int:
    return int(load_library().bsattn_xattn_workspace_bytes(B, H, Sq, Sk, stride))


def _xattn_qk(q, k):
    torch = _torch()
    _dev(q, "q", torch.bfloat16, 4)
    _dev(k, "k", torch.bfloat16, 4)
    B, H, Sq, D = q.shape
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != D:
        raise ValueError("q [B, H, Sq, D] and k [B, H, Sk, D] must agree on B, H, D")
    return B, H, Sq, k.shape[2], D


def _xattn_ws(B, H, Sq, Sk, stride, workspace, device, stream):
    torch = _torch()
    need = bsattn_xattn_workspace_bytes(B, H, Sq, Sk, stride)
    if workspace is None:
        workspace = _empty(max(need, 1), torch.uint8, device, stream)
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def bsattn_xattn_block_sums(q, k, stride: int = 8, norm: float = 1.0, is_causal: bool = True,
                            out=None, workspace=None, stream=None):
    """XAttention block estimate (XAttention guide, phases 1-2): q bf16 [B,H,Sq,D],
    k bf16 [B,H,Sk,D] -> float32 block sums [B,H,ceil(Sq/64),ceil(Sk/64)]."""
    torch = _torch()
    B, H, Sq, Sk, D = _xattn_qk(q, k)
    nbq, nbk = -(-Sq // BLOCK), -(-Sk // BLOCK)
    if out is None:
        out = _empty((B, H, nbq, nbk), torch.float32, q.device, stream)
    _dev(out, "out", torch.float32, 4)
    ws_ptr, ws_bytes = _xattn_ws(B, H, Sq, Sk, stride, workspace, q.device, stream)
    _check("bsattn_xattn_block_sums", load_library().bsattn_xattn_block_sums(
        _ptr(q), _ptr(k), B, H, Sq, Sk, D, int(stride), float(norm), int(bool(is_causal)),
        _ptr(out), ws_ptr, ws_bytes, _stream(stream)))
    return out


def bsattn_build_mask_cumulative(block_sums, threshold: float = 0.9, keep_sink: bool = True,
                                 keep_diagonal: bool = True, is_causal: bool = True, out=None,
                                 stream=None):
    """float32 [B,H,nbq,nbk] -> uint8 0/1 mask, selection by cumulative weight
    (XAttention guide, block-selection section)."""
    torch = _torch()
    _dev(block_sums, "block_sums", torch.float32, 4)
    B, H, nbq, nbk = block_sums.shape
    if out is None:
        out = _empty((B, H, nbq, nbk), torch.uint8, block_sums.device, stream)
    _dev(out, "out", torch.uint8, 4)
    _check("bsattn_build_mask_cumulative", load_library().bsattn_build_mask_cumulative(
        _ptr(block_sums), B, H, nbq, nbk, float(threshold), int(bool(keep_sink)),
        int(bool(keep_diagonal)), int(bool(is_causal)), _ptr(out), _stream(stream)))
    return out


def bsattn_xattn_estimate(q, k, stride: int = 8, norm: float = 1.0, threshold: float = 0.9,
                          keep_sink: bool = True, keep_diagonal: bool = True,
                          is_causal: bool = True, block_sums=None, write_sums: bool = False,
                          out=None, workspace=None, stream=None):
    """The whole estimator (XAttention guide, phases 1-3) -> uint8 mask [B,H,nbq,nbk],
    or (mask, block_sums) when block_sums is given or write_sums is set."""
    torch = _torch()
    B, H, Sq, Sk, D = _xattn_qk(q, k)
    nbq, nbk = -(-Sq // BLOCK), -(-Sk // BLOCK)
    if out is None:
        out = _empty((B, H, nbq, nbk), torch.uint8, q.device, stream)
    _dev(out, "out", torch.uint8, 4)
    if block_sums is None and write_sums:
        block_sums = _empty((B, H, nbq, nbk), torch.float32, q.device, stream)
    if block_sums is not None:
        _dev(block_sums, "block_sums", torch.float32, 4)
    ws_ptr, ws_bytes = _xattn_ws(B, H, Sq, Sk, stride, workspace, q.device, stream)
    _check("bsattn_xattn_estimate", load_library().bsattn_xattn_estimate(
        _ptr(q), _ptr(k), B, H, Sq, Sk, D, int(stride), float(norm), float(threshold),
        int(bool(keep_sink)), int(bool(keep_diagonal)), int(bool(is_causal)),
        None if block_sums is None else _ptr(block_sums), _ptr(out), ws_ptr, ws_bytes,
        _stream(stream)))
    return out if block_sums is None else (out, block_sums)
