"""MI355X (gfx950) MLA speculative-decoding verify attention.

Thin ctypes binding over ``libverify_attn.so`` (C ABI in ``include/verify_attn.h``).
This module only marshals arguments: every step of the computation runs in the
HIP kernels. PyTorch is used for device memory and streams. The library must be
built first (``python -m speculative_decoding_verify_03_amd.build``); there is
no fallback path, and calling into a missing library raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Tuple

LATENT_DIM = 576
VALUE_DIM = 512
MAX_Q = 64

VA_OK, VA_EINVAL, VA_ENOSPC, VA_EHIP = 0, -1, -2, -3

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_lib", "libverify_attn.so")
EXPORTED = (
    "verify_attn",
    "verify_attn_workspace_size",
    "verify_attn_last_error",
    "verify_attn_kv_defrag",
    "verify_attn_tree_accept",
    "verify_attn_noalloc",
    # test and measurement interface (include/verify_attn_testing.h)
    "verify_attn_ex",
    "verify_attn_workspace_size_ex",
    "verify_attn_query_plan",
    "verify_attn_debug_gather",
)


class _TestOptions(ctypes.Structure):
    """va_test_options of include/verify_attn_testing.h."""
    _fields_ = [("chunk_keys", ctypes.c_int32), ("split_start_event", ctypes.c_void_p),
                ("split_stop_event", ctypes.c_void_p)]


_lib = None


class VerifyAttnError(RuntimeError):
    """A non-zero status from the library, with its message."""

    def __init__(self, code: int, msg: str):
        super().__init__(f"verify_attn status {code}: {msg}")
        self.code = code


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load (once) and type the C ABI. Raises if the library is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"HIP library not built: {path} is missing "
            "(run `python -m speculative_decoding_verify_03_amd.build`)")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    lib.verify_attn.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, i32, i32, i32, i64, i64,
                                vp, sz, vp]
    lib.verify_attn.restype = i32
    lib.verify_attn_workspace_size.argtypes = [i32, i32, i32, i64]
    lib.verify_attn_workspace_size.restype = sz
    lib.verify_attn_last_error.argtypes = []
    lib.verify_attn_last_error.restype = ctypes.c_char_p
    lib.verify_attn_noalloc.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, i32, i32, i32, i64, i64, vp]
    lib.verify_attn_noalloc.restype = i32
    lib.verify_attn_ex.argtypes = lib.verify_attn.argtypes + [ctypes.POINTER(_TestOptions)]
    lib.verify_attn_ex.restype = i32
    lib.verify_attn_workspace_size_ex.argtypes = [i32, i32, i32, i64, ctypes.c_int32]
    lib.verify_attn_workspace_size_ex.restype = sz
    lib.verify_attn_debug_gather.argtypes = [vp, vp, i64, i64, vp, vp]
    lib.verify_attn_debug_gather.restype = i32
    p32 = ctypes.POINTER(ctypes.c_int32)
    lib.verify_attn_query_plan.argtypes = [i32, i32, i32, i64, ctypes.c_int32, p32, p32, p32, p32]
    lib.verify_attn_query_plan.restype = i32
    lib.verify_attn_kv_defrag.argtypes = [vp, vp, i64, i64, vp, i64, i64, vp, vp]
    lib.verify_attn_kv_defrag.restype = i32
    lib.verify_attn_tree_accept.argtypes = [vp, vp, vp, i32, i32, vp, vp, vp, vp]
    lib.verify_attn_tree_accept.restype = i32
    _lib = lib
    return lib


def _check(code: int) -> None:
    if code != VA_OK:
        raise VerifyAttnError(code, load_library().verify_attn_last_error().decode())


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream_handle(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def workspace_size(B: int, Q: int, H: int, total_kv: int, chunk_keys: int = 0) -> int:
    """Workspace bytes of a call (chunk_keys > 0: with that forced chunk length)."""
    lib = load_library()
    if chunk_keys:
        n = lib.verify_attn_workspace_size_ex(B, Q, H, total_kv, int(chunk_keys))
    else:
        n = lib.verify_attn_workspace_size(B, Q, H, total_kv)
    if n == 0:
        raise VerifyAttnError(VA_EINVAL, f"invalid sizes B={B} Q={Q} H={H} total_kv={total_kv} "
                                         f"chunk_keys={chunk_keys}")
    return int(n)


def query_plan(B: int, Q: int, H: int, total_kv: int, chunk_keys: int = 0) -> Dict[str, int]:
    vals = [ctypes.c_int32() for _ in range(4)]
    _check(load_library().verify_attn_query_plan(B, Q, H, total_kv, int(chunk_keys),
                                                 *[ctypes.byref(v) for v in vals]))
    return dict(zip(("chunk_keys", "max_chunks", "row_tiles", "grid"), (v.value for v in vals)))


def alloc_workspace(B: int, Q: int, H: int, total_kv: int, device="cuda", chunk_keys: int = 0):
    import torch
    return torch.empty(workspace_size(B, Q, H, total_kv, chunk_keys), dtype=torch.uint8, device=device)


def verify_attn(q, kv_pool, kv_indices, prefix_lens, tree_mask, scale: float,
                out=None, lse=None, workspace=None, stream=None, chunk_keys: int = 0,
                split_events=None) -> Tuple[object, object]:
    """Verify attention over a paged MLA latent cache (see include/verify_attn.h).

    q: bf16 (or int16 bit patterns) [B, Q, H, 576]; kv_pool: bf16 [S, 576];
    kv_indices: int32 [total_kv]; prefix_lens: int32 [B]; tree_mask: uint8
    [B, Q, Q]; all CUDA tensors, contiguous. Returns (out fp32 [B, Q, H, 512],
    lse fp32 [B, Q, H]). Asynchronous on ``stream`` (default: current stream).

    Test and measurement options (include/verify_attn_testing.h), per call:
    ``chunk_keys`` > 0 forces the keys per chunk; ``split_events`` = (start,
    stop) torch.cuda.Events (either may be None) recorded around the split
    kernel. With neither, the plain ``verify_attn`` entry point is called.
    """
    import torch
    lib = load_library()
    B, Q, H, D = q.shape
    if D != LATENT_DIM or kv_pool.shape[-1] != LATENT_DIM:
        raise ValueError("q and kv_pool rows must have 576 elements")
    for name, t in (("q", q), ("kv_pool", kv_pool), ("kv_indices", kv_indices),
                    ("prefix_lens", prefix_lens), ("tree_mask", tree_mask)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous CUDA tensor")
    if q.element_size() != 2 or kv_pool.element_size() != 2:
        raise ValueError("q and kv_pool must hold 16-bit (bf16) elements")
    if kv_indices.dtype != torch.int32 or prefix_lens.dtype != torch.int32:
        raise ValueError("kv_indices and prefix_lens must be int32")
    if tree_mask.dtype != torch.uint8 or tuple(tree_mask.shape) != (B, Q, Q):
        raise ValueError("tree_mask must be uint8 [B, Q, Q]")
    if tuple(prefix_lens.shape) != (B,):
        raise ValueError("prefix_lens must be [B]")
    total_kv = int(kv_indices.numel())
    if out is None:
        out = torch.empty((B, Q, H, VALUE_DIM), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Q, H), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(B, Q, H, total_kv, device=q.device, chunk_keys=chunk_keys)
    args = (_ptr(q), _ptr(kv_pool), _ptr(kv_indices), _ptr(prefix_lens), _ptr(tree_mask), float(scale),
            _ptr(out), _ptr(lse), B, Q, H, int(kv_pool.shape[0]), total_kv, _ptr(workspace),
            int(workspace.numel() * workspace.element_size()), _stream_handle(stream))
    if chunk_keys or split_events is not None:
        ev0, ev1 = split_events if split_events is not None else (None, None)
        h = lambda e: None if e is None else int(e.cuda_event)  # noqa: E731
        opts = _TestOptions(int(chunk_keys), h(ev0), h(ev1))
        code = lib.verify_attn_ex(*args, ctypes.byref(opts))
    else:
        code = lib.verify_attn(*args)
    _check(code)
    return out, lse


def verify_attn_noalloc(q, kv_pool, kv_indices, prefix_lens, tree_mask, scale: float, out, lse,
                        stream=None) -> Tuple[object, object]:
    """verify_attn through the allocation-free entry point: the library's fixed device
    scratch replaces the workspace, and the caller passes preallocated ``out`` (fp32
    [B, Q, H, 512]) and ``lse`` (fp32 [B, Q, H]). Calls that overlap on one device race."""
    import torch
    B, Q, H, D = q.shape
    for name, t in (("q", q), ("kv_pool", kv_pool), ("kv_indices", kv_indices), ("prefix_lens", prefix_lens),
                    ("tree_mask", tree_mask), ("out", out), ("lse", lse)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous CUDA tensor")
    if D != LATENT_DIM or kv_pool.shape[-1] != LATENT_DIM or q.element_size() != 2 or kv_pool.element_size() != 2:
        raise ValueError("q and kv_pool must be 16-bit [.., 576]")
    if kv_indices.dtype != torch.int32 or prefix_lens.dtype != torch.int32 or tree_mask.dtype != torch.uint8:
        raise ValueError("kv_indices and prefix_lens must be int32, tree_mask uint8")
    if tuple(tree_mask.shape) != (B, Q, Q) or tuple(prefix_lens.shape) != (B,):
        raise ValueError("tree_mask must be [B, Q, Q] and prefix_lens [B]")
    if out.dtype != torch.float32 or tuple(out.shape) != (B, Q, H, VALUE_DIM):
        raise ValueError("out must be fp32 [B, Q, H, 512]")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Q, H):
        raise ValueError("lse must be fp32 [B, Q, H]")
    _check(load_library().verify_attn_noalloc(_ptr(q), _ptr(kv_pool), _ptr(kv_indices), _ptr(prefix_lens),
                                              _ptr(tree_mask), float(scale), _ptr(out), _ptr(lse), B, Q, H,
                                              int(kv_pool.shape[0]), int(kv_indices.numel()),
                                              _stream_handle(stream)))
    return out, lse


def debug_gather(kv_pool, kv_indices, stream=None):
    """Rows [n, 576] (int16 bit patterns) produced by the split kernel's own gather."""
    import torch
    n = int(kv_indices.numel())
    rows = torch.empty((n, LATENT_DIM), dtype=torch.int16, device=kv_pool.device)
    _check(load_library().verify_attn_debug_gather(_ptr(kv_pool), _ptr(kv_indices), n,
                                                   int(kv_pool.shape[0]), _ptr(rows),
                                                   _stream_handle(stream)))
    return rows


def kv_defrag(src_pool, kv_indices, dst_pool, dst_base: int, new_indices=None, stream=None):
    """Copy the rows kv_indices names into dst_pool[dst_base:dst_base+n] in position
    order and return the rewritten index table (see include/verify_attn.h)."""
    import torch
    for name, t in (("src_pool", src_pool), ("kv_indices", kv_indices), ("dst_pool", dst_pool)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous CUDA tensor")
    if kv_indices.dtype != torch.int32:
        raise ValueError("kv_indices must be int32")
    n = int(kv_indices.numel())
    if new_indices is None:
        new_indices = torch.empty(n, dtype=torch.int32, device=kv_indices.device)
    _check(load_library().verify_attn_kv_defrag(_ptr(src_pool), _ptr(kv_indices), n, int(src_pool.shape[0]),
                                                _ptr(dst_pool), int(dst_base), int(dst_pool.shape[0]),
                                                _ptr(new_indices), _stream_handle(stream)))
    return new_indices


def tree_accept(parents, draft_tokens, target_tokens, out=None, stream=None):
    """Greedy acceptance over draft trees, int32 [B, Q] inputs; returns
    (accept_len [B], accepted [B, Q], bonus_token [B]) (see include/verify_attn.h)."""
    import torch
    B, Q = parents.shape
    for name, t in (("parents", parents), ("draft_tokens", draft_tokens), ("target_tokens", target_tokens)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.int32 or tuple(t.shape) != (B, Q):
            raise ValueError(f"{name} must be a contiguous int32 CUDA tensor [B, Q]")
    if out is None:
        dev = parents.device
        out = (torch.empty(B, dtype=torch.int32, device=dev), torch.empty((B, Q), dtype=torch.int32, device=dev),
               torch.empty(B, dtype=torch.int32, device=dev))
    accept_len, accepted, bonus = out
    _check(load_library().verify_attn_tree_accept(_ptr(parents), _ptr(draft_tokens), _ptr(target_tokens), B, Q,
                                                  _ptr(accept_len), _ptr(accepted), _ptr(bonus),
                                                  _stream_handle(stream)))
    return accept_len, accepted, bonus
