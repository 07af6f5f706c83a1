"""Fused attention forward for MI355X (gfx950): Python binding of libattn.so.

Thin ctypes layer over the C ABI in include/attn.h.  The functions named
attn_* take raw device pointers and sizes and return the C status code,
exactly like their C counterparts.  `prefill()` and `decode()` marshal torch
tensors onto those calls: they check shapes, dtypes and devices, allocate the
output, pass torch's current HIP stream and keep a decode workspace per
(device, stream).  Every step of the computation runs in the HIP kernels; there is
no fallback path: the library is loaded on first use, and every entry point
raises ImportError if libattn.so has not been built.
"""
import contextlib
import ctypes
import math
import os
import threading

import torch

__all__ = [
    "ATTN_F32", "ATTN_BF16", "AttnError", "attn_prefill_fwd", "attn_decode_fwd",
    "attn_decode_paged_fwd", "attn_decode_noalloc_fwd", "ATTN_DECODE_NOALLOC_SCRATCH_BYTES",
    "attn_prefill_varlen_fwd", "attn_prefill_rope_fwd",
    "attn_prefill_rope_workspace_bytes", "attn_decode_workspace_bytes",
    "attn_status_str", "attn_last_hip_error", "prefill", "prefill_varlen", "decode",
    "decode_paged", "library_path", "lds_poison_library_path", "use_library",
]

ATTN_F32 = 0
ATTN_BF16 = 1
STATUS = {0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_UNSUPPORTED",
          4: "ATTN_ERR_ALIGN", 5: "ATTN_ERR_WORKSPACE", 6: "ATTN_ERR_HIP", 7: "ATTN_ERR_VALUE"}

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libattn.so")
# The same library with each direct global -> LDS copy preceded by a NaN fill
# of its destination (a debug build for the tests; see use_library).
lds_poison_library_path = os.path.join(_HERE, "libattn_lds_poison.so")

_lib = None
_lock = threading.Lock()


def _load():
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(library_path):
            raise ImportError(
                f"{library_path} is missing: build it with "
                "`python -m attention_attn_fwd_11_amd.build` (hipcc, gfx950)")
        _lib = _open(library_path)
    return _lib


def _open(path):
    """Load one build of the library and declare its entry points."""
    # torch is imported first so the library binds to the HIP runtime torch loaded.
    lib = ctypes.CDLL(path)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.attn_prefill_fwd.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32,
                                     vp, ctypes.c_int, vp]
    lib.attn_prefill_fwd.restype = ctypes.c_int
    lib.attn_decode_fwd.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32,
                                    vp, ctypes.c_int, vp, sz, vp]
    lib.attn_decode_fwd.restype = ctypes.c_int
    lib.attn_prefill_varlen_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                            i32, i32, i32, f32, ctypes.c_int, vp]
    lib.attn_prefill_varlen_fwd.restype = ctypes.c_int
    lib.attn_prefill_rope_fwd.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32,
                                          vp, vp, i32, vp, ctypes.c_size_t, ctypes.c_int, vp]
    lib.attn_prefill_rope_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.attn_prefill_rope_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_prefill_rope_fwd.restype = ctypes.c_int
    lib.attn_decode_noalloc_fwd.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                            f32, vp, ctypes.c_int, vp]
    lib.attn_decode_noalloc_fwd.restype = ctypes.c_int
    lib.attn_decode_paged_fwd.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, f32, vp, i32, i32,
                                          i32, vp, ctypes.c_int, vp, sz, vp]
    lib.attn_decode_paged_fwd.restype = ctypes.c_int
    lib.attn_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.attn_decode_workspace_bytes.restype = sz
    lib.attn_status_str.argtypes = [ctypes.c_int]
    lib.attn_status_str.restype = ctypes.c_char_p
    lib.attn_last_hip_error.argtypes = []
    lib.attn_last_hip_error.restype = ctypes.c_char_p
    return lib


@contextlib.contextmanager
def use_library(path):
    """Run the wrappers on another build of the library inside the block (the
    LDS-poison debug build, libattn_lds_poison.so, in the tests); the default
    build is back in use afterwards.  Not for concurrent use."""
    global _lib
    other = _open(path)
    with _lock:
        prev, _lib = _lib, other
    try:
        yield other
    finally:
        with _lock:
            _lib = prev


# ---------------------------------------------------------------------------
# Same-name wrappers of the C ABI (raw pointers as Python ints, C status out).
# ---------------------------------------------------------------------------
def attn_prefill_fwd(q, k, v, o, B, H_q, H_kv, S_q, S_kv, d, causal, scale, kv_lens, dtype, stream):
    return _load().attn_prefill_fwd(q, k, v, o, B, H_q, H_kv, S_q, S_kv, d, causal, scale, kv_lens,
                                    dtype, stream)


def attn_prefill_rope_fwd(q, k, v, o, B, H_q, H_kv, S_q, S_kv, d, causal, scale, kv_lens, rope_table,
                          rope_rows, workspace, workspace_bytes, dtype, stream):
    return _load().attn_prefill_rope_fwd(q, k, v, o, B, H_q, H_kv, S_q, S_kv, d, causal, scale,
                                         kv_lens, rope_table, rope_rows, workspace, workspace_bytes,
                                         dtype, stream)


def attn_prefill_rope_workspace_bytes(B, H_kv, S_kv, d):
    return _load().attn_prefill_rope_workspace_bytes(B, H_kv, S_kv, d)


def attn_prefill_varlen_fwd(q, k, v, o, cu_seqlens_q, cu_seqlens_k, B, H_q, H_kv, max_seqlen_q,
                            max_seqlen_k, total_q, total_k, d, causal, scale, dtype, stream):
    return _load().attn_prefill_varlen_fwd(q, k, v, o, cu_seqlens_q, cu_seqlens_k, B, H_q, H_kv,
                                           max_seqlen_q, max_seqlen_k, total_q, total_k, d, causal,
                                           scale, dtype, stream)


def attn_decode_fwd(q, k_cache, v_cache, o, B, H_q, H_kv, S_q, S_kv, d, causal, scale, kv_lens,
                    dtype, workspace, workspace_bytes, stream):
    return _load().attn_decode_fwd(q, k_cache, v_cache, o, B, H_q, H_kv, S_q, S_kv, d, causal,
                                   scale, kv_lens, dtype, workspace, workspace_bytes, stream)


def attn_decode_noalloc_fwd(q, k_cache, v_cache, o, B, H_q, H_kv, S_q, S_kv, d, causal, scale,
                            kv_lens, dtype, stream):
    return _load().attn_decode_noalloc_fwd(q, k_cache, v_cache, o, B, H_q, H_kv, S_q, S_kv, d,
                                           causal, scale, kv_lens, dtype, stream)


# Size of the static scratch behind attn_decode_noalloc_fwd (include/attn.h).
ATTN_DECODE_NOALLOC_SCRATCH_BYTES = 32 << 20


def attn_decode_paged_fwd(q, k_pages, v_pages, o, B, H_q, H_kv, d, scale, block_table, max_blocks,
                          page_size, num_pages, kv_lens, dtype, workspace, workspace_bytes, stream):
    return _load().attn_decode_paged_fwd(q, k_pages, v_pages, o, B, H_q, H_kv, d, scale,
                                         block_table, max_blocks, page_size, num_pages, kv_lens,
                                         dtype, workspace, workspace_bytes, stream)


def attn_decode_workspace_bytes(B, H_q, H_kv, S_kv, d):
    return int(_load().attn_decode_workspace_bytes(B, H_q, H_kv, S_kv, d))


def attn_status_str(status):
    return _load().attn_status_str(status).decode()


def attn_last_hip_error():
    return _load().attn_last_hip_error().decode()


class AttnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = f"{where}: {STATUS.get(status, status)} ({attn_status_str(status)})"
        if status == 6:
            msg += f": {attn_last_hip_error()}"
        super().__init__(msg)


# ---------------------------------------------------------------------------
# torch-facing helpers
# ---------------------------------------------------------------------------
_DTYPES = {torch.float32: ATTN_F32, torch.bfloat16: ATTN_BF16}
_workspaces = {}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_tensor(name, t, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _lens(kv_lens, B, device):
    if kv_lens is None:
        return None
    _check_tensor("kv_lens", kv_lens, torch.int32)
    if tuple(kv_lens.shape) != (B,) or kv_lens.device != device:
        raise ValueError("kv_lens must be int32 [B] on the same device as q")
    return kv_lens


def prefill(q, k, v, causal=True, scale=None, kv_lens=None, out=None, rope=None, rope_workspace=None):
    """Attention forward.  q [B,H_q,S_q,d]; k, v [B,H_kv,S_kv,d]; fp32 or bf16.

    Returns o [B,H_q,S_q,d] with q's dtype.  kv_lens (optional) is int32 [B]
    on the device.  rope (optional, bf16 only): fp32 [rows, d] cos/sin table;
    Q and K are then rotated (attn_prefill_rope_fwd): K inside the kernel,
    or, with rope_workspace (a uint8 device tensor of at least
    attn_prefill_rope_workspace_bytes bytes), once into that buffer first.
    Runs on torch's current stream for q's device.
    """
    if q.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, q.dtype)
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, S, d]")
    B, H_q, S_q, d = q.shape
    Bk, H_kv, S_kv, dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or dk != d:
        raise ValueError("inconsistent q/k/v shapes")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k, v must be on one device")
    lens = _lens(kv_lens, B, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = out if out is not None else torch.empty_like(q)
    _check_tensor("out", o, q.dtype)
    if o.shape != q.shape:
        raise ValueError("out must have q's shape")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    if rope is not None:
        _check_tensor("rope", rope, torch.float32)
        if rope.dim() != 2 or rope.shape[1] != d or rope.device != q.device:
            raise ValueError("rope must be float32 [rows, d] on q's device")
        ws, ws_bytes = None, 0
        if rope_workspace is not None:
            if not rope_workspace.is_cuda or rope_workspace.device != q.device:
                raise ValueError("rope_workspace must be on q's device")
            ws, ws_bytes = _ptr(rope_workspace), rope_workspace.numel() * rope_workspace.element_size()
        st = attn_prefill_rope_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H_q, H_kv, S_q, S_kv, d,
                                   int(bool(causal)), float(scale), _ptr(lens), _ptr(rope),
                                   rope.shape[0], ws, ws_bytes, _DTYPES[q.dtype],
                                   ctypes.c_void_p(stream))
        if st != 0:
            raise AttnError(st, "attn_prefill_rope_fwd")
        return o
    st = attn_prefill_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H_q, H_kv, S_q, S_kv, d,
                          int(bool(causal)), float(scale), _ptr(lens), _DTYPES[q.dtype],
                          ctypes.c_void_p(stream))
    if st != 0:
        raise AttnError(st, "attn_prefill_fwd")
    return o


def prefill_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, causal=True,
                   scale=None, out=None):
    """Attention over packed sequences.  q [total_q,H_q,d]; k, v [total_k,H_kv,d]
    (bf16); cu_seqlens_q / cu_seqlens_k int32 [B+1] on the device; the
    max_seqlen_* bound every sequence's length.  Returns o [total_q,H_q,d].
    Runs on torch's current stream for q's device."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, torch.bfloat16)
        if t.dim() != 3:
            raise ValueError(f"{name} must be [total, H, d]")
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        _check_tensor(name, t, torch.int32)
        if t.dim() != 1 or t.device != q.device:
            raise ValueError(f"{name} must be int32 [B+1] on q's device")
    if cu_seqlens_q.shape != cu_seqlens_k.shape:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    total_q, H_q, d = q.shape
    total_k, H_kv, dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or dk != d:
        raise ValueError("inconsistent q/k/v shapes")
    B = cu_seqlens_q.shape[0] - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = out if out is not None else torch.empty_like(q)
    _check_tensor("out", o, torch.bfloat16)
    if o.shape != q.shape:
        raise ValueError("out must have q's shape")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = attn_prefill_varlen_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(cu_seqlens_q),
                                 _ptr(cu_seqlens_k), B, H_q, H_kv, int(max_seqlen_q),
                                 int(max_seqlen_k), total_q, total_k, d, int(bool(causal)),
                                 float(scale), ATTN_BF16, ctypes.c_void_p(stream))
    if st != 0:
        raise AttnError(st, "attn_prefill_varlen_fwd")
    return o


def workspace_for(device, nbytes, stream=None):
    """Cached decode scratch buffer of at least nbytes for (device, stream).

    Calls that share a workspace must be ordered on one stream, so the cache
    keeps one buffer per (device, stream): decodes issued on different
    streams never share partials.  The buffer is allocated while its stream
    is current, so when it grows the caching allocator reuses the old memory
    only after the work already queued on that stream.  Under graph capture
    a cached buffer could be regrown (and freed) after the graph has baked
    in its address, so there the caller must pass `workspace=` and keep it
    alive as long as the graph.
    """
    dev = torch.device(device)
    if torch.cuda.is_current_stream_capturing():
        raise RuntimeError("decode under graph capture needs an explicit workspace= tensor that "
                           "outlives the graph (see attn_decode_workspace_bytes)")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    key = (dev.index, stream.cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        with torch.cuda.stream(stream):
            ws = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=dev)
        _workspaces[key] = ws
    return ws


def _decode_buffers(q, o, ws, need, others):
    """Checks shared by the decode wrappers: out has q's shape, dtype and
    device; the cache tensors and the workspace sit on q's device; the
    workspace is large enough.  Returns (o, ws)."""
    for name, t in others:
        if t.device != q.device:
            raise ValueError(f"{name} must be on q's device ({q.device}), got {t.device}")
    if o is None:
        o = torch.empty_like(q)
    _check_tensor("out", o, q.dtype)
    if o.shape != q.shape or o.device != q.device:
        raise ValueError("out must have q's shape and device")
    if ws is None:
        ws = workspace_for(q.device, need)
    else:
        if not isinstance(ws, torch.Tensor) or ws.device != q.device or not ws.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on q's device")
        if ws.numel() * ws.element_size() < need:
            raise ValueError(f"workspace holds {ws.numel() * ws.element_size()} bytes, "
                             f"{need} needed")
    return o, ws


def decode(q, k_cache, v_cache, kv_lens=None, scale=None, out=None, workspace=None):
    """Single-query decode.  q [B,H_q,1,d]; k_cache, v_cache [B,H_kv,S_cap,d]
    (bf16, or all float32); kv_lens int32 [B] on the device (None: every row
    is valid).

    Returns o [B,H_q,1,d] with q's dtype.  Runs the split and combine kernels
    on torch's current stream; the workspace (if not given) is cached per
    (device, stream), and must be given under graph capture.
    """
    if q.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _check_tensor(name, t, q.dtype)
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, S, d]")
    B, H_q, S_q, d = q.shape
    Bk, H_kv, S_kv, dk = k_cache.shape
    if tuple(v_cache.shape) != tuple(k_cache.shape) or Bk != B or dk != d:
        raise ValueError("inconsistent q/k/v shapes")
    lens = _lens(kv_lens, B, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = attn_decode_workspace_bytes(B, H_q, H_kv, S_kv, d)
    o, ws = _decode_buffers(q, out, workspace, need,
                            (("k_cache", k_cache), ("v_cache", v_cache)))
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = attn_decode_fwd(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), B, H_q, H_kv, S_q, S_kv,
                         d, 0, float(scale), _ptr(lens), _DTYPES[q.dtype], _ptr(ws),
                         ws.numel() * ws.element_size(), ctypes.c_void_p(stream))
    if st != 0:
        raise AttnError(st, "attn_decode_fwd")
    return o


def decode_paged(q, k_pages, v_pages, block_table, kv_lens=None, scale=None, out=None,
                 workspace=None):
    """Single-query decode over a paged cache.  q [B,H_q,1,d]; k_pages,
    v_pages [num_pages,H_kv,page_size,d] (bf16, or all float32); block_table
    int32 [B,max_blocks] (page of each sequence's page_size-key block);
    kv_lens int32 [B] or None.

    Returns o [B,H_q,1,d] with q's dtype, on torch's current stream; the
    workspace (if not given) is cached per (device, stream), and must be given
    under graph capture.
    """
    if q.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for name, t in (("q", q), ("k_pages", k_pages), ("v_pages", v_pages)):
        _check_tensor(name, t, q.dtype)
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-dimensional")
    _check_tensor("block_table", block_table, torch.int32)
    B, H_q, S_q, d = q.shape
    num_pages, H_kv, page_size, dk = k_pages.shape
    if tuple(v_pages.shape) != tuple(k_pages.shape) or dk != d or S_q != 1:
        raise ValueError("inconsistent q / page shapes")
    if block_table.dim() != 2 or block_table.shape[0] != B or block_table.device != q.device:
        raise ValueError("block_table must be int32 [B, max_blocks] on q's device")
    max_blocks = block_table.shape[1]
    lens = _lens(kv_lens, B, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = attn_decode_workspace_bytes(B, H_q, H_kv, max_blocks * page_size, d)
    o, ws = _decode_buffers(q, out, workspace, need,
                            (("k_pages", k_pages), ("v_pages", v_pages)))
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = attn_decode_paged_fwd(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(o), B, H_q, H_kv, d,
                               float(scale), _ptr(block_table), max_blocks, page_size, num_pages,
                               _ptr(lens), _DTYPES[q.dtype], _ptr(ws), ws.numel() * ws.element_size(),
                               ctypes.c_void_p(stream))
    if st != 0:
        raise AttnError(st, "attn_decode_paged_fwd")
    return o
