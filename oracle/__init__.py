"""CPU oracle for the attention forward pass -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product library neither imports nor links it, and
the two share no code.

`attention()` and `attention_rows()` call the fp64 three-pass definition in
oracle.c (or, given lib=oracle.rowblock, the same definition evaluated one
block of query rows at a time with fp64 library matrix products, fast enough
for whole outputs of the large workloads) (standard attention as set out in "GPU learning day 24: Operator
Fusion", section 3.4, with the two-pass softmax of "Optimizing Decoder
Attention for LLMs on GPU", traditional-approach step 3).  `decode()` is the
same definition with one query row per head, as in the decoding setting of
the latter page.

Inputs may be numpy arrays (float64, float32, or uint16 holding bf16 bit
patterns) or CPU torch tensors (float64, float32, bfloat16); they are passed
to C in their stored format and upcast there exactly.  Outputs are float64
numpy arrays.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F64, F32, BF16 = 0, 1, 2


def load(path=None):
    """Load (building first if missing) the oracle library at `path`."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        from . import build as _build
        _build.build(p, quiet=True)
    lib = ctypes.CDLL(p)
    vp, i32, f64, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_int64
    lib.oracle_attention.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                     i32, f64, vp, vp, vp, vp]
    lib.oracle_attention.restype = i32
    lib.oracle_attention_rows.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                          i32, f64, vp, vp, i64, vp, vp]
    lib.oracle_attention_rows.restype = i32
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = i32
    if path is None:
        _lib = lib
    return lib


def _as_stored(x):
    """Return (contiguous numpy array in stored format, dtype code)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy().view(np.uint16), BF16
            if x.dtype == torch.float32:
                return x.numpy(), F32
            if x.dtype == torch.float64:
                return x.numpy(), F64
            raise TypeError(f"unsupported tensor dtype {x.dtype}")
    except ImportError:
        pass
    x = np.ascontiguousarray(x)
    if x.dtype == np.float64:
        return x, F64
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.uint16:
        return x, BF16
    raise TypeError(f"unsupported array dtype {x.dtype}")


def _lens(kv_lens, B):
    if kv_lens is None:
        return None
    try:
        import torch
        if isinstance(kv_lens, torch.Tensor):
            kv_lens = kv_lens.detach().cpu().numpy()
    except ImportError:
        pass
    a = np.ascontiguousarray(np.asarray(kv_lens, dtype=np.int32))
    if a.shape != (B,):
        raise ValueError("kv_lens must have shape [B]")
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, S, d]")
    B, Hq, Sq, d = q.shape
    Bk, Hkv, Skv, dk = k.shape
    if k.shape != v.shape or Bk != B or dk != d:
        raise ValueError("inconsistent q/k/v shapes")
    return B, Hq, Hkv, Sq, Skv, d


def _rowblock(lib):
    return getattr(lib, "IS_ROWBLOCK", False)


def attention(q, k, v, causal, scale, kv_lens=None, want_lse=False, want_p=False, lib=None):
    """Full fp64 attention.  Returns o [B,H_q,S_q,d] (and lse, p if asked)."""
    if _rowblock(lib):
        return lib.attention(q, k, v, causal, scale, kv_lens=kv_lens, want_lse=want_lse,
                             want_p=want_p)
    qa, dt = _as_stored(q)
    ka, dtk = _as_stored(k)
    va, dtv = _as_stored(v)
    if not (dt == dtk == dtv):
        raise TypeError("q, k, v must share one dtype")
    B, Hq, Hkv, Sq, Skv, d = _shapes(qa, ka, va)
    lens = _lens(kv_lens, B)
    o = np.empty((B, Hq, Sq, d), np.float64)
    lse = np.empty((B, Hq, Sq), np.float64) if want_lse else None
    p = np.empty((B, Hq, Sq, Skv), np.float64) if want_p else None
    rc = (lib or load()).oracle_attention(_ptr(qa), _ptr(ka), _ptr(va), dt, B, Hq, Hkv, Sq, Skv, d,
                                          int(bool(causal)), float(scale), _ptr(lens),
                                          _ptr(o), _ptr(lse), _ptr(p))
    if rc != 0:
        raise ValueError(f"oracle_attention rejected its arguments (code {rc})")
    out = [o]
    if want_lse:
        out.append(lse)
    if want_p:
        out.append(p)
    return out[0] if len(out) == 1 else tuple(out)


def attention_rows(q, k, v, causal, scale, rows, kv_lens=None, want_lse=False, lib=None):
    """fp64 attention for selected (b, h_q, i) rows.  Returns o [n, d] (and lse [n])."""
    if _rowblock(lib):
        return lib.attention_rows(q, k, v, causal, scale, rows, kv_lens=kv_lens, want_lse=want_lse)
    qa, dt = _as_stored(q)
    ka, dtk = _as_stored(k)
    va, dtv = _as_stored(v)
    if not (dt == dtk == dtv):
        raise TypeError("q, k, v must share one dtype")
    B, Hq, Hkv, Sq, Skv, d = _shapes(qa, ka, va)
    lens = _lens(kv_lens, B)
    sel = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
    n = sel.shape[0]
    o = np.empty((n, d), np.float64)
    lse = np.empty((n,), np.float64)
    rc = (lib or load()).oracle_attention_rows(_ptr(qa), _ptr(ka), _ptr(va), dt, B, Hq, Hkv, Sq,
                                               Skv, d, int(bool(causal)), float(scale),
                                               _ptr(lens), _ptr(sel), n, _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError(f"oracle_attention_rows rejected its arguments (code {rc})")
    return (o, lse) if want_lse else o


def decode(q, k_cache, v_cache, kv_lens, scale, want_lse=False, lib=None):
    """Single-query decode: q [B,H_q,1,d] over the first kv_lens[b] cache rows."""
    if q.shape[2] != 1:
        raise ValueError("decode takes one query row per head")
    return attention(q, k_cache, v_cache, False, scale, kv_lens=kv_lens, want_lse=want_lse,
                     lib=lib)


def num_threads(lib=None):
    """OpenMP threads the oracle uses (follows OMP_NUM_THREADS)."""
    return int((lib or load()).oracle_num_threads())
