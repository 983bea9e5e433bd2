"""Python binding of the MALA operator library (``libmala.so``).

Argument marshalling only: every step of the operator runs in the HIP
kernels behind the C ABI declared in ``include/mala.h``. The functions carry
the C names and take caller-allocated torch tensors (bf16 / fp32 on a gfx950
device); PyTorch supplies device memory and streams, nothing else. If the
library is not built, every call raises: there is no fallback path.

MassAlloc Attention ("MassAlloc Attention: Let Attention Allocate Its Own
Compute"): causal attention that scores every legal Q.K tile and runs a
tile's post-score work only if some valid row's normalised contribution
reaches tau / L_q (Sec. 2.1-2.2; Algorithms 1 and 2; split-KV decode in
Sec. 2.4 and Appendix A.1).
"""
from __future__ import annotations

import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmala.so")

MALA_OK = 0
MALA_ERR_INVALID_ARG = 1
MALA_ERR_UNSUPPORTED = 2
MALA_ERR_WORKSPACE = 3
MALA_ERR_DEVICE = 4
MALA_ERR_LAUNCH = 5


class MalaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {mala_status_string(status)} (status {status})")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32),
                ("heads_kv", ctypes.c_int32), ("seqlen_q", ctypes.c_int32),
                ("seqlen_k", ctypes.c_int32), ("head_dim", ctypes.c_int32)]


class Config(ctypes.Structure):
    _fields_ = [("causal", ctypes.c_int32), ("block_q", ctypes.c_int32),
                ("block_k", ctypes.c_int32), ("tau", ctypes.c_float),
                ("softmax_scale", ctypes.c_float)]


class _CStats(ctypes.Structure):
    _fields_ = [("counters", ctypes.c_void_p), ("decisions", ctypes.c_void_p)]


class Stats:
    """Optional instrumentation: ``counters`` int64[4] and ``decisions``
    uint8 tensors on the device (either may be None); see mala.h."""

    def __init__(self, counters=None, decisions=None):
        self.counters = counters
        self.decisions = decisions

    def _c(self):
        for t, name in ((self.counters, "stats.counters"), (self.decisions, "stats.decisions")):
            if t is not None:
                if not t.is_cuda or not t.is_contiguous():
                    raise ValueError(f"{name}: a contiguous device tensor is required")
                _on_current_device(t, name)
        return _CStats(self.counters.data_ptr() if self.counters is not None else None,
                       self.decisions.data_ptr() if self.decisions is not None else None)


EXPORTS = ("mala_fwd", "fullattn_fwd", "mala_bwd_workspace_bytes", "mala_bwd", "fullattn_bwd",
           "mala_decode_workspace_bytes", "mala_decode_default_splits", "mala_decode",
           "fullattn_decode", "mala_decode_noalloc", "mala_decode_paged", "fullattn_decode_paged",
           "mala_status_string")

# device-resident scratch of mala_decode_noalloc (bytes per GPU; mala.h)
DECODE_NOALLOC_MAX_BYTES = 16 << 20

_lib = None


def lib():
    """Load ``libmala.so`` (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run __graft_entry__.build() "
                              "(or python -m adaptive_softmax_attention_amd.build)")
        # torch ships its own HIP runtime under the same soname; loading it
        # first makes the library bind to that one instance instead of
        # pulling a second runtime into the process
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        P, vp, sz = ctypes.POINTER, ctypes.c_void_p, ctypes.c_size_t
        ps, pc, pst = P(Shape), P(Config), P(_CStats)
        for f in ("mala_fwd", "fullattn_fwd"):
            getattr(L, f).argtypes = [ps, pc, vp, vp, vp, vp, vp, pst, vp]
            getattr(L, f).restype = ctypes.c_int
        for f in ("mala_bwd", "fullattn_bwd"):
            getattr(L, f).argtypes = [ps, pc, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, pst, vp]
            getattr(L, f).restype = ctypes.c_int
        for f in ("mala_decode", "fullattn_decode"):
            getattr(L, f).argtypes = [ps, pc, vp, vp, vp, vp, vp, ctypes.c_int32, vp, sz, pst, vp]
            getattr(L, f).restype = ctypes.c_int
        L.mala_decode_noalloc.argtypes = [ps, pc, vp, vp, vp, vp, vp, ctypes.c_int32, pst, vp]
        L.mala_decode_noalloc.restype = ctypes.c_int
        for f in ("mala_decode_paged", "fullattn_decode_paged"):
            getattr(L, f).argtypes = [ps, pc, vp, vp, vp, vp, vp, ctypes.c_int32, vp, vp,
                                      ctypes.c_int32, vp, sz, pst, vp]
            getattr(L, f).restype = ctypes.c_int
        L.mala_bwd_workspace_bytes.argtypes = [ps, pc]
        L.mala_bwd_workspace_bytes.restype = sz
        L.mala_decode_workspace_bytes.argtypes = [ps, ctypes.c_int32]
        L.mala_decode_workspace_bytes.restype = sz
        L.mala_decode_default_splits.argtypes = [ps]
        L.mala_decode_default_splits.restype = ctypes.c_int32
        L.mala_status_string.argtypes = [ctypes.c_int]
        L.mala_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def mala_status_string(status: int) -> str:
    return lib().mala_status_string(int(status)).decode()


# ------------------------------------------------------------ marshalling --

def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _on_current_device(t, name):
    """The library launches on the current device: a tensor elsewhere would
    hand it a pointer that device cannot use."""
    import torch
    cur = torch.cuda.current_device()
    if t.device.index is not None and t.device.index != cur:
        raise ValueError(f"{name}: on {t.device}, but the current device is cuda:{cur}")


def _check(t, name, dtype, shape):
    import torch
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be on the GPU")
    _on_current_device(t, name)
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    return torch


def make_shape(q, k, decode=False):
    if decode:
        B, Hq, d = q.shape
        return Shape(B, Hq, k.shape[1], 1, k.shape[2], d)
    B, Hq, Nq, d = q.shape
    return Shape(B, Hq, k.shape[1], Nq, k.shape[2], d)


def make_config(causal=True, tau=1.0, block_q=64, block_k=64, softmax_scale=None, head_dim=128):
    sc = softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(head_dim)
    return Config(int(causal), block_q, block_k, float(tau), float(sc))


def _fwd(name, q, k, v, o, lse, causal, tau, block_q, block_k, softmax_scale, stats, stream):
    import torch
    B, Hq, Nq, d = q.shape
    _check(q, "q", torch.bfloat16, q.shape)
    _check(k, "k", torch.bfloat16, (B, k.shape[1], k.shape[2], d))
    _check(v, "v", torch.bfloat16, k.shape)
    _check(o, "o", torch.bfloat16, q.shape)
    _check(lse, "lse", torch.float32, (B, Hq, Nq))
    shp = make_shape(q, k)
    cfg = make_config(causal, tau, block_q, block_k, softmax_scale, d)
    st = stats._c() if stats is not None else None
    rc = getattr(lib(), name)(ctypes.byref(shp), ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v),
                              _ptr(o), _ptr(lse), ctypes.byref(st) if st is not None else None,
                              _stream(stream))
    if rc != MALA_OK:
        raise MalaError(rc, name)


def mala_fwd(q, k, v, o, lse, *, causal=True, tau=1.0, block_q=64, block_k=64,
             softmax_scale=None, stats=None, stream=None):
    """MALA forward into caller-allocated o [B,Hq,Nq,d] bf16, lse [B,Hq,Nq] fp32."""
    _fwd("mala_fwd", q, k, v, o, lse, causal, tau, block_q, block_k, softmax_scale, stats, stream)


def fullattn_fwd(q, k, v, o, lse, *, causal=True, block_q=64, block_k=64, softmax_scale=None,
                 stats=None, stream=None):
    """Dense FullAttn forward from the same kernel (test compiled out)."""
    _fwd("fullattn_fwd", q, k, v, o, lse, causal, 0.0, block_q, block_k, softmax_scale, stats,
         stream)


def mala_bwd_workspace_bytes(q, k, *, causal=True, block_q=64, block_k=64, softmax_scale=None):
    shp = make_shape(q, k)
    cfg = make_config(causal, 0.0, block_q, block_k, softmax_scale, q.shape[-1])
    return int(lib().mala_bwd_workspace_bytes(ctypes.byref(shp), ctypes.byref(cfg)))


def _bwd(name, q, k, v, o, lse, dout, dq, dk, dv, workspace, causal, tau, block_q, block_k,
         softmax_scale, stats, stream):
    import torch
    B, Hq, Nq, d = q.shape
    for t, n, shp in ((q, "q", q.shape), (o, "o", q.shape), (dout, "dout", q.shape),
                      (dq, "dq", q.shape), (k, "k", k.shape), (v, "v", k.shape),
                      (dk, "dk", k.shape), (dv, "dv", k.shape)):
        _check(t, n, torch.bfloat16, shp)
    _check(lse, "lse", torch.float32, (B, Hq, Nq))
    if workspace is None or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace: a contiguous device tensor is required")
    _on_current_device(workspace, "workspace")
    shp = make_shape(q, k)
    cfg = make_config(causal, tau, block_q, block_k, softmax_scale, d)
    st = stats._c() if stats is not None else None
    nbytes = workspace.numel() * workspace.element_size()
    rc = getattr(lib(), name)(ctypes.byref(shp), ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v),
                              _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                              _ptr(workspace), nbytes,
                              ctypes.byref(st) if st is not None else None, _stream(stream))
    if rc != MALA_OK:
        raise MalaError(rc, name)


def mala_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, *, causal=True, tau=1.0, block_q=64,
             block_k=64, softmax_scale=None, stats=None, stream=None):
    """MALA backward into caller-allocated dq/dk/dv (bf16); ``workspace`` is a
    device tensor of at least mala_bwd_workspace_bytes() bytes."""
    _bwd("mala_bwd", q, k, v, o, lse, dout, dq, dk, dv, workspace, causal, tau, block_q, block_k,
         softmax_scale, stats, stream)


def fullattn_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, *, causal=True, block_q=64,
                 block_k=64, softmax_scale=None, stats=None, stream=None):
    """Dense FullAttn backward from the same kernel (test compiled out)."""
    _bwd("fullattn_bwd", q, k, v, o, lse, dout, dq, dk, dv, workspace, causal, 0.0, block_q,
         block_k, softmax_scale, stats, stream)


def mala_decode_workspace_bytes(q, k_cache, num_splits):
    shp = make_shape(q, k_cache, decode=True)
    return int(lib().mala_decode_workspace_bytes(ctypes.byref(shp), int(num_splits)))


def mala_decode_default_splits(q, k_cache):
    shp = make_shape(q, k_cache, decode=True)
    return int(lib().mala_decode_default_splits(ctypes.byref(shp)))


def _decode(name, q, k_cache, v_cache, o, lse, num_splits, workspace, tau, block_k,
            softmax_scale, stats, stream):
    import torch
    B, Hq, d = q.shape
    _check(q, "q", torch.bfloat16, q.shape)
    _check(k_cache, "k_cache", torch.bfloat16, (B, k_cache.shape[1], k_cache.shape[2], d))
    _check(v_cache, "v_cache", torch.bfloat16, k_cache.shape)
    _check(o, "o", torch.bfloat16, q.shape)
    _check(lse, "lse", torch.float32, (B, Hq))
    if workspace is None or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace: a contiguous device tensor is required")
    _on_current_device(workspace, "workspace")
    shp = make_shape(q, k_cache, decode=True)
    cfg = make_config(False, tau, 64, block_k, softmax_scale, d)
    st = stats._c() if stats is not None else None
    nbytes = workspace.numel() * workspace.element_size()
    rc = getattr(lib(), name)(ctypes.byref(shp), ctypes.byref(cfg), _ptr(q), _ptr(k_cache),
                              _ptr(v_cache), _ptr(o), _ptr(lse), int(num_splits), _ptr(workspace),
                              nbytes, ctypes.byref(st) if st is not None else None,
                              _stream(stream))
    if rc != MALA_OK:
        raise MalaError(rc, name)


def mala_decode(q, k_cache, v_cache, o, lse, num_splits, workspace, *, tau=1.0, block_k=64,
                softmax_scale=None, stats=None, stream=None):
    """Split-KV MALA decode: q/o [B,Hq,d] bf16, lse [B,Hq] fp32, caches
    [B,Hkv,Nk,d] bf16 (current token included)."""
    _decode("mala_decode", q, k_cache, v_cache, o, lse, num_splits, workspace, tau, block_k,
            softmax_scale, stats, stream)


def fullattn_decode(q, k_cache, v_cache, o, lse, num_splits, workspace, *, block_k=64,
                    softmax_scale=None, stats=None, stream=None):
    """Dense split-KV decode from the same kernels (test compiled out)."""
    _decode("fullattn_decode", q, k_cache, v_cache, o, lse, num_splits, workspace, 0.0, block_k,
            softmax_scale, stats, stream)


def mala_decode_noalloc(q, k_cache, v_cache, o, lse, num_splits, *, tau=1.0, block_k=64,
                        softmax_scale=None, stats=None, stream=None):
    """mala_decode without a workspace: the split partials go to the
    library's device-resident array (at most DECODE_NOALLOC_MAX_BYTES per
    GPU). For callers that cannot allocate; overlapping calls on one GPU
    race."""
    import torch
    B, Hq, d = q.shape
    _check(q, "q", torch.bfloat16, q.shape)
    _check(k_cache, "k_cache", torch.bfloat16, (B, k_cache.shape[1], k_cache.shape[2], d))
    _check(v_cache, "v_cache", torch.bfloat16, k_cache.shape)
    _check(o, "o", torch.bfloat16, q.shape)
    _check(lse, "lse", torch.float32, (B, Hq))
    shp = make_shape(q, k_cache, decode=True)
    cfg = make_config(False, tau, 64, block_k, softmax_scale, d)
    st = stats._c() if stats is not None else None
    rc = lib().mala_decode_noalloc(ctypes.byref(shp), ctypes.byref(cfg), _ptr(q), _ptr(k_cache),
                                   _ptr(v_cache), _ptr(o), _ptr(lse), int(num_splits),
                                   ctypes.byref(st) if st is not None else None, _stream(stream))
    if rc != MALA_OK:
        raise MalaError(rc, "mala_decode_noalloc")


def _decode_paged(name, q, k_pages, v_pages, block_table, cache_lens, max_len, o, lse,
                  num_splits, workspace, tau, block_k, softmax_scale, stats, stream):
    import torch
    B, Hq, d = q.shape
    P, Hkv = k_pages.shape[0], k_pages.shape[1]
    _check(q, "q", torch.bfloat16, q.shape)
    _check(k_pages, "k_pages", torch.bfloat16, (P, Hkv, 64, d))
    _check(v_pages, "v_pages", torch.bfloat16, k_pages.shape)
    _check(block_table, "block_table", torch.int32, (B, -(-int(max_len) // 64)))
    _check(cache_lens, "cache_lens", torch.int32, (B,))
    _check(o, "o", torch.bfloat16, q.shape)
    _check(lse, "lse", torch.float32, (B, Hq))
    if workspace is None or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace: a contiguous device tensor is required")
    _on_current_device(workspace, "workspace")
    shp = Shape(B, Hq, Hkv, 1, int(max_len), d)
    cfg = make_config(False, tau, 64, block_k, softmax_scale, d)
    st = stats._c() if stats is not None else None
    nbytes = workspace.numel() * workspace.element_size()
    rc = getattr(lib(), name)(ctypes.byref(shp), ctypes.byref(cfg), _ptr(q), _ptr(k_pages),
                              _ptr(v_pages), _ptr(block_table), _ptr(cache_lens), int(P), _ptr(o),
                              _ptr(lse), int(num_splits), _ptr(workspace), nbytes,
                              ctypes.byref(st) if st is not None else None, _stream(stream))
    if rc != MALA_OK:
        raise MalaError(rc, name)


def mala_decode_paged_workspace_bytes(q, max_len, heads_kv, num_splits):
    B, Hq, d = q.shape
    shp = Shape(B, Hq, int(heads_kv), 1, int(max_len), d)
    return int(lib().mala_decode_workspace_bytes(ctypes.byref(shp), int(num_splits)))


def mala_decode_paged(q, k_pages, v_pages, block_table, cache_lens, max_len, o, lse, num_splits,
                      workspace, *, tau=1.0, block_k=64, softmax_scale=None, stats=None,
                      stream=None):
    """Split-KV MALA decode over a paged cache of variable-length sequences:
    q/o [B,Hq,d] bf16, lse [B,Hq] fp32, pages [P,Hkv,64,d] bf16, block_table
    [B, ceil(max_len/64)] int32, cache_lens [B] int32 (1..max_len), all on the
    device. block_k (64 or 128) is the decision tile; pages stay 64 keys."""
    _decode_paged("mala_decode_paged", q, k_pages, v_pages, block_table, cache_lens, max_len, o,
                  lse, num_splits, workspace, tau, block_k, softmax_scale, stats, stream)


def fullattn_decode_paged(q, k_pages, v_pages, block_table, cache_lens, max_len, o, lse,
                          num_splits, workspace, *, block_k=64, softmax_scale=None, stats=None,
                          stream=None):
    """Dense split-KV decode over the same paged cache."""
    _decode_paged("fullattn_decode_paged", q, k_pages, v_pages, block_table, cache_lens, max_len,
                  o, lse, num_splits, workspace, 0.0, block_k, softmax_scale, stats, stream)
