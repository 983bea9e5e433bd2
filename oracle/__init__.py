"""CPU oracle for MassAlloc Attention (MALA) and dense attention.

TEST INFRASTRUCTURE ONLY. Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The operator
library never loads it and shares no code with it.

The arithmetic lives in ``mala_oracle.c`` (fp64, libm exp/log, loops in the
order of the paper's Algorithms 1 and 2); this module only marshals numpy
arrays through ctypes. Citations (paper "MassAlloc Attention: Let Attention
Allocate Its Own Compute"; review "Why exact attention does not need a
quadratic matrix"):

* ``dense_fwd`` / ``dense_bwd``: FullAttn, Sec. 2.1; softmax backward written
  with rowsum(P o dP).
* ``mala_fwd``: Algorithm 1 with the online test of Eqs. (1)-(3), Sec. 2.2.
* ``mala_bwd``: Algorithm 2 with the offline test of Eq. (4), Sec. 2.2.
* ``mala_decode``: split-KV decoding, Sec. 2.4 and Appendix A.1.
* ``merge``: the (m, l, u) merge identity of the review's Method section.

Every function here is pinned by the ``-m "not gpu"`` tests against values
the pages print, closed forms, special cases and brute force.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mala_oracle.c")
# MALA_ORACLE_LIB names another build of mala_oracle.c (the mutation test
# loads deliberately broken builds through it); default: the in-tree build
_LIB = os.environ.get("MALA_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

# rounding flags (mirrors the #defines in mala_oracle.c)
ROUND_P_FWD = 1
ROUND_P_BWD = 2
ROUND_DS = 4
ROUND_OUT = 8
ABS = 16  # magnitude mode: sums of |a|*|b| instead of a*b (error-bound scale)
ABS_D = 32  # backward: dS -> P * sum_d |O||dO| in dQ / dK (sensitivity to D)
# forward model: exponentials against a reference maximum that moves only on
# jumps of more than 8 log2 units (where the kernel rounds P), a 128-key tile
# whose upper 64 keys pass alone taken as those 64 keys and then the lower 64;
# exact results are the same for either reference
LAZY_REF = 64
EXACT = 0
BF16_FWD = ROUND_P_FWD | ROUND_OUT
BF16_BWD = ROUND_P_BWD | ROUND_DS | ROUND_OUT
BF16_DECODE = ROUND_OUT  # the decode kernel forms P V in fp32

ILLEGAL, SKIP, RETAIN = -1, 0, 1


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
             "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32),
        ("heads_kv", ctypes.c_int32), ("seqlen_q", ctypes.c_int32),
        ("seqlen_k", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("causal", ctypes.c_int32), ("block_q", ctypes.c_int32),
        ("block_k", ctypes.c_int32), ("tau", ctypes.c_double),
        ("scale", ctypes.c_double), ("round_flags", ctypes.c_int32),
    ]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = ctypes.CDLL(_LIB)
        P = ctypes.POINTER
        dp, i8, i32 = P(ctypes.c_double), P(ctypes.c_int8), P(ctypes.c_int32)
        pr = P(_Problem)
        _lib.orc_dense_fwd.argtypes = [pr, dp, dp, dp, dp, dp]
        _lib.orc_dense_bwd.argtypes = [pr, dp, dp, dp, dp, dp, dp, dp]
        _lib.orc_mala_fwd.argtypes = [pr, dp, dp, dp, i8, dp, dp, i8, dp, i32, ctypes.c_int64]
        _lib.orc_mala_bwd.argtypes = [pr, dp, dp, dp, dp, dp, dp, i8, dp, dp, dp, i8, dp,
                                      i32, ctypes.c_int64, i32, ctypes.c_int64]
        _lib.orc_mala_decode.argtypes = [pr, dp, dp, dp, ctypes.c_int32, i8, dp, dp, i8, dp]
        _lib.orc_merge.argtypes = [ctypes.c_int32, ctypes.c_int32, dp, dp, dp, dp, dp]
        _lib.orc_round_bf16_array.argtypes = [dp, dp, ctypes.c_int64]
        _lib.orc_num_threads.argtypes = []
    return _lib


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a, ctype):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


@dataclass
class Problem:
    batch: int
    heads_q: int
    heads_kv: int
    seqlen_q: int
    seqlen_k: int
    head_dim: int
    causal: bool = True
    block_q: int = 64
    block_k: int = 64
    tau: float = 1.0
    scale: float | None = None
    round_flags: int = EXACT

    def c(self):
        sc = self.scale if self.scale is not None else 1.0 / math.sqrt(self.head_dim)
        return _Problem(self.batch, self.heads_q, self.heads_kv, self.seqlen_q, self.seqlen_k,
                        self.head_dim, int(bool(self.causal)), self.block_q, self.block_k,
                        float(self.tau), float(sc), int(self.round_flags))

    @property
    def tiles(self):
        return (-(-self.seqlen_q // self.block_q), -(-self.seqlen_k // self.block_k))


def _problem_from(q, k, causal, block_q, block_k, tau, scale, round_flags):
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    return Problem(B, Hq, Hkv, Nq, Nk, d, causal, block_q, block_k, tau, scale, round_flags)


def dense_fwd(q, k, v, causal=True, scale=None):
    """Dense softmax attention. q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d] -> (o, lse)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    p = _problem_from(q, k, causal, 64, 64, 0.0, scale, EXACT)
    o = np.zeros_like(q)
    lse = np.zeros(q.shape[:3])
    _load().orc_dense_fwd(ctypes.byref(p.c()), _ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double),
                          _ptr(v, ctypes.c_double), _ptr(o, ctypes.c_double),
                          _ptr(lse, ctypes.c_double))
    return o, lse


def dense_bwd(q, k, v, dout, causal=True, scale=None):
    """Gradients of dense attention w.r.t. q, k, v (unscaled inputs)."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    p = _problem_from(q, k, causal, 64, 64, 0.0, scale, EXACT)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    _load().orc_dense_bwd(ctypes.byref(p.c()), *[_ptr(a, ctypes.c_double)
                                                 for a in (q, k, v, dout, dq, dk, dv)])
    return dq, dk, dv


def _sel(sel):
    if sel is None:
        return None, 0
    a = np.ascontiguousarray(np.asarray(sel, dtype=np.int32).reshape(-1, 3))
    return a, a.shape[0]


def mala_fwd(q, k, v, tau=1.0, causal=True, block_q=64, block_k=64, scale=None,
             round_flags=EXACT, force=None, sel=None, want_margin=True):
    """MALA forward (Algorithm 1). Returns dict(o, lse, dec, margin).

    dec/margin are [B, Hq, Tr, Tc]: decision per tile (-1 illegal, 0 skip,
    1 retain) and the tile margin (largest row margin of Eq. 3 in nats).
    ``force`` (int8, same shape, -1 = free) overrides decisions; ``sel`` lists
    (b, h, i) query blocks to compute (others stay NaN)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    p = _problem_from(q, k, causal, block_q, block_k, tau, scale, round_flags)
    Tr, Tc = p.tiles
    o = np.full_like(q, np.nan)
    lse = np.full(q.shape[:3], np.nan)
    dec = np.full((p.batch, p.heads_q, Tr, Tc), ILLEGAL, dtype=np.int8)
    mrg = np.full((p.batch, p.heads_q, Tr, Tc), np.nan) if want_margin else None
    f = None if force is None else np.ascontiguousarray(force, dtype=np.int8)
    s, ns = _sel(sel)
    _load().orc_mala_fwd(ctypes.byref(p.c()), _ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double),
                         _ptr(v, ctypes.c_double), _ptr(f, ctypes.c_int8),
                         _ptr(o, ctypes.c_double), _ptr(lse, ctypes.c_double),
                         _ptr(dec, ctypes.c_int8), _ptr(mrg, ctypes.c_double),
                         _ptr(s, ctypes.c_int32), ns)
    return {"o": o, "lse": lse, "dec": dec, "margin": mrg}


def mala_bwd(q, k, v, o, lse, dout, tau=1.0, causal=True, block_q=64, block_k=64, scale=None,
             round_flags=EXACT, force=None, sel_q=None, sel_k=None, want_margin=True):
    """MALA backward (Algorithm 2). Returns dict(dq, dk, dv, dec, margin).

    ``o``/``lse`` are the forward's stored output and log-normaliser. ``sel_q``
    lists (b, h, i) blocks whose dQ rows are computed, ``sel_k`` (b, g, j)
    blocks whose dK/dV rows are computed; both None computes everything."""
    q, k, v, o, lse, dout = (_f64(x) for x in (q, k, v, o, lse, dout))
    p = _problem_from(q, k, causal, block_q, block_k, tau, scale, round_flags)
    Tr, Tc = p.tiles
    dq = np.full_like(q, np.nan)
    dk = np.full_like(k, np.nan)
    dv = np.full_like(v, np.nan)
    dec = np.full((p.batch, p.heads_q, Tr, Tc), ILLEGAL, dtype=np.int8)
    mrg = np.full((p.batch, p.heads_q, Tr, Tc), np.nan) if want_margin else None
    f = None if force is None else np.ascontiguousarray(force, dtype=np.int8)
    sq, nq = _sel(sel_q)
    sk, nk = _sel(sel_k)
    _load().orc_mala_bwd(ctypes.byref(p.c()), *[_ptr(a, ctypes.c_double)
                                                for a in (q, k, v, o, lse, dout)],
                         _ptr(f, ctypes.c_int8), _ptr(dq, ctypes.c_double),
                         _ptr(dk, ctypes.c_double), _ptr(dv, ctypes.c_double),
                         _ptr(dec, ctypes.c_int8), _ptr(mrg, ctypes.c_double),
                         _ptr(sq, ctypes.c_int32), nq, _ptr(sk, ctypes.c_int32), nk)
    return {"dq": dq, "dk": dk, "dv": dv, "dec": dec, "margin": mrg}


def mala_decode(q, k, v, num_splits, tau=1.0, block_k=64, scale=None, round_flags=EXACT,
                force=None):
    """Split-KV decode. q [B,Hq,d] (one new token per sequence), k/v
    [B,Hkv,Nk,d]. Returns dict(o [B,Hq,d], lse [B,Hq], dec/margin [B,Hq,Tc])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    p = Problem(B, Hq, Hkv, 1, Nk, d, False, 1, block_k, tau, scale, round_flags)
    Tc = -(-Nk // block_k)
    o = np.full_like(q, np.nan)
    lse = np.full((B, Hq), np.nan)
    dec = np.full((B, Hq, Tc), ILLEGAL, dtype=np.int8)
    mrg = np.full((B, Hq, Tc), np.nan)
    f = None if force is None else np.ascontiguousarray(force, dtype=np.int8)
    _load().orc_mala_decode(ctypes.byref(p.c()), _ptr(q, ctypes.c_double),
                            _ptr(k, ctypes.c_double), _ptr(v, ctypes.c_double),
                            int(num_splits), _ptr(f, ctypes.c_int8), _ptr(o, ctypes.c_double),
                            _ptr(lse, ctypes.c_double), _ptr(dec, ctypes.c_int8),
                            _ptr(mrg, ctypes.c_double))
    return {"o": o, "lse": lse, "dec": dec, "margin": mrg}


def merge(m, l, u):
    """Merge (m_s, l_s, u_s) summaries of one query row -> (o, lse)."""
    m, l, u = _f64(m).ravel(), _f64(l).ravel(), _f64(u)
    S = m.shape[0]
    u = u.reshape(S, -1)
    d = u.shape[1]
    o = np.zeros(d)
    z = np.zeros(1)
    _load().orc_merge(S, d, _ptr(m, ctypes.c_double), _ptr(l, ctypes.c_double),
                      _ptr(np.ascontiguousarray(u), ctypes.c_double), _ptr(o, ctypes.c_double),
                      _ptr(z, ctypes.c_double))
    return o, float(z[0])


def num_threads():
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().orc_num_threads())


def round_bf16(x):
    """fp64 -> fp32 (RNE) -> bf16 (RNE), returned as fp64."""
    x = _f64(x)
    y = np.empty_like(x)
    _load().orc_round_bf16_array(_ptr(x, ctypes.c_double), _ptr(y, ctypes.c_double), x.size)
    return y
