"""CPU tests of the C ABI: the library loads, exports every function that
include/mala.h declares, and every validation error path returns its status
before any device call. No compute call is made: each call below carries at
least one invalid argument, except the no-device check, which only runs
where no GPU is visible."""
import ctypes
import math
import os
import re

import pytest

import adaptive_softmax_attention_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mala.h")
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:mala|fullattn)_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = m.lib()
    names = declared_functions()
    assert len(names) == 13
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(m.EXPORTS)


def test_status_strings():
    for code in range(6):
        s = m.mala_status_string(code)
        assert isinstance(s, str) and s
    assert m.mala_status_string(99) == "unknown status"


def shape(B=1, Hq=4, Hkv=2, Nq=128, Nk=128, d=128):
    return m.Shape(B, Hq, Hkv, Nq, Nk, d)


def cfg(causal=1, bq=64, bk=64, tau=1.0, scale=None):
    return m.Config(causal, bq, bk, tau, 0.088 if scale is None else scale)


def fwd(s, c, q=FAKE, fn="mala_fwd"):
    return getattr(m.lib(), fn)(ctypes.byref(s) if s is not None else None,
                                ctypes.byref(c) if c is not None else None,
                                q, FAKE, FAKE, FAKE, FAKE, None, None)


@pytest.mark.parametrize("s,c,expect", [
    (None, cfg(), m.MALA_ERR_INVALID_ARG),
    (shape(), None, m.MALA_ERR_INVALID_ARG),
    (shape(B=0), cfg(), m.MALA_ERR_INVALID_ARG),
    (shape(Hq=3, Hkv=2), cfg(), m.MALA_ERR_INVALID_ARG),
    (shape(Nq=0, Nk=0), cfg(), m.MALA_ERR_INVALID_ARG),
    (shape(d=96), cfg(), m.MALA_ERR_UNSUPPORTED),
    (shape(d=0), cfg(), m.MALA_ERR_INVALID_ARG),
    (shape(), cfg(bq=96, bk=64), m.MALA_ERR_UNSUPPORTED),
    (shape(), cfg(bq=64, bk=256), m.MALA_ERR_UNSUPPORTED),
    (shape(), cfg(bq=32, bk=32), m.MALA_ERR_UNSUPPORTED),
    (shape(), cfg(bq=0), m.MALA_ERR_INVALID_ARG),
    (shape(), cfg(tau=float("nan")), m.MALA_ERR_INVALID_ARG),
    (shape(), cfg(tau=-1.0), m.MALA_ERR_INVALID_ARG),
    (shape(), cfg(scale=0.0), m.MALA_ERR_INVALID_ARG),
    (shape(), cfg(scale=float("inf")), m.MALA_ERR_INVALID_ARG),
    (shape(), cfg(scale=float("nan")), m.MALA_ERR_INVALID_ARG),
    (shape(), cfg(causal=2), m.MALA_ERR_INVALID_ARG),
    (shape(Nq=128, Nk=100), cfg(causal=1), m.MALA_ERR_UNSUPPORTED),
    (shape(Nq=1 << 25, Nk=1 << 25), cfg(), m.MALA_ERR_UNSUPPORTED),
])
def test_forward_validation(s, c, expect):
    assert fwd(s, c) == expect


def test_forward_null_pointer():
    assert fwd(shape(), cfg(), q=None) == m.MALA_ERR_INVALID_ARG


def test_fullattn_ignores_tau_but_checks_the_rest():
    # tau NaN is not an error for the dense path; a bad scale still is
    assert fwd(shape(), cfg(scale=-1.0), fn="fullattn_fwd") == m.MALA_ERR_INVALID_ARG
    rc = fwd(shape(B=0), cfg(tau=float("nan")), fn="fullattn_fwd")
    assert rc == m.MALA_ERR_INVALID_ARG


def _no_gpu():
    try:
        import torch
        return torch.cuda.device_count() == 0
    except Exception:
        return True


@pytest.mark.skipif(not _no_gpu(), reason="only meaningful where no GPU is visible")
def test_valid_call_without_device_reports_device_error():
    assert fwd(shape(), cfg()) == m.MALA_ERR_DEVICE
    # causal with fewer queries than keys (prefill against a cache) is accepted
    assert fwd(shape(Nq=100, Nk=128), cfg()) == m.MALA_ERR_DEVICE
    # decision tiles of 64 or 128 rows and keys
    for bq in (64, 128):
        for bk in (64, 128):
            assert fwd(shape(), cfg(bq=bq, bk=bk)) == m.MALA_ERR_DEVICE
    assert fwd(shape(), cfg(tau=float("nan")), fn="fullattn_fwd") == m.MALA_ERR_DEVICE


def test_workspace_sizes():
    L = m.lib()
    s, c = shape(B=2, Hq=4, Nq=100, Nk=100, d=64), cfg()
    a256 = lambda x: (x + 255) // 256 * 256
    # backward: a 256-byte status header, 1 KiB of row terms per 64-row
    # query block, one decision byte per legal tile (lower triangle when
    # causal and Nq = Nk, Tr x Tc when not causal), fp32 partial dK/dV for
    # 4 npair slots per (batch, KV head), npair = Tc/2 + 1, each a pair of
    # key blocks,
    # and int32 tables per (batch, KV head): kept-item count and segment
    # entry per key block, npair key-block pairs, 8 work items per pair and a
    # work count
    bh, tr = 2 * 4, 2
    npair = 2 // 2 + 1
    part = 2 * 2 * 4 * npair * 2 * 2 * 64 * 64 * 4  # B * Hkv * 4 npair * 2 blocks * (dK, dV) * 64 * d * 4
    tabs = 2 * 2 * (2 * 2 + 2 * npair + 8 * npair + 1) * 4
    want = 256 + a256(bh * tr * 1024) + a256(bh * tr * (tr + 1) // 2) + part + tabs
    assert L.mala_bwd_workspace_bytes(ctypes.byref(s), ctypes.byref(c)) == want
    s2 = shape(B=1, Hq=2, Hkv=1, Nq=130, Nk=700, d=128)
    npair = 11 // 2 + 1
    tabs = 1 * 1 * (2 * 11 + 2 * npair + 8 * npair + 1) * 4
    part = 1 * 1 * 4 * npair * 2 * 2 * 64 * 128 * 4
    want = 256 + a256(2 * 3 * 1024) + a256(2 * 3 * 11) + part + tabs
    assert L.mala_bwd_workspace_bytes(ctypes.byref(s2), ctypes.byref(cfg(causal=0))) == want
    # causal with the 130 queries at the end of 700 keys: query blocks 0, 1, 2
    # reach key blocks 0..9, 0..10, 0..10 (32 decision bytes per head)
    want = 256 + a256(2 * 3 * 1024) + a256(2 * 32) + part + tabs
    assert L.mala_bwd_workspace_bytes(ctypes.byref(s2), ctypes.byref(cfg(causal=1))) == want
    # the 128K operator at one GPU's head share (8 query / 1 KV head, d 128):
    # the partial sums take 4100 slots x 128 KiB, about 537 MB (half the 8
    # segments per key block of a plain per-block layout)
    s4 = shape(B=1, Hq=8, Hkv=1, Nq=131072, Nk=131072, d=128)
    ws4 = L.mala_bwd_workspace_bytes(ctypes.byref(s4), ctypes.byref(cfg()))
    assert 560e6 < ws4 < 580e6, ws4
    assert L.mala_bwd_workspace_bytes(ctypes.byref(shape(d=96)), ctypes.byref(c)) == 0
    sd = shape(B=3, Hq=8, Hkv=2, Nq=1, Nk=1000, d=128)
    n = 3 * 8 * 5
    assert L.mala_decode_workspace_bytes(ctypes.byref(sd), 5) == 2 * a256(n * 4) + a256(n * 128 * 4)
    assert L.mala_decode_workspace_bytes(ctypes.byref(sd), 0) == 0
    assert 1 <= L.mala_decode_default_splits(ctypes.byref(sd)) <= 16


def bwd(s, c, ws=FAKE, nbytes=1 << 40, dq=FAKE):
    return m.lib().mala_bwd(ctypes.byref(s), ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                            dq, FAKE, FAKE, ws, nbytes, None, None)


def test_backward_validation():
    assert bwd(shape(), cfg(), ws=None) == m.MALA_ERR_WORKSPACE
    assert bwd(shape(), cfg(), nbytes=16) == m.MALA_ERR_WORKSPACE
    assert bwd(shape(), cfg(), dq=None) == m.MALA_ERR_INVALID_ARG
    assert bwd(shape(Nq=128, Nk=64), cfg()) == m.MALA_ERR_UNSUPPORTED
    assert bwd(shape(), cfg(tau=-2.0)) == m.MALA_ERR_INVALID_ARG


def dec(s, c, S=4, ws=FAKE, nbytes=1 << 40):
    return m.lib().mala_decode(ctypes.byref(s), ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, S,
                               ws, nbytes, None, None)


def test_decode_validation():
    s = shape(Nq=1, Nk=4096)
    assert dec(shape(Nq=2, Nk=4096), cfg()) == m.MALA_ERR_INVALID_ARG
    assert dec(s, cfg(), S=0) == m.MALA_ERR_INVALID_ARG
    assert dec(s, cfg(), S=65) == m.MALA_ERR_INVALID_ARG  # more splits than tiles
    # 128-key decision tiles: 32 of them in 4096 keys
    assert dec(s, cfg(bk=128), S=33) == m.MALA_ERR_INVALID_ARG
    assert dec(s, cfg(), ws=None) == m.MALA_ERR_WORKSPACE
    assert dec(s, cfg(), nbytes=100) == m.MALA_ERR_WORKSPACE
    assert dec(s, cfg(tau=float("nan"))) == m.MALA_ERR_INVALID_ARG
    assert dec(shape(Hq=16, Hkv=1, Nq=1, Nk=4096), cfg()) == m.MALA_ERR_UNSUPPORTED


def test_binding_rejects_bad_tensors():
    import torch
    q = torch.zeros(1, 2, 64, 64, dtype=torch.float32)
    with pytest.raises(ValueError):
        m.mala_fwd(q, q, q, q, q[..., 0])


def test_decode_paged_validation():
    L = m.lib()
    s = shape(Nq=1, Nk=4096)

    def call(table=FAKE, lens=FAKE, pages=8, S=4, fn="mala_decode_paged"):
        return getattr(L, fn)(ctypes.byref(s), ctypes.byref(cfg(causal=0)), FAKE, FAKE, FAKE,
                              table, lens, pages, FAKE, FAKE, S, FAKE, 1 << 40, None, None)
    assert call(table=None) == m.MALA_ERR_INVALID_ARG
    assert call(lens=None) == m.MALA_ERR_INVALID_ARG
    assert call(pages=0) == m.MALA_ERR_INVALID_ARG
    assert call(S=0) == m.MALA_ERR_INVALID_ARG
    assert call(table=None, fn="fullattn_decode_paged") == m.MALA_ERR_INVALID_ARG
    if _no_gpu():
        assert call() == m.MALA_ERR_DEVICE


MIS = ctypes.c_void_p(0x1002)  # 2-byte aligned: below what every tensor needs


def test_misaligned_pointers_are_rejected():
    L = m.lib()
    s, c = shape(), cfg()
    # forward: any bf16 tensor off a 16-byte boundary, or lse off 4 bytes
    for pos in range(4):
        args = [FAKE] * 4
        args[pos] = MIS
        assert L.mala_fwd(ctypes.byref(s), ctypes.byref(c), *args, FAKE, None, None) == \
            m.MALA_ERR_INVALID_ARG, pos
    assert L.mala_fwd(ctypes.byref(s), ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, MIS, None,
                      None) == m.MALA_ERR_INVALID_ARG
    assert L.fullattn_fwd(ctypes.byref(s), ctypes.byref(c), MIS, FAKE, FAKE, FAKE, FAKE, None,
                          None) == m.MALA_ERR_INVALID_ARG
    # counters must be 8-byte aligned
    st = m._CStats(0x1004, None)
    assert L.mala_fwd(ctypes.byref(s), ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE,
                      ctypes.byref(st), None) == m.MALA_ERR_INVALID_ARG
    # backward: each of the nine tensors, then the workspace
    for pos in range(9):
        args = [FAKE] * 9
        args[pos] = MIS
        assert L.mala_bwd(ctypes.byref(s), ctypes.byref(c), *args, FAKE, 1 << 40, None,
                          None) == m.MALA_ERR_INVALID_ARG, pos
    assert L.mala_bwd(ctypes.byref(s), ctypes.byref(c), *([FAKE] * 9), ctypes.c_void_p(0x1008),
                      1 << 40, None, None) == m.MALA_ERR_INVALID_ARG
    # decode: q, caches, o, lse, workspace
    sd = shape(Nq=1, Nk=4096)
    for pos in range(5):
        args = [FAKE] * 5
        args[pos] = MIS
        assert L.mala_decode(ctypes.byref(sd), ctypes.byref(c), *args, 4, FAKE, 1 << 40, None,
                             None) == m.MALA_ERR_INVALID_ARG, pos
    assert L.mala_decode(ctypes.byref(sd), ctypes.byref(c), *([FAKE] * 5), 4,
                         ctypes.c_void_p(0x1008), 1 << 40, None, None) == m.MALA_ERR_INVALID_ARG
    # paged: block table and lengths are int32 words
    for table, lens in ((MIS, FAKE), (FAKE, MIS)):
        assert L.mala_decode_paged(ctypes.byref(sd), ctypes.byref(cfg(causal=0)), FAKE, FAKE, FAKE,
                                   table, lens, 8, FAKE, FAKE, 4, FAKE, 1 << 40, None,
                                   None) == m.MALA_ERR_INVALID_ARG


def test_stats_tensors_must_be_device_tensors():
    import torch
    with pytest.raises(ValueError):
        m.Stats(torch.zeros(4, dtype=torch.int64))._c()
    with pytest.raises(ValueError):
        m.Stats(None, torch.zeros(8, dtype=torch.uint8))._c()
    assert m.Stats()._c().counters is None
