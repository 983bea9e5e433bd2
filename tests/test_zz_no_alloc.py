"""mala_decode_noalloc (the allocation-free decode) against mala_decode,
through the C ABI: the same kernels on the same inputs, so the outputs must
agree bitwise, on two calls in a row (the second smaller) and on a call
after a larger one left its partials in the shared device array."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as W
from parity import bits_to_gpu

pytestmark = pytest.mark.gpu


def mala():
    import adaptive_softmax_attention_amd as m
    m.lib()
    return m


def _case(seed, B, Hq, Hkv, Nk, d, planted):
    inp = W.peaked(W.Spec(seed, B, Hq, Hkv, Nk, d, 3.0, planted), q_rows=[Nk - 1],
                   want_do=False)
    q = bits_to_gpu(np.ascontiguousarray(inp["q"][:, :, 0, :]))
    return q, bits_to_gpu(inp["k"]), bits_to_gpu(inp["v"])


def _both(m, q, k, v, S, tau, bk=64, dense=False):
    o1, o2 = torch.empty_like(q), torch.empty_like(q)
    l1 = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    l2 = torch.empty_like(l1)
    ws = torch.empty(m.mala_decode_workspace_bytes(q, k, S), dtype=torch.uint8, device="cuda")
    assert ws.numel() <= m.DECODE_NOALLOC_MAX_BYTES
    m.mala_decode(q, k, v, o1, l1, S, ws, tau=tau, block_k=bk)
    m.mala_decode_noalloc(q, k, v, o2, l2, S, tau=tau, block_k=bk)
    torch.cuda.synchronize()
    return o1, l1, o2, l2


def test_noalloc_decode_matches_workspace_decode_twice():
    m = mala()
    print("[noalloc] call 1: 16 x 32/8 heads, 16K cache, 16 splits", flush=True)
    big = _case(5101, 16, 32, 8, 16384, 128, 64)
    o1, l1, o2, l2 = _both(m, *big, 16, 1.0)
    assert torch.isfinite(o1.float()).all()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    print("[noalloc] call 2: 3 x 8/2 heads, 1000-token cache, d 64, 5 splits", flush=True)
    small = _case(5102, 3, 8, 2, 1000, 64, 8)
    o1, l1, o2, l2 = _both(m, *small, 5, 4.0)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # 128-key decision tiles and tau = 0 after that
    o1, l1, o2, l2 = _both(m, *small, 3, 0.0, bk=128)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_noalloc_decode_allocates_nothing_and_rejects_oversize():
    m = mala()
    q, k, v = _case(5103, 4, 16, 4, 4096, 128, 16)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    m.mala_decode_noalloc(q, k, v, o, lse, 8, tau=1.0)  # first call on the device: set-up
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for _ in range(20):
        m.mala_decode_noalloc(q, k, v, o, lse, 8, tau=1.0)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0
    # 64 sequences x 64 heads x 16 splits need about 34 MB of partials
    qb = torch.zeros((64, 64, 128), dtype=torch.bfloat16, device="cuda")
    kb = torch.zeros((64, 8, 1024, 128), dtype=torch.bfloat16, device="cuda")
    ob = torch.empty_like(qb)
    lb = torch.empty((64, 64), dtype=torch.float32, device="cuda")
    assert m.mala_decode_workspace_bytes(qb, kb, 16) > m.DECODE_NOALLOC_MAX_BYTES
    with pytest.raises(m.MalaError) as e:
        m.mala_decode_noalloc(qb, kb, kb, ob, lb, 16, tau=1.0)
    assert e.value.status == m.MALA_ERR_WORKSPACE
