"""The entry points under HIP graph capture (test code). The library issues
only kernel launches on the caller's stream (no allocation, memset or
synchronisation), so a call can be captured once and replayed. Each test
captures on small inputs, replays several times with eager work and
synchronisations in between, changes the captured inputs in place between
replays, and checks every replay bitwise against an eager call on the same
inputs (the kernels are deterministic)."""
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


def _decode_inputs(seed, B, Hq, Hkv, Nk, d):
    inp = W.peaked(W.Spec(seed, B, Hq, Hkv, Nk, d, 3.0, 16), q_rows=[Nk - 1], want_do=False)
    q = bits_to_gpu(np.ascontiguousarray(inp["q"][:, :, 0, :]))
    return q, bits_to_gpu(inp["k"]), bits_to_gpu(inp["v"])


def test_decode_noalloc_captured_and_replayed():
    m = mala()
    B, Hq, Hkv, Nk, d, S, tau = 4, 16, 4, 3000, 128, 6, 1.0
    a = dict(zip("qkv", _decode_inputs(9101, B, Hq, Hkv, Nk, d)))
    b = dict(zip("qkv", _decode_inputs(9102, B, Hq, Hkv, Nk, d)))
    q, k, v = (a[x].clone() for x in "qkv")
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    ws = torch.empty(m.mala_decode_workspace_bytes(q, k, S), dtype=torch.uint8, device="cuda")

    def eager(x):
        oe, le = torch.empty_like(o), torch.empty_like(lse)
        m.mala_decode(x["q"], x["k"], x["v"], oe, le, S, ws, tau=tau)
        torch.cuda.synchronize()
        return oe, le

    print("[graph] decode: warm-up and eager references", flush=True)
    m.mala_decode_noalloc(q, k, v, o, lse, S, tau=tau)  # first call on the device: address lookup
    torch.cuda.synchronize()
    ref_a, ref_b = eager(a), eager(b)
    assert not torch.equal(ref_a[0], ref_b[0])

    print("[graph] decode: capture", flush=True)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        m.mala_decode_noalloc(q, k, v, o, lse, S, tau=tau)
    for rep, src in enumerate((a, b, a, b)):
        for dst, x in ((q, "q"), (k, "k"), (v, "v")):
            dst.copy_(src[x])
        o.fill_(0)
        lse.fill_(0)
        print(f"[graph] decode: replay {rep}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        ro, rl = ref_a if src is a else ref_b
        assert torch.equal(o, ro) and torch.equal(lse, rl), rep
        eager(b if src is a else a)  # eager work between replays


def _prefill(seed, N):
    a = W.peaked(W.Spec(seed, 1, 4, 1, N, 128, 3.0, 8))
    return {x: bits_to_gpu(a[x]) for x in ("q", "k", "v", "do")}


def test_forward_and_backward_captured_and_replayed():
    m = mala()
    N, tau = 777, 1.0
    a, b = _prefill(9201, N), _prefill(9202, N)
    q, k, v, do = (a[x].clone() for x in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(m.mala_bwd_workspace_bytes(q, k), dtype=torch.uint8, device="cuda")
    ws_e = torch.empty_like(ws)

    def eager(x):
        oe, le = torch.empty_like(o), torch.empty_like(lse)
        g_ = [torch.empty_like(t) for t in (dq, dk, dv)]
        m.mala_fwd(x["q"], x["k"], x["v"], oe, le, tau=tau)
        m.mala_bwd(x["q"], x["k"], x["v"], oe, le, x["do"], *g_, ws_e, tau=tau)
        torch.cuda.synchronize()
        return [oe, le] + g_

    print("[graph] fwd+bwd: warm-up and eager references", flush=True)
    ref_a, ref_b = eager(a), eager(b)
    assert not torch.equal(ref_a[0], ref_b[0])
    assert all(torch.isfinite(t.float()).all() for t in ref_a)

    print("[graph] fwd+bwd: capture", flush=True)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        m.mala_fwd(q, k, v, o, lse, tau=tau)
        m.mala_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, tau=tau)
    for rep, src in enumerate((a, b, a, b)):
        for dst, x in ((q, "q"), (k, "k"), (v, "v"), (do, "do")):
            dst.copy_(src[x])
        for t in (o, lse, dq, dk, dv):
            t.fill_(0)
        print(f"[graph] fwd+bwd: replay {rep}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        ref = ref_a if src is a else ref_b
        for name, got, want in zip(("o", "lse", "dq", "dk", "dv"), (o, lse, dq, dk, dv), ref):
            assert torch.equal(got, want), (rep, name)
        eager(b if src is a else a)  # eager work between replays
