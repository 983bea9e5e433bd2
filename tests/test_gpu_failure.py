"""The kernels' bounded waits, forced to give up from the host.

The forward's vote exchange and the backward scoring pass's LDS ring both
wait on other waves of their workgroup. Each wait is bounded; the bound comes
from the environment variable MALA_WAIT_BOUND (read per call), and 0 makes
every wait give up at once. These tests set it to 0, so the give-up path runs
while every kernel still exits normally (nothing waits beyond its bound),
and check that the failure is visible: NaN outputs and, for the backward, the
status word at the start of the workspace. The same calls with the default
bound then give the normal results bitwise."""
import os

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


class wait_bound:
    def __init__(self, value):
        self.value = value

    def __enter__(self):
        self.old = os.environ.get("MALA_WAIT_BOUND")
        os.environ["MALA_WAIT_BOUND"] = str(self.value)

    def __exit__(self, *exc):
        if self.old is None:
            del os.environ["MALA_WAIT_BOUND"]
        else:
            os.environ["MALA_WAIT_BOUND"] = self.old


def _inputs():
    inp = W.peaked(W.Spec(91, 1, 8, 2, 2000, 128, 3.0, 16))
    return [bits_to_gpu(inp[x]) for x in ("q", "k", "v", "do")]


def test_forward_wait_give_up_gives_nan():
    m = mala()
    q, k, v, _ = _inputs()
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    m.mala_fwd(q, k, v, o, lse, tau=1.0)
    ref_o, ref_l = o.clone(), lse.clone()
    assert torch.isfinite(ref_o.float()).all() and torch.isfinite(ref_l).all()
    print("[failure] forward with every vote wait bounded at 0 polls", flush=True)
    with wait_bound(0):
        o.zero_()
        m.mala_fwd(q, k, v, o, lse, tau=1.0)
        torch.cuda.synchronize()
    # every query block takes part in a vote exchange, so every row gives up
    assert torch.isnan(o.float()).all() and torch.isnan(lse).all()
    # the dense path has no exchange and is unaffected
    with wait_bound(0):
        m.fullattn_fwd(q, k, v, o, lse)
        torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    # back to the default bound: the normal result, bitwise
    m.mala_fwd(q, k, v, o, lse, tau=1.0)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(lse, ref_l)


@pytest.mark.parametrize("dense", [False, True])
def test_backward_wait_give_up_gives_nan_and_status(dense):
    m = mala()
    q, k, v, do = _inputs()
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    m.mala_fwd(q, k, v, o, lse, tau=1.0)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(m.mala_bwd_workspace_bytes(q, k), dtype=torch.uint8, device="cuda")
    fn = m.fullattn_bwd if dense else m.mala_bwd
    kw = {} if dense else {"tau": 1.0}
    # the dense path only scores (and waits) when instrumented
    stats = m.Stats(torch.zeros(4, dtype=torch.int64, device="cuda")) if dense else None
    fn(q, k, v, o, lse, do, dq, dk, dv, ws, stats=stats, **kw)
    torch.cuda.synchronize()
    ref = [x.clone() for x in (dq, dk, dv)]
    status = lambda: int(ws[:4].view(torch.int32).item())
    assert status() == 0
    assert all(torch.isfinite(x.float()).all() for x in ref)
    print(f"[failure] backward (dense={dense}) with every ring wait bounded at 0 polls",
          flush=True)
    with wait_bound(0):
        fn(q, k, v, o, lse, do, dq, dk, dv, ws, stats=stats, **kw)
        torch.cuda.synchronize()
    assert status() == 1
    for x in (dq, dk, dv):
        assert torch.isnan(x.float()).all()
    # the next call resets the status and gives the normal result, bitwise
    fn(q, k, v, o, lse, do, dq, dk, dv, ws, stats=stats, **kw)
    torch.cuda.synchronize()
    assert status() == 0
    for a, b in zip((dq, dk, dv), ref):
        assert torch.equal(a, b)


def test_malformed_wait_bound_is_ignored():
    m = mala()
    q, k, v, _ = _inputs()
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    m.mala_fwd(q, k, v, o, lse, tau=1.0)
    ref = o.clone()
    for bad in ("", "-1", "12abc", "x"):
        with wait_bound(bad):
            m.mala_fwd(q, k, v, o, lse, tau=1.0)
            torch.cuda.synchronize()
        assert torch.equal(o, ref), bad
