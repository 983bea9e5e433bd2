"""Every entry point writes its outputs and nothing else, through the C ABI.

Each output tensor and the workspace sit in the middle of a larger device
buffer whose guard regions hold a fill pattern: after the call the guards
must be untouched and the inputs unchanged. Each call runs twice, over two
different fill patterns, and must give the same outputs bit for bit (every
sum runs in a fixed order), so that no output element is left as it was
found. Shapes are ragged (partial tiles, rectangular causal, paged caches with
lengths that end mid-page) so that every tail path is exercised."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from parity import bits_to_gpu

pytestmark = pytest.mark.gpu

PAD = 8192  # guard bytes on each side


def mala():
    import adaptive_softmax_attention_amd as m
    m.lib()
    return m


class Guarded:
    """A tensor of `shape` and `dtype` inside a device buffer with PAD guard
    bytes on each side, all bytes set to `fill`."""

    def __init__(self, shape, dtype, fill):
        esz = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(shape)) if len(shape) else 1
        self.nbytes = n * esz
        self.raw = torch.full((PAD + self.nbytes + PAD,), fill, dtype=torch.uint8, device="cuda")
        self.fill = fill
        self.t = self.raw[PAD:PAD + self.nbytes].view(dtype).view(shape)

    def guards_intact(self):
        g = torch.cat([self.raw[:PAD], self.raw[PAD + self.nbytes:]])
        return bool((g == self.fill).all())


def _inputs(seed, B, Hq, Hkv, Nq, Nk, d):
    spec = W.Spec(seed, B, Hq, Hkv, Nk, d, 3.0, 8, local_bias=True)
    inp = W.peaked(spec, q_rows=list(range(Nk - Nq, Nk)))
    return {x: bits_to_gpu(inp[x]) for x in ("q", "k", "v", "do")}


def _prefill(m, t, causal, tau, dense, fill, tile=(64, 64)):
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    B, Hq, Nq, d = q.shape
    o = Guarded(q.shape, torch.bfloat16, fill)
    lse = Guarded((B, Hq, Nq), torch.float32, fill)
    dq, dk, dv = (Guarded(x.shape, torch.bfloat16, fill) for x in (q, k, v))
    tk = {"block_q": tile[0], "block_k": tile[1]}
    ws = Guarded((m.mala_bwd_workspace_bytes(q, k, causal=causal, **tk),), torch.uint8, fill)
    if dense:
        m.fullattn_fwd(q, k, v, o.t, lse.t, causal=causal, **tk)
        m.fullattn_bwd(q, k, v, o.t, lse.t, do, dq.t, dk.t, dv.t, ws.t, causal=causal, **tk)
    else:
        m.mala_fwd(q, k, v, o.t, lse.t, causal=causal, tau=tau, **tk)
        m.mala_bwd(q, k, v, o.t, lse.t, do, dq.t, dk.t, dv.t, ws.t, causal=causal, tau=tau, **tk)
    torch.cuda.synchronize()
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv, "ws": ws}


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,causal", [
    (2, 4, 2, 777, 777, 128, True),    # ragged causal, GQA 2:1, batch 2
    (1, 3, 1, 37, 300, 64, True),      # chunk against a cache, G = 3
    (1, 4, 4, 300, 450, 128, False),   # non-causal rectangular
    (1, 8, 1, 65, 65, 128, True),      # one row past a tile, G = 8
])
@pytest.mark.parametrize("dense,tile", [(False, (64, 64)), (True, (64, 64)), (False, (128, 128))])
def test_prefill_writes_only_its_outputs(B, Hq, Hkv, Nq, Nk, d, causal, dense, tile):
    m = mala()
    t = _inputs(900 + Nq, B, Hq, Hkv, Nq, Nk, d)
    before = {x: y.clone() for x, y in t.items()}
    print(f"[bounds] prefill B{B} Hq{Hq} Hkv{Hkv} Nq{Nq} Nk{Nk} d{d} causal={causal} "
          f"dense={dense} tile={tile}", flush=True)
    r1 = _prefill(m, t, causal, 1.0, dense, 0xA5, tile)
    r2 = _prefill(m, t, causal, 1.0, dense, 0x5A, tile)
    for name in ("o", "lse", "dq", "dk", "dv", "ws"):
        assert r1[name].guards_intact() and r2[name].guards_intact(), name
    for x in t:
        assert torch.equal(t[x], before[x]), f"input {x} changed"
    for name in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(r1[name].t, r2[name].t), name
    assert torch.isfinite(r1["dq"].t.float()).all() and torch.isfinite(r1["o"].t.float()).all()


def _decode_inputs(seed, B, Hq, Hkv, Nk, d):
    inp = W.peaked(W.Spec(seed, B, Hq, Hkv, Nk, d, 3.0, 8), q_rows=[Nk - 1], want_do=False)
    return (bits_to_gpu(np.ascontiguousarray(inp["q"][:, :, 0, :])), bits_to_gpu(inp["k"]),
            bits_to_gpu(inp["v"]))


@pytest.mark.parametrize("B,Hq,Hkv,Nk,d,S", [
    (3, 8, 2, 1000, 128, 3),
    (2, 4, 4, 65, 64, 2),
    (1, 8, 1, 4097, 128, 7),
])
@pytest.mark.parametrize("dense,bk", [(False, 64), (True, 64), (False, 128)])
def test_decode_writes_only_its_outputs(B, Hq, Hkv, Nk, d, S, dense, bk):
    m = mala()
    S = min(S, -(-Nk // bk))  # a split owns at least one decision tile
    q, k, v = _decode_inputs(950 + Nk, B, Hq, Hkv, Nk, d)
    before = [x.clone() for x in (q, k, v)]
    print(f"[bounds] decode B{B} Hq{Hq} Hkv{Hkv} Nk{Nk} d{d} S{S} dense={dense}", flush=True)
    outs = []
    for fill in (0xA5, 0x5A):
        o = Guarded(q.shape, torch.bfloat16, fill)
        lse = Guarded((B, Hq), torch.float32, fill)
        ws = Guarded((m.mala_decode_workspace_bytes(q, k, S),), torch.uint8, fill)
        if dense:
            m.fullattn_decode(q, k, v, o.t, lse.t, S, ws.t, block_k=bk)
        else:
            m.mala_decode(q, k, v, o.t, lse.t, S, ws.t, tau=1.0, block_k=bk)
        torch.cuda.synchronize()
        assert o.guards_intact() and lse.guards_intact() and ws.guards_intact()
        outs.append((o.t.clone(), lse.t.clone()))
    for x, y in zip((q, k, v), before):
        assert torch.equal(x, y)
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert torch.isfinite(outs[0][0].float()).all()


@pytest.mark.parametrize("dense", [False, True])
def test_paged_decode_writes_only_its_outputs(dense):
    m = mala()
    lens = [1, 63, 64, 700, 1000]
    B, Hq, Hkv, d, S = len(lens), 8, 2, 128, 3
    max_len = max(lens)
    inp = W.peaked(W.Spec(77, B, Hq, Hkv, max_len, d, 3.0, 8), want_do=False)
    q = bits_to_gpu(np.stack([inp["q"][b, :, lens[b] - 1] for b in range(B)]))
    tiles = [-(-n // 64) for n in lens]
    P = sum(tiles) + 3
    rng = np.random.default_rng(77)
    order = rng.permutation(P)
    kp = W.f32_to_bf16_bits(rng.standard_normal((P, Hkv, 64, d)).astype(np.float32))
    vp = kp.copy()
    table = np.zeros((B, -(-max_len // 64)), dtype=np.int32)
    t_ = 0
    for b in range(B):
        for j in range(tiles[b]):
            pg = int(order[t_])
            t_ += 1
            table[b, j] = pg
            n = min(64, lens[b] - 64 * j)
            kp[pg, :, :n] = inp["k"][b, :, 64 * j:64 * j + n]
            vp[pg, :, :n] = inp["v"][b, :, 64 * j:64 * j + n]
    kp_g, vp_g = bits_to_gpu(kp), bits_to_gpu(vp)
    table_g = torch.from_numpy(table).cuda()
    lens_g = torch.from_numpy(np.array(lens, dtype=np.int32)).cuda()
    before = [x.clone() for x in (q, kp_g, vp_g, table_g, lens_g)]
    print(f"[bounds] paged decode lens {lens} dense={dense}", flush=True)
    outs = []
    for fill in (0xA5, 0x5A):
        o = Guarded(q.shape, torch.bfloat16, fill)
        lse = Guarded((B, Hq), torch.float32, fill)
        ws = Guarded((m.mala_decode_paged_workspace_bytes(q, max_len, Hkv, S),), torch.uint8,
                     fill)
        if dense:
            m.fullattn_decode_paged(q, kp_g, vp_g, table_g, lens_g, max_len, o.t, lse.t, S, ws.t)
        else:
            m.mala_decode_paged(q, kp_g, vp_g, table_g, lens_g, max_len, o.t, lse.t, S, ws.t,
                                tau=1.0)
        torch.cuda.synchronize()
        assert o.guards_intact() and lse.guards_intact() and ws.guards_intact()
        outs.append((o.t.clone(), lse.t.clone()))
    for x, y in zip((q, kp_g, vp_g, table_g, lens_g), before):
        assert torch.equal(x, y)
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert torch.isfinite(outs[0][0].float()).all() and torch.isfinite(outs[0][1]).all()
