"""GPU parity of the backward entry points (mala_bwd, fullattn_bwd) against
the CPU oracle, through the C ABI. The oracle backward consumes the oracle's
own forward outputs (O rounded to bf16 and LSE to fp32 in the bf16-operand
model), never the GPU's. Tolerances: tests/parity.py."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from parity import (AGREE_MIN, DELTA, LSE_TOL, V2_TOL, bits_to_f64, bits_to_gpu,
                    check_decisions, gpu_to_f64, l2_ok, settle_fwd_branch, v1_exact_metric,
                    v1_exact_ok, v1_ok, v2)

pytestmark = pytest.mark.gpu


def mala():
    import adaptive_softmax_attention_amd as m
    m.lib()
    return m


def run_fwd_bwd(inp, tau, causal=True, dense=False, bq=64, bk=64):
    m = mala()
    q, k, v, do = (bits_to_gpu(inp[x]) for x in ("q", "k", "v", "do"))
    B, Hq, Nq, d = q.shape
    Nk = k.shape[2]
    Tr, Tc = -(-Nq // bq), -(-Nk // bk)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device="cuda")
    fst = m.Stats(torch.zeros(4, dtype=torch.int64, device="cuda"),
                  torch.full((B, Hq, Tr, Tc), 255, dtype=torch.uint8, device="cuda"))
    bst = m.Stats(torch.zeros(4, dtype=torch.int64, device="cuda"),
                  torch.full((B, Hq, Tr, Tc), 255, dtype=torch.uint8, device="cuda"))
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(m.mala_bwd_workspace_bytes(q, k, causal=causal, block_q=bq, block_k=bk),
                     dtype=torch.uint8, device="cuda")
    t = {"block_q": bq, "block_k": bk}
    if dense:
        m.fullattn_fwd(q, k, v, o, lse, causal=causal, stats=fst, **t)
        m.fullattn_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, causal=causal, stats=bst, **t)
    else:
        m.mala_fwd(q, k, v, o, lse, causal=causal, tau=tau, stats=fst, **t)
        m.mala_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, causal=causal, tau=tau, stats=bst, **t)
    torch.cuda.synchronize()
    # the kernels without instrumentation (the timed instances) give the same
    # results bitwise
    o2, lse2 = torch.empty_like(o), torch.empty_like(lse)
    dq2, dk2, dv2 = torch.empty_like(dq), torch.empty_like(dk), torch.empty_like(dv)
    if dense:
        m.fullattn_fwd(q, k, v, o2, lse2, causal=causal, **t)
        m.fullattn_bwd(q, k, v, o, lse, do, dq2, dk2, dv2, ws, causal=causal, **t)
    else:
        m.mala_fwd(q, k, v, o2, lse2, causal=causal, tau=tau, **t)
        m.mala_bwd(q, k, v, o, lse, do, dq2, dk2, dv2, ws, causal=causal, tau=tau, **t)
    torch.cuda.synchronize()
    for a, b_, name in ((o, o2, "o"), (lse, lse2, "lse"), (dq, dq2, "dq"), (dk, dk2, "dk"),
                        (dv, dv2, "dv")):
        assert torch.equal(a, b_), f"{name}: instrumented and plain kernels differ"
    del o2, lse2, dq2, dk2, dv2
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv,
            "fdec": fst.decisions.cpu().numpy().astype(np.int8),
            "bdec": bst.decisions.cpu().numpy().astype(np.int8),
            "fcnt": fst.counters.cpu().numpy(), "bcnt": bst.counters.cpu().numpy()}


def _legal_sel(dec, sel):
    if sel is None:
        return dec >= 0
    m = np.zeros(dec.shape, dtype=bool)
    for (b, h, i) in sel:
        m[b, h, i] = dec[b, h, i] >= 0
    return m


def run_bwd_given(inp, o, lse, tau, causal=True, bq=64, bk=64):
    """The GPU backward alone, on given forward outputs (O as bf16 values,
    LSE as fp32 values)."""
    m = mala()
    q, k, v, do = (bits_to_gpu(inp[x]) for x in ("q", "k", "v", "do"))
    B, Hq, Nq, d = q.shape
    Tr, Tc = -(-Nq // bq), -(-k.shape[2] // bk)
    og = torch.from_numpy(np.ascontiguousarray(o, dtype=np.float32)).to(torch.bfloat16).cuda()
    lg = torch.from_numpy(np.ascontiguousarray(lse, dtype=np.float32)).cuda()
    assert np.array_equal(og.float().cpu().numpy(), np.asarray(o, dtype=np.float32))
    bst = m.Stats(torch.zeros(4, dtype=torch.int64, device="cuda"),
                  torch.full((B, Hq, Tr, Tc), 255, dtype=torch.uint8, device="cuda"))
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(m.mala_bwd_workspace_bytes(q, k, causal=causal, block_q=bq, block_k=bk),
                     dtype=torch.uint8, device="cuda")
    m.mala_bwd(q, k, v, og, lg, do, dq, dk, dv, ws, causal=causal, tau=tau, stats=bst,
               block_q=bq, block_k=bk)
    torch.cuda.synchronize()
    return {"dq": dq, "dk": dk, "dv": dv,
            "bdec": bst.decisions.cpu().numpy().astype(np.int8)}


def _settle_bwd(bwd, o_, lse_, gd):
    """Oracle backward decisions under (o_, lse_); where the GPU took the other
    side of a tile within DELTA of the threshold, the oracle's result on that
    branch. Returns (exact result, legal mask, agreement, flipped tiles)."""
    free = bwd(o_, lse_, O.EXACT)
    legal = free["dec"] >= 0
    assert (gd[legal] >= 0).all()
    agree = check_decisions(gd, free, legal)
    dis = legal & (gd != free["dec"])
    if dis.any():
        force = np.full(gd.shape, -1, dtype=np.int8)
        force[dis] = gd[dis]
        free = bwd(o_, lse_, O.EXACT, force)
    return free, legal, agree, int(dis.sum())


def _fwd_rows(shape, fwd_sel):
    """Mask [B, H, N] of the query rows whose forward the oracle computed."""
    B, H, N, _ = shape
    if fwd_sel is None:
        return np.ones((B, H, N), dtype=bool)
    m = np.zeros((B, H, N), dtype=bool)
    for (b, h, i) in fwd_sel:
        m[b, h, 64 * i:min(N, 64 * i + 64)] = True
    return m


def compare_bwd(inp, tau, causal=True, sel_q=None, sel_k=None, fwd_sel=None, label="", bq=64,
                bk=64):
    """Two checks of the backward.
    End to end (GPU forward, then GPU backward on its outputs): decisions,
    fidelity to the fp64 oracle (relative L2, with the D term for the stored
    O), nesting in the forward support.
    Backward alone (GPU backward on the oracle's bf16-model forward outputs,
    so that both sides form D from the same stored O): decisions, V1 and V2
    against the oracle's bf16-operand backward model."""
    q, k, v, do = (bits_to_f64(inp[x]) for x in ("q", "k", "v", "do"))
    G = q.shape[1] // k.shape[1]
    print(f"[bwd {label}] q{q.shape} k{k.shape} tau={tau} causal={causal} tile {bq}x{bk}",
          flush=True)
    g = run_fwd_bwd(inp, tau, causal, bq=bq, bk=bk)

    # --- oracle forward on the GPU's branch of ambiguous tiles ---
    def fwd(force, flags=O.EXACT):
        return O.mala_fwd(q, k, v, tau, causal, bq, bk, round_flags=flags, force=force,
                          sel=fwd_sel)

    ffree = fwd(None)
    flegal = _legal_sel(ffree["dec"], fwd_sel)
    fex, fflip = settle_fwd_branch(fwd, g["fdec"], flegal, free=ffree)
    # the bf16-operand model follows the exact oracle's settled decisions
    fbf = fwd(fex["dec"].copy(), O.BF16_FWD)

    def bwd(o_, lse_, flags, force=None):
        return O.mala_bwd(q, k, v, o_, lse_, do, tau, causal, bq, bk, round_flags=flags,
                          force=force, sel_q=sel_q, sel_k=sel_k)

    rq = _rows_q(sel_q, q.shape)
    rk = _rows_k(sel_k, k.shape, G)
    names = (("dq", rq), ("dk", rk), ("dv", rk))

    # --- end to end: the oracle backward on the oracle's exact forward ---
    gd = g["bdec"]
    bex, legal, agree, bflip = _settle_bwd(bwd, fex["o"], fex["lse"], gd)
    bmag = bwd(fbf["o"], fbf["lse"], O.BF16_BWD | O.ABS, bex["dec"].copy())
    bmd = bwd(fbf["o"], fbf["lse"], O.ABS_D, bex["dec"].copy())
    out = {"agree": agree, "fflip": fflip, "bflip": bflip}
    for name, rows in names:
        x = gpu_to_f64(g[name])[rows]
        assert np.isfinite(x).all()
        ok, rl2 = l2_ok(x, bex[name][rows], bmag[name][rows], bmd[name][rows])
        assert ok, f"{name} relative L2 vs fp64 {rl2}"
        out[name + "_l2"] = rl2
        out[name + "_v1x"] = v1_exact_metric(x, bex[name][rows])
    # backward support nested in forward support (Sec. 2.2), up to ties
    viol = (gd == 1) & (g["fdec"] == 0) & _legal_sel(fex["dec"], fwd_sel)
    if viol.any():
        fm = fex["margin"][viol]
        assert np.all(np.abs(fm) < DELTA), "backward retained a tile forward skipped"
    out["bret"] = float((gd == 1).sum() / max(1, (gd >= 0).sum()))
    # counters agree with the bitmaps: legal and kept tiles of the scoring pass, and
    # every kept (tile, key block) listed once by the dK/dV pass
    bc, fc = g["bcnt"], g["fcnt"]
    assert bc[0] == int((gd >= 0).sum()) and bc[1] == int((gd == 1).sum())
    # the dK/dV pass loads dO once per legal 64 x 64 sub-tile of a kept tile
    sub = _subtile_counts(q.shape[2], k.shape[2], bq, bk, causal)
    assert bc[3] == int(((gd == 1) * sub[None, None]).sum())
    rows = np.array([min(q.shape[2], (I + 1) * bq) - I * bq for I in range(gd.shape[2])])
    assert bc[2] == int(((gd == 1) * rows[None, None, :, None]).sum()) * bk
    assert fc[0] == int((g["fdec"] >= 0).sum()) and fc[1] == int((g["fdec"] == 1).sum())

    # --- the backward alone, on the oracle's bf16-model forward outputs (the
    #     GPU's own outputs fill the rows the oracle did not compute; no
    #     compared value depends on them) ---
    rows = _fwd_rows(q.shape, fwd_sel)
    o_in = np.where(rows[..., None], fbf["o"], gpu_to_f64(g["o"]))
    lse_in = np.where(rows, fbf["lse"], g["lse"].cpu().numpy().astype(np.float64))
    g2 = run_bwd_given(inp, o_in, lse_in, tau, causal, bq=bq, bk=bk)
    b2, _, agree2, bflip2 = _settle_bwd(bwd, fbf["o"], fbf["lse"], g2["bdec"])
    b2bf = bwd(fbf["o"], fbf["lse"], O.BF16_BWD, b2["dec"].copy())
    b2mag = bwd(fbf["o"], fbf["lse"], O.BF16_BWD | O.ABS, b2["dec"].copy())
    out["agree_alone"] = agree2
    out["bflip_alone"] = bflip2
    for name, rows_ in names:
        x = gpu_to_f64(g2[name])[rows_]
        assert np.isfinite(x).all()
        ok, worst = v1_ok(x, b2bf[name][rows_], b2mag[name][rows_])
        assert ok, f"{name} V1 worst ratio {worst}"
        r2 = v2(x, b2bf[name][rows_])
        assert r2 <= V2_TOL, f"{name} V2 {r2}"
        out[name + "_v2"] = r2
        ok, worst = v1_exact_ok(x, b2[name][rows_], b2mag[name][rows_])
        assert ok, f"{name} V1 vs fp64 worst ratio {worst}"
        out[name + "_v1x_alone"] = v1_exact_metric(x, b2[name][rows_])
    out["g"] = g
    print({k_: v_ for k_, v_ in out.items() if k_ != "g"}, flush=True)
    return out


def _subtile_counts(Nq, Nk, bq, bk, causal):
    """Legal 64 x 64 sub-tiles of every bq x bk decision tile (queries at the
    end of the keys when causal)."""
    off = Nk - Nq if causal else 0
    tr, tc = -(-Nq // 64), -(-Nk // 64)
    kq, kk = bq // 64, bk // 64
    out = np.zeros((-(-Nq // bq), -(-Nk // bk)), dtype=np.int64)
    for i in range(tr):
        for j in range(tc):
            if not causal or 64 * j <= 64 * i + 63 + off:
                out[i // kq, j // kk] += 1
    return out


def _rows_q(sel, shape):
    if sel is None:
        return (slice(None),) * 4
    B, H, N, d = shape
    m = np.zeros((B, H, N), dtype=bool)
    for (b, h, i) in sel:
        m[b, h, 64 * i:min(N, 64 * i + 64)] = True
    return np.nonzero(m)


def _rows_k(sel, shape, G):
    if sel is None:
        return (slice(None),) * 4
    B, H, N, d = shape
    m = np.zeros((B, H, N), dtype=bool)
    for (b, g, j) in sel:
        m[b, g, 64 * j:min(N, 64 * j + 64)] = True
    return np.nonzero(m)


def _gen(seed, B, Hq, Hkv, N, d, planted, sigma=3.0, local=False):
    return W.peaked(W.Spec(seed, B, Hq, Hkv, N, d, sigma, planted, local_bias=local))


@pytest.mark.parametrize("N,Hq,Hkv,d,tau", [
    (1, 2, 1, 128, 1.0),
    (65, 4, 2, 64, 1.0),
    (200, 2, 2, 128, 1.0),
    (777, 4, 1, 128, 1.0),      # ragged, GQA 4:1, odd number of key blocks
    (640, 8, 2, 128, 4.0),
    (1000, 3, 3, 64, 0.25),
])
def test_backward_shapes(N, Hq, Hkv, d, tau):
    compare_bwd(_gen(300 + N, 1, Hq, Hkv, N, d, 10), tau, label=f"N{N}")


def test_backward_batch2_tau_extremes():
    inp = _gen(11, 2, 4, 2, 333, 128, 6)
    compare_bwd(inp, 0.0, label="tau0")
    r = compare_bwd(inp, math.inf, label="tauinf")
    assert not r["g"]["dq"].any() and not r["g"]["dk"].any() and not r["g"]["dv"].any()


def test_backward_noncausal():
    a = W.peaked(W.Spec(51, 1, 4, 2, 300, 128, 3.0, 0))
    b = W.peaked(W.Spec(52, 1, 4, 2, 450, 128, 3.0, 8))
    inp = {"q": a["q"], "do": a["do"], "k": b["k"], "v": b["v"]}
    compare_bwd(inp, 1.0, causal=False, label="noncausal")


def test_backward_dense_identity_and_determinism():
    inp = _gen(61, 1, 8, 2, 900, 128, 12)
    a = run_fwd_bwd(inp, 0.0)
    b = run_fwd_bwd(inp, 0.0, dense=True)
    c = run_fwd_bwd(inp, 0.0)
    # every gradient is summed in a fixed order (dK, dV in registers or in
    # segment partials added in index order, dQ query-major without atomics):
    # bitwise repeatable, and at tau = 0 equal to the dense path
    for x in ("dq", "dk", "dv"):
        assert torch.equal(a[x], c[x]), x
        assert torch.equal(a[x], b[x]), x


def test_backward_eight_segment_pairs():
    """16 query heads on one KV head at 8K with tau 256: the backward keeps
    little besides the sink and the planted hubs, so the dK/dV pass cuts the
    heaviest pairs of key blocks into the maximum of 8 segments and its
    finalize adds 8 partial sums per key (the host model of the pairing
    confirms it on the GPU's own decisions). Every dQ, dK and dV element is
    compared."""
    from bwd_schedule import pairs_and_segments
    inp = _gen(4242, 1, 16, 1, 8192, 128, 16)
    r = compare_bwd(inp, 256.0, label="eight-segments")
    sched = pairs_and_segments(r["g"]["bdec"], 1, 8192, 8192)
    nseg = [row[3] for row in sched[(0, 0)]]
    print("segments per pair (largest first):", sorted(nseg, reverse=True)[:8], flush=True)
    assert max(nseg) == 8


def test_cfg2_forward_backward_full():
    w = W.cfg2()
    r = compare_bwd(W.peaked(w.spec), w.tau, label=w.name)
    print("cfg2 bwd retained", r["bret"])


@pytest.mark.parametrize("length", [1024, 4096])
def test_cfg3_forward_backward(length):
    w = W.cfg3(length)
    compare_bwd(W.peaked(w.spec), w.tau, label=w.name)


def test_cfg4_layout_8k_full():
    """The 128K workload's head layout (8 query / 1 KV head, d 128, 256 planted
    pairs' density) at 8K, every output compared."""
    w = W.cfg4()
    s = w.spec
    inp = W.peaked(W.Spec(s.seed, 1, 8, 1, 8192, 128, s.sigma_s, 16))
    r = compare_bwd(inp, w.tau, label="cfg4-layout-8k")
    g = r["g"]
    assert g["dk"].abs().sum().item() > 0 and g["dv"].abs().sum().item() > 0


@pytest.mark.parametrize("Nq,Nk,Hq,Hkv,d,tau", [
    (37, 300, 4, 2, 128, 1.0),
    (64, 300, 2, 1, 64, 0.25),
    (256, 1024, 8, 1, 128, 1.0),
    (129, 1000, 3, 3, 128, 4.0),
])
def test_backward_causal_chunk_against_cache(Nq, Nk, Hq, Hkv, d, tau):
    """Backward of a causal chunk of the last Nq queries against Nk keys."""
    a = W.peaked(W.Spec(950 + Nq, 1, Hq, Hkv, Nk, d, 3.0, 6))
    inp = {"q": np.ascontiguousarray(a["q"][:, :, Nk - Nq:]), "k": a["k"], "v": a["v"],
           "do": np.ascontiguousarray(a["do"][:, :, Nk - Nq:])}
    compare_bwd(inp, tau, causal=True, label=f"chunk{Nq}of{Nk}")


@pytest.mark.parametrize("bq,bk", [(128, 128), (128, 64), (64, 128)])
@pytest.mark.parametrize("N,Hq,Hkv,d,tau,causal", [
    (777, 4, 2, 128, 1.0, True),     # ragged, GQA 2:1, odd number of 128-key tiles
    (640, 3, 1, 64, 4.0, True),      # G = 3
    (450, 2, 2, 128, 1.0, False),    # non-causal
])
def test_backward_decision_tile_128(bq, bk, N, Hq, Hkv, d, tau, causal):
    """Decision tiles of 128 rows and / or 128 keys, end to end and on the
    oracle's forward outputs, against the oracle run with the same tile."""
    compare_bwd(_gen(800 + N + bq + bk, 1, Hq, Hkv, N, d, 8, local=True), tau, causal,
                label=f"tile{bq}x{bk}", bq=bq, bk=bk)


def test_backward_decision_tile_128_chunk_against_cache():
    a = W.peaked(W.Spec(833, 1, 4, 2, 700, 128, 3.0, 8, local_bias=True),
                 q_rows=list(range(600, 700)))
    compare_bwd(a, 1.0, True, label="chunk128", bq=128, bk=128)
