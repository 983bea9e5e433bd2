"""GPU parity of the forward entry points (mala_fwd, fullattn_fwd) against
the CPU oracle, through the C ABI. Tolerances: tests/parity.py."""
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from parity import (AGREE_MIN, LSE_TOL, V2_TOL, bits_to_f64, bits_to_gpu, check_decisions,
                    gpu_to_f64, l2_ok, settle_fwd_branch, v1_exact_metric, v1_exact_ok, v1_ok,
                    v2)

pytestmark = pytest.mark.gpu

M = None


def mala():
    global M
    if M is None:
        import adaptive_softmax_attention_amd as m
        m.lib()
        M = m
    return M


def run_fwd(inp, tau, causal=True, dense=False, with_stats=True, nk_override=None, bq=64, bk=64):
    m = mala()
    q, k, v = bits_to_gpu(inp["q"]), bits_to_gpu(inp["k"]), bits_to_gpu(inp["v"])
    B, Hq, Nq, d = q.shape
    Nk = k.shape[2]
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device="cuda")
    Tr, Tc = -(-Nq // bq), -(-Nk // bk)
    stats = None
    if with_stats:
        stats = m.Stats(torch.zeros(4, dtype=torch.int64, device="cuda"),
                        torch.full((B, Hq, Tr, Tc), 255, dtype=torch.uint8, device="cuda"))
    if dense:
        m.fullattn_fwd(q, k, v, o, lse, causal=causal, stats=stats, block_q=bq, block_k=bk)
    else:
        m.mala_fwd(q, k, v, o, lse, causal=causal, tau=tau, stats=stats, block_q=bq, block_k=bk)
    torch.cuda.synchronize()
    dec = None
    cnt = None
    if with_stats:
        dec = stats.decisions.cpu().numpy().astype(np.int8)  # 255 (untested) -> -1
        cnt = stats.counters.cpu().numpy()
    return o, lse, dec, cnt


def compare_fwd(inp, tau, causal=True, sel=None, label="", bq=64, bk=64):
    q, k, v = bits_to_f64(inp["q"]), bits_to_f64(inp["k"]), bits_to_f64(inp["v"])
    print(f"[fwd {label}] q{tuple(q.shape)} k{tuple(k.shape)} tau={tau} causal={causal} "
          f"tile {bq}x{bk}", flush=True)
    o, lse, dec, cnt = run_fwd(inp, tau, causal, bq=bq, bk=bk)
    # the kernel without instrumentation (the timed instance) gives the same
    # results bitwise
    o2, lse2, _, _ = run_fwd(inp, tau, causal, with_stats=False, bq=bq, bk=bk)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    del o2, lse2
    go, gl = gpu_to_f64(o), lse.cpu().numpy().astype(np.float64)

    def run(force, flags=O.EXACT):
        return O.mala_fwd(q, k, v, tau, causal, bq, bk, round_flags=flags, force=force, sel=sel)

    free = run(None)
    legal = _legal(free["dec"], sel)
    # GPU decisions: every legal tile tested, nothing else written
    assert (dec[legal] >= 0).all()
    if sel is None:
        assert (dec[~legal] == -1).all()
    agree = check_decisions(dec, free, legal)
    ex, flipped = settle_fwd_branch(lambda f: run(f), dec, legal, free=free)
    # the bf16-operand model follows the exact oracle's settled decisions and
    # rounds P~ where the kernel does (against its lazy reference maximum)
    bf = run(ex["dec"].copy(), O.BF16_FWD | O.LAZY_REF)
    mag = run(ex["dec"].copy(), O.BF16_FWD | O.ABS)
    rows = _rows(sel, q.shape)
    ok, worst = v1_ok(go[rows], bf["o"][rows], mag["o"][rows])
    assert ok, f"V1 worst ratio {worst}"
    r2 = v2(go[rows], bf["o"][rows])
    assert r2 <= V2_TOL, r2
    ok, rl2 = l2_ok(go[rows], ex["o"][rows], mag["o"][rows])
    assert ok, f"relative L2 vs fp64 {rl2}"
    ok, worst = v1_exact_ok(go[rows], ex["o"][rows], mag["o"][rows])
    assert ok, f"V1 vs fp64 worst ratio {worst}"
    v1x = v1_exact_metric(go[rows], ex["o"][rows])
    print(f"  fwd V2 {r2:.2e}  max|dO|/max(1,|O|) vs fp64 {v1x:.2e}  rel L2 vs fp64 {rl2:.2e}",
          flush=True)
    assert np.abs(gl[rows[:3]] - ex["lse"][rows[:3]]).max() <= LSE_TOL
    assert np.isfinite(go[rows]).all() and np.isfinite(gl[rows[:3]]).all()
    if sel is None:
        # counters agree with the bitmap: legal and kept tiles, and block_k
        # slots for each valid row of a kept tile (Eq. 11)
        assert cnt[0] == int((dec >= 0).sum())
        assert cnt[1] == int((dec == 1).sum())
        Nq = q.shape[2]
        rows = np.array([min(Nq, (I + 1) * bq) - I * bq for I in range(dec.shape[2])])
        assert cnt[2] == int(((dec == 1) * rows[None, None, :, None]).sum()) * bk
    return {"agree": agree, "v2": r2, "l2": rl2, "v1x": v1x, "flipped": flipped, "dec": dec,
            "ora": ex, "o": o, "lse": lse}


def _legal(dec, sel):
    legal = dec >= 0
    if sel is not None:
        m = np.zeros_like(legal)
        for (b, h, i) in sel:
            m[b, h, i] = legal[b, h, i]
        legal = m
    return legal


def _rows(sel, shape):
    if sel is None:
        return (slice(None),) * 4
    B, H, N, d = shape
    mask = np.zeros((B, H, N), dtype=bool)
    for (b, h, i) in sel:
        mask[b, h, i * 64:min(N, (i + 1) * 64)] = True
    idx = np.nonzero(mask)
    return idx


def _gen(seed, B, Hq, Hkv, N, d, planted, sigma=3.0, local=False):
    return W.peaked(W.Spec(seed, B, Hq, Hkv, N, d, sigma, planted, local_bias=local), want_do=False)


def test_cfg1_forward():
    w = W.cfg1()
    r = compare_fwd(W.peaked(w.spec, want_do=False), w.tau, label=w.name)
    print("agree", r["agree"], "v2", r["v2"])


@pytest.mark.parametrize("N,Hq,Hkv,d,tau", [
    (1000, 2, 2, 64, 1.0),     # ragged tail, MHA (4 query blocks per workgroup)
    (777, 4, 2, 128, 1.0),     # ragged, GQA 2:1 (2 heads x 2 blocks)
    (1100, 8, 1, 128, 1.0),    # GQA 8:1 (4 heads per workgroup)
    (900, 8, 2, 128, 4.0),     # GQA 4:1, larger tolerance: more skipping
    (640, 3, 1, 64, 0.25),     # G = 3
])
def test_forward_shapes(N, Hq, Hkv, d, tau):
    inp = _gen(7 + N, 1, Hq, Hkv, N, d, 12)
    compare_fwd(inp, tau, label=f"N{N}")


@pytest.mark.parametrize("N", [1, 2, 63, 64, 65, 129])
def test_forward_tiny_and_tile_edges(N):
    inp = _gen(100 + N, 2, 4, 2, N, 64, 0)
    compare_fwd(inp, 1.0, label=f"tiny{N}")


def test_forward_noncausal_rectangular():
    spec_q = W.Spec(31, 1, 4, 2, 300, 128, 3.0, 0)
    spec_k = W.Spec(32, 1, 4, 2, 517, 128, 3.0, 8)
    a, b = W.peaked(spec_q, want_do=False), W.peaked(spec_k, want_do=False)
    inp = {"q": a["q"], "k": b["k"], "v": b["v"]}
    compare_fwd(inp, 1.0, causal=False, label="noncausal")


def test_forward_tau_extremes_and_dense_identity():
    inp = _gen(41, 1, 4, 1, 700, 128, 8)
    # tau = 0: every legal tile retained and bitwise equal to the dense path
    o0, l0, d0, _ = run_fwd(inp, 0.0)
    od, ld, dd, _ = run_fwd(inp, 0.0, dense=True)
    assert (d0[d0 >= 0] == 1).all()
    assert torch.equal(o0, od) and torch.equal(l0, ld)
    compare_fwd(inp, 0.0, label="tau0")
    r = compare_fwd(inp, math.inf, label="tauinf")
    # tau = inf keeps only the diagonal tile of every block
    dec = r["dec"]
    for i in range(dec.shape[2]):
        assert dec[0, 0, i, i] == 1 and (dec[0, 0, i, :i] == 0).all()


def test_forward_deterministic():
    inp = _gen(5, 1, 8, 1, 1500, 128, 16)
    a = run_fwd(inp, 1.0, with_stats=False)
    b = run_fwd(inp, 1.0, with_stats=False)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_cfg2_forward_full():
    w = W.cfg2()
    r = compare_fwd(W.peaked(w.spec, want_do=False), w.tau, label=w.name)
    print("cfg2 fwd agree", r["agree"], "v2", r["v2"], "flipped", r["flipped"])


@pytest.mark.parametrize("length", [1024, 4096])
def test_cfg3_forward(length):
    w = W.cfg3(length)
    compare_fwd(W.peaked(w.spec, want_do=False), w.tau, label=w.name)


@pytest.mark.parametrize("Nq,Nk,Hq,Hkv,d,tau", [
    (1, 300, 4, 2, 128, 1.0),       # one query at the end of the cache
    (37, 300, 4, 2, 128, 1.0),      # ragged chunk, offset not a whole tile
    (64, 300, 2, 1, 64, 0.25),
    (256, 1024, 8, 1, 128, 1.0),    # offset a whole number of tiles
    (129, 1000, 3, 3, 128, 4.0),
])
def test_forward_causal_chunk_against_cache(Nq, Nk, Hq, Hkv, d, tau):
    """Causal prefill of the last Nq queries against Nk keys (bottom-right
    alignment: query q sees keys k <= q + Nk - Nq)."""
    a = W.peaked(W.Spec(900 + Nq, 1, Hq, Hkv, Nk, d, 3.0, 6), want_do=False)
    inp = {"q": np.ascontiguousarray(a["q"][:, :, Nk - Nq:]), "k": a["k"], "v": a["v"]}
    compare_fwd(inp, tau, causal=True, label=f"chunk{Nq}of{Nk}")


@pytest.mark.parametrize("bq,bk", [(128, 128), (128, 64), (64, 128)])
@pytest.mark.parametrize("N,Hq,Hkv,d,tau,causal", [
    (777, 4, 2, 128, 1.0, True),     # ragged: partial 128-row and 128-key tiles
    (1100, 8, 1, 128, 1.0, True),    # GQA 8:1
    (640, 3, 1, 64, 4.0, True),      # G = 3 (one head, four query blocks per workgroup)
    (500, 2, 2, 128, 1.0, False),    # non-causal
])
def test_forward_decision_tile_128(bq, bk, N, Hq, Hkv, d, tau, causal):
    """Decision tiles of 128 rows and / or 128 keys: decisions, counters and
    values against the oracle run with the same tile (its decisions depend on
    the tile, Sec. 2.2)."""
    r = compare_fwd(_gen(700 + N + bq + bk, 1, Hq, Hkv, N, d, 8, local=True), tau, causal,
                    label=f"tile{bq}x{bk}", bq=bq, bk=bk)
    assert r["agree"] >= 0.99


def test_forward_decision_tile_128_chunk_against_cache():
    """A chunk of 100 queries at the end of 700 keys with 128 x 128 tiles:
    the shifted staircase with partial coarse tiles on both axes."""
    a = W.peaked(W.Spec(733, 1, 4, 2, 700, 128, 3.0, 8, local_bias=True), q_rows=list(range(600, 700)),
                 want_do=False)
    compare_fwd(a, 1.0, True, label="chunk128", bq=128, bk=128)


def test_forward_tile_128_tau0_is_dense():
    inp = _gen(741, 1, 4, 2, 600, 128, 8)
    for bq, bk in ((128, 128), (64, 128), (128, 64)):
        o1, l1, _, c1 = run_fwd(inp, 0.0, bq=bq, bk=bk)
        o2, l2, _, _ = run_fwd(inp, 0.0, dense=True, with_stats=False)
        # every tile kept: the same sums as the dense kernel in the same order
        assert c1[0] == c1[1]
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("N,Hkv,bq,bk", [(3000, 2, 128, 128), (3000, 2, 64, 128), (8192, 1, 64, 128)])
def test_forward_tile_128_upper_tile_kept_late(N, Hkv, bq, bk):
    """128-key tiles whose upper half fails the test against the tile's
    state while the lower half passes (the local bias makes this frequent at
    these lengths): the pair is kept, its upper half scored again and both
    halves updated against one reference maximum. Values and decisions
    against the oracle with the same tile."""
    inp = _gen(1700 + N + 64, 1, 2, Hkv, N, 128, 64, local=True)
    compare_fwd(inp, 4.0, True, label=f"late{N}-{bq}x{bk}", bq=bq, bk=bk)
