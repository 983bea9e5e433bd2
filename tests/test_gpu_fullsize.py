"""Full-size GPU parity: the 16K and 32K rows of the length sweep, the 128K
operator workload the benchmark times, and the 128K decode workload on all
its sequences and tolerances, against the CPU oracle run on the host.

For the prefill workloads the oracle runs the exact forward on every query
block of every head (in chunks, with progress lines), which gives

  * the forward's decisions on every legal tile (agreement, and every
    difference within DELTA of the threshold, the oracle then taking the
    GPU's branch of that tile);
  * LSE of every row (|delta| <= 1e-3) and O of every row against the exact
    result, with the elementwise bound 2^-6 (Mbar + |O|) + 1e-4 where Mbar =
    max_k |V_kc| bounds the magnitude sum M = sum_k p_k |V_kc| from above
    (so this is implied by the bound of tests/parity.py), plus the strict
    V1 / V2 / relative-L2 checks on sampled blocks with the oracle's exact
    magnitudes;
  * the final log-normaliser of every row, so that the backward can be
    checked on key blocks every later query keeps: key block 0 (the
    attention sink) and the heaviest hub blocks, which the dK/dV pass cuts
    into the most segments, plus sampled query blocks for dQ.

The backward is checked twice, as in tests/test_gpu_bwd.py: end to end (GPU
forward then GPU backward, against the fp64 oracle with the relative-L2
bound) and alone (the GPU backward fed the oracle's exact forward outputs in
their stored precision, bf16 O and fp32 LSE, against the oracle's bf16-
operand backward on the same inputs: V1, V2 and the fp64 elementwise bound).
"""
import os
import time

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from bwd_schedule import pairs_and_segments, segments_of_block
from parity import (DELTA, LSE_TOL, V2_TOL, bits_to_f64, check_decisions, gpu_to_f64, l2_ok,
                    settle_fwd_branch, v1_exact_metric, v1_exact_ok, v1_ok, v2)
from test_gpu_bwd import run_bwd_given, run_fwd_bwd

pytestmark = pytest.mark.gpu


@pytest.fixture
def say(capsys):
    """Progress lines that reach the terminal while a long oracle run is in
    progress, and also a file fullsize_progress.log in the folder named by
    MALA_PROGRESS_DIR when that variable is set."""
    logdir = os.environ.get("MALA_PROGRESS_DIR", "")
    t0 = time.time()

    def _say(msg):
        line = f"[{time.time() - t0:7.1f}s] {msg}"
        with capsys.disabled():
            print(line, flush=True)
        if logdir and os.path.isdir(logdir):
            with open(os.path.join(logdir, "fullsize_progress.log"), "a") as f:
                f.write(line + "\n")
    return _say


def oracle_fwd_blocks(q, k, v, tau, blocks, say, flags=O.EXACT, force=None, chunks=8,
                      label=""):
    """The oracle forward on the query blocks `blocks` ((b, h, i) list), run
    in `chunks` pieces; returns full-size arrays (NaN / -1 outside)."""
    B, Hq, N, d = q.shape
    Tr, Tc = -(-N // 64), -(-k.shape[2] // 64)
    out = {"o": np.full(q.shape, np.nan), "lse": np.full((B, Hq, N), np.nan),
           "dec": np.full((B, Hq, Tr, Tc), O.ILLEGAL, dtype=np.int8),
           "margin": np.full((B, Hq, Tr, Tc), np.nan)}
    blocks = list(blocks)
    step = -(-len(blocks) // chunks)
    for c0 in range(0, len(blocks), step):
        part = blocks[c0:c0 + step]
        t = time.time()
        r = O.mala_fwd(q, k, v, tau, round_flags=flags, force=force, sel=part)
        for (b, h, i) in part:
            rs = slice(64 * i, min(N, 64 * i + 64))
            out["o"][b, h, rs] = r["o"][b, h, rs]
            out["lse"][b, h, rs] = r["lse"][b, h, rs]
            out["dec"][b, h, i] = r["dec"][b, h, i]
            out["margin"][b, h, i] = r["margin"][b, h, i]
        del r
        say(f"{label} oracle forward: {min(len(blocks), c0 + step)}/{len(blocks)} blocks "
            f"({time.time() - t:.1f}s for this chunk)")
    return out


def settle_forward(q, k, v, tau, fex, gdec, say):
    """Where the GPU took the other side of a forward tile within DELTA of
    the threshold, rerun the oracle on the affected blocks with that branch
    (check_decisions has already bounded every difference)."""
    legal = fex["dec"] >= 0
    dis = legal & (gdec != fex["dec"])
    if not dis.any():
        return fex, 0
    blocks = sorted({(int(b), int(h), int(i)) for (b, h, i, _) in np.argwhere(dis)})
    say(f"forward: {int(dis.sum())} tiles in the delta band, {len(blocks)} blocks rerun")
    base = fex

    def run(force):
        r = O.mala_fwd(q, k, v, tau, force=force, sel=blocks)
        out = {key: base[key].copy() for key in ("o", "lse", "dec", "margin")}
        N = q.shape[2]
        for (b, h, i) in blocks:
            rs = slice(64 * i, min(N, 64 * i + 64))
            out["o"][b, h, rs] = r["o"][b, h, rs]
            out["lse"][b, h, rs] = r["lse"][b, h, rs]
            out["dec"][b, h, i] = r["dec"][b, h, i]
            out["margin"][b, h, i] = r["margin"][b, h, i]
        return out

    return settle_fwd_branch(run, gdec, legal, free=fex)


def heavy_key_blocks(bdec, heads_kv, N, per_group=2):
    """Per KV head: key block 0 and the `per_group` key blocks (other than 0)
    of the pairs the dK/dV pass cuts into the most segments, heaviest first."""
    sched = pairs_and_segments(bdec, heads_kv, N, N)
    B, Hq = bdec.shape[:2]
    G = Hq // heads_kv
    kept = (bdec == 1).reshape(B, heads_kv, G, *bdec.shape[2:]).sum(axis=(2, 3))
    sel = []
    for b in range(B):
        for g in range(heads_kv):
            cand = [j for (jA, jB, _, _) in sched[(b, g)] for j in (jA, jB) if j > 0]
            cand.sort(key=lambda j: (-segments_of_block(sched, b, g, j), -kept[b, g, j]))
            sel += [(b, g, 0)] + [(b, g, j) for j in cand[:per_group]]
    return sel, sched


def check_fullsize(inp, tau, sel_q, say, label, sample_blocks, kv_per_group=2):
    q, k, v, do = (bits_to_f64(inp[x]) for x in ("q", "k", "v", "do"))
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    Tr = -(-N // 64)
    say(f"[{label}] GPU forward + backward, q{q.shape} k{k.shape} tau {tau}")
    g = run_fwd_bwd(inp, tau)
    gdec, bdec = g["fdec"], g["bdec"]

    # ---- forward: every block of every head ----
    blocks = [(b, h, i) for b in range(B) for h in range(Hq) for i in range(Tr)]
    fex = oracle_fwd_blocks(q, k, v, tau, blocks, say, label=label)
    legal = fex["dec"] >= 0
    assert (gdec[legal] >= 0).all() and (gdec[~legal] == -1).all()
    agree = check_decisions(gdec, fex, legal)
    fex, fflip = settle_forward(q, k, v, tau, fex, gdec, say)
    go = gpu_to_f64(g["o"])
    gl = g["lse"].cpu().numpy().astype(np.float64)
    dl = float(np.abs(gl - fex["lse"]).max())
    assert dl <= LSE_TOL, f"LSE max |delta| {dl}"
    # M = sum_k p_k |V_kc| <= max_k |V_kc| for every row (the weights sum to 1)
    vmax = np.abs(v).max(axis=2)                          # [B, Hkv, d]
    mbar = np.repeat(vmax, Hq // Hkv, axis=1)[:, :, None, :]
    err = np.abs(go - fex["o"])
    bound = 2.0 ** -6 * (mbar + np.abs(fex["o"])) + 1e-4
    worst = float((err / bound).max())
    assert worst <= 1.0, f"O vs fp64 on every row: worst ratio {worst}"
    rl2 = float(np.linalg.norm(go - fex["o"]) / np.linalg.norm(fex["o"]))
    say(f"[{label}] forward: {int(legal.sum())} tiles, agreement {agree:.6f}, {fflip} flipped; "
        f"LSE max|d| {dl:.2e}; O rel L2 vs fp64 {rl2:.2e}, worst bound ratio {worst:.3f}, "
        f"max|dO|/max(1,|O|) {v1_exact_metric(go, fex['o']):.2e}")
    # strict checks on sampled blocks (the oracle's exact magnitudes)
    sb = [(b, h, i) for (b, h, i) in sample_blocks]
    fbf = O.mala_fwd(q, k, v, tau, round_flags=O.BF16_FWD | O.LAZY_REF, force=fex["dec"], sel=sb)
    fmag = O.mala_fwd(q, k, v, tau, round_flags=O.BF16_FWD | O.ABS, force=fex["dec"], sel=sb)
    rows = np.zeros((B, Hq, N), dtype=bool)
    for (b, h, i) in sb:
        rows[b, h, 64 * i:min(N, 64 * i + 64)] = True
    ok, w1 = v1_ok(go[rows], fbf["o"][rows], fmag["o"][rows])
    assert ok, f"forward V1 worst ratio {w1}"
    r2 = v2(go[rows], fbf["o"][rows])
    assert r2 <= V2_TOL, f"forward V2 {r2}"
    ok, wx = v1_exact_ok(go[rows], fex["o"][rows], fmag["o"][rows])
    assert ok, f"forward V1 vs fp64 worst ratio {wx}"
    ok, l2s = l2_ok(go[rows], fex["o"][rows], fmag["o"][rows])
    assert ok, f"forward relative L2 vs fp64 {l2s}"
    say(f"[{label}] forward on {len(sb)} sampled blocks: V2 {r2:.2e}, V1 worst {w1:.3f}")

    # ---- backward on sampled query blocks and the heaviest key blocks ----
    sel_k, sched = heavy_key_blocks(bdec, Hkv, N, kv_per_group)
    segs = [segments_of_block(sched, b, g_, j) for (b, g_, j) in sel_k]
    say(f"[{label}] backward key blocks {[j for (_, _, j) in sel_k]} with "
        f"{segs} dK/dV segments; largest pair {max(r[3] for rr in sched.values() for r in rr)}")

    def bwd(o_, lse_, flags, force=None):
        return O.mala_bwd(q, k, v, o_, lse_, do, tau, round_flags=flags, force=force,
                          sel_q=sel_q, sel_k=sel_k)

    def settle(o_, lse_, gd):
        free = bwd(o_, lse_, O.EXACT)
        lg = free["dec"] >= 0
        assert (gd[lg] >= 0).all()
        agree_ = check_decisions(gd, free, lg)
        dis = lg & (gd != free["dec"])
        if dis.any():
            force = np.full(gd.shape, -1, dtype=np.int8)
            force[dis] = gd[dis]
            free = bwd(o_, lse_, O.EXACT, force)
        return free, lg, agree_, int(dis.sum())

    rq = np.zeros((B, Hq, N), dtype=bool)
    for (b, h, i) in sel_q:
        rq[b, h, 64 * i:min(N, 64 * i + 64)] = True
    rk = np.zeros((B, Hkv, N), dtype=bool)
    for (b, g_, j) in sel_k:
        rk[b, g_, 64 * j:min(N, 64 * j + 64)] = True
    names = (("dq", rq), ("dk", rk), ("dv", rk))
    t = time.time()
    bex, blegal, bagree, bflip = settle(fex["o"], fex["lse"], bdec)
    bmag = bwd(fex["o"], fex["lse"], O.BF16_BWD | O.ABS, bex["dec"].copy())
    bmd = bwd(fex["o"], fex["lse"], O.ABS_D, bex["dec"].copy())
    say(f"[{label}] oracle backward (end to end) {time.time() - t:.1f}s, {int(blegal.sum())} "
        f"tiles, agreement {bagree:.6f}, {bflip} flipped")
    res = {}
    for name, rows_ in names:
        x = gpu_to_f64(g[name])[rows_]
        assert np.isfinite(x).all()
        ok, rl = l2_ok(x, bex[name][rows_], bmag[name][rows_], bmd[name][rows_])
        assert ok, f"{name} relative L2 vs fp64 {rl}"
        res[name + "_l2"] = rl
        res[name + "_v1x"] = v1_exact_metric(x, bex[name][rows_])
    # the sink and hub blocks do get gradient: the comparison is not of zeros
    assert np.abs(bex["dk"][rk]).max() > 0 and np.abs(bex["dv"][rk]).max() > 0
    # backward support nested in the forward support (up to ties)
    viol = (bdec == 1) & (gdec == 0)
    if viol.any():
        assert np.all(np.abs(fex["margin"][viol]) < DELTA), "backward kept a tile forward skipped"

    # ---- the backward alone, on the oracle's exact forward outputs stored as
    #      bf16 O and fp32 LSE ----
    o_in = O.round_bf16(fex["o"])
    lse_in = fex["lse"].astype(np.float32).astype(np.float64)
    g2 = run_bwd_given(inp, o_in, lse_in, tau)
    t = time.time()
    b2, _, agree2, flip2 = settle(o_in, lse_in, g2["bdec"])
    b2bf = bwd(o_in, lse_in, O.BF16_BWD, b2["dec"].copy())
    b2mag = bwd(o_in, lse_in, O.BF16_BWD | O.ABS, b2["dec"].copy())
    say(f"[{label}] oracle backward (alone) {time.time() - t:.1f}s, agreement {agree2:.6f}, "
        f"{flip2} flipped")
    for name, rows_ in names:
        x = gpu_to_f64(g2[name])[rows_]
        assert np.isfinite(x).all()
        ok, w1 = v1_ok(x, b2bf[name][rows_], b2mag[name][rows_])
        assert ok, f"{name} V1 worst ratio {w1}"
        r2_ = v2(x, b2bf[name][rows_])
        assert r2_ <= V2_TOL, f"{name} V2 {r2_}"
        ok, wx = v1_exact_ok(x, b2[name][rows_], b2mag[name][rows_])
        assert ok, f"{name} V1 vs fp64 worst ratio {wx}"
        res[name + "_v2"] = r2_
        res[name + "_v1x_alone"] = v1_exact_metric(x, b2[name][rows_])
    say(f"[{label}] backward: " + ", ".join(f"{k_} {v_:.2e}" for k_, v_ in res.items()))
    return {"agree": agree, "bagree": bagree, "res": res, "sel_k": sel_k, "segs": segs}


def _sample_blocks(rng, B, Hq, Tr, n):
    out = {(0, 0, 0), (0, Hq - 1, Tr - 1), (0, 0, Tr // 2)}
    while len(out) < n:
        out.add((int(rng.integers(0, B)), int(rng.integers(0, Hq)), int(rng.integers(0, Tr))))
    return sorted(out)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("length", [16384, 32768])
def test_cfg3_full_forward_and_sink_hub_backward(length, say):
    """Length-sweep rows at 16K and 32K (16 query / 4 KV heads, d 128, local
    bias, tau 1): forward on every row, backward on sampled query blocks and
    on key block 0 and the two heaviest hub blocks of two KV heads."""
    w = W.cfg3(length)
    inp = W.peaked(w.spec)
    Tr = length // 64
    rng = np.random.default_rng(length)
    sel_q = [(0, h, i) for h in (0, 7, 15) for i in (0, Tr // 3, Tr - 1)]
    r = check_fullsize(inp, w.tau, sel_q, say, w.name, _sample_blocks(rng, 1, 16, Tr, 24))
    assert r["agree"] >= 0.999


@pytest.mark.timeout(1200)
def test_cfg4_full_forward_and_sink_hub_backward(say):
    """The 128K operator workload (8 query / 1 KV head, d 128, tau 1), the
    launches the benchmark times: forward on every row of every head,
    backward dQ on sampled query blocks and dK / dV on the sink key block and
    the three heaviest hub blocks, whose pairs the dK/dV pass cuts into the
    most segments."""
    w = W.cfg4()
    inp = W.peaked(w.spec)
    Tr = w.spec.seqlen // 64
    rng = np.random.default_rng(4)
    sel_q = [(0, h, i) for i in (0, 1, 700, Tr - 1) for h in (0, 3)]
    r = check_fullsize(inp, w.tau, sel_q, say, w.name, _sample_blocks(rng, 1, 8, Tr, 24),
                       kv_per_group=3)
    assert r["agree"] >= 0.999
    assert max(r["segs"]) == 8, r["segs"]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("variant", ["peaked", "diffuse"])
def test_cfg5_full_cache_all_sequences_tau_sweep(variant, say):
    """The decode workload at its full size (16 sequences, 128K cache, 32
    query / 8 KV heads, d 128, 16 splits): every sequence and head against
    the oracle for tau in {0, 0.25, 1, 4}."""
    from test_gpu_decode import compare_decode, decode_inputs
    w = W.cfg5(variant, 1.0)
    inp = decode_inputs(w.spec)
    say(f"[cfg5 {variant}] cache generated; converting to fp64")
    f64 = tuple(bits_to_f64(inp[x]) for x in ("q", "k", "v"))
    for tau in W.DECODE_TAUS:
        t = time.time()
        r = compare_decode(inp, tau, w.extra["num_splits"], label=f"cfg5-{variant}", f64=f64)
        c = r["cnt"]
        say(f"[cfg5 {variant}] tau {tau}: agreement {r['agree']:.6f}, {r['flipped']} flipped, "
            f"V2 {r['v2']:.2e}, rel L2 vs fp64 {r['l2']:.2e}, head-tiles kept "
            f"{c[1] / c[0]:.4f} ({time.time() - t:.1f}s)")
