"""GPU parity of split-KV decode (mala_decode, fullattn_decode) against the
CPU oracle, through the C ABI. Tolerances: tests/parity.py."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from parity import (AGREE_MIN, LSE_TOL, V2_TOL, bits_to_f64, bits_to_gpu, check_decisions,
                    gpu_to_f64, l2_ok, settle_fwd_branch, v1_ok, v2)

pytestmark = pytest.mark.gpu


def mala():
    import adaptive_softmax_attention_amd as m
    m.lib()
    return m


def decode_inputs(spec):
    """Cache K/V from the generator; the new query is row N-1 (it sees all
    N keys including its own, L = N)."""
    inp = W.peaked(spec, q_rows=[spec.seqlen - 1], want_do=False)
    inp["q"] = np.ascontiguousarray(inp["q"][:, :, 0, :])
    return inp


def run_decode(inp, tau, S, dense=False, with_stats=True):
    m = mala()
    q, k, v = bits_to_gpu(inp["q"]), bits_to_gpu(inp["k"]), bits_to_gpu(inp["v"])
    B, Hq, d = q.shape
    Nk = k.shape[2]
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    ws = torch.empty(m.mala_decode_workspace_bytes(q, k, S), dtype=torch.uint8, device="cuda")
    stats = None
    if with_stats:
        stats = m.Stats(torch.zeros(4, dtype=torch.int64, device="cuda"),
                        torch.full((B, Hq, -(-Nk // 64)), 255, dtype=torch.uint8, device="cuda"))
    if dense:
        m.fullattn_decode(q, k, v, o, lse, S, ws, stats=stats)
    else:
        m.mala_decode(q, k, v, o, lse, S, ws, tau=tau, stats=stats)
    torch.cuda.synchronize()
    dec = stats.decisions.cpu().numpy().astype(np.int8) if with_stats else None
    cnt = stats.counters.cpu().numpy() if with_stats else None
    return o, lse, dec, cnt


def compare_decode(inp, tau, S, batches=None, label=""):
    o, lse, dec, cnt = run_decode(inp, tau, S)
    print(f"[decode {label}] q{inp['q'].shape} k{inp['k'].shape} tau={tau} S={S}", flush=True)
    bsel = slice(None) if batches is None else list(batches)
    q = bits_to_f64(inp["q"][bsel])
    k = bits_to_f64(inp["k"][bsel])
    v = bits_to_f64(inp["v"][bsel])
    go = gpu_to_f64(o)[bsel]
    gl = lse.cpu().numpy().astype(np.float64)[bsel]
    gd = dec[bsel]

    def run(force, flags=O.EXACT):
        return O.mala_decode(q, k, v, S, tau, 64, round_flags=flags, force=force)

    free = run(None)
    legal = free["dec"] >= 0
    assert (gd[legal] >= 0).all() and (gd[~legal] == -1).all()
    agree = check_decisions(gd, free, legal)
    ex, flipped = settle_fwd_branch(run, gd, legal, free=free)
    bf = run(ex["dec"].copy(), O.BF16_DECODE)  # follows the settled decisions
    mag = run(ex["dec"].copy(), O.BF16_DECODE | O.ABS)
    ok, worst = v1_ok(go, bf["o"], mag["o"])
    assert ok, f"V1 worst ratio {worst}"
    r2 = v2(go, bf["o"])
    assert r2 <= V2_TOL, r2
    ok, rl2 = l2_ok(go, ex["o"], mag["o"])
    assert ok, f"relative L2 vs fp64 {rl2}"
    assert np.abs(gl - ex["lse"]).max() <= LSE_TOL
    assert np.isfinite(go).all() and np.isfinite(gl).all()
    if batches is None:
        assert cnt[0] == int((dec >= 0).sum()) and cnt[1] == int((dec == 1).sum())
    return {"agree": agree, "v2": r2, "flipped": flipped, "dec": dec, "cnt": cnt}


@pytest.mark.parametrize("Nk,Hq,Hkv,d,S", [
    (1, 4, 2, 128, 1),
    (63, 4, 4, 64, 1),
    (65, 8, 2, 128, 2),
    (1000, 8, 2, 128, 3),      # ragged last tile
    (4097, 8, 1, 128, 7),      # G = 8, uneven splits
    (2048, 4, 4, 64, 32),      # one tile per split
    (3000, 6, 2, 128, 5),      # G = 3
])
@pytest.mark.parametrize("tau", [0.0, 1.0, 4.0])
def test_decode_shapes(Nk, Hq, Hkv, d, S, tau):
    spec = W.Spec(900 + Nk, 2, Hq, Hkv, Nk, d, 3.0, 8 if Nk > 200 else 0)
    compare_decode(decode_inputs(spec), tau, S, label=f"Nk{Nk}")


def test_decode_empty_trailing_split():
    # 5 tiles in 4 splits of 2: the last split is empty and must drop out
    spec = W.Spec(77, 1, 4, 1, 5 * 64, 128, 3.0, 4)
    compare_decode(decode_inputs(spec), 1.0, 4, label="empty-split")


def test_decode_dense_identity_and_tau0():
    spec = W.Spec(78, 2, 8, 2, 3000, 128, 3.0, 16)
    inp = decode_inputs(spec)
    a = run_decode(inp, 0.0, 6)
    b = run_decode(inp, 0.0, 6, dense=True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert (a[2][a[2] >= 0] == 1).all()


@pytest.mark.parametrize("variant", ["peaked", "diffuse"])
@pytest.mark.parametrize("tau", [0.0, 0.25, 1.0, 4.0])
def test_cfg5_tau_sweep_reduced_cache(variant, tau):
    """The decode workload (16 sequences, 32 query / 8 KV heads, d 128, 16
    splits) with a 16K cache, all outputs compared."""
    w = W.cfg5(variant, tau)
    spec = w.spec
    spec = W.Spec(spec.seed, spec.batch, spec.heads_q, spec.heads_kv, 16384, spec.head_dim,
                  spec.sigma_s, 64)
    compare_decode(decode_inputs(spec), tau, w.extra["num_splits"], label=f"{variant}-16k")


@pytest.mark.parametrize("variant", ["peaked", "diffuse"])
def test_cfg5_full_cache_sampled(variant):
    """Full 128K cache, the launch the benchmark times; two of the sixteen
    sequences (all heads) recomputed by the oracle."""
    w = W.cfg5(variant, 1.0)
    r = compare_decode(decode_inputs(w.spec), 1.0, w.extra["num_splits"], batches=[0, 15],
                       label=w.name)
    print("retained head-tiles", r["cnt"][1] / r["cnt"][0], "V tiles", r["cnt"][3])
