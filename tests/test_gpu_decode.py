"""GPU parity of split-KV decode (mala_decode, fullattn_decode) against the
CPU oracle, through the C ABI. Tolerances: tests/parity.py."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from parity import (AGREE_MIN, LSE_TOL, V2_TOL, bits_to_f64, bits_to_gpu, check_decisions,
                    gpu_to_f64, l2_ok, settle_fwd_branch, v1_exact_metric, v1_exact_ok, v1_ok,
                    v2)

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


def run_decode(inp, tau, S, dense=False, with_stats=True, bk=64):
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
                        torch.full((B, Hq, -(-Nk // bk)), 255, dtype=torch.uint8, device="cuda"))
    if dense:
        m.fullattn_decode(q, k, v, o, lse, S, ws, stats=stats, block_k=bk)
    else:
        m.mala_decode(q, k, v, o, lse, S, ws, tau=tau, stats=stats, block_k=bk)
    torch.cuda.synchronize()
    dec = stats.decisions.cpu().numpy().astype(np.int8) if with_stats else None
    cnt = stats.counters.cpu().numpy() if with_stats else None
    return o, lse, dec, cnt


def compare_decode(inp, tau, S, batches=None, label="", bk=64, f64=None):
    """GPU decode against the oracle on the sequences `batches` (all when
    None). f64: the (q, k, v) of those sequences already in fp64, to reuse
    one conversion of a large cache across several calls."""
    print(f"[decode {label}] q{inp['q'].shape} k{inp['k'].shape} tau={tau} S={S} block_k={bk}",
          flush=True)
    o, lse, dec, cnt = run_decode(inp, tau, S, bk=bk)
    # the kernels without instrumentation (the timed instances) give the same
    # results bitwise
    o2, lse2, _, _ = run_decode(inp, tau, S, with_stats=False, bk=bk)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    del o2, lse2
    bsel = slice(None) if batches is None else list(batches)
    if f64 is None:
        q = bits_to_f64(inp["q"][bsel])
        k = bits_to_f64(inp["k"][bsel])
        v = bits_to_f64(inp["v"][bsel])
    else:
        q, k, v = f64
    go = gpu_to_f64(o)[bsel]
    gl = lse.cpu().numpy().astype(np.float64)[bsel]
    gd = dec[bsel]

    def run(force, flags=O.EXACT):
        return O.mala_decode(q, k, v, S, tau, bk, round_flags=flags, force=force)

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
    ok, worst = v1_exact_ok(go, ex["o"], mag["o"])
    assert ok, f"V1 vs fp64 worst ratio {worst}"
    v1x = v1_exact_metric(go, ex["o"])
    print(f"  decode V2 {r2:.2e}  max|dO|/max(1,|O|) vs fp64 {v1x:.2e}  rel L2 vs fp64 "
          f"{rl2:.2e}", flush=True)
    assert np.abs(gl - ex["lse"]).max() <= LSE_TOL
    assert np.isfinite(go).all() and np.isfinite(gl).all()
    if batches is None:
        assert cnt[0] == int((dec >= 0).sum()) and cnt[1] == int((dec == 1).sum())
        assert cnt[2] == bk * cnt[1]
    return {"agree": agree, "v2": r2, "v1x": v1x, "l2": rl2, "flipped": flipped, "dec": dec,
            "cnt": cnt}


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


# ---- paged cache of variable-length sequences (mala_decode_paged) ----

def paged_inputs(seed, lens, Hq, Hkv, d, spare=5):
    """Caches of len(lens) sequences from the generator (sequence b keeps its
    first lens[b] keys; its query is its row lens[b] - 1), stored in 64-key
    pages at shuffled page indices, with spare pages of noise."""
    B, max_len = len(lens), max(lens)
    inp = W.peaked(W.Spec(seed, B, Hq, Hkv, max_len, d, 3.0, 8), want_do=False)
    q = np.stack([inp["q"][b, :, lens[b] - 1] for b in range(B)])
    tiles = [-(-n // 64) for n in lens]
    P = sum(tiles) + spare
    rng = np.random.default_rng(seed)
    order = rng.permutation(P)
    noise = W.f32_to_bf16_bits(rng.standard_normal((P, Hkv, 64, d)).astype(np.float32))
    kp, vp = noise.copy(), noise.copy()
    table = np.zeros((B, -(-max_len // 64)), dtype=np.int32)
    t = 0
    for b in range(B):
        for j in range(tiles[b]):
            pg = int(order[t])
            t += 1
            table[b, j] = pg
            rows = slice(64 * j, min(64 * j + 64, lens[b]))
            n = rows.stop - rows.start
            kp[pg, :, :n] = inp["k"][b, :, rows]
            vp[pg, :, :n] = inp["v"][b, :, rows]
    return {"q": q, "k": inp["k"], "v": inp["v"], "kp": kp, "vp": vp, "table": table,
            "lens": np.array(lens, dtype=np.int32), "max_len": max_len}


def run_decode_paged(pin, tau, S, dense=False, lens=None, bk=64):
    m = mala()
    q = bits_to_gpu(pin["q"])
    kp, vp = bits_to_gpu(pin["kp"]), bits_to_gpu(pin["vp"])
    table = torch.from_numpy(pin["table"]).cuda()
    lens_g = torch.from_numpy(pin["lens"] if lens is None else lens).cuda()
    B, Hq, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    ws = torch.empty(m.mala_decode_paged_workspace_bytes(q, pin["max_len"], kp.shape[1], S),
                     dtype=torch.uint8, device="cuda")
    st = m.Stats(torch.zeros(4, dtype=torch.int64, device="cuda"),
                 torch.full((B, Hq, -(-pin["max_len"] // bk)), 255, dtype=torch.uint8,
                            device="cuda"))
    if dense:
        m.fullattn_decode_paged(q, kp, vp, table, lens_g, pin["max_len"], o, lse, S, ws, stats=st,
                                block_k=bk)
    else:
        m.mala_decode_paged(q, kp, vp, table, lens_g, pin["max_len"], o, lse, S, ws, tau=tau,
                            stats=st, block_k=bk)
    torch.cuda.synchronize()
    return o, lse, st.decisions.cpu().numpy().astype(np.int8), st.counters.cpu().numpy()


def compare_decode_paged(pin, lens, tau, S, bk=64):
    """Paged decode of the sequences `lens` against the oracle's decode of
    each sequence's own cache (its own L = cache length), with the decision,
    V1/V2 and LSE checks of compare_decode; tiles past a sequence are never
    tested, and the counters match the bitmaps."""
    o, lse, dec, cnt = run_decode_paged(pin, tau, S, bk=bk)
    go, gl = gpu_to_f64(o), lse.cpu().numpy().astype(np.float64)
    assert np.isfinite(go).all() and np.isfinite(gl).all()
    legal_total = kept_total = 0
    for b, n in enumerate(lens):
        q = bits_to_f64(pin["q"][b:b + 1])
        k = bits_to_f64(pin["k"][b:b + 1, :, :n])
        v = bits_to_f64(pin["v"][b:b + 1, :, :n])
        nt = -(-n // bk)
        gd = dec[b:b + 1, :, :nt]
        assert (dec[b, :, nt:] == -1).all()  # tiles past the sequence are never tested

        def run(force, flags=O.EXACT):
            return O.mala_decode(q, k, v, S, tau, bk, round_flags=flags, force=force)

        free = run(None)
        legal = free["dec"] >= 0
        check_decisions(gd, free, legal)
        ex, _ = settle_fwd_branch(run, gd, legal, free=free)
        bf = run(ex["dec"].copy(), O.BF16_DECODE)
        mag = run(ex["dec"].copy(), O.BF16_DECODE | O.ABS)
        ok, worst = v1_ok(go[b:b + 1], bf["o"], mag["o"])
        assert ok, f"sequence {b}: V1 worst ratio {worst}"
        assert v2(go[b:b + 1], bf["o"]) <= V2_TOL
        assert np.abs(gl[b:b + 1] - ex["lse"]).max() <= LSE_TOL
        legal_total += int(legal.sum())
        kept_total += int((gd == 1).sum())
    assert cnt[0] == legal_total and cnt[1] == kept_total


@pytest.mark.parametrize("tau,S", [(1.0, 3), (0.0, 2), (4.0, 1)])
def test_decode_paged_varlen(tau, S):
    """Each sequence against the oracle's decode of its own cache (its own
    L = cache length), with the same decision, V1/V2 and LSE checks."""
    lens = [1, 63, 64, 700, 1000]
    compare_decode_paged(paged_inputs(41, lens, 8, 2, 128), lens, tau, S)


@pytest.mark.parametrize("bk", [64, 128])
def test_decode_paged_equals_contiguous(bk):
    """Equal lengths and pages in order: the paged path computes exactly what
    mala_decode computes on the contiguous caches (bitwise), MALA and dense,
    for 64- and 128-key decision tiles."""
    m = mala()
    spec = W.Spec(43, 3, 8, 2, 777, 128, 3.0, 8)
    inp = decode_inputs(spec)
    B, Hkv, N, d = inp["k"].shape
    T = -(-N // 64)
    kp = np.zeros((B * T, Hkv, 64, d), dtype=np.uint16)
    vp = np.zeros_like(kp)
    table = np.zeros((B, T), dtype=np.int32)
    for b in range(B):
        for j in range(T):
            rows = slice(64 * j, min(64 * j + 64, N))
            kp[b * T + j, :, :rows.stop - rows.start] = inp["k"][b, :, rows]
            vp[b * T + j, :, :rows.stop - rows.start] = inp["v"][b, :, rows]
            table[b, j] = b * T + j
    pin = {"q": inp["q"], "kp": kp, "vp": vp, "table": table,
           "lens": np.full(B, N, dtype=np.int32), "max_len": N}
    for dense in (False, True):
        o1, l1, d1, _ = run_decode(inp, 1.0, 4, dense=dense, bk=bk)
        o2, l2, d2, _ = run_decode_paged(pin, 1.0, 4, dense=dense, bk=bk)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        assert np.array_equal(d1, d2)


def test_decode_paged_bad_entries_give_nan_for_that_sequence():
    """A cache length or page index out of range is never read from: that
    sequence's outputs become NaN and the others keep their values."""
    lens = [100, 300, 200]
    pin = paged_inputs(47, lens, 4, 2, 128)
    o_ref, l_ref, _, _ = run_decode_paged(pin, 1.0, 2)
    bad_lens = np.array([100, 300 + 10 ** 6, 200], dtype=np.int32)  # sequence 1: too long
    o, l, _, _ = run_decode_paged(pin, 1.0, 2, lens=bad_lens)
    assert torch.isnan(o[1].float()).all() and torch.isnan(l[1]).all()
    assert torch.equal(o[0], o_ref[0]) and torch.equal(o[2], o_ref[2])
    pin2 = dict(pin, table=pin["table"].copy())
    pin2["table"][2, 1] = 10 ** 6  # sequence 2: page index past the pages
    o, l, _, _ = run_decode_paged(pin2, 1.0, 2)
    assert torch.isnan(o[2].float()).all() and torch.isnan(l[2]).all()
    assert torch.equal(o[0], o_ref[0]) and torch.equal(o[1], o_ref[1])


@pytest.mark.parametrize("Nk,Hq,Hkv,d,S", [
    (1000, 8, 2, 128, 3),      # ragged last 128-key tile (its upper half empty)
    (4097, 8, 1, 128, 7),      # one key in the last tile
    (3000, 6, 2, 64, 5),       # G = 3
    (129, 4, 4, 128, 2),       # two decision tiles, one split each
])
@pytest.mark.parametrize("tau", [0.0, 1.0, 4.0])
def test_decode_decision_tile_128(Nk, Hq, Hkv, d, S, tau):
    """1 x 128 decision tiles (split boundaries on 128 keys): against the
    oracle's decode with the same tile."""
    spec = W.Spec(960 + Nk, 2, Hq, Hkv, Nk, d, 3.0, 8 if Nk > 200 else 0)
    compare_decode(decode_inputs(spec), tau, S, label=f"Nk{Nk}-bk128", bk=128)


def test_decode_tile_128_dense_identity():
    inp = decode_inputs(W.Spec(979, 2, 8, 2, 3000, 128, 3.0, 16))
    a = run_decode(inp, 0.0, 6, bk=128)
    b = run_decode(inp, 0.0, 6, dense=True, bk=128)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert (a[2][a[2] >= 0] == 1).all()
