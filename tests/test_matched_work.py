"""CPU pins of the matched-work allocation control that bench.py reports
([MALA] Sec. 3, "Normalized-Mass Allocation at Matched Work", Table 1; App. C.2).

The control's evaluation (torch, any device) is checked against the oracle:
attention restricted to a tile set is the oracle's MALA forward with those
decisions forced, and its omitted mass is 1 - exp(z_kept - z_dense) from the
oracle's two normalizers (App. C.2's definition). The selection is checked
against brute force over every subset, and the allocations against their
definition (exact totals, static where they must be)."""
import itertools
import math

import numpy as np
import pytest
import torch

import bench
import oracle as O
import workloads as W

TILE = 16


def _mala_counts(rng, R, H, Tr):
    # MALA keeps between 1 and i + 1 tiles of causal query block i
    return np.stack([[[rng.integers(1, i + 2) for i in range(Tr)] for _ in range(H)]
                     for _ in range(R)])


def test_allocations_match_mala_total_and_stay_static():
    rng = np.random.default_rng(5)
    R, H, Tr = 3, 5, 9
    n = _mala_counts(rng, R, H, Tr)
    a = bench.matched_allocations(n)
    assert (a["instance"] == n).all()
    legal = np.arange(1, Tr + 1)
    for name in ("position", "head_position"):
        x = a[name]
        assert x.shape == n.shape and x.sum() == n.sum(), name
        assert (x >= 1).all() and (x <= legal).all(), name
    hp = a["head_position"]
    # fixed across inputs up to the rounding unit, and exact per (head, block)
    assert (hp.max(0) - hp.min(0) <= 1).all()
    assert (hp.sum(0) == n.sum(0)).all()
    mean_hi = n.mean(0)
    assert (np.abs(hp - mean_hi[None]) < 1).all()
    pos = a["position"]
    assert (pos.max((0, 1)) - pos.min((0, 1)) <= 1).all()
    assert (pos.sum((0, 1)) == n.sum((0, 1))).all()
    assert (np.abs(pos - n.mean((0, 1))[None, None]) < 1).all()
    # an allocation that is already constant is returned unchanged
    c = np.broadcast_to(np.arange(1, Tr + 1), (R, H, Tr))
    for x in bench.matched_allocations(c).values():
        assert (x == c).all()


def test_top_tiles_keeps_the_heaviest_subset():
    rng = np.random.default_rng(11)
    Tr = Tc = 6
    legal = torch.ones(Tr, Tc, dtype=torch.bool).tril()
    for _ in range(20):
        mass = torch.from_numpy(rng.random((Tr, Tc)))
        alloc = torch.tensor([rng.integers(0, i + 2) for i in range(Tr)])
        keep = bench.top_tiles(mass, alloc, legal)
        assert not (keep & ~legal).any()
        for i in range(Tr):
            a = int(alloc[i])
            assert int(keep[i].sum()) == a
            got = float(mass[i][keep[i]].sum())
            best = max(sum(float(mass[i, j]) for j in sub)
                       for sub in itertools.combinations(range(i + 1), a))
            assert got == pytest.approx(best, rel=1e-12)


def _inputs(seed, R=3, H=2, N=128, d=16):
    """The benchmark's generator at a tiny size: sink, planted keys, local bias."""
    spec = W.Spec(seed, R, H, 1, N, d, 3.0, 4, local_bias=True, block_k=TILE)
    inp = W.peaked(spec, want_do=False)
    return tuple(W.bf16_bits_to_f32(inp[x]).astype(np.float64) for x in ("q", "k", "v"))


def test_policy_errors_match_the_oracle():
    """Per row omitted mass and per block output error of every policy equal
    the oracle's forward with the policy's tiles forced, against the oracle's
    dense forward (fp64 on both sides)."""
    q, k, v = _inputs(3)
    R, H, N, d = q.shape
    Tr = N // TILE
    scale = 1.0 / math.sqrt(d)
    free = O.mala_fwd(q, k, v, tau=1.0, block_q=TILE, block_k=TILE)
    dec = free["dec"]
    legal_np = np.tril(np.ones((Tr, Tr), dtype=bool))
    assert ((dec >= 0) == legal_np).all()
    keep_mala = dec == 1
    assert (~keep_mala & legal_np).any(), "the rule skipped nothing; inputs too flat"
    n = keep_mala.sum(-1)
    alloc = bench.matched_allocations(n)
    o_ref, z_ref = O.dense_fwd(q, k, v)
    legal = torch.from_numpy(legal_np)
    checked = 0
    for r in range(R):
        for h in range(H):
            qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x[r, hh]))
                          for x, hh in ((q, h), (k, 0), (v, 0)))
            p, row, blk = bench.reference_masses(qt, kt, scale, TILE)
            o = p @ vt
            assert np.allclose(o.numpy(), o_ref[r, h], rtol=1e-10, atol=1e-12)
            masks = {"mala": torch.from_numpy(keep_mala[r, h])}
            for name, a in alloc.items():
                masks[name] = bench.top_tiles(blk, torch.from_numpy(a[r, h]), legal)
            for name, keep in masks.items():
                eps, eps_blk, err = bench.policy_errors(p, o, row, vt, keep, TILE)
                force = np.full(dec.shape, -1, dtype=np.int8)
                force[r, h] = np.where(legal_np, keep.numpy().astype(np.int8), -1)
                sel = [(r, h, i) for i in range(Tr)]
                f = O.mala_fwd(q, k, v, tau=1.0, block_q=TILE, block_k=TILE, force=force, sel=sel)
                assert (f["dec"][r, h] == force[r, h]).all()
                want_eps = -np.expm1(f["lse"][r, h] - z_ref[r, h])
                assert np.allclose(eps.numpy(), want_eps, rtol=1e-8, atol=1e-14), name
                diff = (f["o"][r, h] - o_ref[r, h]).reshape(Tr, TILE, d)
                ref = o_ref[r, h].reshape(Tr, TILE, d)
                want_err = np.sqrt((diff ** 2).sum((1, 2)) / (ref ** 2).sum((1, 2)))
                assert np.allclose(err.numpy(), want_err, rtol=1e-7, atol=1e-14), name
                assert np.allclose(eps_blk.numpy(), want_eps.reshape(Tr, TILE).mean(1),
                                   rtol=1e-8, atol=1e-14)
                checked += 1
    assert checked == R * H * 4


def test_instance_control_never_omits_more_than_mala():
    """At the same tile count per query block, the heaviest tiles omit the
    least block mass; MALA's set is one of the candidates."""
    q, k, v = _inputs(9, R=2, H=3)
    R, H, N, d = q.shape
    Tr = N // TILE
    dec = O.mala_fwd(q, k, v, tau=1.0, block_q=TILE, block_k=TILE)["dec"]
    n = (dec == 1).sum(-1)
    legal = torch.ones(Tr, Tr, dtype=torch.bool).tril()
    for r in range(R):
        for h in range(H):
            qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x[r, hh]))
                          for x, hh in ((q, h), (k, 0), (v, 0)))
            p, row, blk = bench.reference_masses(qt, kt, 1.0 / math.sqrt(d), TILE)
            o = p @ vt
            _, om_mala, _ = bench.policy_errors(p, o, row, vt, torch.from_numpy(dec[r, h] == 1),
                                                TILE)
            keep = bench.top_tiles(blk, torch.from_numpy(n[r, h]), legal)
            _, om_inst, _ = bench.policy_errors(p, o, row, vt, keep, TILE)
            assert (om_inst <= om_mala + 1e-15).all()


def test_head_gain_scales_only_that_heads_queries():
    plain = W.Spec(77, 2, 4, 2, 256, 16, 3.0, 4, local_bias=True, block_k=TILE)
    mixed = W.Spec(77, 2, 4, 2, 256, 16, 3.0, 4, local_bias=True, block_k=TILE,
                   head_gain=(0.5, 2.0))
    a, b = W.peaked(plain), W.peaked(mixed)
    for x in ("k", "v", "do"):
        assert np.array_equal(a[x], b[x]), x
    qa, qb = (W.bf16_bits_to_f32(t[x]).astype(np.float64) for t, x in ((a, "q"), (b, "q")))
    gains = set()
    for bb in range(2):
        for h in range(4):
            g = W.head_gain(mixed, bb, h)
            assert 0.5 <= g <= 2.0
            gains.add(round(g, 6))
            # one bf16 rounding on each side: within 2^-8 of the scaled value
            assert np.allclose(qb[bb, h], g * qa[bb, h], rtol=2 ** -7, atol=1e-30)
    assert len(gains) == 8
