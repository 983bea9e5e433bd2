"""The dK/dV pass's fp32 partial sums fit the workspace whatever the
decisions: the workspace holds SLOTS_PER_PAIR partial slots per pair of key
blocks, and the pairing pass gives every pair it cuts into several segments
one slot per segment. The segment rule (segments of at least Lseg =
max(512, ceil(2 K / (4 npair))) kept items, at most 8) keeps the total below
that: a pair cut into n >= 2 segments keeps more than Lseg items, so n < 2
kept / Lseg, and the kept items of all pairs add up to K. These tests check
the bound, the segment limit and the pairing (every key block in exactly one
pair) on the host model of the pairing pass, for dense, structured and random
decision maps, including maps built to reach the limits."""
import numpy as np
import pytest

from bwd_schedule import SEG_MAX, SLOTS_PER_PAIR, pairs_and_segments


def legal_mask(B, Hq, Tr, Tc, nq, nk, causal):
    off = nk - nq if causal else 0
    i = np.arange(Tr)[:, None]
    j = np.arange(Tc)[None, :]
    # causal: query block i reaches key block j iff 64 j <= 64 i + 63 + off
    ok = (64 * j <= 64 * i + 63 + off) if causal else np.ones((Tr, Tc), bool)
    return np.broadcast_to(ok, (B, Hq, Tr, Tc))


def check(bdec, heads_kv, nq, nk, causal):
    sched = pairs_and_segments(bdec, heads_kv, nq, nk, causal)
    Tc = bdec.shape[3]
    npair = Tc // 2 + 1
    for rows in sched.values():
        blocks = [j for (jA, jB, _, _) in rows for j in (jA, jB) if j >= 0]
        assert sorted(blocks) == list(range(Tc)), "every key block in exactly one pair"
        assert len(rows) <= npair
        nslot = 0
        for (_, _, kept, nseg) in rows:
            assert 1 <= nseg <= SEG_MAX
            if nseg > 1:
                nslot += nseg
        assert nslot <= SLOTS_PER_PAIR * npair, (nslot, npair)
    return sched


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("Tr,G", [(2, 1), (17, 3), (128, 8), (512, 4), (2048, 8)])
def test_every_tile_kept(Tr, G, causal):
    nq = nk = 64 * Tr
    legal = legal_mask(1, G, Tr, Tr, nq, nk, causal)
    bdec = np.where(legal, 1, -1).astype(np.int8)
    check(bdec, 1, nq, nk, causal)


@pytest.mark.parametrize("seed", range(12))
def test_random_and_structured_maps(seed):
    rng = np.random.default_rng(seed)
    Tr = int(rng.integers(1, 400))
    causal = bool(rng.integers(0, 2))
    chunk = causal and bool(rng.integers(0, 2))
    Tc = Tr + (int(rng.integers(1, 50)) if chunk else 0)
    nq, nk = 64 * Tr - int(rng.integers(0, 64)), 64 * Tc - int(rng.integers(0, 64))
    Tr, Tc = -(-nq // 64), -(-nk // 64)
    G = int(rng.choice([1, 2, 3, 4, 8]))
    Hkv = int(rng.integers(1, 3))
    legal = legal_mask(1, G * Hkv, Tr, Tc, nq, nk, causal)
    kind = seed % 4
    if kind == 0:    # independent tiles at a random density
        keep = rng.random(legal.shape) < rng.random()
    elif kind == 1:  # sinks and hubs: whole key columns kept, the rest sparse
        keep = rng.random(legal.shape) < 0.05
        hubs = rng.choice(Tc, size=max(1, Tc // int(rng.integers(2, 10))), replace=False)
        keep[..., hubs] = True
    elif kind == 2:  # just enough kept per block to be cut: many blocks slightly over Lseg
        keep = rng.random(legal.shape) < 0.5
        keep[..., ::2] = True
    else:            # diagonal band plus a sink
        i = np.arange(Tr)[:, None]
        j = np.arange(Tc)[None, :]
        band = np.abs((i + (Tc - Tr)) - j) <= int(rng.integers(0, 8))
        keep = np.broadcast_to(band, legal.shape).copy()
        keep[..., 0] = True
    bdec = np.where(legal, keep.astype(np.int8), -1).astype(np.int8)
    check(bdec, Hkv, nq, nk, causal)


def test_bound_is_tight_enough_to_matter():
    """With every tile kept on a long causal sequence the cut pairs use a
    large share of the slots, so the test above exercises the bound rather
    than a trivially small count."""
    Tr, G = 2048, 8
    nq = nk = 64 * Tr
    bdec = np.where(legal_mask(1, G, Tr, Tr, nq, nk, True), 1, -1).astype(np.int8)
    sched = check(bdec, 1, nq, nk, True)
    rows = sched[(0, 0)]
    used = sum(n for (_, _, _, n) in rows if n > 1)
    assert used > SLOTS_PER_PAIR * (Tr // 2 + 1) // 4
