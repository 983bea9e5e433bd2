"""Pins for the CPU oracle: it is checked against things other than itself.

* the review's worked merge example (golden fixture) and the merge identity;
* dense attention against torch's fp64 CPU attention and autograd, and
  finite differences;
* brute force on tiny inputs (tests/twin.py: Eq. 1 and Eq. 2 written with
  explicit sums and ratios, the backward as a masked gradient formula);
* closed-form hand cases with Bq = Bk = 1 (the per-key rule), including the
  visible-key count L_q and the descending traversal;
* tau = 0 reproduces dense attention (paper Sec. 2.3), tau = +inf keeps only
  each block's first legal tiles and the backward skips everything;
* forward output = softmax restricted to the retained tiles (Sec. 2.2);
* backward = autograd of that restricted softmax when the backward keeps the
  forward's tiles;
* Proposition 1 and Eqs. (6)-(10) (App. B) and backward nesting (Sec. 2.2);
* decode: one split equals the forward with one query; tau = 0 equals dense
  for any split count (Sec. 2.4).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from twin import twin_bwd, twin_decode, twin_fwd

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _bf(x):
    return W.bf16_bits_to_f32(x).astype(np.float64)


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ---------------------------------------------------------------- merge ----

def _val(x):
    if isinstance(x, str):
        return math.log(float(x[2:]))
    return float(x)


def test_merge_review_worked_example():
    cases = json.load(open(os.path.join(GOLD, "review_merge_example.json")))["cases"]
    for case in cases:
        m = [_val(b["summary"][0]) for b in case["blocks"]]
        l = [b["summary"][1] for b in case["blocks"]]
        u = [[b["summary"][2]] for b in case["blocks"]]
        o, _ = O.merge(m, l, u)
        assert abs(o[0] - case["merged_output"]) < 1e-14
        # the summaries themselves follow from the scores and values
        for b in case["blocks"]:
            s = np.array([_val(x) for x in b["scores"]])
            vv = np.array(b["values"])
            mm = s.max()
            assert abs(mm - _val(b["summary"][0])) < 1e-15
            assert abs(np.exp(s - mm).sum() - b["summary"][1]) < 1e-14
            assert abs((np.exp(s - mm) * vv).sum() - b["summary"][2]) < 1e-14
        if "direct_weights" in case:
            s = np.concatenate([[_val(x) for x in b["scores"]] for b in case["blocks"]])
            w = np.exp(s) / np.exp(s).sum()
            assert np.allclose(w, case["direct_weights"], atol=1e-15)


def test_merge_identity_random_splits():
    rng = np.random.default_rng(7)
    for _ in range(20):
        n, d = int(rng.integers(2, 200)), int(rng.integers(1, 9))
        s = rng.standard_normal(n) * 5
        v = rng.standard_normal((n, d))
        cuts = np.sort(rng.choice(np.arange(1, n), size=min(n - 1, int(rng.integers(1, 6))), replace=False))
        parts = np.split(np.arange(n), cuts)
        m = [s[p].max() for p in parts]
        l = [np.exp(s[p] - s[p].max()).sum() for p in parts]
        u = [(np.exp(s[p] - s[p].max())[:, None] * v[p]).sum(0) for p in parts]
        o, z = O.merge(m, l, u)
        w = np.exp(s - s.max())
        assert np.allclose(o, (w[:, None] * v).sum(0) / w.sum(), rtol=1e-12, atol=1e-12)
        assert abs(z - (s.max() + np.log(w.sum()))) < 1e-12


def test_merge_skips_empty_summaries():
    o, z = O.merge([0.0, -np.inf], [2.0, 0.0], [[2.0], [0.0]])
    assert o[0] == 1.0 and abs(z - np.log(2.0)) < 1e-15


# ---------------------------------------------------------------- dense ----

def _torch_ref(q, k, v, causal, scale):
    G = q.shape[1] // k.shape[1]
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    ke = tk.repeat_interleave(G, dim=1)
    ve = tv.repeat_interleave(G, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(tq, ke, ve, is_causal=causal, scale=scale)
    return tq, tk, tv, o


@pytest.mark.parametrize("causal,Hq,Hkv,N,d", [(True, 2, 2, 37, 8), (True, 4, 2, 50, 16),
                                                (False, 3, 1, 29, 8)])
def test_dense_matches_torch(causal, Hq, Hkv, N, d):
    q, k, v, do = (_rand(s, i) for i, s in enumerate([(2, Hq, N, d), (2, Hkv, N, d),
                                                        (2, Hkv, N, d), (2, Hq, N, d)]))
    scale = 1 / math.sqrt(d)
    o, lse = O.dense_fwd(q, k, v, causal)
    tq, tk, tv, to = _torch_ref(q, k, v, causal, scale)
    assert np.allclose(o, to.detach().numpy(), rtol=1e-12, atol=1e-12)
    # lse against an explicit logsumexp
    G = Hq // Hkv
    s = scale * np.einsum("bhqd,bhkd->bhqk", q, np.repeat(k, G, axis=1))
    if causal:
        s = np.where(np.tril(np.ones((N, N), bool)), s, -np.inf)
    ref_lse = np.log(np.exp(s - s.max(-1, keepdims=True)).sum(-1)) + s.max(-1)
    assert np.allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)
    to.backward(torch.tensor(do))
    dq, dk, dv = O.dense_bwd(q, k, v, do, causal)
    assert np.allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-11)
    assert np.allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-11)
    assert np.allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-11)


def test_dense_bwd_finite_differences():
    q, k, v, do = (_rand(s, 10 + i) for i, s in enumerate([(1, 2, 6, 3), (1, 1, 6, 3),
                                                             (1, 1, 6, 3), (1, 2, 6, 3)]))
    dq, dk, dv = O.dense_bwd(q, k, v, do, True)
    eps = 1e-6

    def loss(q_, k_, v_):
        return (O.dense_fwd(q_, k_, v_, True)[0] * do).sum()

    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in [(0, 0, 1, 0), (0, 0, 5, 2), (0, 0, 3, 1)]:
            if name == "q":
                idx = (0, 1) + idx[2:]
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = {"q": q, "k": k, "v": v}
            args_p[name], args_m[name] = xp, xm
            fd = (loss(**{a + "_": b for a, b in args_p.items()}) -
                  loss(**{a + "_": b for a, b in args_m.items()})) / (2 * eps)
            assert abs(fd - g[idx]) < 1e-7 * max(1, abs(fd))


# ------------------------------------------------------- brute-force twin --

def _near_zero(m):
    """Margins within rounding of zero but not exactly zero. (An exact zero
    is a structural tie, e.g. row 0 with tau = 1 in the backward where
    P = 1 = tau/L; both formulations then retain, since skipping is strict.)"""
    m = np.nan_to_num(m, nan=1.0)
    return (np.abs(m) < 1e-9) & (m != 0.0)


TINY = [
    # (causal, Hq, Hkv, N, d, bq, bk, tau)
    (True, 1, 1, 13, 4, 1, 1, 1.0),
    (True, 2, 1, 16, 4, 2, 2, 1.0),
    (True, 2, 2, 15, 4, 4, 2, 0.5),
    (True, 2, 1, 14, 4, 2, 4, 2.0),
    (True, 1, 1, 16, 4, 4, 4, 4.0),
    (True, 3, 3, 11, 4, 3, 2, 0.25),
    (False, 2, 1, 12, 4, 4, 4, 1.0),
    (False, 1, 1, 10, 4, 1, 3, 1.0),
]


def _tiny_inputs(N, Hq, Hkv, d, seed):
    # a peaked but overflow-free score distribution: a sink and a few hubs
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, Hq, N, d)) * 1.5
    k = rng.standard_normal((1, Hkv, N, d)) * 1.5
    k[:, :, 0] += 2.0 * q.mean(axis=(1, 2))[:, None]
    hubs = rng.choice(np.arange(1, N), size=2, replace=False)
    k[:, :, hubs] *= 2.5
    v = rng.standard_normal((1, Hkv, N, d))
    do = rng.standard_normal((1, Hq, N, d))
    return q, k, v, do


@pytest.mark.parametrize("case", TINY)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_oracle_matches_bruteforce_twin(case, seed):
    causal, Hq, Hkv, N, d, bq, bk, tau = case
    q, k, v, do = _tiny_inputs(N, Hq, Hkv, d, seed)
    r = O.mala_fwd(q, k, v, tau, causal, bq, bk)
    to, tl, tdec, _ = twin_fwd(q, k, v, tau, causal, bq, bk)
    # a tile whose margin is within rounding of zero could legitimately differ
    assert not _near_zero(r["margin"]).any()
    assert np.array_equal(r["dec"], tdec)
    assert np.allclose(r["o"], to, rtol=1e-12, atol=1e-12)
    assert np.allclose(r["lse"], tl, rtol=1e-12, atol=1e-12)
    b = O.mala_bwd(q, k, v, r["o"], r["lse"], do, tau, causal, bq, bk)
    tq, tk, tv, tbd = twin_bwd(q, k, v, r["o"], r["lse"], do, tau, causal, bq, bk)
    assert not _near_zero(b["margin"]).any()
    assert np.array_equal(b["dec"], tbd)
    for x, y in ((b["dq"], tq), (b["dk"], tk), (b["dv"], tv)):
        assert np.allclose(x, y, rtol=1e-11, atol=1e-12)


def test_twin_cases_exercise_skipping():
    # the tiny cases must actually skip tiles in both passes, otherwise the
    # comparison above would not test the rule
    fs = bs = 0
    for case in TINY:
        causal, Hq, Hkv, N, d, bq, bk, tau = case
        for seed in range(3):
            q, k, v, do = _tiny_inputs(N, Hq, Hkv, d, seed)
            r = O.mala_fwd(q, k, v, tau, causal, bq, bk)
            b = O.mala_bwd(q, k, v, r["o"], r["lse"], do, tau, causal, bq, bk)
            fs += int((r["dec"] == 0).sum())
            bs += int((b["dec"] == 0).sum())
    assert fs > 20 and bs > 40


@pytest.mark.parametrize("S", [1, 2, 3, 7])
def test_decode_matches_bruteforce_twin(S):
    rng = np.random.default_rng(S)
    B, Hq, Hkv, N, d, bk = 2, 4, 2, 37, 4, 4
    k = rng.standard_normal((B, Hkv, N, d)) * 1.5
    v = rng.standard_normal((B, Hkv, N, d))
    q = rng.standard_normal((B, Hq, d)) * 1.5
    k[:, :, [3, 20]] *= 2.5
    for tau in (0.25, 1.0, 4.0):
        r = O.mala_decode(q, k, v, S, tau, bk)
        to, tl, tdec = twin_decode(q, k, v, tau, S, bk)
        assert not _near_zero(r["margin"]).any()
        assert np.array_equal(r["dec"], tdec)
        assert np.allclose(r["o"], to, rtol=1e-12, atol=1e-12)
        assert np.allclose(r["lse"], tl, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------ closed-form cases --

def _one_query_case(scores, values, tau):
    """Keys 0..n-1 with the given scores for query n-1 (causal, d = 1,
    scale = 1, Bq = Bk = 1). Query rows 0..n-2 have q = 0."""
    n = len(scores)
    q = np.zeros((1, 1, n, 1))
    q[0, 0, n - 1, 0] = 1.0
    k = np.array(scores, dtype=np.float64).reshape(1, 1, n, 1)
    v = np.array(values, dtype=np.float64).reshape(1, 1, n, 1)
    r = O.mala_fwd(q, k, v, tau, True, 1, 1, scale=1.0)
    return r["o"][0, 0, n - 1, 0], r["lse"][0, 0, n - 1], r["dec"][0, 0, n - 1]


def test_per_key_rule_hand_case_visible_count_and_order():
    # query at position 2 sees L = 3 keys; visited 2, 1, 0 (Sec. 2.2).
    # key 2 is first (retained); key 1: e^b / e^0 = 1/3 + 0.01/3 >= 1/3 -> kept;
    # key 0: 0.4 / (1 + e^b) < 1/3 -> skipped.
    b = math.log(1 / 3 + 0.01 / 3)
    a = math.log(0.4)
    o, z, dec = _one_query_case([a, b, 0.0], [10.0, 20.0, 30.0], 1.0)
    assert list(dec) == [0, 1, 1]
    assert abs(o - (30.0 + 20.0 * math.exp(b)) / (1.0 + math.exp(b))) < 1e-12
    assert abs(z - math.log(1.0 + math.exp(b))) < 1e-12


def test_per_key_rule_review_scores_threshold_sides():
    # review scores (0, 0, ln 2), values (0, 2, 4): at key 0 the ratio is
    # exactly 1/3 = tau/L for tau = 1; just below tau it is kept (the dense
    # result 2.5 of the review), just above it is dropped ((2 + 8)/3).
    s = [0.0, 0.0, math.log(2.0)]
    o, _, dec = _one_query_case(s, [0.0, 2.0, 4.0], 0.999)
    assert list(dec) == [1, 1, 1] and abs(o - 2.5) < 1e-12
    o, _, dec = _one_query_case(s, [0.0, 2.0, 4.0], 1.001)
    assert list(dec) == [0, 1, 1] and abs(o - 10.0 / 3.0) < 1e-12


def test_exact_tie_retains():
    # query 1 sees L = 2 keys with equal scores 0; tau = 2 makes the ratio
    # e^0 / e^0 = 1 equal to tau / L exactly (margin 0 - log 1 - log 1 = 0).
    # Skipping needs a strict "<" (Eqs. 2-3), so key 0 is kept: O = mean.
    o, z, dec = _one_query_case([0.0, 0.0], [2.0, 6.0], 2.0)
    assert list(dec) == [1, 1] and o == 4.0 and abs(z - math.log(2.0)) < 1e-15


def test_first_legal_tile_always_retained_and_not_forced_in_backward():
    # tau huge: every forward row keeps exactly its first tile (the diagonal)
    q, k, v, do = _tiny_inputs(12, 1, 1, 4, 5)
    r = O.mala_fwd(q, k, v, 1e30, True, 4, 4)
    for i in range(3):
        assert r["dec"][0, 0, i, i] == 1
        assert (r["dec"][0, 0, i, :i] == 0).all()
    b = O.mala_bwd(q, k, v, r["o"], r["lse"], do, 1e30, True, 4, 4)
    assert (b["dec"][b["dec"] >= 0] == 0).all()


# ------------------------------------------------------- special cases ----

def _gen_small(N=300, Hq=4, Hkv=2, d=32, planted=6, seed=11, sigma=3.0, local=False):
    spec = W.Spec(seed, 1, Hq, Hkv, N, d, sigma, planted, local_bias=local, block_k=16)
    inp = W.peaked(spec)
    return _bf(inp["q"]), _bf(inp["k"]), _bf(inp["v"]), _bf(inp["do"])


def test_tau_zero_is_dense():
    q, k, v, do = _gen_small()
    r = O.mala_fwd(q, k, v, 0.0, True, 32, 16)
    od, ld = O.dense_fwd(q, k, v, True)
    assert (r["dec"][r["dec"] >= 0] == 1).all()
    assert np.allclose(r["o"], od, rtol=1e-11, atol=1e-11)
    assert np.allclose(r["lse"], ld, rtol=1e-12, atol=1e-11)
    b = O.mala_bwd(q, k, v, r["o"], r["lse"], do, 0.0, True, 32, 16)
    dq, dk, dv = O.dense_bwd(q, k, v, do, True)
    assert (b["dec"][b["dec"] >= 0] == 1).all()
    for x, y in ((b["dq"], dq), (b["dk"], dk), (b["dv"], dv)):
        assert np.allclose(x, y, rtol=1e-9, atol=1e-9)


def test_tau_inf_keeps_first_tiles_only():
    q, k, v, do = _gen_small(N=130, Hq=2, Hkv=1)
    bq, bk = 32, 16
    r = O.mala_fwd(q, k, v, np.inf, True, bq, bk)
    # expected mask: visiting blocks last-to-first, a tile is retained iff
    # some row of the query block sees its first legal key there
    N = q.shape[2]
    mask = np.zeros((N, N), dtype=bool)
    for i in range(-(-N // bq)):
        rows = np.arange(i * bq, min(N, (i + 1) * bq))
        seen = np.zeros(len(rows), dtype=bool)
        for j in range((rows[-1]) // bk, -1, -1):
            cols = np.arange(j * bk, min(N, (j + 1) * bk))
            has = (cols[None, :] <= rows[:, None]).any(axis=1)
            if (has & ~seen).any():
                mask[np.ix_(rows, cols)] = True
            seen |= has
    mask &= np.tril(np.ones((N, N), bool))
    s = np.einsum("bhqd,bhkd->bhqk", q, np.repeat(k, 2, axis=1)) / math.sqrt(q.shape[-1])
    s = np.where(mask, s, -np.inf)
    w = np.exp(s - s.max(-1, keepdims=True))
    ref = np.einsum("bhqk,bhkd->bhqd", w / w.sum(-1, keepdims=True), np.repeat(v, 2, axis=1))
    assert np.allclose(r["o"], ref, rtol=1e-11, atol=1e-11)
    b = O.mala_bwd(q, k, v, r["o"], r["lse"], do, np.inf, True, bq, bk)
    assert (b["dec"][b["dec"] >= 0] == 0).all()
    assert not b["dq"].any() and not b["dk"].any() and not b["dv"].any()


def _tile_mask(dec, N, bq, bk, causal=True):
    B, H, Tr, Tc = dec.shape
    m = np.repeat(np.repeat(dec == 1, bq, axis=2), bk, axis=3)[:, :, :N, :N]
    if causal:
        m &= np.tril(np.ones((N, N), bool))
    return m


@pytest.mark.parametrize("tau", [0.25, 1.0, 4.0, 64.0])
def test_forward_is_softmax_over_retained_tiles(tau):
    q, k, v, do = _gen_small(N=400, Hq=4, Hkv=1, d=32, planted=12, seed=3)
    bq, bk = 32, 32
    r = O.mala_fwd(q, k, v, tau, True, bq, bk)
    mask = _tile_mask(r["dec"], q.shape[2], bq, bk)
    add = torch.tensor(np.where(mask, 0.0, -np.inf))
    tq, tk, tv = (torch.tensor(x) for x in (q, k, v))
    ke, ve = tk.repeat_interleave(4, dim=1), tv.repeat_interleave(4, dim=1)
    s = (tq @ ke.transpose(-1, -2)) / math.sqrt(q.shape[-1]) + add
    ref = torch.softmax(s, -1) @ ve
    assert np.allclose(r["o"], ref.numpy(), rtol=1e-11, atol=1e-11)
    assert np.allclose(r["lse"], torch.logsumexp(s, -1).numpy(), rtol=1e-12, atol=1e-11)


@pytest.mark.parametrize("tau", [1.0, 4.0])
def test_backward_with_forward_support_is_autograd_of_restricted_softmax(tau):
    q, k, v, do = _gen_small(N=260, Hq=2, Hkv=1, d=16, planted=8, seed=4)
    bq, bk = 32, 32
    r = O.mala_fwd(q, k, v, tau, True, bq, bk)
    # backward forced onto the forward's tiles: then it is the exact gradient
    b = O.mala_bwd(q, k, v, r["o"], r["lse"], do, tau, True, bq, bk, force=r["dec"])
    mask = _tile_mask(r["dec"], q.shape[2], bq, bk)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    ke, ve = tk.repeat_interleave(2, dim=1), tv.repeat_interleave(2, dim=1)
    s = (tq @ ke.transpose(-1, -2)) / math.sqrt(q.shape[-1]) + torch.tensor(np.where(mask, 0.0, -np.inf))
    o = torch.softmax(s, -1) @ ve
    o.backward(torch.tensor(do))
    for x, y in ((b["dq"], tq.grad), (b["dk"], tk.grad), (b["dv"], tv.grad)):
        assert np.allclose(x, y.numpy(), rtol=1e-9, atol=1e-10)


@pytest.mark.parametrize("tau", [0.25, 1.0, 4.0, 32.0])
def test_proposition1_bounds_and_nesting(tau):
    q, k, v, do = _gen_small(N=512, Hq=4, Hkv=2, d=32, planted=16, seed=8)
    bq, bk = 32, 32
    N, d = q.shape[2], q.shape[3]
    r = O.mala_fwd(q, k, v, tau, True, bq, bk)
    od, ld = O.dense_fwd(q, k, v, True)
    mask = _tile_mask(r["dec"], N, bq, bk)
    s = np.einsum("bhqd,bhkd->bhqk", q, np.repeat(k, 2, axis=1)) / math.sqrt(d)
    legal = np.tril(np.ones((N, N), bool))
    s = np.where(legal, s, -np.inf)
    # Eq. (6): omitted dense mass eps_q <= tau / (1 + tau)
    eps = 1.0 - np.exp(r["lse"] - ld)  # the paper's omitted-mass formula (App. C.2)
    Zr = np.where(mask, np.exp(s - ld[..., None]), 0.0).sum(-1)
    assert np.allclose(eps, 1.0 - Zr, atol=1e-12)
    assert (eps <= tau / (1 + tau) + 1e-12).all()
    # Eq. (7): every omitted key has exp(s)/Z_R < tau / L_q
    L = np.arange(1, N + 1)[None, None, :, None]
    omitted = legal & ~mask
    ratio = np.exp(s - r["lse"][..., None])
    assert (ratio[np.broadcast_to(omitted, ratio.shape)] <
            np.broadcast_to(tau / L, ratio.shape)[np.broadcast_to(omitted, ratio.shape)]).all()
    # Eq. (9): ||p - p~||_1 = 2 eps
    p = np.exp(s - ld[..., None])
    pt = np.where(mask, np.exp(s - r["lse"][..., None]), 0.0)
    assert np.allclose(np.abs(p - pt).sum(-1), 2 * eps, atol=1e-12)
    # Eq. (10): ||o - o~|| <= 2 tau/(1+tau) Vmax
    vmax = np.linalg.norm(v, axis=-1).max()
    assert (np.linalg.norm(od - r["o"], axis=-1) <= 2 * tau / (1 + tau) * vmax + 1e-12).all()
    # nesting (Sec. 2.2): backward-retained tiles are forward-retained tiles
    b = O.mala_bwd(q, k, v, r["o"], r["lse"], do, tau, True, bq, bk)
    assert not ((b["dec"] == 1) & (r["dec"] != 1)).any()
    assert ((r["dec"] == 0).sum() > 0) or tau <= 0.25  # skipping does happen


def test_decode_one_split_equals_forward_single_query():
    rng = np.random.default_rng(3)
    B, Hq, Hkv, N, d = 2, 4, 2, 300, 16
    k = rng.standard_normal((B, Hkv, N, d)) * 2
    v = rng.standard_normal((B, Hkv, N, d))
    q = rng.standard_normal((B, Hq, d)) * 2
    k[:, :, 17] *= 3
    for tau in (0.5, 1.0, 4.0):
        r = O.mala_decode(q, k, v, 1, tau, 32)
        f = O.mala_fwd(q[:, :, None, :], k, v, tau, False, 1, 32)
        assert np.array_equal(r["dec"], f["dec"][:, :, 0, :])
        assert np.allclose(r["o"], f["o"][:, :, 0], rtol=1e-13, atol=1e-13)
        assert np.allclose(r["lse"], f["lse"][:, :, 0], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("S", [1, 3, 8, 20])
def test_decode_tau_zero_is_dense_for_any_split(S):
    rng = np.random.default_rng(S)
    B, Hq, Hkv, N, d = 2, 4, 1, 333, 8
    k = rng.standard_normal((B, Hkv, N, d)) * 2
    v = rng.standard_normal((B, Hkv, N, d))
    q = rng.standard_normal((B, Hq, d)) * 2
    r = O.mala_decode(q, k, v, S, 0.0, 32)
    od, ld = O.dense_fwd(q[:, :, None, :], k, v, False)
    assert np.allclose(r["o"], od[:, :, 0], rtol=1e-12, atol=1e-12)
    assert np.allclose(r["lse"], ld[:, :, 0], rtol=1e-13, atol=1e-12)


# ------------------------------------------------------------- rounding ----

def test_round_bf16_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(10000) * 10.0 ** rng.integers(-6, 6, 10000),
                        [1 + 2 ** -8, 1 + 3 * 2 ** -8, -1 - 2 ** -8, 0.0, 1e-40]])
    ref = torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_bf16(x), ref)


def test_bf16_operand_mode_is_close_to_exact():
    q, k, v, do = _gen_small(N=200, Hq=2, Hkv=2, d=32, planted=4, seed=2)
    e = O.mala_fwd(q, k, v, 1.0, True, 32, 32)
    r = O.mala_fwd(q, k, v, 1.0, True, 32, 32, round_flags=O.BF16_FWD, force=e["dec"])
    # P~ rounded to bf16 (rel. 2^-9) and O rounded: error well under 1e-2
    assert np.abs(r["o"] - e["o"]).max() < 2e-2
    assert np.abs(r["o"] - e["o"]).max() > 0
    assert np.abs(r["lse"] - e["lse"]).max() < 1e-5


def test_lazy_reference_changes_where_p_is_rounded_not_the_result():
    """The forward model's lazy reference maximum (the kernel's: it moves only
    on jumps of more than 8 log2 units) leaves the exact result unchanged: the
    online softmax is invariant to its reference (Sec. 2.2, m + log l), so
    without rounding O, LSE and every decision match the plain oracle. With
    bf16 P~ it rounds at other points than the plain model (P~ up to 2^8), and
    both stay within bf16 error of exact."""
    q, k, v, do = _gen_small(N=300, Hq=2, Hkv=1, d=32, planted=6, seed=11)
    for tau in (0.25, 1.0, 4.0):
        e = O.mala_fwd(q, k, v, tau, True, 32, 32)
        z = O.mala_fwd(q, k, v, tau, True, 32, 32, round_flags=O.LAZY_REF)
        legal = e["dec"] >= 0
        same = z["dec"] == e["dec"]
        # a decision may differ only on a tile at the threshold to rounding
        assert (same | (np.abs(e["margin"]) < 1e-9)).all()
        assert same[legal].mean() > 0.99
        if same.all():
            assert np.abs(z["o"] - e["o"]).max() < 1e-12
            assert np.abs(z["lse"] - e["lse"]).max() < 1e-12
    e = O.mala_fwd(q, k, v, 1.0, True, 32, 32)
    a = O.mala_fwd(q, k, v, 1.0, True, 32, 32, round_flags=O.BF16_FWD, force=e["dec"])
    b = O.mala_fwd(q, k, v, 1.0, True, 32, 32, round_flags=O.BF16_FWD | O.LAZY_REF,
                   force=e["dec"])
    assert np.abs(b["o"] - a["o"]).max() > 0          # other rounding points
    assert np.abs(b["o"] - e["o"]).max() < 2e-2       # both within bf16 error
    assert np.abs(b["lse"] - e["lse"]).max() < 1e-5


def _np_bf16_forward(q, k, v, bq, bk, lazy):
    """Restatement in NumPy, row by row, of the causal forward with every
    legal tile retained (tau = 0) and P~ rounded to bf16 (torch's cast,
    through fp32) before the P V product: tiles from the diagonal down, the
    exponentials against the running maximum, or with `lazy` against a
    reference that moves only when a tile's row maximum exceeds it by more
    than 8 ln 2. With `lazy`, a 128-key tile whose upper 64 keys hold a legal
    key for some row of the query block (so that they pass at tau = 0 on
    their own) is taken as those 64 keys and then the lower 64, each with its
    own reference step; otherwise as one."""
    def bf(x):
        return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    B, Hq, N, d = q.shape
    G = Hq // k.shape[1]
    scale = 1.0 / np.sqrt(d)
    o = np.zeros_like(q)
    for b in range(B):
        for h in range(Hq):
            s = scale * q[b, h] @ k[b, h // G].T
            vv = v[b, h // G]
            for r in range(N):
                m, l, acc = -np.inf, 0.0, np.zeros(d)
                r_last = min(N - 1, (r // bq) * bq + bq - 1)  # the block's last row
                for j in range(r_last // bk, -1, -1):
                    k0 = j * bk
                    st = s[r, k0:min(N, k0 + bk)].copy()
                    st[np.arange(k0, k0 + st.size) > r] = -np.inf
                    parts = [(0, st.size)]
                    if lazy and bk == 128 and k0 + 64 <= r_last:
                        parts = [(64, st.size), (0, 64)]  # upper half first
                    for c0, c1 in parts:
                        sp = st[c0:c1]
                        mt = sp.max() if sp.size else -np.inf
                        m_new = (mt if mt > m + 8.0 * np.log(2.0) else m) if lazy else max(m, mt)
                        if m_new == -np.inf:
                            continue
                        alpha = np.exp(m - m_new) if m > -np.inf else 0.0
                        pt = np.exp(sp - m_new)
                        acc = alpha * acc + bf(pt) @ vv[k0 + c0:k0 + c0 + sp.size]
                        l = alpha * l + pt.sum()
                        m = m_new
                o[b, h, r] = acc / l
    return bf(o)


def test_lazy_reference_model_matches_a_numpy_restatement():
    """The LAZY_REF model rounds P~ as a plain restatement of the lazy rule
    does, and the plain model as one with the running maximum: the two
    models differ only in the reference rule."""
    q, k, v, do = _gen_small(N=160, Hq=2, Hkv=1, d=16, planted=4, seed=23)
    for lazy, flags in ((True, O.BF16_FWD | O.LAZY_REF), (False, O.BF16_FWD)):
        r = O.mala_fwd(q, k, v, 0.0, True, 16, 16, round_flags=flags)
        e = _np_bf16_forward(q, k, v, 16, 16, lazy)
        diff = np.abs(r["o"] - e)
        # identical up to a rare bf16 flip at a rounding boundary
        assert (diff == 0).mean() > 0.999
        assert diff.max() <= 2.0 ** -7 * np.abs(e).max()
    a = O.mala_fwd(q, k, v, 0.0, True, 16, 16, round_flags=O.BF16_FWD | O.LAZY_REF)
    b = O.mala_fwd(q, k, v, 0.0, True, 16, 16, round_flags=O.BF16_FWD)
    assert not np.array_equal(a["o"], b["o"])  # the rule is exercised


def test_lazy_reference_model_128_key_tiles_in_halves():
    """With 128-key tiles the LAZY_REF model takes a tile whose upper 64 keys
    pass on their own as those keys and then the lower 64 (the NumPy
    restatement above); a model that takes every tile as one differs."""
    q, k, v, do = _gen_small(N=400, Hq=2, Hkv=1, d=16, planted=6, seed=31, sigma=0.5)
    r = O.mala_fwd(q, k, v, 0.0, True, 64, 128, round_flags=O.BF16_FWD | O.LAZY_REF)
    e = _np_bf16_forward(q, k, v, 64, 128, True)
    diff = np.abs(r["o"] - e)
    assert (diff == 0).mean() > 0.999
    assert diff.max() <= 2.0 ** -7 * np.abs(e).max()
    # the exact result does not depend on how the tile is split
    x = O.mala_fwd(q, k, v, 0.0, True, 64, 128)
    y = O.mala_fwd(q, k, v, 0.0, True, 64, 64)
    assert np.allclose(x["o"], y["o"], rtol=1e-12, atol=1e-12)
    assert np.allclose(x["lse"], y["lse"], rtol=1e-12, atol=1e-12)


def test_bf16_backward_model_matches_a_numpy_restatement():
    """The backward's bf16-operand model (Algorithm 2 with every legal tile
    kept): P from the saved LSE and dS = P (dP - D) with D = rowsum(O dO),
    P rounded to bf16 before the dV product and dS before the dK and dQ
    products, the softmax scale applied to the sums, outputs rounded. A plain
    NumPy restatement with torch's bf16 cast gives the same gradients."""
    q, k, v, do = _gen_small(N=150, Hq=4, Hkv=2, d=16, planted=4, seed=29)
    f = O.mala_fwd(q, k, v, 0.0, True, 16, 16)
    r = O.mala_bwd(q, k, v, f["o"], f["lse"], do, 0.0, True, 16, 16, round_flags=O.BF16_BWD)

    def bf(x):
        return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    B, Hq, N, d = q.shape
    G = Hq // k.shape[1]
    scale = 1.0 / np.sqrt(d)
    legal = np.tril(np.ones((N, N), dtype=bool))
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            s = scale * q[b, h] @ k[b, g].T
            p = np.where(legal, np.exp(s - f["lse"][b, h][:, None]), 0.0)
            dp = do[b, h] @ v[b, g].T
            D = (f["o"][b, h] * do[b, h]).sum(-1)
            ds = np.where(legal, p * (dp - D[:, None]), 0.0)
            dq[b, h] = scale * (bf(ds) @ k[b, g])
            dk[b, g] += bf(ds).T @ q[b, h]
            dv[b, g] += bf(p).T @ do[b, h]
    dk *= scale
    for name, e in (("dq", dq), ("dk", dk), ("dv", dv)):
        e = bf(e)
        diff = np.abs(r[name] - e)
        # one bf16 step where the two summation orders round apart, and an
        # fp64-noise floor for elements that cancel to almost nothing (where
        # dP - D itself is rounding noise of order 1e-16)
        assert (diff <= 2.0 ** -8 * np.abs(e) + 1e-9 * np.abs(e).max()).all(), name
        assert (diff == 0).mean() > 0.98, name
    # and the rounding is exercised: the exact gradients differ
    x = O.mala_bwd(q, k, v, f["o"], f["lse"], do, 0.0, True, 16, 16)
    assert not np.array_equal(x["dq"], r["dq"])


# ------------------------------------------------------- magnitude mode ----

def test_magnitude_mode_bounds_and_matches_twin():
    q, k, v, do = _tiny_inputs(16, 2, 1, 4, 9)
    for tau in (0.5, 2.0):
        r = O.mala_fwd(q, k, v, tau, True, 4, 4)
        m = O.mala_fwd(q, k, v, tau, True, 4, 4, round_flags=O.ABS, force=r["dec"])
        assert (np.abs(r["o"]) <= m["o"] + 1e-12).all()          # triangle inequality
        assert np.array_equal(m["dec"], r["dec"])
        b = O.mala_bwd(q, k, v, r["o"], r["lse"], do, tau, True, 4, 4)
        bm = O.mala_bwd(q, k, v, r["o"], r["lse"], do, tau, True, 4, 4, round_flags=O.ABS,
                        force=b["dec"])
        tq, tk, tv, _ = twin_bwd(q, k, v, r["o"], r["lse"], do, tau, True, 4, 4, mag=True)
        for x, mm, t in ((b["dq"], bm["dq"], tq), (b["dk"], bm["dk"], tk), (b["dv"], bm["dv"], tv)):
            assert (np.abs(x) <= mm + 1e-12).all()
            assert np.allclose(mm, t, rtol=1e-11, atol=1e-12)
        bd = O.mala_bwd(q, k, v, r["o"], r["lse"], do, tau, True, 4, 4, round_flags=O.ABS_D,
                        force=b["dec"])
        tq, tk, tv, _ = twin_bwd(q, k, v, r["o"], r["lse"], do, tau, True, 4, 4, dsens=True)
        assert np.allclose(bd["dq"], tq, rtol=1e-11, atol=1e-12)
        assert np.allclose(bd["dk"], tk, rtol=1e-11, atol=1e-12)
        assert not bd["dv"].any() and not tv.any()


def test_magnitude_mode_equals_value_for_nonnegative_operands():
    q, k, v, do = _tiny_inputs(14, 2, 2, 4, 4)
    v, do = np.abs(v), np.abs(do)
    r = O.mala_fwd(q, k, v, 1.0, True, 2, 2)
    m = O.mala_fwd(q, k, v, 1.0, True, 2, 2, round_flags=O.ABS, force=r["dec"])
    assert np.allclose(m["o"], r["o"], rtol=1e-13, atol=1e-13)
    b = O.mala_bwd(q, k, v, r["o"], r["lse"], do, 1.0, True, 2, 2)
    bm = O.mala_bwd(q, k, v, r["o"], r["lse"], do, 1.0, True, 2, 2, round_flags=O.ABS,
                    force=b["dec"])
    assert np.allclose(bm["dv"], b["dv"], rtol=1e-13, atol=1e-13)


# ------------------------------------------- causal with N_q < N_k (prefill) ----
# Queries sit at the last N_q key positions (a chunk of prefill against a
# cache): query q sees keys k <= q + N_k - N_q, and L_q counts them.

def _rect_inputs(Nq, Nk, Hq, Hkv, d, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, Hq, Nq, d)) * 1.5
    k = rng.standard_normal((1, Hkv, Nk, d)) * 1.5
    k[:, :, 0] += 2.0 * q.mean(axis=(1, 2))[:, None]
    hubs = rng.choice(np.arange(1, Nk), size=2, replace=False)
    k[:, :, hubs] *= 2.5
    v = rng.standard_normal((1, Hkv, Nk, d))
    do = rng.standard_normal((1, Hq, Nq, d))
    return q, k, v, do


@pytest.mark.parametrize("Nq,Nk,Hq,Hkv", [(5, 13, 2, 1), (16, 16, 2, 2), (1, 9, 2, 2), (7, 30, 4, 2)])
def test_dense_bottom_right_matches_torch(Nq, Nk, Hq, Hkv):
    d = 8
    q, k, v, do = _rect_inputs(Nq, Nk, Hq, Hkv, d, 3)
    scale = 1.0 / math.sqrt(d)
    o, lse = O.dense_fwd(q, k, v, True)
    G = Hq // Hkv
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    ke, ve = tk.repeat_interleave(G, dim=1), tv.repeat_interleave(G, dim=1)
    allowed = torch.ones(Nq, Nk, dtype=torch.bool).tril(diagonal=Nk - Nq)  # bottom-right
    to = torch.nn.functional.scaled_dot_product_attention(tq, ke, ve, attn_mask=allowed,
                                                          scale=scale)
    assert np.allclose(o, to.detach().numpy(), rtol=1e-12, atol=1e-12)
    s = (tq @ ke.transpose(-1, -2)) * scale
    tl = torch.logsumexp(s.masked_fill(~allowed, -math.inf), dim=-1)
    assert np.allclose(lse, tl.detach().numpy(), rtol=1e-12, atol=1e-12)
    to.backward(torch.tensor(do))
    dq, dk, dv = O.dense_bwd(q, k, v, do, True)
    for x, y in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.allclose(x, y.numpy(), rtol=1e-10, atol=1e-12)


RECT = [
    # (Nq, Nk, Hq, Hkv, d, bq, bk, tau)
    (5, 13, 2, 1, 4, 2, 2, 1.0),
    (7, 16, 2, 2, 4, 4, 2, 0.5),
    (9, 14, 2, 1, 4, 2, 4, 2.0),
    (1, 11, 2, 2, 4, 1, 3, 1.0),
    (12, 16, 1, 1, 4, 4, 4, 4.0),
]


@pytest.mark.parametrize("case", RECT)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_bottom_right_matches_bruteforce_twin(case, seed):
    Nq, Nk, Hq, Hkv, d, bq, bk, tau = case
    q, k, v, do = _rect_inputs(Nq, Nk, Hq, Hkv, d, seed)
    r = O.mala_fwd(q, k, v, tau, True, bq, bk)
    to, tl, tdec, _ = twin_fwd(q, k, v, tau, True, bq, bk)
    assert not _near_zero(r["margin"]).any()
    assert np.array_equal(r["dec"], tdec)
    assert np.allclose(r["o"], to, rtol=1e-12, atol=1e-12)
    assert np.allclose(r["lse"], tl, rtol=1e-12, atol=1e-12)
    b = O.mala_bwd(q, k, v, r["o"], r["lse"], do, tau, True, bq, bk)
    tq, tk, tv, tbd = twin_bwd(q, k, v, r["o"], r["lse"], do, tau, True, bq, bk)
    assert not _near_zero(b["margin"]).any()
    assert np.array_equal(b["dec"], tbd)
    for x, y in ((b["dq"], tq), (b["dk"], tk), (b["dv"], tv)):
        assert np.allclose(x, y, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("off_blocks,bq,tau", [(1, 4, 1.0), (2, 4, 0.25), (3, 2, 4.0)])
def test_bottom_right_is_the_suffix_of_the_full_problem(off_blocks, bq, tau):
    """A chunk of N_q queries at the end of an N_k-token sequence is exactly the
    last N_q rows of the full causal problem when N_k - N_q is a whole number
    of query blocks (the blocks then coincide): same decisions, O and LSE, and
    the same dQ; dK and dV equal the full backward with dO = 0 on the other
    rows (those rows then contribute dS = 0)."""
    Nq, d, bk, Hq, Hkv = 12, 4, 4, 2, 1
    Nk = Nq + off_blocks * bq
    q_full, k, v, do_full = _rect_inputs(Nk, Nk, Hq, Hkv, d, 7)
    q_full *= 2.0  # more peaked scores, so that these small problems skip tiles
    do_full[:, :, :Nk - Nq] = 0.0
    q, do = q_full[:, :, Nk - Nq:], do_full[:, :, Nk - Nq:]
    full = O.mala_fwd(q_full, k, v, tau, True, bq, bk)
    part = O.mala_fwd(q, k, v, tau, True, bq, bk)
    nb = off_blocks  # query blocks before the chunk
    assert np.array_equal(part["dec"], full["dec"][:, :, nb:])
    assert np.allclose(part["o"], full["o"][:, :, Nk - Nq:], rtol=1e-13, atol=1e-14)
    assert np.allclose(part["lse"], full["lse"][:, :, Nk - Nq:], rtol=1e-13, atol=1e-14)
    bf = O.mala_bwd(q_full, k, v, full["o"], full["lse"], do_full, tau, True, bq, bk)
    bp = O.mala_bwd(q, k, v, part["o"], part["lse"], do, tau, True, bq, bk)
    assert np.allclose(bp["dq"], bf["dq"][:, :, Nk - Nq:], rtol=1e-12, atol=1e-13)
    assert np.allclose(bp["dk"], bf["dk"], rtol=1e-12, atol=1e-13)
    assert np.allclose(bp["dv"], bf["dv"], rtol=1e-12, atol=1e-13)
    assert (bp["dec"] == 0).any() or (part["dec"] == 0).any()  # the rule is exercised


def test_single_causal_query_is_decode():
    """One causal query at the end of the cache sees every key (L = N_k): it is
    the one-split decode of that query (Sec. 2.4)."""
    rng = np.random.default_rng(11)
    Hq, Hkv, Nk, d, bk = 4, 2, 37, 4, 4
    k = rng.standard_normal((1, Hkv, Nk, d)) * 1.5
    k[:, :, [3, 20]] *= 2.5
    v = rng.standard_normal((1, Hkv, Nk, d))
    q = rng.standard_normal((1, Hq, 1, d)) * 1.5
    for tau in (0.25, 1.0, 4.0):
        f = O.mala_fwd(q, k, v, tau, True, 1, bk)
        dd = O.mala_decode(q[:, :, 0], k, v, 1, tau, bk)
        assert np.allclose(f["o"][:, :, 0], dd["o"], rtol=1e-13, atol=1e-14)
        assert np.allclose(f["lse"][:, :, 0], dd["lse"], rtol=1e-13, atol=1e-14)
