"""Seeded random sweep of small problems over the whole parameter space
(test code): forward, backward and split-KV decode against the oracle, 32
cases each, paged variable-length decode, 16 cases, and forward and backward
at 1K-4.5K keys, 6 cases each; every case is drawn from its own seed so that
any one reruns alone.

A case draws the batch (1-2), the KV heads (1-2) and the group size (1, 2,
3, 4 or 8), the head dimension (64 or 128), the lengths (1-900 keys; causal
problems are either square or a chunk of the last queries against the cache,
non-causal ones rectangular), tau in {0, 0.25, 1, 4, inf}, the decision tile
(64 or 128 rows and keys), the logit scale (peaked or diffuse), planted keys
and the local bias, and for decode the split count (1-8, at most the
cache's decision tiles, as the API requires). The comparison is the same as
in the per-entry-point tests (tests/parity.py)."""
import math

import numpy as np
import pytest

import workloads as W
from test_gpu_bwd import compare_bwd
from test_gpu_decode import compare_decode, compare_decode_paged, decode_inputs, paged_inputs
from test_gpu_fwd import compare_fwd

pytestmark = pytest.mark.gpu

TAUS = (0.0, 0.25, 1.0, 4.0, math.inf)
N_CASES = 32


def _draw(seed):
    r = np.random.default_rng(seed)
    B = int(r.integers(1, 3))
    Hkv = int(r.integers(1, 3))
    G = int(r.choice([1, 2, 3, 4, 8]))
    d = int(r.choice([64, 128]))
    Nk = int(r.integers(1, 901))
    causal = bool(r.integers(0, 4) > 0)  # mostly causal
    if causal:
        Nq = Nk if r.integers(0, 2) else int(r.integers(1, Nk + 1))
    else:
        Nq = int(r.integers(1, 901))
    tau = float(r.choice(TAUS))
    bq = int(r.choice([64, 128]))
    bk = int(r.choice([64, 128]))
    sigma = float(r.choice([3.0, 0.5]))
    planted = int(r.choice([0, 4, 8])) if Nk > 130 else 0
    local = bool(r.integers(0, 2)) and G > 1 and Nk > 64
    S = int(r.integers(1, 9))
    return dict(B=B, Hkv=Hkv, Hq=G * Hkv, d=d, Nk=Nk, Nq=Nq, causal=causal, tau=tau, bq=bq,
                bk=bk, sigma=sigma, planted=planted, local=local, S=S)


def _prefill(seed, c, want_do):
    spec = W.Spec(seed, c["B"], c["Hq"], c["Hkv"], c["Nk"], c["d"], c["sigma"], c["planted"],
                  local_bias=c["local"])
    a = W.peaked(spec, want_do=want_do)
    Nq, Nk = c["Nq"], c["Nk"]
    if c["causal"]:
        # the last Nq queries against the whole cache (bottom-right alignment)
        inp = {"q": np.ascontiguousarray(a["q"][:, :, Nk - Nq:]), "k": a["k"], "v": a["v"]}
        if want_do:
            inp["do"] = np.ascontiguousarray(a["do"][:, :, Nk - Nq:])
        return inp
    # non-causal: queries (and dO) from a second draw of another length
    b = W.peaked(W.Spec(seed + 1, c["B"], c["Hq"], c["Hkv"], Nq, c["d"], c["sigma"], 0),
                 want_do=want_do)
    inp = {"q": b["q"], "k": a["k"], "v": a["v"]}
    if want_do:
        inp["do"] = b["do"]
    return inp


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_forward(case):
    seed = 71000 + case
    c = _draw(seed)
    print(f"[random fwd] seed {seed} {c}", flush=True)
    compare_fwd(_prefill(seed, c, False), c["tau"], causal=c["causal"], label=f"rand{case}",
                bq=c["bq"], bk=c["bk"])


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_backward(case):
    seed = 72000 + case
    c = _draw(seed)
    print(f"[random bwd] seed {seed} {c}", flush=True)
    compare_bwd(_prefill(seed, c, True), c["tau"], causal=c["causal"], label=f"rand{case}",
                bq=c["bq"], bk=c["bk"])


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_decode(case):
    seed = 73000 + case
    c = _draw(seed)
    print(f"[random decode] seed {seed} {c}", flush=True)
    spec = W.Spec(seed, c["B"], c["Hq"], c["Hkv"], c["Nk"], c["d"], c["sigma"], c["planted"])
    S = min(c["S"], -(-c["Nk"] // c["bk"]))  # 1 <= num_splits <= decision tiles
    compare_decode(decode_inputs(spec), c["tau"], S, label=f"rand{case}", bk=c["bk"])


@pytest.mark.parametrize("case", range(16))
def test_random_decode_paged(case):
    """Paged, variable-length decode: 1-4 sequences of 1-900 keys in
    shuffled 64-key pages, each compared with the oracle's decode of its own
    cache (its own L)."""
    seed = 74000 + case
    c = _draw(seed)
    r = np.random.default_rng(seed + 1)
    lens = [int(x) for x in r.integers(1, 901, size=int(r.integers(1, 5)))]
    bk, tau = c["bk"], c["tau"]
    S = min(c["S"], -(-max(lens) // bk))
    print(f"[random paged] seed {seed} lens {lens} Hq {c['Hq']} Hkv {c['Hkv']} d {c['d']} "
          f"tau {tau} S {S} bk {bk}", flush=True)
    compare_decode_paged(paged_inputs(seed, lens, c["Hq"], c["Hkv"], c["d"]), lens, tau, S, bk=bk)


def _draw_medium(seed):
    """A longer problem (1K-4.5K keys, ragged): more key blocks per pair and
    longer pipelines, still seconds for the oracle."""
    c = _draw(seed)
    r = np.random.default_rng(seed + 7)
    c["Nk"] = int(r.integers(1000, 4501))
    c["Nq"] = c["Nk"] if (not c["causal"] or r.integers(0, 2)) else int(r.integers(1, c["Nk"] + 1))
    if not c["causal"]:
        c["Nq"] = int(r.integers(1000, 4501))
    c["B"] = 1
    c["planted"] = int(r.choice([8, 32]))
    return c


@pytest.mark.parametrize("case", range(6))
def test_random_medium_forward(case):
    seed = 75000 + case
    c = _draw_medium(seed)
    print(f"[random medium fwd] seed {seed} {c}", flush=True)
    compare_fwd(_prefill(seed, c, False), c["tau"], causal=c["causal"], label=f"rmed{case}",
                bq=c["bq"], bk=c["bk"])


@pytest.mark.parametrize("case", range(6))
def test_random_medium_backward(case):
    seed = 76000 + case
    c = _draw_medium(seed)
    print(f"[random medium bwd] seed {seed} {c}", flush=True)
    compare_bwd(_prefill(seed, c, True), c["tau"], causal=c["causal"], label=f"rmed{case}",
                bq=c["bq"], bk=c["bk"])


@pytest.mark.parametrize("seed", [80092])
def test_random_forward_found_by_a_wider_sweep(seed):
    """A case a wider run of this sweep found: 70 keys in one 128-key
    decision tile, diffuse non-causal rows. The kernel forms the tile's upper
    64 keys, which pass on their own, before the lower 64, each with its own
    lazy reference step; the bf16 model must round P~ the same way."""
    c = _draw(seed)
    print(f"[random fwd] seed {seed} {c}", flush=True)
    compare_fwd(_prefill(seed, c, False), c["tau"], causal=c["causal"], label=f"seed{seed}",
                bq=c["bq"], bk=c["bk"])
