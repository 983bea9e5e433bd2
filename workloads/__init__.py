"""Seeded synthetic inputs shaped like the MALA paper's workloads.

This module holds no attention arithmetic. It only draws Gaussian tensors,
plants the structure described below, and rounds once to bf16. Both the GPU
tests and the CPU oracle consume its output; nothing else is shared between
them.

The paper measures on hidden states of a 14B model, which are not available
here. These inputs stand in for them: lengths 1K-32K and 128K, 8 query / 1 KV
heads per GPU at 128K (the per-rank share of the operator benchmark, App. C.5,
Table 4), d = 128, and score distributions with the features that let MALA
skip work (a sink key, a few large "retrieval" keys, an optional local bias).

Recipe ``peaked(seed, B, Hq, Hkv, N, d, sigma_s, n_planted, local_bias)``,
applied independently to every (batch b, KV head g) with G = Hq / Hkv:

1. Q0, K0 ~ N(0, sigma_e^2) with sigma_e = sqrt(sigma_s), so that
   <q, k> / sqrt(d) has standard deviation sigma_s.
2. (local bias only) for j >= 1: K0[j] += c * mean{Q0[h, i] : h in the group,
   j < i <= min(j + 32, N - 1)} with c = 48 G / (sigma_e^2 sqrt(d)); this adds
   about +1.5 to the scaled score of the next 32 queries on key j.
3. sink: a unit vector u; every query of the group gets Q = Q0 + 2 sigma_e u,
   and K[0] = 4 sigma_e sqrt(d) u (scaled sink score ~ N(8 sigma_s, (4 sigma_s)^2)).
4. planted pairs t = 0..n_planted-1: distinct query positions p_t in
   [Bk + 1, N), query head g*G + (t mod G), distinct key positions p'_t in
   [1, p_t - Bk]; K[p'_t] = 4 Q[h_t, p_t].
5. V ~ N(0, 1), dO ~ N(0, 1).
   (optional head_gain = (lo, hi)) after the planting, every query head h of
   entry b is multiplied by its own gain, log-uniform in [lo, hi].
6. every tensor is rounded once fp32 -> bf16 (round to nearest even).

Random streams: numpy PCG64 seeded by SeedSequence(seed, spawn_key=(b, head,
tensor, chunk)); Q rows come in chunks of 64 rows and K/V/dO in chunks of
4096 rows, so any slice regenerates on its own.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

Q_CHUNK = 64
KV_CHUNK = 4096
_TID_Q, _TID_K, _TID_V, _TID_DO, _TID_U, _TID_PLANT, _TID_GAIN = range(7)


def _rng(seed, b, head, tid, chunk=0):
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence(entropy=seed, spawn_key=(b, head, tid, chunk))))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (RNE); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_rows(seed, b, head, tid, rows, d, chunk, sigma=1.0):
    """Rows `rows` (sorted int array) of an N(0, sigma^2) [*, d] tensor."""
    out = np.empty((len(rows), d), dtype=np.float32)
    if len(rows) == 0:
        return out
    chunks = np.unique(rows // chunk)
    for c in chunks:
        blk = _rng(seed, b, head, tid, int(c)).standard_normal((chunk, d), dtype=np.float32)
        sel = np.nonzero(rows // chunk == c)[0]
        out[sel] = blk[rows[sel] - c * chunk]
    if sigma != 1.0:
        out *= np.float32(sigma)
    return out


def _normal_full(seed, b, head, tid, n, d, chunk, sigma=1.0):
    out = np.empty((n, d), dtype=np.float32)
    for c in range((n + chunk - 1) // chunk):
        r0, r1 = c * chunk, min(n, (c + 1) * chunk)
        blk = _rng(seed, b, head, tid, c).standard_normal((chunk, d), dtype=np.float32)
        out[r0:r1] = blk[: r1 - r0]
    if sigma != 1.0:
        out *= np.float32(sigma)
    return out


@dataclass
class Spec:
    """One generator call: sizes plus the peaked-distribution parameters."""
    seed: int
    batch: int
    heads_q: int
    heads_kv: int
    seqlen: int
    head_dim: int
    sigma_s: float = 3.0
    n_planted: int = 0
    local_bias: bool = False
    block_k: int = 64
    head_gain: tuple | None = None

    @property
    def group(self):
        return self.heads_q // self.heads_kv


def _planted(spec: Spec, b, g):
    """(query pos, query head, key pos) of the planted pairs of group (b, g)."""
    n, N, Bk, G = spec.n_planted, spec.seqlen, spec.block_k, spec.group
    if n == 0 or N <= Bk + 2:
        return np.zeros((0, 3), dtype=np.int64)
    rng = _rng(spec.seed, b, g, _TID_PLANT)
    n = min(n, N - Bk - 1)
    qpos = rng.choice(np.arange(Bk + 1, N), size=n, replace=False)
    used = set()
    out = []
    for t, p in enumerate(qpos):
        hi = int(p) - Bk
        kp = None
        for _ in range(64):
            c = int(rng.integers(1, hi + 1))
            if c not in used:
                kp = c
                break
        if kp is None:  # dense corner of a tiny problem: take the first free slot
            free = [c for c in range(1, hi + 1) if c not in used]
            if not free:
                continue
            kp = free[0]
        used.add(kp)
        out.append((int(p), g * G + (t % G), kp))
    return np.asarray(out, dtype=np.int64).reshape(-1, 3)


def head_gain(spec: Spec, b: int, h: int) -> float:
    """Query gain of head h of batch entry b (1 unless spec.head_gain = (lo, hi)):
    log-uniform in [lo, hi], one draw per (b, h)."""
    if spec.head_gain is None:
        return 1.0
    lo, hi = spec.head_gain
    x = _rng(spec.seed, b, h, _TID_GAIN).random()
    return math.exp(math.log(lo) + x * (math.log(hi) - math.log(lo)))


def _group(spec: Spec, b: int, g: int, q_rows, want_do: bool):
    """All tensors of one (b, g) group, fp32 before rounding."""
    N, d, G = spec.seqlen, spec.head_dim, spec.group
    sig_e = math.sqrt(spec.sigma_s)
    u = _rng(spec.seed, b, g, _TID_U).standard_normal(d).astype(np.float64)
    u = (u / np.linalg.norm(u)).astype(np.float32)
    heads = range(g * G, (g + 1) * G)
    plant = _planted(spec, b, g)

    k = _normal_full(spec.seed, b, g, _TID_K, N, d, KV_CHUNK, sig_e)
    if spec.local_bias:
        # window sums of the un-shifted queries of the group, rows j+1..j+32
        qsum = np.zeros((N, d), dtype=np.float64)
        for h in heads:
            qsum += _normal_full(spec.seed, b, h, _TID_Q, N, d, Q_CHUNK, sig_e)
        cs = np.concatenate([np.zeros((1, d)), np.cumsum(qsum, axis=0)])
        j = np.arange(1, N)
        hi = np.minimum(j + 32, N - 1)
        cnt = (hi - j) * G
        ok = cnt > 0
        c = 48.0 * G / (sig_e ** 2 * math.sqrt(d))
        win = (cs[hi + 1] - cs[j + 1])
        k[j[ok]] += (c * win[ok] / cnt[ok, None]).astype(np.float32)
        del qsum, cs, win
    k[0] = np.float32(4.0 * sig_e * math.sqrt(d)) * u

    full_q = q_rows is None
    rows = np.arange(N) if full_q else np.unique(np.asarray(q_rows, dtype=np.int64))
    q = {}
    for h in heads:
        if full_q:
            qh = _normal_full(spec.seed, b, h, _TID_Q, N, d, Q_CHUNK, sig_e)
        else:
            qh = _normal_rows(spec.seed, b, h, _TID_Q, rows, d, Q_CHUNK, sig_e)
        qh += np.float32(2.0 * sig_e) * u
        q[h] = qh
    for (p, h, kp) in plant:
        if full_q:
            qrow = q[h][p]
        else:
            qrow = _normal_rows(spec.seed, b, h, _TID_Q, np.array([p]), d, Q_CHUNK, sig_e)[0]
            qrow = qrow + np.float32(2.0 * sig_e) * u
        k[kp] = np.float32(4.0) * qrow
    if spec.head_gain is not None:
        for h in heads:
            q[h] *= np.float32(head_gain(spec, b, h))
    v = _normal_full(spec.seed, b, g, _TID_V, N, d, KV_CHUNK)
    do = None
    if want_do:
        do = {h: (_normal_full(spec.seed, b, h, _TID_DO, N, d, KV_CHUNK) if full_q else
                  _normal_rows(spec.seed, b, h, _TID_DO, rows, d, KV_CHUNK)) for h in heads}
    return q, k, v, do, plant, rows


def peaked(spec: Spec, q_rows=None, want_do=True, threads=None):
    """Generate bf16 inputs. Returns a dict of uint16 bf16 bit arrays:
    q [B,Hq,R,d] (R = N, or len(q_rows)), k, v [B,Hkv,N,d], do [B,Hq,R,d]
    (if want_do), plus 'planted' [(b, qpos, head, kpos)] and 'q_rows'."""
    B, Hq, Hkv, N, d = spec.batch, spec.heads_q, spec.heads_kv, spec.seqlen, spec.head_dim
    R = N if q_rows is None else len(np.unique(np.asarray(q_rows)))
    out = {
        "q": np.empty((B, Hq, R, d), dtype=np.uint16),
        "k": np.empty((B, Hkv, N, d), dtype=np.uint16),
        "v": np.empty((B, Hkv, N, d), dtype=np.uint16),
    }
    if want_do:
        out["do"] = np.empty((B, Hq, R, d), dtype=np.uint16)
    planted = []
    rows_out = [None]

    def work(bg):
        b, g = bg
        q, k, v, do, plant, rows = _group(spec, b, g, q_rows, want_do)
        for h, qh in q.items():
            out["q"][b, h] = f32_to_bf16_bits(qh)
            if want_do:
                out["do"][b, h] = f32_to_bf16_bits(do[h])
        out["k"][b, g] = f32_to_bf16_bits(k)
        out["v"][b, g] = f32_to_bf16_bits(v)
        rows_out[0] = rows
        return [(b, int(p), int(h), int(kp)) for (p, h, kp) in plant]

    jobs = [(b, g) for b in range(B) for g in range(Hkv)]
    nthreads = threads or min(len(jobs), max(1, min(16, os.cpu_count() or 1)))
    if nthreads > 1 and len(jobs) > 1:
        with ThreadPoolExecutor(nthreads) as ex:
            for pl in ex.map(work, jobs):
                planted.extend(pl)
    else:
        for j in jobs:
            planted.extend(work(j))
    out["planted"] = np.asarray(planted, dtype=np.int64).reshape(-1, 4)
    out["q_rows"] = rows_out[0]
    return out


def selfcheck(inp: dict, spec: Spec, samples: int = 4096, seed: int = 12345):
    """Input statistics (scaled scores): bulk std, mean sink score, mean planted
    score. Only describes the generated tensors."""
    rng = np.random.default_rng(seed)
    q = inp["q"]
    k = inp["k"]
    B, Hq, R, d = q.shape
    G = spec.group
    sc = 1.0 / math.sqrt(d)
    rows = inp["q_rows"]
    bulk, sink = [], []
    for _ in range(samples):
        b = int(rng.integers(B)); h = int(rng.integers(Hq)); r = int(rng.integers(R))
        qpos = int(rows[r])
        if qpos < 2:
            continue
        kp = int(rng.integers(1, qpos + 1))
        qv = bf16_bits_to_f32(q[b, h, r]).astype(np.float64)
        bulk.append(sc * qv @ bf16_bits_to_f32(k[b, h // G, kp]).astype(np.float64))
        sink.append(sc * qv @ bf16_bits_to_f32(k[b, h // G, 0]).astype(np.float64))
    planted = []
    if len(inp["planted"]) and R == spec.seqlen:
        for (b, p, h, kp) in inp["planted"][:256]:
            qv = bf16_bits_to_f32(q[b, h, p]).astype(np.float64)
            planted.append(sc * qv @ bf16_bits_to_f32(k[b, h // G, kp]).astype(np.float64))
    return {
        "bulk_score_std": float(np.std(bulk)) if bulk else None,
        "sink_score_mean": float(np.mean(sink)) if sink else None,
        "planted_score_mean": float(np.mean(planted)) if planted else None,
    }


# --------------------------------------------------------------------------
# The five measured workloads (paper lengths and head shares; seeds fixed).

@dataclass
class Workload:
    name: str
    spec: Spec
    tau: float = 1.0
    block_q: int = 64
    block_k: int = 64
    passes: tuple = ("fwd",)
    extra: dict = field(default_factory=dict)


def cfg1():
    """MALA forward, causal, B 1, 2 MHA heads, N 1024, d 64, 8 planted pairs."""
    return Workload("cfg1_fwd_1k_mha2_d64", Spec(101, 1, 2, 2, 1024, 64, 3.0, 8), passes=("fwd",))


def cfg2():
    """MALA forward + backward, B 1, 8 MHA heads, N 8192, d 128, 64 planted."""
    return Workload("cfg2_fwdbwd_8k_mha8_d128", Spec(201, 1, 8, 8, 8192, 128, 3.0, 64),
                    passes=("fwd", "bwd"))


CFG3_LENGTHS = (1024, 4096, 16384, 32768)


def cfg3(length: int):
    """Length sweep: B 1, 16 query / 4 KV heads, d 128, 64 planted, local bias."""
    seed = 301 + CFG3_LENGTHS.index(length)
    return Workload(f"cfg3_fwdbwd_{length // 1024}k_gqa16x4_d128",
                    Spec(seed, 1, 16, 4, length, 128, 3.0, 64, local_bias=True),
                    passes=("fwd", "bwd"))


def cfg4():
    """128K operator at one GPU's head share: 8 query / 1 KV head, d 128."""
    return Workload("cfg4_fwdbwd_128k_gqa8x1_d128", Spec(401, 1, 8, 1, 131072, 128, 3.0, 256),
                    passes=("fwd", "bwd"))


def cfg5(variant: str = "peaked", tau: float = 1.0, num_splits: int = 16):
    """Decode: 16 sequences x 1 token, 32 query / 8 KV heads, 128K cache, d 128."""
    seed, sig = (501, 3.0) if variant == "peaked" else (502, 0.5)
    return Workload(f"cfg5_decode_128k_b16_gqa32x8_d128_{variant}",
                    Spec(seed, 16, 32, 8, 131072, 128, sig, 256), tau=tau, passes=("decode",),
                    extra={"num_splits": num_splits, "variant": variant})


DECODE_TAUS = (0.0, 0.25, 1.0, 4.0)


MATCHED_WORK_VARIANTS = ("uniform", "mixed")


def matched_work(variant: str = "uniform"):
    """Matched-work allocation study at 8K: B 4 independent inputs (each batch
    entry draws its own streams), 16 query / 4 KV heads, d 128, 64 planted,
    local bias. "mixed" also scales each (input, query head) by its own query
    gain, log-uniform in [0.5, 2], so that heads and inputs differ in
    sharpness; "uniform" draws them all alike."""
    if variant == "uniform":
        spec = Spec(601, 4, 16, 4, 8192, 128, 3.0, 64, local_bias=True)
    else:
        spec = Spec(602, 4, 16, 4, 8192, 128, 3.0, 64, local_bias=True, head_gain=(0.5, 2.0))
    return Workload(f"matched_work_8k_b4_gqa16x4_d128_{variant}", spec, passes=("fwd",))
