"""Host model of how the backward's dK/dV pass schedules its work (test code).

The pass works on pairs of 64-key blocks of one (batch, KV head), split into
segments whose fp32 partial sums a finalize kernel adds. From the backward's
decision bitmap this module derives what the kernels do, so that a test can
state which code paths an input reaches (for example a pair cut into the
maximum of 8 segments, whose finalize adds 8 partials):

  * kept[j]: the (query head, query block) items that keep key block j;
  * heavy blocks: 4 kept[j] >= the items with a legal tile in block j;
    heavy blocks are paired in index order, then the light ones;
  * K = sum of kept[j], npair = Tc // 2 + 1, Lseg = max(512, ceil(2 K / (4 npair)));
    a pair keeping `kept` items gets min(8, max(1, ceil(kept / Lseg)))
    segments.
"""
import numpy as np

SEG_KEPT = 512
SEG_MAX = 8
SLOTS_PER_PAIR = 4


def pairs_and_segments(bdec, heads_kv, nq, nk, causal=True):
    """bdec: [B, Hq, Tr, Tc] int array of 64 x 64 backward decisions (1 kept,
    0 skipped, -1 illegal). Returns {(b, g): [(jA, jB, kept, nseg), ...]}
    in table order (heavy pairs first)."""
    B, Hq, Tr, Tc = bdec.shape
    G = Hq // heads_kv
    off = nk - nq if causal else 0
    npair = Tc // 2 + 1
    out = {}
    for b in range(B):
        for g in range(heads_kv):
            d = bdec[b, g * G:(g + 1) * G]
            kept = (d == 1).sum(axis=(0, 1)).astype(np.int64)
            first = np.array([min(Tr - 1, max(0, 64 * j - off) // 64) if causal else 0
                              for j in range(Tc)])
            heavy = 4 * kept >= G * (Tr - first)
            hv = [j for j in range(Tc) if heavy[j]]
            lt = [j for j in range(Tc) if not heavy[j]]
            table = [-1] * (2 * npair)
            for x, j in enumerate(hv):
                table[x] = j
            ph = (len(hv) + 1) // 2
            for x, j in enumerate(lt):
                table[2 * ph + x] = j
            K = int(kept.sum())
            lseg = max(SEG_KEPT, -(-2 * K // (SLOTS_PER_PAIR * npair)))
            rows = []
            for p in range(npair):
                jA, jB = table[2 * p], table[2 * p + 1]
                if jA < 0:
                    continue
                k = int(kept[jA] + (kept[jB] if jB >= 0 else 0))
                rows.append((jA, jB, k, min(SEG_MAX, max(1, -(-k // lseg)))))
            out[(b, g)] = rows
    return out


def segments_of_block(sched, b, g, j):
    for (jA, jB, _, nseg) in sched[(b, g)]:
        if j in (jA, jB):
            return nseg
    raise KeyError(j)
