"""Index identities that the backward kernels rely on, checked on the CPU.

Two of the backward passes use an index form that is cheaper than, but
equivalent to, the direct formula:

* the scoring pass steps each item's position in the decision map along the
  order in which a wave visits its items, instead of evaluating the map's
  index (triangular row offset plus head base) for every item;
* the dQ pass splits the address of each transposing K read into one per-lane
  offset per d chunk plus a constant per key subtile and half, which the read
  takes as an immediate.

Each test restates the definitions involved, checks each restatement against
the source text (so that a change of the kernels' layout or swizzle cannot
leave the test checking an old definition), and verifies the identity for
every case over a range of shapes."""
import itertools
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "adaptive_softmax_attention_amd", "csrc")


def source(name):
    with open(os.path.join(CSRC, name)) as f:
        return re.sub(r"\s+", " ", f.read())


# ---- decision-map position of the scoring pass ----------------------------

def causal_row_start(i, tc, cblk):
    istar = max(tc - cblk - 1, 0)
    m = min(i, istar)
    return m * (m - 1) // 2 + m * (cblk + 1) + (i - m) * tc


def test_row_start_restatement_is_the_sources():
    text = source("mala_internal.h")
    for piece in ("const long long istar = tc - cblk - 1 > 0 ? tc - cblk - 1 : 0;",
                  "const long long m = i < istar ? i : istar;",
                  "return m * (m - 1) / 2 + m * (cblk + 1) + (i - m) * tc;"):
        assert piece in text, piece
    # the map index is the head's base plus the row start plus the key block
    assert ("const long long t = p.causal ? causal_row_start(i, p.tc, p.cblk) + j : "
            "(long long)i * p.tc + j; return (long long)bh * p.dmap_per_head + t;"
            in source("mala_bwd.h"))


def test_scoring_pass_steps_are_in_the_kernel():
    text = source("mala_bwd.hip")
    for piece in ("long long hoff = (long long)(b * p.heads_q + kvh * p.group + ch) * ph + jw;",
                  "long long roff = p.causal ? causal_row_start(ci, p.tc, p.cblk) : "
                  "(long long)ci * p.tc;",
                  "p.dmap[hoff + roff] = want ? 1 : 0;",
                  "ch += 2; hoff += 2 * ph; while (ch >= p.group) { ch -= p.group; "
                  "hoff -= p.group * ph; --ci; roff -= (p.causal && ci < istar) ? "
                  "ci + p.cblk + 1 : p.tc; }",
                  "const int istar = max(p.tc - p.cblk - 1, 0);",
                  "int ci = p.tr - 1 - par / p.group, ch = par % p.group;"):
        assert piece in text, piece


def test_stepped_map_position_equals_the_index():
    """Every item that a compute wave of the scoring pass records (wave w
    scores key block 4 G + w % 4 and every other item from w / 4 on, item k
    being group head k % group of query block tr - 1 - k / group) lands on
    the byte the map index gives, inside the map."""
    n = 0
    for nq, nk, causal, B, Hkv, G in itertools.product(
            (1, 64, 65, 200, 1000), (1, 130, 1000, 1300), (0, 1), (1, 2), (1, 3),
            (1, 2, 3, 8)):
        if causal and nq > nk:
            continue
        tr, tc = (nq + 63) // 64, (nk + 63) // 64
        off = nk - nq if causal else 0
        cblk = (63 + off) // 64
        Hq = Hkv * G
        ph = causal_row_start(tr, tc, cblk) if causal else tr * tc
        size = B * Hq * ph
        istar = max(tc - cblk - 1, 0)

        def first_qblock(j):
            t = 64 * j - off
            return min(tr - 1, t // 64) if causal and t > 0 else 0

        for b, kvh, g4 in itertools.product(range(B), range(Hkv), range((tc + 3) // 4)):
            jb0 = 4 * g4
            n_items = G * (tr - first_qblock(jb0))
            for w in range(8):
                jw, par = jb0 + (w & 3), w >> 2
                if jw >= tc:
                    continue
                ci, ch = tr - 1 - par // G, par % G
                hoff = (b * Hq + kvh * G + ch) * ph + jw
                roff = causal_row_start(ci, tc, cblk) if causal else ci * tc
                for _ in range(par, n_items, 2):
                    if not causal or jw <= ci + cblk:
                        bh = b * Hq + kvh * G + ch
                        t = (causal_row_start(ci, tc, cblk) if causal else ci * tc) + jw
                        assert hoff + roff == bh * ph + t
                        assert 0 <= hoff + roff < size
                        n += 1
                    ch += 2
                    hoff += 2 * ph
                    while ch >= G:
                        ch -= G
                        hoff -= G * ph
                        ci -= 1
                        roff -= ci + cblk + 1 if causal and ci < istar else tc
    assert n > 50_000


# ---- transposing K reads of the dQ pass ------------------------------------

def dqswz(D, row):
    if D == 128:
        return ((row & 3) << 1) | (((row >> 3) & 1) << 3)
    return (((row >> 1) & 1) << 1) | (((row >> 3) & 1) << 2)


def test_dq_swizzle_restatement_is_the_sources():
    text = source("mala_common.h")
    assert ("int dqswz(int row) { if constexpr (D == 128) return ((row & 3) << 1) | "
            "(((row >> 3) & 1) << 3); else return (((row >> 1) & 1) << 1) | "
            "(((row >> 3) & 1) << 2); }" in text)
    kern = source("mala_bwd.hip")
    assert ("const int row = 8 * g4 + (l16 >> 2); const int col = 16 * ds + 4 * (l16 & 3); "
            "ktr_off[ds] = row * D + (((col >> 3) ^ dqswz<D>(row)) & (KCH - 1)) * 8 + (col & 7);"
            in kern)
    assert "lds_read_tr4(kt + ktr_off[ds] + (32 * kc + 4 * hh) * D)" in kern


def test_dq_read_offset_split_equals_the_swizzled_address():
    """Row 32 kc + 8 g4 + 4 hh + l16 / 4 and column 16 ds + 4 (l16 % 4) of
    the swizzled K tile are at ktr_off[ds] + (32 kc + 4 hh) D for every lane,
    key subtile pair, half and d chunk, at both head dims."""
    for D in (64, 128):
        kch, nds = D // 8, D // 16
        for lane in range(64):
            l16, g4 = lane & 15, lane >> 4
            base_row = 8 * g4 + (l16 >> 2)
            offs = []
            for ds in range(nds):
                col = 16 * ds + 4 * (l16 & 3)
                offs.append(base_row * D + (((col >> 3) ^ dqswz(D, base_row)) & (kch - 1)) * 8
                            + (col & 7))
            for kc, hh, ds in itertools.product(range(2), range(2), range(nds)):
                row = 32 * kc + 8 * g4 + 4 * hh + (l16 >> 2)
                col = 16 * ds + 4 * (l16 & 3)
                direct = row * D + (((col >> 3) ^ dqswz(D, row)) & (kch - 1)) * 8 + (col & 7)
                assert offs[ds] + (32 * kc + 4 * hh) * D == direct
                # the constant part fits the read's 16-bit byte offset
                assert 2 * (32 * kc + 4 * hh) * D < 1 << 16
