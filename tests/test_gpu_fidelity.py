"""Fidelity of MALA against the screening-disabled reference ([MALA] Sec. 3,
"Operator Fidelity Across Context Lengths", App. C.3), anchored to fp64, and
the matched-work allocation study's evaluation ([MALA] Sec. 3 Table 1, App.
C.2) run on the GPU and checked against the oracle.

The fidelity suite of bench.py (--sweep) compares the MALA and dense bf16
GPU outputs, which mixes the terms MALA skips with the two kernels'
rounding. Here the same quantities are computed twice on identical inputs:

  * in the fp64 oracle, MALA against dense: the omitted mass per query row
    eps = 1 - exp(z_mala - z_dense) and the output's relative L2 error per
    row, from the skipped terms alone; and the gradients' relative L2 per
    head with a Rademacher dO probe (App. C.3);
  * on the GPU, the same figures from the MALA and dense kernels.

Assertions: the oracle's figures obey Proposition 1 (eps <= tau / (1 + tau)
per row, output error <= 2 tau / (1 + tau) max |v| / |o|); the GPU's omitted
mass equals the oracle's up to the LSE rounding of the two kernels
(|delta eps| <= 2 * 1e-3 (1 - eps)); and the GPU's MALA-dense output difference
stays within the oracle's skipped-term difference plus the two kernels'
rounding (the fp64 bound of tests/parity.py applied to each). Both columns
are printed, so the skipped-term error and the rounding error are read apart.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from parity import LSE_TOL, bits_to_f64, bits_to_gpu, gpu_to_f64

pytestmark = pytest.mark.gpu


def mala():
    import adaptive_softmax_attention_amd as m
    m.lib()
    return m


def _gpu_fwd_bwd(inp, do_bits, tau, dense):
    m = mala()
    q, k, v = (bits_to_gpu(inp[x]) for x in ("q", "k", "v"))
    do = bits_to_gpu(do_bits)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(m.mala_bwd_workspace_bytes(q, k), dtype=torch.uint8, device="cuda")
    if dense:
        m.fullattn_fwd(q, k, v, o, lse)
        m.fullattn_bwd(q, k, v, o, lse, do, dq, dk, dv, ws)
    else:
        m.mala_fwd(q, k, v, o, lse, tau=tau)
        m.mala_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, tau=tau)
    torch.cuda.synchronize()
    return {"o": gpu_to_f64(o), "lse": lse.cpu().numpy().astype(np.float64),
            "dq": gpu_to_f64(dq), "dk": gpu_to_f64(dk), "dv": gpu_to_f64(dv)}


def _row_rel(a, b):
    return np.linalg.norm(a - b, axis=-1) / np.maximum(np.linalg.norm(b, axis=-1), 1e-300)


def _head_rel(a, b):
    B, H = a.shape[:2]
    x, y = a.reshape(B, H, -1), b.reshape(B, H, -1)
    return (np.linalg.norm(x - y, axis=-1) / np.linalg.norm(y, axis=-1)).ravel()


@pytest.mark.parametrize("length", [1024, 4096])
def test_fidelity_against_screening_disabled_fp64_anchor(length):
    w = W.cfg3(length)
    inp = W.peaked(w.spec)
    tau = w.tau
    # Rademacher probe dO (exact in bf16), as in App. C.3
    signs = np.random.default_rng(7000 + length).integers(0, 2, size=inp["do"].shape) * 2 - 1
    do_bits = W.f32_to_bf16_bits(signs.astype(np.float32))
    q, k, v = (bits_to_f64(inp[x]) for x in ("q", "k", "v"))
    do = bits_to_f64(do_bits)
    # --- fp64: MALA against dense, the skipped terms alone ---
    fm = O.mala_fwd(q, k, v, tau, want_margin=False)
    od, zd = O.dense_fwd(q, k, v)
    bm = O.mala_bwd(q, k, v, fm["o"], fm["lse"], do, tau, want_margin=False)
    gd = O.dense_bwd(q, k, v, do)
    eps_x = -np.expm1(fm["lse"] - zd)
    rl2_x = _row_rel(fm["o"], od)
    # --- GPU: the MALA and dense kernels on the same inputs ---
    gm = _gpu_fwd_bwd(inp, do_bits, tau, dense=False)
    gdn = _gpu_fwd_bwd(inp, do_bits, tau, dense=True)
    eps_g = -np.expm1(gm["lse"] - gdn["lse"])
    rl2_g = _row_rel(gm["o"], gdn["o"])

    # Proposition 1 in fp64: per row, eps <= tau / (1 + tau), and the output
    # moves by at most 2 tau / (1 + tau) max_k |v_k| (here per row, against
    # the row's own norm)
    assert (eps_x >= -1e-12).all() and (eps_x <= tau / (1 + tau) + 1e-12).all()
    G = q.shape[1] // k.shape[1]
    vmax = np.repeat(np.linalg.norm(v, axis=-1).max(axis=2), G, axis=1)[:, :, None]
    assert (np.linalg.norm(fm["o"] - od, axis=-1) <= 2 * tau / (1 + tau) * vmax + 1e-9).all()
    # the GPU's omitted mass is the oracle's up to the two kernels' LSE rounding
    assert (np.abs(eps_g - eps_x) <= 2 * LSE_TOL * (1 - eps_x) + 1e-12).all()
    # the GPU's MALA - dense difference: the skipped part plus each kernel's
    # rounding (each output within 2^-6 (M + |O|) + 1e-4 of its fp64 value,
    # M <= max |v| per column since the weights sum to 1)
    vcol = np.repeat(np.abs(v).max(axis=2), G, axis=1)[:, :, None, :]
    round_bound = 2 * np.linalg.norm(2.0 ** -6 * (vcol + np.abs(od)) + 1e-4, axis=-1)
    gap = np.linalg.norm((gm["o"] - gdn["o"]) - (fm["o"] - od), axis=-1)
    assert (gap <= round_bound).all()

    names = ("dq", "dk", "dv")
    rel_x = [_head_rel(bm[n], gd[i]) for i, n in enumerate(names)]
    rel_g = [_head_rel(gm[n], gdn[n]) for n in names]
    p95 = lambda a: float(np.percentile(a, 95))
    print(f"\n[fidelity N={length}, tau={tau}] per query row; fp64 oracle (skipped terms only) | "
          f"GPU kernels (skipped terms + rounding)", flush=True)
    print(f"  omitted mass   mean {eps_x.mean():.3e} P95 {p95(eps_x):.3e} | "
          f"mean {eps_g.mean():.3e} P95 {p95(eps_g):.3e}", flush=True)
    print(f"  output rel L2  mean {rl2_x.mean():.3e} P95 {p95(rl2_x):.3e} | "
          f"mean {rl2_g.mean():.3e} P95 {p95(rl2_g):.3e}", flush=True)
    for n, ax, ag in zip(names, rel_x, rel_g):
        print(f"  {n} rel L2 per head  mean {ax.mean():.3e} P95 {p95(ax):.3e} | "
              f"mean {ag.mean():.3e} P95 {p95(ag):.3e}", flush=True)
    # the skipped terms move the gradients by far less than bf16 rounding
    # does: the GPU figure is dominated by rounding, the fp64 one isolates
    # skipping (both are reported; the fp64 one must stay small)
    for ax in rel_x:
        assert ax.max() < 1e-2


def test_matched_work_evaluation_on_gpu_matches_oracle():
    """The matched-work study's evaluation at a reduced size (2 inputs x 4
    query heads, 2K, d 128, query gains that differ per head), run on the GPU
    with the MALA kernel's own decisions: the omitted mass per row and the
    output error per block of every policy equal the oracle's forward with
    that policy's tiles forced, against the oracle's dense forward."""
    import bench
    m = mala()
    spec = W.Spec(611, 2, 4, 1, 2048, 128, 3.0, 16, local_bias=True, head_gain=(0.5, 2.0))
    inp = W.peaked(spec, want_do=False)
    tau, T = 1.0, 64
    qg, kg, vg = (bits_to_gpu(inp[x]) for x in ("q", "k", "v"))
    B, H, N, d = qg.shape
    Tr = N // T
    o = torch.empty_like(qg)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dec = torch.full((B, H, Tr, Tr), 255, dtype=torch.uint8, device="cuda")
    m.mala_fwd(qg, kg, vg, o, lse, tau=tau, stats=m.Stats(decisions=dec))
    torch.cuda.synchronize()
    legal = torch.ones(Tr, Tr, dtype=torch.bool, device="cuda").tril()
    assert bool(((dec != 255) == legal).all())
    keep_mala = dec == 1
    n = keep_mala.sum(-1).cpu().numpy()
    alloc = {k_: torch.from_numpy(a).cuda() for k_, a in bench.matched_allocations(n).items()}
    scale = float(np.float32(1.0 / math.sqrt(d)))
    q, k, v = (bits_to_f64(inp[x]) for x in ("q", "k", "v"))
    od, zd = O.dense_fwd(q, k, v, scale=scale)
    checked = 0
    for r in range(B):
        for h in range(H):
            qf, kf, vf = qg[r, h].float(), kg[r, 0].float(), vg[r, 0].float()
            p, row, blk = bench.reference_masses(qf, kf, scale, T)
            oref = p @ vf
            masks = {"mala": keep_mala[r, h]}
            for name, a in alloc.items():
                masks[name] = bench.top_tiles(blk, a[r, h], legal)
            for name, keep in masks.items():
                eps, eps_blk, err = bench.policy_errors(p, oref, row, vf, keep, T)
                force = np.full((B, H, Tr, Tr), -1, dtype=np.int8)
                kn = keep.cpu().numpy()
                force[r, h] = np.where(np.tril(np.ones((Tr, Tr), dtype=bool)), kn, -1)
                f = O.mala_fwd(q, k, v, tau, scale=scale, force=force,
                               sel=[(r, h, i) for i in range(Tr)], want_margin=False)
                want_eps = -np.expm1(f["lse"][r, h] - zd[r, h])
                e = eps.cpu().numpy().astype(np.float64)
                # fp32 evaluation of the dense reference against fp64
                assert np.all(np.abs(e - want_eps) <= 1e-5 + 1e-3 * want_eps), name
                diff = (f["o"][r, h] - od[r, h]).reshape(Tr, T, d)
                ref = od[r, h].reshape(Tr, T, d)
                want_err = np.sqrt((diff ** 2).sum((1, 2)) / (ref ** 2).sum((1, 2)))
                ge = err.cpu().numpy().astype(np.float64)
                assert np.all(np.abs(ge - want_err) <= 1e-4 + 1e-2 * want_err), name
                checked += 1
    assert checked == B * H * 4
