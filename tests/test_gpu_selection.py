"""GPU parity of the selection comparators and fidelity diagnostics ("Faster Than Flash" Sec. 4.5
Table 3, Sec. 5.1 Fig. 6, Sec. 3.2 Eq. 3 / Sec. 5.2 Fig. 5) against oracle/selection.py.

Bars: block min/max values and scan scores bit-exact; min/max bounds within 1e-4 and exact block
maxima within 2e-3 (fp32 sums against fp64); top-delta and top-k masks bit-exact on the same fp32
scores; top-p masks a valid ranked prefix whose length the fp64 oracle brackets within 1e-5 of
p; masked attention within 2e-3; top-delta on the scan scores followed by masked attention equal
bit for bit to the fused sparse decode.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import selection as S
from conftest import log
from helpers import DEV, assert_close, to_dev
from long_context_decoding_amd import ffd
from long_context_decoding_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-3, "f32": 1e-5}
CASES = [("bf16", 4, 64, 20 * 64 + 5), ("bf16", 1, 128, 9 * 128), ("f32", 2, 64, 12 * 64 + 33),
         ("bf16", 8, 64, 7 * 64 + 1),
         # padded groups and a group cut into two units of 8
         ("bf16", 3, 128, 11 * 128 + 7), ("f32", 7, 64, 13 * 64 + 9), ("bf16", 12, 64, 10 * 64)]


def setup(dtype, G, T, L, seed):
    Hkv = 2 if G <= 4 or G == 12 else 1
    w = W.small(f"sel_{dtype}_G{G}_T{T}_L{L}", B=2, Hq=G * Hkv, Hkv=Hkv, L=L, T=T, dtype=dtype,
                seed=seed, plant="powerlaw" if seed % 2 else "needles")
    q, K, V, _ = W.make_inputs(w)
    qd, Kd, Vd = to_dev(q), to_dev(K), to_dev(V)
    return w, q, K, V, qd, Kd, Vd


@pytest.mark.parametrize("dtype,G,T,L", CASES)
def test_scores_and_bounds(dtype, G, T, L):
    w, q, K, V, qd, Kd, Vd = setup(dtype, G, T, L, seed=G * 10 + T)
    nf = L // T
    Kq, sc = ffd.alloc_kq(Kd, T)
    ffd.quantize_k_append(Kd, 0, L, T, Kq, sc, seq_len=L)
    kmin, kmax = ffd.alloc_bounds(Kd, T)
    ffd.block_bounds(Kd, 0, L, T, kmin, kmax, seq_len=L)
    s_scan = ffd.block_scores(ffd.SCORE_SCAN, qd, Kd, T, L, Kq=Kq, scales=sc)
    s_bnd = ffd.block_scores(ffd.SCORE_BOUNDS, qd, Kd, T, L, kmin=kmin, kmax=kmax)
    s_ex = ffd.block_scores(ffd.SCORE_EXACT, qd, Kd, T, L)
    torch.cuda.synchronize()
    mn_d, mx_d = kmin.float().cpu().numpy(), kmax.float().cpu().numpy()
    s_scan, s_bnd, s_ex = s_scan.cpu().numpy(), s_bnd.cpu().numpy(), s_ex.cpu().numpy()
    Kq_o, sc_o = oracle.quantize_k(K, T)
    for b in range(w.B):
        for g in range(w.Hkv):
            mn, mx = S.block_bounds(K[b, g], T, nf)
            np.testing.assert_array_equal(mn_d[b, g, :nf], mn, err_msg=f"kmin b={b} g={g}")
            np.testing.assert_array_equal(mx_d[b, g, :nf], mx, err_msg=f"kmax b={b} g={g}")
        for h in range(w.Hq):
            g = h // w.G
            ref = oracle.scan_head(q[b, h], Kq_o[b, g], sc_o[b, g], nf, T)
            np.testing.assert_array_equal(s_scan[b, h], ref, err_msg=f"scan b={b} h={h}")
            mn, mx = S.block_bounds(K[b, g], T, nf)
            assert_close(s_bnd[b, h], S.bound_scores(q[b, h], mn, mx), 1e-4, f"bounds b={b} h={h}")
            assert_close(s_ex[b, h], S.exact_block_max(q[b, h], K[b, g], T, nf), TOL[dtype],
                         f"exact b={b} h={h}")
            assert (s_bnd[b, h] >= s_ex[b, h] - 1e-3).all(), "bound below the exact maximum"


@pytest.mark.parametrize("dtype,G,T,L", CASES)
def test_rules_on_identical_scores(dtype, G, T, L):
    w, q, K, V, qd, Kd, Vd = setup(dtype, G, T, L, seed=G + T)
    nf, nb = L // T, math.ceil(L / T)
    rng = np.random.default_rng(G * T)
    s = (rng.standard_normal((w.B, w.Hq, nf)) * 3).astype(np.float32)
    s[..., 5] = s[..., 3]  # ties
    sd = to_dev(s)
    pm = (rng.standard_normal((w.B, w.Hq)) * 3).astype(np.float32)
    for delta in (0.0, 1.0, 4.0, math.inf):
        got = ffd.select_blocks(ffd.SELECT_TOP_DELTA, sd, delta, T, L, w.Hkv).cpu().numpy()
        got_pm = ffd.select_blocks(ffd.SELECT_TOP_DELTA, sd, delta, T, L, w.Hkv,
                                   pseudo_max=to_dev(pm)).cpu().numpy()
        for b in range(w.B):
            for h in range(w.Hq):
                np.testing.assert_array_equal(got[b, h], S.select_top_delta(s[b, h], nf, nb, delta)[0])
                np.testing.assert_array_equal(got_pm[b, h],
                                              S.select_top_delta(s[b, h], nf, nb, delta, pm[b, h])[0])
    for k in (0, 1, 3, nf // 2, nf, nf + 5):
        got = ffd.select_blocks(ffd.SELECT_TOP_K, sd, k, T, L, w.Hkv).cpu().numpy()
        for b in range(w.B):
            for h in range(w.Hq):
                np.testing.assert_array_equal(got[b, h], S.select_top_k(s[b, h], nf, nb, k),
                                              err_msg=f"top-k {k}")
    for p in (1e-6, 0.3, 0.6, 0.9, 0.99, 1.0):
        got = ffd.select_blocks(ffd.SELECT_TOP_P, sd, p, T, L, w.Hkv).cpu().numpy()
        for b in range(w.B):
            for h in range(w.Hq):
                check_top_p(got[b, h], s[b, h], p, nf, nb)


def check_top_p(kept_row, s_row, p, nf, nb):
    """The kept full blocks, forced ones aside, are the n highest-ranked, and the fp64 oracle's
    cumulative mass brackets n: cum[n-1] >= p and cum[n-2] < p, within 1e-5."""
    kept = kept_row.astype(bool)
    n_o, order, cum = S.top_p_prefix(s_row, p)
    forced = S.forced_mask(nf, nb).astype(bool)
    rank_of = {j: i for i, j in enumerate(order)}
    ranks = [rank_of[j] for j in range(nf) if kept[j] and not forced[j]]
    n = 1 + max(ranks + [0])
    # forced blocks are kept anyway, so the prefix may extend over them unseen
    while n < nf and cum[n - 1] < p - 1e-5 and forced[order[n]]:
        n += 1
    assert all(kept[j] for j in order[:n]), "kept blocks are not a ranked prefix"
    assert cum[n - 1] >= p - 1e-5 and (n == 1 or cum[n - 2] < p + 1e-5), (p, n, n_o)
    assert kept[nf:].all() and kept[0] and kept[nf - 1]


def test_rank_rules_on_the_longest_rows():
    rng = np.random.default_rng(9)
    T, nf = 64, 16384
    L = nf * T
    s = (rng.standard_normal((1, 2, nf)) * 2).astype(np.float32)
    sd = to_dev(s)
    k = 1234
    got = ffd.select_blocks(ffd.SELECT_TOP_K, sd, k, T, L, 2).cpu().numpy()
    for h in range(2):
        np.testing.assert_array_equal(got[0, h], S.select_top_k(s[0, h], nf, nf, k))
    got = ffd.select_blocks(ffd.SELECT_TOP_P, sd, 0.5, T, L, 2).cpu().numpy()
    for h in range(2):
        check_top_p(got[0, h], s[0, h], 0.5, nf, nf)


@pytest.mark.parametrize("dtype,G,T,L", CASES)
def test_masked_attention_and_fused_equivalence(dtype, G, T, L):
    w, q, K, V, qd, Kd, Vd = setup(dtype, G, T, L, seed=3 * G + T)
    nf, nb = L // T, math.ceil(L / T)
    Kq, sc = ffd.alloc_kq(Kd, T)
    ffd.quantize_k_append(Kd, 0, L, T, Kq, sc, seq_len=L)
    s_scan = ffd.block_scores(ffd.SCORE_SCAN, qd, Kd, T, L, Kq=Kq, scales=sc)
    for delta in (0.5, 5.0):
        keep_sel = ffd.select_blocks(ffd.SELECT_TOP_DELTA, s_scan, delta, T, L, w.Hkv)
        o_m, l_m = ffd.decode_masked(qd, Kd, Vd, keep_sel, T, L)
        keep_f = torch.zeros_like(keep_sel)
        o_f, l_f = ffd.decode_sparse(qd, Kd, Vd, Kq, sc, delta, T, L, keep_mask=keep_f)
        torch.cuda.synchronize()
        assert torch.equal(keep_sel, keep_f), "top-delta on the scan scores differs from fused"
        # same kept set; the fused kernel may visit the kept blocks in another order, so the
        # two agree to rounding, not bit for bit
        assert_close(o_m.cpu().numpy(), o_f.cpu().numpy(), TOL[dtype], "masked vs fused out")
        assert_close(l_m.cpu().numpy(), l_f.cpu().numpy(), TOL[dtype], "masked vs fused lse")
    # an arbitrary mask (top-k on exact scores) against the oracle's attention over it
    s_ex = ffd.block_scores(ffd.SCORE_EXACT, qd, Kd, T, L)
    keep = ffd.select_blocks(ffd.SELECT_TOP_K, s_ex, max(1, nf // 4), T, L, w.Hkv)
    out, lse = ffd.decode_masked(qd, Kd, Vd, keep, T, L)
    torch.cuda.synchronize()
    keep, out, lse = keep.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()
    for b in range(w.B):
        for h in range(w.Hq):
            g = h // w.G
            o_ref, l_ref = oracle.attend_head(q[b, h], K[b, g], V[b, g], L, T, keep=keep[b, h])
            assert_close(out[b, h], o_ref, TOL[dtype], f"masked out b={b} h={h}")
            assert_close(lse[b, h], l_ref, TOL[dtype], f"masked lse b={b} h={h}")


def test_eq3_exact_pseudo_max_variant():
    """Eq. 3: the pseudo-max from the exact scores of the sink and local blocks.  The GPU's exact
    block maxima are fp32, so blocks within 1e-3 of the threshold may fall either way; every
    other decision matches the oracle, and mtilde never exceeds the true maximum."""
    w, q, K, V, qd, Kd, Vd = setup("bf16", 4, 64, 30 * 64, seed=5)
    T, L = 64, 30 * 64
    nf, nb = L // T, math.ceil(L / T)
    Kq, sc = ffd.alloc_kq(Kd, T)
    ffd.quantize_k_append(Kd, 0, L, T, Kq, sc, seq_len=L)
    s_scan = ffd.block_scores(ffd.SCORE_SCAN, qd, Kd, T, L, Kq=Kq, scales=sc)
    s_ex = ffd.block_scores(ffd.SCORE_EXACT, qd, Kd, T, L)
    pm = torch.maximum(s_ex[..., 0], s_ex[..., nf - 1]).contiguous()
    keep = ffd.select_blocks(ffd.SELECT_TOP_DELTA, s_scan, 5.0, T, L, w.Hkv, pseudo_max=pm)
    torch.cuda.synchronize()
    keep, s_scan_h, s_ex_h = keep.cpu().numpy(), s_scan.cpu().numpy(), s_ex.cpu().numpy()
    gaps = []
    for b in range(w.B):
        for h in range(w.Hq):
            g = h // w.G
            ex = S.exact_block_max(q[b, h], K[b, g], T, nf)
            mt = max(ex[0], ex[nf - 1])
            assert mt <= ex.max() + 1e-12
            gaps.append(ex.max() - mt)
            ref, _, theta = S.select_top_delta(s_scan_h[b, h], nf, nb, 5.0, np.float32(mt))
            diff = np.nonzero(ref != keep[b, h])[0]
            assert all(abs(float(s_scan_h[b, h, j]) - theta) <= 1e-3 for j in diff), diff
    log(f"Eq. 3 pseudo-max gap m - mtilde: max {max(gaps):.3f}, mean {np.mean(gaps):.3f}")
