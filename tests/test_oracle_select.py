"""Pins for the oracle's pseudo-max and top-delta block selection.

"Faster Than Flash" Sec. 3.2: Eq. 1 keeps tokens whose score is within delta of the maximum;
Eq. 3 replaces the maximum by a pseudo-max over sink and local tokens; Alg. 1 applies the test
per block to the block's estimated maximum.  Pins: closed forms (delta = +inf keeps everything,
delta = 0 keeps exactly the blocks at or above the pseudo-max), monotonicity in delta, the forced
blocks, and brute-force enumeration of the breakpoints delta_j = mtilde - shat_j on tiny inputs.
"""
import numpy as np
import pytest

import oracle
from long_context_decoding_amd import workloads as W


def test_pseudo_max_is_max_of_sink_and_local():
    sb = np.array([1.0, 9.0, 2.5, -3.0, 4.0, 0.5], np.float32)
    keep, mt, th = oracle.select_head(sb, n_full=6, n_blocks=6, delta=1.0)
    assert mt == 1.0 and th == 0.0  # max(block 0 = 1.0, last full block = 0.5)
    np.testing.assert_array_equal(keep, [1, 1, 1, 0, 1, 1])
    # with a partial tail block: local = last *full* block, tail forced
    keep, mt, th = oracle.select_head(sb, n_full=6, n_blocks=7, delta=0.25)
    assert mt == 1.0
    np.testing.assert_array_equal(keep, [1, 1, 1, 0, 1, 1, 1])


def test_degenerate_block_counts():
    keep, mt, th = oracle.select_head(np.zeros(0, np.float32), n_full=0, n_blocks=1, delta=0.0)
    assert keep.tolist() == [1] and np.isnan(mt)
    keep, mt, _ = oracle.select_head(np.array([3.0], np.float32), n_full=1, n_blocks=2, delta=0.0)
    assert keep.tolist() == [1, 1] and mt == 3.0
    keep, _, _ = oracle.select_head(np.array([3.0, -50.0], np.float32), 2, 2, 0.0)
    assert keep.tolist() == [1, 1]  # both forced


@pytest.mark.parametrize("seed", range(5))
def test_closed_forms_and_monotone(seed):
    rng = np.random.default_rng(seed)
    n = 40
    sb = (rng.standard_normal(n) * 3).astype(np.float32)
    keep_inf, mt, th = oracle.select_head(sb, n, n, float("inf"))
    assert keep_inf.all() and th == -np.inf
    keep0, mt, _ = oracle.select_head(sb, n, n, 0.0)
    expect0 = (sb >= mt).astype(np.uint8)
    expect0[0] = expect0[-1] = 1
    np.testing.assert_array_equal(keep0, expect0)
    prev = keep0
    for delta in np.linspace(0, 20, 81)[1:]:
        k, _, _ = oracle.select_head(sb, n, n, float(delta))
        assert (k >= prev).all(), "selection must be monotone in delta"
        assert k[0] == 1 and k[-1] == 1
        prev = k


@pytest.mark.parametrize("seed", range(8))
def test_brute_force_breakpoints_tiny(seed):
    """Tiny inputs (d=8, T=4, up to 8 blocks): for each block the mask flips exactly at
    delta_j = mtilde - shat_j, found by enumerating the sorted breakpoints."""
    rng = np.random.default_rng(seed)
    d, T = 8, 4
    n = int(rng.integers(3, 9))
    K = rng.standard_normal((1, 1, n * T, d)).astype(np.float32) * 2
    Kq, sc = oracle.quantize_k(K, T)
    q = rng.standard_normal(d).astype(np.float32)
    sb = oracle.scan_head(q, Kq[0, 0], sc[0, 0], n, T)
    mt = max(sb[0], sb[n - 1])
    bps = sorted(set(float(mt) - float(x) for x in sb))
    probes = [0.0]
    for b in bps:
        probes += [b - 1e-3, b + 1e-3]
    for delta in probes:
        if delta < 0:
            continue
        k, m2, _ = oracle.select_head(sb, n, n, delta)
        assert m2 == mt
        for j in range(n):
            forced = j == 0 or j == n - 1
            brute = forced or (float(mt) - float(sb[j]) <= delta)
            assert bool(k[j]) == brute, (delta, j)


def test_decode_keep_mask_matches_stagewise():
    """The batch driver's mask equals scan + select applied head by head."""
    w = W.small("t", B=2, Hq=8, Hkv=2, L=7 * 64 + 17, T=64, seed=3)
    q, K, V, _ = W.make_inputs(w)
    Kq, sc = oracle.quantize_k(K, w.T)
    res = oracle.decode(q, K, V, w.L, w.T, delta=2.0, Kq=Kq, scales=sc, want_shat=True)
    for b in range(2):
        for h in range(8):
            g = h // 4
            sb = oracle.scan_head(q[b, h], Kq[b, g], sc[b, g], w.n_full, w.T)
            np.testing.assert_array_equal(res["shat"][b, h], sb)
            keep, mt, _ = oracle.select_head(sb, w.n_full, w.n_blocks, 2.0)
            np.testing.assert_array_equal(res["keep"][b, h], keep)
            assert res["mtilde"][b, h] == mt
    assert res["keep"][:, :, -1].all()  # the ragged tail is always kept
