"""Pins for the oracle's low-bit key quantizer.

"Faster Than Flash" App. A, Eqs. 5-7 define a symmetric mid-rise quantizer (no zero codeword):
s = max|x| / 1.5 and x_q = nearest codeword of x / s in {-1.5, -0.5, +0.5, +1.5}.  The oracle
generalizes it to 2^bits levels (value (u - (2^bits - 1)/2) * s).  These tests pin it to the
definition by brute force (argmin over the whole codebook), to the 2-bit worked example, and to
closed forms; none of them re-types the oracle's floor-based formula.
"""
from pathlib import Path

import numpy as np
import pytest
import torch

import oracle
from long_context_decoding_amd import workloads as W

GOLDEN = Path(__file__).resolve().parent / "golden"


def codebook(bits):
    half = (2 ** bits - 1) / 2
    return np.arange(2 ** bits, dtype=np.float64) - half


def brute_force_codes(x, s, bits):
    """Eq. 7 by exhaustive search: index of the codeword nearest to x/s (fp64)."""
    cb = codebook(bits)
    y = np.asarray(x, np.float64) / s
    dist = np.abs(y[:, None] - cb[None, :])
    best = dist.min(axis=1)
    # all codewords within a hair of the minimum (ties and near-ties)
    cand = dist <= best[:, None] + 1e-6
    return dist.argmin(axis=1), cand


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("seed", range(6))
def test_codes_are_nearest_codeword(bits, seed):
    rng = np.random.default_rng(seed)
    n = 257
    x = (rng.standard_normal(n) * rng.uniform(0.01, 30)).astype(np.float32)
    codes, s = oracle.quantize_channel(x, bits)
    assert s == np.float32(np.float32(np.abs(x).max()) / np.float32((2 ** bits - 1) / 2))
    ref, cand = brute_force_codes(x, s, bits)
    ok = cand[np.arange(n), codes]
    assert ok.all(), f"codes not nearest at {np.nonzero(~ok)[0][:5]}"
    # away from ties the choice is unique
    unique = cand.sum(axis=1) == 1
    assert (codes[unique] == ref[unique]).all()


@pytest.mark.parametrize("bits", [2, 4])
def test_boundaries_go_to_upper_codeword(bits):
    """Values exactly on a bin boundary (integer multiples of s) take the upper codeword."""
    half = (2 ** bits - 1) / 2
    s = 0.25  # power of two: x / s exact
    amax = half * s
    bounds = np.arange(-(2 ** (bits - 1) - 1), 2 ** (bits - 1), dtype=np.float64)  # interior
    x = np.concatenate([[amax], bounds * s]).astype(np.float32)
    codes, s_out = oracle.quantize_channel(x, bits)
    assert s_out == s
    cb = codebook(bits)
    for xi, ci in zip(x[1:], codes[1:]):
        y = xi / s
        assert cb[ci] == y + 0.5, (xi, ci)


def test_app_a_worked_example():
    rows = [l.split() for l in (GOLDEN / "appA_2bit_worked_example.txt").read_text().splitlines()
            if l.strip() and not l.startswith("#")]
    tab = np.array(rows, dtype=np.float64)
    x = tab[:, 0].astype(np.float32)
    codes, s = oracle.quantize_channel(x, 2)
    assert abs(s - 0.8) < 1e-7
    assert (codes == tab[:, 3].astype(int)).all()
    recon = codebook(2)[codes] * s
    np.testing.assert_allclose(recon, tab[:, 4], atol=1e-6)
    np.testing.assert_allclose(codebook(2)[codes], tab[:, 2])


@pytest.mark.parametrize("bits", [2, 4])
def test_closed_forms(bits):
    rng = np.random.default_rng(7)
    x = rng.standard_normal(64).astype(np.float32)
    i_max, i_min = 5, 9
    x[i_max] = 3.0
    x[i_min] = -3.0
    codes, s = oracle.quantize_channel(x, bits)
    assert codes[i_max] == 2 ** bits - 1 and codes[i_min] == 0
    recon = codebook(bits)[codes] * s
    err = np.abs(recon - x.astype(np.float64))
    assert (err <= s / 2 * (1 + 2 ** -14)).all()
    # a zero channel reconstructs to zero
    z, s0 = oracle.quantize_channel(np.zeros(16, np.float32), bits)
    assert s0 == 0.0 and (codebook(bits)[z] * s0 == 0).all()
    # sign symmetry away from boundaries
    y = rng.uniform(-1, 1, 200).astype(np.float32)
    y[0] = 1.0
    c1, s1 = oracle.quantize_channel(y, bits)
    c2, s2 = oracle.quantize_channel(-y, bits)
    cb = codebook(bits)
    interior = np.abs(y / s1 - np.round(y / s1)) > 1e-4
    assert s1 == s2
    assert (cb[c1][interior] == -cb[c2][interior]).all()


def torch_bf16_bits(x):
    """bf16 bit patterns of float32 values by torch's CPU conversion (round to nearest, ties to
    even): an independent implementation of the scales' storage rounding."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_scale_storage_rounding():
    """The block scales are stored as bf16, rounded to nearest with ties to even."""
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(4096).astype(np.float32) * np.float32(3.0),
        np.exp(rng.uniform(-80, 80, 4096)).astype(np.float32),
        # exact ties between two bf16 values (lower 16 bits 0x8000), both parities of the kept
        # bit, a tie that carries into the next binade, the largest finite value (rounds to
        # infinity), subnormals, zero and infinity
        np.array([0x3F808000, 0x3F818000, 0x3FFF8000, 0x7F7FFFFF, 0x7F7F7FFF, 0x00000001,
                  0x00018000, 0x00028000, 0x00000000, 0x7F800000],
                 dtype=np.uint32).view(np.float32),
    ])
    got = oracle.round_bf16(x)
    assert (got == torch_bf16_bits(x)).all()
    assert got[-10:].tolist() == [0x3F80, 0x3F82, 0x4000, 0x7F80, 0x7F7F, 0x0000, 0x0002,
                                  0x0002, 0x0000, 0x7F80]
    nan = oracle.round_bf16(np.array([np.nan], np.float32))[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x007F) != 0


def test_quantize_k_packing_and_blocks():
    """Kq nibble order, per-(block, channel) scales (stored as bf16) and the append window."""
    rng = np.random.default_rng(3)
    T, d, L_cap = 64, 128, 5 * 64
    K32 = rng.standard_normal((1, 2, L_cap, d)).astype(np.float32)
    K = W.f32_to_bf16_bits(K32)
    Kq, sc = oracle.quantize_k(K, T)
    Kv = W.bf16_bits_to_f32(K)
    for g in range(2):
        for j in range(L_cap // T):
            for c in (0, 1, 2, 77, 127):
                codes, s = oracle.quantize_channel(Kv[0, g, j * T:(j + 1) * T, c], 4)
                assert sc[0, g, j, c] == torch_bf16_bits(np.array([s]))[0]
                byte = Kq[0, g, j * T:(j + 1) * T, c // 2]
                got = (byte >> 4) if c % 2 else (byte & 15)
                assert (got == codes).all()
    # append window: only blocks whose last token lies in [tok_begin, tok_end)
    Kq2 = np.full_like(Kq, 0xAB)
    sc2 = np.full_like(sc, 0xFFFF)
    oracle.quantize_k(K, T, tok_begin=2 * T - 1, tok_end=4 * T - 1, Kq=Kq2, scales=sc2)
    for j in range(L_cap // T):
        written = j in (1, 2)
        blk = slice(j * T, (j + 1) * T)
        assert (Kq2[:, :, blk] == Kq[:, :, blk]).all() == written
        assert (Kq2[:, :, blk] == 0xAB).all() == (not written)
        assert (sc2[:, :, j] == sc[:, :, j]).all() == written
    # incremental appends, one token at a time, give the one-shot bytes
    Kq3 = np.zeros_like(Kq)
    sc3 = np.zeros_like(sc)
    for t in range(L_cap):
        oracle.quantize_k(K, T, tok_begin=t, tok_end=t + 1, Kq=Kq3, scales=sc3)
    assert (Kq3 == Kq).all() and (sc3 == sc).all()
