"""Running-max variant of top-delta on the GPU (ffd_decode_sparse_running; "Faster Than Flash"
Sec. 1 Fig. 1: a threshold relative to the local max; Alg. 1: the pseudo-max it starts from).

- masks equal the oracle's select_running on the oracle's own scan estimates and pseudo-max,
  bit for bit, for windows from 1 block to more than the sequence and for ragged lengths;
- out and lse equal the oracle's exact attention over that mask within 2e-3 (bf16) / 1e-5 (fp32);
- at a 32K-token size (512 blocks, so windows of at least 2 blocks: at most 256 windows): every
  window keeps a subset of ffd_decode_sparse's Alg. 1 mask (the running maximum never lies below
  the pseudo-max), and a window of more than 256 blocks is rejected.
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
CASES = [("bf16", 4, 64, 20 * 64 + 5, 2), ("bf16", 1, 128, 9 * 128, 1), ("f32", 2, 64, 12 * 64 + 33, 2),
         ("bf16", 8, 64, 7 * 64 + 1, 1),
         # padded groups and a group cut into two units of 8
         ("bf16", 5, 64, 17 * 64 + 3, 2), ("f32", 3, 128, 8 * 128 + 1, 1), ("bf16", 16, 64, 9 * 64, 1)]


@pytest.mark.parametrize("dtype,G,T,L,Hkv", CASES)
def test_running_matches_oracle(dtype, G, T, L, Hkv):
    w = W.small(f"run_{dtype}_G{G}_T{T}_L{L}", B=2, Hq=G * Hkv, Hkv=Hkv, L=L, T=T, dtype=dtype,
                seed=G * 7 + T, plant="needles")
    q, K, V, _ = W.make_inputs(w)
    qd, Kd, Vd = to_dev(q), to_dev(K), to_dev(V)
    nf, nb = L // T, math.ceil(L / T)
    Kq, sc = ffd.alloc_kq(Kd, T)
    ffd.quantize_k_append(Kd, 0, L, T, Kq, sc, seq_len=L)
    Kq_o, sc_o = oracle.quantize_k(K, T)
    ref = oracle.decode(q, K, V, L, T, 5.0, Kq=Kq_o, scales=sc_o, want_shat=True)
    for delta in (0.5, 2.0, 5.0):
        for window in (1, 3, 8, nb, nb + 5):
            log(f"running {dtype} G={G} T={T} L={L} delta={delta} window={window}")
            keep = torch.full((w.B, w.Hq, nb), 7, dtype=torch.uint8, device=DEV)
            out, lse = ffd.decode_sparse_running(qd, Kd, Vd, Kq, sc, delta, T, window, L,
                                                 keep_mask=keep)
            torch.cuda.synchronize()
            keep, out, lse = keep.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()
            for b in range(w.B):
                for h in range(w.Hq):
                    want = S.select_running(ref["shat"][b, h], float(ref["mtilde"][b, h]), nf, nb,
                                            delta, window)
                    np.testing.assert_array_equal(keep[b, h], want,
                                                  err_msg=f"b={b} h={h} delta={delta} W={window}")
                    g = h // w.G
                    o_ref, l_ref = oracle.attend_head(q[b, h], K[b, g], V[b, g], L, T, keep=want)
                    assert_close(out[b, h], o_ref, TOL[dtype], f"out b={b} h={h} W={window}")
                    assert_close(lse[b, h], l_ref, TOL[dtype], f"lse b={b} h={h} W={window}")


def test_running_subset_at_32k():
    w = W.WORKLOADS["gqa4_32k_sink_needles"]
    q, K, V, _ = W.make_inputs(w)
    qd, Kd, Vd = to_dev(q), to_dev(K), to_dev(V)
    Kq, sc = ffd.alloc_kq(Kd, w.T)
    ffd.quantize_k_append(Kd, 0, w.L, w.T, Kq, sc, seq_len=w.L)
    keep_a = torch.zeros((w.B, w.Hq, w.n_blocks), dtype=torch.uint8, device=DEV)
    ffd.decode_sparse(qd, Kd, Vd, Kq, sc, 5.0, w.T, w.L, keep_mask=keep_a)
    for window in (2, 4, 16, 64, 256):
        keep_r = torch.zeros_like(keep_a)
        ffd.decode_sparse_running(qd, Kd, Vd, Kq, sc, 5.0, w.T, window, w.L, keep_mask=keep_r)
        torch.cuda.synchronize()
        a, r = keep_a.cpu().numpy().astype(bool), keep_r.cpu().numpy().astype(bool)
        log(f"32K window {window}: keep {r.mean():.4f} vs Alg. 1 {a.mean():.4f}")
        assert not (r & ~a).any(), f"window {window} keeps a block Alg. 1 drops"
        assert r.sum() > 0
    with pytest.raises(ffd.FFDError):
        ffd.decode_sparse_running(qd, Kd, Vd, Kq, sc, 5.0, w.T, 257, w.L)
