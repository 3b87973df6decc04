"""Helpers shared by the GPU tests: upload seeded inputs, run the HIP path, run the oracle."""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
from long_context_decoding_amd import ffd
from long_context_decoding_amd import workloads as W

DEV = "cuda:0"
TOL = {"bf16": 2e-3, "f32": 1e-5}


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    """A device tensor as numpy; bf16 as its bit patterns (uint16), the oracle's convention."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def upload(w: W.Workload, q, K, V):
    return to_dev(q), to_dev(K), to_dev(V)


def gpu_quantize(w: W.Workload, Kd: torch.Tensor, tok_begin=0, tok_end=None, Kq=None, sc=None):
    if Kq is None:
        Kq, sc = ffd.alloc_kq(Kd, w.T)
    ffd.quantize_k_append(Kd, tok_begin, w.L if tok_end is None else tok_end, w.T, Kq, sc,
                          seq_len=w.L)
    return Kq, sc


def gpu_sparse(w: W.Workload, qd, Kd, Vd, Kq, sc, delta):
    keep = torch.full((w.B, w.Hq, w.n_blocks), 7, dtype=torch.uint8, device=DEV)
    out, lse = ffd.decode_sparse(qd, Kd, Vd, Kq, sc, delta, w.T, w.L, keep_mask=keep)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), keep.cpu().numpy()


def gpu_dense(w: W.Workload, qd, Kd, Vd):
    out, lse = ffd.decode_dense(qd, Kd, Vd, w.T, w.L)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def oracle_masks(w: W.Workload, q, Kq, sc, delta, heads=None, workers=16):
    """keep [B, Hq, n_blocks] from the oracle's scan + select, head by head (threads)."""
    keep = np.zeros((w.B, w.Hq, w.n_blocks), dtype=np.uint8)
    heads = heads or [(b, h) for b in range(w.B) for h in range(w.Hq)]

    def one(bh):
        b, h = bh
        g = h // w.G
        sb = oracle.scan_head(q[b, h], Kq[b, g], sc[b, g], w.n_full, w.T)
        k, _, _ = oracle.select_head(sb, w.n_full, w.n_blocks, delta)
        return bh, k

    with ThreadPoolExecutor(workers) as ex:
        for (b, h), k in ex.map(one, heads):
            keep[b, h] = k
    return keep


def oracle_attend(w: W.Workload, q, K, V, heads, keep=None, workers=16):
    """{(b, h): (out f64[d], lse)} for the sampled heads (dense if keep is None)."""
    def one(bh):
        b, h = bh
        g = h // w.G
        kp = None if keep is None else keep[b, h]
        return bh, oracle.attend_head(q[b, h], K[b, g], V[b, g], w.L, w.T, kp)

    with ThreadPoolExecutor(workers) as ex:
        return dict(ex.map(one, heads))


def sample_heads(w: W.Workload, n: int, seed: int = 0):
    rng = np.random.default_rng(seed)
    all_h = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    if len(all_h) <= n:
        return all_h
    idx = rng.choice(len(all_h), size=n, replace=False)
    return [all_h[i] for i in sorted(idx)]


def assert_close(got, ref, tol, what):
    err = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    bad = ~(err <= tol)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(np.isnan(err), np.inf, err)), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} values off, max err {np.nanmax(err):.3g} "
                             f"at {i} (got {np.asarray(got)[i]}, ref {np.asarray(ref)[i]}), "
                             f"tol {tol}")
