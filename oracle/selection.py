"""Oracle (test infrastructure, CPU only) for the block-selection comparators of "Faster Than
Flash": Quest-style min/max block bounds, exact block maxima, and the selection rules top-delta,
top-k and top-p on per-block scores (Sec. 3.2 Eqs. 1 and 3; Sec. 4.5 Table 3; Sec. 5.1 Fig. 6;
Sec. 5.2 Fig. 5).  Plain numpy, fp64 unless a rule's decision is defined in fp32.  Nothing here
is used by the HIP path; only tests, the smoke check and the bench's CPU baseline import oracle/.

Readings (the pages name these rules but do not define them at block granularity):
  - a block's score is one of: the scan estimate of its largest score (Alg. 1), a Quest-style
    upper bound from per-channel min/max metadata, or its exact largest score q.k / sqrt(d);
  - every rule keeps the forced blocks (block 0, the last full block, a partial tail), as top-delta
    does, and ranks the full blocks by score, ties going to the lower block index;
  - top-k keeps the k highest-ranked full blocks;
  - top-p treats each full block's score as the logit of its share of the attention mass,
    pi_j = exp(s_j - max s) / sum_i exp(s_i - max s), and keeps the shortest ranked prefix whose
    mass reaches p (all full blocks when rounding keeps the total just below p);
  - top-delta is Eq. 1 with a pseudo-max: theta = RN32(mtilde - delta), keep s_j >= theta, with
    mtilde = max(s_0, s_{nf-1}) (Alg. 1) or a given value (Eq. 3 with exact scores);
  - the running-max variant of top-delta (a threshold "from the local max", Sec. 1 Fig. 1, kept
    local to a window of consecutive blocks): the blocks are cut into windows of W blocks; in each
    window, in increasing block order, a non-forced full block j is kept iff
    s_j >= RN32(M - delta), where M starts at the Alg. 1 pseudo-max and, after block j is judged,
    becomes max(M, s_j).
"""
from __future__ import annotations

import math

import numpy as np

from . import to_f32


def forced_mask(n_full: int, n_blocks: int) -> np.ndarray:
    """Blocks every rule keeps: 0, the last full block and a partial tail (Alg. 1's sink and
    local sets, Sec. 3.2)."""
    keep = np.zeros(n_blocks, dtype=np.uint8)
    if n_blocks:
        keep[0] = 1
        keep[max(n_full - 1, 0):] = 1
    return keep


def block_bounds(K_slice: np.ndarray, T: int, n_full: int):
    """Per full block and channel: min and max of the keys over its T tokens (Quest's page
    metadata with a page of T tokens) -> (mn, mx) float32 [n_full, d]."""
    K = to_f32(K_slice)[: n_full * T]
    d = K.shape[1]
    mn = np.empty((n_full, d), dtype=np.float32)
    mx = np.empty((n_full, d), dtype=np.float32)
    for j in range(n_full):
        blk = K[j * T:(j + 1) * T]
        mn[j] = blk.min(axis=0)
        mx[j] = blk.max(axis=0)
    return mn, mx


def bound_scores(qh: np.ndarray, mn: np.ndarray, mx: np.ndarray) -> np.ndarray:
    """Quest-style upper bound of each block's largest score:
    sum_c max(q_c mn_c, q_c mx_c) / sqrt(d), in fp64."""
    q = to_f32(qh).astype(np.float64)
    d = q.shape[0]
    lo = q[None, :] * mn.astype(np.float64)
    hi = q[None, :] * mx.astype(np.float64)
    return np.maximum(lo, hi).sum(axis=1) / math.sqrt(d)


def exact_block_max(qh: np.ndarray, K_slice: np.ndarray, T: int, n_full: int) -> np.ndarray:
    """Exact largest score of each full block, max_t q.k_t / sqrt(d), in fp64 (Eq. 1's s_ij)."""
    q = to_f32(qh).astype(np.float64)
    K = to_f32(K_slice)[: n_full * T].astype(np.float64)
    d = q.shape[0]
    out = np.empty(n_full, dtype=np.float64)
    for j in range(n_full):
        out[j] = (K[j * T:(j + 1) * T] @ q).max() / math.sqrt(d)
    return out


def ranked(scores: np.ndarray) -> list[int]:
    """Full blocks by decreasing score, ties to the lower index."""
    s = np.asarray(scores, dtype=np.float64)
    return sorted(range(s.shape[0]), key=lambda j: (-s[j], j))


def select_top_delta(scores: np.ndarray, n_full: int, n_blocks: int, delta: float,
                     pseudo_max: float | None = None):
    """Eq. 1 with a pseudo-max, decided in fp32 -> (keep u8[n_blocks], mtilde, theta)."""
    s = np.asarray(scores, dtype=np.float32)
    keep = forced_mask(n_full, n_blocks)
    if n_full == 0:
        return keep, float("-inf"), float("-inf")
    mt = np.float32(max(s[0], s[n_full - 1])) if pseudo_max is None else np.float32(pseudo_max)
    theta = np.float32(mt - np.float32(delta))  # one fp32 subtraction, round to nearest
    for j in range(n_full):
        if s[j] >= theta:
            keep[j] = 1
    return keep, float(mt), float(theta)


def select_top_k(scores: np.ndarray, n_full: int, n_blocks: int, k: int) -> np.ndarray:
    """The k highest-ranked full blocks, plus the forced blocks (Table 3's top-k)."""
    keep = forced_mask(n_full, n_blocks)
    for j in ranked(np.asarray(scores)[:n_full])[: max(0, min(k, n_full))]:
        keep[j] = 1
    return keep


def top_p_prefix(scores: np.ndarray, p: float):
    """Length of the shortest ranked prefix whose mass reaches p, and the cumulative masses."""
    s = np.asarray(scores, dtype=np.float64)
    order = ranked(s)
    w = np.exp(s[order] - s[order[0]])
    cum = np.cumsum(w) / w.sum()
    n = int(np.searchsorted(cum, p, side="left")) + 1
    return min(n, s.shape[0]), order, cum


def select_top_p(scores: np.ndarray, n_full: int, n_blocks: int, p: float) -> np.ndarray:
    """The shortest ranked prefix of full blocks holding mass >= p, plus the forced blocks
    (Table 3's top-p at block granularity)."""
    keep = forced_mask(n_full, n_blocks)
    if n_full == 0:
        return keep
    n, order, _ = top_p_prefix(np.asarray(scores)[:n_full], p)
    for j in order[:n]:
        keep[j] = 1
    return keep


def select_running(scores: np.ndarray, mtilde: float, n_full: int, n_blocks: int, delta: float,
                   window: int) -> np.ndarray:
    """Top-delta against a running maximum local to each window of `window` blocks (the module
    docstring's reading), decided in fp32 -> keep u8[n_blocks]."""
    s = np.asarray(scores, dtype=np.float32)
    forced = forced_mask(n_full, n_blocks)
    keep = forced.copy()
    dl = np.float32(delta)
    for w0 in range(0, n_blocks, window):
        M = np.float32(mtilde)
        for j in range(w0, min(w0 + window, n_blocks)):
            if forced[j]:  # kept, and its score does not enter the running maximum
                continue
            if s[j] >= np.float32(M - dl):  # one fp32 subtraction, round to nearest
                keep[j] = 1
            M = max(M, s[j])
    return keep
