"""Seeded synthetic decode-attention workloads.

This module only draws inputs (queries, keys, values) with the shapes and structure of the
long-context decode workloads studied in "Faster Than Flash: Exploiting Attention Sparsity for
Efficient Long-Context Decoding" (Sec. 4.1-4.2: Llama-3.1-8B-shaped attention, 4K-256K
contexts; Sec. 3.2: attention dominated by sink and local tokens).  It holds none of the
method's arithmetic: no quantization, scan, selection or attention.  Both the CPU oracle and the
HIP library consume the same arrays it returns.

The paper measures on real model traces and public long-context suites, which are not available
here; these synthetic inputs stand in for them.  Keys are ``plant + noise``: noise, queries and
values are i.i.d. N(0, 1); a *plant* adds ``a * e`` to every key of selected blocks, where ``e``
is a direction built from the queries of the kv-head's query group:

* ``literal``  e = qbar / |qbar| with qbar the group's mean query: logit shift a*|qbar|/sqrt(d),
  about a for a single head with |q| ~ sqrt(d).
* ``logit``    the minimum-norm e with q_h . e = sqrt(d) for every query head h of the group
  (e = sqrt(d) Q^T (Q Q^T)^-1 1 for the group's G x d query matrix Q), so the plant raises every
  head's logit q_h . k / sqrt(d) by exactly a.

Queries enter after rounding to the storage dtype.

Arrays: bf16 tensors are numpy ``uint16`` bit patterns (round-to-nearest-even from float32),
fp32 tensors are ``float32``.  Shapes: q [B, Hq, d]; K, V [B, Hkv, L_cap, d].  Rows at token
index >= L (padding up to L_cap) are filled with NaN so that any read of them shows up.

Random streams: ``numpy.random.Generator(PCG64(SeedSequence([seed, stream, ...])))`` with
stream 0 for q, (1, b) for per-sequence draws and (2, b, g) for the kv slice (b, g), drawn in the
order: key noise, values, then plant choices.  Every slice can therefore be regenerated on its
own.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

BF16_NAN = np.uint16(0x7FC0)


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    L: int
    T: int
    dtype: str = "bf16"          # "bf16" or "f32" for q, K and V
    d: int = 128
    deltas: tuple = (5.0,)
    plant: str = "flat"          # "flat" | "needles" | "powerlaw"
    plant_dir: str = "logit"     # "literal" | "logit"
    n_needles: int = 0           # needle blocks per (b, kv head)
    needle_a: float = 0.0
    sink_a: float = 0.0          # plant on block 0 (0 = none)
    power_a: float = 0.0         # powerlaw: block offset power_a * u**power_exp
    power_exp: float = 4.0
    recent_tokens: int = 0       # powerlaw: extra plant on the last tokens
    recent_a: float = 0.0
    seed: int = 0
    L_cap: int = 0               # 0 -> ceil(L / T) * T
    description: str = field(default="", compare=False)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def cap(self) -> int:
        return self.L_cap or -(-self.L // self.T) * self.T

    @property
    def n_full(self) -> int:
        return self.L // self.T

    @property
    def n_blocks(self) -> int:
        return -(-self.L // self.T)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five decode workloads, named by what they are.
WORKLOADS = {
    w.name: w
    for w in [
        Workload("h1_4k_f32_needles", B=1, Hq=1, Hkv=1, L=4096, T=64, dtype="f32",
                 deltas=(5.0,), plant="needles", plant_dir="literal", n_needles=4,
                 needle_a=8.0, seed=20260901,
                 description="single head, fp32, 4 needle blocks at logit ~8"),
        Workload("gqa4_32k_sink_needles", B=1, Hq=32, Hkv=8, L=32768, T=64, deltas=(3.0, 5.0, 8.0),
                 plant="needles", n_needles=round(0.01 * 512), needle_a=6.0, sink_a=10.0,
                 seed=20260902,
                 description="Llama-3-8B-shaped layer, 32K, sink block + 1% needle blocks"),
        Workload("b8_gqa4_128k_powerlaw", B=8, Hq=32, Hkv=8, L=131072, T=64, deltas=(5.0,),
                 plant="powerlaw", power_a=8.0, power_exp=4.0, sink_a=10.0, recent_tokens=256,
                 recent_a=4.0, seed=20260903,
                 description="batch 8, 128K, power-law block relevance + sink + recency"),
        Workload("gqa4_256k_sink_needles", B=1, Hq=32, Hkv=8, L=262144, T=128, deltas=(5.0,),
                 plant="needles", n_needles=round(0.005 * 2048), needle_a=6.0, sink_a=10.0,
                 seed=20260904,
                 description="256K, block 128, sink block + 0.5% needle blocks"),
        Workload("b16_gqa4_64k_flat", B=16, Hq=32, Hkv=8, L=65536, T=64, deltas=(5.0,),
                 plant="flat", seed=20260905,
                 description="batch 16, 64K, all keys N(0,1): scan-overhead case"),
    ]
}


# Further shapes the paper runs the method on (Sec. 4.5 and App. F: Qwen2.5 with grouped-query
# attention); parity cases, not benchmark lines.
EXTRA_WORKLOADS = {
    w.name: w
    for w in [
        Workload("gqa7_32k_sink_needles", B=1, Hq=28, Hkv=4, L=32768, T=64, deltas=(5.0,),
                 plant="needles", n_needles=round(0.01 * 512), needle_a=6.0, sink_a=10.0,
                 seed=20260906,
                 description="Qwen2.5-7B-shaped layer (28 query / 4 kv heads), 32K, sink block + "
                             "1% needle blocks"),
    ]
}


def _gen(seed: int, *stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *stream])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, np.float32)


def _values(a: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_to_f32(a) if dtype == "bf16" else a


def make_q(w: Workload) -> np.ndarray:
    q32 = _gen(w.seed, 0).standard_normal((w.B, w.Hq, w.d), dtype=np.float32)
    return _store(q32, w.dtype)


def plant_direction(w: Workload, q_group: np.ndarray) -> np.ndarray:
    """Plant direction e for one kv head from its group's stored queries (float64 [d])."""
    Q = _values(q_group, w.dtype).astype(np.float64)
    if w.plant_dir == "literal":
        qbar = Q.mean(axis=0)
        n = math.sqrt(float(qbar @ qbar))
        return qbar / n if n > 0 else np.zeros(w.d)
    gram = Q @ Q.T
    coef = np.linalg.lstsq(gram, np.ones(Q.shape[0]), rcond=None)[0]
    return math.sqrt(w.d) * (Q.T @ coef)


def sequence_offsets(w: Workload, b: int) -> np.ndarray | None:
    """Per-sequence block offsets (powerlaw plant), shared by the kv heads of sequence b."""
    if w.plant != "powerlaw":
        return None
    u = _gen(w.seed, 1, b).random(w.n_blocks)
    return w.power_a * u ** w.power_exp


def make_slice(w: Workload, q: np.ndarray, b: int, g: int, offsets: np.ndarray | None = None):
    """Keys and values of kv slice (b, g): (K [L_cap, d], V [L_cap, d], info dict)."""
    rng = _gen(w.seed, 2, b, g)
    L, cap, d, T = w.L, w.cap, w.d, w.T
    z = rng.standard_normal((L, d), dtype=np.float32)
    v = rng.standard_normal((L, d), dtype=np.float32)
    info = {"needles": np.zeros(0, dtype=np.int64)}
    e = plant_direction(w, q[b, g * w.G:(g + 1) * w.G])
    # per-token plant amplitude
    amp = np.zeros(L, dtype=np.float64)
    if w.plant == "needles" and w.n_needles > 0 and w.n_full >= 3:
        pool = np.arange(1, w.n_full - 1)
        k = min(w.n_needles, pool.size)
        needles = np.sort(rng.choice(pool, size=k, replace=False))
        info["needles"] = needles
        for j in needles:
            amp[j * T:(j + 1) * T] = w.needle_a
    elif w.plant == "powerlaw":
        if offsets is None:
            offsets = sequence_offsets(w, b)
        amp[:] = np.repeat(offsets, T)[:L]
    if w.sink_a:                      # the sink block replaces whatever block 0 had
        amp[:min(T, L)] = w.sink_a
    if w.recent_tokens:               # recency boost on the last tokens, on top
        amp[max(0, L - w.recent_tokens):] += w.recent_a
    nz = np.nonzero(amp)[0]
    if nz.size:
        z[nz] += (amp[nz, None] * e[None, :]).astype(np.float32)
    K = np.empty((cap, d), dtype=np.uint16 if w.dtype == "bf16" else np.float32)
    V = np.empty_like(K)
    K[:L] = _store(z, w.dtype)
    V[:L] = _store(v, w.dtype)
    if cap > L:
        K[L:] = BF16_NAN if w.dtype == "bf16" else np.float32(np.nan)
        V[L:] = K[L:]
    return K, V, info


def make_inputs(w: Workload, slices=None, workers: int | None = None):
    """q [B,Hq,d] and K, V [B,Hkv,L_cap,d] for the whole workload (or only `slices` = [(b,g)],
    the other slices left zero).  Returns (q, K, V, info) with info["needles"][(b, g)].
    Slices are drawn in a thread pool; each has its own random stream, so the result does not
    depend on the number of workers."""
    q = make_q(w)
    shape = (w.B, w.Hkv, w.cap, w.d)
    dt = np.uint16 if w.dtype == "bf16" else np.float32
    K = np.zeros(shape, dtype=dt)
    V = np.zeros(shape, dtype=dt)
    info = {"needles": {}}
    want = [(b, g) for b in range(w.B) for g in range(w.Hkv)]
    if slices is not None:
        sel = set(slices)
        want = [bg for bg in want if bg in sel]
    offs = {b: sequence_offsets(w, b) for b in {b for b, _ in want}}

    def one(bg):
        b, g = bg
        K[b, g], V[b, g], inf = make_slice(w, q, b, g, offs[b])
        return bg, inf["needles"]

    if workers is None:
        workers = min(16, max(1, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(max(1, workers)) as ex:
        for bg, nd in ex.map(one, want):
            info["needles"][bg] = nd
    return q, K, V, info


def small(name: str, B: int, Hq: int, Hkv: int, L: int, T: int, dtype: str = "bf16",
          seed: int = 1, plant: str = "needles", **kw) -> Workload:
    """A small workload for parity sweeps (defaults: sink 10, needles at 6, logit plant)."""
    n_full = L // T
    base = dict(n_needles=max(1, n_full // 8), needle_a=6.0, sink_a=10.0)
    if plant == "powerlaw":
        base = dict(power_a=8.0, power_exp=4.0, sink_a=10.0, recent_tokens=min(L, 2 * T),
                    recent_a=4.0)
    elif plant == "flat":
        base = {}
    base.update(kw)
    return Workload(name, B=B, Hq=Hq, Hkv=Hkv, L=L, T=T, dtype=dtype, plant=plant,
                    plant_dir="literal" if Hq == Hkv else "logit", seed=seed, **base)
