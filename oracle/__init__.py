"""CPU oracle for Faster Flash Decoding sparse decode attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline`` leg import this
package.  The product (the HIP library and its Python binding) never does.  It shares no code
with the HIP path.

The arithmetic lives in ``ffd_oracle.c`` (plain C, built with ``-ffp-contract=off``, no fast-math,
OpenMP over (batch, query head)); this module compiles it with gcc and wraps it with ctypes on
numpy arrays.  See that file's header for what each stage computes and which passage of
"Faster Than Flash: Exploiting Attention Sparsity for Efficient Long-Context Decoding" it follows.

Array conventions: bf16 tensors are numpy ``uint16`` arrays holding bf16 bit patterns; fp32
tensors are ``float32``.  Block scales of the low-bit key copies are stored as bf16 (``uint16``);
the residual scales of the storage form are ``float32``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "ffd_oracle.c"
_LIB_PATH = _HERE / "libffd_oracle.so"

DTYPE_F32 = 0
DTYPE_BF16 = 1

_lib = None


def build(force: bool = True) -> Path:
    """Compile the oracle with gcc (fp-contract off, no fast-math)."""
    if not force and _LIB_PATH.exists() and _LIB_PATH.stat().st_mtime >= _SRC.stat().st_mtime:
        return _LIB_PATH
    tmp = _LIB_PATH.with_suffix(".so.tmp")
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-o", str(tmp), str(_SRC), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not _LIB_PATH.exists() or _LIB_PATH.stat().st_mtime < _SRC.stat().st_mtime:
        build()
    lib = ctypes.CDLL(str(_LIB_PATH))
    P = ctypes.c_void_p
    i32 = ctypes.c_int
    f32 = ctypes.c_float
    lib.ffdo_version.restype = i32
    lib.ffdo_round_bf16.argtypes = [P, P, i32]
    lib.ffdo_round_bf16.restype = None
    lib.ffdo_quantize_channel.argtypes = [P, i32, i32, i32, P, P]
    lib.ffdo_quantize_channel.restype = None
    lib.ffdo_quantize_k.argtypes = [P, i32, i32, i32, i32, i32, i32, P, P]
    lib.ffdo_quantize_k.restype = i32
    lib.ffdo_kappa.argtypes = [i32]
    lib.ffdo_kappa.restype = f32
    lib.ffdo_requant.argtypes = [P, P, i32, P]
    lib.ffdo_requant.restype = f32
    lib.ffdo_scan_head.argtypes = [P, P, P, i32, i32, i32, P, P, P]
    lib.ffdo_scan_head.restype = None
    lib.ffdo_select_head.argtypes = [P, i32, i32, f32, P, P, P]
    lib.ffdo_select_head.restype = None
    lib.ffdo_attend_head.argtypes = [P, P, P, i32, i32, i32, i32, P, P, P]
    lib.ffdo_attend_head.restype = None
    lib.ffdo_decode.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, P, P, P, P, P, f32, i32,
                                P, P, P, P, P, i32]
    lib.ffdo_decode.restype = i32
    lib.ffdo_quantize_residual.argtypes = [P, i32, P, P]
    lib.ffdo_quantize_residual.restype = None
    lib.ffdo_quantize_k_res.argtypes = [P, i32, i32, i32, i32, i32, i32, i32, P, P, P, P]
    lib.ffdo_quantize_k_res.restype = i32
    lib.ffdo_dequant.argtypes = [P, P, P, P, i32, i32, i32, i32, i32]
    lib.ffdo_dequant.restype = ctypes.c_double
    lib.ffdo_scan_head_bits.argtypes = [P, P, P, i32, i32, i32, i32, P, P, P]
    lib.ffdo_scan_head_bits.restype = None
    lib.ffdo_attend_head_res.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, i32, P, P, P]
    lib.ffdo_attend_head_res.restype = None
    lib.ffdo_decode_res.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, P,
                                    f32, i32, P, P, P, P, P, i32]
    lib.ffdo_decode_res.restype = i32
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return DTYPE_F32
    if a.dtype == np.uint16:
        return DTYPE_BF16
    raise TypeError(f"oracle takes float32 or bf16-bits (uint16) arrays, got {a.dtype}")


def _need_bf16(a: np.ndarray, name: str) -> np.ndarray:
    if a.dtype != np.uint16:
        raise TypeError(f"{name}: block scales are bf16 bits (uint16), got {a.dtype}")
    return np.ascontiguousarray(a)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to bf16 (nearest, ties to even) -> bf16 bits (uint16), as the
    block scales are stored."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, dtype=np.uint16)
    _load().ffdo_round_bf16(_ptr(x), _ptr(y), x.size)
    return y


def to_f32(a: np.ndarray) -> np.ndarray:
    """Values of an fp32 or bf16-bits array as float32."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32)
    return np.asarray(a, dtype=np.float32)


def n_threads_default() -> int:
    return max(1, len(os.sched_getaffinity(0)))


# ------------------------------------------------------------------------------------------
# Stage wrappers
# ------------------------------------------------------------------------------------------
def quantize_channel(x: np.ndarray, bits: int):
    """App. A quantizer on one channel vector -> (codes uint8[n], scale float)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    codes = np.empty(x.shape[0], dtype=np.uint8)
    s = np.empty(1, dtype=np.float32)
    _load().ffdo_quantize_channel(_ptr(x), x.shape[0], 1, bits, _ptr(codes), _ptr(s))
    return codes, float(s[0])


def quantize_k(K: np.ndarray, T: int, tok_begin: int = 0, tok_end: int | None = None,
               Kq: np.ndarray | None = None, scales: np.ndarray | None = None):
    """Quantize the completed blocks of K [B, Hkv, L_cap, d] -> (Kq u8 [..., d/2], scales bf16
    bits u16 [..., L_cap/T, d])."""
    B, Hkv, L_cap, d = K.shape
    if tok_end is None:
        tok_end = L_cap
    K = np.ascontiguousarray(K)
    if Kq is None:
        Kq = np.zeros((B, Hkv, L_cap, d // 2), dtype=np.uint8)
    if scales is None:
        scales = np.zeros((B, Hkv, L_cap // T, d), dtype=np.uint16)
    _need_bf16(scales, "scales")
    lib = _load()
    dt = _dtype_code(K)
    for b in range(B):
        for g in range(Hkv):
            rc = lib.ffdo_quantize_k(_ptr(K[b, g]), dt, L_cap, d, T, tok_begin, tok_end,
                                     _ptr(Kq[b, g]), _ptr(scales[b, g]))
            if rc < 0:
                raise ValueError("oracle quantize_k: bad sizes")
    return Kq, scales


def kappa(d: int) -> float:
    return float(_load().ffdo_kappa(d))


def requant(qh: np.ndarray, s: np.ndarray):
    """Integer requantization of q (.) s for one (head, block) -> (wi int32[d], f float)."""
    qh = np.ascontiguousarray(qh, dtype=np.float32)
    s = np.ascontiguousarray(s, dtype=np.float32)
    wi = np.empty(qh.shape[0], dtype=np.int32)
    f = _load().ffdo_requant(_ptr(qh), _ptr(s), qh.shape[0], _ptr(wi))
    return wi, float(f)


def scan_head(qh: np.ndarray, Kq_slice: np.ndarray, scales_slice: np.ndarray, n_full: int,
              T: int, per_token: bool = False):
    """Scan of one query head over a kv slice -> shat_block[n_full] (+ shat_tok, E_tok)."""
    qh = np.ascontiguousarray(to_f32(qh))
    d = qh.shape[0]
    Kq_slice = np.ascontiguousarray(Kq_slice)
    scales_slice = _need_bf16(scales_slice, "scales")
    sb = np.empty(max(n_full, 1), dtype=np.float32)
    st = np.empty(max(n_full * T, 1), dtype=np.float32) if per_token else None
    Et = np.empty(max(n_full * T, 1), dtype=np.int32) if per_token else None
    _load().ffdo_scan_head(_ptr(qh), _ptr(Kq_slice), _ptr(scales_slice), n_full, T, d,
                           _ptr(sb), _ptr(st), _ptr(Et))
    if per_token:
        return sb[:n_full], st[: n_full * T], Et[: n_full * T]
    return sb[:n_full]


def select_head(shat_block: np.ndarray, n_full: int, n_blocks: int, delta: float):
    """Pseudo-max, threshold and block mask of one head -> (keep u8[n_blocks], mtilde, theta)."""
    sb = np.ascontiguousarray(shat_block, dtype=np.float32)
    if sb.size == 0:
        sb = np.zeros(1, dtype=np.float32)
    keep = np.empty(max(n_blocks, 1), dtype=np.uint8)
    mt = np.empty(1, dtype=np.float32)
    th = np.empty(1, dtype=np.float32)
    _load().ffdo_select_head(_ptr(sb), n_full, n_blocks, float(delta), _ptr(keep), _ptr(mt),
                             _ptr(th))
    return keep[:n_blocks], float(mt[0]), float(th[0])


def attend_head(qh: np.ndarray, K_slice: np.ndarray, V_slice: np.ndarray, L: int, T: int,
                keep: np.ndarray | None = None):
    """Exact fp64 attention of one head over kept blocks (or all if keep is None)."""
    qv = np.ascontiguousarray(to_f32(qh))
    d = qv.shape[0]
    K_slice = np.ascontiguousarray(K_slice)
    V_slice = np.ascontiguousarray(V_slice)
    out = np.empty(d, dtype=np.float64)
    lse = np.empty(1, dtype=np.float64)
    kp = None if keep is None else np.ascontiguousarray(keep, dtype=np.uint8)
    _load().ffdo_attend_head(_ptr(qv), _ptr(K_slice), _ptr(V_slice), _dtype_code(K_slice), L, d,
                             T, _ptr(kp), _ptr(out), _ptr(lse))
    return out, float(lse[0])


def decode(q, K, V, L: int, T: int, delta: float = float("inf"), Kq=None, scales=None,
           sparse: bool = True, n_threads: int | None = None, want_shat: bool = False):
    """Whole decode step.  Returns dict(out f64 [B,Hq,d], lse f64 [B,Hq], keep u8, shat, mtilde)."""
    B, Hq, d = q.shape
    _, Hkv, L_cap, _ = K.shape
    dt = _dtype_code(K)
    if _dtype_code(q) != dt or _dtype_code(V) != dt:
        raise TypeError("q, K and V must share a dtype")
    q = np.ascontiguousarray(q)
    K = np.ascontiguousarray(K)
    V = np.ascontiguousarray(V)
    n_blocks = (L + T - 1) // T
    n_full = L // T
    out = np.empty((B, Hq, d), dtype=np.float64)
    lse = np.empty((B, Hq), dtype=np.float64)
    keep = shat = mtilde = None
    if sparse:
        if Kq is None or scales is None:
            raise ValueError("sparse decode needs Kq and scales")
        Kq = np.ascontiguousarray(Kq)
        scales = _need_bf16(scales, "scales")
        keep = np.empty((B, Hq, max(n_blocks, 1)), dtype=np.uint8)
        mtilde = np.empty((B, Hq), dtype=np.float32)
        if want_shat:
            shat = np.empty((B, Hq, max(n_full, 1)), dtype=np.float32)
    rc = _load().ffdo_decode(B, Hq, Hkv, d, L, L_cap, T, dt, _ptr(q), _ptr(K), _ptr(V),
                             _ptr(Kq), _ptr(scales), float(delta), 1 if sparse else 0,
                             _ptr(out), _ptr(lse), _ptr(keep), _ptr(shat), _ptr(mtilde),
                             n_threads or n_threads_default())
    if rc < 0:
        raise ValueError("oracle decode: bad sizes")
    res = {"out": out, "lse": lse}
    if sparse:
        res["keep"] = keep[:, :, :n_blocks]
        res["mtilde"] = mtilde
        if want_shat:
            res["shat"] = shat[:, :, :n_full]
    return res


# ------------------------------------------------------------------------------------------
# Residual storage form: low-bit thumbnail + 8-bit residual (Sec. 3.1, Fig. 2, Alg. 1 Dequant)
# ------------------------------------------------------------------------------------------
def quantize_residual(r: np.ndarray):
    """8-bit symmetric quantizer of one residual vector -> (codes int8[n], scale float)."""
    r = np.ascontiguousarray(r, dtype=np.float32)
    rq = np.empty(r.shape[0], dtype=np.int8)
    s = np.empty(1, dtype=np.float32)
    _load().ffdo_quantize_residual(_ptr(r), r.shape[0], _ptr(rq), _ptr(s))
    return rq, float(s[0])


def quantize_k_res(K: np.ndarray, T: int, bits: int, tok_begin: int = 0, tok_end: int | None = None,
                   out=None):
    """Thumbnail + residual of the completed blocks of K [B, Hkv, L_cap, d] ->
    (Kc u8 [.., d*bits/8], sc bf16 bits u16 [.., L_cap/T, d], Kr i8 [.., d], sr f32 [.., L_cap/T, d])."""
    B, Hkv, L_cap, d = K.shape
    if tok_end is None:
        tok_end = L_cap
    K = np.ascontiguousarray(K)
    if out is None:
        out = (np.zeros((B, Hkv, L_cap, d * bits // 8), np.uint8),
               np.zeros((B, Hkv, L_cap // T, d), np.uint16),
               np.zeros((B, Hkv, L_cap, d), np.int8),
               np.zeros((B, Hkv, L_cap // T, d), np.float32))
    Kc, sc, Kr, sr = out
    _need_bf16(sc, "sc")
    lib = _load()
    dt = _dtype_code(K)
    for b in range(B):
        for g in range(Hkv):
            rc = lib.ffdo_quantize_k_res(_ptr(K[b, g]), dt, L_cap, d, T, bits, tok_begin, tok_end,
                                         _ptr(Kc[b, g]), _ptr(sc[b, g]), _ptr(Kr[b, g]),
                                         _ptr(sr[b, g]))
            if rc < 0:
                raise ValueError("oracle quantize_k_res: bad sizes")
    return Kc, sc, Kr, sr


def dequant(Kc, sc, Kr, sr, T: int, bits: int, t: int, c: int) -> float:
    """Alg. 1 Dequant of key element (t, c) of one slice (double)."""
    d = Kr.shape[-1]
    return float(_load().ffdo_dequant(_ptr(np.ascontiguousarray(Kc)), _ptr(_need_bf16(sc, "sc")),
                                      _ptr(np.ascontiguousarray(Kr)), _ptr(np.ascontiguousarray(sr)),
                                      d, T, bits, t, c))


def scan_head_bits(qh, Kc_slice, sc_slice, n_full: int, T: int, bits: int, per_token=False):
    """Scan of one head over a thumbnail slice (bits = 2 or 4)."""
    qh = np.ascontiguousarray(to_f32(qh))
    d = qh.shape[0]
    Kc_slice = np.ascontiguousarray(Kc_slice)
    sc_slice = _need_bf16(sc_slice, "sc")
    sb = np.empty(max(n_full, 1), dtype=np.float32)
    st = np.empty(max(n_full * T, 1), dtype=np.float32) if per_token else None
    Et = np.empty(max(n_full * T, 1), dtype=np.int32) if per_token else None
    _load().ffdo_scan_head_bits(_ptr(qh), _ptr(Kc_slice), _ptr(sc_slice), n_full, T, d, bits,
                                _ptr(sb), _ptr(st), _ptr(Et))
    if per_token:
        return sb[:n_full], st[: n_full * T], Et[: n_full * T]
    return sb[:n_full]


def attend_head_res(qh, Kc, sc, Kr, sr, Ktail, V, L: int, T: int, bits: int, keep=None):
    """Exact fp64 attention of one head over Dequant keys (full blocks) + 16-bit tail keys."""
    qv = np.ascontiguousarray(to_f32(qh))
    d = qv.shape[0]
    out = np.empty(d, dtype=np.float64)
    lse = np.empty(1, dtype=np.float64)
    kp = None if keep is None else np.ascontiguousarray(keep, dtype=np.uint8)
    V = np.ascontiguousarray(V)
    _load().ffdo_attend_head_res(_ptr(qv), _ptr(np.ascontiguousarray(Kc)),
                                 _ptr(_need_bf16(sc, "sc")), _ptr(np.ascontiguousarray(Kr)),
                                 _ptr(np.ascontiguousarray(sr)),
                                 None if Ktail is None else _ptr(np.ascontiguousarray(Ktail)),
                                 _ptr(V), _dtype_code(V), L, d, T, bits, _ptr(kp), _ptr(out),
                                 _ptr(lse))
    return out, float(lse[0])


def decode_res(q, Ktail, V, Kc, sc, Kr, sr, L: int, T: int, bits: int, delta: float = float("inf"),
               sparse: bool = True, n_threads: int | None = None, want_shat: bool = False):
    """Whole decode step in the residual storage form (q, Ktail, V bf16 bits)."""
    B, Hq, d = q.shape
    _, Hkv, L_cap, _ = V.shape
    for a in (q, V) + (() if Ktail is None else (Ktail,)):
        if _dtype_code(a) != DTYPE_BF16:
            raise TypeError("the residual form takes bf16 q, tail keys and values")
    n_blocks = (L + T - 1) // T
    n_full = L // T
    out = np.empty((B, Hq, d), dtype=np.float64)
    lse = np.empty((B, Hq), dtype=np.float64)
    keep = np.empty((B, Hq, max(n_blocks, 1)), dtype=np.uint8) if sparse else None
    mtilde = np.empty((B, Hq), dtype=np.float32) if sparse else None
    shat = np.empty((B, Hq, max(n_full, 1)), dtype=np.float32) if (sparse and want_shat) else None
    _need_bf16(sc, "sc")
    arrs = [np.ascontiguousarray(a) for a in (q, V, Kc, sc, Kr, sr)]
    Kt = None if Ktail is None else np.ascontiguousarray(Ktail)
    rc = _load().ffdo_decode_res(B, Hq, Hkv, d, L, L_cap, T, bits, _ptr(arrs[0]), _ptr(Kt),
                                 _ptr(arrs[1]), _ptr(arrs[2]), _ptr(arrs[3]), _ptr(arrs[4]),
                                 _ptr(arrs[5]), float(delta), 1 if sparse else 0, _ptr(out),
                                 _ptr(lse), _ptr(keep), _ptr(shat), _ptr(mtilde),
                                 n_threads or n_threads_default())
    if rc < 0:
        raise ValueError("oracle decode_res: bad sizes")
    res = {"out": out, "lse": lse}
    if sparse:
        res["keep"] = keep[:, :, :n_blocks]
        res["mtilde"] = mtilde
        if want_shat:
            res["shat"] = shat[:, :, :n_full]
    return res
