"""Python binding of libffd (include/ffd.h): argument marshalling only.

Every step of the decode path runs in the HIP kernels of ``libffd.so``; this module checks torch
tensor shapes, dtypes, devices and contiguity, passes ``data_ptr()`` and the current HIP stream
through ctypes, and raises on a non-OK status.  There is no fallback: if the library is not built
or cannot be loaded, every call raises.

Names follow the C ABI: ``quantize_k_append``, ``decode_sparse``, ``decode_dense``,
``quantize_k_residual_append``, ``decode_sparse_residual``, ``append_token``,
``decode_sparse_varlen``, ``decode_sparse_append``, ``decode_dense_varlen``, ``block_bounds``,
``block_scores``, ``select_blocks``, ``decode_masked``, ``workspace_bytes``, ``workspace_init``,
``num_splits``.
"""
from __future__ import annotations

import contextlib
import ctypes
import math
from pathlib import Path

import torch

LIB_PATH = Path(__file__).resolve().parent / "libffd.so"

FFD_OK, FFD_ERR_INVALID_ARG, FFD_ERR_UNSUPPORTED, FFD_ERR_WORKSPACE, FFD_ERR_HIP = range(5)
FFD_F32, FFD_BF16 = 0, 1
HEAD_DIM = 128


class FFDError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libffd: {msg} (status {status})")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "n_q_heads", "n_kv_heads", "head_dim", "seq_len", "seq_cap", "dtype")]


_lib = None
ABI_VERSION = 2  # include/ffd.h FFD_ABI_VERSION (2: bf16 block scales)


def lib():
    """The loaded libffd (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise FileNotFoundError(
                f"{LIB_PATH} is not built; run `python -m long_context_decoding_amd.build`")
        L = ctypes.CDLL(str(LIB_PATH))
        P, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
        D = ctypes.POINTER(Dims)
        L.ffd_abi_version.restype = i32
        if L.ffd_abi_version() != ABI_VERSION:
            raise RuntimeError(
                f"{LIB_PATH} has ABI version {L.ffd_abi_version()}, this binding expects "
                f"{ABI_VERSION}; rebuild with `python -m long_context_decoding_amd.build`")
        L.ffd_status_string.argtypes = [i32]
        L.ffd_status_string.restype = ctypes.c_char_p
        L.ffd_workspace_bytes.argtypes = [D, i32]
        L.ffd_workspace_bytes.restype = sz
        L.ffd_workspace_init.argtypes = [D, i32, P, sz, P]
        L.ffd_workspace_init.restype = i32
        L.ffd_num_splits.argtypes = [D, i32, i32]
        L.ffd_num_splits.restype = i32
        L.ffd_quantize_k_append.argtypes = [D, P, i32, i32, i32, P, P, P]
        L.ffd_quantize_k_append.restype = i32
        L.ffd_decode_sparse.argtypes = [D, P, P, P, P, P, f32, i32, P, P, P, P, sz, P]
        L.ffd_decode_sparse.restype = i32
        L.ffd_decode_dense.argtypes = [D, P, P, P, i32, P, P, P, sz, P]
        L.ffd_decode_dense.restype = i32
        L.ffd_quantize_k_residual_append.argtypes = [D, P, i32, i32, i32, i32, P, P, P, P, P]
        L.ffd_quantize_k_residual_append.restype = i32
        L.ffd_decode_sparse_residual.argtypes = [D, P, P, P, P, P, P, P, i32, f32, i32, P, P, P, P,
                                                 sz, P]
        L.ffd_decode_sparse_residual.restype = i32
        L.ffd_append_token.argtypes = [D, P, P, P, P, P, i32, P, P, P]
        L.ffd_append_token.restype = i32
        L.ffd_decode_sparse_varlen.argtypes = [D, P, P, P, P, P, P, f32, i32, P, P, P, P, sz, P]
        L.ffd_decode_sparse_varlen.restype = i32
        L.ffd_decode_sparse_append.argtypes = [D, P, P, P, P, P, P, P, P, f32, i32, P, P, P, P, sz,
                                               P]
        L.ffd_decode_sparse_append.restype = i32
        L.ffd_decode_dense_varlen.argtypes = [D, P, P, P, P, i32, P, P, P, sz, P]
        L.ffd_decode_dense_varlen.restype = i32
        L.ffd_block_bounds.argtypes = [D, P, i32, i32, i32, P, P, P]
        L.ffd_block_bounds.restype = i32
        L.ffd_block_scores.argtypes = [D, i32, P, P, P, P, P, P, i32, P, P]
        L.ffd_block_scores.restype = i32
        L.ffd_select_blocks.argtypes = [D, i32, P, P, f32, i32, P, P]
        L.ffd_select_blocks.restype = i32
        L.ffd_decode_masked.argtypes = [D, P, P, P, P, i32, P, P, P, sz, P]
        L.ffd_decode_masked.restype = i32
        L.ffd_decode_sparse_running.argtypes = [D, P, P, P, P, P, f32, i32, i32, P, P, P, P, sz,
                                                P]
        L.ffd_decode_sparse_running.restype = i32
        L.ffd_workspace_bytes_window.argtypes = [D, i32, i32]
        L.ffd_workspace_bytes_window.restype = sz
        L.ffd_decode_sparse_noalloc.argtypes = [D, P, P, P, P, P, f32, i32, P, P, P, P]
        L.ffd_decode_sparse_noalloc.restype = i32
        _lib = L
    return _lib


def abi_version() -> int:
    return int(lib().ffd_abi_version())


def status_string(status: int) -> str:
    return lib().ffd_status_string(status).decode()


def _check(status: int) -> None:
    if status != FFD_OK:
        raise FFDError(status, status_string(status))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return FFD_BF16
    if t.dtype == torch.float32:
        return FFD_F32
    raise TypeError(f"q, K and V must be bfloat16 or float32, got {t.dtype}")


def make_dims(B: int, Hq: int, Hkv: int, seq_len: int, seq_cap: int, dtype: int,
              head_dim: int = HEAD_DIM) -> Dims:
    return Dims(B, Hq, Hkv, head_dim, seq_len, seq_cap, dtype)


def dims_of(q: torch.Tensor, K: torch.Tensor, seq_len: int) -> Dims:
    if q.dim() != 3 or K.dim() != 4:
        raise ValueError("q must be [B, Hq, d] and K [B, Hkv, seq_cap, d]")
    B, Hq, d = q.shape
    B2, Hkv, cap, d2 = K.shape
    if B2 != B or d2 != d:
        raise ValueError(f"shape mismatch q {tuple(q.shape)} vs K {tuple(K.shape)}")
    return make_dims(B, Hq, Hkv, seq_len, cap, _dtype_code(K), d)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on(stream):
    """Context in which temporary buffers of a call on `stream` are allocated: torch's caching
    allocator then ties them to that stream, so that their memory is not handed to other work
    before the call's kernels on `stream` are done with it."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _need(t: torch.Tensor, name: str, dtype=None, shape=None, device=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def workspace_bytes(dims: Dims, block: int) -> int:
    return int(lib().ffd_workspace_bytes(ctypes.byref(dims), block))


def num_splits(dims: Dims, block: int, sparse: bool = True) -> int:
    return int(lib().ffd_num_splits(ctypes.byref(dims), block, 1 if sparse else 0))


def workspace_init(dims: Dims, block: int, workspace: torch.Tensor, stream=None) -> None:
    """Prepare a workspace (zero its counters) on `stream` (default: the current stream)."""
    _need(workspace, "workspace", torch.uint8)
    _check(lib().ffd_workspace_init(ctypes.byref(dims), block, _ptr(workspace),
                                    workspace.numel(), _stream(stream)))


def alloc_workspace(dims: Dims, block: int, device, stream=None) -> torch.Tensor:
    """A workspace for decode calls with these dims and block, allocated for and prepared on
    `stream` (default: the current stream)."""
    n = workspace_bytes(dims, block)
    if n == 0:
        raise FFDError(FFD_ERR_INVALID_ARG, "invalid dims for workspace")
    with _on(stream):
        ws = torch.empty(n, dtype=torch.uint8, device=device)
        workspace_init(dims, block, ws)
    return ws


def alloc_workspace_window(dims: Dims, block: int, window: int, device,
                           stream=None) -> torch.Tensor:
    """A workspace for decode_sparse_running with this window, allocated for and prepared on
    `stream`."""
    n = lib().ffd_workspace_bytes_window(ctypes.byref(dims), block, window)
    if n == 0:
        raise FFDError(FFD_ERR_UNSUPPORTED, "invalid dims or window for workspace")
    with _on(stream):
        ws = torch.empty(n, dtype=torch.uint8, device=device)
        workspace_init(dims, block, ws)
    return ws


def alloc_kq(K: torch.Tensor, block: int):
    """Zero-filled Kq [B, Hkv, seq_cap, d/2] u8 and scales [B, Hkv, seq_cap/block, d] bf16."""
    B, Hkv, cap, d = K.shape
    Kq = torch.zeros((B, Hkv, cap, d // 2), dtype=torch.uint8, device=K.device)
    sc = torch.zeros((B, Hkv, cap // block, d), dtype=torch.bfloat16, device=K.device)
    return Kq, sc


def quantize_k_append(K: torch.Tensor, tok_begin: int, tok_end: int, block: int,
                      Kq: torch.Tensor, scales: torch.Tensor, seq_len: int | None = None,
                      stream=None) -> None:
    """Quantize the blocks of K completed by tokens [tok_begin, tok_end) into Kq / scales."""
    B, Hkv, cap, d = K.shape
    _need(K, "K")
    _need(Kq, "Kq", torch.uint8, (B, Hkv, cap, d // 2), K.device)
    _need(scales, "scales", torch.bfloat16, (B, Hkv, cap // block if block > 0 else 0, d),
          K.device)
    dims = make_dims(B, Hkv, Hkv, seq_len if seq_len is not None else cap, cap, _dtype_code(K), d)
    _check(lib().ffd_quantize_k_append(ctypes.byref(dims), _ptr(K), tok_begin, tok_end, block,
                                       _ptr(Kq), _ptr(scales), _stream(stream)))


def _decode_outputs(q, out, lse, want_lse, stream=None):
    B, Hq, d = q.shape
    if out is None:
        with _on(stream):
            out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (B, Hq, d), q.device)
    if lse is None and want_lse:
        with _on(stream):
            lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, Hq), q.device)
    return out, lse


def decode_sparse(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, Kq: torch.Tensor,
                  scales: torch.Tensor, delta: float, block: int, seq_len: int,
                  out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                  keep_mask: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                  want_lse: bool = True, stream=None):
    """Sparse decode step.  Returns (out [B,Hq,d] fp32, lse [B,Hq] fp32 or None)."""
    dims = dims_of(q, K, seq_len)
    for name, t in (("q", q), ("K", K), ("V", V)):
        _need(t, name, K.dtype, None, K.device)
    _need(V, "V", K.dtype, K.shape, K.device)
    B, Hkv, cap, d = K.shape
    _need(Kq, "Kq", torch.uint8, (B, Hkv, cap, d // 2), K.device)
    _need(scales, "scales", torch.bfloat16, (B, Hkv, cap // block if block > 0 else 0, d),
          K.device)
    out, lse = _decode_outputs(q, out, lse, want_lse, stream)
    if keep_mask is not None:
        _need(keep_mask, "keep_mask", torch.uint8,
              (q.shape[0], q.shape[1], math.ceil(seq_len / block)), q.device)
    if workspace is None:
        workspace = alloc_workspace(dims, block, q.device, stream)
    _need(workspace, "workspace", torch.uint8, None, q.device)
    _check(lib().ffd_decode_sparse(ctypes.byref(dims), _ptr(q), _ptr(K), _ptr(V), _ptr(Kq),
                                   _ptr(scales), float(delta), block, _ptr(out), _ptr(lse),
                                   _ptr(keep_mask), _ptr(workspace), workspace.numel(),
                                   _stream(stream)))
    return out, lse


NOALLOC_SCRATCH_BYTES = 16 << 20  # FFD_NOALLOC_SCRATCH_BYTES


def decode_sparse_noalloc(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, Kq: torch.Tensor,
                          scales: torch.Tensor, delta: float, block: int, seq_len: int,
                          out: torch.Tensor, lse: torch.Tensor | None = None,
                          keep_mask: torch.Tensor | None = None, stream=None):
    """Sparse decode step on the library's fixed scratch area (no workspace, nothing
    allocated: `out` and `lse` are the caller's).  Calls that overlap on one GPU race."""
    dims = dims_of(q, K, seq_len)
    for name, t in (("q", q), ("K", K), ("V", V)):
        _need(t, name, K.dtype, None, K.device)
    _need(V, "V", K.dtype, K.shape, K.device)
    B, Hkv, cap, d = K.shape
    _need(Kq, "Kq", torch.uint8, (B, Hkv, cap, d // 2), K.device)
    _need(scales, "scales", torch.bfloat16, (B, Hkv, cap // block if block > 0 else 0, d),
          K.device)
    _need(out, "out", torch.float32, (q.shape[0], q.shape[1], d), q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, (q.shape[0], q.shape[1]), q.device)
    if keep_mask is not None:
        _need(keep_mask, "keep_mask", torch.uint8,
              (q.shape[0], q.shape[1], math.ceil(seq_len / block)), q.device)
    _check(lib().ffd_decode_sparse_noalloc(ctypes.byref(dims), _ptr(q), _ptr(K), _ptr(V),
                                           _ptr(Kq), _ptr(scales), float(delta), block, _ptr(out),
                                           _ptr(lse), _ptr(keep_mask), _stream(stream)))
    return out, lse


def decode_sparse_running(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, Kq: torch.Tensor,
                          scales: torch.Tensor, delta: float, block: int, window: int,
                          seq_len: int, out: torch.Tensor | None = None,
                          lse: torch.Tensor | None = None, keep_mask: torch.Tensor | None = None,
                          workspace: torch.Tensor | None = None, want_lse: bool = True,
                          stream=None):
    """Sparse step with top-delta against the running maximum of each window of `window`
    blocks.  Returns (out, lse) as decode_sparse."""
    dims = dims_of(q, K, seq_len)
    for name, t in (("q", q), ("K", K), ("V", V)):
        _need(t, name, K.dtype, None, K.device)
    _need(V, "V", K.dtype, K.shape, K.device)
    B, Hkv, cap, d = K.shape
    _need(Kq, "Kq", torch.uint8, (B, Hkv, cap, d // 2), K.device)
    _need(scales, "scales", torch.bfloat16, (B, Hkv, cap // block if block > 0 else 0, d),
          K.device)
    out, lse = _decode_outputs(q, out, lse, want_lse, stream)
    if keep_mask is not None:
        _need(keep_mask, "keep_mask", torch.uint8,
              (q.shape[0], q.shape[1], math.ceil(seq_len / block)), q.device)
    if workspace is None:
        workspace = alloc_workspace_window(dims, block, window, q.device, stream)
    _need(workspace, "workspace", torch.uint8, None, q.device)
    _check(lib().ffd_decode_sparse_running(ctypes.byref(dims), _ptr(q), _ptr(K), _ptr(V),
                                           _ptr(Kq), _ptr(scales), float(delta), block,
                                           int(window), _ptr(out), _ptr(lse), _ptr(keep_mask),
                                           _ptr(workspace), workspace.numel(), _stream(stream)))
    return out, lse


def decode_dense(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, block: int, seq_len: int,
                 out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                 workspace: torch.Tensor | None = None, want_lse: bool = True, stream=None):
    """Dense (exact flash-decoding) step.  Returns (out, lse)."""
    dims = dims_of(q, K, seq_len)
    for name, t in (("q", q), ("K", K), ("V", V)):
        _need(t, name, K.dtype, None, K.device)
    _need(V, "V", K.dtype, K.shape, K.device)
    out, lse = _decode_outputs(q, out, lse, want_lse, stream)
    if workspace is None:
        workspace = alloc_workspace(dims, block, q.device, stream)
    _need(workspace, "workspace", torch.uint8, None, q.device)
    _check(lib().ffd_decode_dense(ctypes.byref(dims), _ptr(q), _ptr(K), _ptr(V), block,
                                  _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                                  _stream(stream)))
    return out, lse


# ------------------------------------------------------------------------------------------
# Residual storage form: low-bit thumbnail + 8-bit residual instead of 16-bit keys
# ------------------------------------------------------------------------------------------
def alloc_kres(K: torch.Tensor, block: int, bits: int):
    """Zero-filled (Kc u8 [B,Hkv,cap,d*bits/8], scales bf16 [B,Hkv,cap/block,d],
    Kr int8 [B,Hkv,cap,d], res_scales f32 [B,Hkv,cap/block,d])."""
    B, Hkv, cap, d = K.shape
    dev = K.device
    return (torch.zeros((B, Hkv, cap, d * bits // 8), dtype=torch.uint8, device=dev),
            torch.zeros((B, Hkv, cap // block, d), dtype=torch.bfloat16, device=dev),
            torch.zeros((B, Hkv, cap, d), dtype=torch.int8, device=dev),
            torch.zeros((B, Hkv, cap // block, d), dtype=torch.float32, device=dev))


def _need_kres(K_shape, block, bits, Kc, sc, Kr, sr, device):
    B, Hkv, cap, d = K_shape
    _need(Kc, "Kc", torch.uint8, (B, Hkv, cap, d * bits // 8), device)
    _need(sc, "scales", torch.bfloat16, (B, Hkv, cap // block if block > 0 else 0, d), device)
    _need(Kr, "Kr", torch.int8, (B, Hkv, cap, d), device)
    _need(sr, "res_scales", torch.float32, (B, Hkv, cap // block if block > 0 else 0, d), device)


def quantize_k_residual_append(K: torch.Tensor, tok_begin: int, tok_end: int, block: int,
                               bits: int, kres, seq_len: int | None = None, stream=None) -> None:
    """Thumbnail + residual of the blocks of K (bf16) completed by tokens [tok_begin, tok_end)."""
    B, Hkv, cap, d = K.shape
    _need(K, "K")
    Kc, sc, Kr, sr = kres
    _need_kres(K.shape, block, bits, Kc, sc, Kr, sr, K.device)
    dims = make_dims(B, Hkv, Hkv, seq_len if seq_len is not None else cap, cap, _dtype_code(K), d)
    _check(lib().ffd_quantize_k_residual_append(ctypes.byref(dims), _ptr(K), tok_begin, tok_end,
                                                block, bits, _ptr(Kc), _ptr(sc), _ptr(Kr),
                                                _ptr(sr), _stream(stream)))


def decode_sparse_residual(q: torch.Tensor, K_tail: torch.Tensor | None, V: torch.Tensor, kres,
                           bits: int, delta: float, block: int, seq_len: int,
                           out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                           keep_mask: torch.Tensor | None = None,
                           workspace: torch.Tensor | None = None, want_lse: bool = True,
                           stream=None):
    """Sparse decode step in the residual storage form.  K_tail (bf16 [B,Hkv,cap,d]) supplies
    the keys of a partial tail block and may be None when seq_len % block == 0."""
    dims = dims_of(q, V, seq_len)
    _need(V, "V", torch.bfloat16, None, V.device)
    _need(q, "q", torch.bfloat16, None, V.device)
    if K_tail is not None:
        _need(K_tail, "K_tail", torch.bfloat16, V.shape, V.device)
    Kc, sc, Kr, sr = kres
    _need_kres(V.shape, block, bits, Kc, sc, Kr, sr, V.device)
    out, lse = _decode_outputs(q, out, lse, want_lse, stream)
    if keep_mask is not None:
        _need(keep_mask, "keep_mask", torch.uint8,
              (q.shape[0], q.shape[1], math.ceil(seq_len / block)), q.device)
    if workspace is None:
        workspace = alloc_workspace(dims, block, q.device, stream)
    _need(workspace, "workspace", torch.uint8, None, q.device)
    _check(lib().ffd_decode_sparse_residual(ctypes.byref(dims), _ptr(q), _ptr(K_tail), _ptr(V),
                                            _ptr(Kc), _ptr(sc), _ptr(Kr), _ptr(sr), bits,
                                            float(delta), block, _ptr(out), _ptr(lse),
                                            _ptr(keep_mask), _ptr(workspace), workspace.numel(),
                                            _stream(stream)))
    return out, lse


def append_token(k_new: torch.Tensor, v_new: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
                 seq_lens: torch.Tensor, block: int, Kq: torch.Tensor, scales: torch.Tensor,
                 stream=None) -> None:
    """Decode-loop cache update on the device: the new token's rows go to position seq_lens[b],
    a key block it completes is quantized, and seq_lens advances by one (capped at capacity)."""
    B, Hkv, cap, d = K.shape
    _need(k_new, "k_new", K.dtype, (B, Hkv, d), K.device)
    _need(v_new, "v_new", K.dtype, (B, Hkv, d), K.device)
    _need(V, "V", K.dtype, K.shape, K.device)
    _need(seq_lens, "seq_lens", torch.int32, (B,), K.device)
    _need(Kq, "Kq", torch.uint8, (B, Hkv, cap, d // 2), K.device)
    _need(scales, "scales", torch.bfloat16, (B, Hkv, cap // block if block > 0 else 0, d), K.device)
    dims = make_dims(B, Hkv, Hkv, cap, cap, _dtype_code(K), d)
    _check(lib().ffd_append_token(ctypes.byref(dims), _ptr(k_new), _ptr(v_new), _ptr(K), _ptr(V),
                                  _ptr(seq_lens), block, _ptr(Kq), _ptr(scales), _stream(stream)))


def decode_sparse_varlen(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, Kq: torch.Tensor,
                         scales: torch.Tensor, seq_lens: torch.Tensor, delta: float, block: int,
                         max_len: int | None = None, out: torch.Tensor | None = None,
                         lse: torch.Tensor | None = None, keep_mask: torch.Tensor | None = None,
                         workspace: torch.Tensor | None = None, want_lse: bool = True,
                         stream=None):
    """Sparse decode step with per-sequence lengths in device memory (seq_lens int32 [B]);
    max_len (default: the cache capacity) bounds them and sets the split coverage."""
    B, Hkv, cap, d = K.shape
    max_len = cap if max_len is None else max_len
    dims = dims_of(q, K, max_len)
    _need(V, "V", K.dtype, K.shape, K.device)
    _need(q, "q", K.dtype, None, K.device)
    _need(Kq, "Kq", torch.uint8, (B, Hkv, cap, d // 2), K.device)
    _need(scales, "scales", torch.bfloat16, (B, Hkv, cap // block if block > 0 else 0, d),
          K.device)
    _need(seq_lens, "seq_lens", torch.int32, (B,), K.device)
    out, lse = _decode_outputs(q, out, lse, want_lse, stream)
    if keep_mask is not None:
        _need(keep_mask, "keep_mask", torch.uint8,
              (q.shape[0], q.shape[1], math.ceil(max_len / block)), q.device)
    if workspace is None:
        workspace = alloc_workspace(dims, block, q.device, stream)
    _need(workspace, "workspace", torch.uint8, None, q.device)
    _check(lib().ffd_decode_sparse_varlen(ctypes.byref(dims), _ptr(q), _ptr(K), _ptr(V), _ptr(Kq),
                                          _ptr(scales), _ptr(seq_lens), float(delta), block,
                                          _ptr(out), _ptr(lse), _ptr(keep_mask), _ptr(workspace),
                                          workspace.numel(), _stream(stream)))
    return out, lse


def decode_sparse_append(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                         K: torch.Tensor, V: torch.Tensor, Kq: torch.Tensor, scales: torch.Tensor,
                         seq_lens: torch.Tensor, delta: float, block: int,
                         max_len: int | None = None, out: torch.Tensor | None = None,
                         lse: torch.Tensor | None = None, keep_mask: torch.Tensor | None = None,
                         workspace: torch.Tensor | None = None, want_lse: bool = True,
                         stream=None):
    """One decode-loop step in one launch: append_token(k_new, v_new) then decode_sparse_varlen,
    with the same results; K, V, Kq, scales and seq_lens are updated in place."""
    B, Hkv, cap, d = K.shape
    max_len = cap if max_len is None else max_len
    dims = dims_of(q, K, max_len)
    _need(V, "V", K.dtype, K.shape, K.device)
    _need(q, "q", K.dtype, None, K.device)
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _need(t, name, K.dtype, (B, Hkv, d), K.device)
    _need(Kq, "Kq", torch.uint8, (B, Hkv, cap, d // 2), K.device)
    _need(scales, "scales", torch.bfloat16, (B, Hkv, cap // block if block > 0 else 0, d),
          K.device)
    _need(seq_lens, "seq_lens", torch.int32, (B,), K.device)
    out, lse = _decode_outputs(q, out, lse, want_lse, stream)
    if keep_mask is not None:
        _need(keep_mask, "keep_mask", torch.uint8,
              (q.shape[0], q.shape[1], math.ceil(max_len / block)), q.device)
    if workspace is None:
        workspace = alloc_workspace(dims, block, q.device, stream)
    _need(workspace, "workspace", torch.uint8, None, q.device)
    _check(lib().ffd_decode_sparse_append(ctypes.byref(dims), _ptr(q), _ptr(k_new), _ptr(v_new),
                                          _ptr(K), _ptr(V), _ptr(Kq), _ptr(scales),
                                          _ptr(seq_lens), float(delta), block, _ptr(out),
                                          _ptr(lse), _ptr(keep_mask), _ptr(workspace),
                                          workspace.numel(), _stream(stream)))
    return out, lse


def decode_dense_varlen(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, seq_lens: torch.Tensor,
                        block: int, max_len: int | None = None, out: torch.Tensor | None = None,
                        lse: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                        want_lse: bool = True, stream=None):
    """Dense decode step with per-sequence lengths in device memory."""
    B, Hkv, cap, d = K.shape
    max_len = cap if max_len is None else max_len
    dims = dims_of(q, K, max_len)
    _need(V, "V", K.dtype, K.shape, K.device)
    _need(q, "q", K.dtype, None, K.device)
    _need(seq_lens, "seq_lens", torch.int32, (B,), K.device)
    out, lse = _decode_outputs(q, out, lse, want_lse, stream)
    if workspace is None:
        workspace = alloc_workspace(dims, block, q.device, stream)
    _need(workspace, "workspace", torch.uint8, None, q.device)
    _check(lib().ffd_decode_dense_varlen(ctypes.byref(dims), _ptr(q), _ptr(K), _ptr(V),
                                         _ptr(seq_lens), block, _ptr(out), _ptr(lse),
                                         _ptr(workspace), workspace.numel(), _stream(stream)))
    return out, lse


SCORE_SCAN, SCORE_BOUNDS, SCORE_EXACT = 0, 1, 2
SELECT_TOP_DELTA, SELECT_TOP_K, SELECT_TOP_P = 0, 1, 2


def alloc_bounds(K: torch.Tensor, block: int):
    """Zeroed (kmin, kmax) [B, Hkv, cap/block, d] in K's dtype."""
    B, Hkv, cap, d = K.shape
    shape = (B, Hkv, cap // block, d)
    return (torch.zeros(shape, dtype=K.dtype, device=K.device),
            torch.zeros(shape, dtype=K.dtype, device=K.device))


def block_bounds(K: torch.Tensor, tok_begin: int, tok_end: int, block: int, kmin: torch.Tensor,
                 kmax: torch.Tensor, seq_len: int | None = None, stream=None) -> None:
    """Per-channel min/max of every key block completed by tokens [tok_begin, tok_end)."""
    B, Hkv, cap, d = K.shape
    _need(K, "K", None, None, K.device)
    for name, t in (("kmin", kmin), ("kmax", kmax)):
        _need(t, name, K.dtype, (B, Hkv, cap // block, d), K.device)
    dims = make_dims(B, Hkv, Hkv, cap if seq_len is None else seq_len, cap, _dtype_code(K), d)
    _check(lib().ffd_block_bounds(ctypes.byref(dims), _ptr(K), tok_begin, tok_end, block,
                                  _ptr(kmin), _ptr(kmax), _stream(stream)))


def block_scores(kind: int, q: torch.Tensor, K: torch.Tensor, block: int, seq_len: int,
                 Kq: torch.Tensor | None = None, scales: torch.Tensor | None = None,
                 kmin: torch.Tensor | None = None, kmax: torch.Tensor | None = None,
                 out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Per-block scores [B, Hq, seq_len // block] fp32 of one kind (SCORE_*)."""
    dims = dims_of(q, K, seq_len)
    B, Hq, d = q.shape
    _need(q, "q", K.dtype, None, K.device)
    nf = seq_len // block
    if out is None:
        with _on(stream):
            out = torch.empty((B, Hq, nf), dtype=torch.float32, device=q.device)
    _need(out, "scores", torch.float32, (B, Hq, nf), q.device)
    Hkv, cap = K.shape[1], K.shape[2]
    if Kq is not None:
        _need(Kq, "Kq", torch.uint8, (B, Hkv, cap, d // 2), K.device)
    if scales is not None:
        _need(scales, "scales", torch.bfloat16, (B, Hkv, cap // block if block > 0 else 0, d),
              K.device)
    _check(lib().ffd_block_scores(ctypes.byref(dims), kind, _ptr(q), _ptr(K), _ptr(Kq),
                                  _ptr(scales), _ptr(kmin), _ptr(kmax), block, _ptr(out),
                                  _stream(stream)))
    return out


def select_blocks(rule: int, scores: torch.Tensor, param: float, block: int, seq_len: int,
                  Hkv: int, pseudo_max: torch.Tensor | None = None,
                  keep_mask: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """One selection rule (SELECT_*) over scores [B, Hq, nf] -> keep_mask [B, Hq, n_blocks]."""
    B, Hq, nf = scores.shape
    _need(scores, "scores", torch.float32, None, scores.device)
    n_blocks = math.ceil(seq_len / block)
    if keep_mask is None:
        with _on(stream):
            keep_mask = torch.empty((B, Hq, n_blocks), dtype=torch.uint8, device=scores.device)
    _need(keep_mask, "keep_mask", torch.uint8, (B, Hq, n_blocks), scores.device)
    if pseudo_max is not None:
        _need(pseudo_max, "pseudo_max", torch.float32, (B, Hq), scores.device)
    cap = n_blocks * block
    dims = make_dims(B, Hq, Hkv, seq_len, cap, FFD_BF16)
    _check(lib().ffd_select_blocks(ctypes.byref(dims), rule, _ptr(scores), _ptr(pseudo_max),
                                   float(param), block, _ptr(keep_mask), _stream(stream)))
    return keep_mask


def decode_masked(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, keep_mask: torch.Tensor,
                  block: int, seq_len: int, out: torch.Tensor | None = None,
                  lse: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                  want_lse: bool = True, stream=None):
    """Exact attention over the blocks keep_mask [B, Hq, n_blocks] marks."""
    dims = dims_of(q, K, seq_len)
    _need(V, "V", K.dtype, K.shape, K.device)
    _need(q, "q", K.dtype, None, K.device)
    _need(keep_mask, "keep_mask", torch.uint8,
          (q.shape[0], q.shape[1], math.ceil(seq_len / block)), q.device)
    out, lse = _decode_outputs(q, out, lse, want_lse, stream)
    if workspace is None:
        workspace = alloc_workspace(dims, block, q.device, stream)
    _need(workspace, "workspace", torch.uint8, None, q.device)
    _check(lib().ffd_decode_masked(ctypes.byref(dims), _ptr(q), _ptr(K), _ptr(V),
                                   _ptr(keep_mask), block, _ptr(out), _ptr(lse), _ptr(workspace),
                                   workspace.numel(), _stream(stream)))
    return out, lse
