"""ctypes binding of libffd_probe.so (include/ffd_probe.h): a plain streaming read, the
measured ceiling of HBM read bandwidth beside the vendor peak.  Marshalling only."""
from __future__ import annotations

import ctypes
from pathlib import Path

import torch

LIB_PATH = Path(__file__).resolve().parent / "libffd_probe.so"
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is not built: run long_context_decoding_amd.build")
        L = ctypes.CDLL(str(LIB_PATH))
        L.ffd_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32,
                                            ctypes.c_void_p, ctypes.c_void_p]
        L.ffd_probe_stream_read.restype = ctypes.c_int32
        _lib = L
    return _lib


def stream_read(src: torch.Tensor, n_groups: int, sink: torch.Tensor, stream=None) -> None:
    """Read all of src (contiguous, 16-byte aligned, size a multiple of 16 bytes) with n_groups
    work-groups; sink (>= 16 * n_groups bytes) receives each work-group's XOR of 16-byte words."""
    if not (src.is_cuda and sink.is_cuda and src.is_contiguous() and sink.is_contiguous()):
        raise ValueError("src and sink must be contiguous device tensors")
    nbytes = src.numel() * src.element_size()
    if sink.numel() * sink.element_size() < 16 * n_groups:
        raise ValueError("sink too small")
    s = stream if stream is not None else torch.cuda.current_stream()
    rc = lib().ffd_probe_stream_read(ctypes.c_void_p(src.data_ptr()), nbytes, int(n_groups),
                                     ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(s.cuda_stream))
    if rc != 0:
        raise RuntimeError(f"ffd_probe_stream_read failed ({rc})")
