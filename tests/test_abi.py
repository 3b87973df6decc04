"""C-ABI checks that need no GPU: the library loads, exports every function declared in
include/ffd.h, and rejects bad arguments before any HIP call (so nothing is launched)."""
import ctypes
import re
import subprocess
from pathlib import Path

import pytest

from long_context_decoding_amd import ffd

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "ffd.h"

# fake, 16-byte aligned device addresses: validation must fail before anything dereferences them
A = ctypes.c_void_p(0x10000)
MISALIGNED = ctypes.c_void_p(0x10008)
COUNTER_BYTES = 524288  # fixed counter region: one 8-byte slot per work unit, 65535 units


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(ffd_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not ffd.LIB_PATH.exists():
        pytest.skip("libffd.so not built")
    return ffd.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert {"ffd_quantize_k_append", "ffd_decode_sparse", "ffd_decode_dense",
            "ffd_workspace_bytes", "ffd_workspace_init", "ffd_status_string",
            "ffd_abi_version"} <= set(names)
    nm = subprocess.run(["nm", "-D", "--defined-only", str(ffd.LIB_PATH)], capture_output=True,
                        text=True, check=True).stdout
    exported = set(re.findall(r"\bT (ffd_\w+)", nm))
    for n in names:
        assert n in exported, f"{n} declared in ffd.h but not exported"
        assert hasattr(L, n)


def test_version_and_status_strings(L):
    m = re.search(r"#define FFD_ABI_VERSION (\d+)", HEADER.read_text())
    assert ffd.abi_version() == ffd.ABI_VERSION == int(m.group(1))
    for s in range(5):
        assert ffd.status_string(s)
    assert ffd.status_string(99) == "unknown status"


def test_build_entry_post_check(L):
    # the checks build() runs after compiling: package import, ABI version, both libraries
    import __graft_entry__

    __graft_entry__.check_built()


def dims(**kw):
    base = dict(B=1, Hq=32, Hkv=8, seq_len=4096, seq_cap=4096, dtype=ffd.FFD_BF16)
    base.update(kw)
    return ffd.make_dims(base["B"], base["Hq"], base["Hkv"], base["seq_len"], base["seq_cap"],
                         base["dtype"], base.get("head_dim", 128))


def sparse_call(L, d, block=64, delta=5.0, q=A, ws=A, ws_bytes=1 << 30, K=A, keep=None):
    return L.ffd_decode_sparse(ctypes.byref(d), q, K, A, A, A, delta, block, A, A, keep, ws,
                               ws_bytes, None)





def ws_need(units, S, width, d=128):
    """Bytes one call needs: the counter region, then (m, l) and o of every (unit, split, head
    of the unit) record, each region on a 256-byte boundary."""
    rec = units * S * width
    return COUNTER_BYTES + -(-rec * 8 // 256) * 256 + rec * d * 4


def test_workspace_and_splits(L):
    d = dims()
    S = ffd.num_splits(d, 64)
    assert S >= 1
    # 64 blocks over 8 kv heads: one block per wave (16 splits) for the sparse step; the dense
    # step keeps two blocks per split (32), and the workspace covers both
    assert S == 16 and ffd.num_splits(d, 64, sparse=False) == 32
    rec = 1 * 8 * 32 * 4                      # (unit, split, query head of the unit)
    r256 = lambda x: -(-x // 256) * 256
    assert ffd.workspace_bytes(d, 64) == COUNTER_BYTES + r256(rec * 8) + rec * 128 * 4
    big = dims(B=8, seq_len=131072, seq_cap=131072)
    S = ffd.num_splits(big, 64)
    assert -(-2048 // S) <= 256
    # the dense step splits further (at most 8192 tokens per split); the workspace covers both
    Sd = ffd.num_splits(big, 64, sparse=False)
    assert Sd == 131072 // 8192 and Sd > S
    rec = 8 * 8 * Sd * 4
    assert ffd.workspace_bytes(big, 64) == COUNTER_BYTES + r256(rec * 8) + rec * 128 * 4
    long1 = dims(seq_len=262144, seq_cap=262144)
    assert ffd.num_splits(long1, 128, sparse=False) == ffd.num_splits(long1, 128) == 32
    assert ffd.workspace_bytes(dims(head_dim=64), 64) == 0
    assert ffd.workspace_bytes(d, 96) == 0


@pytest.mark.parametrize("Hq,Hkv,units,width", [
    (24, 8, 8, 4),     # G = 3: one unit of 4 heads per kv head, the last one padding
    (28, 4, 4, 8),     # G = 7 (Qwen2.5-7B's 28 query / 4 kv heads): padded to 8
    (40, 8, 8, 8),     # G = 5
    (12, 2, 2, 8),     # G = 6
    (64, 4, 8, 8),     # G = 16: two units of 8 per kv head
    (48, 4, 8, 8),     # G = 12: units of 8 and of 4 (+4 padding)
    (9, 1, 2, 8),      # G = 9
])
def test_group_sizes_and_units(L, Hq, Hkv, units, width):
    """Every group size is accepted; the workspace holds one partial per (unit, split, head of
    the unit), the unit being the kernel width that holds the group (or 8 heads)."""
    d = dims(Hq=Hq, Hkv=Hkv)
    S = ffd.num_splits(d, 64)
    Sd = ffd.num_splits(d, 64, sparse=False)
    assert S >= 1 and Sd >= 1
    # one work-group per CU: the split count follows the unit count (4096 tokens: 64 blocks,
    # so at most 32 splits of two blocks each); the sparse step takes one block per wave (16
    # splits) when its work-groups still fill half of the 256 CUs
    s0 = min(-(-256 // units), 32)
    assert Sd == s0
    assert S == (16 if s0 > 16 and units * 16 >= 128 else s0)
    assert ffd.workspace_bytes(d, 64) == ws_need(units, max(S, Sd), width)
    assert sparse_call(L, d, ws_bytes=ws_need(units, S, width) - 1) == ffd.FFD_ERR_WORKSPACE


def test_too_many_units_unsupported(L):
    # 65535 units at most: 4096 sequences x 8 kv heads x 2 units (G = 16) is 65536
    assert sparse_call(L, dims(B=4096, Hq=128, Hkv=8)) == ffd.FFD_ERR_UNSUPPORTED
    assert ffd.workspace_bytes(dims(B=4096, Hq=128, Hkv=8), 64) == 0
    assert ffd.workspace_bytes(dims(B=4095, Hq=128, Hkv=8), 64) > 0


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), ffd.FFD_ERR_UNSUPPORTED),
    (dict(Hq=30, Hkv=8), ffd.FFD_ERR_INVALID_ARG),      # not a multiple
    (dict(seq_len=0), ffd.FFD_ERR_INVALID_ARG),
    (dict(seq_cap=4000), ffd.FFD_ERR_INVALID_ARG),      # < seq_len
    (dict(seq_len=100, seq_cap=100), ffd.FFD_ERR_INVALID_ARG),  # cap not a block multiple
    (dict(dtype=7), ffd.FFD_ERR_INVALID_ARG),
    (dict(B=-1), ffd.FFD_ERR_INVALID_ARG),
])
def test_bad_dims(L, kw, status):
    assert sparse_call(L, dims(**kw)) == status


def test_bad_arguments(L):
    d = dims()
    assert sparse_call(L, d, block=96) == ffd.FFD_ERR_UNSUPPORTED
    assert sparse_call(L, d, block=0) == ffd.FFD_ERR_INVALID_ARG
    assert sparse_call(L, d, delta=float("nan")) == ffd.FFD_ERR_INVALID_ARG
    assert sparse_call(L, d, delta=-1.0) == ffd.FFD_ERR_INVALID_ARG
    assert sparse_call(L, d, q=None) == ffd.FFD_ERR_INVALID_ARG
    assert sparse_call(L, d, K=MISALIGNED) == ffd.FFD_ERR_INVALID_ARG
    assert sparse_call(L, d, keep=MISALIGNED) == ffd.FFD_ERR_INVALID_ARG
    assert sparse_call(L, d, ws=None) == ffd.FFD_ERR_WORKSPACE
    assert sparse_call(L, d, ws_bytes=ws_need(8, ffd.num_splits(d, 64), 4) - 1) == \
        ffd.FFD_ERR_WORKSPACE
    assert L.ffd_decode_dense(ctypes.byref(d), A, A, A, 64, A, A, A, 16, None) == \
        ffd.FFD_ERR_WORKSPACE
    assert L.ffd_decode_dense(ctypes.byref(d), A, A, None, 64, A, A, A, 1 << 30, None) == \
        ffd.FFD_ERR_INVALID_ARG


def test_quantize_validation(L):
    d = dims()
    q = L.ffd_quantize_k_append
    assert q(ctypes.byref(d), A, 0, 4097, 64, A, A, None) == ffd.FFD_ERR_INVALID_ARG
    assert q(ctypes.byref(d), A, 10, 5, 64, A, A, None) == ffd.FFD_ERR_INVALID_ARG
    assert q(ctypes.byref(d), A, -1, 5, 64, A, A, None) == ffd.FFD_ERR_INVALID_ARG
    assert q(ctypes.byref(d), None, 0, 64, 64, A, A, None) == ffd.FFD_ERR_INVALID_ARG
    assert q(ctypes.byref(d), A, 0, 64, 128, A, MISALIGNED, None) == ffd.FFD_ERR_INVALID_ARG
    # ranges that complete no block launch nothing and succeed
    assert q(ctypes.byref(d), A, 0, 63, 64, A, A, None) == ffd.FFD_OK
    assert q(ctypes.byref(d), A, 64, 127, 64, A, A, None) == ffd.FFD_OK


def test_workspace_init_validation(L):
    d = dims()
    n = ffd.workspace_bytes(d, 64)
    wi = L.ffd_workspace_init
    assert wi(ctypes.byref(d), 64, None, n, None) == ffd.FFD_ERR_WORKSPACE
    assert wi(ctypes.byref(d), 64, MISALIGNED, n, None) == ffd.FFD_ERR_WORKSPACE
    # only the counter region needs to fit: its fixed size, whatever the dims
    assert wi(ctypes.byref(d), 64, A, COUNTER_BYTES - 1, None) == ffd.FFD_ERR_WORKSPACE
    big = dims(B=40)
    assert wi(ctypes.byref(big), 64, A, COUNTER_BYTES - 1, None) == ffd.FFD_ERR_WORKSPACE
    assert wi(ctypes.byref(d), 96, A, n, None) == ffd.FFD_ERR_UNSUPPORTED
    assert wi(ctypes.byref(dims(B=0)), 64, None, 0, None) == ffd.FFD_OK


def test_too_many_blocks_unsupported(L):
    d = dims(seq_len=256 * 256 * 64 + 1, seq_cap=256 * 256 * 64 + 64)
    assert sparse_call(L, d) == ffd.FFD_ERR_UNSUPPORTED


def test_empty_batch_is_a_noop(L):
    d = dims(B=0)
    assert sparse_call(L, d, q=None, ws=None, ws_bytes=0) == ffd.FFD_OK
    assert L.ffd_decode_dense(ctypes.byref(d), None, None, None, 64, None, None, None, 0,
                              None) == ffd.FFD_OK
    assert L.ffd_quantize_k_append(ctypes.byref(d), None, 0, 4096, 64, None, None, None) == \
        ffd.FFD_OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(ffd, "LIB_PATH", tmp_path / "missing.so")
    monkeypatch.setattr(ffd, "_lib", None)
    with pytest.raises(FileNotFoundError):
        ffd.lib()


def test_residual_validation(L):
    d = dims()
    n = ffd.workspace_bytes(d, 64)
    dec = L.ffd_decode_sparse_residual
    qa = L.ffd_quantize_k_residual_append

    def call(dd=d, bits=2, Kt=None, Kr=A, delta=5.0, block=64):
        return dec(ctypes.byref(dd), A, Kt, A, A, A, Kr, A, bits, delta, block, A, A, None, A, n,
                   None)

    assert call(bits=3) == ffd.FFD_ERR_UNSUPPORTED
    assert call(bits=0) == ffd.FFD_ERR_UNSUPPORTED
    assert call(dd=dims(dtype=ffd.FFD_F32)) == ffd.FFD_ERR_UNSUPPORTED
    assert call(Kr=None) == ffd.FFD_ERR_INVALID_ARG
    assert call(delta=float("nan")) == ffd.FFD_ERR_INVALID_ARG
    # a partial tail block needs the 16-bit tail keys
    assert call(dd=dims(seq_len=4000, seq_cap=4096)) == ffd.FFD_ERR_INVALID_ARG
    assert qa(ctypes.byref(d), A, 0, 64, 64, 3, A, A, A, A, None) == ffd.FFD_ERR_UNSUPPORTED
    assert qa(ctypes.byref(dims(dtype=ffd.FFD_F32)), A, 0, 64, 64, 2, A, A, A, A, None) == \
        ffd.FFD_ERR_UNSUPPORTED
    assert qa(ctypes.byref(d), A, 0, 64, 64, 2, A, A, None, A, None) == ffd.FFD_ERR_INVALID_ARG
    assert qa(ctypes.byref(d), A, 0, 63, 64, 2, A, A, A, A, None) == ffd.FFD_OK  # no block


def test_decode_loop_validation(L):
    """ffd_append_token and the per-sequence-length decode calls reject bad arguments before any
    launch (so the fake pointers are never dereferenced)."""
    d = dims()
    lens = ctypes.c_void_p(0x20000)
    lens_odd = ctypes.c_void_p(0x20002)
    app = L.ffd_append_token
    assert app(ctypes.byref(d), None, A, A, A, lens, 64, A, A, None) == ffd.FFD_ERR_INVALID_ARG
    assert app(ctypes.byref(d), A, A, A, A, None, 64, A, A, None) == ffd.FFD_ERR_INVALID_ARG
    assert app(ctypes.byref(d), A, A, A, A, lens_odd, 64, A, A, None) == ffd.FFD_ERR_INVALID_ARG
    assert app(ctypes.byref(d), A, MISALIGNED, A, A, lens, 64, A, A, None) == \
        ffd.FFD_ERR_INVALID_ARG
    assert app(ctypes.byref(d), A, A, A, A, lens, 96, A, A, None) == ffd.FFD_ERR_UNSUPPORTED
    assert app(ctypes.byref(dims(B=0)), A, A, A, A, lens, 64, A, A, None) == ffd.FFD_OK

    sv = L.ffd_decode_sparse_varlen
    assert sv(ctypes.byref(d), A, A, A, A, A, None, 5.0, 64, A, A, None, A, 1 << 30,
              None) == ffd.FFD_ERR_INVALID_ARG
    assert sv(ctypes.byref(d), A, A, A, A, A, lens_odd, 5.0, 64, A, A, None, A, 1 << 30,
              None) == ffd.FFD_ERR_INVALID_ARG
    assert sv(ctypes.byref(d), A, A, A, A, A, lens, float("nan"), 64, A, A, None, A, 1 << 30,
              None) == ffd.FFD_ERR_INVALID_ARG
    assert sv(ctypes.byref(d), A, A, A, A, A, lens, 5.0, 64, A, A, None, A, 16,
              None) == ffd.FFD_ERR_WORKSPACE
    dv = L.ffd_decode_dense_varlen
    assert dv(ctypes.byref(d), A, A, A, None, 64, A, A, A, 1 << 30, None) == \
        ffd.FFD_ERR_INVALID_ARG
    assert dv(ctypes.byref(d), A, A, A, lens, 64, A, A, A, 16, None) == ffd.FFD_ERR_WORKSPACE

    # the fused decode-loop step: (dims, q, k_new, v_new, K, V, Kq, scales, seq_lens, delta,
    # block, out, lse, keep_mask, workspace, bytes, stream)
    fs = L.ffd_decode_sparse_append

    def fused(dd=d, k_new=A, v_new=A, K=A, seq=lens, delta=5.0, block=64, ws_bytes=1 << 30):
        return fs(ctypes.byref(dd), A, k_new, v_new, K, A, A, A, seq, delta, block, A, A, None,
                  A, ws_bytes, None)
    assert fused(seq=None) == ffd.FFD_ERR_INVALID_ARG
    assert fused(k_new=None) == ffd.FFD_ERR_INVALID_ARG
    assert fused(v_new=None) == ffd.FFD_ERR_INVALID_ARG
    assert fused(K=None) == ffd.FFD_ERR_INVALID_ARG
    assert fused(k_new=MISALIGNED) == ffd.FFD_ERR_INVALID_ARG
    assert fused(seq=lens_odd) == ffd.FFD_ERR_INVALID_ARG
    assert fused(delta=float("nan")) == ffd.FFD_ERR_INVALID_ARG
    assert fused(block=96) == ffd.FFD_ERR_UNSUPPORTED
    assert fused(ws_bytes=16) == ffd.FFD_ERR_WORKSPACE
    # the per-sequence counts need B slots above the work units' (65535 in all)
    many = dims(B=32768, Hq=1, Hkv=1, seq_len=64, seq_cap=64)
    assert fused(dd=many) == ffd.FFD_ERR_UNSUPPORTED
    assert sv(ctypes.byref(many), A, A, A, A, A, lens, 5.0, 64, A, A, None, A, 16,
              None) == ffd.FFD_ERR_WORKSPACE  # the varlen step itself takes that shape
    assert fused(dd=dims(B=0)) == ffd.FFD_OK


def test_comparator_validation(L):
    """Block scores, selection rules and masked decode reject bad arguments before any launch."""
    d = dims()
    sc = L.ffd_block_scores
    assert sc(ctypes.byref(d), 3, A, A, A, A, A, A, 64, A, None) == ffd.FFD_ERR_INVALID_ARG
    assert sc(ctypes.byref(d), 0, A, A, None, A, None, None, 64, A, None) == ffd.FFD_ERR_INVALID_ARG
    assert sc(ctypes.byref(d), 1, A, A, A, A, None, A, 64, A, None) == ffd.FFD_ERR_INVALID_ARG
    assert sc(ctypes.byref(d), 2, A, None, None, None, None, None, 64, A, None) == \
        ffd.FFD_ERR_INVALID_ARG
    assert sc(ctypes.byref(d), 2, A, A, None, None, None, None, 64, None, None) == \
        ffd.FFD_ERR_INVALID_ARG
    sel = L.ffd_select_blocks
    assert sel(ctypes.byref(d), 3, A, None, 1.0, 64, A, None) == ffd.FFD_ERR_INVALID_ARG
    assert sel(ctypes.byref(d), 0, A, None, -1.0, 64, A, None) == ffd.FFD_ERR_INVALID_ARG
    assert sel(ctypes.byref(d), 0, A, None, float("nan"), 64, A, None) == ffd.FFD_ERR_INVALID_ARG
    assert sel(ctypes.byref(d), 1, A, None, -2.0, 64, A, None) == ffd.FFD_ERR_INVALID_ARG
    assert sel(ctypes.byref(d), 2, A, None, 0.0, 64, A, None) == ffd.FFD_ERR_INVALID_ARG
    assert sel(ctypes.byref(d), 2, A, None, 1.5, 64, A, None) == ffd.FFD_ERR_INVALID_ARG
    assert sel(ctypes.byref(d), 1, None, None, 4.0, 64, A, None) == ffd.FFD_ERR_INVALID_ARG
    big = dims(seq_len=16385 * 64, seq_cap=16385 * 64)
    assert sel(ctypes.byref(big), 1, A, None, 4.0, 64, A, None) == ffd.FFD_ERR_UNSUPPORTED
    assert sel(ctypes.byref(big), 2, A, None, 0.5, 64, A, None) == ffd.FFD_ERR_UNSUPPORTED
    dm = L.ffd_decode_masked
    assert dm(ctypes.byref(d), A, A, A, None, 64, A, A, A, 1 << 30, None) == \
        ffd.FFD_ERR_INVALID_ARG
    assert dm(ctypes.byref(d), A, A, A, A, 64, A, A, A, 16, None) == ffd.FFD_ERR_WORKSPACE
    bb = L.ffd_block_bounds
    assert bb(ctypes.byref(d), A, 0, 4096, 64, None, A, None) == ffd.FFD_ERR_INVALID_ARG
    assert bb(ctypes.byref(d), A, 0, 4097, 64, A, A, None) == ffd.FFD_ERR_INVALID_ARG
    assert bb(ctypes.byref(d), A, 0, 4096, 96, A, A, None) == ffd.FFD_ERR_UNSUPPORTED


def test_running_validation(L):
    """The running-max step rejects bad windows and small workspaces before any launch."""
    d = dims()  # 4096 tokens: 64 blocks of 64
    run = L.ffd_decode_sparse_running
    for window in (0, -3, 257):
        assert run(ctypes.byref(d), A, A, A, A, A, 5.0, 64, window, A, A, None, A, 1 << 30,
                   None) == ffd.FFD_ERR_UNSUPPORTED
        assert L.ffd_workspace_bytes_window(ctypes.byref(d), 64, window) == 0
    assert run(ctypes.byref(d), A, A, A, A, A, float("nan"), 64, 8, A, A, None, A, 1 << 30,
               None) == ffd.FFD_ERR_INVALID_ARG
    assert run(ctypes.byref(d), A, A, A, None, A, 5.0, 64, 8, A, A, None, A, 1 << 30,
               None) == ffd.FFD_ERR_INVALID_ARG
    need = L.ffd_workspace_bytes_window(ctypes.byref(d), 64, 8)
    assert need > 0
    # fewer, longer windows need no more workspace than more, shorter ones
    assert L.ffd_workspace_bytes_window(ctypes.byref(d), 64, 64) <= need
    assert run(ctypes.byref(d), A, A, A, A, A, 5.0, 64, 8, A, A, None, A, need - 16,
               None) == ffd.FFD_ERR_WORKSPACE
    # more than 256 windows
    big = dims(seq_len=257 * 64, seq_cap=257 * 64)
    assert run(ctypes.byref(big), A, A, A, A, A, 5.0, 64, 1, A, A, None, A, 1 << 30,
               None) == ffd.FFD_ERR_UNSUPPORTED
    assert L.ffd_workspace_bytes_window(ctypes.byref(big), 64, 1) == 0


def test_probe_library_exports_and_validates():
    """The measurement aid's header and library agree, and invalid arguments launch nothing."""
    from long_context_decoding_amd import probe
    if not probe.LIB_PATH.exists():
        pytest.skip("libffd_probe.so not built")
    header = Path(__file__).resolve().parents[1] / "include" / "ffd_probe.h"
    text = re.sub(r"/\*.*?\*/", "", header.read_text(), flags=re.S)
    names = set(re.findall(r"\b(ffd_[a-z_0-9]+)\s*\(", text))
    assert names == {"ffd_probe_stream_read"}
    nm = subprocess.run(["nm", "-D", "--defined-only", str(probe.LIB_PATH)], capture_output=True,
                        text=True, check=True).stdout
    assert names <= set(re.findall(r"\bT (ffd_\w+)", nm))
    f = probe.lib().ffd_probe_stream_read
    assert f(None, 1024, 4, A, None) == 1
    assert f(A, 1024, 4, None, None) == 1
    assert f(MISALIGNED, 1024, 4, A, None) == 1
    assert f(A, 1000, 4, A, None) == 1
    assert f(A, 0, 4, A, None) == 1
    assert f(A, 1024, 0, A, None) == 1
    assert f(A, 1024, 65536, A, None) == 1
