"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

Bar: Kq / scales byte-exact, keep masks bit-exact, out and lse within 2e-3 (bf16 q/K/V) or 1e-5
(fp32) absolute.  Small cases span several blocks, every group size, both block sizes and a
ragged tail; the named workloads run at full size in the same launch configuration as the
benchmark, with masks compared for every head and outputs for sampled heads.
"""
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from conftest import log
from helpers import (DEV, TOL, assert_close, gpu_dense, gpu_quantize, gpu_sparse, oracle_attend,
                     oracle_masks, sample_heads, to_host, upload)
from long_context_decoding_amd import ffd
from long_context_decoding_amd import workloads as W

pytestmark = pytest.mark.gpu

INF = float("inf")
DELTAS = (0.0, 0.5, 2.0, 5.0, INF)

CASES = ([(dt, G, T, L)
          for dt in ("bf16", "f32")
          for G in (1, 2, 4, 8)
          for T in (64, 128)
          for L in (T, 2 * T, 3 * T + 17, 20 * T + 5)]
         # group sizes the kernels run padded (3 as 4; 5, 6, 7 as 8)
         + [(dt, G, T, L)
            for dt in ("bf16", "f32")
            for G in (3, 5, 6, 7)
            for T in (64, 128)
            for L in (T, 3 * T + 17, 20 * T + 5)]
         # groups wider than the kernel: cut into units of 8 heads (9 = 8 + 1, 12 = 8 + 4,
         # 16 = 8 + 8)
         + [(dt, G, T, L)
            for dt in ("bf16", "f32")
            for G in (9, 12, 16)
            for T in (64, 128)
            for L in (3 * T + 17, 20 * T + 5)])


def small_case(dt, G, T, L):
    B = 2 if (G + L) % 2 == 0 else 1
    Hkv = 2 if G <= 4 or G % 3 == 0 else 1
    plant = "powerlaw" if (L // T) % 2 == 0 else "needles"
    seed = 1000 * G + 7 * T + L + (0 if dt == "bf16" else 1)
    return W.small(f"case_{dt}_G{G}_T{T}_L{L}", B=B, Hq=G * Hkv, Hkv=Hkv, L=L, T=T, dtype=dt,
                   seed=seed, plant=plant)


def oracle_quantize(w, K):
    return oracle.quantize_k(K, w.T, 0, w.L)


@pytest.mark.parametrize("dt,G,T,L", CASES)
def test_small_sparse_and_dense(dt, G, T, L):
    w = small_case(dt, G, T, L)
    q, K, V, _ = W.make_inputs(w)
    log(f"[gpu] {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv}")
    qd, Kd, Vd = upload(w, q, K, V)
    Kq_d, sc_d = gpu_quantize(w, Kd)
    Kq, sc = oracle_quantize(w, K)
    np.testing.assert_array_equal(Kq_d.cpu().numpy(), Kq)
    np.testing.assert_array_equal(to_host(sc_d), sc)
    tol = TOL[dt]
    for delta in DELTAS:
        out, lse, keep = gpu_sparse(w, qd, Kd, Vd, Kq_d, sc_d, delta)
        ref = oracle.decode(q, K, V, w.L, w.T, delta=delta, Kq=Kq, scales=sc)
        np.testing.assert_array_equal(keep, ref["keep"], err_msg=f"mask delta={delta}")
        assert_close(out, ref["out"], tol, f"out delta={delta}")
        assert_close(lse, ref["lse"], tol, f"lse delta={delta}")
    out, lse = gpu_dense(w, qd, Kd, Vd)
    ref = oracle.decode(q, K, V, w.L, w.T, sparse=False)
    assert_close(out, ref["out"], tol, "dense out")
    assert_close(lse, ref["lse"], tol, "dense lse")


def test_append_incremental_equals_one_shot():
    w = W.small("append", B=2, Hq=8, Hkv=2, L=9 * 64 + 30, T=64, seed=5)
    q, K, V, _ = W.make_inputs(w)
    _, Kd, _ = upload(w, q, K, V)
    Kq1, sc1 = gpu_quantize(w, Kd)
    Kq2, sc2 = ffd.alloc_kq(Kd, w.T)
    bounds = [0, 1, 63, 64, 65, 200, 383, 384, 500, w.L]
    for a, b in zip(bounds[:-1], bounds[1:]):
        ffd.quantize_k_append(Kd, a, b, w.T, Kq2, sc2, seq_len=w.L)
    torch.cuda.synchronize()
    assert torch.equal(Kq1, Kq2) and torch.equal(sc1, sc2)
    Kq, sc = oracle.quantize_k(K, w.T, 0, w.L)
    np.testing.assert_array_equal(Kq2.cpu().numpy(), Kq)


def oracle_quantize_threaded(w, K, slices):
    Kq = np.zeros((w.B, w.Hkv, w.cap, w.d // 2), np.uint8)
    sc = np.zeros((w.B, w.Hkv, w.cap // w.T, w.d), np.uint16)

    def one(bg):
        b, g = bg
        oracle.quantize_k(K[b:b + 1, g:g + 1], w.T, 0, w.L, Kq=Kq[b:b + 1, g:g + 1],
                          scales=sc[b:b + 1, g:g + 1])

    with ThreadPoolExecutor(16) as ex:
        list(ex.map(one, slices))
    return Kq, sc


@pytest.mark.parametrize("name", list(W.WORKLOADS) + list(W.EXTRA_WORKLOADS))
def test_named_workload_full_size(name):
    """Full size, in the benchmark's launch configuration: Kq and scales byte-exact, masks of
    every head bit-exact, out and lse of every head within the tolerance, sparse and dense."""
    w = W.WORKLOADS.get(name) or W.EXTRA_WORKLOADS[name]
    log(f"[gpu] full-size {name}: generating")
    q, K, V, info = W.make_inputs(w)
    all_slices = [(b, g) for b in range(w.B) for g in range(w.Hkv)]
    log(f"[gpu] full-size {name}: oracle quantize")
    Kq, sc = oracle_quantize_threaded(w, K, all_slices)
    log(f"[gpu] full-size {name}: upload + quantize on GPU")
    qd, Kd, Vd = upload(w, q, K, V)
    Kq_d, sc_d = gpu_quantize(w, Kd)
    torch.cuda.synchronize()
    assert torch.equal(Kq_d.cpu(), torch.from_numpy(Kq)), "Kq bytes differ"
    assert (to_host(sc_d) == sc).all(), "scales differ"
    heads = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    tol = TOL[w.dtype]
    for delta in w.deltas:
        log(f"[gpu] full-size {name}: sparse delta={delta}")
        out, lse, keep = gpu_sparse(w, qd, Kd, Vd, Kq_d, sc_d, delta)
        ref_keep = oracle_masks(w, q, Kq, sc, delta)
        np.testing.assert_array_equal(keep, ref_keep, err_msg=f"{name} mask delta={delta}")
        ref = oracle_attend(w, q, K, V, heads, keep=ref_keep)
        for (b, h) in heads:
            assert_close(out[b, h], ref[(b, h)][0], tol, f"{name} out b={b} h={h}")
            assert_close(lse[b, h], ref[(b, h)][1], tol, f"{name} lse b={b} h={h}")
        log(f"[gpu] full-size {name}: delta={delta} union keep "
            f"{keep.reshape(w.B, w.Hkv, w.G, -1).max(axis=2).mean():.4f}")
    log(f"[gpu] full-size {name}: dense")
    out, lse = gpu_dense(w, qd, Kd, Vd)
    ref = oracle_attend(w, q, K, V, heads, keep=None)
    for (b, h) in heads:
        assert_close(out[b, h], ref[(b, h)][0], tol, f"{name} dense out b={b} h={h}")
        assert_close(lse[b, h], ref[(b, h)][1], tol, f"{name} dense lse b={b} h={h}")
    del qd, Kd, Vd, Kq_d, sc_d
    torch.cuda.empty_cache()


@pytest.mark.parametrize("L,T", [(4096, 64), (4096 + 3 * 64 + 9, 64), (8192, 128)])
def test_short_context_one_block_per_wave(L, T):
    """The 32/8-head shape with a sink block and 0.5% needle blocks at short contexts, where the
    sparse step runs one scan block per wave and so fewer splits than the dense step (a ragged
    tail among them): Kq and scales byte-exact, every head's mask bit-exact, out and lse within
    the tolerance, sparse and dense."""
    base = W.WORKLOADS["gqa4_256k_sink_needles"]
    nb = L // T
    w = base.with_(name=f"short_L{L}_T{T}", L=L, T=T, n_needles=max(1, round(0.005 * nb)),
                   seed=base.seed + 3 * L + T)
    q, K, V, _ = W.make_inputs(w)
    qd, Kd, Vd = upload(w, q, K, V)
    dims = ffd.dims_of(qd, Kd, w.L)
    S, Sd = ffd.num_splits(dims, T), ffd.num_splits(dims, T, False)
    log(f"[gpu] {w.name}: sparse splits {S}, dense splits {Sd}")
    assert S == -(-L // T) // 4 and S < Sd
    Kq_d, sc_d = gpu_quantize(w, Kd)
    Kq, sc = oracle_quantize(w, K)
    np.testing.assert_array_equal(Kq_d.cpu().numpy(), Kq)
    np.testing.assert_array_equal(to_host(sc_d), sc)
    tol = TOL[w.dtype]
    for delta in (2.0, 5.0):
        out, lse, keep = gpu_sparse(w, qd, Kd, Vd, Kq_d, sc_d, delta)
        ref = oracle.decode(q, K, V, w.L, w.T, delta=delta, Kq=Kq, scales=sc)
        np.testing.assert_array_equal(keep, ref["keep"], err_msg=f"mask delta={delta}")
        assert_close(out, ref["out"], tol, f"out delta={delta}")
        assert_close(lse, ref["lse"], tol, f"lse delta={delta}")
    out, lse = gpu_dense(w, qd, Kd, Vd)
    ref = oracle.decode(q, K, V, w.L, w.T, sparse=False)
    assert_close(out, ref["out"], tol, "dense out")
    assert_close(lse, ref["lse"], tol, "dense lse")


# --------------------------------------------------------------------------------------------
# Properties of the HIP path itself
# --------------------------------------------------------------------------------------------
@pytest.fixture(scope="module")
def mid_case():
    w = W.WORKLOADS["gqa4_32k_sink_needles"].with_(L=200 * 64 + 33, B=2)
    q, K, V, _ = W.make_inputs(w)
    qd, Kd, Vd = upload(w, q, K, V)
    Kq_d, sc_d = gpu_quantize(w, Kd)
    return w, (q, K, V), (qd, Kd, Vd, Kq_d, sc_d)


def test_delta_inf_equals_dense(mid_case):
    w, _, (qd, Kd, Vd, Kq_d, sc_d) = mid_case
    out, lse, keep = gpu_sparse(w, qd, Kd, Vd, Kq_d, sc_d, INF)
    assert keep.all()
    out2, lse2 = gpu_dense(w, qd, Kd, Vd)
    assert_close(out, out2, 1e-5, "sparse(inf) vs dense out")
    assert_close(lse, lse2, 1e-5, "sparse(inf) vs dense lse")


def test_masks_nested_in_delta(mid_case):
    w, _, (qd, Kd, Vd, Kq_d, sc_d) = mid_case
    prev = None
    for delta in (0.0, 1.0, 3.0, 5.0, 8.0, 12.0):
        _, _, keep = gpu_sparse(w, qd, Kd, Vd, Kq_d, sc_d, delta)
        if prev is not None:
            assert (keep >= prev).all(), f"mask not monotone at delta={delta}"
        prev = keep


@pytest.mark.parametrize("splits", ["1", "2", "7", "33"])
def test_split_invariance(mid_case, splits, monkeypatch):
    w, _, (qd, Kd, Vd, Kq_d, sc_d) = mid_case
    out0, lse0, keep0 = gpu_sparse(w, qd, Kd, Vd, Kq_d, sc_d, 5.0)
    d0, dl0 = gpu_dense(w, qd, Kd, Vd)
    monkeypatch.setenv("FFD_NUM_SPLITS", splits)
    dims = ffd.dims_of(qd, Kd, w.L)
    log(f"[gpu] split invariance S={ffd.num_splits(dims, w.T)}")
    out, lse, keep = gpu_sparse(w, qd, Kd, Vd, Kq_d, sc_d, 5.0)
    np.testing.assert_array_equal(keep, keep0)
    assert_close(out, out0, 1e-5, "out vs default split")
    assert_close(lse, lse0, 1e-5, "lse vs default split")
    d, dl = gpu_dense(w, qd, Kd, Vd)
    assert_close(d, d0, 1e-5, "dense out vs default split")


def test_side_stream_without_workspace(mid_case):
    """A call on a non-default stream with no workspace given: the binding allocates and
    prepares the temporary workspace on that stream, so the result equals the oracle's."""
    w, (q, K, V), (qd, Kd, Vd, Kq_d, sc_d) = mid_case
    Kq, sc = oracle.quantize_k(K, w.T, 0, w.L)
    ref = oracle.decode(q, K, V, w.L, w.T, delta=5.0, Kq=Kq, scales=sc)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for i in range(3):
        keep = torch.full((w.B, w.Hq, w.n_blocks), 7, dtype=torch.uint8, device=DEV)
        side.wait_stream(torch.cuda.current_stream())
        out, lse = ffd.decode_sparse(qd, Kd, Vd, Kq_d, sc_d, 5.0, w.T, w.L, keep_mask=keep,
                                     stream=side)
        # other work on the current stream meanwhile allocates and fills fresh memory
        junk = torch.full((1 << 20,), float("nan"), device=DEV)
        del junk
        side.synchronize()
        np.testing.assert_array_equal(keep.cpu().numpy(), ref["keep"])
        assert_close(out.cpu().numpy(), ref["out"], TOL[w.dtype], f"out call {i}")
        assert_close(lse.cpu().numpy(), ref["lse"], TOL[w.dtype], f"lse call {i}")
    torch.cuda.synchronize()


def test_deterministic(mid_case):
    w, _, (qd, Kd, Vd, Kq_d, sc_d) = mid_case
    a = gpu_sparse(w, qd, Kd, Vd, Kq_d, sc_d, 5.0)
    b = gpu_sparse(w, qd, Kd, Vd, Kq_d, sc_d, 5.0)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_errors_launch_nothing(mid_case):
    w, _, (qd, Kd, Vd, Kq_d, sc_d) = mid_case
    with pytest.raises(ffd.FFDError) as e:
        ffd.decode_sparse(qd, Kd, Vd, Kq_d, sc_d, float("nan"), w.T, w.L)
    assert e.value.status == ffd.FFD_ERR_INVALID_ARG
    small_ws = torch.empty(64, dtype=torch.uint8, device=DEV)
    with pytest.raises(ffd.FFDError) as e:
        ffd.decode_sparse(qd, Kd, Vd, Kq_d, sc_d, 5.0, w.T, w.L, workspace=small_ws)
    assert e.value.status == ffd.FFD_ERR_WORKSPACE
    with pytest.raises(ffd.FFDError) as e:
        ffd.decode_dense(qd, Kd, Vd, 96, w.L)
    assert e.value.status in (ffd.FFD_ERR_UNSUPPORTED, ffd.FFD_ERR_INVALID_ARG)


def test_workspace_reuse_across_calls(mid_case):
    """One workspace serves many calls: each call returns its counters to zero."""
    w, _, (qd, Kd, Vd, Kq_d, sc_d) = mid_case
    dims = ffd.dims_of(qd, Kd, w.L)
    ws = ffd.alloc_workspace(dims, w.T, qd.device)
    ref_s = ffd.decode_sparse(qd, Kd, Vd, Kq_d, sc_d, 5.0, w.T, w.L)
    ref_d = ffd.decode_dense(qd, Kd, Vd, w.T, w.L)
    for i in range(6):
        if i % 2 == 0:
            o, l = ffd.decode_sparse(qd, Kd, Vd, Kq_d, sc_d, 5.0, w.T, w.L, workspace=ws)
            r = ref_s
        else:
            o, l = ffd.decode_dense(qd, Kd, Vd, w.T, w.L, workspace=ws)
            r = ref_d
        torch.cuda.synchronize()
        assert torch.equal(o, r[0]) and torch.equal(l, r[1]), f"call {i} differs"


def test_graph_replay_matches_eager(mid_case):
    """The decode calls can be recorded into a HIP graph; every replay equals the eager result."""
    w, _, (qd, Kd, Vd, Kq_d, sc_d) = mid_case
    dims = ffd.dims_of(qd, Kd, w.L)
    ws = ffd.alloc_workspace(dims, w.T, qd.device)
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=DEV)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=DEV)
    ref = ffd.decode_sparse(qd, Kd, Vd, Kq_d, sc_d, 5.0, w.T, w.L)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ffd.decode_sparse(qd, Kd, Vd, Kq_d, sc_d, 5.0, w.T, w.L, out=out, lse=lse, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ffd.decode_sparse(qd, Kd, Vd, Kq_d, sc_d, 5.0, w.T, w.L, out=out, lse=lse, workspace=ws)
        ffd.decode_sparse(qd, Kd, Vd, Kq_d, sc_d, 5.0, w.T, w.L, out=out, lse=lse, workspace=ws)
    for i in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1]), f"replay {i} differs"
        # eager work between replays on the same workspace
        ffd.decode_dense(qd, Kd, Vd, w.T, w.L, workspace=ws)
        torch.cuda.synchronize()


# --------------------------------------------------------------------------------------------
# Edge cases: no full block, spare cache capacity, the largest supported block count
# --------------------------------------------------------------------------------------------
@pytest.mark.parametrize("dt,T,L", [("bf16", 64, 17), ("bf16", 128, 127), ("f32", 64, 1)])
def test_no_full_block_keeps_everything(dt, T, L):
    w = W.small(f"short_{dt}_{T}_{L}", B=2, Hq=8, Hkv=2, L=L, T=T, dtype=dt, seed=L + T)
    q, K, V, _ = W.make_inputs(w)
    log(f"[gpu] {w.name}")
    qd, Kd, Vd = upload(w, q, K, V)
    Kq_d, sc_d = gpu_quantize(w, Kd)
    Kq, sc = oracle.quantize_k(K, w.T, 0, w.L)
    out, lse, keep = gpu_sparse(w, qd, Kd, Vd, Kq_d, sc_d, 0.0)
    ref = oracle.decode(q, K, V, w.L, w.T, delta=0.0, Kq=Kq, scales=sc)
    assert keep.all()
    np.testing.assert_array_equal(keep, ref["keep"])
    assert_close(out, ref["out"], TOL[dt], "out")
    assert_close(lse, ref["lse"], TOL[dt], "lse")


@pytest.mark.parametrize("T", [64, 128])
def test_spare_capacity_rows_are_ignored(T):
    """seq_cap well beyond L: the padding rows (NaN in the inputs) never reach the outputs."""
    L = 9 * T + 5
    w = W.small(f"cap_{T}", B=1, Hq=8, Hkv=2, L=L, T=T, seed=33, L_cap=16 * T)
    q, K, V, _ = W.make_inputs(w)
    log(f"[gpu] {w.name} cap={w.cap}")
    qd, Kd, Vd = upload(w, q, K, V)
    Kq_d, sc_d = gpu_quantize(w, Kd)
    Kq, sc = oracle.quantize_k(K, w.T, 0, w.L)
    np.testing.assert_array_equal(Kq_d.cpu().numpy()[:, :, :w.n_full * T], Kq[:, :, :w.n_full * T])
    for delta in (2.0, INF):
        out, lse, keep = gpu_sparse(w, qd, Kd, Vd, Kq_d, sc_d, delta)
        ref = oracle.decode(q, K, V, w.L, w.T, delta=delta, Kq=Kq, scales=sc)
        np.testing.assert_array_equal(keep, ref["keep"])
        assert_close(out, ref["out"], 2e-3, f"out delta={delta}")
        assert_close(lse, ref["lse"], 2e-3, f"lse delta={delta}")
    out, lse = gpu_dense(w, qd, Kd, Vd)
    ref = oracle.decode(q, K, V, w.L, w.T, sparse=False)
    assert_close(out, ref["out"], 2e-3, "dense out")


def test_largest_block_count():
    """65536 blocks of 64 tokens (4M tokens, the most one call supports): 256 splits, so the
    merge takes its general path; masks compared for the head, outputs against the oracle."""
    w = W.Workload("max_blocks", B=1, Hq=2, Hkv=1, L=256 * 256 * 64, T=64, plant="needles",
                   n_needles=40, needle_a=6.0, sink_a=10.0, seed=77)
    log(f"[gpu] {w.name}: generating {w.L} tokens")
    q, K, V, _ = W.make_inputs(w)
    qd, Kd, Vd = upload(w, q, K, V)
    Kq_d, sc_d = gpu_quantize(w, Kd)
    dims = ffd.dims_of(qd, Kd, w.L)
    assert ffd.num_splits(dims, w.T) == 256
    log(f"[gpu] {w.name}: sparse")
    out, lse, keep = gpu_sparse(w, qd, Kd, Vd, Kq_d, sc_d, 5.0)
    Kq, sc = oracle.quantize_k(K, w.T, 0, w.L)
    np.testing.assert_array_equal(Kq_d.cpu().numpy(), Kq)
    ref_keep = oracle_masks(w, q, Kq, sc, 5.0)
    np.testing.assert_array_equal(keep, ref_keep)
    ref = oracle_attend(w, q, K, V, [(0, 0), (0, 1)], keep=ref_keep)
    for h in range(2):
        assert_close(out[0, h], ref[(0, h)][0], 2e-3, f"out h={h}")
        assert_close(lse[0, h], ref[(0, h)][1], 2e-3, f"lse h={h}")
    del qd, Kd, Vd, Kq_d, sc_d
    torch.cuda.empty_cache()


def test_most_work_units():
    """65528 work units, near the 65535 a call supports: 8191 sequences of one kv head with a
    64-head query group, cut into 8 units of 8 heads each, 5 blocks of 64 tokens (block 0 the
    sink, block 4 the local block, one needle among blocks 1-3).  Masks are compared for every
    head of the first and last sequences and for sampled heads elsewhere; sparse and dense
    outputs for sampled heads."""
    w = W.Workload("max_units", B=8191, Hq=64, Hkv=1, L=5 * 64, T=64, plant="needles",
                   n_needles=1, needle_a=6.0, sink_a=10.0, seed=91)
    log(f"[gpu] {w.name}: generating {w.B} sequences")
    q, K, V, _ = W.make_inputs(w)
    qd, Kd, Vd = upload(w, q, K, V)
    dims = ffd.dims_of(qd, Kd, w.L)
    assert w.B * w.Hkv * (w.G // 8) == 65528
    Kq_d, sc_d = gpu_quantize(w, Kd)
    log(f"[gpu] {w.name}: sparse and dense")
    out, lse, keep = gpu_sparse(w, qd, Kd, Vd, Kq_d, sc_d, 5.0)
    out_dn, lse_dn = gpu_dense(w, qd, Kd, Vd)
    Kq, sc = oracle.quantize_k(K, w.T, 0, w.L)
    np.testing.assert_array_equal(Kq_d.cpu().numpy(), Kq)
    np.testing.assert_array_equal(to_host(sc_d), sc)
    out_heads = sample_heads(w, 96, seed=6) + [(w.B - 1, w.Hq - 1)]
    heads = sorted(set([(0, h) for h in range(w.Hq)] + [(w.B - 1, h) for h in range(w.Hq)]
                       + sample_heads(w, 1024, seed=5) + out_heads))
    ref_keep = oracle_masks(w, q, Kq, sc, 5.0, heads=heads)
    for b, h in heads:
        np.testing.assert_array_equal(keep[b, h], ref_keep[b, h], err_msg=f"mask b={b} h={h}")
    # every head keeps its sink and local blocks
    assert keep[:, :, 0].all() and keep[:, :, 4].all()
    ref = oracle_attend(w, q, K, V, out_heads, keep=ref_keep)
    ref_dn = oracle_attend(w, q, K, V, out_heads)
    for b, h in out_heads:
        assert_close(out[b, h], ref[(b, h)][0], 2e-3, f"out b={b} h={h}")
        assert_close(lse[b, h], ref[(b, h)][1], 2e-3, f"lse b={b} h={h}")
        assert_close(out_dn[b, h], ref_dn[(b, h)][0], 2e-3, f"dense out b={b} h={h}")
        assert_close(lse_dn[b, h], ref_dn[(b, h)][1], 2e-3, f"dense lse b={b} h={h}")
    del qd, Kd, Vd, Kq_d, sc_d
    torch.cuda.empty_cache()
