"""Decode-loop integration on the GPU ("Faster Than Flash" Sec. 3.3: one fused step per generated
token; Fig. 2: the key copy is quantized as blocks complete; App. G: the step replayed as a graph).

- per-sequence lengths read from device memory give, for every sequence, the oracle's result on
  that sequence's own prefix (masks bit-exact, out and lse within 2e-3);
- one captured step (ffd_append_token + ffd_decode_sparse_varlen, or the fused
  ffd_decode_sparse_append) replayed across several block boundaries matches, after every replay,
  the oracle run on a host mirror of the growing cache; the cache rows and the key copy of every
  completed block are byte-exact at the end;
- the fused step gives, step after step, the same bytes as the pair of calls: outputs, masks,
  caches, key copy and lengths, also for groups cut into several units, fp32, a sequence at the
  capacity and one that starts empty.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from conftest import log
from helpers import DEV, assert_close, to_dev, to_host
from long_context_decoding_amd import ffd
from long_context_decoding_amd import workloads as W

pytestmark = pytest.mark.gpu

INF = float("inf")
TOL = 2e-3


def bf16(x: np.ndarray) -> np.ndarray:
    return W.f32_to_bf16_bits(x.astype(np.float32))


@pytest.mark.parametrize("T,G", [(64, 4), (128, 1), (64, 8), (128, 2), (64, 7), (128, 6), (64, 16)])
def test_varlen_matches_oracle_per_sequence(T, G):
    Hkv = 2 if G <= 4 else 1
    cap = 12 * T
    w = W.small(f"varlen_T{T}_G{G}", B=5, Hq=G * Hkv, Hkv=Hkv, L=cap, T=T, seed=7 * T + G)
    q, K, V, _ = W.make_inputs(w)
    lens = np.array([cap, T, 3 * T + 17, 5, 7 * T], dtype=np.int32)
    log(f"varlen T={T} G={G} lens={lens.tolist()}")
    qd, Kd, Vd = to_dev(q), to_dev(K), to_dev(V)
    Kq, sc = ffd.alloc_kq(Kd, T)
    ffd.quantize_k_append(Kd, 0, cap, T, Kq, sc, seq_len=cap)
    Kq_o, sc_o = oracle.quantize_k(K, T)
    lens_d = torch.from_numpy(lens).to(DEV)
    nbc = cap // T
    for delta in (0.5, 5.0, INF):
        keep = torch.full((w.B, w.Hq, nbc), 7, dtype=torch.uint8, device=DEV)
        out, lse = ffd.decode_sparse_varlen(qd, Kd, Vd, Kq, sc, lens_d, delta, T, keep_mask=keep)
        outd, lsed = ffd.decode_dense_varlen(qd, Kd, Vd, lens_d, T)
        torch.cuda.synchronize()
        out, lse, keep = out.cpu().numpy(), lse.cpu().numpy(), keep.cpu().numpy()
        outd, lsed = outd.cpu().numpy(), lsed.cpu().numpy()
        for b, L in enumerate(lens):
            sl = slice(b, b + 1)
            ref = oracle.decode(q[sl], K[sl], V[sl], int(L), T, delta, Kq=Kq_o[sl], scales=sc_o[sl])
            nb = math.ceil(L / T)
            np.testing.assert_array_equal(keep[b, :, :nb], ref["keep"][0, :, :nb],
                                          err_msg=f"mask b={b} L={L} delta={delta}")
            assert (keep[b, :, nb:] == 7).all(), "entries past the sequence's blocks were written"
            assert_close(out[b], ref["out"][0], TOL, f"out b={b} L={L} delta={delta}")
            assert_close(lse[b], ref["lse"][0], TOL, f"lse b={b} L={L} delta={delta}")
            dref = oracle.decode(q[sl], K[sl], V[sl], int(L), T, sparse=False)
            assert_close(outd[b], dref["out"][0], TOL, f"dense out b={b} L={L}")
            assert_close(lsed[b], dref["lse"][0], TOL, f"dense lse b={b} L={L}")


def test_varlen_empty_sequence():
    T = 64
    w = W.small("varlen_empty", B=2, Hq=8, Hkv=2, L=4 * T, T=T, seed=3)
    q, K, V, _ = W.make_inputs(w)
    qd, Kd, Vd = to_dev(q), to_dev(K), to_dev(V)
    Kq, sc = ffd.alloc_kq(Kd, T)
    ffd.quantize_k_append(Kd, 0, 4 * T, T, Kq, sc, seq_len=4 * T)
    lens_d = torch.tensor([0, 2 * T + 3], dtype=torch.int32, device=DEV)
    out, lse = ffd.decode_sparse_varlen(qd, Kd, Vd, Kq, sc, lens_d, 5.0, T)
    outd, lsed = ffd.decode_dense_varlen(qd, Kd, Vd, lens_d, T)
    torch.cuda.synchronize()
    Kq_o, sc_o = oracle.quantize_k(K, T)
    L1 = 2 * T + 3
    ref = oracle.decode(q[1:2], K[1:2], V[1:2], L1, T, 5.0, Kq=Kq_o[1:2], scales=sc_o[1:2])
    dref = oracle.decode(q[1:2], K[1:2], V[1:2], L1, T, sparse=False)
    for (o, l), r in (((out, lse), ref), ((outd, lsed), dref)):
        o, l = o.cpu().numpy(), l.cpu().numpy()
        assert (o[0] == 0).all() and np.isneginf(l[0]).all(), "length 0: out = 0, lse = -inf"
        assert_close(o[1], r["out"][0], TOL, "out b=1")
        assert_close(l[1], r["lse"][0], TOL, "lse b=1")


def _loop_setup(B, Hq, Hkv, T, cap, init, seed):
    w = W.small("decode_loop", B=B, Hq=Hq, Hkv=Hkv, L=cap, T=T, seed=seed)
    q0, K, V, _ = W.make_inputs(w)
    K = K.copy()
    V = V.copy()
    for b, L in enumerate(init):  # rows past the initial lengths are written by the loop
        K[b, :, L:] = 0
        V[b, :, L:] = 0
    return w, q0, K, V


@pytest.mark.parametrize("fused", [False, True])
def test_graph_replayed_decode_loop(fused):
    B, Hq, Hkv, T, cap = 2, 8, 2, 64, 8 * 64
    init = [60, 126]
    n_steps, delta = 80, 5.0
    w, q0, K_host, V_host = _loop_setup(B, Hq, Hkv, T, cap, init, seed=11)
    rng = np.random.default_rng(20261202)
    q_f = W.bf16_bits_to_f32(q0)
    qs = bf16(q_f[None] + 0.3 * rng.standard_normal((n_steps, B, Hq, 128)))
    ks = bf16(rng.standard_normal((n_steps, B, Hkv, 128)))
    vs = bf16(rng.standard_normal((n_steps, B, Hkv, 128)))

    Kd, Vd = to_dev(K_host), to_dev(V_host)
    Kq, sc = ffd.alloc_kq(Kd, T)
    ffd.quantize_k_append(Kd, 0, cap, T, Kq, sc, seq_len=cap)
    q_buf = torch.empty((B, Hq, 128), dtype=torch.bfloat16, device=DEV)
    k_buf = torch.empty((B, Hkv, 128), dtype=torch.bfloat16, device=DEV)
    v_buf = torch.empty_like(k_buf)
    lens_d = torch.tensor(init, dtype=torch.int32, device=DEV)
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    keep = torch.zeros((B, Hq, cap // T), dtype=torch.uint8, device=DEV)
    ws = ffd.alloc_workspace(ffd.dims_of(q_buf, Kd, cap), T, DEV)

    # load the kernels once outside the capture: sequences at capacity are left untouched
    full = torch.full((B,), cap, dtype=torch.int32, device=DEV)
    q_buf.copy_(to_dev(qs[0]))

    def step(lens_t, **kw):
        if fused:
            ffd.decode_sparse_append(q_buf, k_buf, v_buf, Kd, Vd, Kq, sc, lens_t, delta, T, **kw)
        else:
            ffd.append_token(k_buf, v_buf, Kd, Vd, lens_t, T, Kq, sc)
            ffd.decode_sparse_varlen(q_buf, Kd, Vd, Kq, sc, lens_t, delta, T, **kw)

    step(full, workspace=ws)
    torch.cuda.synchronize()
    assert full.tolist() == [cap, cap]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(lens_d, out=out, lse=lse, keep_mask=keep, workspace=ws)
    lens = list(init)
    for step in range(n_steps):
        q_buf.copy_(to_dev(qs[step]))
        k_buf.copy_(to_dev(ks[step]))
        v_buf.copy_(to_dev(vs[step]))
        g.replay()
        torch.cuda.synchronize()
        for b in range(B):
            K_host[b, :, lens[b]] = ks[step, b]
            V_host[b, :, lens[b]] = vs[step, b]
            lens[b] += 1
        Kq_o, sc_o = oracle.quantize_k(K_host, T)
        o, l, kp = out.cpu().numpy(), lse.cpu().numpy(), keep.cpu().numpy()
        for b in range(B):
            sl = slice(b, b + 1)
            ref = oracle.decode(qs[step][sl], K_host[sl], V_host[sl], lens[b], T, delta,
                                Kq=Kq_o[sl], scales=sc_o[sl])
            nb = math.ceil(lens[b] / T)
            np.testing.assert_array_equal(kp[b, :, :nb], ref["keep"][0, :, :nb],
                                          err_msg=f"step {step} b={b} L={lens[b]}")
            assert_close(o[b], ref["out"][0], TOL, f"out step {step} b={b} L={lens[b]}")
            assert_close(l[b], ref["lse"][0], TOL, f"lse step {step} b={b} L={lens[b]}")
    log(f"decode loop (fused={fused}): {n_steps} graph replays, lengths {init} -> {lens}")
    assert lens_d.cpu().tolist() == lens
    K_dev = Kd.view(torch.int16).cpu().numpy().view(np.uint16)
    V_dev = Vd.view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(K_dev, K_host)
    np.testing.assert_array_equal(V_dev, V_host)
    Kq_o, sc_o = oracle.quantize_k(K_host, T)
    Kq_d, sc_d = Kq.cpu().numpy(), to_host(sc)
    for b in range(B):
        nf = lens[b] // T
        np.testing.assert_array_equal(Kq_d[b, :, :nf * T], Kq_o[b, :, :nf * T], err_msg=f"Kq b={b}")
        np.testing.assert_array_equal(sc_d[b, :, :nf], sc_o[b, :, :nf], err_msg=f"scales b={b}")


def test_append_at_capacity_is_a_noop():
    B, Hq, Hkv, T, cap = 2, 4, 1, 64, 2 * 64
    w, q0, K_host, V_host = _loop_setup(B, Hq, Hkv, T, cap, [cap, cap - 1], seed=2)
    Kd, Vd = to_dev(K_host), to_dev(V_host)
    Kq, sc = ffd.alloc_kq(Kd, T)
    ffd.quantize_k_append(Kd, 0, cap, T, Kq, sc, seq_len=cap)
    rng = np.random.default_rng(5)
    k_new = bf16(rng.standard_normal((B, Hkv, 128)))
    v_new = bf16(rng.standard_normal((B, Hkv, 128)))
    lens_d = torch.tensor([cap, cap - 1], dtype=torch.int32, device=DEV)
    for _ in range(2):
        ffd.append_token(to_dev(k_new), to_dev(v_new), Kd, Vd, lens_d, T, Kq, sc)
    torch.cuda.synchronize()
    assert lens_d.cpu().tolist() == [cap, cap]
    K_dev = Kd.view(torch.int16).cpu().numpy().view(np.uint16)
    expect = K_host.copy()
    expect[1, :, cap - 1] = k_new[1]
    np.testing.assert_array_equal(K_dev, expect)
    Kq_o, sc_o = oracle.quantize_k(expect, T)
    np.testing.assert_array_equal(Kq.cpu().numpy()[1], Kq_o[1])
    np.testing.assert_array_equal(to_host(sc)[1], sc_o[1])


@pytest.mark.parametrize("dtype,T,G,Hkv", [("bf16", 64, 4, 2), ("f32", 128, 1, 2),
                                           ("bf16", 64, 12, 1), ("bf16", 128, 8, 2)])
def test_fused_step_equals_append_then_decode(dtype, T, G, Hkv):
    B, cap = 4, 4 * T
    init = [T - 3, 2 * T - 2, cap, 0]  # crossing block boundaries, at the capacity, empty
    n_steps, delta = T + 6, 5.0
    w = W.small(f"fused_{dtype}_T{T}_G{G}", B=B, Hq=G * Hkv, Hkv=Hkv, L=cap, T=T, dtype=dtype,
                seed=5 * T + G)
    q, K, V, _ = W.make_inputs(w)
    log(f"fused step {dtype} T={T} G={G} Hkv={Hkv}: lengths {init}, {n_steps} steps")
    rng = np.random.default_rng(31 * T + G)
    new = rng.standard_normal((n_steps, 2, B, Hkv, 128)).astype(np.float32)
    if dtype == "bf16":
        new = bf16(new)
    qd = to_dev(q)
    caches = []
    for _ in range(2):
        Kd, Vd = to_dev(K), to_dev(V)
        Kq, sc = ffd.alloc_kq(Kd, T)
        ffd.quantize_k_append(Kd, 0, cap, T, Kq, sc, seq_len=cap)
        lens = torch.tensor(init, dtype=torch.int32, device=DEV)
        ws = ffd.alloc_workspace(ffd.dims_of(qd, Kd, cap), T, DEV)
        caches.append((Kd, Vd, Kq, sc, lens, ws))
    (Ka, Va, Kqa, sca, la, wsa), (Kb, Vb, Kqb, scb, lb, wsb) = caches
    nbc = cap // T
    for step in range(n_steps):
        kn, vn = to_dev(new[step, 0]), to_dev(new[step, 1])
        keep_a = torch.full((B, w.Hq, nbc), 7, dtype=torch.uint8, device=DEV)
        keep_b = keep_a.clone()
        ffd.append_token(kn, vn, Ka, Va, la, T, Kqa, sca)
        oa, lsa = ffd.decode_sparse_varlen(qd, Ka, Va, Kqa, sca, la, delta, T, keep_mask=keep_a,
                                           workspace=wsa)
        ob, lsb = ffd.decode_sparse_append(qd, kn, vn, Kb, Vb, Kqb, scb, lb, delta, T,
                                           keep_mask=keep_b, workspace=wsb)
        torch.cuda.synchronize()
        msg = f"step {step}, lengths {la.tolist()}"
        assert torch.equal(la, lb), msg
        assert torch.equal(keep_a, keep_b), msg
        assert torch.equal(oa, ob), msg
        assert torch.equal(lsa, lsb), msg
    for name, x, y in (("K", Ka, Kb), ("V", Va, Vb), ("Kq", Kqa, Kqb), ("scales", sca, scb)):
        assert torch.equal(x, y), name
    final = [min(L + n_steps, cap) if L < cap else L for L in init]
    assert lb.tolist() == final
    # and the whole loop against the oracle on the final cache (each sequence's own prefix)
    Kh, Vh = to_host(Kb), to_host(Vb)
    Kq_o, sc_o = oracle.quantize_k(Kh, T)
    o, l = ob.cpu().numpy(), lsb.cpu().numpy()
    for b, L in enumerate(final):
        nf = L // T
        np.testing.assert_array_equal(Kqb.cpu().numpy()[b, :, :nf * T], Kq_o[b, :, :nf * T])
        np.testing.assert_array_equal(to_host(scb)[b, :, :nf], sc_o[b, :, :nf])
        if L == 0:
            assert (o[b] == 0).all() and np.isneginf(l[b]).all()
            continue
        sl = slice(b, b + 1)
        ref = oracle.decode(q[sl], Kh[sl], Vh[sl], L, T, delta, Kq=Kq_o[sl], scales=sc_o[sl])
        tol = 2e-3 if dtype == "bf16" else 1e-5
        assert_close(o[b], ref["out"][0], tol, f"out b={b} L={L}")
        assert_close(l[b], ref["lse"][0], tol, f"lse b={b} L={L}")


def test_fused_step_streaming_kernels_128k():
    """The fused step at a length whose splits run the streaming-policy kernels (32 splits of 33
    blocks of 128), over the step that completes a block: bit-identical to the pair of calls at
    every step, and the last step against the oracle for every head."""
    T, Hkv, G = 128, 8, 4
    nbc = 1040
    cap = nbc * T
    init = 1025 * T - 2  # the second step completes block 1024
    n_steps, delta = 4, 5.0
    base = W.WORKLOADS["gqa4_256k_sink_needles"]
    w = base.with_(name="fused_stream_128k", L=cap, n_needles=5, seed=base.seed + 17)
    q, K, V, _ = W.make_inputs(w)
    qd = to_dev(q)
    caches = []
    for _ in range(2):
        Kd, Vd = to_dev(K), to_dev(V)
        Kq, sc = ffd.alloc_kq(Kd, T)
        ffd.quantize_k_append(Kd, 0, cap, T, Kq, sc, seq_len=cap)
        lens = torch.tensor([init], dtype=torch.int32, device=DEV)
        ws = ffd.alloc_workspace(ffd.dims_of(qd, Kd, cap), T, DEV)
        caches.append((Kd, Vd, Kq, sc, lens, ws))
    S = ffd.num_splits(ffd.dims_of(qd, caches[0][0], cap), T)
    assert S == 32 and -(-nbc // S) >= 32, "the splits must be long enough for the streaming kernels"
    log(f"fused step at 128K: {S} splits of {-(-nbc // S)} blocks, lengths from {init}")
    rng = np.random.default_rng(2026)
    new = bf16(rng.standard_normal((n_steps, 2, 1, Hkv, 128)).astype(np.float32))
    (Ka, Va, Kqa, sca, la, wsa), (Kb, Vb, Kqb, scb, lb, wsb) = caches
    for step in range(n_steps):
        kn, vn = to_dev(new[step, 0]), to_dev(new[step, 1])
        keep_a = torch.full((1, Hkv * G, nbc), 7, dtype=torch.uint8, device=DEV)
        keep_b = keep_a.clone()
        ffd.append_token(kn, vn, Ka, Va, la, T, Kqa, sca)
        oa, lsa = ffd.decode_sparse_varlen(qd, Ka, Va, Kqa, sca, la, delta, T, keep_mask=keep_a,
                                           workspace=wsa)
        ob, lsb = ffd.decode_sparse_append(qd, kn, vn, Kb, Vb, Kqb, scb, lb, delta, T,
                                           keep_mask=keep_b, workspace=wsb)
        torch.cuda.synchronize()
        msg = f"step {step}, length {la.tolist()}"
        assert torch.equal(la, lb), msg
        assert torch.equal(keep_a, keep_b), msg
        assert torch.equal(oa, ob), msg
        assert torch.equal(lsa, lsb), msg
    for name, x, y in (("K", Ka, Kb), ("V", Va, Vb), ("Kq", Kqa, Kqb), ("scales", sca, scb)):
        assert torch.equal(x, y), name
    L = init + n_steps
    assert lb.tolist() == [L]
    # the last step against the oracle over the grown cache
    Kh, Vh = to_host(Kb), to_host(Vb)
    nf = L // T
    Kq_o, sc_o = oracle.quantize_k(Kh, T, 0, L)
    np.testing.assert_array_equal(Kqb.cpu().numpy()[:, :, :nf * T], Kq_o[:, :, :nf * T])
    np.testing.assert_array_equal(to_host(scb)[:, :, :nf], sc_o[:, :, :nf])
    ref = oracle.decode(q, Kh, Vh, L, T, delta, Kq=Kq_o, scales=sc_o)
    np.testing.assert_array_equal(keep_b.cpu().numpy()[:, :, :-(-L // T)], ref["keep"])
    assert_close(ob.cpu().numpy(), ref["out"], TOL, "out")
    assert_close(lsb.cpu().numpy(), ref["lse"], TOL, "lse")
