"""GPU parity of the residual storage form (low-bit thumbnail + 8-bit residual instead of 16-bit
keys; "Faster Than Flash" Sec. 3.1, Fig. 2, Alg. 1 Dequant, Eq. 4) against the CPU oracle.

Bar: thumbnail codes, scales, residual codes and residual scales byte-exact; keep masks bit-exact;
out and lse within 2e-3 absolute (bf16 q and V; fp32 accumulation against the fp64 oracle over
the same Dequant keys).
"""
import numpy as np
import pytest
import torch

import oracle
from conftest import log
from helpers import DEV, assert_close, oracle_attend, to_dev, to_host, upload
from long_context_decoding_amd import ffd
from long_context_decoding_amd import workloads as W

pytestmark = pytest.mark.gpu

INF = float("inf")
TOL = 2e-3

CASES = ([(bits, G, T, L)
          for bits in (2, 4)
          for G in (1, 4, 8)
          for T in (64, 128)
          for L in (T, 3 * T + 17, 20 * T + 5)] + [(2, 2, 64, 64 * 7), (4, 2, 128, 128 * 5 + 99)]
         # padded groups (3 as 4, 7 as 8) and a group cut into two units of 8
         + [(bits, G, T, 20 * T + 5) for bits in (2, 4) for G in (3, 7, 16) for T in (64, 128)])


def gpu_kres(w, Kd, bits, tok_begin=0, tok_end=None, kres=None):
    if kres is None:
        kres = ffd.alloc_kres(Kd, w.T, bits)
    ffd.quantize_k_residual_append(Kd, tok_begin, w.L if tok_end is None else tok_end, w.T, bits,
                                   kres, seq_len=w.L)
    return kres


def gpu_sparse_res(w, qd, Kd, Vd, kres, bits, delta, pass_tail=True):
    keep = torch.full((w.B, w.Hq, w.n_blocks), 7, dtype=torch.uint8, device=DEV)
    out, lse = ffd.decode_sparse_residual(qd, Kd if pass_tail else None, Vd, kres, bits, delta,
                                          w.T, w.L, keep_mask=keep)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), keep.cpu().numpy()


def check_kres(kres_d, kres_o, n_rows):
    names = ("Kc", "scales", "Kr", "res_scales")
    for name, a, b in zip(names, kres_d, kres_o):
        a = to_host(a)
        if name in ("Kc", "Kr"):
            a, b = a[:, :, :n_rows], b[:, :, :n_rows]
        np.testing.assert_array_equal(a, b, err_msg=name)


@pytest.mark.parametrize("bits,G,T,L", CASES)
def test_small_residual(bits, G, T, L):
    Hkv = 2 if G <= 4 else 1
    w = W.small(f"res_b{bits}_G{G}_T{T}_L{L}", B=2 if G < 7 else 1, Hq=G * Hkv, Hkv=Hkv, L=L, T=T,
                seed=100 * bits + 10 * G + L, plant="powerlaw" if (L // T) % 2 else "needles")
    q, K, V, _ = W.make_inputs(w)
    log(f"[gpu] {w.name}")
    qd, Kd, Vd = upload(w, q, K, V)
    kres_d = gpu_kres(w, Kd, bits)
    kres_o = oracle.quantize_k_res(K, w.T, bits, 0, w.L)
    check_kres(kres_d, kres_o, w.n_full * T)
    for delta in (0.0, 2.0, 5.0, INF):
        out, lse, keep = gpu_sparse_res(w, qd, Kd, Vd, kres_d, bits, delta)
        ref = oracle.decode_res(q, K, V, *kres_o, w.L, w.T, bits, delta=delta)
        np.testing.assert_array_equal(keep, ref["keep"], err_msg=f"mask delta={delta}")
        assert_close(out, ref["out"], TOL, f"out delta={delta}")
        assert_close(lse, ref["lse"], TOL, f"lse delta={delta}")


def test_residual_without_tail_buffer():
    w = W.small("res_notail", B=1, Hq=8, Hkv=2, L=9 * 64, T=64, seed=9)
    q, K, V, _ = W.make_inputs(w)
    qd, Kd, Vd = upload(w, q, K, V)
    kres_d = gpu_kres(w, Kd, 2)
    a = gpu_sparse_res(w, qd, Kd, Vd, kres_d, 2, 5.0, pass_tail=True)
    b = gpu_sparse_res(w, qd, Kd, Vd, kres_d, 2, 5.0, pass_tail=False)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    w2 = w.with_(L=9 * 64 + 3)
    dims = ffd.dims_of(qd, Vd, w2.L)
    with pytest.raises(ffd.FFDError) as e:
        ffd.decode_sparse_residual(qd, None, Vd, kres_d, 2, 5.0, 64, w2.L)
    assert e.value.status == ffd.FFD_ERR_INVALID_ARG


def test_residual_append_incremental_equals_one_shot():
    w = W.small("res_append", B=2, Hq=8, Hkv=2, L=9 * 64 + 30, T=64, seed=5)
    q, K, V, _ = W.make_inputs(w)
    _, Kd, _ = upload(w, q, K, V)
    one = gpu_kres(w, Kd, 2)
    inc = ffd.alloc_kres(Kd, w.T, 2)
    bounds = [0, 1, 63, 64, 65, 200, 383, 384, 500, w.L]
    for a, b in zip(bounds[:-1], bounds[1:]):
        gpu_kres(w, Kd, 2, a, b, kres=inc)
    torch.cuda.synchronize()
    for x, y in zip(one, inc):
        assert torch.equal(x, y)


@pytest.mark.parametrize("name,bits", [("gqa4_256k_sink_needles", 2), ("gqa4_256k_sink_needles", 4),
                                       ("gqa4_32k_sink_needles", 2),
                                       ("b8_gqa4_128k_powerlaw", 2)])
def test_named_workload_residual(name, bits):
    w = W.WORKLOADS[name]
    log(f"[gpu] residual {name} bits={bits}: generating")
    q, K, V, _ = W.make_inputs(w)
    qd, Kd, Vd = upload(w, q, K, V)
    kres_d = gpu_kres(w, Kd, bits)
    torch.cuda.synchronize()
    log(f"[gpu] residual {name}: oracle quantize")
    np_of = {torch.uint8: np.uint8, torch.float32: np.float32, torch.bfloat16: np.uint16,
             torch.int8: np.int8}
    kres_o = tuple(np.zeros(t.shape, dtype=np_of[t.dtype]) for t in kres_d)
    from concurrent.futures import ThreadPoolExecutor

    def one(bg):
        b, g = bg
        sl = tuple(a[b:b + 1, g:g + 1] for a in kres_o)
        oracle.quantize_k_res(K[b:b + 1, g:g + 1], w.T, bits, 0, w.L, out=sl)

    with ThreadPoolExecutor(16) as ex:
        list(ex.map(one, [(b, g) for b in range(w.B) for g in range(w.Hkv)]))
    check_kres(kres_d, kres_o, w.n_full * w.T)
    delta = w.deltas[0] if name != "gqa4_32k_sink_needles" else 5.0
    log(f"[gpu] residual {name}: sparse delta={delta}")
    out, lse, keep = gpu_sparse_res(w, qd, Kd, Vd, kres_d, bits, delta, pass_tail=False)
    keep_ref = np.zeros_like(keep)

    def mask(bh):
        b, h = bh
        g = h // w.G
        sb = oracle.scan_head_bits(q[b, h], kres_o[0][b, g], kres_o[1][b, g], w.n_full, w.T, bits)
        k, _, _ = oracle.select_head(sb, w.n_full, w.n_blocks, delta)
        return bh, k

    with ThreadPoolExecutor(16) as ex:
        for (b, h), k in ex.map(mask, [(b, h) for b in range(w.B) for h in range(w.Hq)]):
            keep_ref[b, h] = k
    np.testing.assert_array_equal(keep, keep_ref)

    def attend(bh):
        b, h = bh
        g = h // w.G
        return bh, oracle.attend_head_res(q[b, h], kres_o[0][b, g], kres_o[1][b, g],
                                          kres_o[2][b, g], kres_o[3][b, g], None, V[b, g],
                                          w.L, w.T, bits, keep_ref[b, h])

    log(f"[gpu] residual {name}: oracle attention, every head")
    with ThreadPoolExecutor(16) as ex:
        refs = dict(ex.map(attend, [(b, h) for b in range(w.B) for h in range(w.Hq)]))
    for (b, h), (ref_o, ref_l) in refs.items():
        assert_close(out[b, h], ref_o, TOL, f"out b={b} h={h}")
        assert_close(lse[b, h], ref_l, TOL, f"lse b={b} h={h}")
    log(f"[gpu] residual {name} bits={bits}: union keep "
        f"{keep.reshape(w.B, w.Hkv, w.G, -1).max(axis=2).mean():.4f}")
    del qd, Kd, Vd, kres_d
    torch.cuda.empty_cache()
