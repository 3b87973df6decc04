"""HIP-graph capture of the running-max and storage-form steps ("Faster Than Flash" App. G /
Table 9: the fused step replayed as a graph).  Each graph holds two steps on one workspace; it is
replayed four times, with eager decode work on the same workspace between the replays, and
every replay must equal the eager result bit for bit."""
import pytest
import torch

from conftest import log
from helpers import DEV, to_dev
from long_context_decoding_amd import ffd
from long_context_decoding_amd import workloads as W

pytestmark = pytest.mark.gpu


def _replays_equal(step, eager_between, out, lse, ref, what):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
        step()
    for i in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1]), f"{what}: replay {i} differs"
        eager_between()
        torch.cuda.synchronize()


def _case(T, L, seed):
    w = W.small(f"graphs_T{T}_L{L}", B=2, Hq=8, Hkv=2, L=L, T=T, seed=seed, plant="needles")
    q, K, V, _ = W.make_inputs(w)
    return w, to_dev(q), to_dev(K), to_dev(V)


@pytest.mark.parametrize("window", [3, 16])
def test_running_step_in_a_graph(window):
    w, qd, Kd, Vd = _case(64, 40 * 64 + 9, seed=31)
    log(f"graph running window={window}")
    Kq, sc = ffd.alloc_kq(Kd, w.T)
    ffd.quantize_k_append(Kd, 0, w.L, w.T, Kq, sc, seq_len=w.L)
    ws = ffd.alloc_workspace_window(ffd.dims_of(qd, Kd, w.L), w.T, window, DEV)
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=DEV)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=DEV)
    ref = ffd.decode_sparse_running(qd, Kd, Vd, Kq, sc, 2.0, w.T, window, w.L)
    torch.cuda.synchronize()

    def step():
        ffd.decode_sparse_running(qd, Kd, Vd, Kq, sc, 2.0, w.T, window, w.L, out=out, lse=lse,
                                  workspace=ws)

    def between():
        ffd.decode_sparse_running(qd, Kd, Vd, Kq, sc, 5.0, w.T, window, w.L, workspace=ws)

    _replays_equal(step, between, out, lse, ref, f"running window {window}")


@pytest.mark.parametrize("bits", [2, 4])
def test_residual_step_in_a_graph(bits):
    w, qd, Kd, Vd = _case(128, 12 * 128 + 40, seed=17 + bits)
    log(f"graph residual bits={bits}")
    kres = ffd.alloc_kres(Kd, w.T, bits)
    ffd.quantize_k_residual_append(Kd, 0, w.L, w.T, bits, kres, seq_len=w.L)
    ws = ffd.alloc_workspace(ffd.dims_of(qd, Kd, w.L), w.T, DEV)
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=DEV)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=DEV)
    ref = ffd.decode_sparse_residual(qd, Kd, Vd, kres, bits, 5.0, w.T, w.L)
    torch.cuda.synchronize()

    def step():
        ffd.decode_sparse_residual(qd, Kd, Vd, kres, bits, 5.0, w.T, w.L, out=out, lse=lse,
                                   workspace=ws)

    def between():
        ffd.decode_dense(qd, Kd, Vd, w.T, w.L, workspace=ws)

    _replays_equal(step, between, out, lse, ref, f"residual bits {bits}")
