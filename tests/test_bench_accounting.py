"""Host logic of the benchmark: the algorithmic byte counts behind its GB/s and roofline figures,
and the lookup of the counter-measured traffic.  No GPU is used.

Bytes of one sparse step: the packed 4-bit keys (T*d/2 bytes) and bf16 scales (2*d bytes) of every
full block, for every (sequence, kv head); the 16-bit keys and values (2*d*e bytes per token) of
every block that at least one query head of the group keeps, a partial tail block counted at its
real length; and the query rows.
"""
import json

import numpy as np

import bench
from long_context_decoding_amd import workloads as W


def test_sparse_bytes_on_a_hand_built_mask():
    T, d = 64, 128
    w = W.small("t", B=1, Hq=4, Hkv=2, L=3 * T + 17, T=T, dtype="bf16", seed=1)
    assert (w.G, w.n_full, w.n_blocks) == (2, 3, 4)
    keep = np.zeros((1, 4, 4), np.uint8)
    keep[0, 0, [0, 2]] = 1          # group 0: head 0 keeps blocks 0 and 2
    keep[0, 1, 2] = 1               # head 1 keeps block 2 again (counted once for the group)
    keep[0, 3, [1, 3]] = 1          # group 1: head 3 keeps block 1 and the 17-token tail
    b = bench.bytes_sparse(w, keep)
    assert b["scan"] == 1 * 2 * 3 * (T * d // 2 + 2 * d)
    assert b["exact"] == (2 * T + (T + 17)) * 2 * d * 2
    assert b["q"] == 4 * d * 2
    assert b["total"] == b["scan"] + b["exact"] + b["q"]
    assert b["union_keep"] == 4 / 8 and b["head_keep"] == 5 / 16


def test_headline_bytes_of_the_256k_step():
    # 8 kv heads x 2048 full blocks of 128 tokens scanned (8,448 bytes each), 96 union-kept
    # blocks of bf16 keys and values (64 KiB each), 32 query rows: 144,711,680 bytes
    w = W.WORKLOADS["gqa4_256k_sink_needles"]
    keep = np.zeros((w.B, w.Hq, w.n_blocks), np.uint8)
    rng = np.random.default_rng(0)
    for g in range(w.Hkv):
        blocks = rng.choice(w.n_blocks, 12, replace=False)
        for i, j in enumerate(blocks):
            keep[0, g * w.G + i % w.G, j] = 1
    b = bench.bytes_sparse(w, keep)
    assert b["scan"] == 138_412_032 and b["exact"] == 96 * 65_536 and b["q"] == 8_192
    assert b["total"] == 144_711_680


def test_dense_and_residual_bytes():
    T, d = 128, 128
    w = W.small("t", B=2, Hq=8, Hkv=2, L=5 * T, T=T, dtype="bf16", seed=2)
    assert bench.bytes_dense(w) == 2 * 2 * 2 * 5 * T * d * 2 + 2 * 8 * d * 2
    keep = np.zeros((2, 8, 5), np.uint8)
    keep[0, 1, 0] = keep[0, 2, 0] = 1   # sequence 0, group 0 (heads 0-3): block 0 once
    keep[1, 7, 4] = 1                   # sequence 1, group 1: block 4
    for bits in (2, 4):
        r = bench.bytes_residual(w, keep, bits)
        code = T * d * bits // 8
        # bf16 thumbnail scales (2 d bytes per block), fp32 residual scales (4 d)
        assert r["scan"] == 2 * 2 * 5 * (code + 2 * d)
        assert r["exact"] == 2 * (code + T * d + 2 * d + 4 * d + 2 * T * d)
        assert r["total"] == r["scan"] + r["exact"] + 2 * 8 * d * 2


def test_traffic_lookup_is_per_workload_and_tied_to_the_kernel_source(tmp_path, monkeypatch):
    rec = {"kernel_src_sha256_16": bench.kernel_hash(), "workload": "w256",
           "hbm_bytes_per_launch": 123,
           "other_workloads": {"w128": {"hbm_bytes_per_launch": 456}}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", f)
    assert bench.traffic_entry("w256") == 123
    assert bench.traffic_entry("w128") == 456
    assert bench.traffic_entry("w32") is None          # no counters for that workload
    rec["kernel_src_sha256_16"] = "0" * 16               # counters taken on another kernel source
    f.write_text(json.dumps(rec))
    assert bench.traffic_entry("w256") is None


def test_committed_traffic_record_is_within_the_counter_check():
    # (the bench itself reports no traffic once the kernel source differs from the record's)
    rec = json.loads(bench.TRAFFIC_FILE.read_text())
    assert len(rec["kernel_src_sha256_16"]) == 16
    assert rec["workload"] == bench.PRIMARY
    hb, alg = rec["hbm_bytes_per_launch"], rec["algorithmic_bytes_per_launch"]
    assert alg <= hb <= 1.1 * alg   # the counter check: within 10% of the algorithmic bytes
    for other in rec.get("other_workloads", {}).values():
        assert other["algorithmic_bytes_per_launch"] <= other["hbm_bytes_per_launch"] \
            <= 1.1 * other["algorithmic_bytes_per_launch"]
