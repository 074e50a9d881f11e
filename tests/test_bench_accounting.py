"""The figures bench.py reports rest on a few counting functions; each is checked
here against a brute-force count on small shapes (CPU only).

  attention_flops    4*D per valid (query, key) pair of every kept (row, block),
                     causal inside the diagonal block, ragged last block exact,
                     times the heads one selection row serves
  dense_causal_flops the same count for the full causal mask
  quest_flops        4*D per (query row, causal key block) of every query head
  traffic record     used only for the kernel source and workload it was taken on
"""

from __future__ import annotations

import itertools
import json
import os
from types import SimpleNamespace

import numpy as np

import bench


def _cfg(S, B, D, Hq, Hkv, granularity="qhead"):
    nb = -(-S // B)
    G = Hq // Hkv
    return SimpleNamespace(seq_len=S, block_size=B, head_dim=D, num_q_heads=Hq,
                           num_kv_heads=Hkv, num_blocks=nb, group_size=G,
                           granularity=granularity,
                           num_units=Hkv if granularity == "group" else Hq)


def _brute_pairs(S, B, i, j):
    # valid (query t, key s) pairs of query block i against key block j: s <= t
    return sum(1 for t in range(i * B, min((i + 1) * B, S))
               for s in range(j * B, min((j + 1) * B, S)) if s <= t)


def _random_csr(cfg, rng):
    nb = cfg.num_blocks
    rows = []
    for _u, i in itertools.product(range(cfg.num_units), range(nb)):
        others = [j for j in range(i) if rng.random() < 0.5]
        rows.append(sorted(others + [i]))
    rp = np.zeros(len(rows) + 1, dtype=np.int64)
    rp[1:] = np.cumsum([len(r) for r in rows])
    ci = np.concatenate([np.array(r, dtype=np.int64) for r in rows])
    return rows, rp, ci


def test_attention_flops_matches_pair_count():
    rng = np.random.default_rng(7)
    for S, B, gran in ((18, 4, "qhead"), (20, 4, "qhead"), (13, 4, "group"), (9, 8, "group")):
        cfg = _cfg(S, B, D=2, Hq=4, Hkv=2, granularity=gran)
        rows, rp, ci = _random_csr(cfg, rng)
        heads = cfg.group_size if gran == "group" else 1
        want = 0
        for r, kept in enumerate(rows):
            i = r % cfg.num_blocks
            want += sum(_brute_pairs(S, B, i, j) for j in kept)
        want *= 4 * cfg.head_dim * heads
        assert bench.attention_flops(rp, ci, cfg) == float(want)


def test_dense_causal_flops_is_the_full_mask():
    for S, B in ((18, 4), (16, 4), (7, 8)):
        cfg = _cfg(S, B, D=2, Hq=3, Hkv=1)
        nb = cfg.num_blocks
        rows = [list(range(i + 1)) for _u in range(cfg.num_units) for i in range(nb)]
        rp = np.zeros(len(rows) + 1, dtype=np.int64)
        rp[1:] = np.cumsum([len(r) for r in rows])
        ci = np.concatenate([np.array(r, dtype=np.int64) for r in rows])
        assert bench.dense_causal_flops(cfg) == bench.attention_flops(rp, ci, cfg)
        # and the closed form: every head, every (t, s <= t) pair
        assert bench.dense_causal_flops(cfg) == 4.0 * 2 * 3 * sum(t + 1 for t in range(S))


def test_quest_flops_counts_rows_times_causal_blocks():
    for S, B in ((18, 4), (16, 8)):
        cfg = _cfg(S, B, D=4, Hq=2, Hkv=1)
        want = 0
        for i in range(cfg.num_blocks):
            rows_in_tile = min(B, S - i * B)
            want += rows_in_tile * (i + 1)
        want *= cfg.num_q_heads * 4 * cfg.head_dim
        assert bench.quest_flops(cfg) == float(want)


def test_pool_select_bytes_counts_each_csr_entry_once():
    cfg = SimpleNamespace(seq_len=1024, num_q_heads=4, num_kv_heads=2, head_dim=64,
                          num_blocks=16, num_units=4, dtype="bf16", backbone="mean_pool")
    assert bench.pool_select_bytes(cfg, 101) - bench.pool_select_bytes(cfg, 100) == 4.0
    # Q and K are read once: doubling S adds exactly their bytes (plus nothing else
    # that scales with S at a fixed block count)
    c2 = SimpleNamespace(**{**cfg.__dict__, "seq_len": 2048})
    assert (bench.pool_select_bytes(c2, 0) - bench.pool_select_bytes(cfg, 0)
            == 1024 * (4 + 2) * 64 * 2)


def test_traffic_record_is_used_only_where_it_was_taken():
    path = os.path.join(bench.ROOT, "profiles", "attention_dual128k_counters.json")
    rec = json.load(open(path))
    h, w = rec["kernel_source_hash"], rec["workload"]
    assert bench.traffic_from_profile(h, w) == rec["hbm_bytes_per_launch"]
    assert bench.traffic_from_profile(h, "msa1m") is None
    assert bench.traffic_from_profile("0" * 16, w) is None


def test_realized_stats_count_by_hand():
    """Needle recall, planted-pair recall, gate rates and outlier recall on a
    hand-built CSR (2 query heads over 1 kv head, 6 blocks)."""
    cfg = _cfg(6 * 8, 8, 4, 2, 1)
    cfg.force_sink = False
    cfg.gate = "top12_gap"
    nb = 6
    rows = {  # (u, i) -> kept
        (0, 0): [0], (0, 1): [0, 1], (0, 2): [1, 2], (0, 3): [0, 1, 3], (0, 4): [2, 4],
        (0, 5): [1, 2, 3, 5], (1, 0): [0], (1, 1): [1], (1, 2): [1, 2], (1, 3): [3],
        (1, 4): [1, 4], (1, 5): [5]}
    counts = [len(rows[(u, i)]) for u in range(2) for i in range(nb)]
    rp = np.concatenate([[0], np.cumsum(counts)])
    ci = np.array([j for u in range(2) for i in range(nb) for j in rows[(u, i)]])
    # needle block 1: eligible rows i > 1, both heads -> 8 pairs; kept in
    # (0,2) (0,3) (0,5) (1,2) (1,4) -> 5
    st = bench.realized_stats(cfg, {"needle_blocks": [1]}, rp, ci, None)
    assert st["needle_pairs"] == 8 and st["needle_recall"] == round(5 / 8, 4)
    # pairs (needle 1, decoy 2) planted in query blocks 3 and 5; gate fired on
    # (0,3), (0,4), (1,5)
    gate = np.zeros(2 * nb, dtype=np.uint8)
    gate[[3, 4, nb + 5]] = 1
    meta = {"pairs": {0: [(1, 2)]}, "planted_query_blocks": {0: {3: 0, 5: 0}}}
    st = bench.realized_stats(cfg, meta, rp, ci, gate)
    # planted rows: (0,3) needle yes decoy no; (0,5) both; (1,3) neither; (1,5) neither
    assert st["planted_rows"] == 4
    assert st["planted_needle_recall"] == 0.5 and st["planted_pair_recall"] == 0.25
    assert st["gate_fire_rate_planted"] == 0.5  # (0,3) and (1,5)
    assert st["gate_fire_rate_background"] == round(1 / 8, 4)  # (0,4)
    # a wide block 2 whose outlier aims at query block 4 of head 0 (kept there),
    # and block 3 aimed at block 5 of head 1 (not kept)
    st = bench.realized_stats(cfg, {"wide_blocks": {0: {2: (17, 4, 0), 3: (30, 5, 1)}}},
                              rp, ci, None)
    assert st["outlier_rows"] == 2 and st["outlier_block_recall"] == 0.5


def test_cpu_full_runs_the_whole_tiny_workload():
    import torch
    from workloads import config_by_name, generate, scaled
    cfg = scaled(config_by_name("tiny"), 300)
    inp = generate(cfg, "cpu")
    res = bench.cpu_full(cfg, inp)
    assert res["kind"] == "oracle" and res["value"] > 0 and res["cores"] >= 1
    assert res["cpu_model"] and res["affinity_cores"] >= 1


def test_bench_refuses_more_than_one_gpu():
    """The bench measures one GPU's share; asked for several it exits with a
    message before touching a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr and r.stdout == ""
