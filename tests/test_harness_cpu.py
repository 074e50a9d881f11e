"""The GPU parity harness, exercised on the CPU: it must accept results built by
the oracle itself and reject a planted wrong decision.  This checks the checker
(its sigma-gate tile logic in particular); no GPU and no library are involved."""

import math

import numpy as np
import pytest
import torch

import bsa_check as K
from oracle import bsa_oracle as O
from random_layers import random_layers
from workloads import config_by_name, generate, scaled


def _oracle_run(cfg, inp):
    """A GpuRun-shaped record computed by the oracle (fp32 where the library
    exports fp32, selection re-run on the fp32 scores and bounds as the harness does)."""
    scales = [None if x is None else x.cpu().numpy() for x in (inp.q_scale, inp.k_scale,
                                                               inp.v_scale)]
    Q, Kk, V = O.decode_inputs(*(K._raw(t) for t in (inp.q, inp.k, inp.v)), cfg.dtype,
                               cfg.block_size, *scales)
    qbar, qn = O.pool_queries(Q, cfg.block_size, cfg.num_kv_heads, cfg.granularity)
    kbar, kr = O.pool_keys(Kk, cfg.block_size)
    kmin, kmax = O.key_block_bounds(Kk, cfg.block_size)
    if cfg.backbone == "quest":
        s = O.quest_scores(Q, kmin, kmax, cfg.block_size, cfg.num_kv_heads, cfg.granularity)
    else:
        s = O.block_scores(qbar, kbar, cfg.num_q_heads, cfg.num_kv_heads, cfg.granularity)
    s32 = np.nan_to_num(s).astype(np.float32)
    p = K.params_of(cfg)
    b32 = None
    if cfg.rescue_fraction > 0:
        b = O.rescue_bounds(s32.astype(np.float64), np.asarray(qn, np.float32).astype(np.float64),
                            np.asarray(kr, np.float32).astype(np.float64), cfg.num_q_heads,
                            cfg.num_kv_heads, cfg.granularity)
        b32 = np.nan_to_num(b).astype(np.float32)
    kept, fired = O.select(s32.astype(np.float64),
                           None if b32 is None else b32.astype(np.float64), p)
    rp, ci = O.to_csr(kept)
    out, lse = O.attention(Q, Kk, V, kept, cfg.block_size, 1 / math.sqrt(cfg.head_dim),
                           cfg.granularity)
    f32 = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float32))  # noqa: E731
    return K.GpuRun(torch.from_numpy(out).to(torch.bfloat16), f32(lse), rp, ci, f32(qbar),
                    f32(qn), f32(kbar), f32(kr), torch.from_numpy(s32),
                    None if b32 is None else torch.from_numpy(b32),
                    fired.reshape(-1).astype(np.uint8), f32(kmin), f32(kmax))


@pytest.fixture(scope="module")
def small_sigma():
    cfg = scaled(config_by_name("sigma64k"), 64 * 48 + 5, num_q_heads=2, num_kv_heads=1,
                 block_size=64, head_dim=64, top_k=6, name="sigma-cpu")
    inp = generate(cfg, "cpu")
    return cfg, inp, _oracle_run(cfg, inp)


def test_harness_accepts_the_oracles_own_results(small_sigma):
    cfg, inp, run = small_sigma
    rep = K.check_all(cfg, inp, run)
    assert rep.rows_checked == cfg.num_units * cfg.num_blocks
    T = sum(1 for i in range(cfg.num_blocks) if i - 1 > cfg.top_k)
    assert rep.gate_fired_tiles == int(math.floor(float(np.float32(0.3)) * T))
    assert rep.max_abs < 1e-2


def test_harness_rejects_a_wrong_tile_decision(small_sigma):
    cfg, inp, run = small_sigma
    nb, U = cfg.num_blocks, cfg.num_units
    g = run.gate.reshape(U, nb)
    tile = int(np.nonzero(g[0])[0][0])
    bad = g.copy()
    bad[:, tile] = 0  # the tile decision flipped in every unit, CSR unchanged
    run2 = K.GpuRun(**{**run.__dict__, "gate": bad.reshape(-1)})
    with pytest.raises(AssertionError, match="sigma gate"):
        K.check_all(cfg, inp, run2)
    bad1 = g.copy()
    bad1[0, tile] = 0  # one unit disagrees with the others
    run3 = K.GpuRun(**{**run.__dict__, "gate": bad1.reshape(-1)})
    with pytest.raises(AssertionError, match="disagree"):
        K.check_all(cfg, inp, run3)


def test_boundary_band_marks_only_near_ties():
    sbar = np.array([0.1, 0.2, math.nan, 0.2 + 5e-6, 0.5])
    # T = 4, q = 0.5: r = 2, the boundary is the 3rd smallest (0.2 + 5e-6)
    band = K.sigma_boundary_band(sbar, 0.5, 1e-5)
    assert list(band) == [False, True, False, True, False]
    assert not K.sigma_boundary_band(sbar, 1.0, 1e-5).any()
    # a boundary with room on both sides leaves nothing in doubt, the boundary tile included
    assert not K.sigma_boundary_band(np.array([0.1, 0.2, 0.3, 0.5]), 0.5, 1e-5).any()
    assert not K.sigma_boundary_band(np.array([0.1, 0.2, 0.3, 0.5]), 0.2, 1e-5).any()


@pytest.mark.parametrize("gran", ["qhead", "group"])
def test_harness_accepts_oracle_quest_results_and_rejects_a_wrong_bound(gran):
    cfg = scaled(config_by_name("quest64k"), 64 * 40 + 9, num_q_heads=4, num_kv_heads=2,
                 block_size=64, head_dim=64, top_k=5, granularity=gran, name=f"quest-cpu-{gran}")
    inp = generate(cfg, "cpu")
    run = _oracle_run(cfg, inp)
    rep = K.check_all(cfg, inp, run)
    assert rep.rows_checked == cfg.num_units * cfg.num_blocks and rep.max_abs < 1e-2
    bad = run.kmax.clone()
    bad[0, 3, 5] += 1e-3
    with pytest.raises(AssertionError, match="k_max block 3"):
        K.check_all(cfg, inp, K.GpuRun(**{**run.__dict__, "kmax": bad}))
    sc = run.scores.clone()
    sc[0, 7, 2] *= 1.01
    with pytest.raises(AssertionError, match="quest score"):
        K.check_all(cfg, inp, K.GpuRun(**{**run.__dict__, "scores": sc}))


@pytest.mark.parametrize("cfg", random_layers(48), ids=lambda c: c.name)
def test_harness_accepts_oracle_results_on_the_random_layers(cfg):
    """Every random layer the GPU parity test runs is decidable by the checker: the
    oracle's own results pass in full with no row or tile left in doubt."""
    inp = generate(cfg, "cpu")
    rep = K.check_all(cfg, inp, _oracle_run(cfg, inp))
    assert rep.rows_checked == cfg.num_units * cfg.num_blocks
    assert rep.ambiguous_rows == 0 and rep.ambiguous_tiles == 0
    assert rep.max_abs < 2e-2
