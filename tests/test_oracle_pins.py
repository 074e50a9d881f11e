"""Pins for the CPU oracle: it is checked against things other than itself.

Each test fixes one step of the oracle to a closed form, an invariant, a
library routine on a special case, brute force on a tiny input, or a worked
example the pages give, so that a plausible slip (a dropped term, a wrong sign
or index, a transposed operand) fails at least one of them.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import bsa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- decoding

def test_e4m3_decode_exhaustive_against_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.decode_e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    m = ~np.isnan(ref)
    assert np.array_equal(ours[m], ref[m])
    assert np.nanmax(ours) == 448.0 and np.nanmin(ours) == -448.0
    assert np.isnan(ours).sum() == 2  # +-NaN only: the fn variant has no infinities


def test_bf16_decode_against_torch():
    rng = np.random.default_rng(1)
    x = torch.from_numpy(rng.standard_normal(4096).astype(np.float32) * 100).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.decode_bf16(bits), x.to(torch.float64).numpy())


def test_dequantize_uses_head_and_block_scale():
    S, H, D, B = 10, 2, 3, 4
    codes = np.full((S, H, D), 0x38, dtype=np.uint8)  # 0x38 = 1.0 in E4M3
    scales = np.array([[1.0, 2.0, 3.0], [10.0, 20.0, 30.0]])
    x = O.dequantize(codes, scales, B)
    assert x[0, 0, 0] == 1.0 and x[4, 0, 1] == 2.0 and x[9, 0, 2] == 3.0
    assert x[9, 1, 0] == 30.0 and x[3, 1, 0] == 10.0


# ---------------------------------------------------------------- pooling

def test_pool_identical_rows_closed_form():
    rng = np.random.default_rng(2)
    S, H, D, B = 12, 2, 5, 4
    rows = rng.standard_normal((S // B, H, D))
    K = np.repeat(rows, B, axis=0)
    kbar, r = O.pool_keys(K, B)
    for g in range(H):
        assert np.allclose(kbar[g], rows[:, g, :], rtol=0, atol=1e-15)
        assert np.all(r[g] < 1e-12)


def test_pool_radius_plus_minus_closed_form():
    rng = np.random.default_rng(3)
    D, B = 6, 4
    c = rng.standard_normal(D)
    a = rng.standard_normal(D)
    K = np.stack([c + a, c - a, c + a, c - a])[:, None, :]
    kbar, r = O.pool_keys(K, B)
    assert np.allclose(kbar[0, 0], c, atol=1e-14)
    assert abs(r[0, 0] - np.linalg.norm(a)) < 1e-12


def test_pool_radius_is_max_not_mean():
    # three keys at the centroid, one far away: the radius is the far key's distance
    D, B = 4, 4
    K = np.zeros((4, 1, D))
    K[3, 0, 0] = 4.0
    kbar, r = O.pool_keys(K, B)
    assert np.allclose(kbar[0, 0], [1.0, 0, 0, 0])
    assert abs(r[0, 0] - 3.0) < 1e-12


def test_pool_queries_group_mean_is_mean_of_head_means():
    rng = np.random.default_rng(4)
    S, Hq, Hkv, D, B = 16, 4, 2, 3, 8
    Q = rng.standard_normal((S, Hq, D))
    per_head, qn_h = O.pool_queries(Q, B, Hkv, "qhead")
    grp, qn_g = O.pool_queries(Q, B, Hkv, "group")
    assert np.allclose(grp[0], per_head[0:2].mean(axis=0), atol=1e-15)
    assert np.allclose(grp[1], per_head[2:4].mean(axis=0), atol=1e-15)
    assert np.allclose(qn_h, np.linalg.norm(per_head, axis=-1))
    # block means by hand for one entry
    assert np.allclose(per_head[3, 1], Q[8:16, 3, :].sum(axis=0) / 8)


def test_pool_ragged_last_block_averages_rows_it_has():
    rng = np.random.default_rng(5)
    S, B, D = 10, 4, 3
    K = rng.standard_normal((S, 1, D))
    kbar, r = O.pool_keys(K, B)
    assert kbar.shape[1] == 3
    assert np.allclose(kbar[0, 2], K[8:10, 0].mean(axis=0))
    Q = rng.standard_normal((S, 1, D))
    qbar, _ = O.pool_queries(Q, B, 1, "qhead")
    assert np.allclose(qbar[0, 2], Q[8:10, 0].mean(axis=0))


# ---------------------------------------------------------------- scores and bound

def test_scores_bilinear_identity_against_dense_logits():
    """qbar_i . kbar_j equals the mean of the dense logit block Q_i K_j^T."""
    rng = np.random.default_rng(6)
    S, Hq, Hkv, D, B = 40, 4, 2, 8, 8
    Q = rng.standard_normal((S, Hq, D))
    K = rng.standard_normal((S, Hkv, D))
    for gran in ("qhead", "group"):
        qbar, _ = O.pool_queries(Q, B, Hkv, gran)
        kbar, _ = O.pool_keys(K, B)
        s = O.block_scores(qbar, kbar, Hq, Hkv, gran)
        nb = S // B
        for u in range(s.shape[0]):
            heads = [u] if gran == "qhead" else [2 * u, 2 * u + 1]
            g = u // 2 if gran == "qhead" else u
            for i in range(nb):
                for j in range(nb):
                    if j > i:
                        assert np.isnan(s[u, i, j])
                        continue
                    dense = np.mean([Q[i * B:(i + 1) * B, h] @ K[j * B:(j + 1) * B, g].T for h in heads])
                    assert abs(s[u, i, j] - dense) < 1e-12


def test_rescue_bound_cauchy_schwarz_invariant():
    # GQA shape (4 query heads per kv head): each unit's bound must use its own
    # kv head's keys and radius
    rng = np.random.default_rng(7)
    S, Hq, Hkv, D, B = 64, 8, 2, 8, 8
    G = Hq // Hkv
    Q = rng.standard_normal((S, Hq, D))
    K = rng.standard_normal((S, Hkv, D)) * rng.uniform(0.1, 3.0, size=(S, Hkv, 1))
    qbar, qn = O.pool_queries(Q, B, Hkv, "qhead")
    kbar, r = O.pool_keys(K, B)
    s = O.block_scores(qbar, kbar, Hq, Hkv, "qhead")
    b = O.rescue_bounds(s, qn, r, Hq, Hkv, "qhead")
    nb = S // B
    for u in range(Hq):
        g = u // G
        for i in range(nb):
            for j in range(i + 1):
                best_key = (K[j * B:(j + 1) * B, g] @ qbar[u, i]).max()
                assert b[u, i, j] >= best_key - 1e-12
                assert b[u, i, j] >= s[u, i, j]
    # equality when the block's keys are identical (radius 0)
    K2 = np.repeat(rng.standard_normal((nb, Hkv, D)), B, axis=0)
    kbar2, r2 = O.pool_keys(K2, B)
    s2 = O.block_scores(qbar, kbar2, Hq, Hkv, "qhead")
    b2 = O.rescue_bounds(s2, qn, r2, Hq, Hkv, "qhead")
    m = ~np.isnan(s2)
    assert np.allclose(b2[m], s2[m], atol=1e-12)


def test_rescue_bound_closed_form_and_tight_on_aligned_blocks():
    """Closed form, from the construction alone: every query row of head h is the
    same vector w_h, so qbar[h, i] = w_h for all i; block j of kv head g holds
    keys c_gj + a_gj*e and c_gj - a_gj*e (e a unit vector), so its centroid is
    c_gj and its radius a_gj.  Hence b[h, i, j] = w_h.c_gj + ||w_h||*a_gj exactly,
    with g = h // 4.  For the head whose w points along its kv head's e, the
    bound is attained by the key c + a*e: b equals the best key's dot product.
    The radii differ per kv head, so a bound built from another kv head's
    radius, or with 2*||qbar||*r, misses the closed form."""
    rng = np.random.default_rng(71)
    S, Hq, Hkv, D, B = 48, 8, 2, 6, 8
    G = Hq // Hkv
    nb = S // B
    e = rng.standard_normal((Hkv, D))
    e /= np.linalg.norm(e, axis=1, keepdims=True)
    w = rng.standard_normal((Hq, D))
    aligned = [g * G + 1 for g in range(Hkv)]  # head 1 of each group looks along e_g
    for g, h in enumerate(aligned):
        w[h] = 2.5 * e[g]
    c = rng.standard_normal((Hkv, nb, D))
    a = np.stack([rng.uniform(0.5, 1.0, nb), rng.uniform(2.0, 4.0, nb)])  # [Hkv, nb]
    Q = np.broadcast_to(w[None], (S, Hq, D)).copy()
    K = np.zeros((S, Hkv, D))
    for g in range(Hkv):
        for j in range(nb):
            for t in range(B):
                sign = 1.0 if t % 2 == 0 else -1.0
                K[j * B + t, g] = c[g, j] + sign * a[g, j] * e[g]
    qbar, qn = O.pool_queries(Q, B, Hkv, "qhead")
    kbar, r = O.pool_keys(K, B)
    s = O.block_scores(qbar, kbar, Hq, Hkv, "qhead")
    b = O.rescue_bounds(s, qn, r, Hq, Hkv, "qhead")
    for h in range(Hq):
        g = h // G
        for i in range(nb):
            for j in range(i + 1):
                expect = w[h] @ c[g, j] + np.linalg.norm(w[h]) * a[g, j]
                assert abs(b[h, i, j] - expect) < 1e-10, (h, i, j)
                best_key = (K[j * B:(j + 1) * B, g] @ w[h]).max()
                if h in aligned:
                    assert abs(b[h, i, j] - best_key) < 1e-10, (h, i, j)
                else:
                    assert b[h, i, j] > best_key + 1e-6, (h, i, j)


# ---------------------------------------------------------------- Quest backbone

def test_quest_bound_is_the_box_maximum_by_corner_enumeration():
    # the largest of a linear function over a box sits at one of its 2^D corners
    rng = np.random.default_rng(50)
    for _ in range(50):
        D = int(rng.integers(1, 7))
        a, b = rng.normal(size=D), rng.normal(size=D)
        kmin, kmax = np.minimum(a, b), np.maximum(a, b)
        q = rng.normal(size=(3, D))
        got = O.quest_row_bound(q, kmin[None], kmax[None])[:, 0]
        corners = np.array(list(itertools.product(*zip(kmin, kmax))))
        assert np.allclose(got, (q @ corners.T).max(axis=1), rtol=0, atol=1e-12)


def test_quest_bound_sign_picks_the_right_end():
    # q = -e0: the bound uses the minimum of coordinate 0 (-(-2) = 2), not its maximum
    kmin, kmax = np.array([[-2.0, 0.0]]), np.array([[3.0, 0.0]])
    assert O.quest_row_bound(np.array([[-1.0, 0.0]]), kmin, kmax)[0, 0] == 2.0
    assert O.quest_row_bound(np.array([[1.0, 0.0]]), kmin, kmax)[0, 0] == 3.0


def test_key_block_bounds_closed_forms():
    B, D = 4, 3
    c, a = np.array([1.0, -2.0, 0.5]), np.array([0.5, -1.0, 2.0])
    K = np.stack([c + a, c - a, c, c + 0.5 * a, c - a])[:, None, :]  # 5 rows: 1 full block + ragged
    kmin, kmax = O.key_block_bounds(K, B)
    assert np.array_equal(kmin[0, 0], c - np.abs(a)) and np.array_equal(kmax[0, 0], c + np.abs(a))
    assert np.array_equal(kmin[0, 1], c - a) and np.array_equal(kmax[0, 1], c - a)


def test_quest_scores_upper_bound_every_logit_and_are_tight_on_constant_blocks():
    rng = np.random.default_rng(51)
    S, Hq, Hkv, D, B = 7 * 16 - 5, 4, 2, 8, 16
    Q = rng.normal(size=(S, Hq, D))
    K = rng.normal(size=(S, Hkv, D))
    K[2 * B:3 * B, 1] = K[2 * B, 1]  # block 2 of kv head 1: every key the same
    kmin, kmax = O.key_block_bounds(K, B)
    for gran in ("qhead", "group"):
        s = O.quest_scores(Q, kmin, kmax, B, Hkv, gran)
        U = s.shape[0]
        G = Hq // Hkv
        for u in range(U):
            heads = [u] if gran == "qhead" else list(range(u * G, (u + 1) * G))
            g = O.kv_of_unit(u, Hq, Hkv, gran)
            for i in range(s.shape[1]):
                qi = Q[i * B:(i + 1) * B, heads].reshape(-1, D)
                for j in range(i + 1):
                    logits = qi @ K[j * B:(j + 1) * B, g].T
                    assert s[u, i, j] >= logits.max() - 1e-12
                    if g == 1 and j == 2:
                        assert s[u, i, j] == pytest.approx(logits.max(), abs=1e-12)
                assert np.all(np.isnan(s[u, i, i + 1:]))


def test_quest_scores_take_the_row_maximum_and_the_group_maximum():
    # one loud row in a quiet tile sets the tile's score (a mean would divide it by B)
    S, D, B = 8, 2, 4
    Q = np.zeros((S, 2, D))
    Q[5, 0] = [10.0, 0.0]
    Q[6, 1] = [0.0, -3.0]
    K = np.zeros((S, 1, D))
    K[:, 0] = [1.0, -1.0]
    kmin, kmax = O.key_block_bounds(K, B)
    s = O.quest_scores(Q, kmin, kmax, B, 1, "qhead")
    assert s[0, 1, 0] == 10.0 and s[1, 1, 0] == 3.0 and s[0, 0, 0] == 0.0
    sg = O.quest_scores(Q, kmin, kmax, B, 1, "group")
    fill = lambda a: np.where(np.isnan(a), -np.inf, a)  # noqa: E731
    assert sg[0, 1, 0] == 10.0 and np.array_equal(fill(s).max(axis=0), fill(sg[0]))


# ---------------------------------------------------------------- selection

def test_top_k_brute_force_with_ties():
    rng = np.random.default_rng(8)
    for trial in range(300):
        n = int(rng.integers(1, 9))
        vals = rng.integers(0, 4, size=n).astype(np.float64)  # many exact ties
        k = int(rng.integers(0, n + 2))
        got = sorted(O.top_k(vals, list(range(n)), k))
        kk = min(k, n)
        best = None
        for sub in itertools.combinations(range(n), kk):
            key = (-sum(vals[list(sub)]), sub)
            if best is None or key < best:
                best = key
        assert got == list(best[1]), (vals, k, got, best)


def test_top_k_lowest_index_tie_break():
    vals = np.array([1.0, 5.0, 3.0, 5.0, 3.0, 3.0])
    assert O.top_k(vals, [0, 1, 2, 3, 4, 5], 3) == [1, 3, 2]
    assert O.top_k(vals, [0, 2, 4, 5], 2) == [2, 4]


def test_gate_two_candidate_closed_form():
    rng = np.random.default_rng(9)
    for _ in range(100):
        a, b = rng.normal(0, 3, size=2)
        tau = float(rng.uniform(0.1, 2.0))
        s = np.array([0.0, a, b])  # block 0 forced as sink, candidates {1, 2}
        gap = O.gate_gap(s, [1, 2], tau)
        assert abs(gap - math.tanh(tau * abs(a - b) / 2)) < 1e-12


def test_gate_worked_example_from_page():
    fx = json.load(open(os.path.join(GOLDEN, "gate_worked_example.json")))
    p = O.SelectParams(top_k=fx["top_k"], force_sink=False, gate="top12_gap",
                       gate_threshold=fx["gate_threshold"], gate_factor=fx["gate_factor"],
                       score_temperature=fx["score_temperature"]).as_library_precision()
    # row i = 2: block 2 is the forced diagonal, candidates are blocks 0 and 1
    s = np.array(fx["scores"] + [0.0])
    gap = O.gate_gap(s, [0, 1], p.score_temperature)
    assert abs(gap - math.tanh(0.05)) < 1e-12
    kept, fired = O.select_row(2, s, None, p)
    assert fired is fx["expected_fires"]
    assert kept == sorted(fx["expected_kept_candidates"] + [2])
    # without the gate the plain top-1 drops the runner-up
    kept0, _ = O.select_row(2, s, None, O.SelectParams(top_k=1))
    assert kept0 == [0, 2]


def test_gate_does_not_fire_on_clear_winner_and_gated_is_superset():
    rng = np.random.default_rng(10)
    p = O.SelectParams(top_k=3, force_sink=True, gate="top12_gap", gate_threshold=0.05)
    p0 = O.SelectParams(top_k=3, force_sink=True)
    n_fired = 0
    for _ in range(200):
        i = int(rng.integers(1, 30))
        s = rng.normal(0, float(rng.uniform(0.01, 5)), size=i + 1)
        kept, fired = O.select_row(i, s, None, p)
        kept0, _ = O.select_row(i, s, None, p0)
        assert set(kept0) <= set(kept)
        _, cands = O.candidate_sets(i, True)
        assert len(kept) == len(set(kept))
        expect = min(len(cands), 6 if fired else 3) + (2 if i > 0 else 1)
        assert len(kept) == expect
        n_fired += fired
    assert 0 < n_fired < 200
    s = np.array([0.0, 10.0, 0.0, 0.0, 0.0])
    assert not O.select_row(4, s, None, p)[1]


# ---------------------------------------------------------------- sigma gate

def test_sigma_hand_worked_rows():
    # scores of five candidates, sorted 10, 7, 6, 2, 0
    vals = np.array([6.0, 0.0, 10.0, 2.0, 7.0])
    c = [0, 1, 2, 3, 4]
    assert O.sigma_cut_margin(vals, c, 2) == pytest.approx((7 - 6) / (10 - 6), abs=1e-15)
    assert O.sigma_cut_margin(vals, c, 3) == pytest.approx((6 - 2) / (10 - 2), abs=1e-15)
    assert O.sigma_cut_margin(vals, c, 4) == pytest.approx((2 - 0) / (10 - 0), abs=1e-15)
    # only the listed candidates count: dropping block 2 (the 10) changes the top
    assert O.sigma_cut_margin(vals, [0, 1, 3, 4], 2) == pytest.approx((6 - 2) / (7 - 2), abs=1e-15)


def test_sigma_arithmetic_progression_is_one_over_k():
    # scores n, n-1, ..., 1 in shuffled positions: s(0) = n, s(k-1) = n-k+1 and
    # s(k) = n-k, so sigma = 1/k; reading the cut one place off gives 1/(k+1)
    rng = np.random.default_rng(40)
    for n in (3, 5, 9, 17):
        vals = rng.permutation(np.arange(1, n + 1)).astype(np.float64)
        for k in range(1, n):
            assert O.sigma_cut_margin(vals, list(range(n)), k) == pytest.approx(1.0 / k, abs=1e-15)


def test_sigma_limits_and_no_cut():
    c = [0, 1, 2, 3]
    # tie between the last kept and the first dropped score: fully ambiguous
    assert O.sigma_cut_margin(np.array([3.0, 9.0, 3.0, 1.0]), c, 2) == 0.0
    # everything down to the cut tied: 0 by definition
    assert O.sigma_cut_margin(np.array([4.0, 4.0, 4.0, 1.0]), c, 2) == 0.0
    # kept set tied at the top and far above the rest: decisive
    assert O.sigma_cut_margin(np.array([9.0, 1.0, 9.0, 0.0]), c, 2) == 1.0
    # no cut when |C| <= k, and k = 0 has none either
    assert math.isnan(O.sigma_cut_margin(np.arange(4.0), c, 4))
    assert math.isnan(O.sigma_cut_margin(np.arange(4.0), c, 0))
    rng = np.random.default_rng(41)
    for _ in range(300):
        n = int(rng.integers(2, 40))
        vals = rng.normal(0, float(rng.uniform(0.01, 5)), size=n)
        k = int(rng.integers(1, n))
        sg = O.sigma_cut_margin(vals, list(range(n)), k)
        assert 0.0 <= sg <= 1.0
        # invariant under positive affine maps and under reordering of the candidates
        a, b = float(rng.uniform(0.1, 10)), float(rng.normal(0, 10))
        assert O.sigma_cut_margin(a * vals + b, list(range(n)), k) == pytest.approx(sg, abs=1e-9)
        perm = rng.permutation(n)
        assert O.sigma_cut_margin(vals[perm], list(range(n)), k) == pytest.approx(sg, abs=1e-15)


def test_sigma_k1_degeneracy_and_the_lay_example():
    # with k = 1 the kept score is the top one, so sigma is 1 unless s(0) = s(1)
    rng = np.random.default_rng(42)
    for _ in range(100):
        n = int(rng.integers(2, 30))
        vals = rng.normal(size=n)
        assert O.sigma_cut_margin(vals, list(range(n)), 1) == 1.0
    fx = json.load(open(os.path.join(GOLDEN, "gate_worked_example.json")))
    s = np.array(fx["scores"] + [0.0])  # tile 2: candidates are blocks 0 and 1
    assert O.sigma_cut_margin(s, [0, 1], 1) == 1.0
    # a layer of such tiles: the gap gate fires on each, the sigma gate never does
    nb = 6
    srow = np.zeros((1, nb, nb))
    for i in range(2, nb):
        srow[0, i, i - 2:i] = fx["scores"]
        srow[0, i, :i - 2] = -50.0
    for q in (0.05, 0.5, 0.99):
        p = O.SelectParams(top_k=1, gate="sigma_cut", gate_threshold=q)
        sbar, fired = O.tile_gate(srow, p)
        assert np.all(sbar[2:] == 1.0) and not fired.any()
    pg = O.SelectParams(top_k=1, gate="top12_gap", gate_threshold=0.05)
    assert all(O.select_row(i, srow[0, i], None, pg)[1] for i in range(2, nb))


def test_sigma_tile_decision_hand_cases():
    nan = math.nan
    # one unit; tile 3 has no cut.  T = 4 tiles, q = 0.5: at most 2 may sit at or below
    sbar, fired = O.sigma_gate_tiles(np.array([[0.5, 0.1, 0.3, nan, 0.2]]), 0.5)
    assert list(fired) == [False, True, False, False, True]
    # a tie across the boundary: three tiles share the lowest value, so with room for
    # two none fires, with room for three all three do
    sg = np.array([[0.2, 0.2, 0.2, 0.9]])
    assert not O.sigma_gate_tiles(sg, 0.5)[1].any()
    assert list(O.sigma_gate_tiles(sg, 0.75)[1]) == [True, True, True, False]
    assert list(O.sigma_gate_tiles(sg, 1.0)[1]) == [True, True, True, True]
    assert not O.sigma_gate_tiles(sg, 0.2)[1].any()
    # the tile signal is the mean over units of each tile's column (3 units, 2 tiles)
    sbar, _ = O.sigma_gate_tiles(np.array([[0.1, 0.9], [0.2, 0.6], [0.3, 0.3]]), 0.5)
    assert sbar == pytest.approx([0.2, 0.6], abs=1e-15)


def test_sigma_tile_decision_brute_force_by_sorting():
    rng = np.random.default_rng(43)
    for _ in range(100):
        U, nb = int(rng.integers(1, 5)), int(rng.integers(1, 40))
        sg = rng.uniform(0, 1, size=(U, nb))
        sg[:, rng.random(nb) < 0.2] = math.nan
        q = float(rng.uniform(0, 1))
        sbar, fired = O.sigma_gate_tiles(sg, q)
        elig = np.nonzero(~np.isnan(sbar))[0]
        order = elig[np.argsort(sbar[elig], kind="stable")]
        expect = set(order[: int(math.floor(q * len(elig)))].tolist())  # distinct values
        assert set(np.nonzero(fired)[0].tolist()) == expect


def test_sigma_gate_fires_on_planted_ambiguous_tiles():
    # k = 2, sink forced: tile i has candidates 1..i-1, a cut from i = 4 on (8 tiles).
    # Decisive tiles: two scores near 10 over a tail at 0 (sigma ~ 0.99); planted
    # tiles: the 2nd and 3rd score nearly tied (sigma ~ 0.002).
    nb, k, U = 12, 2, 2
    s = np.full((U, nb, nb), -1.0)
    planted = {5, 8, 11}
    for u in range(U):
        for i in range(nb):
            s[u, i, 1:i] = 0.0
            if i >= 4:
                s[u, i, 1] = 10.0
                if i in planted:
                    s[u, i, 2], s[u, i, 3] = 5.0, 4.99
                else:
                    s[u, i, 2] = 9.9
    p = O.SelectParams(top_k=k, force_sink=True, gate="sigma_cut", gate_threshold=3 / 8,
                       gate_factor=2)
    sbar, fired = O.tile_gate(s, p)
    assert set(np.nonzero(fired)[0].tolist()) == planted
    kept, flags = O.select(s, None, p)
    for u in range(U):
        for i in range(nb):
            _, cands = O.candidate_sets(i, True)
            forced = 2 if i > 0 else 1
            assert flags[u, i] == (i in planted)
            assert len(kept[u][i]) == min(len(cands), 2 * k if i in planted else k) + forced
    # with room for two, the three planted tiles (equal sigma: the zero tail does
    # not enter it) all stay off, since the percentile counts ties inclusively;
    # once tile 11 is strictly the most ambiguous it fires alone
    p2 = O.SelectParams(top_k=k, force_sink=True, gate="sigma_cut", gate_threshold=2 / 8)
    assert not O.tile_gate(s, p2)[1].any()
    s[:, 11, 3] = 4.999
    assert set(np.nonzero(O.tile_gate(s, p2)[1])[0].tolist()) == {11}


def test_sigma_gate_layer_superset_and_budget():
    rng = np.random.default_rng(44)
    U, nb, k = 3, 20, 3
    s = rng.normal(0, 2, size=(U, nb, nb))
    p = O.SelectParams(top_k=k, force_sink=True, gate="sigma_cut", gate_threshold=0.3,
                       gate_factor=2).as_library_precision()
    p0 = O.SelectParams(top_k=k, force_sink=True)
    kept, flags = O.select(s, None, p)
    kept0, _ = O.select(s, None, p0)
    T = sum(1 for i in range(nb) if len(O.candidate_sets(i, True)[1]) > k)
    fired_tiles = set(np.nonzero(flags[0])[0].tolist())
    assert len(fired_tiles) == int(math.floor(p.gate_threshold * T))
    for u in range(U):
        assert set(np.nonzero(flags[u])[0].tolist()) == fired_tiles  # one decision per tile
        for i in range(nb):
            assert set(kept0[u][i]) <= set(kept[u][i])


def test_mass_prefix_invariants():
    rng = np.random.default_rng(11)
    mu = float(np.float32(0.9))
    for _ in range(200):
        n = int(rng.integers(1, 40))
        s = rng.normal(0, float(rng.uniform(0.1, 6)), size=n + 1)
        order, cum = O.mass_cumulative(s, list(range(n)), 1.0)
        m = O.mass_prefix_length(cum, mu)
        p = np.exp(s[:n] - s[:n].max())
        p /= p.sum()
        kept = order[:m]
        assert p[kept].sum() >= mu - 1e-12
        assert p[kept[:-1]].sum() < mu
        # kept blocks are exactly the m largest
        assert set(kept) == set(np.argsort(-s[:n], kind="stable")[:m])


def test_mass_single_dominant_block():
    s = np.array([0.0, 0.0, 8.0, 0.0, 0.0])  # p(block 2) > 0.99
    p = O.SelectParams(mass_threshold=0.9)
    kept, _ = O.select_row(4, s, None, p)
    assert kept == [2, 4]


def test_rescue_count_and_ranking_by_bound():
    assert O.rescue_count(20, 0.05) == 1
    assert O.rescue_count(21, 0.05) == 2
    assert O.rescue_count(1, 0.05) == 1
    assert O.rescue_count(0, 0.05) == 0
    assert O.rescue_count(1022, 0.05) == 52
    s = np.zeros(41)
    b = np.zeros(41)
    b[[3, 17, 30]] = [5.0, 7.0, 5.0]
    p = O.SelectParams(rescue_fraction=0.05)  # ceil(0.05 * 40) = 2
    kept, _ = O.select_row(40, s, b, p)
    assert kept == [3, 17, 40]


def test_union_and_forced_identities():
    rng = np.random.default_rng(12)
    p = O.SelectParams(top_k=2, force_sink=True, mass_threshold=0.5, rescue_fraction=0.1)
    for _ in range(200):
        i = int(rng.integers(0, 50))
        s = rng.normal(0, 3, size=i + 1)
        b = s + rng.uniform(0, 5, size=i + 1)
        kept, _ = O.select_row(i, s, b, p)
        forced, cands = O.candidate_sets(i, True)
        tk = set(O.top_k(s, cands, 2))
        order, cum = O.mass_cumulative(s, cands, 1.0)
        base = set(order[:O.mass_prefix_length(cum, 0.5)])
        resc = set(O.top_k(b, cands, O.rescue_count(len(cands), 0.1)))
        assert set(kept) == set(forced) | tk | base | resc
        assert len(kept) <= len(forced) + len(tk) + len(base) + len(resc)
        assert kept == sorted(set(kept)) and kept[-1] == i and kept[0] == 0
        assert all(0 <= j <= i for j in kept)


def test_padded_width_fits_every_row_and_is_attained():
    # brute force over random layers: every kept set fits, and with top-k (gated or
    # not) some row fills the width exactly
    rng = np.random.default_rng(60)
    for p in (O.SelectParams(top_k=3, force_sink=True),
              O.SelectParams(top_k=3, force_sink=True, gate="top12_gap", gate_threshold=1.0),
              O.SelectParams(top_k=3, force_sink=False, gate="sigma_cut", gate_threshold=1.0),
              O.SelectParams(top_k=2, rescue_fraction=0.25),
              O.SelectParams(mass_threshold=0.9)):
        nb = 14
        s = rng.normal(0, 3, size=(2, nb, nb))
        b = s + rng.uniform(0, 2, size=s.shape)
        kept, _ = O.select(s, b, p.as_library_precision())
        w = O.padded_width(nb, p)
        lens = [len(r) for unit in kept for r in unit]
        assert max(lens) <= w
        if p.mass_threshold == 0.0 and p.rescue_fraction == 0.0 and p.gate != "top12_gap":
            assert max(lens) == w  # (branches of a union may overlap, so only top-k attains)
    # closed forms: top-k + sink + diagonal, gated to rho*k: rho*k + 2 once rows are long
    assert O.padded_width(100, O.SelectParams(top_k=32, force_sink=True, gate="sigma_cut")) == 66
    assert O.padded_width(100, O.SelectParams(top_k=32, force_sink=True)) == 34
    assert O.padded_width(10, O.SelectParams(top_k=32, force_sink=True)) == 10  # whole rows
    assert O.padded_width(7, O.SelectParams(mass_threshold=0.9)) == 7


def test_padded_rows_hold_the_kept_sets_then_sentinels():
    kept = [[[0], [0, 1], [1, 2]], [[0], [1], [0, 2]]]
    pad = O.to_padded(kept, 3)
    assert pad.tolist() == [[0, -1, -1], [0, 1, -1], [1, 2, -1], [0, -1, -1], [1, -1, -1],
                            [0, 2, -1]]
    rp, ci = O.to_csr(kept)
    for r in range(6):
        assert [x for x in pad[r] if x >= 0] == list(ci[rp[r]:rp[r + 1]])


def test_csr_round_trip():
    kept = [[[0], [0, 1], [0, 2]], [[0], [1], [1, 2]]]
    rp, ci = O.to_csr(kept)
    assert list(rp) == [0, 1, 3, 5, 6, 7, 9]
    assert O.from_csr(rp, ci, 2, 3) == kept


def test_acceptable_sets_cover_near_threshold():
    # two candidates whose gate gap sits right at the threshold: both decisions allowed
    theta = 0.05
    delta = math.atanh(theta) * 2  # tau*|a-b| so that tanh(.../2) == theta
    s = np.array([0.0, delta, 0.0])  # row 2: candidates {0, 1}, block 2 forced
    p = O.SelectParams(top_k=1, gate="top12_gap", gate_threshold=theta)
    sets, amb = O.acceptable_row_sets(2, s, None, p, 1e-5)
    assert amb and len(sets) == 2
    sets, amb = O.acceptable_row_sets(2, np.array([0.0, 3.0, 0.0]), None, p, 1e-5)
    assert not amb and len(sets) == 1


def _mass_row(cum_targets):
    """Scores whose softmax (temperature 1) over candidates 0..n-1 has the given
    cumulative sums (candidate j has the j-th largest probability); the row's
    last entry is its forced diagonal block."""
    cum = np.asarray(cum_targets, dtype=np.float64)
    p = np.diff(np.concatenate([[0.0], cum]))
    assert np.all(p > 0) and np.all(np.diff(p) <= 0) and abs(cum[-1] - 1.0) < 1e-15
    return np.concatenate([np.log(p), [0.0]])


@pytest.mark.parametrize("mu,cum,accepted", [
    # cumulative mass of the first 3 candidates just above mu, within delta:
    # stopping at 3 (float64 decision) or at 4 (a float32 sum a hair low)
    (0.9, [0.5, 0.8, 0.9 + 5e-6, 0.95, 0.98, 1.0], [3, 4]),
    # just below mu, within delta: 4 in float64, 3 if a float32 sum is a hair high
    (0.9, [0.5, 0.8, 0.9 - 5e-6, 0.95, 0.98, 1.0], [3, 4]),
    # outside the band on either side: only the float64 decision
    (0.9, [0.5, 0.8, 0.9 + 2e-5, 0.95, 0.98, 1.0], [3]),
    (0.9, [0.5, 0.8, 0.9 - 2e-5, 0.95, 0.98, 1.0], [4]),
    # every prefix short of the whole row stays below mu - delta: all of them
    (0.9, [0.3, 0.5, 0.65, 0.78, 0.9 - 2e-5, 1.0], [6]),
    # the whole row is reachable when the prefix before it sits inside the band
    (0.9, [0.3, 0.5, 0.65, 0.78, 0.9 - 5e-6, 1.0], [5, 6]),
    # two consecutive prefix masses inside the band (mu close to 1, so that the
    # tail after the band can hold candidates no larger than the one inside it):
    # three lengths reachable
    (0.99998, [0.6, 0.9, 0.99998 - 5e-6, 0.99998 + 4e-6, 0.999992, 1.0], [3, 4, 5]),
])
def test_acceptable_sets_mass_branch_hand_cases(mu, cum, accepted):
    """The base branch's accepted prefix lengths near mu with delta = 1e-5, worked
    out by hand: a prefix length m is reachable when its own mass is within delta
    of reaching mu (or it is the whole row) and the mass before it is within
    delta of not reaching mu."""
    delta = 1e-5
    n = len(cum)
    i = n  # candidates 0..n-1, forced diagonal n
    s = _mass_row(cum)
    p = O.SelectParams(mass_threshold=mu)
    sets, amb = O.acceptable_row_sets(i, s, None, p, delta)
    lengths = sorted(len(kept) - 1 for kept, _ in sets)
    assert lengths == accepted
    for kept, fired in sets:
        m = len(kept) - 1
        assert kept == list(range(m)) + [i] and not fired
    assert amb == (len(accepted) > 1)
    # the plain decision is one of them
    kept, _ = O.select_row(i, s, None, p)
    assert len(kept) - 1 in accepted



# ---------------------------------------------------------------- attention

def _rand_qkv(rng, S, Hq, Hkv, D):
    return (rng.standard_normal((S, Hq, D)), rng.standard_normal((S, Hkv, D)),
            rng.standard_normal((S, Hkv, D)))


def test_full_budget_equals_dense_causal_and_sdpa():
    """With every causal block kept, block-sparse attention is dense causal attention."""
    rng = np.random.default_rng(13)
    S, Hq, Hkv, D, B = 50, 4, 2, 8, 8  # ragged last block (50 = 6*8 + 2)
    Q, K, V = _rand_qkv(rng, S, Hq, Hkv, D)
    nb = -(-S // B)
    kept = [[list(range(i + 1)) for i in range(nb)] for _ in range(Hq)]
    scale = 1 / math.sqrt(D)
    Os, lse_s = O.attention(Q, K, V, kept, B, scale, "qhead")
    Od, lse_d = O.dense_causal_attention(Q, K, V, scale)
    assert np.allclose(Os, Od, atol=1e-12) and np.allclose(lse_s, lse_d, atol=1e-12)
    qt = torch.from_numpy(Q).permute(1, 0, 2)
    kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
    vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    assert np.allclose(Os, ref.permute(1, 0, 2).numpy(), atol=1e-12)
    # lse against torch.logsumexp of the masked logits
    lg = scale * torch.einsum("hsd,htd->hst", qt, kt)
    lg = lg.masked_fill(~torch.tril(torch.ones(S, S, dtype=torch.bool)), float("-inf"))
    assert np.allclose(lse_s, torch.logsumexp(lg, dim=-1).numpy(), atol=1e-12)


def test_sparse_mask_matches_sdpa_with_explicit_mask():
    rng = np.random.default_rng(14)
    S, Hq, Hkv, D, B = 48, 2, 1, 8, 8
    Q, K, V = _rand_qkv(rng, S, Hq, Hkv, D)
    nb = S // B
    kept = [[sorted({i} | set(rng.choice(i + 1, size=min(i + 1, 2), replace=False).tolist()))
             for i in range(nb)] for _ in range(Hq)]
    scale = 0.3
    Os, _ = O.attention(Q, K, V, kept, B, scale, "qhead")
    for h in range(Hq):
        allow = torch.zeros(S, S, dtype=torch.bool)
        for i in range(nb):
            for j in kept[h][i]:
                allow[i * B:(i + 1) * B, j * B:(j + 1) * B] = True
        allow &= torch.tril(torch.ones(S, S, dtype=torch.bool))
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(Q[:, h])[None], torch.from_numpy(K[:, 0])[None],
            torch.from_numpy(V[:, 0])[None], attn_mask=allow[None], scale=scale)[0]
        assert np.allclose(Os[:, h], ref.numpy(), atol=1e-12)


def test_attention_row_invariants():
    rng = np.random.default_rng(15)
    S, Hq, Hkv, D, B = 32, 2, 2, 4, 8
    Q, K, V = _rand_qkv(rng, S, Hq, Hkv, D)
    nb = S // B
    kept = [[[0, i] if i else [0] for i in range(nb)] for _ in range(Hq)]
    Os, _ = O.attention(Q, K, V, kept, B, 0.5, "qhead")
    assert np.array_equal(Os[0], V[0])  # row 0 sees only key 0
    ones = np.ones_like(V)
    O1, _ = O.attention(Q, K, ones, kept, B, 0.5, "qhead")
    assert np.allclose(O1, 1.0, atol=1e-14)  # softmax rows sum to 1
    const = np.broadcast_to(np.arange(D, dtype=np.float64), V.shape).copy()
    Oc, _ = O.attention(Q, K, const, kept, B, 0.5, "qhead")
    assert np.allclose(Oc, const, atol=1e-13)


def test_group_granularity_shares_rows_across_heads():
    rng = np.random.default_rng(16)
    S, Hq, Hkv, D, B = 32, 4, 2, 4, 8
    Q, K, V = _rand_qkv(rng, S, Hq, Hkv, D)
    nb = S // B
    kept_g = [[[0, i] if i else [0] for i in range(nb)], [[i] for i in range(nb)]]
    Og, _ = O.attention(Q, K, V, kept_g, B, 0.5, "group")
    kept_h = [kept_g[0], kept_g[0], kept_g[1], kept_g[1]]
    Oh, _ = O.attention(Q, K, V, kept_h, B, 0.5, "qhead")
    assert np.array_equal(Og, Oh)


# ---------------------------------------------------------------- needles

def test_planted_needle_must_be_selected():
    """Every key of the needle block beats every other candidate's centroid score, so by
    bilinearity the needle's centroid score is the row maximum and top-k keeps it."""
    rng = np.random.default_rng(17)
    S, D, B = 128, 16, 8
    nb = S // B
    Q = rng.standard_normal((S, 1, D)) * 0.1
    K = rng.standard_normal((S, 1, D)) * 0.1
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    Q[:, 0, :] += u  # every query leans on u
    needle = 5
    K[needle * B:(needle + 1) * B, 0, :] = 3 * u + rng.standard_normal((B, D)) * 0.01
    qbar, _ = O.pool_queries(Q, B, 1, "qhead")
    kbar, _ = O.pool_keys(K, B)
    s = O.block_scores(qbar, kbar, 1, 1, "qhead")
    p = O.SelectParams(top_k=1, force_sink=True)
    for i in range(needle + 2, nb):
        # the precondition that makes selection provable
        others = [s[0, i, j] for j in range(i) if j not in (0, needle)]
        assert (K[needle * B:(needle + 1) * B, 0] @ qbar[0, i]).min() > max(others)
        kept, _ = O.select_row(i, s[0, i], None, p)
        assert needle in kept
