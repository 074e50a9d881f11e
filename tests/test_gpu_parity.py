"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Small workloads are checked exhaustively (every pool entry, score, row and
output); the five full-size workloads are checked on seeded samples, in the
launch configuration the benchmark times.
"""

import math

import numpy as np
import pytest
import torch

from workloads import CONFIGS, EXTRA_CONFIGS, config_by_name, generate, scaled

pytestmark = pytest.mark.gpu


def _gpu_or_skip():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _small(name):
    c = config_by_name(name)
    if name == "tiny":
        return [c, scaled(c, 1000)]
    if name == "msa1m":
        return [scaled(c, 8192 + 1, num_q_heads=16, num_kv_heads=2)]
    if name == "dual128k":
        return [scaled(c, 8192 + 100, num_q_heads=8, num_kv_heads=1)]
    if name == "gated64k":
        return [scaled(c, 8192 + 5, num_q_heads=8, num_kv_heads=2)]
    return [scaled(c, 4096 + 77, num_q_heads=8, num_kv_heads=2)]


SMALL = [s for c in CONFIGS for s in _small(c.name)]
# the sigma gate beside the mass and rescue branches (one union), and on
# per-group E4M3 rows (one list per GQA group)
SMALL += [scaled(config_by_name("dual128k"), 4096 + 77, num_q_heads=8, num_kv_heads=2, top_k=8,
                 gate="sigma_cut", gate_threshold=0.3, name="sigma-with-mass-and-rescue"),
          scaled(config_by_name("msa1m"), 8192 + 1, num_q_heads=16, num_kv_heads=2, top_k=16,
                 gate="sigma_cut", gate_threshold=0.3, name="sigma-per-group-fp8")]
# every supported (head_dim, block_size) pair in both input formats, ragged tails
SHAPES = [scaled(config_by_name(base), 4096 + tail, num_q_heads=8, num_kv_heads=2,
                 head_dim=d, block_size=b, name=f"{base}-D{d}-B{b}")
          for base, tail in (("gqa32k", 37), ("msa1m", 70))
          for d, b in ((64, 64), (64, 128), (128, 64), (128, 128))]


@pytest.mark.parametrize("cfg", SMALL + SHAPES, ids=[c.name for c in SMALL + SHAPES])
def test_small_full_parity(cfg):
    _gpu_or_skip()
    import bsa_check as K
    print(f"[parity] {cfg.name} S={cfg.seq_len} Hq={cfg.num_q_heads} Hkv={cfg.num_kv_heads}",
          flush=True)
    inp = generate(cfg, "cpu").to("cuda")
    run = K.run_gpu(cfg, inp)
    rep = K.check_all(cfg, inp, run)
    print(f"  rows={rep.rows_checked} ambiguous={rep.ambiguous_rows} fired={rep.gate_fired} "
          f"kept={rep.kept_blocks} max_abs={rep.max_abs:.3g} mean_abs={rep.mean_abs:.3g} "
          f"lse={rep.lse_max:.3g}", flush=True)
    assert rep.ambiguous_rows <= max(1, rep.rows_checked // 100)


@pytest.mark.parametrize("cfg", CONFIGS, ids=[c.name for c in CONFIGS])
def test_full_size_sampled_parity(cfg):
    _gpu_or_skip()
    import bsa_check as K
    print(f"[parity-full] {cfg.name} S={cfg.seq_len}", flush=True)
    inp = generate(cfg, "cuda")
    run = K.run_gpu(cfg, inp)
    rep = K.check_all(cfg, inp, run, row_sample=48, unit_sample=24, score_sample=256)
    print(f"  rows={rep.rows_checked} ambiguous={rep.ambiguous_rows} fired={rep.gate_fired} "
          f"max_abs={rep.max_abs:.3g} mean_abs={rep.mean_abs:.3g} lse={rep.lse_max:.3g}",
          flush=True)
    del inp, run
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cfg", EXTRA_CONFIGS, ids=[c.name for c in EXTRA_CONFIGS])
def test_extra_workloads(cfg):
    """Workloads beyond the five (the 128K dual-branch selection on E4M3 inputs):
    a small scaled copy checked in full, then the full size on samples."""
    _gpu_or_skip()
    import bsa_check as K
    small = scaled(cfg, 8192 + 100, num_q_heads=8, num_kv_heads=1)
    for c, kw in ((small, {}), (cfg, dict(row_sample=48, unit_sample=24, score_sample=256))):
        print(f"[parity-extra] {c.name} S={c.seq_len} {c.dtype}", flush=True)
        inp = generate(c, "cuda")
        run = K.run_gpu(c, inp)
        rep = K.check_all(c, inp, run, **kw)
        print(f"  rows={rep.rows_checked} ambiguous={rep.ambiguous_rows} fired={rep.gate_fired} "
              f"max_abs={rep.max_abs:.3g} mean_abs={rep.mean_abs:.3g} lse={rep.lse_max:.3g}",
              flush=True)
        assert rep.ambiguous_rows <= max(1, rep.rows_checked // 100)
        del inp, run
        torch.cuda.empty_cache()


# the Quest backbone over every (head_dim, block_size) pair and input format, plus
# per-group units (the maximum over a group's heads), ragged tails
QUEST = [scaled(config_by_name("quest64k"), 2048 + tail, num_q_heads=8, num_kv_heads=2,
                head_dim=d, block_size=b, dtype=dt, top_k=8, granularity=gran,
                name=f"quest-{dt}-{gran}-D{d}-B{b}")
         for (dt, gran, tail) in (("bf16", "qhead", 37), ("fp8", "qhead", 70),
                                  ("bf16", "group", 5))
         for d, b in ((64, 64), (64, 128), (128, 64), (128, 128))]


@pytest.mark.parametrize("cfg", QUEST, ids=[c.name for c in QUEST])
def test_quest_backbone_parity(cfg):
    _gpu_or_skip()
    import bsa_check as K
    print(f"[parity-quest] {cfg.name} S={cfg.seq_len}", flush=True)
    inp = generate(cfg, "cpu").to("cuda")
    run = K.run_gpu(cfg, inp)
    rep = K.check_all(cfg, inp, run)
    print(f"  rows={rep.rows_checked} ambiguous={rep.ambiguous_rows} tiles_fired="
          f"{rep.gate_fired_tiles} max_abs={rep.max_abs:.3g} lse={rep.lse_max:.3g}", flush=True)
    assert rep.ambiguous_rows <= max(1, rep.rows_checked // 100)


# the padded list against CSR: the same selection, sentinels after each row's
# blocks, and attention bitwise equal to the CSR run (same blocks, same order)
PADDED = [scaled(config_by_name(n), 4096 + 77, num_q_heads=8, num_kv_heads=2, name=f"padded-{n}")
          for n in ("gqa32k", "gated64k", "sigma64k", "quest64k", "dual128k")]


@pytest.mark.parametrize("cfg", PADDED, ids=[c.name for c in PADDED])
def test_padded_list_matches_csr(cfg):
    _gpu_or_skip()
    import block_sparse_attention_36_amd as bsa
    import bsa_check as K
    from oracle import bsa_oracle as O
    print(f"[padded] {cfg.name} S={cfg.seq_len}", flush=True)
    inp = generate(cfg, "cpu").to("cuda")
    run = K.run_gpu(cfg, inp)
    problem = bsa.make_problem(inp.q, inp.k, cfg.block_size, K.granularity_code(cfg))
    params = K.lib_params(cfg)
    if cfg.backbone == "quest":
        pb = bsa.bsa_score_select_padded(problem, params, scores=run.scores, export=True)
    else:
        pool = bsa.bsa_pool(problem, inp.q, inp.k, inp.q_scale, inp.k_scale)
        pb = bsa.bsa_score_select_padded(problem, params, pool=pool, export=True)
    out, lse = bsa.bsa_attention_fwd_padded(problem, inp.q, inp.k, inp.v, pb.kv_idx,
                                            1.0 / math.sqrt(cfg.head_dim), inp.q_scale,
                                            inp.k_scale, inp.v_scale)
    torch.cuda.synchronize()
    U, nb = cfg.num_units, cfg.num_blocks
    kept = O.from_csr(run.row_ptr, run.col_idx, U, nb)
    width = O.padded_width(nb, K.params_of(cfg))
    assert pb.width == width
    assert np.array_equal(pb.kv_idx.cpu().numpy(), O.to_padded(kept, width))
    assert np.array_equal(pb.gate.cpu().numpy(), run.gate)
    assert torch.equal(out, run.out) and torch.equal(lse, run.lse)
    print(f"  width={width} rows={U * nb} fired={int(run.gate.sum())}", flush=True)


MID = [scaled(config_by_name("msa1m"), 2000 * 128 + 17, num_q_heads=4, num_kv_heads=2),
       scaled(config_by_name("dual128k"), 4000 * 128 - 3, num_q_heads=2, num_kv_heads=1),
       scaled(config_by_name("gated64k"), 3000 * 128, num_q_heads=2, num_kv_heads=1),
       # rows past 64 register slots: the register form runs once per range of query
       # blocks, and here the widest range holds the last query block alone
       scaled(config_by_name("gated64k"), 4096 * 128 + 5, num_q_heads=2, num_kv_heads=1),
       # the sigma gate in the 128-slot register form and, past 8192 blocks, in the
       # LDS form with the tile keys in global memory
       scaled(config_by_name("sigma64k"), 6000 * 128, num_q_heads=2, num_kv_heads=1),
       scaled(config_by_name("sigma64k"), 8300 * 64 + 11, num_q_heads=1, num_kv_heads=1,
              block_size=64, name="sigma64k@8301x64")]


@pytest.mark.parametrize("cfg", MID, ids=[c.name for c in MID])
def test_long_rows_sampled_parity(cfg):
    """Rows of 2000-4000 candidate blocks (the selection's wider register forms)."""
    _gpu_or_skip()
    import bsa_check as K
    print(f"[parity-mid] {cfg.name} S={cfg.seq_len} nb={cfg.num_blocks}", flush=True)
    inp = generate(cfg, "cuda")
    run = K.run_gpu(cfg, inp)
    rep = K.check_all(cfg, inp, run, row_sample=64, unit_sample=16, score_sample=256)
    print(f"  rows={rep.rows_checked} ambiguous={rep.ambiguous_rows} fired={rep.gate_fired} "
          f"tiles_fired={rep.gate_fired_tiles} max_abs={rep.max_abs:.3g}", flush=True)
    assert rep.ambiguous_rows <= max(1, rep.rows_checked // 100)


def test_full_budget_equals_dense_causal():
    """k >= every candidate set: the mask is the full causal triangle, so the output is
    dense causal attention (checked against the oracle's dense routine)."""
    _gpu_or_skip()
    import bsa_check as K
    from oracle import bsa_oracle as O
    base = config_by_name("gqa32k")
    cfg = scaled(base, 1536 + 40, num_q_heads=4, num_kv_heads=2, top_k=10_000)
    inp = generate(cfg, "cpu").to("cuda")
    run = K.run_gpu(cfg, inp)
    nb = cfg.num_blocks
    assert run.row_ptr[-1] == cfg.num_units * nb * (nb + 1) // 2
    host = K.HostInputs(cfg, inp)
    Q, Kk, V = (host.rows(w, list(range(nb))) for w in "qkv")
    Od, lsed = O.dense_causal_attention(Q, Kk, V, 1 / math.sqrt(cfg.head_dim))
    got = run.out.float().cpu().numpy()
    err = np.abs(got - Od)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3
    assert np.abs(run.lse.cpu().numpy() - lsed).max() <= 1e-3


def test_degenerate_csr_rows():
    """Entries outside [0, i] are ignored; a row without its diagonal keeps only the
    listed blocks; an empty row yields O = 0 and lse = -inf."""
    _gpu_or_skip()
    import block_sparse_attention_36_amd as bsa
    from oracle import bsa_oracle as O
    import bsa_check as K
    cfg = scaled(config_by_name("gqa32k"), 512, num_q_heads=1, num_kv_heads=1)
    inp = generate(cfg, "cpu").to("cuda")
    nb = cfg.num_blocks  # 4
    rows = [[], [0, 1, 7, -3], [1], [0, 2, 3, 99]]
    rp = np.zeros(nb + 1, dtype=np.int32)
    for i, r in enumerate(rows):
        rp[i + 1] = rp[i] + len(r)
    ci = np.array([x for r in rows for x in r], dtype=np.int32)
    problem = bsa.make_problem(inp.q, inp.k, cfg.block_size)
    out, lse = bsa.bsa_attention_fwd(problem, inp.q, inp.k, inp.v, torch.from_numpy(rp).cuda(),
                                     torch.from_numpy(ci).cuda(), 1 / math.sqrt(cfg.head_dim))
    torch.cuda.synchronize()
    B = cfg.block_size
    assert torch.all(out[:B].float() == 0) and torch.all(torch.isinf(lse[0, :B]))
    host = K.HostInputs(cfg, inp)
    for i, r in enumerate(rows):
        valid = [j for j in r if 0 <= j <= i]
        if not valid:
            continue
        q = host.rows("q", [i])[:, 0]
        keys = O.block_tokens(valid, B, cfg.seq_len)
        ref, lref = O.attend(q, i * B + np.arange(B), host.rows("k", valid)[:, 0],
                             host.rows("v", valid)[:, 0], keys, 1 / math.sqrt(cfg.head_dim))
        got = out[i * B:(i + 1) * B, 0].float().cpu().numpy()
        # a row without its diagonal has queries with no allowed key only if valid is empty
        assert np.abs(got - ref).max() <= 2e-2


def test_empty_sequence_is_a_no_op():
    _gpu_or_skip()
    import block_sparse_attention_36_amd as bsa
    q = torch.empty(0, 2, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.empty(0, 1, 128, dtype=torch.bfloat16, device="cuda")
    problem = bsa.make_problem(q, k, 128)
    lib = bsa.load_library()
    import ctypes
    assert lib.bsa_pool(ctypes.byref(problem), None, None, None, None, None, None, None, None,
                        None) == 0


def test_repeat_runs_are_bitwise_identical():
    _gpu_or_skip()
    import bsa_check as K
    cfg = scaled(config_by_name("dual128k"), 4096 + 3, num_q_heads=4, num_kv_heads=1)
    inp = generate(cfg, "cpu").to("cuda")
    a = K.run_gpu(cfg, inp)
    b = K.run_gpu(cfg, inp)
    assert np.array_equal(a.row_ptr, b.row_ptr) and np.array_equal(a.col_idx, b.col_idx)
    assert torch.equal(a.out, b.out) and torch.equal(a.lse, b.lse)
