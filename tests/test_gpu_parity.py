"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Small workloads are checked exhaustively (every pool entry, score, row and
output); the five full-size workloads are checked on seeded samples, in the
launch configuration the benchmark times.
"""

import math

import numpy as np
import pytest
import torch

from random_layers import random_layers
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
    # (the 1M layer's rows hold 8192 candidates each: fewer of them keep the test short)
    rows = 192 if cfg.seq_len > 500000 else 512
    rep = K.check_all(cfg, inp, run, row_sample=rows, unit_sample=128, score_sample=2048)
    print(f"  rows={rep.rows_checked} ambiguous={rep.ambiguous_rows} fired={rep.gate_fired} "
          f"max_abs={rep.max_abs:.3g} mean_abs={rep.mean_abs:.3g} lse={rep.lse_max:.3g}",
          flush=True)
    assert rep.ambiguous_rows <= max(1, rep.rows_checked // 100)
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


# the padded list: checked against the oracle on its own (selection, exported
# scores and outputs), and against the CSR run of the same inputs (the same
# selection, attention bitwise equal: same blocks, same order)
PADDED = [scaled(config_by_name(n), 4096 + 77, num_q_heads=8, num_kv_heads=2, name=f"padded-{n}")
          for n in ("gqa32k", "gated64k", "sigma64k", "quest64k", "dual128k")]


@pytest.mark.parametrize("cfg", PADDED, ids=[c.name for c in PADDED])
def test_padded_list_parity(cfg):
    _gpu_or_skip()
    import bsa_check as K
    from oracle import bsa_oracle as O
    print(f"[padded] {cfg.name} S={cfg.seq_len}", flush=True)
    inp = generate(cfg, "cpu").to("cuda")
    run = K.run_gpu(cfg, inp)
    prun = K.run_gpu_padded(cfg, inp, run)
    rep = K.check_all(cfg, inp, prun)
    print(f"  rows={rep.rows_checked} ambiguous={rep.ambiguous_rows} fired={rep.gate_fired} "
          f"max_abs={rep.max_abs:.3g} lse={rep.lse_max:.3g}", flush=True)
    assert rep.ambiguous_rows <= max(1, rep.rows_checked // 100)
    # the same bytes as the CSR run
    U, nb = cfg.num_units, cfg.num_blocks
    assert np.array_equal(prun.row_ptr, run.row_ptr) and np.array_equal(prun.col_idx, run.col_idx)
    assert np.array_equal(prun.gate, run.gate)
    assert torch.equal(prun.out, run.out) and torch.equal(prun.lse, run.lse)
    width = O.padded_width(nb, K.params_of(cfg))
    print(f"  width={width} rows={U * nb}", flush=True)


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
              block_size=64, name="sigma64k@8301x64"),
       # rows past 4096 blocks with the mass and rescue branches: the LDS form of
       # the select kernel, with under 64 KiB of LDS and with more (the raised limit)
       scaled(config_by_name("dual128k"), 4500 * 128 + 9, num_q_heads=1, num_kv_heads=1,
              name="dual128k@4501-lds"),
       scaled(config_by_name("dual128k"), 5600 * 128, num_q_heads=1, num_kv_heads=1,
              name="dual128k@5600-lds96k")]


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


def test_fp8_zero_blocks_with_zero_scales():
    """An all-zero E4M3 block has scale 0 (its amax is 0).  Zero query blocks and
    zero key blocks, the diagonal among them, give finite outputs equal to the
    oracle's (uniform softmax where every logit is 0)."""
    _gpu_or_skip()
    import bsa_check as K
    cfg = scaled(config_by_name("msa1m"), 2048 + 70, num_q_heads=4, num_kv_heads=2, top_k=4)
    inp = generate(cfg, "cpu")
    for blk in (0, 5, cfg.num_blocks - 1):
        t0, t1 = blk * cfg.block_size, min(cfg.seq_len, (blk + 1) * cfg.block_size)
        inp.q[t0:t1, 1] = 0
        inp.q_scale[1, blk] = 0.0
        inp.k[t0:t1, 0] = 0
        inp.k_scale[0, blk] = 0.0
    inp = inp.to("cuda")
    run = K.run_gpu(cfg, inp)
    assert torch.isfinite(run.out.float()).all() and not torch.isnan(run.lse).any()
    rep = K.check_all(cfg, inp, run)
    print(f"  zero blocks: max_abs={rep.max_abs:.3g} lse={rep.lse_max:.3g}", flush=True)
    # zero value blocks with scale 0 as well, through the prepared V tiles: the same
    # bytes as the codes path
    import block_sparse_attention_36_amd as bsa
    for blk in (2, cfg.num_blocks - 1):
        t0, t1 = blk * cfg.block_size, min(cfg.seq_len, (blk + 1) * cfg.block_size)
        inp.v[t0:t1, 1] = 0
        inp.v_scale[1, blk] = 0.0
    problem = bsa.make_problem(inp.q, inp.k, cfg.block_size, K.granularity_code(cfg))
    rp = torch.from_numpy(run.row_ptr.astype(np.int32)).to("cuda")
    ci = torch.from_numpy(run.col_idx.astype(np.int32)).to("cuda")
    scale = 1.0 / math.sqrt(cfg.head_dim)
    out0, lse0 = bsa.bsa_attention_fwd(problem, inp.q, inp.k, inp.v, rp, ci, scale,
                                       inp.q_scale, inp.k_scale, inp.v_scale)
    out1, lse1 = bsa.bsa_attention_fwd_prepared_v(problem, inp.q, inp.k,
                                                  bsa.bsa_prepare_v(problem, inp.v), rp, ci,
                                                  scale, inp.q_scale, inp.k_scale, inp.v_scale)
    torch.cuda.synchronize()
    assert torch.isfinite(out0.float()).all() and not torch.isnan(lse0).any()
    assert torch.equal(out0.view(torch.int16), out1.view(torch.int16))
    assert torch.equal(lse0, lse1)


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


# E4M3 shapes (every (head_dim, block_size) pair, ragged tails, both granularities)
# and the 1M workload at full size for the expanded-V attention
# the score kernel's own arithmetic: bf16 products of fp32 centroids split into two
# bf16 parts each, against float64 products of the same centroids
SCORE_ERR = [scaled(config_by_name("gqa32k"), 4096 + 77, num_q_heads=8, num_kv_heads=2,
                    name="scores-D128"),
             scaled(config_by_name("gqa32k"), 4096 + 77, num_q_heads=8, num_kv_heads=2,
                    head_dim=64, block_size=64, name="scores-D64"),
             scaled(config_by_name("msa1m"), 8192 + 1, num_q_heads=16, num_kv_heads=2,
                    name="scores-group-fp8")]


@pytest.mark.parametrize("cfg", SCORE_ERR, ids=[c.name for c in SCORE_ERR])
def test_score_kernel_error_bound(cfg):
    """Every exported score within 1e-5 * ||qbar|| * ||kbar|| of the float64 product of
    the centroids the library itself pooled (the split operands carry about 2^-17 of
    each product; the parity bound against the oracle is 1e-4)."""
    _gpu_or_skip()
    import block_sparse_attention_36_amd as bsa
    import bsa_check as K
    print(f"[scores] {cfg.name} S={cfg.seq_len}", flush=True)
    inp = generate(cfg, "cpu").to("cuda")
    problem = bsa.make_problem(inp.q, inp.k, cfg.block_size, K.granularity_code(cfg))
    pool = bsa.bsa_pool(problem, inp.q, inp.k, inp.q_scale, inp.k_scale)
    sel = bsa.bsa_score_select(problem, K.lib_params(cfg), pool, export=True)
    torch.cuda.synchronize()
    qc = pool.q_centroid.double().cpu()
    kc = pool.k_centroid.double().cpu()
    s = sel.scores.double().cpu()
    U, nb = qc.shape[0], qc.shape[1]
    G = 1 if cfg.granularity == "group" else cfg.num_q_heads // cfg.num_kv_heads
    tri = torch.tril(torch.ones(nb, nb, dtype=torch.bool))
    worst = 0.0
    for u in range(U):
        g = u if cfg.granularity == "group" else u // G
        exact = qc[u] @ kc[g].T
        norm = qc[u].norm(dim=1)[:, None] * kc[g].norm(dim=1)[None, :] + 1e-30
        err = ((s[u] - exact).abs() / norm)[tri]
        worst = max(worst, float(err.max()))
    print(f"  worst normwise score error {worst:.3g}", flush=True)
    assert worst <= 1e-5


EXPANDED_V = [c for c in SHAPES if c.dtype == "fp8"] + [
    scaled(config_by_name("dual128k_fp8"), 4096 + 77, num_q_heads=8, num_kv_heads=2),
    config_by_name("msa1m")]


@pytest.mark.parametrize("cfg", EXPANDED_V, ids=[c.name for c in EXPANDED_V])
def test_expanded_v_attention_equals_the_codes_path(cfg):
    """bsa_expand_e4m3 decodes every code exactly (against torch's E4M3 decoding),
    and attention on the expanded V equals attention on the codes bit for bit
    (outputs and log-sum-exp), so the oracle parity of the codes path carries over."""
    _gpu_or_skip()
    import block_sparse_attention_36_amd as bsa
    import bsa_check as K
    print(f"[expanded-v] {cfg.name} S={cfg.seq_len} Hq={cfg.num_q_heads} Hkv={cfg.num_kv_heads}",
          flush=True)
    inp = generate(cfg, "cpu" if cfg.seq_len < 100000 else "cuda").to("cuda")
    problem = bsa.make_problem(inp.q, inp.k, cfg.block_size, K.granularity_code(cfg))
    params = K.lib_params(cfg)
    pool = bsa.bsa_pool(problem, inp.q, inp.k, inp.q_scale, inp.k_scale)
    sel = bsa.bsa_score_select(problem, params, pool)
    v16 = bsa.bsa_expand_e4m3(problem, inp.v)
    ref16 = inp.v.view(torch.float8_e4m3fn).float().to(torch.bfloat16)
    assert torch.equal(v16.view(torch.int16), ref16.view(torch.int16))
    del ref16
    scale = 1.0 / math.sqrt(cfg.head_dim)
    out0, lse0 = bsa.bsa_attention_fwd(problem, inp.q, inp.k, inp.v, sel.row_ptr, sel.col_idx,
                                       scale, inp.q_scale, inp.k_scale, inp.v_scale)
    out1, lse1 = bsa.bsa_attention_fwd_expanded_v(problem, inp.q, inp.k, v16, sel.row_ptr,
                                                  sel.col_idx, scale, inp.q_scale, inp.k_scale,
                                                  inp.v_scale)
    torch.cuda.synchronize()
    assert torch.equal(out0.view(torch.int16), out1.view(torch.int16))
    assert torch.equal(lse0, lse1)


# the prepared (transposed) V tiles: bf16 and E4M3, one list per head and per GQA
# group, ragged tails, and the 1M-token layer the benchmark runs on them
PREPARED_V = [
    scaled(config_by_name("dual128k"), 4096 + 77, num_q_heads=8, num_kv_heads=2,
           name="prepared-bf16"),
    scaled(config_by_name("gqa32k"), 2 * 4096 + 5, num_q_heads=8, num_kv_heads=2,
           name="prepared-bf16-topk"),
    scaled(config_by_name("dual128k_fp8"), 4096 + 77, num_q_heads=8, num_kv_heads=2,
           name="prepared-fp8"),
    scaled(config_by_name("msa1m"), 8192 + 1, num_q_heads=16, num_kv_heads=2,
           name="prepared-fp8-group"),
    config_by_name("msa1m")]


@pytest.mark.parametrize("cfg", PREPARED_V, ids=[c.name for c in PREPARED_V])
def test_prepared_v_attention_equals_the_plain_path(cfg):
    """bsa_prepare_v writes every value of V (E4M3 codes decoded exactly) at its place
    in the transposed tiles, zero past the sequence, and attention on them equals
    bsa_attention_fwd on V as given bit for bit (outputs and log-sum-exp), so the
    oracle parity of the plain path carries over."""
    _gpu_or_skip()
    import block_sparse_attention_36_amd as bsa
    import bsa_check as K
    print(f"[prepared-v] {cfg.name} S={cfg.seq_len} Hq={cfg.num_q_heads} "
          f"Hkv={cfg.num_kv_heads} {cfg.dtype}", flush=True)
    inp = generate(cfg, "cpu" if cfg.seq_len < 100000 else "cuda").to("cuda")
    problem = bsa.make_problem(inp.q, inp.k, cfg.block_size, K.granularity_code(cfg))
    params = K.lib_params(cfg)
    pool = bsa.bsa_pool(problem, inp.q, inp.k, inp.q_scale, inp.k_scale)
    sel = bsa.bsa_score_select(problem, params, pool)
    vp = bsa.bsa_prepare_v(problem, inp.v)
    # the tiles against the layout, from V decoded by torch: [nb, Hkv, 128 dims, 128 keys]
    # with each 16-key group stored as keys 0-3, 8-11, 4-7, 12-15, zero past S
    S, Hkv, D = inp.v.shape
    nb = -(-S // 128)
    vf = (inp.v.view(torch.float8_e4m3fn).float() if cfg.dtype == "fp8" else inp.v.float())
    vpad = torch.zeros(nb * 128, Hkv, D, device="cuda")
    vpad[:S] = vf
    order = torch.tensor([0, 1, 2, 3, 8, 9, 10, 11, 4, 5, 6, 7, 12, 13, 14, 15], device="cuda")
    perm = (torch.arange(8, device="cuda")[:, None] * 16 + order[None, :]).reshape(-1)
    want = vpad.view(nb, 128, Hkv, D)[:, perm].permute(0, 2, 3, 1).to(torch.bfloat16)
    assert torch.equal(vp.view(nb, Hkv, D, 128).view(torch.int16),
                       want.contiguous().view(torch.int16))
    del vf, vpad, want
    scale = 1.0 / math.sqrt(cfg.head_dim)
    out0, lse0 = bsa.bsa_attention_fwd(problem, inp.q, inp.k, inp.v, sel.row_ptr, sel.col_idx,
                                       scale, inp.q_scale, inp.k_scale, inp.v_scale)
    out1, lse1 = bsa.bsa_attention_fwd_prepared_v(problem, inp.q, inp.k, vp, sel.row_ptr,
                                                  sel.col_idx, scale, inp.q_scale, inp.k_scale,
                                                  inp.v_scale)
    torch.cuda.synchronize()
    assert torch.equal(out0.view(torch.int16), out1.view(torch.int16))
    assert torch.equal(lse0, lse1)
    del inp, pool, sel, vp, out0, out1, lse0, lse1
    torch.cuda.empty_cache()


RANDOM = random_layers(48)


@pytest.mark.parametrize("cfg", RANDOM, ids=[c.name for c in RANDOM])
def test_random_small_layers_parity(cfg):
    _gpu_or_skip()
    import bsa_check as K
    print(f"[parity-random] {cfg.name} S={cfg.seq_len} Hq={cfg.num_q_heads} "
          f"Hkv={cfg.num_kv_heads} D={cfg.head_dim} B={cfg.block_size} {cfg.dtype} "
          f"{cfg.granularity} {cfg.backbone} k={cfg.top_k} gate={cfg.gate} "
          f"mass={cfg.mass_threshold} rescue={cfg.rescue_fraction} sink={cfg.force_sink}",
          flush=True)
    inp = generate(cfg, "cpu").to("cuda")
    run = K.run_gpu(cfg, inp)
    rep = K.check_all(cfg, inp, run)
    print(f"  rows={rep.rows_checked} ambiguous={rep.ambiguous_rows} kept={rep.kept_blocks} "
          f"max_abs={rep.max_abs:.3g} mean_abs={rep.mean_abs:.3g} lse={rep.lse_max:.3g}",
          flush=True)
    assert rep.ambiguous_rows <= max(1, rep.rows_checked // 100)
    if cfg.head_dim == 128 and cfg.block_size == 128:
        # attention on the prepared V tiles gives the checked outputs bit for bit
        import block_sparse_attention_36_amd as bsa
        problem = bsa.make_problem(inp.q, inp.k, cfg.block_size, K.granularity_code(cfg))
        rp = torch.from_numpy(run.row_ptr.astype(np.int32)).to("cuda")
        ci = torch.from_numpy(run.col_idx.astype(np.int32)).to("cuda")
        out, lse = bsa.bsa_attention_fwd_prepared_v(
            problem, inp.q, inp.k, bsa.bsa_prepare_v(problem, inp.v), rp, ci,
            1.0 / math.sqrt(cfg.head_dim), inp.q_scale, inp.k_scale, inp.v_scale)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), run.out.view(torch.int16))
        assert torch.equal(lse, run.lse)
