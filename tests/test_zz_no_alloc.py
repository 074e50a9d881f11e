"""The allocation-free selection entry point (bsa_score_select_noalloc) against
bsa_score_select on the same inputs: the same kernels on the library's fixed
scratch instead of a caller workspace, so the kept lists, gate flags, scores and
bounds must be bitwise equal.  Two calls in a row, the second on a smaller
problem, then a request beyond the scratch."""

import ctypes

import numpy as np
import pytest
import torch

from workloads import config_by_name, generate, scaled

pytestmark = pytest.mark.gpu


def _gpu_or_skip():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


CASES = [
    # mass + rescue branches, scores kept in the scratch (no export)
    scaled(config_by_name("dual128k"), 4096 + 77, num_q_heads=8, num_kv_heads=2),
    # smaller, the gap gate with a sink
    scaled(config_by_name("gated64k"), 2048 + 5, num_q_heads=4, num_kv_heads=2),
    # smaller still, the sigma gate (its tile buffers in the scratch too)
    scaled(config_by_name("sigma64k"), 1024 + 3, num_q_heads=4, num_kv_heads=1),
]


def _csr(sel):
    rp = sel.row_ptr.cpu().numpy()
    return rp, sel.col_idx[: int(rp[-1])].cpu().numpy()


def test_noalloc_matches_the_workspace_entry_point():
    _gpu_or_skip()
    import block_sparse_attention_36_amd as bsa
    import bsa_check as K
    for cfg in CASES:
        print(f"[noalloc] {cfg.name} S={cfg.seq_len} Hq={cfg.num_q_heads}", flush=True)
        inp = generate(cfg, "cpu").to("cuda")
        problem = bsa.make_problem(inp.q, inp.k, cfg.block_size, K.granularity_code(cfg))
        params = K.lib_params(cfg)
        pool = bsa.bsa_pool(problem, inp.q, inp.k, inp.q_scale, inp.k_scale)
        for export in (False, True):
            ref = bsa.bsa_score_select(problem, params, pool, export=export)
            got = bsa.bsa_score_select_noalloc(problem, params, pool, export=export)
            torch.cuda.synchronize()
            assert not ref.overflowed()
            rp0, ci0 = _csr(ref)
            rp1, ci1 = _csr(got)
            assert np.array_equal(rp0, rp1) and np.array_equal(ci0, ci1)
            if export:
                nb = cfg.num_blocks
                tri = torch.tril(torch.ones(nb, nb, dtype=torch.bool, device="cuda"))
                assert torch.equal(ref.scores[:, tri], got.scores[:, tri])
                if ref.bounds is not None:
                    assert torch.equal(ref.bounds[:, tri], got.bounds[:, tri])
                assert torch.equal(ref.gate, got.gate)
        print(f"  rows={len(rp0) - 1} kept={int(rp0[-1])}", flush=True)


def test_noalloc_rejects_a_request_beyond_its_scratch():
    """The 1M-token per-group layer without a score export would need the
    8 x 8192 x 8192 score matrix in the scratch: rejected before any launch."""
    _gpu_or_skip()
    import block_sparse_attention_36_amd as bsa
    lib = bsa.load_library()
    cfg = config_by_name("msa1m")
    p = bsa.Problem(cfg.seq_len, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                    cfg.block_size, bsa.BSA_FP8_E4M3, bsa.BSA_SEL_PER_GROUP)
    s = bsa.make_params(top_k=cfg.top_k)
    cap = lib.bsa_csr_capacity_bound(ctypes.byref(p), ctypes.byref(s))
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    st = lib.bsa_score_select_noalloc(ctypes.byref(p), ctypes.byref(s), fake, None, fake, None,
                                      fake, fake, cap, None, None, None, None)
    assert st == 4 and b"scratch" in lib.bsa_last_error()
