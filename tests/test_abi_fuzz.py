"""Randomised checks of the C ABI's host layer, no GPU.

Problems and selection parameters are drawn from valid, edge and invalid values
(zero, negative and huge sizes, unsupported head and block sizes, NaN and
infinite thresholds).  Every sizing call must return, and the sizes must agree
with each other and with the closed forms of the problem.  Every entry point is
called with all of its pointers NULL: it must fail its validation before any
device call (or do nothing for an empty sequence) and name the reason.  The
sanitized build of the host layer runs this file again under ASan and UBSan."""

import ctypes
import os
import zlib

import numpy as np
import pytest

import block_sparse_attention_36_amd as bsa

NAN, INF = float("nan"), float("inf")
SEQ = [-1, 0, 1, 63, 64, 65, 127, 128, 129, 4096, 131072 + 5, 1 << 20, (1 << 31) - 1, 1 << 31,
       1 << 40, 1 << 62]
HEADS = [-1, 0, 1, 2, 3, 4, 8, 16, 64, 65, (1 << 31) - 1]
DIMS = [-64, 0, 32, 64, 96, 128, 256]
BLOCKS = [-128, 0, 16, 32, 64, 128, 256]
CODES = [-1, 0, 1, 2]
FLOATS = [NAN, INF, -INF, -1.0, 0.0, 1e-30, 0.05, 0.3, 0.5, 0.9, 1.0, 1.0000001, 2.0]
INTS = [-1, 0, 1, 2, 4, 32, 64, 1 << 20, (1 << 31) - 1]
N_CASES = 1500


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bsa.LIB_PATH):
        from block_sparse_attention_36_amd import build
        build.build()
    return bsa.load_library()


def _pick(rng, values, valid=None, p_valid=0.6):
    if valid is not None and rng.random() < p_valid:
        return valid[rng.integers(len(valid))]
    return values[rng.integers(len(values))]


def _problem(rng):
    hkv = _pick(rng, HEADS, [1, 2, 4, 8])
    hq = _pick(rng, HEADS, [hkv, 2 * hkv, 4 * hkv, 8 * hkv] if hkv > 0 else None)
    return bsa.Problem(seq_len=int(_pick(rng, SEQ, [0, 1, 129, 4096, 65536 + 17])),
                       num_q_heads=int(hq), num_kv_heads=int(hkv),
                       head_dim=int(_pick(rng, DIMS, [64, 128])),
                       block_size=int(_pick(rng, BLOCKS, [64, 128])),
                       dtype=int(_pick(rng, CODES, [0, 1])),
                       granularity=int(_pick(rng, CODES, [0, 1])))


def _params(rng):
    s = bsa.SelectParams()
    s.top_k = int(_pick(rng, INTS, [0, 4, 32]))
    s.force_sink = int(_pick(rng, CODES, [0, 1]))
    s.gate = int(_pick(rng, CODES + [3], [0, 1, 2]))
    s.gate_threshold = float(_pick(rng, FLOATS, [0.05, 0.3]))
    s.gate_factor = int(_pick(rng, INTS, [1, 2]))
    s.score_temperature = float(_pick(rng, FLOATS, [1.0]))
    s.mass_threshold = float(_pick(rng, FLOATS, [0.0, 0.9]))
    s.reserved = 0 if rng.random() < 0.9 else 1
    s.rescue_fraction = float(_pick(rng, FLOATS, [0.0, 0.05]))
    return s


def _valid_shape(p):
    """(nb, units) when the problem's counts are consistent, else None (sizes aside)."""
    if p.seq_len < 0 or p.num_q_heads < 1 or p.num_kv_heads < 1:
        return None
    if p.num_q_heads % p.num_kv_heads or p.dtype not in (0, 1) or p.granularity not in (0, 1):
        return None
    if p.block_size <= 0:
        return None
    nb = -(-p.seq_len // p.block_size)
    units = p.num_kv_heads if p.granularity == bsa.BSA_SEL_PER_GROUP else p.num_q_heads
    return nb, units


def _fails_with_reason(lib, st):
    assert st in (1, 2, 3, 4), st
    assert lib.bsa_last_error() not in (None, b"")
    assert lib.bsa_status_string(st) not in (None, b"")


def test_sizes_agree_on_random_problems(lib):
    rng = np.random.default_rng(20251)
    accepted = 0
    for _ in range(N_CASES):
        p, s = _problem(rng), _params(rng)
        P, S = ctypes.byref(p), ctypes.byref(s)
        nb = lib.bsa_num_blocks(P)
        rows = lib.bsa_num_select_rows(P)
        shape = _valid_shape(p)
        if nb == -1:
            assert rows == -1
            assert lib.bsa_csr_capacity_bound(P, S) == -1
            assert lib.bsa_score_select_workspace_size(P, S, 0) == 0
            assert lib.bsa_quest_scores_workspace_size(P) == 0
            assert lib.bsa_padded_width(P, S) == -1
            assert lib.bsa_select_overflow_offset(P, S, 0) == -1
            continue
        # an accepted problem has consistent counts and a supported head and block size
        assert shape is not None, (p.seq_len, p.num_q_heads, p.num_kv_heads)
        assert p.head_dim in (64, 128) and p.block_size in (64, 128)
        assert (nb, rows) == (shape[0], shape[0] * shape[1])
        accepted += 1
        cap = lib.bsa_csr_capacity_bound(P, S)
        if cap == -1:  # the parameters were rejected: every size that needs them says so
            assert lib.bsa_score_select_workspace_size(P, S, 1) == 0
            assert lib.bsa_padded_width(P, S) == -1
            assert lib.bsa_select_overflow_offset(P, S, 1) == -1
            assert lib.bsa_select_scores_workspace_size(P, S) == 0
            continue
        # every row keeps its diagonal block and at most its i + 1 candidates
        assert rows <= cap <= shape[1] * nb * (nb + 1) // 2
        width = lib.bsa_padded_width(P, S)
        assert (width == 0) if nb == 0 else (1 <= width <= nb)
        for export in (0, 1):
            ws = lib.bsa_score_select_workspace_size(P, S, export)
            off = lib.bsa_select_overflow_offset(P, S, export)
            assert ws > 0 and 0 <= off and off + 4 <= ws
    assert accepted > N_CASES // 5  # the draw reaches the accepted region often


ENTRY_POINTS = {
    "bsa_pool": lambda L, P, S: L.bsa_pool(P, *([None] * 9)),
    "bsa_score_select": lambda L, P, S: L.bsa_score_select(P, S, *([None] * 6), 10**9, None,
                                                           None, None, None, 10**12, None),
    "bsa_score_select_noalloc": lambda L, P, S: L.bsa_score_select_noalloc(
        P, S, *([None] * 6), 10**9, None, None, None, None),
    "bsa_score_select_padded": lambda L, P, S: L.bsa_score_select_padded(
        P, S, *([None] * 6), 10**9, None, None, None, None, 10**12, None),
    "bsa_attention_fwd": lambda L, P, S: L.bsa_attention_fwd(P, *([None] * 8), 0.125, None,
                                                             None, None),
    "bsa_attention_fwd_padded": lambda L, P, S: L.bsa_attention_fwd_padded(
        P, *([None] * 7), 64, 0.125, None, None, None),
    "bsa_attention_fwd_expanded_v": lambda L, P, S: L.bsa_attention_fwd_expanded_v(
        P, *([None] * 8), 0.125, None, None, None),
    "bsa_expand_e4m3": lambda L, P, S: L.bsa_expand_e4m3(P, None, None, None),
    "bsa_prepare_v": lambda L, P, S: L.bsa_prepare_v(P, None, None, None),
    "bsa_attention_fwd_prepared_v": lambda L, P, S: L.bsa_attention_fwd_prepared_v(
        P, *([None] * 8), 0.125, None, None, None),
    "bsa_pool_key_bounds": lambda L, P, S: L.bsa_pool_key_bounds(P, *([None] * 5)),
    "bsa_quest_scores": lambda L, P, S: L.bsa_quest_scores(P, *([None] * 6), 10**12, None),
    "bsa_select_scores": lambda L, P, S: L.bsa_select_scores(P, S, None, None, None, 10**9,
                                                             None, None, 10**12, None),
}


@pytest.mark.parametrize("name", sorted(ENTRY_POINTS))
def test_entry_points_reject_missing_pointers_on_random_problems(lib, name):
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    call = ENTRY_POINTS[name]
    for _ in range(300):
        p, s = _problem(rng), _params(rng)
        st = call(lib, ctypes.byref(p), ctypes.byref(s))
        if st == 0:
            # only an accepted empty sequence succeeds without buffers (nothing launched)
            assert p.seq_len == 0 and lib.bsa_num_blocks(ctypes.byref(p)) == 0, name
        else:
            _fails_with_reason(lib, st)


def test_non_finite_scales_and_thresholds_never_pass_validation(lib):
    p = bsa.Problem(seq_len=4096, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=128,
                    dtype=0, granularity=0)
    P = ctypes.byref(p)
    for field, values in (("score_temperature", (NAN, INF, -INF, 0.0)),
                          ("mass_threshold", (NAN, INF, -0.5, 1.5)),
                          ("rescue_fraction", (NAN, INF, -0.5, 1.5))):
        for v in values:
            s = bsa.make_params(top_k=4)
            setattr(s, field, v)
            assert lib.bsa_csr_capacity_bound(P, ctypes.byref(s)) == -1, (field, v)
    for gate in (1, 2):
        for v in (NAN, INF, 0.0, -1.0, 1.5):
            s = bsa.make_params(top_k=4, gate=gate, gate_threshold=0.05, gate_factor=2)
            s.gate_threshold = v
            assert lib.bsa_csr_capacity_bound(P, ctypes.byref(s)) == -1, (gate, v)


def test_last_error_is_per_thread(lib):
    """Threads that fail in different ways each read back their own reason."""
    import threading

    reasons = {}
    barrier = threading.Barrier(4)

    def worker(t):
        p = bsa.Problem(seq_len=4096, num_q_heads=8, num_kv_heads=2, head_dim=128,
                        block_size=128, dtype=0, granularity=0)
        if t == 0:
            p.head_dim = 96
        elif t == 1:
            p.num_q_heads = 6
            p.num_kv_heads = 4
        elif t == 2:
            p.dtype = 7
        # (thread 3 keeps a valid problem: it fails on the missing buffers)
        P = ctypes.byref(p)
        barrier.wait()
        for _ in range(200):
            st = lib.bsa_pool(P, *([None] * 9))
            reasons.setdefault(t, set()).add((st, lib.bsa_last_error()))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    for t in range(4):
        assert len(reasons[t]) == 1, (t, reasons[t])  # the same reason on every call
    assert len({next(iter(reasons[t]))[1] for t in range(4)}) == 4  # and four different ones
