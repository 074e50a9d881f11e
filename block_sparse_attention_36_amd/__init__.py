"""Python binding of libbsa, the block-sparse attention prefill library for MI355X.

The binding marshals arguments only: every step runs in the HIP kernels of
``libbsa.so`` (built in-tree by ``python -m block_sparse_attention_36_amd.build``).
PyTorch provides device memory and the current stream.  If the library is not
built, every call raises ``RuntimeError``; there is no CPU fallback.

Entry points (same names as the C ABI in include/bsa.h):
  bsa_pool(q, k, ...)            -> PoolResult (centroids, norms, radii)
  bsa_score_select(pool, ...)    -> Selection (row_ptr, col_idx, optional exports)
  bsa_attention_fwd(q, k, v, ...) -> (out, lse)
and ``prefill`` chaining the three for one layer.

Tensor layout: q [S, Hq, D], k/v [S, Hkv, D]; torch.bfloat16, or uint8 /
torch.float8_e4m3fn holding OCP E4M3 codes with float32 scales [H, ceil(S/B)].
"""

from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
# BSA_LIBRARY overrides the in-tree build (e.g. the sanitized build of the C ABI)
LIB_PATH = os.environ.get("BSA_LIBRARY") or os.path.join(_HERE, "libbsa.so")

BSA_OK = 0
BSA_BF16, BSA_FP8_E4M3 = 0, 1
BSA_SEL_PER_QHEAD, BSA_SEL_PER_GROUP = 0, 1
BSA_GATE_NONE, BSA_GATE_TOP12_GAP, BSA_GATE_SIGMA_CUT = 0, 1, 2
GATE_CODES = {"none": BSA_GATE_NONE, "top12_gap": BSA_GATE_TOP12_GAP, "sigma_cut": BSA_GATE_SIGMA_CUT}
STATUS_NAMES = {0: "BSA_OK", 1: "BSA_ERR_INVALID_ARGUMENT", 2: "BSA_ERR_UNSUPPORTED",
                3: "BSA_ERR_CAPACITY", 4: "BSA_ERR_WORKSPACE", 5: "BSA_ERR_DEVICE"}


class Problem(ctypes.Structure):
    _fields_ = [("seq_len", ctypes.c_int64), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("granularity", ctypes.c_int32)]


class SelectParams(ctypes.Structure):
    _fields_ = [("top_k", ctypes.c_int32), ("force_sink", ctypes.c_int32),
                ("gate", ctypes.c_int32), ("gate_threshold", ctypes.c_float),
                ("gate_factor", ctypes.c_int32), ("score_temperature", ctypes.c_float),
                ("mass_threshold", ctypes.c_float), ("reserved", ctypes.c_int32),
                ("rescue_fraction", ctypes.c_double)]


class BsaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {detail}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libbsa.so and declare its C signatures (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libbsa.so is not built ({path}); run "
                           "`python -m block_sparse_attention_36_amd.build`")
    L = ctypes.CDLL(path)
    P, V, I32, I64, F, SZ = (ctypes.c_void_p, None, ctypes.c_int32, ctypes.c_int64,
                             ctypes.c_float, ctypes.c_size_t)
    PP, PS = ctypes.POINTER(Problem), ctypes.POINTER(SelectParams)
    sigs = {
        "bsa_abi_version": ([], ctypes.c_int),
        "bsa_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "bsa_last_error": ([], ctypes.c_char_p),
        "bsa_num_blocks": ([PP], I64),
        "bsa_num_select_rows": ([PP], I64),
        "bsa_pool": ([PP, P, P, P, P, P, P, P, P, P], ctypes.c_int),
        "bsa_csr_capacity_bound": ([PP, PS], I64),
        "bsa_score_select_workspace_size": ([PP, PS, ctypes.c_int], SZ),
        "bsa_score_select": ([PP, PS, P, P, P, P, P, P, I64, P, P, P, P, SZ, P], ctypes.c_int),
        "bsa_score_select_noalloc": ([PP, PS, P, P, P, P, P, P, I64, P, P, P, P], ctypes.c_int),
        "bsa_attention_fwd": ([PP, P, P, P, P, P, P, P, P, F, P, P, P], ctypes.c_int),
        "bsa_expand_e4m3": ([PP, P, P, P], ctypes.c_int),
        "bsa_attention_fwd_expanded_v": ([PP, P, P, P, P, P, P, P, P, F, P, P, P], ctypes.c_int),
        "bsa_pool_key_bounds": ([PP, P, P, P, P, P], ctypes.c_int),
        "bsa_quest_scores_workspace_size": ([PP], SZ),
        "bsa_quest_scores": ([PP, P, P, P, P, P, P, SZ, P], ctypes.c_int),
        "bsa_select_scores_workspace_size": ([PP, PS], SZ),
        "bsa_select_scores": ([PP, PS, P, P, P, I64, P, P, SZ, P], ctypes.c_int),
        "bsa_padded_width": ([PP, PS], I64),
        "bsa_select_overflow_offset": ([PP, PS, ctypes.c_int], I64),
        "bsa_score_select_padded_workspace_size": ([PP, PS, ctypes.c_int], SZ),
        "bsa_score_select_padded": ([PP, PS, P, P, P, P, P, P, I64, P, P, P, P, SZ, P],
                                    ctypes.c_int),
        "bsa_attention_fwd_padded": ([PP, P, P, P, P, P, P, P, I64, F, P, P, P], ctypes.c_int),
        "bsa_prepared_v_bytes": ([PP], SZ),
        "bsa_prepare_v": ([PP, P, P, P], ctypes.c_int),
        "bsa_attention_fwd_prepared_v": ([PP, P, P, P, P, P, P, P, P, F, P, P, P], ctypes.c_int),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    del V
    _lib = L
    return L


def _check(status: int):
    if status != BSA_OK:
        raise BsaError(status, load_library().bsa_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BSA_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return BSA_FP8_E4M3
    raise TypeError(f"unsupported input dtype {t.dtype} (bfloat16 or E4M3 codes)")


def make_problem(q, k, block_size: int, granularity: int = BSA_SEL_PER_QHEAD) -> Problem:
    S, Hq, D = q.shape
    return Problem(S, Hq, k.shape[1], D, block_size, _dtype_code(q), granularity)


def make_params(top_k=0, force_sink=False, gate=BSA_GATE_NONE, gate_threshold=0.05, gate_factor=2,
                score_temperature=1.0, mass_threshold=0.0, rescue_fraction=0.0) -> SelectParams:
    return SelectParams(int(top_k), int(bool(force_sink)), int(gate), float(gate_threshold),
                        int(gate_factor), float(score_temperature), float(mass_threshold), 0,
                        float(rescue_fraction))


@dataclass
class PoolResult:
    q_centroid: object
    q_norm: object
    k_centroid: object
    k_radius: object


@dataclass
class Selection:
    row_ptr: object
    col_idx: object
    nnz: int | None = None
    scores: object = None
    bounds: object = None
    gate: object = None
    buffers: object = None

    def overflowed(self) -> bool:
        """Whether the call reported a kept set too large for its output (reads the
        workspace word back, so it synchronises with the device)."""
        return self.buffers.overflowed()


def _overflow_offset(problem, params, scores_given_or_exported) -> int:
    L = load_library()
    off = L.bsa_select_overflow_offset(ctypes.byref(problem), ctypes.byref(params),
                                       int(scores_given_or_exported))
    if off < 0:
        raise BsaError(1, load_library().bsa_last_error().decode())
    return int(off)


def _read_overflow(workspace, offset: int) -> bool:
    return bool(workspace[offset:offset + 4].view(__import__("torch").int32).item())


def _u8(t):
    import torch
    return None if t is None else (t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t)


def bsa_pool(problem: Problem, q, k, q_scale=None, k_scale=None, want_norm=True,
             want_radius=True, out: PoolResult | None = None) -> PoolResult:
    import torch
    L = load_library()
    nb = L.bsa_num_blocks(ctypes.byref(problem))
    if nb < 0:
        _check(L.bsa_pool(ctypes.byref(problem), None, None, None, None, None, None, None, None, None))
    U = problem.num_kv_heads if problem.granularity == BSA_SEL_PER_GROUP else problem.num_q_heads
    dev = q.device
    f32 = dict(dtype=torch.float32, device=dev)
    if out is None:
        out = PoolResult(torch.empty(U, nb, problem.head_dim, **f32),
                         torch.empty(U, nb, **f32) if want_norm else None,
                         torch.empty(problem.num_kv_heads, nb, problem.head_dim, **f32),
                         torch.empty(problem.num_kv_heads, nb, **f32) if want_radius else None)
    _check(L.bsa_pool(ctypes.byref(problem), _ptr(_u8(q)), _ptr(_u8(k)), _ptr(q_scale),
                      _ptr(k_scale), _ptr(out.q_centroid), _ptr(out.q_norm), _ptr(out.k_centroid),
                      _ptr(out.k_radius), _stream(dev)))
    return out


class SelectBuffers:
    """Device buffers for bsa_score_select (or, with given_scores, bsa_select_scores)
    sized once for a (problem, params) pair."""

    def __init__(self, problem: Problem, params: SelectParams, device, export=False,
                 given_scores=False):
        import torch
        L = load_library()
        rows = L.bsa_num_select_rows(ctypes.byref(problem))
        cap = L.bsa_csr_capacity_bound(ctypes.byref(problem), ctypes.byref(params))
        if rows < 0 or cap < 0:
            _check(L.bsa_score_select(ctypes.byref(problem), ctypes.byref(params), None, None,
                                      None, None, None, None, 0, None, None, None, None, 0, None))
        nb = L.bsa_num_blocks(ctypes.byref(problem))
        U = rows // max(nb, 1)
        if given_scores:
            ws = L.bsa_select_scores_workspace_size(ctypes.byref(problem), ctypes.byref(params))
        else:
            ws = L.bsa_score_select_workspace_size(ctypes.byref(problem), ctypes.byref(params),
                                                   int(export))
        self.row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=device)
        self.col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=device)
        self.capacity = cap
        self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=device)
        self.overflow_offset = _overflow_offset(problem, params, export or given_scores)
        self.scores = self.bounds = self.gate = None
        if export:
            if not given_scores:
                self.scores = torch.empty(U, nb, nb, dtype=torch.float32, device=device)
                if params.rescue_fraction > 0:
                    self.bounds = torch.empty(U, nb, nb, dtype=torch.float32, device=device)
            self.gate = torch.empty(rows, dtype=torch.uint8, device=device)

    def overflowed(self) -> bool:
        return _read_overflow(self.workspace, self.overflow_offset)


def bsa_score_select(problem: Problem, params: SelectParams, pool: PoolResult, export=False,
                     buffers: SelectBuffers | None = None) -> Selection:
    L = load_library()
    dev = pool.q_centroid.device
    b = buffers or SelectBuffers(problem, params, dev, export)
    _check(L.bsa_score_select(ctypes.byref(problem), ctypes.byref(params), _ptr(pool.q_centroid),
                              _ptr(pool.q_norm), _ptr(pool.k_centroid), _ptr(pool.k_radius),
                              _ptr(b.row_ptr), _ptr(b.col_idx), b.capacity, _ptr(b.scores),
                              _ptr(b.bounds), _ptr(b.gate), _ptr(b.workspace),
                              b.workspace.numel(), _stream(dev)))
    return Selection(b.row_ptr, b.col_idx, None, b.scores, b.bounds, b.gate, b)


def bsa_score_select_noalloc(problem: Problem, params: SelectParams, pool: PoolResult,
                             export=False, buffers: SelectBuffers | None = None) -> Selection:
    """bsa_score_select on the library's own fixed scratch instead of a workspace
    (for callers that cannot allocate; the buffers' workspace is not used)."""
    L = load_library()
    dev = pool.q_centroid.device
    b = buffers or SelectBuffers(problem, params, dev, export)
    _check(L.bsa_score_select_noalloc(ctypes.byref(problem), ctypes.byref(params),
                                      _ptr(pool.q_centroid), _ptr(pool.q_norm),
                                      _ptr(pool.k_centroid), _ptr(pool.k_radius), _ptr(b.row_ptr),
                                      _ptr(b.col_idx), b.capacity, _ptr(b.scores), _ptr(b.bounds),
                                      _ptr(b.gate), _stream(dev)))
    return Selection(b.row_ptr, b.col_idx, None, b.scores, b.bounds, b.gate, None)


def bsa_pool_key_bounds(problem: Problem, k, k_scale=None, out=None):
    """(k_min, k_max), each f32 [Hkv, nb, D]: the coordinate-wise extremes of every key block."""
    import torch
    L = load_library()
    nb = L.bsa_num_blocks(ctypes.byref(problem))
    if nb < 0:
        _check(L.bsa_pool_key_bounds(ctypes.byref(problem), None, None, None, None, None))
    if out is None:
        shape = (problem.num_kv_heads, nb, problem.head_dim)
        out = (torch.empty(shape, dtype=torch.float32, device=k.device),
               torch.empty(shape, dtype=torch.float32, device=k.device))
    _check(L.bsa_pool_key_bounds(ctypes.byref(problem), _ptr(_u8(k)), _ptr(k_scale), _ptr(out[0]),
                                 _ptr(out[1]), _stream(k.device)))
    return out


class QuestBuffers:
    """Scores [U, nb, nb] and the repacking workspace of bsa_quest_scores."""

    def __init__(self, problem: Problem, device):
        import torch
        L = load_library()
        nb = L.bsa_num_blocks(ctypes.byref(problem))
        rows = L.bsa_num_select_rows(ctypes.byref(problem))
        if nb < 0 or rows < 0:
            _check(L.bsa_quest_scores(ctypes.byref(problem), None, None, None, None, None, None, 0,
                                      None))
        U = rows // max(nb, 1)
        ws = L.bsa_quest_scores_workspace_size(ctypes.byref(problem))
        self.scores = torch.empty(U, nb, nb, dtype=torch.float32, device=device)
        self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=device)


def bsa_quest_scores(problem: Problem, q, k_min, k_max, q_scale=None,
                     buffers: QuestBuffers | None = None):
    """Quest tile scores f32 [U, nb, nb] (entries j <= i written)."""
    L = load_library()
    b = buffers or QuestBuffers(problem, q.device)
    _check(L.bsa_quest_scores(ctypes.byref(problem), _ptr(_u8(q)), _ptr(q_scale), _ptr(k_min),
                              _ptr(k_max), _ptr(b.scores), _ptr(b.workspace), b.workspace.numel(),
                              _stream(q.device)))
    return b.scores


def bsa_select_scores(problem: Problem, params: SelectParams, scores, export=False,
                      buffers: SelectBuffers | None = None) -> Selection:
    """Selection on given scores; with export the gate flags are returned too."""
    L = load_library()
    dev = scores.device
    b = buffers or SelectBuffers(problem, params, dev, export, given_scores=True)
    _check(L.bsa_select_scores(ctypes.byref(problem), ctypes.byref(params), _ptr(scores),
                               _ptr(b.row_ptr), _ptr(b.col_idx), b.capacity, _ptr(b.gate),
                               _ptr(b.workspace), b.workspace.numel(), _stream(dev)))
    return Selection(b.row_ptr, b.col_idx, None, scores if export else None, None, b.gate, b)


class PaddedBuffers:
    """The padded list [U*nb, width] and the workspace of bsa_score_select_padded."""

    def __init__(self, problem: Problem, params: SelectParams, device, export=False,
                 given_scores=False):
        import torch
        L = load_library()
        rows = L.bsa_num_select_rows(ctypes.byref(problem))
        width = L.bsa_padded_width(ctypes.byref(problem), ctypes.byref(params))
        if rows < 0 or width < 0:
            _check(L.bsa_score_select_padded(ctypes.byref(problem), ctypes.byref(params), None,
                                             None, None, None, None, None, 0, None, None, None,
                                             None, 0, None))
        nb = L.bsa_num_blocks(ctypes.byref(problem))
        U = rows // max(nb, 1)
        ws = L.bsa_score_select_padded_workspace_size(ctypes.byref(problem), ctypes.byref(params),
                                                      int(export or given_scores))
        self.width = max(int(width), 1)
        self.kv_idx = torch.empty(rows, self.width, dtype=torch.int32, device=device)
        self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=device)
        self.overflow_offset = _overflow_offset(problem, params, export or given_scores)
        self.scores = self.bounds = self.gate = None
        if export:
            if not given_scores:
                self.scores = torch.empty(U, nb, nb, dtype=torch.float32, device=device)
                if params.rescue_fraction > 0:
                    self.bounds = torch.empty(U, nb, nb, dtype=torch.float32, device=device)
            self.gate = torch.empty(rows, dtype=torch.uint8, device=device)

    def overflowed(self) -> bool:
        return _read_overflow(self.workspace, self.overflow_offset)


def bsa_score_select_padded(problem: Problem, params: SelectParams, pool: PoolResult | None = None,
                            scores=None, export=False, buffers: PaddedBuffers | None = None):
    """Selection as a padded list (centroid scores from pool, or the given scores).
    Returns the buffers (kv_idx, width, and with export the scores/bounds/gate)."""
    L = load_library()
    dev = (scores if scores is not None else pool.q_centroid).device
    b = buffers or PaddedBuffers(problem, params, dev, export, given_scores=scores is not None)
    pc = (None, None, None, None) if pool is None else (pool.q_centroid, pool.q_norm,
                                                       pool.k_centroid, pool.k_radius)
    _check(L.bsa_score_select_padded(ctypes.byref(problem), ctypes.byref(params), _ptr(pc[0]),
                                     _ptr(pc[1]), _ptr(pc[2]), _ptr(pc[3]), _ptr(scores),
                                     _ptr(b.kv_idx), b.width, _ptr(b.scores), _ptr(b.bounds),
                                     _ptr(b.gate), _ptr(b.workspace), b.workspace.numel(),
                                     _stream(dev)))
    return b


def bsa_attention_fwd_padded(problem: Problem, q, k, v, kv_idx, softmax_scale=None, q_scale=None,
                             k_scale=None, v_scale=None, want_lse=True, out=None, lse=None):
    import torch
    L = load_library()
    S, Hq, D = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty(S, Hq, D, dtype=torch.bfloat16, device=q.device)
    if want_lse and lse is None:
        lse = torch.empty(Hq, S, dtype=torch.float32, device=q.device)
    _check(L.bsa_attention_fwd_padded(ctypes.byref(problem), _ptr(_u8(q)), _ptr(_u8(k)),
                                      _ptr(_u8(v)), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale),
                                      _ptr(kv_idx), kv_idx.shape[1], float(softmax_scale),
                                      _ptr(out), _ptr(lse) if want_lse else None,
                                      _stream(q.device)))
    return out, (lse if want_lse else None)


def bsa_attention_fwd(problem: Problem, q, k, v, row_ptr, col_idx, softmax_scale=None,
                      q_scale=None, k_scale=None, v_scale=None, want_lse=True, out=None, lse=None):
    import torch
    L = load_library()
    S, Hq, D = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty(S, Hq, D, dtype=torch.bfloat16, device=q.device)
    if want_lse and lse is None:
        lse = torch.empty(Hq, S, dtype=torch.float32, device=q.device)
    _check(L.bsa_attention_fwd(ctypes.byref(problem), _ptr(_u8(q)), _ptr(_u8(k)), _ptr(_u8(v)),
                               _ptr(q_scale), _ptr(k_scale), _ptr(v_scale), _ptr(row_ptr),
                               _ptr(col_idx), float(softmax_scale), _ptr(out),
                               _ptr(lse) if want_lse else None, _stream(q.device)))
    return out, (lse if want_lse else None)


def bsa_expand_e4m3(problem: Problem, v, out=None):
    """The E4M3 V codes [S, Hkv, D] as their exact bf16 values (v_scale not applied)."""
    import torch
    L = load_library()
    if out is None:
        out = torch.empty(v.shape, dtype=torch.bfloat16, device=v.device)
    _check(L.bsa_expand_e4m3(ctypes.byref(problem), _ptr(_u8(v)), _ptr(out), _stream(v.device)))
    return out


def bsa_attention_fwd_expanded_v(problem: Problem, q, k, v_bf16, row_ptr, col_idx,
                                 softmax_scale=None, q_scale=None, k_scale=None, v_scale=None,
                                 want_lse=True, out=None, lse=None):
    """bsa_attention_fwd for E4M3 inputs with V given as bsa_expand_e4m3's bf16 values."""
    import torch
    L = load_library()
    S, Hq, D = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty(S, Hq, D, dtype=torch.bfloat16, device=q.device)
    if want_lse and lse is None:
        lse = torch.empty(Hq, S, dtype=torch.float32, device=q.device)
    _check(L.bsa_attention_fwd_expanded_v(
        ctypes.byref(problem), _ptr(_u8(q)), _ptr(_u8(k)), _ptr(v_bf16), _ptr(q_scale),
        _ptr(k_scale), _ptr(v_scale), _ptr(row_ptr), _ptr(col_idx), float(softmax_scale),
        _ptr(out), _ptr(lse) if want_lse else None, _stream(q.device)))
    return out, (lse if want_lse else None)


def bsa_prepare_v(problem: Problem, v, out=None):
    """V [S, Hkv, 128] (bf16 or E4M3 codes) as the transposed bf16 tiles
    [nb, Hkv, 128, 128] bsa_attention_fwd_prepared_v reads (head_dim = block_size =
    128; E4M3 codes expanded exactly, v_scale not applied)."""
    import torch
    L = load_library()
    nbytes = L.bsa_prepared_v_bytes(ctypes.byref(problem))
    if nbytes == 0:
        _check(L.bsa_prepare_v(ctypes.byref(problem), None, None, None))
    if out is None:
        out = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=v.device)
    _check(L.bsa_prepare_v(ctypes.byref(problem), _ptr(_u8(v)), _ptr(out), _stream(v.device)))
    return out


def bsa_attention_fwd_prepared_v(problem: Problem, q, k, v_prepared, row_ptr, col_idx,
                                 softmax_scale=None, q_scale=None, k_scale=None, v_scale=None,
                                 want_lse=True, out=None, lse=None):
    """bsa_attention_fwd with V given as bsa_prepare_v's tiles (bitwise the same results)."""
    import torch
    L = load_library()
    S, Hq, D = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty(S, Hq, D, dtype=torch.bfloat16, device=q.device)
    if want_lse and lse is None:
        lse = torch.empty(Hq, S, dtype=torch.float32, device=q.device)
    _check(L.bsa_attention_fwd_prepared_v(
        ctypes.byref(problem), _ptr(_u8(q)), _ptr(_u8(k)), _ptr(v_prepared), _ptr(q_scale),
        _ptr(k_scale), _ptr(v_scale), _ptr(row_ptr), _ptr(col_idx), float(softmax_scale),
        _ptr(out), _ptr(lse) if want_lse else None, _stream(q.device)))
    return out, (lse if want_lse else None)


def prefill_quest(q, k, v, block_size: int, params: SelectParams, granularity=BSA_SEL_PER_QHEAD,
                  q_scale=None, k_scale=None, v_scale=None, softmax_scale=None, export=False):
    """One layer on the Quest backbone: key bounds -> tile scores -> select -> attention.
    Returns (out, lse, selection, (k_min, k_max))."""
    problem = make_problem(q, k, block_size, granularity)
    bounds = bsa_pool_key_bounds(problem, k, k_scale)
    scores = bsa_quest_scores(problem, q, bounds[0], bounds[1], q_scale)
    sel = bsa_select_scores(problem, params, scores, export=export)
    out, lse = bsa_attention_fwd(problem, q, k, v, sel.row_ptr, sel.col_idx, softmax_scale,
                                 q_scale, k_scale, v_scale)
    return out, lse, sel, bounds


def prefill(q, k, v, block_size: int, params: SelectParams, granularity=BSA_SEL_PER_QHEAD,
            q_scale=None, k_scale=None, v_scale=None, softmax_scale=None, export=False):
    """One layer: pool -> score/select -> attention.  Returns (out, lse, selection, pool)."""
    problem = make_problem(q, k, block_size, granularity)
    rescue = params.rescue_fraction > 0
    pool = bsa_pool(problem, q, k, q_scale, k_scale, want_norm=rescue, want_radius=rescue)
    sel = bsa_score_select(problem, params, pool, export=export)
    if problem.dtype == BSA_FP8_E4M3 and problem.head_dim == 128 and problem.block_size == 128:
        # V codes expanded once into the transposed bf16 tiles the P V products read
        out, lse = bsa_attention_fwd_prepared_v(problem, q, k, bsa_prepare_v(problem, v),
                                                sel.row_ptr, sel.col_idx, softmax_scale,
                                                q_scale, k_scale, v_scale)
    elif problem.dtype == BSA_FP8_E4M3:  # V codes expanded to bf16 once, attention reads those
        out, lse = bsa_attention_fwd_expanded_v(problem, q, k, bsa_expand_e4m3(problem, v),
                                                sel.row_ptr, sel.col_idx, softmax_scale,
                                                q_scale, k_scale, v_scale)
    else:
        out, lse = bsa_attention_fwd(problem, q, k, v, sel.row_ptr, sel.col_idx, softmax_scale,
                                     q_scale, k_scale, v_scale)
    return out, lse, sel, pool
