"""Plain float64 CPU oracle for block-sparse attention prefill.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg, never by the library.  It shares no
code with the HIP path.  Every function is the plain definition of one step,
written for a reader to check against the pages by eye; there is no blocking,
fusion or online rescaling.

The method, as the source pages describe it:
  * Keys are split into fixed blocks and each block is summarised by its mean
    (centroid); a query block is summarised the same way, and the block score
    is the inner product of the two means ("Uncertainty-gated selection for
    block-sparse attention", technical summary, Methodology step 1, the
    SSA-style mean-pooling backbone; RBS-Attention article, second and third
    paragraphs, centroid relevance).
  * Per query tile, the k best-scoring key blocks are kept (same page,
    Methodology step 2, the kv_idx list).
  * Uncertainty gate: when the best two candidates are nearly tied, the budget
    doubles from k to 2k (same page, lay summary "The Solution"; Methodology
    step 5 names the expansion factor rho = 2).
  * Sigma gate (the page's own formulation): per (tile, head) the normalised
    cut margin sigma = (s(k-1) - s(k)) / (s(0) - s(k)) of the sorted scores,
    averaged over heads per tile; tiles whose mean falls in the lowest part of
    the layer's empirical distribution expand to rho*k (same page, Methodology
    steps 3-5).
  * Quest backbone: each key block is summarised by the coordinate-wise minimum
    and maximum of its keys; a query row's score against the block is the
    largest q.k over that box, sum_d max(q_d kmin_d, q_d kmax_d), an upper
    bound on every key of the block; a tile scores a block by the maximum over
    its query rows (same page, Methodology steps 1-2: per-coordinate upper
    bounds as the second backbone, tile score = max over the tile's rows).
  * RBS-Attention: a base branch keeps centroid-relevant blocks under its own
    threshold, a rescue branch flags blocks whose centroid may underestimate
    them using a per-(prompt, layer, head) key-block radius; the two masks are
    unioned (RBS-Attention article, third and fourth paragraphs).
  * MSA: one index selection per GQA group, shared by the group's query heads;
    the main branch attends only over the kept blocks (MiniMax MSA article,
    "What is MSA and how does it work").
  * Attention itself is softmax(q.k / sqrt(D)) v restricted to the kept blocks
    and to causal key positions.

Readings where the pages are silent (each also listed in the design notes):
  temperature 1 for the softmax over block scores; the forced blocks (the
  diagonal, plus block 0 when a sink is requested) are outside the candidate
  set that top-k, gate, mass and rescue rank; ties break toward the lowest
  block index; the gate compares the top-two softmax probabilities with a
  strict "<"; the base branch keeps the shortest prefix whose mass reaches the
  threshold; the rescue branch keeps ceil(fraction * |candidates|) blocks by
  the bound s + ||q_mean|| * r; the radius is the largest distance of a key of
  the block from the block's own mean; a ragged last block is pooled over the
  rows it has.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

__all__ = [
    "SelectParams", "decode_bf16", "decode_e4m3", "dequantize", "decode_inputs",
    "pool_queries", "pool_keys", "block_scores", "rescue_bounds", "candidate_sets",
    "descending_order", "top_k", "gate_gap", "sigma_cut_margin", "sigma_gate_tiles",
    "sigma_matrix", "tile_gate", "key_block_bounds", "quest_row_bound", "quest_scores", "mass_prefix_length", "rescue_count",
    "select_row", "acceptable_row_sets", "select", "to_csr", "from_csr", "padded_width",
    "to_padded",
    "attend", "block_tokens", "attention_unit", "attention", "dense_causal_attention", "block_of", "unit_of_head",
    "kv_of_unit",
]


# ----------------------------------------------------------------------------
# parameters

@dataclass(frozen=True)
class SelectParams:
    """Selection rule parameters, in the precision the library receives them.

    top_k            k, the per-row budget beyond the forced blocks (0 = branch off)
    force_sink       also force block 0
    gate             "none", "top12_gap" or "sigma_cut"
    gate_threshold   top12_gap: theta, a row fires when p(0) - p(1) < theta;
                     sigma_cut: q, a tile fires when its head-mean sigma lies in
                     the lowest q fraction of the layer's tiles (float32)
    gate_factor      rho: the budget a fired row keeps is rho * k
    score_temperature tau in softmax(tau * s) (float32)
    mass_threshold   mu for the base branch (0 = branch off) (float32)
    rescue_fraction  phi for the rescue branch (0 = branch off) (float64)
    """
    top_k: int = 0
    force_sink: bool = False
    gate: str = "none"
    gate_threshold: float = 0.05
    gate_factor: int = 2
    score_temperature: float = 1.0
    mass_threshold: float = 0.0
    rescue_fraction: float = 0.0

    def as_library_precision(self) -> "SelectParams":
        f32 = lambda x: float(np.float32(x))  # noqa: E731
        return SelectParams(int(self.top_k), bool(self.force_sink), self.gate,
                            f32(self.gate_threshold), int(self.gate_factor),
                            f32(self.score_temperature), f32(self.mass_threshold),
                            float(self.rescue_fraction))


# ----------------------------------------------------------------------------
# decoding the stored bytes

def decode_bf16(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64.  bf16 is the top half of an
    IEEE binary32, so the conversion is exact."""
    b = np.asarray(bits).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def decode_e4m3(codes) -> np.ndarray:
    """OCP 8-bit E4M3 ('fn' variant) codes (uint8) -> float64.

    1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 is
    subnormal (m/8 * 2^-6); there is no infinity and only S.1111.111 is NaN;
    the largest finite magnitude is 1.75 * 2^8 = 448.
    """
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    val = np.where(e == 0, sub, normal)
    val = np.where((e == 15) & ((c & 7) == 7), np.nan, val)
    return sign * val


def block_of(S: int, B: int) -> np.ndarray:
    return np.arange(S) // B


def dequantize(codes, scales, B: int) -> np.ndarray:
    """codes [S, H, D] uint8, scales [H, nb] -> value = decode(code) * scale[h, block]."""
    x = decode_e4m3(codes)
    S = x.shape[0]
    sc = np.asarray(scales, dtype=np.float64)  # [H, nb]
    return x * sc[:, block_of(S, B)].T[:, :, None]


def decode_inputs(q, k, v, dtype: str, B: int, q_scale=None, k_scale=None, v_scale=None):
    """Raw stored arrays (uint16 bf16 bits or uint8 E4M3 codes) -> float64 Q, K, V."""
    if dtype == "bf16":
        return decode_bf16(q), decode_bf16(k), decode_bf16(v)
    return dequantize(q, q_scale, B), dequantize(k, k_scale, B), dequantize(v, v_scale, B)


# ----------------------------------------------------------------------------
# step 1: pooling ("Uncertainty-gated selection ...", Methodology step 1;
# RBS-Attention article, third paragraph: centroid and key-block radius)

def _block_ranges(S: int, B: int):
    nb = -(-S // B)
    return [(i * B, min(S, (i + 1) * B)) for i in range(nb)]


def unit_of_head(h: int, num_q_heads: int, num_kv_heads: int, granularity: str) -> int:
    """Selection unit that owns query head h: the head itself, or its GQA group."""
    return h if granularity == "qhead" else h // (num_q_heads // num_kv_heads)


def kv_of_unit(u: int, num_q_heads: int, num_kv_heads: int, granularity: str) -> int:
    return u // (num_q_heads // num_kv_heads) if granularity == "qhead" else u


def pool_queries(Q: np.ndarray, B: int, num_kv_heads: int, granularity: str):
    """Mean-pooled query blocks.

    qhead: qbar[h, i] = mean over the rows t of block i of Q[t, h].
    group: qbar[g, i] = mean over the group's heads and the block's rows (one
           index vector per GQA group, as MSA's index branch scores per group).
    Returns (qbar [U, nb, D], qnorm [U, nb] = ||qbar||_2).
    """
    S, Hq, D = Q.shape
    ranges = _block_ranges(S, B)
    G = Hq // num_kv_heads
    U = Hq if granularity == "qhead" else num_kv_heads
    qbar = np.zeros((U, len(ranges), D))
    for u in range(U):
        heads = [u] if granularity == "qhead" else list(range(u * G, (u + 1) * G))
        for i, (t0, t1) in enumerate(ranges):
            qbar[u, i] = Q[t0:t1, heads, :].reshape(-1, D).mean(axis=0)
    return qbar, np.sqrt((qbar * qbar).sum(axis=-1))


def pool_keys(K: np.ndarray, B: int):
    """Key-block centroids and radii.

    kbar[g, j]   = mean of block j's keys of kv head g.
    radius[g, j] = max over keys t of block j of ||K[t, g] - kbar[g, j]||_2.
    """
    S, Hkv, D = K.shape
    ranges = _block_ranges(S, B)
    kbar = np.zeros((Hkv, len(ranges), D))
    radius = np.zeros((Hkv, len(ranges)))
    for g in range(Hkv):
        for j, (t0, t1) in enumerate(ranges):
            rows = K[t0:t1, g, :]
            c = rows.mean(axis=0)
            kbar[g, j] = c
            radius[g, j] = np.sqrt(((rows - c) ** 2).sum(axis=1)).max()
    return kbar, radius


# ----------------------------------------------------------------------------
# step 1b: the Quest backbone's key-block summaries

def key_block_bounds(K: np.ndarray, B: int):
    """Coordinate-wise minimum and maximum of each key block ("Uncertainty-gated
    selection ...", technical summary, Methodology step 1: Quest's K-min/K-max).

    kmin[g, j, d] = min over keys t of block j of K[t, g, d]; kmax likewise.
    Returns (kmin, kmax), each [Hkv, nb, D]; a ragged last block uses its rows.
    """
    S, Hkv, D = K.shape
    ranges = _block_ranges(S, B)
    kmin = np.zeros((Hkv, len(ranges), D))
    kmax = np.zeros((Hkv, len(ranges), D))
    for j, (t0, t1) in enumerate(ranges):
        kmin[:, j] = K[t0:t1].min(axis=0)
        kmax[:, j] = K[t0:t1].max(axis=0)
    return kmin, kmax


def quest_row_bound(q_rows: np.ndarray, kmin: np.ndarray, kmax: np.ndarray) -> np.ndarray:
    """Largest q.k over the box kmin <= k <= kmax, for every query row and block:
    coordinate d contributes max(q_d * kmin_d, q_d * kmax_d).  [n_rows, n_blocks]."""
    lo = q_rows[:, None, :] * kmin[None, :, :]
    hi = q_rows[:, None, :] * kmax[None, :, :]
    return np.maximum(lo, hi).sum(axis=-1)


def quest_scores(Q: np.ndarray, kmin: np.ndarray, kmax: np.ndarray, B: int, num_kv_heads: int,
                 granularity: str) -> np.ndarray:
    """Tile scores of the Quest backbone with per-row scoring (same page,
    Methodology step 2: a tile's score is the maximum over its rows).

    s[u, i, j] = max over the query rows t of tile i, and over the heads of unit u,
    of quest_row_bound(Q[t, h], kmin[g, j], kmax[g, j]), for j <= i; NaN above
    the diagonal (g = the unit's kv head).
    """
    S, Hq, D = Q.shape
    ranges = _block_ranges(S, B)
    nb = len(ranges)
    G = Hq // num_kv_heads
    U = Hq if granularity == "qhead" else num_kv_heads
    s = np.full((U, nb, nb), np.nan)
    for u in range(U):
        heads = [u] if granularity == "qhead" else list(range(u * G, (u + 1) * G))
        g = kv_of_unit(u, Hq, num_kv_heads, granularity)
        for i, (t0, t1) in enumerate(ranges):
            rows = Q[t0:t1, heads, :].reshape(-1, D)
            s[u, i, : i + 1] = quest_row_bound(rows, kmin[g, : i + 1], kmax[g, : i + 1]).max(axis=0)
    return s


# ----------------------------------------------------------------------------
# step 2: block scores and the rescue bound

def block_scores(qbar: np.ndarray, kbar: np.ndarray, num_q_heads: int, num_kv_heads: int,
                 granularity: str) -> np.ndarray:
    """s[u, i, j] = qbar[u, i] . kbar[kv(u), j] for j <= i; NaN above the diagonal."""
    U, nb, _ = qbar.shape
    s = np.full((U, nb, nb), np.nan)
    for u in range(U):
        g = kv_of_unit(u, num_q_heads, num_kv_heads, granularity)
        full = qbar[u] @ kbar[g].T
        tri = np.tril(np.ones((nb, nb), dtype=bool))
        s[u][tri] = full[tri]
    return s


def rescue_bounds(s: np.ndarray, qnorm: np.ndarray, radius: np.ndarray, num_q_heads: int,
                  num_kv_heads: int, granularity: str) -> np.ndarray:
    """b[u, i, j] = s[u, i, j] + ||qbar[u, i]|| * radius[kv(u), j].

    By Cauchy-Schwarz, qbar . k <= qbar . kbar + ||qbar|| * ||k - kbar|| for every
    key k of block j, so b bounds every single key's dot product with the mean
    query: the block's best key cannot hide below it (RBS-Attention article,
    third paragraph: blocks at risk of being underestimated).
    """
    b = np.full_like(s, np.nan)
    U = s.shape[0]
    for u in range(U):
        g = kv_of_unit(u, num_q_heads, num_kv_heads, granularity)
        b[u] = s[u] + qnorm[u][:, None] * radius[g][None, :]
    return b


# ----------------------------------------------------------------------------
# step 3: selection of one row (unit u, query block i)

def candidate_sets(i: int, force_sink: bool):
    """Forced blocks F_i (the causal diagonal i, plus block 0 with a sink) and the
    candidates C_i = {0..i} minus F_i that the ranking rules choose among."""
    forced = {i} | ({0} if force_sink else set())
    cands = [j for j in range(i + 1) if j not in forced]
    return sorted(forced), cands


def descending_order(values: np.ndarray, idx: list) -> list:
    """idx sorted by (-value, index): descending score, lowest index first on ties."""
    return sorted(idx, key=lambda j: (-values[j], j))


def top_k(values: np.ndarray, cands: list, k: int) -> list:
    """The first min(k, |C|) candidates of the descending order ("Uncertainty-gated
    selection ...", Methodology step 2: a top-k over the tile's block scores)."""
    return descending_order(values, cands)[: max(0, min(k, len(cands)))]


def _softmax(x: np.ndarray) -> np.ndarray:
    z = np.exp(x - x.max())
    return z / z.sum()


def gate_gap(s_row: np.ndarray, cands: list, tau: float) -> float:
    """p(0) - p(1) of softmax(tau * s) over the candidates, sorted descending
    ("Uncertainty-gated selection ...", lay summary "The Solution": compare the
    best and second-best chunk).  +inf when there are fewer than two candidates."""
    if len(cands) < 2:
        return math.inf
    p = np.sort(_softmax(tau * s_row[cands]))[::-1]
    return float(p[0] - p[1])


def sigma_cut_margin(s_row: np.ndarray, cands: list, k: int) -> float:
    """Normalised cut margin of the top-k decision ("Uncertainty-gated selection
    ...", technical summary, Methodology step 3):

        sigma = (s(k-1) - s(k)) / (s(0) - s(k)),

    with s(0) >= s(1) >= ... the candidates' raw scores sorted descending and
    0-indexed, so s(k-1) is the last kept score and s(k) the first dropped one.
    sigma near 1: the kept set stands well above the tail; near 0: the k-th and
    (k+1)-th are (nearly) tied.  Only a row with a cut (|C| > k >= 1) has a
    sigma (nan otherwise); when s(0) = s(k) every score down to the cut is tied
    and sigma is 0.  With k = 1 the numerator equals the denominator, so sigma is
    1 for every row without a tie at the top."""
    if k < 1 or len(cands) <= k:
        return math.nan
    v = np.sort(np.asarray(s_row, dtype=np.float64)[cands])[::-1]
    top, last_kept, first_dropped = v[0], v[k - 1], v[k]
    if top == first_dropped:
        return 0.0
    return float((last_kept - first_dropped) / (top - first_dropped))


def sigma_matrix(s: np.ndarray, k: int, force_sink: bool) -> np.ndarray:
    """sigma[u, i] for every selection row (nan where tile i has no cut)."""
    U, nb, _ = s.shape
    sig = np.full((U, nb), np.nan)
    for i in range(nb):
        _, cands = candidate_sets(i, force_sink)
        for u in range(U):
            sig[u, i] = sigma_cut_margin(s[u, i], cands, k)
    return sig


def sigma_gate_tiles(sigma: np.ndarray, q: float):
    """Per-tile decision of the sigma gate (same page, Methodology step 4).

    sigma_bar[i] is the mean of sigma[:, i] over the selection units (each unit's
    sigma stands for every head that shares its list, so this is the mean over
    heads).  The layer's empirical distribution is that of sigma_bar over its
    T tiles with a cut; tile i fires when the fraction of those tiles whose
    sigma_bar is at most its own is at most q, i.e. when
        #{t : sigma_bar[t] <= sigma_bar[i]} <= q * T   (q * T in IEEE double).
    With distinct values that is the floor(q*T) most ambiguous tiles; a tile
    without a cut never fires.  Returns (sigma_bar [nb], fired [nb] bool)."""
    sbar = np.asarray(sigma, dtype=np.float64).mean(axis=0)
    elig = ~np.isnan(sbar)
    vals = sbar[elig]
    limit = float(q) * float(len(vals))
    fired = np.zeros(sbar.shape[0], dtype=bool)
    for i in np.nonzero(elig)[0]:
        fired[i] = np.count_nonzero(vals <= sbar[i]) <= limit
    return sbar, fired


def tile_gate(s: np.ndarray, p: "SelectParams"):
    """(sigma_bar, fired) of every tile for the sigma gate, or None when the gate
    is not the sigma gate or the top-k branch is off."""
    if p.gate != "sigma_cut" or p.top_k <= 0:
        return None
    return sigma_gate_tiles(sigma_matrix(s, p.top_k, p.force_sink), p.gate_threshold)


def mass_cumulative(s_row: np.ndarray, cands: list, tau: float):
    """(order, cum): candidates in descending order and the running sums of their
    softmax(tau * s) probabilities, cum[n] = mass of the first n (cum[0] = 0)."""
    order = descending_order(s_row, cands)
    if not order:
        return order, np.zeros(1)
    p = _softmax(tau * s_row[order])
    return order, np.concatenate([[0.0], np.cumsum(p)])


def mass_prefix_length(cum: np.ndarray, mu: float) -> int:
    """Shortest prefix whose mass reaches mu (RBS-Attention base branch: keep
    blocks up to a cumulative-mass threshold); all candidates if none does."""
    n = len(cum) - 1
    for m in range(1, n + 1):
        if cum[m] >= mu:
            return m
    return n


def rescue_count(num_cands: int, phi: float) -> int:
    """ceil(phi * |C|), evaluated in IEEE double."""
    if phi <= 0.0 or num_cands == 0:
        return 0
    return min(num_cands, int(math.ceil(phi * num_cands)))


def _kept_set(i, s_row, b_row, p: SelectParams, gate_fired: bool, n_mass: int | None):
    forced, cands = candidate_sets(i, p.force_sink)
    kept = set(forced)
    if p.top_k > 0:
        keff = p.top_k * (p.gate_factor if gate_fired else 1)
        kept |= set(top_k(s_row, cands, keff))
    if p.mass_threshold > 0.0 and n_mass is not None:
        order = descending_order(s_row, cands)
        kept |= set(order[:n_mass])
    if p.rescue_fraction > 0.0:
        kept |= set(top_k(b_row, cands, rescue_count(len(cands), p.rescue_fraction)))
    return sorted(kept)


def select_row(i: int, s_row: np.ndarray, b_row: np.ndarray | None, p: SelectParams,
               tile_fired: bool = False):
    """Kept key blocks of one selection row, plus the gate decision.

    kept = forced  U  top-k (k doubled when the gate fires)  U  mass prefix  U  rescue,
    each branch present only when its parameter is on (RBS-Attention article,
    third paragraph: independent thresholds per branch, masks fused).  The sigma
    gate is decided per tile over the whole layer (``tile_gate``); its decision
    for this row's tile comes in as ``tile_fired``.
    """
    _, cands = candidate_sets(i, p.force_sink)
    fired = False
    if p.gate == "top12_gap" and p.top_k > 0:
        fired = gate_gap(s_row, cands, p.score_temperature) < p.gate_threshold
    elif p.gate == "sigma_cut" and p.top_k > 0:
        fired = bool(tile_fired)
    n_mass = None
    if p.mass_threshold > 0.0:
        _, cum = mass_cumulative(s_row, cands, p.score_temperature)
        n_mass = mass_prefix_length(cum, p.mass_threshold)
    return _kept_set(i, s_row, b_row, p, fired, n_mass), fired


def acceptable_row_sets(i: int, s_row: np.ndarray, b_row, p: SelectParams, delta: float,
                        tile_fired_options=(False,)):
    """All kept sets reachable when a threshold decision whose float64 quantity lies
    within delta of its threshold is taken either way (a float32 evaluation of the
    same softmax may land on the other side).  For the sigma gate the caller
    passes the tile decisions it accepts.  Returns (list of (kept, fired),
    ambiguous flag)."""
    _, cands = candidate_sets(i, p.force_sink)
    gate_opts = [False]
    if p.gate == "sigma_cut" and p.top_k > 0:
        gate_opts = [bool(f) for f in tile_fired_options]
    if p.gate == "top12_gap" and p.top_k > 0:
        gap = gate_gap(s_row, cands, p.score_temperature)
        fired = gap < p.gate_threshold
        gate_opts = [fired]
        if math.isfinite(gap) and abs(gap - p.gate_threshold) < delta:
            gate_opts = [True, False]
    mass_opts = [None]
    if p.mass_threshold > 0.0:
        _, cum = mass_cumulative(s_row, cands, p.score_temperature)
        n0 = mass_prefix_length(cum, p.mass_threshold)
        mu = p.mass_threshold
        n = len(cum) - 1
        mass_opts = [m for m in range(0, n + 1)
                     if (m == n or cum[m] >= mu - delta) and (m == 0 or cum[m - 1] < mu + delta)]
        if n0 not in mass_opts:
            mass_opts.append(n0)
    out = []
    for f in gate_opts:
        for m in mass_opts:
            ks = _kept_set(i, s_row, b_row, p, f, m)
            if (ks, f) not in out:
                out.append((ks, f))
    return out, len(out) > 1


def select(s: np.ndarray, b: np.ndarray | None, p: SelectParams):
    """Selection for every row: returns (kept [U][nb] lists, gate flags [U, nb])."""
    U, nb, _ = s.shape
    kept = [[None] * nb for _ in range(U)]
    fired = np.zeros((U, nb), dtype=bool)
    tg = tile_gate(s, p)
    tiles = tg[1] if tg is not None else np.zeros(nb, dtype=bool)
    for u in range(U):
        for i in range(nb):
            kept[u][i], fired[u, i] = select_row(i, s[u, i], None if b is None else b[u, i], p,
                                                 bool(tiles[i]))
    return kept, fired


def to_csr(kept):
    """Row-major CSR over rows (u, i): row_ptr[u*nb + i] .. col_idx ascending."""
    rows = [r for unit in kept for r in unit]
    row_ptr = np.zeros(len(rows) + 1, dtype=np.int64)
    for n, r in enumerate(rows):
        row_ptr[n + 1] = row_ptr[n] + len(r)
    col_idx = np.array([j for r in rows for j in r], dtype=np.int64)
    return row_ptr, col_idx


def padded_width(nb: int, p: SelectParams) -> int:
    """Slots per row of the sentinel-padded index list: the largest kept set the
    rule can produce in any row, so one uniform shape holds every row whether
    or not its gate fired ("Uncertainty-gated selection ...", technical summary,
    Methodology step 5: non-triggered tiles padded with sentinels).  A row keeps
    its forced blocks plus at most rho*k (gated) or k by top-k, at most
    ceil(phi*|C|) by rescue, and every candidate when the mass branch is on."""
    width = 0
    for i in range(nb):
        forced, cands = candidate_sets(i, p.force_sink)
        n = len(forced)
        if p.mass_threshold > 0.0:
            n += len(cands)
        else:
            if p.top_k > 0:
                n += min(len(cands), p.top_k * (p.gate_factor if p.gate != "none" else 1))
            if p.rescue_fraction > 0.0:
                n += rescue_count(len(cands), p.rescue_fraction)
        width = max(width, min(n, i + 1))
    return width


def to_padded(kept, width: int) -> np.ndarray:
    """[rows, width] block ids: each row's kept blocks ascending, then -1."""
    rows = [r for unit in kept for r in unit]
    out = np.full((len(rows), width), -1, dtype=np.int64)
    for n, r in enumerate(rows):
        assert len(r) <= width
        out[n, : len(r)] = r
    return out


def from_csr(row_ptr, col_idx, U: int, nb: int):
    row_ptr = np.asarray(row_ptr)
    col_idx = np.asarray(col_idx)
    return [[list(col_idx[row_ptr[u * nb + i]: row_ptr[u * nb + i + 1]]) for i in range(nb)]
            for u in range(U)]


# ----------------------------------------------------------------------------
# step 4: attention restricted to the kept blocks (RBS-Attention article, third
# paragraph, sparse FlashAttention over the fused mask; MSA article, the main
# branch attends only over the preselected blocks)

def attend(q: np.ndarray, q_pos: np.ndarray, k: np.ndarray, v: np.ndarray, k_pos: np.ndarray,
           scale: float):
    """Attention of query rows q (token positions q_pos) over key/value rows k, v
    (positions k_pos): for row t, allowed keys A_t = {s : k_pos[s] <= q_pos[t]};
    logits l_s = scale * q_t . k_s; O_t = sum_s softmax(l)_s v_s; lse_t = log sum_s
    exp(l_s) (natural log).  Written directly: all allowed logits at once."""
    logits = scale * (q @ k.T)
    allowed = k_pos[None, :] <= q_pos[:, None]
    logits = np.where(allowed, logits, -np.inf)
    mx = logits.max(axis=1, keepdims=True)
    w = np.exp(logits - mx)
    z = w.sum(axis=1, keepdims=True)
    return (w / z) @ v, (mx + np.log(z))[:, 0]


def block_tokens(blocks, B: int, S: int) -> np.ndarray:
    """Token positions of the given blocks, in order (the last block may be ragged)."""
    return np.concatenate([np.arange(j * B, min(S, (j + 1) * B)) for j in blocks])


def attention_unit(Q, K, V, h: int, i: int, kept_blocks, B: int, scale: float, kvh: int):
    """Output rows and log-sum-exp of query block i, head h, over the kept blocks."""
    S = Q.shape[0]
    t0, t1 = i * B, min(S, (i + 1) * B)
    keys = block_tokens(kept_blocks, B, S)
    return attend(Q[t0:t1, h, :], np.arange(t0, t1), K[keys, kvh, :], V[keys, kvh, :], keys, scale)


def attention(Q, K, V, kept, B: int, scale: float, granularity: str, heads=None, blocks=None):
    """Block-sparse attention for the given heads x query blocks (all by default).

    kept[u][i] lists the kept key blocks of selection row (u, i).  Returns
    (O [S, Hq, D] with NaN where not computed, lse [Hq, S]).
    """
    S, Hq, D = Q.shape
    Hkv = K.shape[1]
    nb = -(-S // B)
    O = np.full((S, Hq, D), np.nan)
    lse = np.full((Hq, S), np.nan)
    for h in (range(Hq) if heads is None else heads):
        u = unit_of_head(h, Hq, Hkv, granularity)
        kvh = h // (Hq // Hkv)
        for i in (range(nb) if blocks is None else blocks):
            t0, t1 = i * B, min(S, (i + 1) * B)
            O[t0:t1, h, :], lse[h, t0:t1] = attention_unit(Q, K, V, h, i, kept[u][i], B, scale, kvh)
    return O, lse


def dense_causal_attention(Q, K, V, scale: float):
    """softmax(scale * Q K^T with keys s > t masked) V, per head, as one S x S matrix."""
    S, Hq, D = Q.shape
    Hkv = K.shape[1]
    O = np.zeros((S, Hq, D))
    lse = np.zeros((Hq, S))
    causal = np.tril(np.ones((S, S), dtype=bool))
    for h in range(Hq):
        g = h // (Hq // Hkv)
        logits = np.where(causal, scale * (Q[:, h, :] @ K[:, g, :].T), -np.inf)
        mx = logits.max(axis=1, keepdims=True)
        w = np.exp(logits - mx)
        z = w.sum(axis=1, keepdims=True)
        O[:, h, :] = (w / z) @ V[:, g, :]
        lse[h] = (mx + np.log(z))[:, 0]
    return O, lse
