"""Seeded generators for the synthetic prefill inputs.

Layout of what is produced (the layout the library consumes):
  q : [S, Hq, D]   k, v : [S, Hkv, D]   token-major, contiguous, batch 1.
  bf16 workloads: torch.bfloat16 tensors.
  fp8 workloads : torch.uint8 tensors holding OCP E4M3 codes, plus float32
                  scales q_scale [Hq, nb], k_scale/v_scale [Hkv, nb]; the real
                  value of an element is decode(code) * scale[head, block].

Values are drawn in float32 with ``torch.Generator`` seeded per stream
(seed = index*1000 + stream: Q=1, K=2, V=3, structure=4, needles=5, pairs=6,
mixture=7) and then rounded once (RNE to bf16, or scaled-and-rounded to E4M3).
The same call on the same device returns the same bytes.  A CUDA generator
draws a different stream than the CPU one, so each consumer must take its bytes
from a single ``generate`` call (tests copy GPU-generated inputs to the host).

Planted structure:
  low-rank: per kv head g an orthonormal basis U_g (D x r) shared by the
      group's query heads and by K and V; per (tensor, head, token block) a
      coefficient vector a ~ N(0, I_r), constant over the block's rows; the term
      scale * U_g a is added to every row of the block.
  needles : a seeded set of key blocks (shared by all kv heads) whose every key
      row is 3 * u_g, u_g the unit mean query direction of group g.
  pairs   : per kv head, (needle, decoy) block pairs along directions w_p
      orthogonal to U_g; needle rows m*w_p, decoy rows m*w_p + delta_p with
      delta_p ~ N(0, sigma^2 I) shared by the decoy's rows; a seeded 30% of
      query blocks (each with a pair strictly earlier) get gamma*w_p added to
      every query row of the group's heads.
  mixture : per (kv head, block) a centre mu_b = N(0, I) + low-rank term; half
      the blocks (seeded) are tight (rows mu_b + 0.1 N(0, I)), the rest wide
      (rows mu_b + 1.5 N(0, I)) with one seeded row replaced by an outlier
      mu_b + 3*1.5*sqrt(D) * v, v the unit mean query of a seeded later block.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

from .configs import WorkloadConfig

E4M3_MAX = 448.0
STREAM_Q, STREAM_K, STREAM_V, STREAM_STRUCT, STREAM_NEEDLE, STREAM_PAIR, STREAM_MIX = 1, 2, 3, 4, 5, 6, 7


@dataclass
class Inputs:
    cfg: WorkloadConfig
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    q_scale: torch.Tensor | None = None
    k_scale: torch.Tensor | None = None
    v_scale: torch.Tensor | None = None
    meta: dict = field(default_factory=dict)

    def to(self, device) -> "Inputs":
        mv = (lambda t: None if t is None else t.to(device))
        return Inputs(self.cfg, mv(self.q), mv(self.k), mv(self.v), mv(self.q_scale),
                      mv(self.k_scale), mv(self.v_scale), self.meta)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _block_rows(S: int, B: int) -> torch.Tensor:
    """Token -> block index (the last block may be ragged)."""
    return torch.arange(S) // B


def _low_rank_term(U: torch.Tensor, nb: int, S: int, B: int, scale: float,
                   g: torch.Generator, device) -> torch.Tensor:
    """scale * U a_b for each token row t in block b (a_b constant within the block)."""
    r = U.shape[1]
    a = torch.randn(nb, r, generator=g, device=device)
    per_block = scale * (a @ U.T)  # [nb, D]
    return per_block[_block_rows(S, B).to(device)]  # [S, D]


def _orthonormal(D: int, r: int, g: torch.Generator, device) -> torch.Tensor:
    m = torch.randn(D, r, generator=g, device=device, dtype=torch.float64)
    qm, _ = torch.linalg.qr(m.cpu())
    return qm.to(device=device, dtype=torch.float32)


def quantize_e4m3(x: torch.Tensor, B: int):
    """Per-block E4M3 quantisation of one head's rows x [S, D] (float32).

    scale[b] = amax(block b) / 448 (1.0 for an all-zero block); the code is
    x / scale rounded to nearest-even, clamped to +-448.  Returns (codes uint8
    [S, D], scales float32 [nb]).
    """
    S, D = x.shape
    nb = -(-S // B)
    pad = nb * B - S
    xp = torch.nn.functional.pad(x, (0, 0, 0, pad)) if pad else x
    amax = xp.view(nb, B, D).abs().amax(dim=(1, 2))
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax)).to(torch.float32)
    y = (x / scale[_block_rows(S, B).to(x.device)][:, None]).clamp(-E4M3_MAX, E4M3_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale


def _store(dst: torch.Tensor, h: int, rows: torch.Tensor, dtype: str, B: int, scales):
    if dtype == "bf16":
        dst[:, h, :] = rows.to(torch.bfloat16)
    else:
        codes, sc = quantize_e4m3(rows, B)
        dst[:, h, :] = codes
        scales[h] = sc


def _rounded(rows: torch.Tensor, dtype: str, B: int) -> torch.Tensor:
    """The value a consumer will see for rows (used to derive planted directions)."""
    if dtype == "bf16":
        return rows.to(torch.bfloat16).to(torch.float32)
    codes, sc = quantize_e4m3(rows, B)
    val = codes.view(torch.float8_e4m3fn).to(torch.float32)
    return val * sc[_block_rows(rows.shape[0], B).to(rows.device)][:, None]


@torch.no_grad()
def generate(cfg: WorkloadConfig, device="cpu") -> Inputs:
    S, Hq, Hkv, D, B = cfg.seq_len, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size
    G = Hq // Hkv
    nb = cfg.num_blocks
    dev = torch.device(device)
    seed0 = cfg.index * 1000
    gq, gk, gv = _gen(seed0 + STREAM_Q, dev), _gen(seed0 + STREAM_K, dev), _gen(seed0 + STREAM_V, dev)
    gs = _gen(seed0 + STREAM_STRUCT, dev)
    # host-side generators for small discrete choices (positions), device independent
    gn = _gen(seed0 + STREAM_NEEDLE, "cpu")
    gp = _gen(seed0 + STREAM_PAIR, "cpu")
    gm = _gen(seed0 + STREAM_MIX, "cpu")

    fp8 = cfg.dtype == "fp8"
    store_dtype = torch.uint8 if fp8 else torch.bfloat16
    q = torch.empty(S, Hq, D, dtype=store_dtype, device=dev)
    k = torch.empty(S, Hkv, D, dtype=store_dtype, device=dev)
    v = torch.empty(S, Hkv, D, dtype=store_dtype, device=dev)
    q_scale = torch.empty(Hq, nb, dtype=torch.float32, device=dev) if fp8 else None
    k_scale = torch.empty(Hkv, nb, dtype=torch.float32, device=dev) if fp8 else None
    v_scale = torch.empty(Hkv, nb, dtype=torch.float32, device=dev) if fp8 else None
    meta: dict = {"structure": cfg.structure}
    blk = _block_rows(S, B).to(dev)

    # seeded needle positions shared by all kv heads
    needles: list[int] = []
    if cfg.structure == "needles" and cfg.num_needles > 0:
        lo = cfg.needle_range[0]
        hi = nb + cfg.needle_range[1]
        pool = torch.arange(lo, max(hi, lo + 1))
        perm = torch.randperm(len(pool), generator=gn)[: min(cfg.num_needles, len(pool))]
        needles = sorted(int(pool[i]) for i in perm)
    meta["needle_blocks"] = needles
    meta["pairs"] = {}
    meta["planted_query_blocks"] = {}
    meta["wide_blocks"] = {}

    for g in range(Hkv):
        U = _orthonormal(D, cfg.low_rank, gs, dev) if cfg.low_rank > 0 else None
        # ---- pairs structure: directions orthogonal to the low-rank span
        pair_dirs, pair_pos, planted = [], [], {}
        if cfg.structure == "pairs":
            npairs = cfg.pairs_per_kv_head
            for _ in range(npairs):
                w = torch.randn(D, generator=gs, device=dev)
                if U is not None:
                    w = w - U @ (U.T @ w)
                pair_dirs.append(w / w.norm())
            slots = torch.randperm(max(nb - 2, 1), generator=gp)[: 2 * npairs] + 1
            for p in range(npairs):
                pair_pos.append((int(slots[2 * p]), int(slots[2 * p + 1])))
            eligible = [i for i in range(nb) if any(max(a, b_) < i for a, b_ in pair_pos)]
            nplant = min(len(eligible), int(round(cfg.planted_query_fraction * nb)))
            pick = torch.randperm(len(eligible), generator=gp)[:nplant]
            for idx in sorted(int(x) for x in pick):
                i = eligible[idx]
                cands = [p for p, (a, b_) in enumerate(pair_pos) if max(a, b_) < i]
                p = cands[int(torch.randint(len(cands), (1,), generator=gp))]
                planted[i] = p
            meta["pairs"][g] = pair_pos
            meta["planted_query_blocks"][g] = planted

        # ---- queries of the group's heads
        qsum = torch.zeros(D, dtype=torch.float64, device=dev)
        for hh in range(G):
            h = g * G + hh
            rows = torch.randn(S, D, generator=gq, device=dev)
            if U is not None:
                rows += _low_rank_term(U, nb, S, B, cfg.low_rank_scale, gq, dev)
            if planted:
                add = torch.zeros(nb, D, device=dev)
                for i, p in planted.items():
                    add[i] = cfg.pair_query_gain * pair_dirs[p]
                rows += add[blk]
            _store(q, h, rows, cfg.dtype, B, q_scale)
            qsum += _rounded(rows, cfg.dtype, B).sum(0, dtype=torch.float64)
        u = (qsum / qsum.norm()).to(torch.float32)

        # ---- keys
        if cfg.structure == "mixture":
            centre = torch.randn(nb, D, generator=gk, device=dev)
            if U is not None:
                centre += cfg.low_rank_scale * (torch.randn(nb, cfg.low_rank, generator=gk, device=dev) @ U.T)
            wide = torch.rand(nb, generator=gm) < 0.5
            sig = torch.where(wide, torch.tensor(cfg.wide_sigma), torch.tensor(cfg.tight_sigma)).to(dev)
            rows = centre[blk] + sig[blk][:, None] * torch.randn(S, D, generator=gk, device=dev)
            outliers = {}
            for b_ in range(nb):
                if not bool(wide[b_]):
                    continue
                b0, b1 = b_ * B, min(S, (b_ + 1) * B)
                t = b0 + int(torch.randint(b1 - b0, (1,), generator=gm))
                later = int(torch.randint(b_ + 1, nb, (1,), generator=gm)) if b_ + 1 < nb else b_
                hsel = g * G + int(torch.randint(G, (1,), generator=gm))
                l0, l1 = later * B, min(S, (later + 1) * B)
                qv = _decode_rows(q[l0:l1, hsel, :], q_scale, hsel, l0, B, cfg.dtype).mean(0)
                vdir = qv / qv.norm().clamp_min(1e-30)
                rows[t] = centre[b_] + 3.0 * cfg.wide_sigma * math.sqrt(D) * vdir
                outliers[b_] = (t, later, hsel)
            meta["wide_blocks"][g] = outliers
        else:
            rows = torch.randn(S, D, generator=gk, device=dev)
            if U is not None:
                rows += _low_rank_term(U, nb, S, B, cfg.low_rank_scale, gk, dev)
            for nbk in needles:
                rows[nbk * B: min(S, (nbk + 1) * B)] = 3.0 * u
            for p, (a, b_) in enumerate(pair_pos):
                w = pair_dirs[p]
                rows[a * B: min(S, (a + 1) * B)] = cfg.pair_magnitude * w
                delta = cfg.decoy_sigma * torch.randn(D, generator=gs, device=dev)
                rows[b_ * B: min(S, (b_ + 1) * B)] = cfg.pair_magnitude * w + delta
        _store(k, g, rows, cfg.dtype, B, k_scale)

        # ---- values
        rows = torch.randn(S, D, generator=gv, device=dev)
        if U is not None and cfg.structure != "mixture":
            rows += _low_rank_term(U, nb, S, B, cfg.low_rank_scale, gv, dev)
        _store(v, g, rows, cfg.dtype, B, v_scale)

    return Inputs(cfg, q, k, v, q_scale, k_scale, v_scale, meta)


def _decode_rows(codes_or_bf16, scales, h, row0, B, dtype):
    if dtype == "bf16":
        return codes_or_bf16.to(torch.float32)
    val = codes_or_bf16.view(torch.float8_e4m3fn).to(torch.float32)
    S = val.shape[0]
    blocks = (torch.arange(S, device=val.device) + row0) // B
    return val * scales[h][blocks][:, None]
