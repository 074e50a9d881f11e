"""Benchmark: one block-sparse prefill layer (pool -> score/select -> attention)
on the 128K dual-branch workload, on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dual128k]

Prints ONE JSON line.  A step is one pass of the whole hot path over the
resident inputs; ``value`` is effective TFLOP/s = algorithmic FLOPs of the kept
blocks / step time.  ``roofline`` describes the attention kernel (HIP events
around each launch on the launching stream); ``cpu_baseline`` times the CPU
oracle on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block-sparse prefill ms/layer + effective TFLOP/s at 128k (frac of MFMA peak)"
PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA, vendor figure
PEAK_FP8_TFLOPS = 5033.2   # MI355X dense fp8 MFMA, vendor figure
# E4M3 inputs: QK^T on the fp8 matrix cores, PV on the bf16 ones, half the FLOPs each,
# so each contraction is priced at its own dtype's peak
PEAK_MIXED_TFLOPS = 2.0 / (1.0 / PEAK_FP8_TFLOPS + 1.0 / PEAK_BF16_TFLOPS)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, vendor figure


def attention_flops(row_ptr, col_idx, cfg) -> float:
    """Kept algorithmic FLOPs of one attention launch: 4*D per valid (query, key)
    pair of every kept (row, block); B^2 pairs off the diagonal and B(B+1)/2 on
    it (ragged last block counted exactly); times the heads a row serves."""
    import numpy as np
    B, S, D, nb = cfg.block_size, cfg.seq_len, cfg.head_dim, cfg.num_blocks
    heads_per_row = cfg.group_size if cfg.granularity == "group" else 1
    rp = np.asarray(row_ptr, dtype=np.int64)
    ci = np.asarray(col_idx, dtype=np.int64)
    rows = np.repeat(np.arange(len(rp) - 1), np.diff(rp))
    i = rows % nb
    nq = np.minimum(B, S - i * B)                # queries in block i
    nk = np.minimum(B, S - ci * B)               # keys in block j
    diag = ci == i
    pairs = np.where(diag, nq * (nq + 1) // 2, nq * nk)
    return float(4 * D * heads_per_row * pairs.sum())


def dense_causal_flops(cfg) -> float:
    S, D, Hq = cfg.seq_len, cfg.head_dim, cfg.num_q_heads
    return 4.0 * D * Hq * S * (S + 1) / 2


def pool_select_bytes(cfg, nnz: int) -> float:
    """Algorithmic HBM bytes of pool + score/select: Q and K read once (plus E4M3
    scales), the block summaries written and read once (centroids/norms/radii, or
    the Quest key bounds), CSR written."""
    S, Hq, Hkv, D, nb, U = (cfg.seq_len, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                            cfg.num_blocks, cfg.num_units)
    es = 1 if cfg.dtype == "fp8" else 2
    b = S * (Hq + Hkv) * D * es
    if cfg.dtype == "fp8":
        b += (Hq + Hkv) * nb * 4
    if cfg.backbone == "quest":
        b += 2 * (2 * Hkv * nb * D * 4)
    else:
        b += 2 * ((U * nb * D + Hkv * nb * D) * 4 + (U * nb + Hkv * nb) * 4)
    b += 4 * (U * nb + 1) + 4 * nnz
    return float(b)


def quest_flops(cfg) -> float:
    """Algorithmic FLOPs of the Quest tile scores: per query row of every head and
    every causal key block, sum_d max(q_d kmin_d, q_d kmax_d) as 2D multiply-adds."""
    S, B, nb = cfg.seq_len, cfg.block_size, cfg.num_blocks
    rows_by_tile = sum(min(B, S - i * B) * (i + 1) for i in range(nb))
    return float(cfg.num_q_heads * rows_by_tile * 4 * cfg.head_dim)


def pool_bytes(cfg) -> float:
    """Algorithmic HBM bytes of the pool stage alone: Q and K read once (plus E4M3
    scales), centroids, norms and radii written once; on the Quest backbone K read
    once and its bounds written."""
    S, Hq, Hkv, D, nb, U = (cfg.seq_len, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                            cfg.num_blocks, cfg.num_units)
    es = 1 if cfg.dtype == "fp8" else 2
    if cfg.backbone == "quest":
        return float(S * Hkv * D * es + (Hkv * nb * 4 if cfg.dtype == "fp8" else 0)
                     + 2 * Hkv * nb * D * 4)
    b = S * (Hq + Hkv) * D * es
    if cfg.dtype == "fp8":
        b += (Hq + Hkv) * nb * 4
    b += (U * nb * D + Hkv * nb * D) * 4 + (U * nb + Hkv * nb) * 4
    return float(b)


def copy_bandwidth(torch, dev, nbytes: int = 1 << 30, reps: int = 5) -> float:
    """GB/s (read + write bytes) of a plain device-to-device copy of nbytes: the
    HBM rate this GPU reaches on a trivially coalesced stream."""
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2.0 * nbytes / (ms * 1e-3) / 1e9


def source_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "block_sparse_attention_36_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel_hash: str, workload: str):
    """HBM bytes per attention launch from the committed counter summary, if it was
    taken on the current kernel source and on this workload; else None."""
    path = os.path.join(ROOT, "profiles", "attention_dual128k_counters.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_hash or rec.get("workload") != workload:
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, inp, sel_rows, budget_s: float = 15.0):
    """Time the CPU oracle on a sample of the workload: for sampled selection rows,
    pool the query block, score it against every key block of its kv head, select,
    and run attention for the row's heads; key pooling for the touched kv heads is
    included.  Reported as oracle TFLOP/s on the same kept-FLOP definition."""
    import numpy as np
    import torch
    from oracle import bsa_oracle as O
    B, S, D, nb = cfg.block_size, cfg.seq_len, cfg.head_dim, cfg.num_blocks
    Hq, Hkv, G = cfg.num_q_heads, cfg.num_kv_heads, cfg.group_size
    gran = cfg.granularity
    p = O.SelectParams(cfg.top_k, cfg.force_sink, cfg.gate, cfg.gate_threshold, cfg.gate_factor,
                       cfg.score_temperature, cfg.mass_threshold,
                       cfg.rescue_fraction).as_library_precision()
    rng = np.random.default_rng(0)
    kv = 0
    fp8 = cfg.dtype == "fp8"
    quest = cfg.backbone == "quest"

    def host_raw(t):
        t = t.cpu()
        return t.numpy() if fp8 else t.view(torch.int16).numpy().view(np.uint16)

    def decode(raw, scale):  # raw [rows, H, D] -> float64, with [H, nb] scales for E4M3
        return O.dequantize(raw, scale, B) if fp8 else O.decode_bf16(raw)

    t_host = time.perf_counter()
    kraw = host_raw(inp.k[:, kv:kv + 1])
    vraw = host_raw(inp.v[:, kv:kv + 1])
    ks = inp.k_scale[kv:kv + 1].cpu().numpy().astype(np.float64) if fp8 else None
    vs = inp.v_scale[kv:kv + 1].cpu().numpy().astype(np.float64) if fp8 else None
    qs_all = inp.q_scale.cpu().numpy().astype(np.float64) if fp8 else None
    copy_s = time.perf_counter() - t_host
    t0 = time.perf_counter()
    K = decode(kraw, ks)
    V = decode(vraw, vs)
    if quest:
        kmin, kmax = O.key_block_bounds(K, B)
    else:
        kbar, rad = O.pool_keys(K, B)
    flops = 0.0
    units = 0
    ambiguous = 0
    heads = [h for h in range(Hq) if h // G == kv]
    c0 = time.process_time()
    while time.perf_counter() - t0 < budget_s:
        i = int(rng.integers(nb))
        h = heads[int(rng.integers(len(heads)))]
        u = h if gran == "qhead" else kv
        qh = decode(host_raw(inp.q[i * B:min(S, (i + 1) * B)]),
                    None if qs_all is None else qs_all[:, i:i + 1])
        hs = [h] if gran == "qhead" else heads
        if quest:
            rows = qh[:, hs, :].reshape(-1, D)
            s = O.quest_row_bound(rows, kmin[0, : i + 1], kmax[0, : i + 1]).max(axis=0)
            b = None
        else:
            qbar, qn = O.pool_queries(qh, B, Hkv, gran)
            s = qbar[u, 0] @ kbar[0, : i + 1].T
            b = s + qn[u, 0] * rad[0, : i + 1]
        if p.gate == "sigma_cut":
            O.sigma_cut_margin(s, O.candidate_sets(i, p.force_sink)[1], p.top_k)
        kept, _ = O.select_row(i, s, b, p)
        ambiguous += int(O.acceptable_row_sets(i, s, b, p, 1e-5)[1])
        keys = O.block_tokens(kept, B, S)
        O.attend(qh[:, h], i * B + np.arange(qh.shape[0]), K[keys, 0], V[keys, 0], keys,
                 1 / math.sqrt(D))
        nq = min(B, S - i * B)
        for j in kept:
            nk = min(B, S - j * B)
            flops += 4 * D * (nq * (nq + 1) // 2 if j == i else nq * nk)
        units += 1
    el = time.perf_counter() - t0
    cpu = time.process_time() - c0
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "kind": "oracle",
            "sample": (f"{units} random (query block, head) rows of kv head 0 at S={S}: "
                       + ("Quest row bounds vs all key blocks" if quest
                          else "pool + score vs all key blocks")
                       + " + select"
                       + (" (per-row sigma; the layer-wide tile percentile not sampled)"
                          if p.gate == "sigma_cut" else "")
                       + f" + attention, plus {'bounds' if quest else 'pooling'} of "
                       f"kv head 0's {nb} key blocks, {el:.1f} s of float64 NumPy "
                       f"(host copy {copy_s:.1f} s excluded)"),
            "seconds": round(el, 2), "rows": units,
            "ambiguous_rows": ambiguous, **_cpu_fields(el, cpu)}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_fields(wall_s: float, cpu_s: float) -> dict:
    """Core accounting of an oracle run: the process's CPU time over its wall time is
    the number of cores it kept busy on average (NumPy's BLAS calls are threaded,
    the row loop is not); the affinity set and the BLAS thread count are the
    ceiling it had."""
    try:
        from threadpoolctl import threadpool_info
        blas = max([x.get("num_threads", 1) for x in threadpool_info()] + [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        blas = None
    return {"cores": max(1, int(round(cpu_s / wall_s))) if wall_s > 0 else 1,
            "cores_busy_avg": round(cpu_s / wall_s, 2) if wall_s > 0 else None,
            "affinity_cores": len(os.sched_getaffinity(0)), "blas_threads": blas,
            "cpu_model": _cpu_model()}


def cpu_full(cfg, inp):
    """The CPU oracle over the whole workload (every pool entry, score, row and
    attention output), timed: for the workloads small enough to finish in
    minutes.  Host copies and the decoding of the stored bytes are excluded."""
    import numpy as np
    import torch
    from oracle import bsa_oracle as O
    B, D = cfg.block_size, cfg.head_dim
    Hq, Hkv, gran = cfg.num_q_heads, cfg.num_kv_heads, cfg.granularity
    p = O.SelectParams(cfg.top_k, cfg.force_sink, cfg.gate, cfg.gate_threshold, cfg.gate_factor,
                       cfg.score_temperature, cfg.mass_threshold,
                       cfg.rescue_fraction).as_library_precision()
    fp8 = cfg.dtype == "fp8"

    def host(t, sc):
        t = t.cpu()
        raw = t.numpy() if fp8 else t.view(torch.int16).numpy().view(np.uint16)
        return O.dequantize(raw, sc.cpu().numpy().astype(np.float64), B) if fp8 \
            else O.decode_bf16(raw)

    Q, K, V = host(inp.q, inp.q_scale), host(inp.k, inp.k_scale), host(inp.v, inp.v_scale)
    t0, c0 = time.perf_counter(), time.process_time()
    b = None
    if cfg.backbone == "quest":
        kmin, kmax = O.key_block_bounds(K, B)
        s = O.quest_scores(Q, kmin, kmax, B, Hkv, gran)
    else:
        qbar, qn = O.pool_queries(Q, B, Hkv, gran)
        kbar, rad = O.pool_keys(K, B)
        s = O.block_scores(qbar, kbar, Hq, Hkv, gran)
        if p.rescue_fraction > 0:
            b = O.rescue_bounds(s, qn, rad, Hq, Hkv, gran)
    kept, _ = O.select(s, b, p)
    print(f"[bench] oracle: pool, scores and selection done ({time.perf_counter() - t0:.1f} s)",
          file=sys.stderr, flush=True)
    for h in range(Hq):
        O.attention(Q, K, V, kept, B, 1 / math.sqrt(D), gran, heads=[h])
        if (h + 1) % 4 == 0 or h + 1 == Hq:
            print(f"[bench] oracle: attention of {h + 1}/{Hq} heads "
                  f"({time.perf_counter() - t0:.1f} s)", file=sys.stderr, flush=True)
    el, cpu = time.perf_counter() - t0, time.process_time() - c0
    rp, ci = O.to_csr(kept)
    flops = attention_flops(rp, ci, cfg)
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "kind": "oracle",
            "sample": f"the whole workload: {cfg.num_units * cfg.num_blocks} selection rows, "
                      f"{Hq * cfg.num_blocks} attention units, {el:.1f} s of float64 NumPy",
            "seconds": round(el, 2), **_cpu_fields(el, cpu)}


def realized_stats(cfg, meta, rp, ci, gate):
    """What the synthetic structure did under the selection (reported, never
    tuned): recall of the planted needle blocks, of the planted pairs and of the
    wide blocks' outlier keys, and the gate's firing rate on rows with a planted
    near tie against the other rows."""
    import numpy as np
    nb, U, G = cfg.num_blocks, cfg.num_units, cfg.group_size
    kept = {}

    def row(u, i):
        r = u * nb + i
        if r not in kept:
            kept[r] = set(int(x) for x in ci[rp[r]:rp[r + 1]])
        return kept[r]

    kv_of = (lambda u: u // G) if cfg.granularity == "qhead" else (lambda u: u)
    out = {}
    needles = meta.get("needle_blocks") or []
    if needles:
        hit = tot = 0
        for u in range(U):
            for i in range(nb):
                elig = [n for n in needles if n < i and not (cfg.force_sink and n == 0)]
                if elig:
                    r = row(u, i)
                    hit += sum(n in r for n in elig)
                    tot += len(elig)
        out["needle_recall"] = round(hit / tot, 4) if tot else None
        out["needle_pairs"] = tot
    planted = meta.get("planted_query_blocks") or {}
    pairs = meta.get("pairs") or {}
    if planted:
        both = needle = tot = 0
        fire_p = n_p = fire_b = n_b = 0
        for u in range(U):
            g = kv_of(u)
            pl = planted.get(g, {})
            for i in range(nb):
                if i in pl:
                    a, b_ = pairs[g][pl[i]]
                    r = row(u, i)
                    needle += a in r
                    both += (a in r) and (b_ in r)
                    tot += 1
                if gate is not None:
                    f = bool(gate[u * nb + i])
                    if i in pl:
                        fire_p += f
                        n_p += 1
                    else:
                        fire_b += f
                        n_b += 1
        out["planted_rows"] = tot
        out["planted_needle_recall"] = round(needle / tot, 4) if tot else None
        out["planted_pair_recall"] = round(both / tot, 4) if tot else None
        if gate is not None and cfg.gate != "none":
            out["gate_fire_rate_planted"] = round(fire_p / n_p, 4) if n_p else None
            out["gate_fire_rate_background"] = round(fire_b / n_b, 4) if n_b else None
    wide = meta.get("wide_blocks") or {}
    if wide:
        hit = tot = 0
        for g, outl in wide.items():
            for b_, (_, later, hsel) in outl.items():
                if later <= b_:
                    continue
                u = hsel if cfg.granularity == "qhead" else g
                hit += b_ in row(u, later)
                tot += 1
        out["outlier_block_recall"] = round(hit / tot, 4) if tot else None
        out["outlier_rows"] = tot
    if gate is not None:
        out["gate_fire_rate"] = round(float(np.mean(gate)), 4)
    return out


COPY_BYTES = 1 << 30


def _pmc_rows(d: str, counter: str):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r.get("Counter_Name") == counter:
                rows.append(r)
    return rows


ATTN_KERNEL = "attn_whole_kernel"


# How the counter record is made (run from /tmp with TMPDIR=/tmp; $R is the repository,
# $OUT the folder the profiler writes to).
PMC_COMMANDS = [
    "rocprofv3 --pmc {c} --kernel-include-regex \"attn_|pool_|select_|score_|copy|scan_|compact_|run_sum_\" "
    "--output-format csv -d $OUT/pmc_{d} -o run -- python3 $R/bench.py --steps 1 --warmup 1 "
    "--no-cpu-baseline --calibrate-copy".format(c=c, d=d)
    for c, d in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write"))
] + ["python3 $R/bench.py --summarize-pmc $OUT/pmc_fetch $OUT/pmc_write "
     "$R/profiles/attention_dual128k_counters.json"]


def summarize_pmc(fetch_dir: str, write_dir: str, out_json: str) -> int:
    """HBM bytes per attention launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
    each scaled by what the same counter reads for a plain copy of COPY_BYTES."""
    import statistics
    out = {"kernel": "attn_whole_kernel<128, 128, false, false, false>", "workload": "dual128k",
           "kernel_source_hash": source_hash("attention.hip", "common.h"),
           "commands": PMC_COMMANDS}
    others = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _pmc_rows(d, counter)
        att = [float(r["Counter_Value"]) * 1024 for r in rows if ATTN_KERNEL in r["Kernel_Name"]]
        cp = [float(r["Counter_Value"]) * 1024 for r in rows
              if "copy" in r["Kernel_Name"].lower() and float(r["Counter_Value"]) * 1024 > COPY_BYTES / 2]
        if not att or not cp:
            print(f"missing {counter} rows (attention {len(att)}, copy {len(cp)})", file=sys.stderr)
            return 1
        factor = statistics.mean(cp) / COPY_BYTES
        out[counter.lower()] = {"raw_bytes_per_launch": statistics.mean(att),
                                "copy_raw_bytes": statistics.mean(cp), "copy_bytes": COPY_BYTES,
                                "scale": factor,
                                "bytes_per_launch": statistics.mean(att) / factor}
        # the pool and selection kernels of the same run, per launch, calibrated alike
        for r in rows:
            name = r["Kernel_Name"]
            short = next((k for k in ("pool_q_kernel", "pool_k_kernel", "score_kernel",
                                      "select_reg_kernel", "select_kernel", "run_sum_kernel",
                                      "scan_kernel", "compact_kernel") if k in name), None)
            if short:
                others.setdefault(short, {}).setdefault(counter.lower(), []).append(
                    float(r["Counter_Value"]) * 1024 / factor)
    out["hbm_bytes_per_launch"] = (out["fetch_size"]["bytes_per_launch"] +
                                   out["write_size"]["bytes_per_launch"])
    out["pool_select_kernels_bytes_per_launch"] = {
        k: {c: round(statistics.mean(v)) for c, v in d.items()} for k, d in others.items()}
    with open(out_json, "w") as f:
        json.dump(out, f, indent=2)
    print(json.dumps(out))
    return 0


def dense_context(bsa, torch, problem, cfg, inp, scale, out, lse, attn_ms: float,
                  step_ms: float, v16=None, vprep=None) -> dict:
    """The same attention kernel on the full causal mask of the same problem (every
    row keeps blocks 0..i): the dense prefill the sparse step stands against (for
    E4M3 inputs on the same expanded or prepared V as the step, when it uses one).
    Context, not a target; run after the timed steps, so nothing here is timed in them."""
    dev = out.device
    nb, U = cfg.num_blocks, cfg.num_units
    counts = (torch.arange(nb, device=dev, dtype=torch.int64) + 1).repeat(U)
    rp = torch.zeros(U * nb + 1, dtype=torch.int64, device=dev)
    rp[1:] = torch.cumsum(counts, 0)
    row_of = torch.repeat_interleave(torch.arange(U * nb, device=dev), counts)
    ci = (torch.arange(int(rp[-1]), device=dev, dtype=torch.int64) - rp[:-1][row_of]).to(torch.int32)
    rp = rp.to(torch.int32)
    del row_of
    if vprep is not None:
        run = lambda: bsa.bsa_attention_fwd_prepared_v(problem, inp.q, inp.k, vprep, rp, ci, scale,
                                                       inp.q_scale, inp.k_scale, inp.v_scale,
                                                       out=out, lse=lse)
    elif v16 is not None:
        run = lambda: bsa.bsa_attention_fwd_expanded_v(problem, inp.q, inp.k, v16, rp, ci, scale,
                                                       inp.q_scale, inp.k_scale, inp.v_scale,
                                                       out=out, lse=lse)
    else:
        run = lambda: bsa.bsa_attention_fwd(problem, inp.q, inp.k, inp.v, rp, ci, scale,
                                            inp.q_scale, inp.k_scale, inp.v_scale, out=out,
                                            lse=lse)
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(2):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 2
    flops = dense_causal_flops(cfg)
    return {"dense_attention_ms": round(ms, 3),
            "dense_attention_tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "dense_attention_frac_bf16_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "speedup_sparse_attention": round(ms / attn_ms, 2),
            "speedup_sparse_step": round(ms / step_ms, 2)}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="dual128k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--index-format", choices=("csr", "padded"), default="csr",
                    help="kept-block lists as CSR, or as the uniform sentinel-padded list")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--cpu-full", action="store_true",
                    help="time the CPU oracle on the whole workload instead of a sample "
                         "(minutes for tiny, gqa32k and gated64k; not for the larger ones)")
    ap.add_argument("--dense-context", action="store_true",
                    help="after timing, run the same attention kernel on the full causal mask "
                         "(dense prefill, context: speedup of the sparse step over it)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after timing, run one plain device copy of 1 GiB (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT_JSON"),
                    help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) into HBM bytes "
                         "per attention launch, calibrated on the 1 GiB copy; no GPU needed")
    args = ap.parse_args(argv)
    if args.summarize_pmc:
        return summarize_pmc(*args.summarize_pmc)
    if args.dense_context and args.calibrate_copy:
        print("--dense-context adds attention launches that --calibrate-copy counter runs "
              "would average in; use one or the other", file=sys.stderr)
        return 2
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}): the block-sparse "
              "prefill path here has no multi-GPU mode.", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import block_sparse_attention_36_amd as bsa
    from workloads import config_by_name, generate

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    bsa.load_library()
    cfg = config_by_name(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {cfg.name} S={cfg.seq_len} Hq={cfg.num_q_heads} "
          f"Hkv={cfg.num_kv_heads} on the GPU", file=sys.stderr, flush=True)
    inp = generate(cfg, dev)
    torch.cuda.synchronize()

    gran = bsa.BSA_SEL_PER_GROUP if cfg.granularity == "group" else bsa.BSA_SEL_PER_QHEAD
    problem = bsa.make_problem(inp.q, inp.k, cfg.block_size, gran)
    params = bsa.make_params(cfg.top_k, cfg.force_sink,
                             bsa.GATE_CODES[cfg.gate],
                             cfg.gate_threshold, cfg.gate_factor, cfg.score_temperature,
                             cfg.mass_threshold, cfg.rescue_fraction)
    rescue = cfg.rescue_fraction > 0
    quest = cfg.backbone == "quest"
    if quest:
        kb = bsa.bsa_pool_key_bounds(problem, inp.k, inp.k_scale)
        qbufs = bsa.QuestBuffers(problem, dev)
    else:
        pool = bsa.bsa_pool(problem, inp.q, inp.k, inp.q_scale, inp.k_scale, want_norm=rescue,
                            want_radius=rescue)
    padded = args.index_format == "padded"
    if padded:
        pbufs = bsa.PaddedBuffers(problem, params, dev, export=False, given_scores=quest)
    else:
        bufs = bsa.SelectBuffers(problem, params, dev, export=False, given_scores=quest)
    # E4M3 V is expanded to its exact bf16 values inside each step (a lossless change
    # of format), and attention reads those; the padded-list path reads the codes
    # (at head_dim = block_size = 128 into the transposed tiles the P V products read
    # with one 16-byte LDS read per operand, bsa_prepare_v)
    expand = cfg.dtype == "fp8" and not padded
    prepared = expand and cfg.head_dim == 128 and cfg.block_size == 128
    v16 = (torch.empty(inp.v.shape, dtype=torch.bfloat16, device=dev)
           if expand and not prepared else None)
    vprep = bsa.bsa_prepare_v(problem, inp.v) if prepared else None
    out = torch.empty(cfg.seq_len, cfg.num_q_heads, cfg.head_dim, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(cfg.num_q_heads, cfg.seq_len, dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(cfg.head_dim)

    sc_last = [None]

    def step(ev=None):
        if ev:
            ev[0].record()
        if quest:
            bsa.bsa_pool_key_bounds(problem, inp.k, inp.k_scale, out=kb)
        else:
            bsa.bsa_pool(problem, inp.q, inp.k, inp.q_scale, inp.k_scale, out=pool)
        if ev:
            ev[1].record()
        sc = None
        if quest:
            sc = bsa.bsa_quest_scores(problem, inp.q, kb[0], kb[1], inp.q_scale, buffers=qbufs)
            sc_last[0] = sc
            if ev:
                ev[4].record()
        if padded:
            bsa.bsa_score_select_padded(problem, params, pool=None if quest else pool, scores=sc,
                                        buffers=pbufs)
        elif quest:
            sel = bsa.bsa_select_scores(problem, params, sc, buffers=bufs)
        else:
            sel = bsa.bsa_score_select(problem, params, pool, buffers=bufs)
        if ev:
            ev[2].record()
        if prepared:
            bsa.bsa_prepare_v(problem, inp.v, out=vprep)
        elif expand:
            bsa.bsa_expand_e4m3(problem, inp.v, out=v16)
        if ev:
            ev[5].record()
        if padded:
            bsa.bsa_attention_fwd_padded(problem, inp.q, inp.k, inp.v, pbufs.kv_idx, scale,
                                         inp.q_scale, inp.k_scale, inp.v_scale, out=out, lse=lse)
        elif prepared:
            bsa.bsa_attention_fwd_prepared_v(problem, inp.q, inp.k, vprep, sel.row_ptr,
                                             sel.col_idx, scale, inp.q_scale, inp.k_scale,
                                             inp.v_scale, out=out, lse=lse)
        elif expand:
            bsa.bsa_attention_fwd_expanded_v(problem, inp.q, inp.k, v16, sel.row_ptr, sel.col_idx,
                                             scale, inp.q_scale, inp.k_scale, inp.v_scale,
                                             out=out, lse=lse)
        else:
            bsa.bsa_attention_fwd(problem, inp.q, inp.k, inp.v, sel.row_ptr, sel.col_idx, scale,
                                  inp.q_scale, inp.k_scale, inp.v_scale, out=out, lse=lse)
        if ev:
            ev[3].record()

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if padded:  # the kept lists of the timed steps (deterministic), as CSR for counting
        pad = pbufs.kv_idx.cpu().numpy()
        counts = (pad >= 0).sum(axis=1)
        rp = np.concatenate([[0], np.cumsum(counts)])
        ci = pad[pad >= 0]
    else:
        rp = bufs.row_ptr.cpu().numpy()  # the CSR of the timed steps (deterministic)
        ci = bufs.col_idx[:int(rp[-1])].cpu().numpy()
    nnz = int(rp[-1])
    kept_flops = attention_flops(rp, ci, cfg)
    pool_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    sel_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    exp_ms = np.array([e[2].elapsed_time(e[5]) for e in evs])
    att_ms = np.array([e[5].elapsed_time(e[3]) for e in evs])
    ms_per_step = wall * 1e3 / args.steps
    attn_avg = float(att_ms.mean())
    achieved = kept_flops / (attn_avg * 1e-3) / 1e12
    ps_bytes = pool_select_bytes(cfg, nnz)
    ps_ms = float(pool_ms.mean() + sel_ms.mean())
    khash = source_hash("attention.hip", "common.h")
    dense = dense_causal_flops(cfg)
    causal_blocks = cfg.num_units * cfg.num_blocks * (cfg.num_blocks + 1) / 2
    if cfg.dtype == "fp8":
        peak = PEAK_MIXED_TFLOPS
        peak_basis = ("QK^T at the dense fp8 peak (5033.2) and PV at the dense bf16 peak "
                      "(2516.6), half the FLOPs each")
    else:
        peak, peak_basis = PEAK_BF16_TFLOPS, "dense bf16 MFMA peak"
    res = {
        "metric": METRIC,
        "value": round(kept_flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "fp8-e4m3 (QK on fp8 MFMA, PV on bf16 MFMA)",
        "data": "synthetic (seeded generator, random structure; no model weights)",
        "config": {"workload": cfg.name, "seq_len": cfg.seq_len, "num_q_heads": cfg.num_q_heads,
                   "num_kv_heads": cfg.num_kv_heads, "head_dim": cfg.head_dim,
                   "block_size": cfg.block_size, "selection": {
                       "top_k": cfg.top_k, "force_sink": cfg.force_sink, "gate": cfg.gate,
                       "mass_threshold": cfg.mass_threshold,
                       "rescue_fraction": cfg.rescue_fraction}},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak, 1),
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "peak_basis": peak_basis,
                     "frac_of_bf16_peak": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_from_profile(khash, cfg.name),
                     "kernel": f"{ATTN_KERNEL}<{cfg.head_dim},{cfg.block_size},"
                               f"{str(cfg.dtype == 'fp8').lower()},{str(expand).lower()},"
                               f"{str(prepared).lower()}>",
                     "kernel_source_hash": khash},
        "stages_ms": {"pool": round(float(pool_ms.mean()), 4),
                      "score_select": round(float(sel_ms.mean()), 4),
                      **({"prepare_v" if prepared else "expand_v": round(float(exp_ms.mean()), 4)}
                         if expand else {}),
                      "attention": round(attn_avg, 4)},
        "frac_of_bf16_peak_whole_step": round(kept_flops / (ms_per_step * 1e-3) / 1e12
                                              / PEAK_BF16_TFLOPS, 4),
        "kept_tflop": round(kept_flops / 1e12, 4),
        "density": round(nnz / causal_blocks, 5),
        "dense_causal_tflop": round(dense / 1e12, 3),
        "backbone": cfg.backbone,
        "index_format": args.index_format,
        "pool_select": {"algorithmic_gb": round(ps_bytes / 1e9, 4),
                        "gbs": round(ps_bytes / (ps_ms * 1e-3) / 1e9, 1),
                        "frac_hbm": round(ps_bytes / (ps_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
    }
    if quest:
        qs_ms = float(np.mean([e[1].elapsed_time(e[4]) for e in evs]))
        qf = quest_flops(cfg)
        res["quest_scores"] = {"ms": round(qs_ms, 4), "tflop": round(qf / 1e12, 4),
                               "tflops": round(qf / (qs_ms * 1e-3) / 1e12, 2),
                               "frac_bf16_peak": round(qf / (qs_ms * 1e-3) / 1e12
                                                       / PEAK_BF16_TFLOPS, 4)}
    copy_gbs = copy_bandwidth(torch, dev)
    pb = pool_bytes(cfg)
    res["pool_select"]["copy_gbs"] = round(copy_gbs, 1)
    res["pool_select"]["frac_copy"] = round(ps_bytes / (ps_ms * 1e-3) / 1e9 / copy_gbs, 4)
    res["pool_select"]["pool_only"] = {
        "gb": round(pb / 1e9, 4), "gbs": round(pb / (float(pool_ms.mean()) * 1e-3) / 1e9, 1),
        "frac_hbm": round(pb / (float(pool_ms.mean()) * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "frac_copy": round(pb / (float(pool_ms.mean()) * 1e-3) / 1e9 / copy_gbs, 4)}
    gate = None
    if cfg.gate != "none" and not padded:
        if quest:
            xs = bsa.bsa_select_scores(problem, params, sc_last[0], export=True)
        else:
            xs = bsa.bsa_score_select(problem, params, pool, export=True)
        torch.cuda.synchronize()
        gate = xs.gate.cpu().numpy()
        del xs
        torch.cuda.empty_cache()
    res["realized"] = realized_stats(cfg, inp.meta, rp, ci, gate)
    res["realized"]["density"] = res["density"]
    if args.calibrate_copy:
        src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.dense_context:
        print("[bench] dense causal attention (context)", file=sys.stderr, flush=True)
        res["dense_context"] = dense_context(bsa, torch, problem, cfg, inp, scale, out, lse,
                                             attn_avg, ms_per_step, v16, vprep)
    if args.cpu_full:
        print("[bench] cpu baseline (oracle, whole workload)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_full(cfg, inp)
    elif not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(cfg, inp, None, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res))
    return 0


if __name__ == "__main__":
    sys.exit(main())
