"""Seeded random small layers for the parity tests (GPU against the oracle, and the
checker against oracle-built results on the CPU)."""

import numpy as np

from workloads import config_by_name, scaled


def random_layers(n, seed=4242):
    """Seeded random small layers: ragged lengths, head counts, head and block sizes,
    input formats, list granularity, backbone and every selection branch mixed (the
    structure of the named workload plants the needles, pairs or mixture)."""
    rng = np.random.default_rng(seed)
    bases = ["tiny", "gqa32k", "gated64k", "dual128k", "msa1m", "sigma64k", "quest64k"]
    out = []
    for c in range(n):
        base = bases[rng.integers(len(bases))]
        d, b = (64, 128)[rng.integers(2)], (64, 128)[rng.integers(2)]
        hkv, g = (1, 2)[rng.integers(2)], (1, 2, 4)[rng.integers(3)]
        top_k = int((0, 1, 3, 8)[rng.integers(4)])
        mass = float((0.0, 0.0, 0.5, 0.9)[rng.integers(4)])
        rescue = float((0.0, 0.0, 0.05, 0.2)[rng.integers(3 + (top_k == 0 and mass == 0.0))])
        gate = "none" if top_k == 0 else ("none", "top12_gap", "sigma_cut")[rng.integers(3)]
        if gate == "sigma_cut":
            # the layer-wide percentile of the tiles' cut margins is decided only where the
            # margins do not tie: on the planted near-tie structure, and never at k = 1
            # (there the margin is 1 on every row)
            base = ("gated64k", "sigma64k", "quest64k")[rng.integers(3)]
            top_k = max(top_k, 3)
        if base == "quest64k":
            rescue = 0.0  # the radius bound belongs to the centroid scores, not to Quest's
        kw = dict(head_dim=d, block_size=b, dtype=("bf16", "fp8")[rng.integers(2)],
                  granularity=("qhead", "group")[rng.integers(2)], top_k=top_k,
                  force_sink=bool(rng.integers(2)), gate=gate,
                  gate_threshold=0.05 if gate == "top12_gap" else 0.3,
                  gate_factor=int((2, 3)[rng.integers(2)]), mass_threshold=mass,
                  rescue_fraction=rescue, name=f"random{c}-{base}")
        seq = int(rng.integers(5 * b + 1, (24 if c % 2 == 0 else 96) * b))  # odd: past 64 slots
        out.append(scaled(config_by_name(base), seq, num_q_heads=hkv * g, num_kv_heads=hkv, **kw))
    return out
