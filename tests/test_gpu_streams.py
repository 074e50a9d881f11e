"""Streams and graph capture through the C ABI.

Every entry point enqueues its kernels on the stream it is given and makes no
allocation, copy, memset or synchronisation of its own.  So a layer run on a
side stream gives the same bytes as on the default stream, and a layer captured
into a HIP graph (with the allocation-free selection, the case that entry point
serves) gives the eager bytes on every replay, with eager work in between."""

import math

import pytest
import torch

import block_sparse_attention_36_amd as bsa
from workloads import config_by_name, generate, scaled

pytestmark = pytest.mark.gpu

CASES = [scaled(config_by_name("gqa32k"), 4096 + 77, num_q_heads=8, num_kv_heads=2),
         scaled(config_by_name("dual128k"), 4096 + 100, num_q_heads=8, num_kv_heads=2),
         scaled(config_by_name("msa1m"), 4096 + 70, num_q_heads=8, num_kv_heads=2),
         scaled(config_by_name("quest64k"), 4096 + 5, num_q_heads=8, num_kv_heads=2),
         scaled(config_by_name("sigma64k"), 4096 + 33, num_q_heads=8, num_kv_heads=2,
                name="padded-sigma64k"),
         scaled(config_by_name("msa1m"), 4096 + 70, num_q_heads=8, num_kv_heads=2,
                name="prepared-msa1m"),
         scaled(config_by_name("dual128k"), 4096 + 100, num_q_heads=8, num_kv_heads=2,
                name="prepared-dual128k")]


def _gpu_or_skip():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


class Layer:
    """One layer's inputs and preallocated outputs; run() enqueues the layer's calls
    (pool or key bounds, selection in CSR or padded form, attention) on the current
    stream without allocating."""

    def __init__(self, cfg, inp, noalloc):
        import bsa_check as K
        self.cfg, self.inp, self.noalloc = cfg, inp, noalloc
        self.quest = cfg.backbone == "quest"
        self.padded = cfg.name.startswith("padded")
        self.prepared = cfg.name.startswith("prepared")
        self.problem = bsa.make_problem(inp.q, inp.k, cfg.block_size, K.granularity_code(cfg))
        self.params = K.lib_params(cfg)
        if self.quest:
            self.kb = bsa.bsa_pool_key_bounds(self.problem, inp.k, inp.k_scale)
            self.qbufs = bsa.QuestBuffers(self.problem, "cuda")
        else:
            self.pool = bsa.bsa_pool(self.problem, inp.q, inp.k, inp.q_scale, inp.k_scale)
        if self.padded:
            self.pbufs = bsa.PaddedBuffers(self.problem, self.params, "cuda")
        self.bufs = bsa.SelectBuffers(self.problem, self.params, "cuda", given_scores=self.quest)
        S, Hq, D = inp.q.shape
        self.out = torch.empty(S, Hq, D, dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty(Hq, S, dtype=torch.float32, device="cuda")
        self.v16 = (torch.empty(inp.v.shape, dtype=torch.bfloat16, device="cuda")
                    if cfg.dtype == "fp8" and not self.prepared else None)
        self.vp = bsa.bsa_prepare_v(self.problem, inp.v) if self.prepared else None

    def run(self):
        i, p = self.inp, self.problem
        scale = 1.0 / math.sqrt(self.cfg.head_dim)
        if self.quest:
            bsa.bsa_pool_key_bounds(p, i.k, i.k_scale, out=self.kb)
            sc = bsa.bsa_quest_scores(p, i.q, self.kb[0], self.kb[1], i.q_scale,
                                      buffers=self.qbufs)
            sel = bsa.bsa_select_scores(p, self.params, sc, buffers=self.bufs)
        else:
            bsa.bsa_pool(p, i.q, i.k, i.q_scale, i.k_scale, out=self.pool)
            if self.padded:
                pl = bsa.bsa_score_select_padded(p, self.params, self.pool, buffers=self.pbufs)
                bsa.bsa_attention_fwd_padded(p, i.q, i.k, i.v, pl.kv_idx, scale, i.q_scale,
                                             i.k_scale, i.v_scale, out=self.out, lse=self.lse)
                return
            select = bsa.bsa_score_select_noalloc if self.noalloc else bsa.bsa_score_select
            sel = select(p, self.params, self.pool, buffers=self.bufs)
        if self.vp is not None:
            bsa.bsa_prepare_v(p, i.v, out=self.vp)
            bsa.bsa_attention_fwd_prepared_v(p, i.q, i.k, self.vp, sel.row_ptr, sel.col_idx,
                                             scale, i.q_scale, i.k_scale, i.v_scale,
                                             out=self.out, lse=self.lse)
        elif self.v16 is not None:
            bsa.bsa_expand_e4m3(p, i.v, out=self.v16)
            bsa.bsa_attention_fwd_expanded_v(p, i.q, i.k, self.v16, sel.row_ptr, sel.col_idx,
                                             scale, i.q_scale, i.k_scale, i.v_scale,
                                             out=self.out, lse=self.lse)
        else:
            bsa.bsa_attention_fwd(p, i.q, i.k, i.v, sel.row_ptr, sel.col_idx, scale, i.q_scale,
                                  i.k_scale, i.v_scale, out=self.out, lse=self.lse)

    def snapshot(self):
        if self.padded:
            lists = (self.pbufs.kv_idx.clone(),)
        else:
            nnz = int(self.bufs.row_ptr[-1].item())
            lists = (self.bufs.row_ptr.clone(), self.bufs.col_idx[:nnz].clone())
        return lists + (self.out.view(torch.int16).clone(), self.lse.clone())

    def clear_lists(self):
        (self.pbufs.kv_idx if self.padded else self.bufs.col_idx).zero_()


def _same(a, b):
    return all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_side_stream_gives_the_same_bytes(cfg):
    _gpu_or_skip()
    print(f"[streams] side stream {cfg.name}", flush=True)
    inp = generate(cfg, "cpu").to("cuda")
    layer = Layer(cfg, inp, noalloc=False)
    layer.run()
    torch.cuda.synchronize()
    ref = layer.snapshot()
    other = Layer(cfg, inp, noalloc=False)
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        other.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert _same(ref, other.snapshot())


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_graph_replays_match_eager(cfg):
    _gpu_or_skip()
    print(f"[streams] graph {cfg.name}", flush=True)
    inp = generate(cfg, "cpu").to("cuda")
    eager = Layer(cfg, inp, noalloc=True)
    eager.run()  # first call per device: attributes and the scratch address are set up here
    torch.cuda.synchronize()
    ref = eager.snapshot()
    captured = Layer(cfg, inp, noalloc=True)
    captured.run()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured.run()
    torch.cuda.synchronize()
    for replay in range(3):
        # outputs cleared between replays, so each replay is seen to write them again
        captured.out.zero_()
        captured.lse.zero_()
        captured.clear_lists()
        graph.replay()
        torch.cuda.synchronize()
        assert _same(ref, captured.snapshot()), f"replay {replay}"
        eager.run()  # the program's own eager work between replays
        torch.cuda.synchronize()
        assert _same(ref, eager.snapshot())
