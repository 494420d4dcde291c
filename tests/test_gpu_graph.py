"""HIP graph capture and replay of whole cycles ([KAP] shape stabilization:
fixed shapes, tables and metadata so that proposal and verification replay as
graphs).

Every entry point enqueues on the caller's stream with no host sync, memset or
allocation, so a cycle can be captured once and replayed.  Each replay gets
new query data in the captured input buffers, runs with eager library work and
synchronizations in between, and must equal the same cycle run eagerly, bit
for bit (the kernels are deterministic).
"""
import numpy as np
import pytest
import torch

import block_sparse_paged_page_amd as kap
import oracle
import workloads as W
from _gpu_util import Case, t

pytestmark = pytest.mark.gpu


class Cycle:
    """Route -> compact -> selected decode -> verify into preallocated buffers."""

    def __init__(self, c):
        w = c.w
        self.c = c
        dev = c.q.device
        cap = c.budget()
        self.cap = cap
        self.q = c.q.clone()
        self.qv = c.qv.clone()
        self.scores = torch.empty((w.B, w.Hkv, c.max_pages), dtype=torch.float32, device=dev)
        self.sel = torch.empty((w.B, 1, cap), dtype=torch.int32, device=dev)
        self.cnt = torch.empty((w.B, 1), dtype=torch.int32, device=dev)
        self.cv = (torch.empty((w.B, 1, cap), dtype=torch.int32, device=dev),
                   torch.empty((w.B, 1, cap), dtype=torch.int32, device=dev),
                   torch.empty((w.B, 1), dtype=torch.int32, device=dev),
                   torch.empty((w.B, 1), dtype=torch.int64, device=dev))
        self.ws = torch.empty(kap.attn_workspace_bytes(w.B, w.q_len, w.Hq, w.Hkv, w.D),
                              dtype=torch.uint8, device=dev)
        self.out = torch.empty_like(c.q)
        self.lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=dev)
        self.vout = torch.empty_like(c.qv)
        self.vlse = torch.empty((w.B, w.q_len, w.Hq), dtype=torch.float32, device=dev)

    def run(self):
        c, w = self.c, self.c.w
        kap.score_blocks(self.q, c.pos, c.S, c.bt, c.L, w.Hkv, scores=self.scores)
        kap.select_topk(self.scores, c.L, c.anchor, c.recent, c.k_mid, self.cap, self.cap,
                        sel=self.sel, cnt=self.cnt)
        kap.compact_view(self.sel, self.cnt, c.bt, c.L, c.pos, 1, out=self.cv)
        kap.decode_attn(self.q, c.pos, c.K, c.V, self.cv[0], self.cv[2], out=self.out,
                        lse=self.lse, workspace=self.ws, logical=self.cv[1])
        kap.verify_attn(self.qv, c.pos, c.K, c.V, c.bt, c.L, out=self.vout, lse=self.vlse,
                        workspace=self.ws)

    def results(self):
        return [x.clone() for x in (self.scores, self.sel, self.cnt, *self.cv, self.out, self.lse,
                                    self.vout, self.vlse)]


def _other_queries(c, seed):
    """Fresh bf16 query bit patterns of the same shapes (new draws, not GPU output)."""
    rng = np.random.default_rng(seed)
    q = oracle.round_to_bf16(rng.standard_normal(c.b["q"].shape))
    qv = oracle.round_to_bf16(rng.standard_normal(c.b["qv"].shape))
    return t(q), t(qv)


def test_cycle_replays_from_a_graph():
    c = Case(W.spec("llama8b_32k", B=3, seq_lens=[4096, 3007, 1234]), aim_needles=True)
    graph_cycle = Cycle(c)
    eager_cycle = Cycle(c)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm up on a side stream before capture
        graph_cycle.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graph_cycle.run()
    torch.cuda.synchronize()
    inputs = [(c.q, c.qv)] + [_other_queries(c, 100 + k) for k in range(3)] + [(c.q, c.qv)]
    first = None
    for rep, (q, qv) in enumerate(inputs):
        graph_cycle.q.copy_(q)
        graph_cycle.qv.copy_(qv)
        g.replay()
        torch.cuda.synchronize()
        got = graph_cycle.results()
        eager_cycle.q.copy_(q)
        eager_cycle.qv.copy_(qv)
        eager_cycle.run()                  # eager library work between replays
        torch.cuda.synchronize()
        want = eager_cycle.results()
        for i, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a, b), f"replay {rep}, output {i}"
        if rep == 0:
            first = got
        elif rep < len(inputs) - 1:
            # the replay followed the new queries (scores and outputs changed)
            assert not torch.equal(got[0], first[0]) and not torch.equal(got[7], first[7])
        else:
            assert all(torch.equal(a, b) for a, b in zip(got, first))


def test_commit_cycle_replays_from_a_graph():
    """Append of the window's K/V, summary update and causal verify, captured once.
    The append rewrites the same slots with the same rows, so every replay must
    reproduce the eager result exactly."""
    w = W.spec("qwen32b_128k", B=2, seq_lens=[16384, 9999], q_len=5)
    c = Case(w)
    kn, vn = W.draft_kv(w)
    kn, vn = t(kn), t(vn)
    L2 = t((c.b["seq_lens"] + w.q_len).astype(np.int32))
    sel = t(np.full((w.B, 1, 1), -1, np.int32))
    cnt = t(np.zeros((w.B, 1), np.int32))
    dev = c.q.device

    def buffers():
        return dict(K=c.K.clone(), V=c.V.clone(), S=c.S.clone(),
                    cv=(torch.empty((w.B, 1, 1), dtype=torch.int32, device=dev),
                        torch.empty((w.B, 1, 1), dtype=torch.int32, device=dev),
                        torch.empty((w.B, 1), dtype=torch.int32, device=dev),
                        torch.empty((w.B, w.q_len), dtype=torch.int64, device=dev)),
                    ws=torch.empty(kap.attn_workspace_bytes(w.B, w.q_len, w.Hq, w.Hkv, w.D),
                                   dtype=torch.uint8, device=dev),
                    out=torch.empty_like(c.qv),
                    lse=torch.empty((w.B, w.q_len, w.Hq), dtype=torch.float32, device=dev))

    def run(x):
        kap.compact_view(sel, cnt, c.bt, c.L, c.pos, w.q_len, out=x["cv"])
        kap.append_kv(kn, vn, x["cv"][3], x["K"], x["V"])
        kap.update_summary(x["K"], c.bt, L2, c.pos, w.q_len, x["S"])
        kap.verify_attn(c.qv, c.pos, x["K"], x["V"], c.bt, L2, out=x["out"], lse=x["lse"],
                        workspace=x["ws"])

    gx, ex = buffers(), buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(gx)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(gx)
    run(ex)
    torch.cuda.synchronize()
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        for key in ("K", "V", "S", "out", "lse"):
            assert torch.equal(gx[key], ex[key]), f"replay {rep}, {key}"
        assert torch.equal(gx["cv"][3], ex["cv"][3])
        run(ex)                            # eager work between replays
        torch.cuda.synchronize()


def test_early_route_side_flow_replays_from_a_graph():
    """The early-routing side flow as the 32-layer line replays it: proxy query
    over the packed W_q, per-head scores, per-head top-8 with the compact view,
    and the decode over those views.  Each replay gets a new hidden state in the
    captured buffer and must equal the eager flow bit for bit."""
    w = W.spec("early_route_40k", B=2, seq_lens=[9000, 6123])
    c = Case(w)
    dev = c.q.device
    Hq, Hkv, D, cap = w.Hq, w.Hkv, w.D, 8
    wq = t(c.b["wq"])
    wp = kap.proxy_pack_weights(wq)
    n_out = Hq * D

    def buffers():
        return dict(hid=t(c.b["hidden"]).clone(),
                    qp=torch.empty((w.B, n_out), dtype=torch.float32, device=dev),
                    scores=torch.empty((w.B, Hkv, c.max_pages), dtype=torch.float32, device=dev),
                    cnt=torch.empty((w.B, Hkv), dtype=torch.int32, device=dev),
                    cv=(torch.empty((w.B, Hkv, cap), dtype=torch.int32, device=dev),
                        torch.empty((w.B, Hkv, cap), dtype=torch.int32, device=dev),
                        torch.empty((w.B, Hkv), dtype=torch.int32, device=dev),
                        torch.empty((w.B, 1), dtype=torch.int64, device=dev)),
                    ws=torch.empty(kap.attn_workspace_bytes(w.B, 1, Hq, Hkv, D), dtype=torch.uint8,
                                   device=dev),
                    out=torch.empty_like(c.q))

    def run(x):
        kap.proxy_query_packed(x["hid"], wp, n_out, q_out=x["qp"])
        kap.score_blocks(x["qp"].view(w.B, Hq, D), c.pos, c.S, c.bt, c.L, Hkv, scores=x["scores"])
        kap.select_compact(x["scores"], c.L, c.anchor, c.recent, c.k_mid, cap, cap, c.bt, c.pos, 1,
                           per_head=True, cnt=x["cnt"], out=x["cv"])
        kap.decode_attn(c.q, c.pos, c.K, c.V, x["cv"][0], x["cv"][2], G=Hkv, out=x["out"],
                        workspace=x["ws"], logical=x["cv"][1])

    gx, ex = buffers(), buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(gx)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(gx)
    torch.cuda.synchronize()
    rng = np.random.default_rng(77)
    first = None
    for rep in range(4):
        hid = t(oracle.round_to_bf16(rng.standard_normal(c.b["hidden"].shape))) if rep % 3 else t(c.b["hidden"])
        gx["hid"].copy_(hid)
        g.replay()
        torch.cuda.synchronize()
        ex["hid"].copy_(hid)
        run(ex)                            # eager library work between replays
        torch.cuda.synchronize()
        for key in ("qp", "scores", "cnt", "out"):
            assert torch.equal(gx[key], ex[key]), f"replay {rep}, {key}"
        for i in range(3):
            assert torch.equal(gx["cv"][i], ex["cv"][i]), f"replay {rep}, view {i}"
        if rep == 0:
            first = gx["qp"].clone()
        elif rep % 3:
            assert not torch.equal(gx["qp"], first)  # the replay followed the new hidden state
        else:
            assert torch.equal(gx["qp"], first)
