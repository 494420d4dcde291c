"""CPU-offloaded routing feeding the GPU: pages picked on the host (proxy query,
scores over a host copy of the K summaries, per-head top-8), uploaded as
indices, then compacted and decoded on the GPU; compared with the oracle's
decode over the oracle's own picks (EarlySelectKV news item, Interpretation)."""
import numpy as np
import pytest
import torch

import block_sparse_paged_page_amd as kap
import oracle
import workloads as W
from _gpu_util import TOL, Case, host, row_errors, t

pytestmark = pytest.mark.gpu


def test_host_routed_decode_matches_oracle():
    w = W.spec("early_route_40k", B=2, seq_lens=[40000, 23456])
    c = Case(w)
    b = c.b
    # host side flow over the host summary copy (local page order, local table)
    qp = kap.host_proxy_query(b["hidden"], b["wq"]).reshape(w.B, w.Hq, w.D)
    scores = kap.host_score_blocks(qp, b["positions"], c.summ_l, c.btl, b["seq_lens"], w.Hkv)
    cap = int((b["anchor"] + b["recent"] + b["k_mid"]).max())
    sel, cnt = kap.host_select_topk(scores, b["seq_lens"], b["anchor"], b["recent"], b["k_mid"],
                                    cap, per_head=True)
    # oracle chain on its own proxy query
    qref = oracle.proxy_query(b["hidden"], b["wq"]).astype(np.float32).reshape(w.B, w.Hq, w.D)
    s_ref = oracle.score(qref, b["positions"], c.summ_l, c.btl, b["seq_lens"], w.Hkv)
    sel_ref, cnt_ref = oracle.select(s_ref.astype(np.float32), b["seq_lens"], b["anchor"],
                                     b["recent"], b["k_mid"], cap, per_head=True)
    np.testing.assert_array_equal(sel, sel_ref)       # no near-ties in this seeded case
    np.testing.assert_array_equal(cnt, cnt_ref)
    # upload the indices; the GPU compacts and decodes with the real query
    cbt, clog, clen, _ = kap.compact_view(t(sel), t(cnt), c.bt, c.L, c.pos, 1)
    out = kap.decode_attn(c.q, c.pos, c.K, c.V, cbt, clen, G=w.Hkv, logical=clog)
    torch.cuda.synchronize()
    keys = oracle.keys_selected(sel_ref, cnt_ref, b["seq_lens"])
    ref, _ = oracle.attend(b["q"][:, None], b["positions"], c.Kl, c.Vl, c.btl, keys, w.Hkv, w.Hkv)
    assert row_errors(host(out, True), ref[:, 0]).max() <= TOL["bf16"]
