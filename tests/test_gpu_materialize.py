"""Compact KV workspace: the selected pages copied into a contiguous workspace
([KAP] selected-KV view: the executor materializes a compact physical view;
shape stabilization: a reusable compact KV workspace), then decoded there.

The copy must match the oracle's bit for bit, and a decode over the workspace
must give the same bits as a decode over the compact table into the pool
(same kernel, same plan, only the page placement differs).
"""
import numpy as np
import pytest
import torch

import block_sparse_paged_page_amd as kap
import oracle
import workloads as W
from _gpu_util import TOL, Case, host, row_errors, t

pytestmark = pytest.mark.gpu

CASES = {
    "llama": lambda: W.spec("llama8b_32k", B=3, seq_lens=[4096, 3007, 1234]),       # pooled
    "early": lambda: W.spec("early_route_40k", B=2, seq_lens=[40000, 23456]),      # per head
    "mixed": lambda: W.spec("mixed_serving", B=8, len_range=(100, 20000), pool_pages=None),
}


def _views(c):
    """Oracle selection on oracle scores; compact views from both sides (checked equal)."""
    w, b = c.w, c.b
    cap = c.budget()
    s_ref = oracle.score(b["q"], b["positions"], c.summ_l, c.btl, b["seq_lens"], w.Hkv)
    sel, cnt = oracle.select(s_ref.astype(np.float32), b["seq_lens"], b["anchor"], b["recent"],
                             c.k_mid_h, cap, per_head=w.per_head)
    cv = kap.compact_view(t(sel), t(cnt), c.bt, c.L, c.pos, 1)
    ref = oracle.compact(sel, cnt, b["bt"], b["seq_lens"], b["positions"], 1)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(cv[0].cpu().numpy(), ref[0])
    return sel, cnt, cv, ref


def _bits(x):
    a = x.cpu().numpy()
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16)


@pytest.mark.parametrize("name", list(CASES))
def test_materialize_bit_exact(name):
    c = Case(CASES[name]())
    w = c.w
    sel, cnt, cv, ref = _views(c)
    cbt = cv[0]
    B, G, cap = cbt.shape
    k_ws = torch.zeros((B * cap,) + tuple(c.K.shape[1:]), dtype=c.K.dtype, device="cuda")
    v_ws = torch.zeros((B * cap,) + tuple(c.V.shape[1:]), dtype=c.V.dtype, device="cuda")
    k_ws, v_ws, tab = kap.materialize_view(c.K, c.V, cbt, k_ws, v_ws)
    torch.cuda.synchronize()
    Kp, Vp = W.dense_pool(c.b)
    Kw, Vw, tab_ref = oracle.materialize(Kp, Vp, ref[0])
    np.testing.assert_array_equal(tab.cpu().numpy(), tab_ref)
    got_k, got_v = _bits(k_ws), _bits(v_ws)
    want_k = Kw.view(np.uint32) if Kw.dtype == np.float32 else Kw
    want_v = Vw.view(np.uint32) if Vw.dtype == np.float32 else Vw
    np.testing.assert_array_equal(got_k, want_k)
    np.testing.assert_array_equal(got_v, want_v)
    print(f"[{name}] materialized {int((tab_ref >= 0).sum())} table entries into {B * cap} pages",
          flush=True)


@pytest.mark.parametrize("name", list(CASES))
def test_decode_over_workspace_is_bit_identical(name):
    c = Case(CASES[name]())
    w = c.w
    sel, cnt, cv, ref = _views(c)
    cbt, clog, clen, _ = cv
    G = cbt.shape[1]
    k_ws, v_ws, tab = kap.materialize_view(c.K, c.V, cbt)
    lse1 = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
    lse2 = torch.empty_like(lse1)
    o_pool = kap.decode_attn(c.q, c.pos, c.K, c.V, cbt, clen, G=G, lse=lse1, logical=clog)
    o_ws = kap.decode_attn(c.q, c.pos, k_ws, v_ws, tab, clen, G=G, lse=lse2, logical=clog)
    torch.cuda.synchronize()
    assert torch.equal(o_pool, o_ws) and torch.equal(lse1, lse2)
    # and both are the oracle's selected-KV decode
    keys = oracle.keys_selected(sel, cnt, c.b["seq_lens"])
    oref, _ = oracle.attend(c.b["q"][:, None], c.b["positions"], c.Kl, c.Vl, c.btl, keys, G, w.Hkv)
    assert row_errors(host(o_ws, c.bf16), oref[:, 0]).max() <= TOL[w.dtype]


def test_workspace_reuse_across_plans():
    """The workspace is reusable: a second, smaller plan written over the first
    decodes exactly like its own compact table."""
    c = Case(CASES["llama"]())
    w = c.w
    sel, cnt, cv, _ = _views(c)
    cbt, _, clen, _ = cv
    k_ws, v_ws, tab = kap.materialize_view(c.K, c.V, cbt)
    # a smaller plan: keep only the first half of each selection
    half = (cnt // 2).astype(np.int32)
    sel2 = np.where(np.arange(sel.shape[2])[None, None, :] < half[:, :, None], sel, -1).astype(np.int32)
    cv2 = kap.compact_view(t(sel2), t(half), c.bt, c.L, c.pos, 1)
    k_ws, v_ws, tab2 = kap.materialize_view(c.K, c.V, cv2[0], k_ws, v_ws)
    o_pool = kap.decode_attn(c.q, c.pos, c.K, c.V, cv2[0], cv2[2], logical=cv2[1])
    o_ws = kap.decode_attn(c.q, c.pos, k_ws, v_ws, tab2, cv2[2], logical=cv2[1])
    torch.cuda.synchronize()
    assert torch.equal(o_pool, o_ws)
