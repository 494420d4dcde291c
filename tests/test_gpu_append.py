"""Committed-state advance: the verify window's K/V appended through the slot
mapping, the touched pages' summaries recomputed, and the k+1-token verify
attending causally to the appended tokens ([KAP] verifier: the verify window
is scored against the full KV and moves the committed state forward; [KAP]
selected-KV view: the slot mapping gives each new token its page and offset).

The oracle side appends on its own host copies (local page order) with the
oracle's slot mapping; nothing the GPU writes is read back into the oracle.
"""
import numpy as np
import pytest
import torch

import block_sparse_paged_page_amd as kap
import oracle
import workloads as W
from _gpu_util import LSE_TOL, TOL, Case, host, row_errors, t

pytestmark = pytest.mark.gpu

CASES = {
    # fp32, the window opens a new page (1024 = 64 full pages)
    "tiny": lambda: W.spec("tiny", q_len=5),
    # bf16, GQA 4:1; request 0's window crosses a page boundary (4094..4098),
    # request 1's starts mid-page, request 2 is short
    "llama": lambda: W.spec("llama8b_32k", B=3, seq_lens=[4094, 3007, 1234], q_len=5),
    # bf16, GQA 8:1, 40 verify rows per KV head (two row slices)
    "qwen": lambda: W.spec("qwen32b_128k", B=2, seq_lens=[16384, 9999], q_len=5),
}
_cache = {}


def get_case(name):
    if name not in _cache:
        print(f"[case] building {name}", flush=True)
        _cache[name] = Case(CASES[name]())
    return _cache[name]


def _no_selection(w):
    return (np.full((w.B, 1, 1), -1, np.int32), np.zeros((w.B, 1), np.int32))


def _oracle_slots(c, table, positions):
    w = c.w
    sel, cnt = _no_selection(w)
    return oracle.compact(sel, cnt, table, c.b["seq_lens"], positions, w.q_len)[3]


def _gpu_append(c, kn, vn):
    """GPU: slot mapping from kap_compact_view, then kap_append_kv on pool copies."""
    w = c.w
    sel, cnt = _no_selection(w)
    slot = kap.compact_view(t(sel), t(cnt), c.bt, c.L, c.pos, w.q_len)[3]
    K2, V2 = c.K.clone(), c.V.clone()
    kap.append_kv(t(kn), t(vn), slot, K2, V2)
    torch.cuda.synchronize()
    return slot, K2, V2


def _oracle_append_local(c, kn, vn):
    """oracle: the same append on host copies of the allocated pages (local order)."""
    Kl, Vl = c.Kl.copy(), c.Vl.copy()
    oracle.append_kv(kn, vn, _oracle_slots(c, c.btl, c.b["positions"]), Kl, Vl)
    return Kl, Vl


def _bits(x: torch.Tensor) -> np.ndarray:
    a = x.cpu().numpy()
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16)


@pytest.mark.parametrize("name", list(CASES))
def test_append_is_bit_exact(name):
    c = get_case(name)
    w = c.w
    kn, vn = W.draft_kv(w)
    slot, K2, V2 = _gpu_append(c, kn, vn)
    slot_ref = _oracle_slots(c, c.b["bt"], c.b["positions"])
    np.testing.assert_array_equal(slot.cpu().numpy(), slot_ref)
    # oracle append into a host copy of the whole pool
    Kp, Vp = _bits(c.K).copy(), _bits(c.V).copy()
    Kp = Kp.view(np.float32) if not c.bf16 else Kp
    Vp = Vp.view(np.float32) if not c.bf16 else Vp
    oracle.append_kv(kn, vn, slot_ref, Kp, Vp)
    np.testing.assert_array_equal(_bits(K2), Kp.view(np.uint32) if not c.bf16 else Kp)
    np.testing.assert_array_equal(_bits(V2), Vp.view(np.uint32) if not c.bf16 else Vp)


def test_append_skips_unmapped_slots():
    """A window past the block table maps to slot -1: nothing is written."""
    c = get_case("llama")
    w = c.w
    kn, vn = W.draft_kv(w)
    pos = c.b["positions"].copy()
    pos[1] = 16 * c.max_pages              # request 1's window lies past its table
    sel, cnt = _no_selection(w)
    slot = kap.compact_view(t(sel), t(cnt), c.bt, c.L, t(pos), w.q_len)[3]
    K2, V2 = c.K.clone(), c.V.clone()
    kap.append_kv(t(kn), t(vn), slot, K2, V2)
    torch.cuda.synchronize()
    s = slot.cpu().numpy()
    assert np.all(s[1] == -1) and np.all(s[[0, 2]] >= 0)
    slot_ref = _oracle_slots(c, c.b["bt"], pos)
    np.testing.assert_array_equal(s, slot_ref)
    Kp, Vp = _bits(c.K).copy(), _bits(c.V).copy()
    oracle.append_kv(kn, vn, slot_ref, Kp, Vp)
    np.testing.assert_array_equal(_bits(K2), Kp)
    np.testing.assert_array_equal(_bits(V2), Vp)


def _aimed_drafts(c):
    """Draft K/V whose last window token is aimed at the last verify query's
    rotated group direction, strongly enough to dominate that query's softmax:
    attending to it (or leaking it to the earlier queries) is then far outside
    the tolerance."""
    w = c.w
    kn, vn = W.draft_kv(w)
    grp = w.Hq // w.Hkv
    j = w.q_len - 1
    kf = oracle.widen(kn) if c.bf16 else kn.astype(np.float64)
    for bi in range(w.B):
        qj = oracle.widen(c.b["qv"][bi, j]) if c.bf16 else c.b["qv"][bi, j].astype(np.float64)
        u = oracle.rope(qj, float(c.b["positions"][bi] + j)).reshape(w.Hkv, grp, w.D).sum(axis=1)
        # logit of the aimed key ~ alpha * sigma * sqrt(D / grp) / sqrt(D) = 20 (noise keys: ~sigma^2)
        alpha = 20.0 * np.sqrt(grp) / w.sigma
        kf[bi, j] += alpha * u / np.linalg.norm(u, axis=1, keepdims=True)
    kn = oracle.round_to_bf16(kf) if c.bf16 else kf.astype(np.float32)
    return kn, vn


@pytest.mark.parametrize("name", list(CASES))
def test_causal_verify_over_appended_window(name):
    """Query i at L+i sees the context and window tokens 0..i: L+i+1 keys."""
    c = get_case(name)
    w = c.w
    kn, vn = _aimed_drafts(c)
    _, K2, V2 = _gpu_append(c, kn, vn)
    L2 = (c.b["seq_lens"] + w.q_len).astype(np.int32)
    lse = torch.empty((w.B, w.q_len, w.Hq), dtype=torch.float32, device="cuda")
    out = kap.verify_attn(c.qv, c.pos, K2, V2, c.bt, t(L2), lse=lse)
    torch.cuda.synchronize()
    Kl, Vl = _oracle_append_local(c, kn, vn)
    ref, lref = oracle.attend(c.b["qv"], c.b["positions"], Kl, Vl, c.btl, oracle.keys_full(L2), 1,
                              w.Hkv)
    err = row_errors(host(out, c.bf16), ref)
    assert err.max() <= TOL[w.dtype], err.max()
    # the aimed logits are ~20: the bf16 rounding of the rotated query (the MFMA
    # operand) moves them by up to ~2^-8 relative, and the log-sum-exp with them
    lse_tol = LSE_TOL[w.dtype] + (2.0 ** -8 if c.bf16 else 0.0) * np.abs(lref)
    assert np.all(np.abs(lse.cpu().numpy() - lref) <= lse_tol)
    # the aimed key dominates the last query (so attending to it is pinned)...
    ref_wo, _ = oracle.attend(c.b["qv"], c.b["positions"], Kl, Vl, c.btl,
                              oracle.keys_full(L2 - 1), 1, w.Hkv)
    assert row_errors(ref_wo[:, -1], ref[:, -1]).min() > 5 * TOL["bf16"]
    # ...and the earlier queries do not see it (causal)
    np.testing.assert_array_equal(ref_wo[:, :-1], ref[:, :-1])
    print(f"[{name}] causal verify over appended window max rel err {err.max():.2e}", flush=True)


@pytest.mark.parametrize("name", list(CASES))
def test_summary_update_after_append(name):
    """Only the window's pages are recomputed, like the builder; the rest keep every bit."""
    c = get_case(name)
    w = c.w
    kn, vn = W.draft_kv(w)
    _, K2, V2 = _gpu_append(c, kn, vn)
    L2 = (c.b["seq_lens"] + w.q_len).astype(np.int32)
    S2 = c.S.clone()
    kap.update_summary(K2, c.bt, t(L2), c.pos, w.q_len, S2)
    torch.cuda.synchronize()
    Kl, _ = _oracle_append_local(c, kn, vn)
    ref = oracle.summary(Kl, c.btl, L2)                       # fp64, local page order
    phys = c.b["phys"]
    got = host(S2, c.bf16)[phys]
    before = _bits(c.S)[phys]
    after = _bits(S2)[phys]
    touched = np.zeros(len(phys), bool)
    for bi in range(w.B):
        P = int(c.b["positions"][bi])
        for lp in range(P // 16, (P + w.q_len - 1) // 16 + 1):
            touched[c.btl[bi, lp]] = True
    assert touched.sum() >= w.B
    tol = 2.0 ** -8 if c.bf16 else 2.0 ** -20
    d = np.abs(got[touched] - ref[touched])
    assert np.all(d <= np.abs(ref[touched]) * tol + 1e-6)
    np.testing.assert_array_equal(after[~touched], before[~touched])
