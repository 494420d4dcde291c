"""CPU-offloaded routing (EarlySelectKV news item, Interpretation: proxy-query
construction, routing and K-summary state moved to the CPU) against the oracle.

These entry points run on host threads over host memory, so they are checked
here without a GPU: selection bit for bit on the oracle's scores (adversarial
keys included), scores and proxy query within the same tolerances as the GPU
path, and the whole host chain against the oracle chain.
"""
import numpy as np
import pytest

import block_sparse_paged_page_amd as kap
import oracle
import workloads as W

SCORE_TOL = 1e-5


@pytest.mark.parametrize("per_head", [False, True])
@pytest.mark.parametrize("threads", [1, 4])
def test_host_select_bit_exact_on_adversarial_keys(per_head, threads):
    rng = np.random.default_rng(31)
    palette = np.array([0.0, -0.0, 1.0, -1.0, 2.5, np.inf, -np.inf, np.nan, 1.0, 0.5], np.float32)
    B, H, P = 6, 4, 3000
    S = palette[rng.integers(0, len(palette), size=(B, H, P))]
    L = np.array([16 * 3000, 16 * 2999 + 1, 100, 16 * 5, 1, 0], np.int32)
    a = np.array([1, 4, 0, 2, 0, 1], np.int32)
    r = np.array([2, 4, 3, 3, 0, 0], np.int32)
    k = np.array([110, 1000, 2, 0, 5, 3], np.int32)
    cap = 2000
    sel, cnt = kap.host_select_topk(S, L, a, r, k, cap, per_head=per_head, threads=threads)
    sref, cref = oracle.select(S, L, a, r, k, cap, per_head=per_head)
    np.testing.assert_array_equal(sel, sref)
    np.testing.assert_array_equal(cnt, cref)


def test_host_select_random_scores_and_capacity_cue():
    rng = np.random.default_rng(32)
    B, H, P = 4, 8, 8193
    S = rng.standard_normal((B, H, P)).astype(np.float32)
    S[:, :, 100:140] = 3.0                             # a block of exact ties
    L = np.array([131072, 131077, 70000, 12345], np.int32)
    a, r = np.full(B, 1, np.int32), np.full(B, 2, np.int32)
    k = np.full(B, 448, np.int32)
    for per_head in (False, True):
        sel, cnt = kap.host_select_topk(S, L, a, r, k, 451, per_head=per_head)
        sref, cref = oracle.select(S, L, a, r, k, 451, per_head=per_head)
        np.testing.assert_array_equal(sel, sref)
        np.testing.assert_array_equal(cnt, cref)
    with pytest.raises(kap.KapError) as ei:
        kap.host_select_topk(S, L, a, r, k, 450)
    assert ei.value.status == 3


def _small_case(name, **over):
    w = W.spec(name, **over)
    b = W.make(w)
    summ = oracle.round_to_bf16(oracle.summary(b["K_pages"], b["bt_local"], b["seq_lens"]))
    return w, b, summ


@pytest.mark.parametrize("name,over", [
    ("llama8b_32k", dict(B=2, seq_lens=[4096, 1234])),
    ("qwen32b_128k", dict(B=1, seq_lens=[9999])),
])
def test_host_scores_match_oracle(name, over):
    w, b, summ = _small_case(name, **over)
    qf = oracle.widen(b["q"]).astype(np.float32)      # bf16 values, exactly
    got = kap.host_score_blocks(qf, b["positions"], summ, b["bt_local"], b["seq_lens"], w.Hkv)
    ref = oracle.score(b["q"], b["positions"], summ, b["bt_local"], b["seq_lens"], w.Hkv)
    grp = w.Hq // w.Hkv
    for bi in range(w.B):
        n = int(w.n_pages[bi])
        qr = oracle.rope(oracle.widen(b["q"][bi]), float(b["positions"][bi]))
        un = np.linalg.norm(qr.reshape(w.Hkv, grp, w.D).sum(axis=1), axis=1)
        rn = np.linalg.norm(oracle.widen(summ[b["bt_local"][bi, :n]]), axis=-1)
        bound = SCORE_TOL * un[:, None] * rn.T + 1e-30
        assert np.all(np.abs(got[bi, :, :n] - ref[bi, :, :n]) <= bound)
        assert np.all(np.isneginf(got[bi, :, n:]))


def test_host_proxy_query_matches_oracle():
    rng = np.random.default_rng(33)
    B, dm, n = 8, 512, 1024
    hidden = oracle.round_to_bf16(rng.standard_normal((B, dm)))
    wq = oracle.round_to_bf16(rng.standard_normal((dm, n)) / np.sqrt(dm))
    got = kap.host_proxy_query(hidden, wq)
    ref = oracle.proxy_query(hidden, wq)
    e = np.abs(got - ref).max(axis=1) / np.linalg.norm(ref, axis=1)
    assert e.max() <= 1e-5
    # deterministic, whatever the thread count
    assert np.array_equal(kap.host_proxy_query(hidden, wq, threads=1), got)


def test_host_early_routing_chain_matches_oracle_chain():
    """Proxy query -> per-head scores -> per-head top-8, all on the host, against
    the same chain in the oracle; picks may differ only between near-tied pages."""
    w, b, summ = _small_case("early_route_40k", B=2, seq_lens=[12000, 7777])
    qp = kap.host_proxy_query(b["hidden"], b["wq"]).reshape(w.B, w.Hq, w.D)
    scores = kap.host_score_blocks(qp, b["positions"], summ, b["bt_local"], b["seq_lens"], w.Hkv)
    cap = int((b["anchor"] + b["recent"] + b["k_mid"]).max())
    sel, cnt = kap.host_select_topk(scores, b["seq_lens"], b["anchor"], b["recent"], b["k_mid"],
                                    cap, per_head=True)
    qref = oracle.proxy_query(b["hidden"], b["wq"]).astype(np.float32).reshape(w.B, w.Hq, w.D)
    s_ref = oracle.score(qref, b["positions"], summ, b["bt_local"], b["seq_lens"], w.Hkv)
    sel_ref, cnt_ref = oracle.select(s_ref.astype(np.float32), b["seq_lens"], b["anchor"],
                                     b["recent"], b["k_mid"], cap, per_head=True)
    np.testing.assert_array_equal(cnt, cnt_ref)
    for bi in range(w.B):
        for g in range(w.Hkv):
            A, R = set(sel[bi, g].tolist()), set(sel_ref[bi, g].tolist())
            key = s_ref[bi, g]
            scale = np.abs(key[np.isfinite(key)]).max()
            for p_ in A - R:
                for q_ in R - A:
                    assert abs(key[p_] - key[q_]) <= 1e-4 * scale, (bi, g, p_, q_)


def test_host_routing_validation():
    S = np.zeros((1, 2, 8), np.float32)
    one = np.ones(1, np.int32)
    with pytest.raises(kap.KapError) as ei:
        kap.host_select_topk(S, one * 100, one, one, one, 2)       # budget 3 > capacity 2
    assert ei.value.status == 3
    lib = kap.load()
    assert lib.kap_host_score_blocks(None, None, 1e4, None, 1, None, 8, None, 1, 8, 2, 96, 16,
                                     None, 0) == 2
    assert lib.kap_host_proxy_query(None, None, 65, 8, 8, None, 0) == 2
    assert lib.kap_host_proxy_query(None, None, 1, 8, 8, None, 0) == 1
