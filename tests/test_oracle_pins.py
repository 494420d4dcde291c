"""Pins of the CPU oracle against what the pages and mathematics fix.

Nothing here retypes the oracle's formulas: each check is a hand-derived value
(tests/golden/), a closed form, an invariant, brute force on tiny inputs, or a
library routine (torch scaled_dot_product_attention, numpy matmul, math.cos).
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle import costmodel as cm

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                out.append(line)
    return out


# ----------------------------------------------------------------------------- RoPE
def test_rope_golden_basis_vectors():
    for line in _rows("rope_d4.txt"):
        v = line.split()
        pos, idx = float(v[0]), int(v[1])
        want = np.array([float(x) for x in v[2:6]])
        x = np.zeros(4)
        x[idx] = 1.0
        got = oracle.rope(x, pos, 1e4)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-15)


def test_rope_identity_at_zero_and_norm():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 128))
    np.testing.assert_array_equal(oracle.rope(x, 0.0), x)
    for pos in (1.0, 1024.0, 131075.0):
        y = oracle.rope(x, pos)
        np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)


def test_rope_relative_position_property():
    # R(P) q . R(t) k depends on P - t only
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    a = oracle.rope(q, 1000.0) @ oracle.rope(k, 400.0)
    b = oracle.rope(q, 600.0) @ oracle.rope(k, 0.0)
    c = oracle.rope(q, 131075.0) @ oracle.rope(k, 130475.0)
    assert abs(a - b) < 1e-11 and abs(a - c) < 1e-9


def test_rope_large_position_matches_libm():
    # D = 2: one pair at frequency 1, so the angle is the position itself
    for pos in (131072.0, 131075.0, 1e6 + 3):
        got = oracle.rope(np.array([1.0, 0.0]), pos)
        assert got[0] == pytest.approx(math.cos(pos), abs=1e-12)
        assert got[1] == pytest.approx(math.sin(pos), abs=1e-12)


# ----------------------------------------------------------------------------- summary
def test_summary_constant_page_and_partial_page():
    P, H, ps, D = 6, 2, 16, 8
    K = np.full((P, H, ps, D), np.nan, dtype=np.float32)
    bt = np.array([[3, 1, 5]], dtype=np.int32)
    L = 2 * ps + 5                      # last page holds 5 valid tokens
    K[3] = 2.0
    K[1] = np.arange(ps, dtype=np.float32)[None, :, None]  # token t holds value t
    K[5, :, :5, :] = 7.0                # slots >= 5 stay NaN (must not be read)
    s = oracle.summary(K, bt, np.array([L]), ps)
    np.testing.assert_array_equal(s[3], 2.0)
    np.testing.assert_allclose(s[1], (ps - 1) / 2.0)
    np.testing.assert_array_equal(s[5], 7.0)


def test_summary_linearity():
    rng = np.random.default_rng(2)
    K1 = rng.standard_normal((4, 2, 16, 8)).astype(np.float32)
    K2 = rng.standard_normal((4, 2, 16, 8)).astype(np.float32)
    bt = np.array([[0, 1, 2, 3]], dtype=np.int32)
    L = np.array([64])
    s = oracle.summary(K1 + K2, bt, L) - oracle.summary(K1, bt, L) - oracle.summary(K2, bt, L)
    assert np.abs(s).max() < 1e-6


# ----------------------------------------------------------------------------- score
def _tiny_batch(**over):
    w = W.spec("tiny", **over)
    b = W.make(w)
    K, V = W.dense_pool(b)
    return w, b, K, V


def test_score_gqa_map_and_beyond_length():
    w, b, K, V = _tiny_batch()
    summ = oracle.summary(K, b["bt"], b["seq_lens"]).astype(np.float32)
    grp = w.Hq // w.Hkv
    q = np.zeros((1, w.Hq, w.D), np.float32)
    h = 1                                         # contiguous groups: head 1 is in group 0
    q[0, h, 3] = 1.0
    S = oracle.score(q, np.array([0]), summ, b["bt"], b["seq_lens"], w.Hkv)
    N = int(w.n_pages[0])
    assert np.all(S[0, 1, :N] == 0.0)             # group 1 sees nothing
    # pos 0 leaves q unrotated: the score is the summary element directly
    np.testing.assert_array_equal(S[0, 0, :N], summ[b["bt"][0, :N], 0, 3])
    assert grp > 1
    assert np.all(np.isneginf(S[0, :, N:]))


def test_score_rotation_closed_form():
    # q = e_0 at position P rotates to (cos P, 0.., sin P at D/2, 0..); a summary row
    # equal to that rotated vector scores cos^2 + sin^2 = 1.
    D, H, P = 8, 1, 777
    summ = np.zeros((2, H, D), np.float32)
    summ[1, 0, 0] = np.float32(math.cos(P))
    summ[1, 0, D // 2] = np.float32(math.sin(P))
    q = np.zeros((1, 1, D), np.float32)
    q[0, 0, 0] = 1.0
    S = oracle.score(q, np.array([P]), summ, np.array([[1]], np.int32), np.array([16]), H)
    assert S[0, 0, 0] == pytest.approx(1.0, abs=1e-7)


def test_score_placement_invariance_and_needles():
    w, b, K, V = _tiny_batch()
    # aim needles at the rotated, group-summed query
    grp = w.Hq // w.Hkv
    qr = oracle.rope(oracle.widen(b["q"][0]), float(b["positions"][0]))
    u = qr.reshape(w.Hkv, grp, w.D).sum(axis=1)
    dirs = (u / np.linalg.norm(u, axis=1, keepdims=True))[None]
    b = W.make(w, needle_dir=dirs)
    K, V = W.dense_pool(b)
    summ = oracle.round_to_bf16(oracle.summary(K, b["bt"], b["seq_lens"]))
    S = oracle.score(b["q"], b["positions"], summ, b["bt"], b["seq_lens"], w.Hkv)
    # permute physical placement: same scores bit for bit
    perm = np.random.default_rng(9).permutation(K.shape[0])
    inv = np.argsort(perm)
    summ2 = summ[perm]
    bt2 = np.where(b["bt"] >= 0, inv[np.maximum(b["bt"], 0)], -1).astype(np.int32)
    S2 = oracle.score(b["q"], b["positions"], summ2, bt2, b["seq_lens"], w.Hkv)
    np.testing.assert_array_equal(S, S2)
    # Cauchy-Schwarz bound
    N = int(w.n_pages[0])
    for g in range(w.Hkv):
        rows = oracle.widen(summ[b["bt"][0, :N], g])
        assert np.all(np.abs(S[0, g, :N]) <= np.linalg.norm(u[g]) * np.linalg.norm(rows, axis=1) + 1e-9)
    # needle pages are the top-scoring middle pages under the pooled key
    pooled = S[0, :, :N].mean(axis=0)
    mid = np.arange(1, N - 2)
    top = mid[np.argsort(-pooled[mid], kind="stable")[:len(b["needle_pages"][0])]]
    assert set(top.tolist()) == set(b["needle_pages"][0].tolist())


def test_proxy_query_matches_matmul():
    rng = np.random.default_rng(3)
    hid = oracle.round_to_bf16(rng.standard_normal((3, 64)))
    wq = oracle.round_to_bf16(rng.standard_normal((64, 40)) / 8)
    got = oracle.proxy_query(hid, wq)
    want = oracle.widen(hid) @ oracle.widen(wq)
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)


# ----------------------------------------------------------------------------- select
def _rank_before(x, y):
    """(key_x, idx_x) ranks before (key_y, idx_y): key descending, NaN last, index ascending."""
    (kx, ix), (ky, iy) = x, y
    nx, ny = math.isnan(kx), math.isnan(ky)
    if nx != ny:
        return ny
    if not nx and kx != ky:
        return kx > ky
    return ix < iy


def _brute_force_middle(keys, a, r, k, N):
    if a + r >= N:
        return list(range(N))
    mid = list(range(a, N - r))
    take = min(k, len(mid))
    valid = []
    for T in itertools.combinations(mid, take):
        rest = [u for u in mid if u not in T]
        if all(_rank_before((keys[t], t), (keys[u], u)) for t in T for u in rest):
            valid.append(T)
    assert len(valid) == 1, "exactly one dominating subset must exist"
    return sorted(list(range(a)) + list(valid[0]) + list(range(N - r, N)))


def test_select_brute_force_per_head():
    rng = np.random.default_rng(4)
    palette = np.array([0.0, -0.0, 1.0, -1.0, 2.5, np.inf, -np.inf, np.nan, 1.0, 0.5],
                       dtype=np.float32)
    for trial in range(300):
        N = int(rng.integers(1, 13))
        L = int(rng.integers(16 * (N - 1) + 1, 16 * N + 1))
        a, r = int(rng.integers(0, 3)), int(rng.integers(0, 3))
        k = int(rng.integers(0, N + 1))
        H = 2
        S = palette[rng.integers(0, len(palette), size=(1, H, N + 2))]
        cap = N + 2
        sel, cnt = oracle.select(S, [L], a, r, k, cap, per_head=True)
        for g in range(H):
            want = _brute_force_middle([float(x) for x in S[0, g]], a, r, k, N)
            got = sel[0, g, :cnt[0, g]].tolist()
            assert got == want, (trial, g, S[0, g], a, r, k, N)
            assert np.all(sel[0, g, cnt[0, g]:] == -1)


def test_select_all_equal_keys_takes_lowest_middle():
    N, a, r, k = 40, 3, 2, 7
    S = np.zeros((1, 2, N), np.float32)
    sel, cnt = oracle.select(S, [16 * N], a, r, k, 64, per_head=False)
    assert sel[0, 0, :cnt[0, 0]].tolist() == list(range(a)) + list(range(a, a + k)) + [38, 39]


def test_select_tag_examples():
    rng = np.random.default_rng(5)
    for line in _rows("arkt_tags.txt"):
        v = line.split()
        N, a, r, k, total = map(int, v[:5])
        pinned = [] if v[5] == "-" else [int(x) for x in v[5].split(",")]
        S = rng.standard_normal((1, 4, N)).astype(np.float32)
        sel, cnt = oracle.select(S, [16 * N], a, r, k, 32)
        got = sel[0, 0, :cnt[0, 0]].tolist()
        assert len(got) == total
        assert set(pinned) <= set(got)
        assert got == sorted(got)
        middle = [p for p in got if a <= p < N - r]
        assert len(middle) == k
        if (a, r, k) == (1, 2, 13):
            assert all(1 <= p < 126 for p in middle)


def test_select_short_and_full_budget():
    S = np.random.default_rng(6).standard_normal((2, 2, 10)).astype(np.float32)
    sel, cnt = oracle.select(S, [16 * 3, 16 * 10], [2, 1], [2, 2], [5, 100], 12)
    assert sel[0, 0, :cnt[0, 0]].tolist() == [0, 1, 2]          # a + r >= N
    assert sel[1, 0, :cnt[1, 0]].tolist() == list(range(10))    # budget beyond N


def test_select_pooled_fold_golden():
    for line in _rows("pooled_fold.txt"):
        case, rest = line.split(None, 1)
        c1, c2, expect = [x.strip() for x in rest.split("|")]
        S = np.zeros((1, 4, 2), np.float32)
        S[0, :, 0] = [float(x) for x in c1.split()]
        S[0, :, 1] = [float(x) for x in c2.split()]
        sel, cnt = oracle.select(S, [32], 0, 0, 1, 2, per_head=False)
        assert sel[0, 0, 0] == (0 if expect == "p1" else 1), case


def test_select_mean_equals_sum_ranking_for_power_of_two_heads():
    rng = np.random.default_rng(7)
    S = (rng.standard_normal((1, 8, 300)) * 3).astype(np.float32)
    sel, cnt = oracle.select(S, [300 * 16], 1, 2, 40, 64)
    acc = S[0, 0].copy()
    for g in range(1, 8):
        acc = (acc + S[0, g]).astype(np.float32)
    mid = np.arange(1, 298)
    order = sorted(mid.tolist(), key=lambda p: (-float(acc[p]), p))[:40]
    assert sel[0, 0, :cnt[0, 0]].tolist() == sorted([0, 298, 299] + order)


def test_budget_from_ratio():
    assert oracle.budget_from_ratio(2048, 55, 1000, 1, 2) == 113
    assert oracle.budget_from_ratio(8192, 55, 1000, 1, 2) == 451
    assert oracle.budget_from_ratio(2000, 55, 1000, 1, 2) == 110   # exact: no rounding up
    assert oracle.budget_from_ratio(100, 1, 100, 4, 4) == 8        # raised to a + r
    assert oracle.budget_from_ratio(7, 1, 1, 1, 2) == 7            # capped at N


# ----------------------------------------------------------------------------- compact
def test_compact_identity_and_slots():
    bt = np.array([[5, 9, 2, 7, -1]], dtype=np.int32)
    L = 16 * 3 + 4
    sel = np.array([[[0, 1, 2, 3, -1, -1]]], dtype=np.int32)
    cnt = np.array([[4]], dtype=np.int32)
    cbt, clog, clen, slot = oracle.compact(sel, cnt, bt, [L], [L], 14)
    assert cbt[0, 0].tolist() == [5, 9, 2, 7, -1, -1]
    assert clog[0, 0].tolist() == [0, 1, 2, 3, -1, -1]
    assert clen[0, 0] == L
    # positions 52..65: page 3 (phys 7) slots 4..15, then page 4 unallocated
    assert slot[0].tolist() == [7 * 16 + t for t in range(4, 16)] + [-1, -1]


def test_compact_subset_lengths():
    bt = np.array([[11, 12, 13, 14]], dtype=np.int32)
    sel = np.array([[[1, 3, -1]], ], dtype=np.int32)
    cbt, clog, clen, slot = oracle.compact(sel, np.array([[2]]), bt, [16 * 3 + 1], [49], 1)
    assert cbt[0, 0].tolist() == [12, 14, -1] and clog[0, 0].tolist() == [1, 3, -1]
    assert clen[0, 0] == 16 + 1
    assert slot[0, 0] == 14 * 16 + 1


# ----------------------------------------------------------------------------- attention
def _sdpa_reference(qr, Kd, Vd, mask=None):
    """torch SDPA in fp64 on CPU: qr [Hq][n_q][D], Kd/Vd [Hq][n_k][D]."""
    q = torch.from_numpy(qr)[None]
    k = torch.from_numpy(Kd)[None]
    v = torch.from_numpy(Vd)[None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m)[0].numpy()


def _gather(K, V, bt, b, g, toks, ps=16):
    pages = bt[b, toks // ps]
    slots = toks % ps
    Kd = oracle.widen(K[pages, g, slots, :])
    Vd = oracle.widen(V[pages, g, :, slots])
    return Kd, Vd


def test_attend_matches_sdpa_on_selected_keys():
    w, b, K, V = _tiny_batch()
    S = oracle.score(b["q"], b["positions"], oracle.summary(K, b["bt"], b["seq_lens"]).astype(np.float32),
                     b["bt"], b["seq_lens"], w.Hkv)
    sel, cnt = oracle.select(S.astype(np.float32), b["seq_lens"], 1, 2, 5, 16)
    keys = oracle.keys_selected(sel, cnt, b["seq_lens"])
    q = b["q"][:, None]
    out, lse = oracle.attend(q, b["positions"], K, V, b["bt"], keys, 1, w.Hkv)
    grp = w.Hq // w.Hkv
    qr = oracle.rope(oracle.widen(b["q"][0]), float(b["positions"][0]))
    toks = keys[0]
    for h in range(w.Hq):
        Kd, Vd = _gather(K, V, b["bt"], 0, h // grp, toks)
        ref = _sdpa_reference(qr[h][None, None], Kd[None], Vd[None])[0, 0]
        np.testing.assert_allclose(out[0, 0, h], ref, rtol=1e-12, atol=1e-13)
        z = torch.from_numpy(Kd @ qr[h] / math.sqrt(w.D))
        assert lse[0, 0, h] == pytest.approx(float(torch.logsumexp(z, 0)), abs=1e-12)


def test_attend_causal_window_matches_sdpa_mask():
    w, b, K, V = _tiny_batch()
    L = int(b["seq_lens"][0])
    P = L - 3                                       # window overlapping the context end
    qv = b["qv"]
    keys = oracle.keys_full([L])
    out, lse = oracle.attend(qv, np.array([P]), K, V, b["bt"], keys, 1, w.Hkv)
    grp = w.Hq // w.Hkv
    toks = np.arange(L)
    for h in range(w.Hq):
        qr = np.stack([oracle.rope(oracle.widen(qv[0, i, h]), float(P + i)) for i in range(w.q_len)])
        mask = toks[None, :] <= (P + np.arange(w.q_len))[:, None]
        Kd, Vd = _gather(K, V, b["bt"], 0, h // grp, toks)
        ref = _sdpa_reference(qr[None], Kd[None], Vd[None], mask)[0]
        np.testing.assert_allclose(out[0, :, h], ref, rtol=1e-11, atol=1e-12)


def test_attend_special_cases():
    ps, H, D = 16, 1, 8
    K = np.zeros((3, H, ps, D), np.float32)
    V = np.zeros((3, H, D, ps), np.float32)
    rng = np.random.default_rng(8)
    V[1, 0] = rng.standard_normal((D, ps)).astype(np.float32)
    K[1, 0] = rng.standard_normal((ps, D)).astype(np.float32)
    bt = np.array([[1, 2]], np.int32)
    q = rng.standard_normal((1, 1, 1, D)).astype(np.float32)
    # one key: out = v
    out, lse = oracle.attend(q, [40], K, V, bt, [np.array([5], np.int32)], 1, H)
    np.testing.assert_allclose(out[0, 0, 0], V[1, 0, :, 5], rtol=0, atol=1e-7)
    # all keys equal (zero): uniform weights -> mean of V, lse = log n
    K0 = K.copy()
    K0[1, 0] = 0
    out, lse = oracle.attend(q, [40], K0, V, bt, [np.arange(16, dtype=np.int32)], 1, H)
    np.testing.assert_allclose(out[0, 0, 0], V[1, 0].astype(np.float64).mean(axis=1), atol=1e-12)
    assert lse[0, 0, 0] == pytest.approx(math.log(16), abs=1e-12)
    # all values equal: out = that value
    V1 = V.copy()
    V1[1, 0] = 0.25
    out, lse = oracle.attend(q, [40], K, V1, bt, [np.arange(16, dtype=np.int32)], 1, H)
    np.testing.assert_allclose(out[0, 0, 0], 0.25, atol=1e-12)
    # no visible key: zeros and -inf
    out, lse = oracle.attend(q, [2], K, V, bt, [np.array([5], np.int32)], 1, H)
    assert np.all(out == 0) and np.isneginf(lse[0, 0, 0])


def test_attend_placement_invariance_and_full_selection():
    w, b, K, V = _tiny_batch()
    N = int(w.n_pages[0])
    full = oracle.keys_full(b["seq_lens"])
    o1, l1 = oracle.attend(b["q"][:, None], b["positions"], K, V, b["bt"], full, 1, w.Hkv)
    # selecting every page is the full context
    sel, cnt = oracle.select(np.zeros((1, w.Hkv, N), np.float32), b["seq_lens"], 1, 2, N, N)
    o2, l2 = oracle.attend(b["q"][:, None], b["positions"], K, V, b["bt"],
                           oracle.keys_selected(sel, cnt, b["seq_lens"]), 1, w.Hkv)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    # moving pages in the pool (with the table) changes nothing
    perm = np.random.default_rng(10).permutation(K.shape[0])
    inv = np.argsort(perm)
    bt2 = np.where(b["bt"] >= 0, inv[np.maximum(b["bt"], 0)], -1).astype(np.int32)
    o3, l3 = oracle.attend(b["q"][:, None], b["positions"], K[perm], V[perm], bt2, full, 1, w.Hkv)
    np.testing.assert_array_equal(o1, o3)
    np.testing.assert_array_equal(l1, l3)


def test_append_then_attend_sees_new_tokens():
    ps, H, D = 16, 2, 8
    K = np.zeros((4, H, ps, D), np.float32)
    V = np.zeros((4, H, D, ps), np.float32)
    bt = np.array([[2, 0]], np.int32)
    rng = np.random.default_rng(11)
    kn = rng.standard_normal((1, 3, H, D)).astype(np.float32)
    vn = rng.standard_normal((1, 3, H, D)).astype(np.float32)
    _, _, _, slot = oracle.compact(np.zeros((1, 1, 1), np.int32), np.array([[0]]), bt, [15], [15], 3)
    assert slot[0].tolist() == [2 * 16 + 15, 0 * 16 + 0, 0 * 16 + 1]
    oracle.append_kv(kn, vn, slot, K, V)
    np.testing.assert_array_equal(K[2, :, 15], kn[0, 0])
    np.testing.assert_array_equal(V[0, :, :, 1], vn[0, 2])
    # a single visible key after the append is returned verbatim
    q = rng.standard_normal((1, 1, 2, D)).astype(np.float32)
    out, _ = oracle.attend(q, [17], K, V, bt, [np.array([17], np.int32)], 1, H)
    np.testing.assert_allclose(out[0, 0, 0], vn[0, 2, 0], atol=1e-7)


def test_materialize_places_each_head_of_each_selected_page():
    """Every K/V element encodes its (page, head); the workspace must show, in page
    b*cap + j and head slot g, the code of compact page j of row (b, g or 0)."""
    ps, H, D, P = 16, 4, 8, 12
    code = (100 * np.arange(P)[:, None] + np.arange(H)[None, :]).astype(np.float32)  # [P][H]
    K = np.broadcast_to(code[:, :, None, None], (P, H, ps, D)).copy()
    V = np.broadcast_to(-code[:, :, None, None], (P, H, D, ps)).copy()
    B, cap = 2, 3
    for G in (1, H):
        cbt = np.full((B, G, cap), -1, np.int32)
        rng = np.random.default_rng(40 + G)
        for b in range(B):
            for gr in range(G):
                n = int(rng.integers(1, cap + 1))
                cbt[b, gr, :n] = rng.choice(P, size=n, replace=False)
        Kws, Vws, tab = oracle.materialize(K, V, cbt)
        for b in range(B):
            for j in range(cap):
                for g in range(H):
                    src = cbt[b, 0 if G == 1 else g, j]
                    want = 100 * src + g if src >= 0 else 0.0
                    assert np.all(Kws[b * cap + j, g] == want) and np.all(Vws[b * cap + j, g] == -want)
        expect = np.where(cbt >= 0, (np.arange(B)[:, None, None] * cap + np.arange(cap)[None, None, :]), -1)
        np.testing.assert_array_equal(tab, np.broadcast_to(expect, cbt.shape))


def test_attention_over_materialized_view_is_unchanged():
    """Selected-page decode reads the same keys through the workspace table."""
    rng = np.random.default_rng(41)
    ps, H, Hq, D, P = 16, 2, 4, 8, 10
    K = rng.standard_normal((P, H, ps, D)).astype(np.float32)
    V = rng.standard_normal((P, H, D, ps)).astype(np.float32)
    bt = rng.permutation(P).astype(np.int32)[None, :8]
    L = [8 * ps - 5]
    sel = np.array([[[0, 3, 7, -1]]], np.int32)
    cnt = np.array([[3]], np.int32)
    cbt, clog, clen, _ = oracle.compact(sel, cnt, bt, L, L, 0)
    Kws, Vws, tab = oracle.materialize(K, V, cbt)
    # the workspace view as a logical table: selected logical page -> workspace page
    bt_ws = np.full_like(bt, -1)
    bt_ws[0, clog[0, 0, :3]] = tab[0, 0, :3]
    keys = oracle.keys_selected(sel, cnt, L)
    q = rng.standard_normal((1, 1, Hq, D)).astype(np.float32)
    o1, l1 = oracle.attend(q, L, K, V, bt, keys, 1, H)
    o2, l2 = oracle.attend(q, L, Kws, Vws, bt_ws, keys, 1, H)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


# ----------------------------------------------------------------------------- cost model
def test_phase_boundary_identity():
    rng = np.random.default_rng(12)
    for _ in range(20000):
        k = int(rng.integers(1, 12))
        h, s = rng.uniform(0, 1), rng.uniform(0.001, 1)
        wm, kv = rng.uniform(0.1, 100), rng.uniform(0.1, 100)
        plan = cm.cost_plan(k, s, wm, wm, kv)
        base = cm.cost_base(k, h, wm, kv)
        if abs(plan - base) < 1e-9 * base:
            continue
        assert (plan < base) == cm.phase_boundary_holds(h, s, wm, kv)


def test_table5_break_even():
    for line in _rows("table5_phase.txt"):
        ctx, s, margin, h, be = line.split()
        s, margin, h, be = float(s), float(margin), float(h), float(be)
        assert s + margin == pytest.approx(h, abs=1e-12)
        assert cm.break_even_w_over_kv(h, s) == pytest.approx(be, rel=1e-9)
        # at exactly the break-even weight cost the plan neither wins nor loses
        kv = 1.0
        w = be * kv
        assert cm.cost_plan(6, s, w, w, kv) == pytest.approx(cm.cost_base(6, h, w, kv), rel=1e-12)
        assert cm.kv_crit(h, s, w) == pytest.approx(kv, rel=1e-12)
    assert cm.kv_crit(0.3, 0.4, 1.0) == float("inf")


# ----------------------------------------------------------------------------- stored inputs
def test_stored_needle_directions_match_the_oracle():
    """workloads/aim/*.npz (the benchmark's needle directions) are the unit
    vectors of the group-summed rotated query, as tests/golden/make_needle_dirs.py
    computes them with the oracle's RoPE, for the current query draws."""
    import importlib.util
    import workloads as W
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "make_needle_dirs.py")
    spec = importlib.util.spec_from_file_location("make_needle_dirs", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    for name, B in mod.WORKLOADS.items():
        dirs, keys = mod.aimed(name, B)
        w = W.spec(name, B=B) if name != "mixed_serving" else W.spec(name)
        stored = W.aimed_dirs(w)
        np.testing.assert_allclose(stored, dirs, rtol=0, atol=1e-6)
        np.testing.assert_allclose(np.linalg.norm(stored, axis=-1), 1.0, atol=1e-6)
