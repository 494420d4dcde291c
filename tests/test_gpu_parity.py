"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Inputs come from the seeded generators (workloads/); expected values come from
the oracle on the same host arrays.  Nothing the GPU produces is fed to the
oracle: integer stages (selection, compaction) are fed oracle-made inputs on
both sides and must match bit for bit; the full GPU chain is then compared
with the full oracle chain.
"""
import numpy as np
import pytest
import torch

import block_sparse_paged_page_amd as kap
import oracle
import workloads as W
from _gpu_util import (LSE_TOL, TOL, Case, check_scores, host, row_errors, t, workspace)

pytestmark = pytest.mark.gpu

CASES = {
    # tiny fp32 case: 1 x 1024 tokens, GQA 4:1, D 64, A1R2K5
    "tiny": lambda: W.spec("tiny"),
    # Llama-3-8B-shaped attention, ragged and short rows (one shorter than its budget)
    "llama": lambda: W.spec("llama8b_32k", B=3, seq_lens=[4096, 3007, 1234]),
    # 32B-shaped, GQA 8:1 (verify rows = 32), ragged
    "qwen": lambda: W.spec("qwen32b_128k", B=2, seq_lens=[16384, 9999]),
    # mixed serving batch: ragged lengths, per-request retention and A/R splits
    "mixed": lambda: W.spec("mixed_serving", B=8, len_range=(100, 20000), pool_pages=None),
}
_cache = {}


def get_case(name):
    if name not in _cache:
        print(f"[case] building {name}", flush=True)
        _cache[name] = Case(CASES[name](), aim_needles=True)
    return _cache[name]


def _oracle_chain(c, cap):
    w, b = c.w, c.b
    s_ref = oracle.score(b["q"], b["positions"], c.summ_l, c.btl, b["seq_lens"], w.Hkv)
    sel, cnt = oracle.select(s_ref.astype(np.float32), b["seq_lens"], b["anchor"], b["recent"],
                             c.k_mid_h, cap, per_head=w.per_head)
    return s_ref, sel, cnt


def _gpu_chain(c, cap):
    w = c.w
    scores = kap.score_blocks(c.q, c.pos, c.S, c.bt, c.L, w.Hkv)
    sel, cnt = kap.select_topk(scores, c.L, c.anchor, c.recent, c.k_mid, c.budget(), cap,
                               per_head=w.per_head)
    return scores, sel, cnt


@pytest.mark.parametrize("name", list(CASES))
def test_score_parity(name):
    c = get_case(name)
    scores = kap.score_blocks(c.q, c.pos, c.S, c.bt, c.L, c.w.Hkv)
    torch.cuda.synchronize()
    check_scores(c, scores.cpu().numpy())


def _check_pooled(c):
    """kap_score_pool_blocks: per-head scores within the scoring tolerance, the
    pooled key equal to the head-order fp32 fold of those scores (bit for
    bit), and top-K on the pooled key (one row, Hkv = 1) equal to the oracle's
    pooled top-K on the per-head scores."""
    w = c.w
    scores, pooled = kap.score_pool_blocks(c.q, c.pos, c.S, c.bt, c.L, w.Hkv)
    _, pooled_only = kap.score_pool_blocks(c.q, c.pos, c.S, c.bt, c.L, w.Hkv, with_scores=False)
    torch.cuda.synchronize()
    s = scores.cpu().numpy()
    check_scores(c, s)
    fold = s[:, 0].copy()
    for g in range(1, w.Hkv):
        fold = fold + s[:, g]                      # float32 adds, round to nearest
    fold = fold / np.float32(w.Hkv)
    got = pooled.cpu().numpy()
    np.testing.assert_array_equal(got.view(np.uint32), fold.view(np.uint32))
    np.testing.assert_array_equal(pooled_only.cpu().numpy().view(np.uint32), got.view(np.uint32))
    cap = c.budget() + 3
    sel, cnt = kap.select_topk(pooled.view(w.B, 1, -1), c.L, c.anchor, c.recent, c.k_mid,
                               c.budget(), cap)
    sel_ref, cnt_ref = oracle.select(s, c.b["seq_lens"], c.b["anchor"], c.b["recent"], c.k_mid_h,
                                     cap, per_head=False)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sel.cpu().numpy(), sel_ref)
    np.testing.assert_array_equal(cnt.cpu().numpy(), cnt_ref)


@pytest.mark.parametrize("name", list(CASES))
def test_pooled_scoring(name):
    _check_pooled(get_case(name))


@pytest.mark.parametrize("name", list(CASES))
def test_select_bit_exact_on_oracle_scores(name):
    c = get_case(name)
    cap = c.budget() + 3
    s_ref, sel_ref, cnt_ref = _oracle_chain(c, cap)
    s32 = torch.from_numpy(s_ref.astype(np.float32)).cuda()
    sel, cnt = kap.select_topk(s32, c.L, c.anchor, c.recent, c.k_mid, c.budget(), cap,
                               per_head=c.w.per_head)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sel.cpu().numpy(), sel_ref)
    np.testing.assert_array_equal(cnt.cpu().numpy(), cnt_ref)


@pytest.mark.parametrize("name", list(CASES))
def test_chain_selection_matches_oracle_chain(name):
    c = get_case(name)
    cap = c.budget() + 3
    s_ref, sel_ref, cnt_ref = _oracle_chain(c, cap)
    _, sel, cnt = _gpu_chain(c, cap)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(cnt.cpu().numpy(), cnt_ref)
    sel_h = sel.cpu().numpy()
    # picks may differ only by swapping near-tied pages (scores agree to SCORE_TOL, not bits)
    flips = 0
    for bi in range(c.w.B):
        for gr in range(sel_h.shape[1]):
            n = int(cnt_ref[bi, gr])
            a, b = set(sel_h[bi, gr, :n].tolist()), set(sel_ref[bi, gr, :n].tolist())
            if a == b:
                continue
            key = s_ref[bi, gr] if c.w.per_head else s_ref[bi].mean(axis=0)
            scale = np.abs(key[np.isfinite(key)]).max()
            for p_ in a - b:
                for q_ in b - a:
                    assert abs(key[p_] - key[q_]) <= 1e-4 * scale, (bi, gr, p_, q_)
            flips += len(a - b)
    print(f"[{name}] near-tie flips between GPU and oracle chains: {flips}", flush=True)
    # aimed needles are picked
    for bi, pages in enumerate(c.b["needle_pages"]):
        chosen = set(sel_h[bi, 0, :cnt_ref[bi, 0]].tolist())
        k = int(c.k_mid_h[bi])
        if k >= len(pages):
            assert set(pages.tolist()) <= chosen


@pytest.mark.parametrize("name", list(CASES))
def test_compact_bit_exact(name):
    c = get_case(name)
    cap = c.budget() + 3
    _, sel_ref, cnt_ref = _oracle_chain(c, cap)
    q_new = 5
    cbt, clog, clen, slot = kap.compact_view(t(sel_ref), t(cnt_ref), c.bt, c.L, c.pos, q_new)
    torch.cuda.synchronize()
    r = oracle.compact(sel_ref, cnt_ref, c.b["bt"], c.b["seq_lens"], c.b["positions"], q_new)
    for got, want in zip((cbt, clog, clen, slot), r):
        np.testing.assert_array_equal(got.cpu().numpy(), want)


def _check_attn(c, out, lse, ref, lref):
    tol = TOL[c.w.dtype]
    o = host(out, c.bf16)
    e = row_errors(o.reshape(ref.shape), ref)
    assert e.max() <= tol, f"attention error {e.max():.3e} > {tol}"
    lg = lse.cpu().numpy().reshape(lref.shape)
    fin = np.isfinite(lref)
    assert np.array_equal(np.isfinite(lg), fin)
    if fin.any():
        d = np.abs(lg[fin] - lref[fin]).max()
        assert d <= LSE_TOL[c.w.dtype], f"lse error {d:.3e}"
    return float(e.max())


@pytest.mark.parametrize("name", list(CASES))
def test_selected_decode_parity(name):
    c = get_case(name)
    w = c.w
    cap = c.budget() + 3
    _, sel_ref, cnt_ref = _oracle_chain(c, cap)
    cbt, clog, clen, slot = kap.compact_view(t(sel_ref), t(cnt_ref), c.bt, c.L, c.pos, 1)
    G = w.Hkv if w.per_head else 1
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
    out = kap.decode_attn(c.q, c.pos, c.K, c.V, cbt, clen, G=G, lse=lse, logical=clog)
    torch.cuda.synchronize()
    keys = oracle.keys_selected(sel_ref, cnt_ref, c.b["seq_lens"])
    ref, lref = oracle.attend(c.b["q"][:, None], c.b["positions"], c.Kl, c.Vl, c.btl, keys, G, w.Hkv)
    err = _check_attn(c, out, lse, ref[:, 0], lref[:, 0])
    print(f"[{name}] selected decode max rel err {err:.2e}", flush=True)


@pytest.mark.parametrize("name,per_head", [("tiny", False), ("llama", False), ("llama", True),
                                           ("qwen", False), ("mixed", False)])
def test_selected_decode_position_inside_context(name, per_head):
    """The decode's causal rule is on logical positions (the compact view keeps
    them): with the query placed inside the context, selected pages past it
    (the recent pages, the later middle picks) must be hidden exactly as the
    oracle hides them over the selected keys, although their compact indices
    are below the query position.  The rotation is at the same position."""
    c = get_case(name)
    w = c.w
    b = c.b
    cap = c.budget() + 3
    s_ref = oracle.score(b["q"], b["positions"], c.summ_l, c.btl, b["seq_lens"], w.Hkv)
    sel_ref, cnt_ref = oracle.select(s_ref.astype(np.float32), b["seq_lens"], b["anchor"],
                                     b["recent"], c.k_mid_h, cap, per_head=per_head)
    cbt, clog, clen, _ = kap.compact_view(t(sel_ref), t(cnt_ref), c.bt, c.L, c.pos, 1)
    G = w.Hkv if per_head else 1
    pin = np.maximum(b["seq_lens"].astype(np.int64) * 2 // 3 - 3, 1).astype(np.int32)
    keys = oracle.keys_selected(sel_ref, cnt_ref, b["seq_lens"])
    hidden = [int((k > pin[i // G]).sum()) for i, k in enumerate(keys)]
    shown = [int((k <= pin[i // G]).sum()) for i, k in enumerate(keys)]
    assert min(hidden) > 0 and min(shown) > 0, (hidden, shown)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
    out = kap.decode_attn(c.q, t(pin), c.K, c.V, cbt, clen, G=G, lse=lse, logical=clog)
    torch.cuda.synchronize()
    ref, lref = oracle.attend(b["q"][:, None], pin, c.Kl, c.Vl, c.btl, keys, G, w.Hkv)
    err = _check_attn(c, out, lse, ref[:, 0], lref[:, 0])
    print(f"[{name}, per_head={per_head}] decode inside the context: hidden keys per row "
          f"{min(hidden)}..{max(hidden)}, max rel err {err:.2e}", flush=True)


@pytest.mark.parametrize("name", list(CASES))
def test_full_decode_parity(name):
    c = get_case(name)
    w = c.w
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
    out = kap.decode_attn(c.q, c.pos, c.K, c.V, c.bt, c.L, G=1, lse=lse)
    torch.cuda.synchronize()
    ref, lref = oracle.attend(c.b["q"][:, None], c.b["positions"], c.Kl, c.Vl, c.btl,
                              oracle.keys_full(c.b["seq_lens"]), 1, w.Hkv)
    err = _check_attn(c, out, lse, ref[:, 0], lref[:, 0])
    print(f"[{name}] full decode max rel err {err:.2e}", flush=True)


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("shift", [0, -3])
def test_verify_parity(name, shift):
    """Window at the context end (shift 0) and overlapping it (causal masking)."""
    c = get_case(name)
    w = c.w
    start = np.maximum(c.b["positions"] + shift, 0).astype(np.int32)
    lse = torch.empty((w.B, w.q_len, w.Hq), dtype=torch.float32, device="cuda")
    out = kap.verify_attn(c.qv, t(start), c.K, c.V, c.bt, c.L, lse=lse)
    torch.cuda.synchronize()
    ref, lref = oracle.attend(c.b["qv"], start, c.Kl, c.Vl, c.btl,
                              oracle.keys_full(c.b["seq_lens"]), 1, w.Hkv)
    err = _check_attn(c, out, lse, ref, lref)
    print(f"[{name}] verify (shift {shift}) max rel err {err:.2e}", flush=True)


@pytest.mark.parametrize("name", ["llama", "qwen"])
def test_gpu_chain_end_to_end(name):
    """score -> select -> compact -> decode, all on the GPU, against the oracle chain."""
    c = get_case(name)
    w = c.w
    cap = c.budget()
    _, sel_ref, cnt_ref = _oracle_chain(c, cap)
    _, sel, cnt = _gpu_chain(c, cap)
    cbt, clog, clen, slot = kap.compact_view(sel, cnt, c.bt, c.L, c.pos, 1)
    out = kap.decode_attn(c.q, c.pos, c.K, c.V, cbt, clen, G=1, logical=clog)
    torch.cuda.synchronize()
    keys = oracle.keys_selected(sel_ref, cnt_ref, c.b["seq_lens"])
    ref, _ = oracle.attend(c.b["q"][:, None], c.b["positions"], c.Kl, c.Vl, c.btl, keys, 1, w.Hkv)
    e = row_errors(host(out, c.bf16), ref[:, 0])
    assert e.max() <= TOL[w.dtype]


@pytest.mark.parametrize("name,q_len,D", [
    ("qwen", 5, 128),    # 40 rows per KV head: one 48-row tile
    ("qwen", 8, 128),    # 64 rows: one 64-row tile
    ("qwen", 16, 128),   # 128 rows: two 64-row slices
    ("llama", 16, 128),  # GQA 4:1, 64 rows
    ("llama", 12, 64),   # head_dim 64, 48 rows
    ("llama", 16, 64),   # head_dim 64, 64 rows
])
def test_verify_row_tiles(name, q_len, D):
    """Windows whose row group (GQA group x window) needs 48- and 64-row tiles,
    in causal overlap with the context end."""
    base = CASES[name]()
    w = W.spec(base.name, B=base.B, seq_lens=list(base.seq_lens), q_len=q_len, D=D)
    c = Case(w)
    start = np.maximum(c.b["positions"] - 7, 0).astype(np.int32)
    lse = torch.empty((w.B, q_len, w.Hq), dtype=torch.float32, device="cuda")
    out = kap.verify_attn(c.qv, t(start), c.K, c.V, c.bt, c.L, lse=lse)
    torch.cuda.synchronize()
    ref, lref = oracle.attend(c.b["qv"], start, c.Kl, c.Vl, c.btl,
                              oracle.keys_full(c.b["seq_lens"]), 1, w.Hkv)
    err = _check_attn(c, out, lse, ref, lref)
    print(f"[{name} q_len {q_len} D {D}] verify max rel err {err:.2e}", flush=True)


_long_cache = {}


@pytest.mark.parametrize("q_len,D", [(4, 128), (2, 128), (4, 64)])
def test_long_ragged_items(q_len, D):
    """Work items longer than 32 pages, whose length is not a multiple of the
    kernel's 4-page step, and a shorter last item in every row: the disciplines
    for long page runs (the staggered loop for 32-row tiles, the throttled ring
    for 16-row tiles and the q = 1 decode).  4 requests of 33K-52K tokens under
    GQA 8:1 with 4 KV heads make 16 rows of 2084-3251 pages; on MI355X the plan
    splits them into items of 41 pages (32-row tiles, 1024 resident waves) or 32
    pages (16-row tiles, 1280 items), every row ending in a shorter item.  Head
    dim 128 and 64."""
    if (q_len, D) not in _long_cache:
        _long_cache.clear()
        w = W.spec("qwen32b_128k", B=4, seq_lens=[52001, 41111, 36000, 33333], Hq=32, Hkv=4,
                   q_len=q_len, D=D)
        _long_cache[(q_len, D)] = Case(w)
    c = _long_cache[(q_len, D)]
    w = c.w
    start = np.maximum(c.b["positions"] - 3, 0).astype(np.int32)
    lse = torch.empty((w.B, q_len, w.Hq), dtype=torch.float32, device="cuda")
    out = kap.verify_attn(c.qv, t(start), c.K, c.V, c.bt, c.L, lse=lse)
    torch.cuda.synchronize()
    ref, lref = oracle.attend(c.b["qv"], start, c.Kl, c.Vl, c.btl,
                              oracle.keys_full(c.b["seq_lens"]), 1, w.Hkv)
    err = _check_attn(c, out, lse, ref, lref)
    print(f"[long items, q_len {q_len}, D {D}] verify max rel err {err:.2e}", flush=True)
    if q_len == 2:
        lse1 = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
        out1 = kap.decode_attn(c.q, c.pos, c.K, c.V, c.bt, c.L, G=1, lse=lse1)
        torch.cuda.synchronize()
        ref1, lref1 = oracle.attend(c.b["q"][:, None], c.b["positions"], c.Kl, c.Vl, c.btl,
                                    oracle.keys_full(c.b["seq_lens"]), 1, w.Hkv)
        err1 = _check_attn(c, out1, lse1, ref1[:, 0], lref1[:, 0])
        print(f"[long items] full decode max rel err {err1:.2e}", flush=True)
        # the long-item discipline with a logical table (here the identity, so
        # bit-identical to no table) and the query inside the context
        width = c.b["bt"].shape[1]
        ident = t(np.tile(np.arange(width, dtype=np.int32), (w.B, 1)))
        pin = (c.b["positions"].astype(np.int64) * 3 // 5 + 7).astype(np.int32)
        lse2, lse3 = (torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda") for _ in range(2))
        out2 = kap.decode_attn(c.q, t(pin), c.K, c.V, c.bt, c.L, G=1, lse=lse2, logical=ident)
        out3 = kap.decode_attn(c.q, t(pin), c.K, c.V, c.bt, c.L, G=1, lse=lse3)
        torch.cuda.synchronize()
        assert torch.equal(out2, out3) and torch.equal(lse2, lse3)
        ref2, lref2 = oracle.attend(c.b["q"][:, None], pin, c.Kl, c.Vl, c.btl,
                                    oracle.keys_full(c.b["seq_lens"]), 1, w.Hkv)
        err2 = _check_attn(c, out2, lse2, ref2[:, 0], lref2[:, 0])
        print(f"[long items] decode inside the context max rel err {err2:.2e}", flush=True)
    _long_cache.clear()


@pytest.mark.parametrize("counts,D", [([700, 613, 651, 590], 128), ([587, 598, 609, 602], 128),
                                      ([700, 613, 651, 590], 64)])
def test_two_pairs_in_flight_tails(counts, D):
    """The pair loop with two pairs in flight (views with one row tile whose
    items have at least eight pages): 4 requests with compact views of the
    given page counts (ragged) under GQA 8:1 with 4 KV heads make 16 rows.  On
    MI355X the plan splits them into items of 9 pages (first and last sets) or
    8 pages (second set), and every row ends in a shorter item, so the tails
    after the unrolled loop take every length from one to seven pages (9-page
    items: 5 after one pass; last items 7, 1, 3, 5 and 3, 6, 1, 2).  The query
    sits at the sequence end and inside the context (the causal rule on the
    compact view's logical pages)."""
    w = W.spec("qwen32b_128k", B=4, seq_lens=[23000, 20011, 30000, 25555], Hq=32, Hkv=4, D=D)
    c = Case(w)
    N = w.n_pages
    counts = np.array(counts, np.int32)
    rng = np.random.default_rng(77)
    cap = int(counts.max())
    sel = np.full((w.B, 1, cap), -1, np.int32)
    for bi in range(w.B):
        pages = rng.choice(int(N[bi]), size=int(counts[bi]), replace=False)
        sel[bi, 0, :counts[bi]] = np.sort(pages).astype(np.int32)
    cnt = counts.reshape(w.B, 1)
    cbt, clog, clen, _ = kap.compact_view(t(sel), t(cnt), c.bt, c.L, c.pos, 1)
    keys = oracle.keys_selected(sel, cnt, c.b["seq_lens"])
    inside = (c.b["positions"].astype(np.int64) * 2 // 3).astype(np.int32)
    for pos in (c.b["positions"], inside):
        lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
        out = kap.decode_attn(c.q, t(pos), c.K, c.V, cbt, clen, G=1, lse=lse, logical=clog)
        torch.cuda.synchronize()
        ref, lref = oracle.attend(c.b["q"][:, None], pos, c.Kl, c.Vl, c.btl, keys, 1, w.Hkv)
        err = _check_attn(c, out, lse, ref[:, 0], lref[:, 0])
        print(f"[two pairs, counts {counts.tolist()}, D {D}] max rel err {err:.2e}", flush=True)


@pytest.mark.parametrize("D", [128, 64])
def test_short_items_made_eight_pages(D):
    """Views whose items would be four to seven pages run as eight-page items
    with two pairs in flight: 2 requests x 8 KV heads (16 rows) with compact
    views of 300 and 277 pages bound the item length at ceil(300 * 16 / 1264)
    = 4 pages on the host, so the item cap drops to 16 * ceil(300 / 8) and the
    device plan splits the ragged rows into items of 8 pages, each row ending
    in a shorter one (4 and 5 pages).  The query sits at the sequence end and
    inside the context."""
    w = W.spec("qwen32b_128k", B=2, seq_lens=[9000, 7777], Hq=64, Hkv=8, D=D)
    c = Case(w)
    N = w.n_pages
    counts = np.array([300, 277], np.int32)
    rng = np.random.default_rng(78)
    cap = int(counts.max())
    sel = np.full((w.B, 1, cap), -1, np.int32)
    for bi in range(w.B):
        pages = rng.choice(int(N[bi]), size=int(counts[bi]), replace=False)
        sel[bi, 0, :counts[bi]] = np.sort(pages).astype(np.int32)
    cnt = counts.reshape(w.B, 1)
    cbt, clog, clen, _ = kap.compact_view(t(sel), t(cnt), c.bt, c.L, c.pos, 1)
    keys = oracle.keys_selected(sel, cnt, c.b["seq_lens"])
    inside = (c.b["positions"].astype(np.int64) * 3 // 4).astype(np.int32)
    for pos in (c.b["positions"], inside):
        lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
        out = kap.decode_attn(c.q, t(pos), c.K, c.V, cbt, clen, G=1, lse=lse, logical=clog)
        torch.cuda.synchronize()
        ref, lref = oracle.attend(c.b["q"][:, None], pos, c.Kl, c.Vl, c.btl, keys, 1, w.Hkv)
        err = _check_attn(c, out, lse, ref[:, 0], lref[:, 0])
        print(f"[eight-page items, D {D}] max rel err {err:.2e}", flush=True)


def test_values_beyond_the_fp16_range():
    """The split partials are bf16 outputs normalized by their own sums, so
    they keep the range of the KV values: with every V value scaled by 2^17
    (up to about 1e5, past fp16's 65504, exact in bf16) the selected decode,
    the full decode and a 4-token verify still match the oracle."""
    w = W.spec("qwen32b_128k", B=2, seq_lens=[8192, 6001])
    c = Case(w)
    scale = np.float32(2.0 ** 17)
    vl = (oracle.widen(c.Vl).astype(np.float32) * scale)
    assert np.nanmax(np.abs(vl)) > 65504.0
    vbits = W.gen._to_bf16_bits(vl)
    assert np.array_equal(oracle.widen(vbits)[np.isfinite(vl)], vl[np.isfinite(vl)].astype(np.float64))
    phys = torch.from_numpy(c.b["phys"].astype(np.int64)).cuda()
    V = torch.zeros_like(c.V)
    V[phys] = t(vbits)
    cap = c.budget()
    sel, cnt = oracle.select(oracle.score(c.b["q"], c.b["positions"], c.summ_l, c.btl,
                                          c.b["seq_lens"], w.Hkv).astype(np.float32),
                             c.b["seq_lens"], c.b["anchor"], c.b["recent"], c.k_mid_h, cap)
    cbt, clog, clen, _ = kap.compact_view(t(sel), t(cnt), c.bt, c.L, c.pos, 1)
    for name, keys, tab in (("selected", oracle.keys_selected(sel, cnt, c.b["seq_lens"]), (cbt, clen, clog)),
                            ("full", oracle.keys_full(c.b["seq_lens"]), (c.bt, c.L, None))):
        lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
        out = kap.decode_attn(c.q, c.pos, c.K, V, tab[0], tab[1], G=1, lse=lse, logical=tab[2])
        torch.cuda.synchronize()
        ref, lref = oracle.attend(c.b["q"][:, None], c.b["positions"], c.Kl, vbits, c.btl, keys, 1,
                                  w.Hkv)
        err = _check_attn(c, out, lse, ref[:, 0], lref[:, 0])
        print(f"[V x 2^17, {name} decode] max rel err {err:.2e}", flush=True)
    vl_ = torch.empty((w.B, w.q_len, w.Hq), dtype=torch.float32, device="cuda")
    vout = kap.verify_attn(c.qv, c.pos, c.K, V, c.bt, c.L, lse=vl_)
    torch.cuda.synchronize()
    ref, lref = oracle.attend(c.b["qv"], c.b["positions"], c.Kl, vbits, c.btl,
                              oracle.keys_full(c.b["seq_lens"]), 1, w.Hkv)
    err = _check_attn(c, vout, vl_, ref, lref)
    print(f"[V x 2^17, verify] max rel err {err:.2e}", flush=True)


@pytest.mark.parametrize("Hq,Hkv,D,dtype", [
    (8, 8, 128, "bf16"),     # MHA: one query row per KV head
    (16, 1, 64, "bf16"),     # MQA, head_dim 64
    (128, 8, 128, "bf16"),   # GQA 16:1 (decode 16 rows, verify 64 rows per KV head)
    (32, 8, 64, "f32"),      # fp32 path, head_dim 64, verify 64 rows (two 32-row slices)
    (32, 16, 128, "bf16"),   # 16 KV heads: the widest pooled-scoring block
    (32, 32, 64, "bf16"),    # 32 KV heads: per-head scores from the one-head-per-block kernel
])
def test_head_layouts(Hq, Hkv, D, dtype):
    """Score (per head and pooled), top-K, selected decode and a 16-token verify on
    other head shapes."""
    over = dict(B=2, seq_lens=[3000, 1777], Hq=Hq, Hkv=Hkv, D=D, q_len=16, dtype=dtype)
    if dtype == "f32":
        over["sigma"] = 1.0 / 8.0
    c = Case(W.spec("llama8b_32k", **over))
    w = c.w
    s = kap.score_blocks(c.q, c.pos, c.S, c.bt, c.L, w.Hkv)
    torch.cuda.synchronize()
    check_scores(c, s.cpu().numpy())
    if w.Hkv <= 16:
        _check_pooled(c)
    else:
        with pytest.raises(kap.KapError) as ei:
            kap.score_pool_blocks(c.q, c.pos, c.S, c.bt, c.L, w.Hkv)
        assert ei.value.status == 2
    cap = c.budget()
    s_ref = oracle.score(c.b["q"], c.b["positions"], c.summ_l, c.btl, c.b["seq_lens"], w.Hkv)
    sel_ref, cnt_ref = oracle.select(s_ref.astype(np.float32), c.b["seq_lens"], c.b["anchor"],
                                     c.b["recent"], c.k_mid_h, cap)
    sel, cnt = kap.select_topk(t(s_ref.astype(np.float32)), c.L, c.anchor, c.recent, c.k_mid, cap,
                               cap)
    cbt, clog, clen, _ = kap.compact_view(sel, cnt, c.bt, c.L, c.pos, 1)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
    out = kap.decode_attn(c.q, c.pos, c.K, c.V, cbt, clen, lse=lse, logical=clog)
    start = np.maximum(c.b["positions"] - 9, 0).astype(np.int32)
    vlse = torch.empty((w.B, w.q_len, w.Hq), dtype=torch.float32, device="cuda")
    vout = kap.verify_attn(c.qv, t(start), c.K, c.V, c.bt, c.L, lse=vlse)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sel.cpu().numpy(), sel_ref)
    keys = oracle.keys_selected(sel_ref, cnt_ref, c.b["seq_lens"])
    ref, lref = oracle.attend(c.b["q"][:, None], c.b["positions"], c.Kl, c.Vl, c.btl, keys, 1,
                              w.Hkv)
    e1 = _check_attn(c, out, lse, ref[:, 0], lref[:, 0])
    vref, vlref = oracle.attend(c.b["qv"], start, c.Kl, c.Vl, c.btl,
                                oracle.keys_full(c.b["seq_lens"]), 1, w.Hkv)
    e2 = _check_attn(c, vout, vlse, vref, vlref)
    print(f"[Hq {Hq} Hkv {Hkv} D {D} {dtype}] decode {e1:.2e} verify {e2:.2e}", flush=True)


def test_verify_window_k_plus_one():
    """The KAP paper's verify window is k+1 tokens (carry + k drafts): q_len 5 on the tiny case."""
    w = W.spec("tiny", q_len=5)
    c = Case(w)
    out = kap.verify_attn(c.qv, c.pos, c.K, c.V, c.bt, c.L)
    torch.cuda.synchronize()
    ref, _ = oracle.attend(c.b["qv"], c.b["positions"], c.Kl, c.Vl, c.btl,
                           oracle.keys_full(c.b["seq_lens"]), 1, w.Hkv)
    assert row_errors(host(out, False), ref).max() <= TOL["f32"]


# ----------------------------------------------------------------------------- invariants
def test_full_selection_is_bit_identical_to_full_decode():
    """s = 1: the compact view is the full table, so the result is bit-identical."""
    c = get_case("llama")
    w = c.w
    N = w.n_pages
    kall = t(N.astype(np.int32))
    cap = int(N.max())
    sel, cnt = kap.select_topk(kap.score_blocks(c.q, c.pos, c.S, c.bt, c.L, w.Hkv), c.L, c.anchor,
                               c.recent, kall, cap, cap)
    cbt, clog, clen, _ = kap.compact_view(sel, cnt, c.bt, c.L, c.pos, 1)
    o_sel = kap.decode_attn(c.q, c.pos, c.K, c.V, cbt, clen, logical=clog)
    o_full = kap.decode_attn(c.q, c.pos, c.K, c.V, c.bt, c.L)
    torch.cuda.synchronize()
    assert np.array_equal(clen.cpu().numpy()[:, 0], c.b["seq_lens"])
    assert torch.equal(o_sel, o_full)


def test_placement_invariance_and_determinism():
    """Moving pages in the pool (table moved with them), placing the K and V pools
    in one allocation (kap_kv_pool_layout) and re-running change no bit."""
    c = get_case("qwen")
    pool = c.K.shape[0]
    g = torch.Generator().manual_seed(7)
    perm = torch.randperm(pool, generator=g).cuda()
    inv = torch.argsort(perm)
    K2, V2 = c.K[perm].contiguous(), c.V[perm].contiguous()
    bt2 = torch.where(c.bt >= 0, inv[c.bt.clamp(min=0).long()].int(), c.bt).contiguous()
    o1 = kap.verify_attn(c.qv, c.pos, c.K, c.V, c.bt, c.L)
    o2 = kap.verify_attn(c.qv, c.pos, K2, V2, bt2, c.L)
    o3 = kap.verify_attn(c.qv, c.pos, c.K, c.V, c.bt, c.L)
    d1 = kap.decode_attn(c.q, c.pos, c.K, c.V, c.bt, c.L)
    d2 = kap.decode_attn(c.q, c.pos, K2, V2, bt2, c.L)
    K3, V3 = kap.copy_kv_pools(c.K, c.V)
    v_off, _ = kap.kv_pool_layout(pool, c.w.Hkv, c.w.D, 2)
    assert V3.data_ptr() - K3.data_ptr() == v_off
    o4 = kap.verify_attn(c.qv, c.pos, K3, V3, c.bt, c.L)
    d3 = kap.decode_attn(c.q, c.pos, K3, V3, c.bt, c.L)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(o1, o3) and torch.equal(d1, d2)
    assert torch.equal(o1, o4) and torch.equal(d1, d3)


# ----------------------------------------------------------------------------- edge cases
def test_adversarial_selection_keys():
    """Ties, +-0, +-inf and NaN keys: GPU top-K equals the oracle's bit for bit."""
    rng = np.random.default_rng(21)
    palette = np.array([0.0, -0.0, 1.0, -1.0, 2.5, np.inf, -np.inf, np.nan, 1.0, 0.5], np.float32)
    B, H, P = 6, 4, 3000
    S = palette[rng.integers(0, len(palette), size=(B, H, P))]
    L = np.array([16 * 3000, 16 * 2999 + 1, 100, 16 * 5, 1, 0], np.int32)
    a = np.array([1, 4, 0, 2, 0, 1], np.int32)
    r = np.array([2, 4, 3, 3, 0, 0], np.int32)
    k = np.array([110, 1000, 2, 0, 5, 3], np.int32)
    cap = 2000
    for per_head in (False, True):
        sel, cnt = kap.select_topk(t(S), t(L), t(a), t(r), t(k), int((a + r + k).max()), cap,
                                   per_head=per_head)
        torch.cuda.synchronize()
        sref, cref = oracle.select(S, L, a, r, k, cap, per_head=per_head)
        np.testing.assert_array_equal(sel.cpu().numpy(), sref)
        np.testing.assert_array_equal(cnt.cpu().numpy(), cref)


def test_select_radix_exits():
    """The top-K's radix passes stop once the chosen bin holds exactly the keys
    still needed.  Three key families reach each exit: one key per power of two
    (decided by the first 12-bit digit), normal draws (usually decided by the
    second digit), and a threshold inside a run of equal keys (all three
    digits, then the tie ranks).  Bit-exact against the oracle, per head and
    pooled."""
    rng = np.random.default_rng(25)
    B, H, P = 3, 2, 4096
    S = np.empty((B, H, P), np.float32)
    # row 0: 4000 keys with distinct top 12 bits (sign, exponent, 3 mantissa
    # bits), then -inf
    sgn, ex, m3 = np.meshgrid([-1.0, 1.0], np.arange(-124, 126), np.arange(8), indexing="ij")
    vals = (sgn * np.exp2(ex.astype(np.float64)) * (1.0 + m3 / 8.0)).ravel().astype(np.float32)
    for h in range(H):
        S[0, h] = np.concatenate([rng.permutation(vals), np.full(P - vals.size, -np.inf, np.float32)])
    S[1] = rng.standard_normal((H, P)).astype(np.float32)
    S[2] = np.where(rng.random((H, P)) < 0.3, np.float32(1.5), rng.standard_normal((H, P)).astype(np.float32))
    L = np.full(B, 16 * P, np.int32)
    a, r = np.full(B, 1, np.int32), np.full(B, 2, np.int32)
    k = np.array([300, 448, 700], np.int32)
    cap = 1024
    for per_head in (True, False):
        sel, cnt = kap.select_topk(t(S), t(L), t(a), t(r), t(k), cap, cap, per_head=per_head)
        torch.cuda.synchronize()
        sref, cref = oracle.select(S, L, a, r, k, cap, per_head=per_head)
        np.testing.assert_array_equal(sel.cpu().numpy(), sref)
        np.testing.assert_array_equal(cnt.cpu().numpy(), cref)


@pytest.mark.parametrize("P", [3000, 12000])
def test_select_small_takes(P):
    """Small middle counts (per-head early routing takes 8): takes 0..17 on
    adversarial keys (ties, +-0, +-inf, NaN), normal draws and a threshold
    inside a run of equal keys, one take per request, with tables staged in
    LDS (3000 pages) and read directly (12000 pages).  Bit-exact against the
    oracle, per head and pooled, and through the fused top-K with compact
    view."""
    rng = np.random.default_rng(31 + P)
    palette = np.array([0.0, -0.0, 1.0, -1.0, 2.5, np.inf, -np.inf, np.nan, 1.0, 0.5], np.float32)
    takes = np.array([1, 2, 3, 7, 8, 15, 16, 17, 8, 5, 16, 0], np.int32)
    B, H = len(takes), 4
    S = np.empty((B, H, P), np.float32)
    for i in range(B):
        fam = i % 3
        if fam == 0:
            S[i] = palette[rng.integers(0, len(palette), size=(H, P))]
        elif fam == 1:
            S[i] = rng.standard_normal((H, P)).astype(np.float32)
        else:
            S[i] = np.where(rng.random((H, P)) < 0.3, np.float32(1.5),
                            rng.standard_normal((H, P)).astype(np.float32) - 3.0)
    L = np.full(B, 16 * P, np.int32)
    L[3] = 16 * (P - 7) + 5                    # a short row with a partial last page
    a = np.array([1, 0, 2, 1, 0, 4, 1, 1, 0, 3, 1, 2], np.int32)
    r = np.array([2, 0, 3, 2, 1, 4, 2, 2, 0, 3, 2, 2], np.int32)
    cap = 64
    for per_head in (True, False):
        sel, cnt = kap.select_topk(t(S), t(L), t(a), t(r), t(takes), cap, cap, per_head=per_head)
        torch.cuda.synchronize()
        sref, cref = oracle.select(S, L, a, r, takes, cap, per_head=per_head)
        np.testing.assert_array_equal(sel.cpu().numpy(), sref)
        np.testing.assert_array_equal(cnt.cpu().numpy(), cref)
    bt = np.stack([rng.permutation(4 * P)[:P] for _ in range(B)]).astype(np.int32)
    pos = L.copy()
    cnt2, cv = kap.select_compact(t(S), t(L), t(a), t(r), t(takes), cap, cap, t(bt), t(pos), 1,
                                  per_head=True)
    torch.cuda.synchronize()
    sref, cref = oracle.select(S, L, a, r, takes, cap, per_head=True)
    np.testing.assert_array_equal(cv[1].cpu().numpy(), sref)
    np.testing.assert_array_equal(cnt2.cpu().numpy(), cref)


def test_select_compact_matches_the_two_calls():
    """kap_select_compact writes exactly what kap_select_topk then kap_compact_view
    write, and what the oracle's selection then compaction give, on adversarial
    keys, ragged and empty rows, unallocated table entries, a window past the
    table, and rows the device budget truncates to the capacity."""
    _select_compact_case(22, 3000)


def test_select_compact_on_a_long_table():
    """Past 11264 pages the keys are not staged in LDS: the other load path."""
    _select_compact_case(23, 12500)


def test_select_compact_at_the_widest_table():
    """65536 pages (a 1M-token context), the widest row the top-K takes."""
    _select_compact_case(24, 65536)


def test_attention_at_the_row_limit():
    """4096 (request, KV head) rows, the most one attention call takes: past 512
    rows the plan reads row lengths outside its register cache, and the rows
    outnumber the work-item target, so most rows are one item.  512 ragged
    requests of 0-399 tokens (empty, 1- and 16-token rows among them), GQA 2:1,
    8 KV heads, D 64: full-table decode, selected decode over per-head compact
    tables, and a 2-token verify."""
    rng = np.random.default_rng(31)
    L = rng.integers(0, 400, size=512)
    L[:3] = [0, 1, 16]
    w = W.spec("llama8b_32k", B=512, seq_lens=[int(x) for x in L], Hq=16, D=64, needles=0,
               q_len=2, per_head=True, k_mid=5)
    c = Case(w)
    b = c.b
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
    out = kap.decode_attn(c.q, c.pos, c.K, c.V, c.bt, c.L, G=1, lse=lse)
    torch.cuda.synchronize()
    ref, lref = oracle.attend(b["q"][:, None], b["positions"], c.Kl, c.Vl, c.btl,
                              oracle.keys_full(b["seq_lens"]), 1, w.Hkv)
    e_full = _check_attn(c, out, lse, ref[:, 0], lref[:, 0])
    cap = c.budget()
    _, sel_ref, cnt_ref = _oracle_chain(c, cap)
    cbt, clog, clen, slot = kap.compact_view(t(sel_ref), t(cnt_ref), c.bt, c.L, c.pos, 1)
    out = kap.decode_attn(c.q, c.pos, c.K, c.V, cbt, clen, G=w.Hkv, lse=lse, logical=clog)
    torch.cuda.synchronize()
    keys = oracle.keys_selected(sel_ref, cnt_ref, b["seq_lens"])
    ref, lref = oracle.attend(b["q"][:, None], b["positions"], c.Kl, c.Vl, c.btl, keys, w.Hkv, w.Hkv)
    e_sel = _check_attn(c, out, lse, ref[:, 0], lref[:, 0])
    start = np.maximum(b["positions"] - 1, 0).astype(np.int32)
    vlse = torch.empty((w.B, w.q_len, w.Hq), dtype=torch.float32, device="cuda")
    vout = kap.verify_attn(c.qv, t(start), c.K, c.V, c.bt, c.L, lse=vlse)
    torch.cuda.synchronize()
    vref, vlref = oracle.attend(b["qv"], start, c.Kl, c.Vl, c.btl,
                                oracle.keys_full(b["seq_lens"]), 1, w.Hkv)
    e_ver = _check_attn(c, vout, vlse, vref, vlref)
    print(f"[4096 rows] max rel err: full {e_full:.2e} selected {e_sel:.2e} verify {e_ver:.2e}",
          flush=True)


def _select_compact_case(seed, P):
    rng = np.random.default_rng(seed)
    palette = np.array([0.0, -0.0, 1.0, -1.0, 2.5, np.inf, -np.inf, np.nan, 1.0, 0.5], np.float32)
    B, H = 6, 4
    S = palette[rng.integers(0, len(palette), size=(B, H, P))]
    L = np.array([16 * P, 16 * (P - 1) + 1, 100, 16 * 5, 1, 0], np.int32)
    a = np.array([1, 4, 0, 2, 0, 1], np.int32)
    r = np.array([2, 4, 3, 3, 0, 0], np.int32)
    k = np.array([110, 1000, 2, 0, 5, 3], np.int32)
    bt = np.stack([rng.permutation(B * P)[:P] for _ in range(B)]).astype(np.int32)
    bt[1, P - 1] = -1                                  # an unallocated last page
    pos = L.copy()                                     # request 0's window lies past its table
    q_new = 5
    for per_head in (False, True):
        for cap in (2000, 600):                        # 600: request 1's 1008 pages are cut
            sel, cnt = kap.select_topk(t(S), t(L), t(a), t(r), t(k), cap, cap, per_head=per_head)
            cv = kap.compact_view(sel, cnt, t(bt), t(L), t(pos), q_new)
            cnt2, cv2 = kap.select_compact(t(S), t(L), t(a), t(r), t(k), cap, cap, t(bt), t(pos),
                                           q_new, per_head=per_head)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(cnt2.cpu().numpy(), cnt.cpu().numpy())
            np.testing.assert_array_equal(cv2[1].cpu().numpy(), sel.cpu().numpy())
            for x, y in zip(cv2, cv):
                np.testing.assert_array_equal(x.cpu().numpy(), y.cpu().numpy())
            # and the oracle's selection then compaction, on the same host arrays
            sref, cref = oracle.select(S, L, a, r, k, cap, per_head=per_head)
            ref = oracle.compact(sref, cref, bt, L, pos, q_new)
            np.testing.assert_array_equal(cnt2.cpu().numpy(), cref)
            for x, y in zip(cv2, ref):
                np.testing.assert_array_equal(x.cpu().numpy(), y)
            if cap == 600:
                assert int(cnt.cpu().numpy()[1].max()) == 600


def test_empty_and_single_token_rows():
    w = W.spec("llama8b_32k", B=3, seq_lens=[0, 1, 17], needles=0)
    c = Case(w)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
    out = kap.decode_attn(c.q, c.pos, c.K, c.V, c.bt, c.L, lse=lse)
    vlse = torch.empty((w.B, w.q_len, w.Hq), dtype=torch.float32, device="cuda")
    vout = kap.verify_attn(c.qv, c.pos, c.K, c.V, c.bt, c.L, lse=vlse)
    scores = kap.score_blocks(c.q, c.pos, c.S, c.bt, c.L, w.Hkv)
    sel, cnt = kap.select_topk(scores, c.L, c.anchor, c.recent, c.k_mid, c.budget(), c.budget())
    torch.cuda.synchronize()
    o = host(out, True)
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse.cpu().numpy()[0]))
    ref, lref = oracle.attend(c.b["q"][:, None], c.b["positions"], c.Kl, c.Vl, c.btl,
                              oracle.keys_full(c.b["seq_lens"]), 1, w.Hkv)
    assert row_errors(o[1:], ref[1:, 0]).max() <= TOL["bf16"]
    vref, _ = oracle.attend(c.b["qv"], c.b["positions"], c.Kl, c.Vl, c.btl,
                            oracle.keys_full(c.b["seq_lens"]), 1, w.Hkv)
    assert row_errors(host(vout, True), vref).max() <= TOL["bf16"]
    assert cnt.cpu().numpy().ravel().tolist() == [0, 1, 2]
    assert np.all(np.isneginf(scores.cpu().numpy()[0]))


def test_capacity_error_is_the_fallback_cue():
    c = get_case("tiny")
    s = kap.score_blocks(c.q, c.pos, c.S, c.bt, c.L, c.w.Hkv)
    with pytest.raises(kap.KapError) as ei:
        kap.select_topk(s, c.L, c.anchor, c.recent, c.k_mid, max_budget=8, capacity=7)
    assert ei.value.status == 3


def test_summary_builder_matches_oracle():
    c = get_case("mixed")
    S2 = torch.zeros_like(c.S)
    kap.build_summary(c.K, c.bt, c.L, S2)
    torch.cuda.synchronize()
    got = oracle.widen(S2.cpu().numpy().view(np.uint16))[c.b["phys"]]
    ref = oracle.summary(c.Kl, c.btl, c.b["seq_lens"])
    used = np.zeros(len(c.b["phys"]), bool)
    for bi in range(c.w.B):
        used[c.btl[bi, :int(c.w.n_pages[bi])]] = True
    # one bf16 rounding of a value that differs from the fp64 mean by fp32 summation error
    d = np.abs(got[used] - ref[used])
    assert np.all(d <= np.abs(ref[used]) * 2.0 ** -8 + 1e-6)


def test_proxy_query_and_per_head_routing():
    """Early routing: proxy query GEMV -> per-head scores -> per-head top-8 -> decode."""
    w = W.spec("early_route_40k", B=2, seq_lens=[40000, 23456])
    c = Case(w)
    hid, wq = t(c.b["hidden"]), t(c.b["wq"])
    qp = kap.proxy_query(hid, wq)
    torch.cuda.synchronize()
    qref = oracle.proxy_query(c.b["hidden"], c.b["wq"])
    e = np.abs(qp.cpu().numpy() - qref).max(axis=1) / np.linalg.norm(qref, axis=1)
    assert e.max() <= 1e-5
    # per-head routing on the proxy query (oracle chain from the oracle's own proxy query)
    Hq, D = w.Hq, w.D
    q32 = qp.view(w.B, Hq, D).contiguous()
    scores = kap.score_blocks(q32, c.pos, c.S, c.bt, c.L, w.Hkv)
    qref32 = qref.astype(np.float32).reshape(w.B, Hq, D)
    s_ref = oracle.score(qref32, c.b["positions"], c.summ_l, c.btl, c.b["seq_lens"], w.Hkv)
    torch.cuda.synchronize()
    s_gpu = scores.cpu().numpy()
    N = w.n_pages
    for bi in range(w.B):
        n = int(N[bi])
        scale = np.abs(s_ref[bi, :, :n]).max()
        assert np.abs(s_gpu[bi, :, :n] - s_ref[bi, :, :n]).max() <= 1e-4 * scale
    cap = 8
    sel_ref, cnt_ref = oracle.select(s_ref.astype(np.float32), c.b["seq_lens"], 0, 0, 8, cap,
                                     per_head=True)
    sel, cnt = kap.select_topk(t(s_ref.astype(np.float32)), c.L, c.anchor, c.recent, c.k_mid, 8,
                               cap, per_head=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sel.cpu().numpy(), sel_ref)
    cbt, clog, clen, _ = kap.compact_view(sel, cnt, c.bt, c.L, c.pos, 1)
    out = kap.decode_attn(c.q, c.pos, c.K, c.V, cbt, clen, G=w.Hkv, logical=clog)
    torch.cuda.synchronize()
    keys = oracle.keys_selected(sel_ref, cnt_ref, c.b["seq_lens"])
    ref, _ = oracle.attend(c.b["q"][:, None], c.b["positions"], c.Kl, c.Vl, c.btl, keys, w.Hkv,
                           w.Hkv)
    assert row_errors(host(out, True), ref[:, 0]).max() <= TOL["bf16"]


def _packed_index(dm, n_out):
    """Position in the packed weight of every W_q element (r, c), from the
    layout kap.h states."""
    r = np.arange(dm)[:, None]
    c = np.arange(n_out)[None, :]
    return (((((c // 16) * (dm // 32) + r // 32) * 4 + (r % 32) // 8) * 16 + c % 16) * 8 + r % 8)


@pytest.mark.parametrize("B,dm,n_out", [(1, 32, 16), (5, 96, 528), (3, 640, 1024), (8, 4096, 4096),
                                        (16, 8192, 256), (7, 4128, 48)])
def test_proxy_query_packed(B, dm, n_out):
    """Packed W_q: the packing is a permutation (bit-exact against the stated
    index), and the one-launch GEMV over it is within 1e-5 |q| of the oracle
    per batch row, deterministic, and agrees with the row-major two-launch
    kernel to fp32 rounding where both apply.  Shapes cover one k-step per
    wave with idle waves (d_model 32, 96), several rounds per wave (8192),
    a share that ends mid-round (4128: 129 steps over 8 waves of 17), and
    batch rows padded to 16."""
    rng = np.random.default_rng(2000 + B + dm)
    hidden = W.gen._to_bf16_bits(rng.standard_normal((B, dm)).astype(np.float32))
    wq = W.gen._to_bf16_bits((rng.standard_normal((dm, n_out)) / 64).astype(np.float32))
    wq_d = t(wq)
    packed = kap.proxy_pack_weights(wq_d)
    q1 = kap.proxy_query_packed(t(hidden), packed, n_out)
    q2 = kap.proxy_query_packed(t(hidden), packed, n_out)
    torch.cuda.synchronize()
    want = np.empty(dm * n_out, dtype=np.uint16)
    want[_packed_index(dm, n_out).ravel()] = wq.ravel()
    np.testing.assert_array_equal(packed.cpu().numpy().view(np.uint16), want)
    assert torch.equal(q1, q2)
    ref = oracle.proxy_query(hidden, wq)
    e = np.abs(q1.cpu().numpy() - ref).max(axis=1) / np.linalg.norm(ref, axis=1)
    assert e.max() <= 1e-5, e.max()
    if dm % 128 == 0 and n_out % 512 == 0:
        q3 = kap.proxy_query(t(hidden), wq_d)
        torch.cuda.synchronize()
        d = (q1 - q3).abs().max(dim=1).values / q3.norm(dim=1)
        assert d.max().item() <= 1e-6


@pytest.mark.parametrize("B,dm,n_out", [(1, 4096, 4096), (3, 256, 512), (8, 4096, 4096),
                                        (16, 1024, 1536), (5, 640, 1024)])
def test_proxy_query_shapes(B, dm, n_out):
    """The proxy GEMV on the matrix cores: batch rows padded to 16 (B = 1, 3,
    5, 8, 16), row splits of 128 added in groups of four (d_model 256 and 640
    end in a partial group), column tiles of 128; within 1e-5 |q| of the
    oracle's fp64 sum of exact bf16 products, per batch row."""
    rng = np.random.default_rng(1000 + B)
    hidden = W.gen._to_bf16_bits(rng.standard_normal((B, dm)).astype(np.float32))
    wq = W.gen._to_bf16_bits((rng.standard_normal((dm, n_out)) / 64).astype(np.float32))
    qp = kap.proxy_query(t(hidden), t(wq))
    torch.cuda.synchronize()
    ref = oracle.proxy_query(hidden, wq)
    e = np.abs(qp.cpu().numpy() - ref).max(axis=1) / np.linalg.norm(ref, axis=1)
    assert e.max() <= 1e-5, e.max()
