"""Parity at the workloads' full sizes, in the launch configuration bench.py times.

K/V are drawn on the GPU by the seeded device generator; the oracle gets host
copies of exactly the pages and KV head it needs and computes sampled output
rows (one KV group of one request at a time).  Routing (scores, selection,
compaction) is checked on every page.
"""
import numpy as np
import pytest
import torch

import block_sparse_paged_page_amd as kap
import oracle
import workloads as W
from _gpu_util import LSE_TOL, TOL, row_errors

pytestmark = pytest.mark.gpu


def _u16(x: torch.Tensor) -> np.ndarray:
    return x.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _pools(pages, Hkv, D, dtype, device):
    return kap.alloc_kv_pools(pages, Hkv, D, dtype, device, zero=True)


class Big:
    def __init__(self, w):
        self.w = w
        dev = torch.device("cuda:0")
        self.b = b = W.make_device(w, dev, alloc_pools=_pools)  # placed as bench.py places them
        to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
        self.bt, self.L, self.pos = to(b["bt"]), to(b["seq_lens"]), to(b["positions"])
        self.anchor, self.recent = to(b["anchor"]), to(b["recent"])
        if "k_mid" in b:
            self.k_mid_h = b["k_mid"]
        else:
            N = w.n_pages
            self.k_mid_h = np.array([
                oracle.budget_from_ratio(int(N[i]), r[0], r[1], int(b["anchor"][i]),
                                         int(b["recent"][i])) - int(b["anchor"][i]) - int(b["recent"][i])
                for i, r in enumerate(b["ratio"])], dtype=np.int32)
        self.k_mid = to(self.k_mid_h)
        self.q = to(b["q"].view(np.int16))
        self.qv = to(b["qv"].view(np.int16))
        self.K, self.V = b["K"], b["V"]
        self.S = torch.zeros((b["pool_pages"], w.Hkv, w.D), dtype=torch.bfloat16, device=dev)
        kap.build_summary(self.K, self.bt, self.L, self.S)
        NA = w.alloc_pages
        self.starts = np.concatenate([[0], np.cumsum(NA)[:-1]]).astype(np.int64)
        torch.cuda.synchronize()

    def budget(self):
        return int((self.b["anchor"] + self.b["recent"] + self.k_mid_h).max())

    def pages(self, bi):
        NA = self.w.alloc_pages
        return self.b["phys"][self.starts[bi]:self.starts[bi] + NA[bi]]

    def host_group(self, bi, g):
        """Request bi's allocated pages of KV head g, local table, oracle summary rows."""
        ph = torch.from_numpy(self.pages(bi).astype(np.int64)).cuda()
        Kh = _u16(self.K[ph][:, g:g + 1])
        Vh = _u16(self.V[ph][:, g:g + 1])
        btl = np.arange(len(ph), dtype=np.int32)[None]
        return Kh, Vh, btl

    def host_selected(self, bi, g, lpages):
        """K/V of KV head g on request bi's logical pages `lpages` only, with a
        full-width local table whose entry for each of those pages points at
        its local copy (the other entries are never read: the key list holds
        only tokens of those pages)."""
        allp = self.pages(bi)
        ph = torch.from_numpy(allp[lpages].astype(np.int64)).cuda()
        Kh = _u16(self.K[ph][:, g:g + 1])
        Vh = _u16(self.V[ph][:, g:g + 1])
        btl = np.zeros((1, len(allp)), dtype=np.int32)
        btl[0, lpages] = np.arange(len(lpages), dtype=np.int32)
        return Kh, Vh, btl

    def host_summary(self, bi):
        """oracle summary of request bi (all heads), rounded to bf16, local page order."""
        ph = torch.from_numpy(self.pages(bi).astype(np.int64)).cuda()
        Kh = _u16(self.K[ph])
        btl = np.arange(len(ph), dtype=np.int32)[None]
        s = oracle.summary(Kh, btl, self.b["seq_lens"][bi:bi + 1])
        return oracle.round_to_bf16(s), btl


def _routing(big):
    """GPU routing vs oracle routing on every page: scores within tolerance,
    top-K bit-exact on the oracle's scores, compaction bit-exact."""
    w, b = big.w, big.b
    cap = big.budget()
    # both sides score the oracle's summary rows; the GPU summary builder is
    # checked against them separately (one bf16 rounding apart at most)
    S_o = torch.zeros_like(big.S)
    summs = []
    for bi in range(w.B):
        summ, btl = big.host_summary(bi)
        summs.append((summ, btl))
        ph = torch.from_numpy(big.pages(bi).astype(np.int64)).cuda()
        n = int(w.n_pages[bi])
        S_o[ph[:n]] = torch.from_numpy(summ[:n].view(np.int16)).cuda().view(torch.bfloat16)
        got = oracle.widen(_u16(big.S[ph[:n]]))
        want = oracle.widen(summ[:n])
        assert np.all(np.abs(got - want) <= np.abs(want) * 2.0 ** -7 + 1e-30), f"summary, request {bi}"
    scores = kap.score_blocks(big.q, big.pos, S_o, big.bt, big.L, w.Hkv)
    torch.cuda.synchronize()
    s_gpu = scores.cpu().numpy()
    max_pages = b["bt"].shape[1]
    s_ref = np.full((w.B, w.Hkv, max_pages), -np.inf)
    grp = w.Hq // w.Hkv
    for bi in range(w.B):
        summ, btl = summs[bi]
        btl_full = np.full((1, max_pages), -1, np.int32)
        btl_full[0, :btl.shape[1]] = btl[0]
        s_ref[bi] = oracle.score(b["q"][bi:bi + 1], b["positions"][bi:bi + 1], summ, btl_full,
                                 b["seq_lens"][bi:bi + 1], w.Hkv)[0]
        n = int(w.n_pages[bi])
        qr = oracle.rope(oracle.widen(b["q"][bi]), float(b["positions"][bi]))
        un = np.linalg.norm(qr.reshape(w.Hkv, grp, w.D).sum(axis=1), axis=1)
        rn = np.linalg.norm(oracle.widen(summ[:n]), axis=-1)          # [n][Hkv]
        bound = 1e-5 * un[:, None] * rn.T + 1e-30
        assert np.all(np.abs(s_gpu[bi, :, :n] - s_ref[bi, :, :n]) <= bound), f"scores, request {bi}"
        assert np.all(np.isneginf(s_gpu[bi, :, n:]))
    s32 = s_ref.astype(np.float32)
    sel_ref, cnt_ref = oracle.select(s32, b["seq_lens"], b["anchor"], b["recent"], big.k_mid_h, cap,
                                     per_head=w.per_head)
    sel, cnt = kap.select_topk(torch.from_numpy(s32).cuda(), big.L, big.anchor, big.recent,
                               big.k_mid, cap, cap, per_head=w.per_head)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sel.cpu().numpy(), sel_ref)
    np.testing.assert_array_equal(cnt.cpu().numpy(), cnt_ref)
    cv = kap.compact_view(sel, cnt, big.bt, big.L, big.pos, 1)
    torch.cuda.synchronize()
    r = oracle.compact(sel_ref, cnt_ref, b["bt"], b["seq_lens"], b["positions"], 1)
    for got, want in zip(cv, r):
        np.testing.assert_array_equal(got.cpu().numpy(), want)
    # the one-launch top-K + compact view on the same scores
    cnt2, cv2 = kap.select_compact(torch.from_numpy(s32).cuda(), big.L, big.anchor, big.recent,
                                   big.k_mid, cap, cap, big.bt, big.pos, 1, per_head=w.per_head)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(cnt2.cpu().numpy(), cnt_ref)
    for got, want in zip(cv2, r):
        np.testing.assert_array_equal(got.cpu().numpy(), want)
    if not w.per_head:
        # the bench's route: pooled key folded in the scoring launch, top-K on it
        s2, pooled = kap.score_pool_blocks(big.q, big.pos, S_o, big.bt, big.L, w.Hkv)
        cnt3, cv3 = kap.select_compact(pooled.view(w.B, 1, -1), big.L, big.anchor, big.recent,
                                       big.k_mid, cap, cap, big.bt, big.pos, 1)
        torch.cuda.synchronize()
        s2h = s2.cpu().numpy()
        np.testing.assert_array_equal(s2h.view(np.uint32), s_gpu.view(np.uint32))
        fold = s2h[:, 0].copy()
        for g in range(1, w.Hkv):
            fold = fold + s2h[:, g]
        fold = fold / np.float32(w.Hkv)
        np.testing.assert_array_equal(pooled.cpu().numpy().view(np.uint32), fold.view(np.uint32))
        sel4, cnt4 = oracle.select(s2h, b["seq_lens"], b["anchor"], b["recent"], big.k_mid_h, cap)
        r4 = oracle.compact(sel4, cnt4, b["bt"], b["seq_lens"], b["positions"], 1)
        np.testing.assert_array_equal(cnt3.cpu().numpy(), cnt4)
        for got, want in zip(cv3, r4):
            np.testing.assert_array_equal(got.cpu().numpy(), want)
    return sel_ref, cnt_ref, cv


def _check_rows(big, out, lse, samples, keys_for, qsrc, q_len, start, host_for=None):
    """Oracle on the given (request, KV group) pairs: every query row of each."""
    w, b = big.w, big.b
    grp = w.Hq // w.Hkv
    o = out.view(torch.int16).cpu().numpy().view(np.uint16)
    lg = lse.cpu().numpy()
    worst = 0.0
    for bi, g in samples:
        Kh, Vh, btl = host_for(bi, g) if host_for else big.host_group(bi, g)
        qsub = qsrc[bi:bi + 1, :, g * grp:(g + 1) * grp]
        ref, lref = oracle.attend(qsub, start[bi:bi + 1], Kh, Vh, btl, [keys_for(bi, g)], 1, 1)
        got = oracle.widen(o.reshape(w.B, q_len, w.Hq, w.D)[bi, :, g * grp:(g + 1) * grp])
        e = row_errors(got, ref[0])
        worst = max(worst, float(e.max()))
        d = np.abs(lg.reshape(w.B, q_len, w.Hq)[bi, :, g * grp:(g + 1) * grp] - lref[0]).max()
        assert d <= LSE_TOL["bf16"], (bi, g, d)
    assert worst <= TOL["bf16"], worst
    return worst


def _attention(big, sel_ref, cnt_ref, cv, sel_requests=None, samples=()):
    """Selected decode on every KV group of the requests `sel_requests` (all
    requests by default; only their selected pages go to the host); full decode
    and verify on every KV group of request 0 and every request of KV group 0,
    plus `samples`."""
    w, b = big.w, big.b
    G = w.Hkv if w.per_head else 1
    sel_requests = range(w.B) if sel_requests is None else sel_requests
    sel_rows = [(bi, g) for bi in sel_requests for g in range(w.Hkv)]
    samples = sorted(set([(0, g) for g in range(w.Hkv)] + [(bi, 0) for bi in range(w.B)] +
                         list(samples)))
    cbt, clog, clen, _ = cv
    ws = torch.empty(kap.attn_workspace_bytes(w.B, w.q_len, w.Hq, w.Hkv, w.D), dtype=torch.uint8,
                     device="cuda")
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
    out = kap.decode_attn(big.q, big.pos, big.K, big.V, cbt, clen, G=G, lse=lse, workspace=ws,
                          logical=clog)
    torch.cuda.synchronize()
    keys_sel = oracle.keys_selected(sel_ref, cnt_ref, b["seq_lens"])
    row = lambda bi, g: bi * G + (g if G > 1 else 0)  # noqa: E731
    e1 = _check_rows(big, out, lse, sel_rows, lambda bi, g: keys_sel[row(bi, g)],
                     b["q"][:, None], 1, b["positions"],
                     host_for=lambda bi, g: big.host_selected(
                         bi, g, sel_ref[bi, row(bi, g) % G, :cnt_ref[bi, row(bi, g) % G]]))
    out = kap.decode_attn(big.q, big.pos, big.K, big.V, big.bt, big.L, G=1, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    e2 = _check_rows(big, out, lse, samples,
                     lambda bi, g: np.arange(int(b["seq_lens"][bi]), dtype=np.int32),
                     b["q"][:, None], 1, b["positions"])
    e3 = 0.0
    if w.q_len > 1:
        vl = torch.empty((w.B, w.q_len, w.Hq), dtype=torch.float32, device="cuda")
        vout = kap.verify_attn(big.qv, big.pos, big.K, big.V, big.bt, big.L, lse=vl, workspace=ws)
        torch.cuda.synchronize()
        e3 = _check_rows(big, vout, vl, samples,
                         lambda bi, g: np.arange(int(b["seq_lens"][bi]), dtype=np.int32),
                         b["qv"], w.q_len, b["positions"])
    print(f"[{w.name}] max rel err: selected {e1:.2e} ({len(sel_rows)} rows), full {e2:.2e} and "
          f"verify {e3:.2e} ({len(samples)} rows)", flush=True)


def test_qwen32b_128k_b4_full_size():
    """The benchmarked configuration: 4 x 131072 tokens, 64/8 heads, s = 451/8192."""
    big = Big(W.spec("qwen32b_128k", B=4))
    sel_ref, cnt_ref, cv = _routing(big)
    assert np.all(cnt_ref == 451)
    _attention(big, sel_ref, cnt_ref, cv, samples=[(1, 3), (2, 7), (3, 5)])


def test_llama8b_32k_b8_full_size():
    big = Big(W.spec("llama8b_32k"))
    sel_ref, cnt_ref, cv = _routing(big)
    assert np.all(cnt_ref == 113)
    _attention(big, sel_ref, cnt_ref, cv, samples=[(3, 4), (7, 7)])


def test_mixed_serving_b64_full_size():
    """64 ragged requests (4K-128K) scattered over the 1,525,878-page (100 GB) pool."""
    big = Big(W.spec("mixed_serving"))
    sel_ref, cnt_ref, cv = _routing(big)
    L = big.b["seq_lens"]
    order = np.argsort(L)
    # every KV group of 8 requests across the length range for the selected
    # decode; request 0 and KV group 0 in full for the full decode
    span = [int(order[i]) for i in np.linspace(0, len(order) - 1, 8).round().astype(int)]
    samples = [(int(order[0]), 0), (int(order[len(order) // 2]), 5), (int(order[-1]), 7)]
    _attention(big, sel_ref, cnt_ref, cv, sel_requests=span, samples=samples)
    del big
    torch.cuda.empty_cache()


def test_early_route_40k_b8_full_size():
    """Proxy query (4096 x 4096 W_q) -> per-head scores -> per-head top-8 -> decode."""
    w = W.spec("early_route_40k", B=8)
    big = Big(w)
    b = big.b
    hid, wq = torch.from_numpy(b["hidden"].view(np.int16)).cuda(), torch.from_numpy(b["wq"].view(np.int16)).cuda()
    qp = kap.proxy_query(hid, wq)
    torch.cuda.synchronize()
    qref = oracle.proxy_query(b["hidden"], b["wq"])
    e = np.abs(qp.cpu().numpy() - qref).max(axis=1) / np.linalg.norm(qref, axis=1)
    assert e.max() <= 1e-5
    sel_ref, cnt_ref, cv = _routing(big)
    assert np.all(cnt_ref == 8)
    _attention(big, sel_ref, cnt_ref, cv, samples=[(5, 6)])


def test_qwen32b_128k_b4_append_and_causal_verify():
    """The k+1 = 5 token window at 131072..131076: its K/V appended through the
    slot mapping, then the causal verify over 131077 tokens, sampled rows."""
    w = W.spec("qwen32b_128k", B=4, q_len=5)
    big = Big(w)
    b = big.b
    kn, vn = W.draft_kv(w)
    samples = [(0, 2), (3, 6)]
    hosts = {s: big.host_group(*s) for s in samples}     # oracle copies, taken before the append
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    sel, cnt = np.full((w.B, 1, 1), -1, np.int32), np.zeros((w.B, 1), np.int32)
    slot = kap.compact_view(to(sel), to(cnt), big.bt, big.L, big.pos, w.q_len)[3]
    kap.append_kv(to(kn.view(np.int16)), to(vn.view(np.int16)), slot, big.K, big.V)
    L2 = (b["seq_lens"] + w.q_len).astype(np.int32)
    ws = torch.empty(kap.attn_workspace_bytes(w.B, w.q_len, w.Hq, w.Hkv, w.D), dtype=torch.uint8,
                     device="cuda")
    vl = torch.empty((w.B, w.q_len, w.Hq), dtype=torch.float32, device="cuda")
    vout = kap.verify_attn(big.qv, big.pos, big.K, big.V, big.bt, to(L2), lse=vl, workspace=ws)
    torch.cuda.synchronize()
    s_ref = oracle.compact(sel, cnt, b["bt"], b["seq_lens"], b["positions"], w.q_len)[3]
    np.testing.assert_array_equal(slot.cpu().numpy(), s_ref)
    grp = w.Hq // w.Hkv
    o = vout.view(torch.int16).cpu().numpy().view(np.uint16).reshape(w.B, w.q_len, w.Hq, w.D)
    lg = vl.cpu().numpy()
    worst = 0.0
    for (bi, g), (Kh, Vh, btl) in hosts.items():
        P = int(b["positions"][bi])
        local_slot = np.arange(P, P + w.q_len, dtype=np.int64)[None]   # pages in logical order
        oracle.append_kv(kn[bi:bi + 1, :, g:g + 1], vn[bi:bi + 1, :, g:g + 1], local_slot, Kh, Vh)
        qsub = b["qv"][bi:bi + 1, :, g * grp:(g + 1) * grp]
        ref, lref = oracle.attend(qsub, b["positions"][bi:bi + 1], Kh, Vh, btl,
                                  [np.arange(int(L2[bi]), dtype=np.int32)], 1, 1)
        got = oracle.widen(o[bi, :, g * grp:(g + 1) * grp])
        worst = max(worst, float(row_errors(got, ref[0]).max()))
        assert np.abs(lg[bi, :, g * grp:(g + 1) * grp] - lref[0]).max() <= LSE_TOL["bf16"]
    assert worst <= TOL["bf16"], worst
    print(f"[qwen32b_128k append] causal verify over 131077 tokens max rel err {worst:.2e}", flush=True)
