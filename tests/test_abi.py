"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

import block_sparse_paged_page_amd as kap

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kap.h")

OK, INVALID, UNSUPPORTED, CAPACITY, WORKSPACE = 0, 1, 2, 3, 4
NP = ctypes.c_void_p(0x1000)   # a non-null pointer that validation never dereferences


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^KAP_API\s+[\w\s\*]*?\b(kap_\w+)\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return kap.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version(lib):
    assert lib.kap_status_string(0) == b"ok"
    assert b"capacity" in lib.kap_status_string(3)
    assert b"gfx950" in lib.kap_version()


def test_budget_helper_matches_closed_forms(lib):
    assert kap.budget_from_ratio(2048, 55, 1000, 1, 2) == 113
    assert kap.budget_from_ratio(8192, 55, 1000, 1, 2) == 451
    assert kap.budget_from_ratio(100, 1, 100, 4, 4) == 8
    assert kap.budget_from_ratio(7, 1, 1, 1, 2) == 7
    assert kap.budget_from_ratio(-1, 1, 1, 0, 0) == -1


def test_budget_helper_agrees_with_oracle(lib):
    import oracle
    for N in (1, 7, 100, 2000, 2048, 8192, 65536):
        for num, den in ((1, 100), (55, 1000), (25, 100), (1, 1), (0, 1)):
            for a, r in ((1, 2), (4, 4), (0, 0)):
                assert kap.budget_from_ratio(N, num, den, a, r) == oracle.budget_from_ratio(N, num, den, a, r)


def test_kv_pool_layout(lib):
    # K at byte 0, V at the K pool's bytes rounded up to 16 KiB plus 4 KiB
    for pages, hkv, d, eb in ((32772, 8, 128, 2), (1, 1, 64, 4), (0, 8, 128, 2), (4096, 8, 128, 2),
                              (12345, 4, 64, 2)):
        kb = pages * hkv * d * 16 * eb
        v_off, total = kap.kv_pool_layout(pages, hkv, d, eb)
        assert v_off % 16384 == 4096 and kb <= v_off < kb + 16384 + 4096
        assert total == v_off + kb
    assert kap.kv_pool_layout(32772, 8, 128, 2) == (1073876992, 2147749888)
    out = ctypes.c_int64(0)
    for args, st in (((-1, 8, 128, 16, 2), INVALID), ((10, 0, 128, 16, 2), INVALID),
                     ((10, 8, 128, 16, 3), INVALID), ((10, 8, 96, 16, 2), UNSUPPORTED),
                     ((10, 8, 128, 8, 2), UNSUPPORTED), ((1 << 60, 8, 128, 16, 2), INVALID)):
        assert lib.kap_kv_pool_layout(*args, ctypes.byref(out), ctypes.byref(out)) == st, args
    assert lib.kap_kv_pool_layout(10, 8, 128, 16, 2, None, ctypes.byref(out)) == INVALID


def _score(lib, **kw):
    args = dict(q=NP, q_dtype=1, positions=NP, theta=1e4, summary=NP, sum_dtype=1, num_pages=10,
                bt=NP, max_pages=4, seq_lens=NP, B=1, Hq=8, Hkv=2, D=128, page_size=16,
                scores=NP)
    args.update(kw)
    return lib.kap_score_blocks(args["q"], args["q_dtype"], args["positions"], args["theta"],
                                args["summary"], args["sum_dtype"], args["num_pages"], args["bt"],
                                args["max_pages"], args["seq_lens"], args["B"], args["Hq"],
                                args["Hkv"], args["D"], args["page_size"], args["scores"], None)


def test_score_validation(lib):
    assert _score(lib, D=96) == UNSUPPORTED
    assert _score(lib, page_size=32) == UNSUPPORTED
    assert _score(lib, Hq=6, Hkv=4) == UNSUPPORTED
    assert _score(lib, q_dtype=7) == UNSUPPORTED
    assert _score(lib, B=-1) == INVALID
    assert _score(lib, theta=0.5) == INVALID
    assert _score(lib, q=None) == INVALID
    assert b"null" in lib.kap_last_error()
    assert _score(lib, B=0) == OK   # empty batch: nothing to do, no launch


def _score_pool(lib, **kw):
    args = dict(q=NP, q_dtype=1, positions=NP, theta=1e4, summary=NP, sum_dtype=1, num_pages=10,
                bt=NP, max_pages=4, seq_lens=NP, B=1, Hq=8, Hkv=2, D=128, page_size=16,
                scores=None, pooled=NP)
    args.update(kw)
    return lib.kap_score_pool_blocks(args["q"], args["q_dtype"], args["positions"], args["theta"],
                                     args["summary"], args["sum_dtype"], args["num_pages"],
                                     args["bt"], args["max_pages"], args["seq_lens"], args["B"],
                                     args["Hq"], args["Hkv"], args["D"], args["page_size"],
                                     args["scores"], args["pooled"], None)


def test_score_pool_validation(lib):
    assert _score_pool(lib, D=96) == UNSUPPORTED
    assert _score_pool(lib, Hq=6, Hkv=4) == UNSUPPORTED
    assert _score_pool(lib, Hq=32, Hkv=32) == UNSUPPORTED          # more than 16 KV heads
    assert b"Hkv" in lib.kap_last_error()
    assert _score_pool(lib, Hq=256, Hkv=16, q_dtype=0) == UNSUPPORTED  # 128 KiB of fp32 queries
    assert _score_pool(lib, pooled=None) == INVALID                # neither output given
    assert _score_pool(lib, q=None) == INVALID
    assert _score_pool(lib, theta=0.5) == INVALID
    assert _score_pool(lib, B=0) == OK


def test_select_validation(lib):
    def sel(**kw):
        a = dict(scores=NP, B=2, Hkv=8, max_pages=2048, seq_lens=NP, page_size=16, per_head=0,
                 anchor=NP, recent=NP, k_mid=NP, budget=113, cap=128, sel=NP, cnt=NP)
        a.update(kw)
        return lib.kap_select_topk(a["scores"], a["B"], a["Hkv"], a["max_pages"], a["seq_lens"],
                                   a["page_size"], a["per_head"], a["anchor"], a["recent"],
                                   a["k_mid"], a["budget"], a["cap"], a["sel"], a["cnt"], None)
    assert sel(budget=129) == CAPACITY          # the fallback cue
    assert b"capacity" in lib.kap_last_error()
    assert sel(max_pages=70000) == UNSUPPORTED
    assert sel(max_pages=65537) == UNSUPPORTED  # one past the widest row the top-K takes
    assert sel(per_head=2) == INVALID
    assert sel(k_mid=None) == INVALID
    assert sel(B=0) == OK


def test_select_compact_validation(lib):
    def call(**kw):
        args = dict(scores=NP, B=2, Hkv=8, max_pages=100, L=NP, ps=16, per_head=0, a=NP, r=NP, k=NP,
                    budget=10, cap=10, bt=NP, pos=NP, q_new=1, cnt=NP, cbt=NP, clog=NP, clen=NP,
                    slot=NP)
        args.update(kw)
        return lib.kap_select_compact(*args.values(), None)
    assert call(budget=11) == CAPACITY
    assert call(ps=8) == UNSUPPORTED
    assert call(max_pages=70000) == UNSUPPORTED
    assert call(per_head=2) == INVALID
    assert call(q_new=-1) == INVALID
    assert call(bt=None) == INVALID
    assert call(slot=None) == INVALID                 # q_new > 0 needs an output
    assert b"slot" in lib.kap_last_error()
    assert call(B=0) == OK


def test_compact_validation(lib):
    def cv(**kw):
        a = dict(sel=NP, cnt=NP, B=1, G=1, cap=8, bt=NP, max_pages=8, seq_lens=NP, page_size=16,
                 pos=NP, q_new=1, cbt=NP, clog=NP, clen=NP, slot=NP)
        a.update(kw)
        return lib.kap_compact_view(a["sel"], a["cnt"], a["B"], a["G"], a["cap"], a["bt"],
                                    a["max_pages"], a["seq_lens"], a["page_size"], a["pos"],
                                    a["q_new"], a["cbt"], a["clog"], a["clen"], a["slot"], None)
    assert cv(slot=None) == INVALID
    assert cv(G=0) == INVALID
    assert cv(page_size=8) == UNSUPPORTED
    assert cv(B=0) == OK


def _attn(lib, fn, **kw):
    a = dict(q=NP, q_dtype=1, pos=NP, q_len=4, theta=1e4, scale=0.088, k=NP, v=NP, kv_dtype=1,
             num_pages=100, Hkv=8, D=128, page_size=16, table=NP, width=64, G=1, lens=NP, B=2,
             Hq=64, out=NP, lse=None, ws=NP, ws_bytes=1 << 40)
    a.update(kw)
    if fn == "decode":
        return lib.kap_decode_attn(a["q"], a["q_dtype"], a["pos"], a["theta"], a["scale"], a["k"],
                                   a["v"], a["kv_dtype"], a["num_pages"], a["Hkv"], a["D"],
                                   a["page_size"], a["table"], None, a["width"], a["G"], a["lens"],
                                   a["B"], a["Hq"], a["out"], a["lse"], a["ws"], a["ws_bytes"],
                                   None)
    return lib.kap_verify_attn(a["q"], a["q_dtype"], a["pos"], a["q_len"], a["theta"], a["scale"],
                               a["k"], a["v"], a["kv_dtype"], a["num_pages"], a["Hkv"], a["D"],
                               a["page_size"], a["table"], a["width"], a["lens"], a["B"], a["Hq"],
                               a["out"], a["lse"], a["ws"], a["ws_bytes"], None)


def test_attention_validation(lib):
    for fn in ("decode", "verify"):
        assert _attn(lib, fn, D=256) == UNSUPPORTED
        assert _attn(lib, fn, q_dtype=0) == UNSUPPORTED       # q and KV dtypes differ
        assert _attn(lib, fn, Hq=60) == UNSUPPORTED
        assert _attn(lib, fn, ws_bytes=16) == WORKSPACE
        assert _attn(lib, fn, ws=None) == WORKSPACE
        assert _attn(lib, fn, out=None) == INVALID
        assert _attn(lib, fn, scale=0.0) == INVALID
        assert _attn(lib, fn, B=0) == OK
    assert _attn(lib, "verify", q_len=17) == UNSUPPORTED
    for fn in ("decode", "verify"):                            # more than 4096 (request, KV head) rows
        assert _attn(lib, fn, B=513, Hkv=8, Hq=64) == UNSUPPORTED
        assert _attn(lib, fn, B=4097, Hkv=1, Hq=8) == UNSUPPORTED
    assert _attn(lib, "decode", G=3) == INVALID
    odd = ctypes.c_void_p(0x1008)                              # 8-byte but not 16-byte aligned
    for fn in ("decode", "verify"):
        for arg in ("q", "k", "v", "out", "ws"):
            assert _attn(lib, fn, **{arg: odd}) == INVALID, (fn, arg)


def test_bulk_pointers_must_be_16_byte_aligned(lib):
    odd = ctypes.c_void_p(0x1008)
    assert _score(lib, q=odd) == INVALID
    assert _score(lib, summary=odd) == INVALID
    assert lib.kap_proxy_query(odd, NP, 1, 4096, 4096, NP, NP, 1 << 30, None) == INVALID
    assert lib.kap_proxy_query(NP, NP, 1, 4096, 4096, NP, odd, 1 << 30, None) == INVALID
    assert lib.kap_proxy_pack_weights(NP, 4096, 4096, odd, None) == INVALID
    assert lib.kap_proxy_query_packed(NP, odd, 1, 4096, 4096, NP, None) == INVALID
    assert lib.kap_diag_stream_read(odd, 1 << 20, NP, None) == INVALID


def test_workspace_sizes_are_monotone(lib):
    a = kap.attn_workspace_bytes(1, 1, 64, 8, 128)
    b = kap.attn_workspace_bytes(4, 4, 64, 8, 128)
    assert 0 < a < b
    assert kap.attn_workspace_bytes(0, 1, 8, 2, 64) == 0
    # one partial per group of four 128-row splits of W_q
    assert kap.proxy_workspace_bytes(8, 4096, 4096) == (4096 // 128 // 4) * 8 * 4096 * 4
    assert kap.proxy_workspace_bytes(3, 640, 512) == 2 * 3 * 512 * 4


def test_proxy_validation(lib):
    f = lib.kap_proxy_query
    assert f(NP, NP, 0, 4096, 4096, NP, NP, 1 << 30, None) == UNSUPPORTED
    assert f(NP, NP, 17, 4096, 4096, NP, NP, 1 << 30, None) == UNSUPPORTED
    assert f(NP, NP, 1, 1000, 4096, NP, NP, 1 << 30, None) == UNSUPPORTED
    assert f(NP, NP, 1, 4096, 4000, NP, NP, 1 << 30, None) == UNSUPPORTED
    assert f(NP, NP, 1, 4096, 4096, NP, NP, 16, None) == WORKSPACE
    pk, pq = lib.kap_proxy_pack_weights, lib.kap_proxy_query_packed
    assert pk(NP, 4016, 4096, ctypes.c_void_p(0x2000), None) == UNSUPPORTED   # d_model % 32
    assert pk(NP, 4096, 4088, ctypes.c_void_p(0x2000), None) == UNSUPPORTED   # n_out % 16
    assert pk(None, 4096, 4096, NP, None) == INVALID
    assert pk(NP, 4096, 4096, NP, None) == INVALID                            # in place
    assert pq(NP, NP, 0, 4096, 4096, NP, None) == UNSUPPORTED
    assert pq(NP, NP, 17, 4096, 4096, NP, None) == UNSUPPORTED
    assert pq(NP, NP, 1, 48, 4096, NP, None) == UNSUPPORTED
    assert pq(NP, NP, 1, 4096, 40, NP, None) == UNSUPPORTED
    assert pq(NP, None, 1, 4096, 4096, NP, None) == INVALID


def test_append_and_summary_update_validation(lib):
    ap = lib.kap_append_kv
    #        k_new v_new dt slot B  q  Hkv  D   ps  pages k   v   stream
    assert ap(NP, NP, 1, NP, 2, 5, 8, 96, 16, 100, NP, NP, None) == UNSUPPORTED
    assert ap(NP, NP, 1, NP, 2, 5, 8, 128, 32, 100, NP, NP, None) == UNSUPPORTED
    assert ap(NP, NP, 5, NP, 2, 5, 8, 128, 16, 100, NP, NP, None) == UNSUPPORTED
    assert ap(NP, NP, 1, None, 2, 5, 8, 128, 16, 100, NP, NP, None) == INVALID
    assert ap(NP, NP, 1, NP, -1, 5, 8, 128, 16, 100, NP, NP, None) == INVALID
    assert ap(None, None, 1, None, 0, 5, 8, 128, 16, 100, None, None, None) == OK  # nothing to do
    up = lib.kap_update_summary
    #        k  dt pages Hkv D   ps  bt  maxp lens pos q  B  summ sdt stream
    assert up(NP, 1, 100, 8, 128, 16, NP, 64, NP, None, 5, 2, NP, 1, None) == INVALID
    assert up(NP, 1, 100, 8, 64, 8, NP, 64, NP, NP, 5, 2, NP, 1, None) == UNSUPPORTED
    assert up(NP, 1, 100, 8, 128, 16, NP, 64, NP, NP, -1, 2, NP, 1, None) == INVALID
    assert up(None, 1, 100, 8, 128, 16, None, 64, None, None, 0, 2, None, 1, None) == OK


def test_materialize_validation(lib):
    m = lib.kap_materialize_view
    #        k   v  dt pages Hkv D   ps cbt  B  G  cap kws vws wsp tab stream
    assert m(NP, NP, 1, 100, 8, 128, 16, NP, 2, 1, 10, NP, NP, 19, NP, None) == WORKSPACE
    assert m(NP, NP, 1, 100, 8, 128, 16, NP, 2, 3, 10, NP, NP, 20, NP, None) == INVALID
    assert m(NP, NP, 1, 100, 8, 96, 16, NP, 2, 1, 10, NP, NP, 20, NP, None) == UNSUPPORTED
    assert m(NP, NP, 1, 100, 8, 128, 16, None, 2, 1, 10, NP, NP, 20, NP, None) == INVALID
    assert m(None, None, 1, 100, 8, 128, 16, None, 0, 1, 10, None, None, 0, None, None) == OK


def test_product_binding_never_imports_oracle():
    pkg = os.path.join(ROOT, "block_sparse_paged_page_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, fn)).read()
                assert "import oracle" not in text and "from oracle" not in text, fn
                assert "kap_oracle" not in text and "liboracle" not in text, fn


def test_noalloc_decode_rejects_oversize_before_any_hip_call(lib):
    """The allocation-free decode holds its split-K partials in a static
    scratch of KAP_NOALLOC_SCRATCH_BYTES; a call that needs more is refused
    with KAP_ERR_WORKSPACE before any HIP call (so this runs without a GPU)."""
    text = open(HEADER).read()
    m = re.search(r"#define KAP_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    cap = int(m.group(1)) << int(m.group(2))
    B, Hq, Hkv, D = 512, 128, 8, 128
    assert kap.attn_workspace_bytes(B, 1, Hq, Hkv, D) > cap
    st = lib.kap_decode_attn_noalloc(NP, 1, NP, 1e4, 0.088, NP, NP, 1, 100, Hkv, D, 16, NP, None,
                                     64, 1, NP, B, Hq, NP, None, None)
    assert st == WORKSPACE
    assert b"scratch" in lib.kap_last_error()
    assert kap.attn_workspace_bytes(4, 1, 64, 8, 128) <= cap   # the 128K, B = 4 decode fits
