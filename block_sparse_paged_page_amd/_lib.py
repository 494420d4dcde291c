"""ctypes binding of libkap.so; argument marshalling only."""
import ctypes
import math
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# KAP_LIB may name another build of the same library (e.g. for side-by-side timing)
_LIB = os.environ.get("KAP_LIB") or os.path.join(_HERE, "libkap.so")

F32, BF16 = 0, 1
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "capacity", 4: "workspace",
           5: "HIP error"}


class KapLibraryMissing(RuntimeError):
    pass


class KapError(RuntimeError):
    def __init__(self, status, what, detail):
        self.status = status
        super().__init__(f"{what}: {_STATUS.get(status, status)}: {detail}")


_P, _I32, _I64, _F, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "kap_status_string": ([_I32], ctypes.c_char_p),
    "kap_last_error": ([], ctypes.c_char_p),
    "kap_version": ([], ctypes.c_char_p),
    "kap_score_blocks": ([_P, _I32, _P, _F, _P, _I32, _I32, _P, _I32, _P, _I32, _I32, _I32, _I32,
                          _I32, _P, _P], _I32),
    "kap_score_pool_blocks": ([_P, _I32, _P, _F, _P, _I32, _I32, _P, _I32, _P, _I32, _I32, _I32,
                               _I32, _I32, _P, _P, _P], _I32),
    "kap_proxy_workspace_bytes": ([_I32, _I32, _I32], _SZ),
    "kap_proxy_query": ([_P, _P, _I32, _I32, _I32, _P, _P, _SZ, _P], _I32),
    "kap_proxy_pack_weights": ([_P, _I32, _I32, _P, _P], _I32),
    "kap_proxy_query_packed": ([_P, _P, _I32, _I32, _I32, _P, _P], _I32),
    "kap_select_topk": ([_P, _I32, _I32, _I32, _P, _I32, _I32, _P, _P, _P, _I32, _I32, _P, _P, _P],
                        _I32),
    "kap_select_compact": ([_P, _I32, _I32, _I32, _P, _I32, _I32, _P, _P, _P, _I32, _I32, _P, _P,
                            _I32, _P, _P, _P, _P, _P, _P], _I32),
    "kap_budget_from_ratio": ([_I32, _I64, _I64, _I32, _I32], _I32),
    "kap_kv_pool_layout": ([_I64, _I32, _I32, _I32, _I32, _P, _P], _I32),
    "kap_choose_plan": ([ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.c_double, _I32,
                         _I32, _I32, _P, _P], _I32),
    "kap_compact_view": ([_P, _P, _I32, _I32, _I32, _P, _I32, _P, _I32, _P, _I32, _P, _P, _P, _P,
                          _P], _I32),
    "kap_attn_workspace_bytes": ([_I32, _I32, _I32, _I32, _I32], _SZ),
    "kap_decode_attn": ([_P, _I32, _P, _F, _F, _P, _P, _I32, _I32, _I32, _I32, _I32, _P, _P, _I32,
                         _I32, _P, _I32, _I32, _P, _P, _P, _SZ, _P], _I32),
    "kap_decode_attn_noalloc": ([_P, _I32, _P, _F, _F, _P, _P, _I32, _I32, _I32, _I32, _I32, _P,
                                 _P, _I32, _I32, _P, _I32, _I32, _P, _P, _P], _I32),
    "kap_verify_attn": ([_P, _I32, _P, _I32, _F, _F, _P, _P, _I32, _I32, _I32, _I32, _I32, _P, _I32,
                         _P, _I32, _I32, _P, _P, _P, _SZ, _P], _I32),
    "kap_diag_stream_read": ([_P, _SZ, _P, _P], _I32),
    "kap_build_summary": ([_P, _I32, _I32, _I32, _I32, _I32, _P, _I32, _P, _I32, _P, _I32, _P], _I32),
    "kap_update_summary": ([_P, _I32, _I32, _I32, _I32, _I32, _P, _I32, _P, _P, _I32, _I32, _P, _I32,
                            _P], _I32),
    "kap_append_kv": ([_P, _P, _I32, _P, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _P], _I32),
    "kap_materialize_view": ([_P, _P, _I32, _I32, _I32, _I32, _I32, _P, _I32, _I32, _I32, _P, _P,
                              _I32, _P, _P], _I32),
    "kap_host_proxy_query": ([_P, _P, _I32, _I32, _I32, _P, _I32], _I32),
    "kap_host_score_blocks": ([_P, _P, ctypes.c_float, _P, _I32, _P, _I32, _P, _I32, _I32, _I32,
                               _I32, _I32, _P, _I32], _I32),
    "kap_host_select_topk": ([_P, _I32, _I32, _I32, _P, _I32, _I32, _P, _P, _P, _I32, _P, _P,
                              _I32], _I32),
}
_lib = None


def lib_path() -> str:
    return _LIB


def load():
    """Load libkap.so (built in-tree by __graft_entry__.build()); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        raise KapLibraryMissing(
            f"{_LIB} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(_LIB)
    for name, (args, res) in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def version() -> str:
    return load().kap_version().decode()


def _check(status, what):
    if status != 0:
        raise KapError(status, what, load().kap_last_error().decode())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return BF16
    raise TypeError(f"unsupported element type {t.dtype}")


def _p(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def attn_workspace_bytes(B, q_len, Hq, Hkv, D) -> int:
    return int(load().kap_attn_workspace_bytes(B, q_len, Hq, Hkv, D))


def proxy_workspace_bytes(B, d_model, n_out) -> int:
    return int(load().kap_proxy_workspace_bytes(B, d_model, n_out))


def budget_from_ratio(n_pages, s_num, s_den, anchor, recent) -> int:
    return int(load().kap_budget_from_ratio(n_pages, s_num, s_den, anchor, recent))


def kv_pool_layout(num_pages, Hkv, D, elem_bytes=2, page_size=16):
    """kap_kv_pool_layout -> (v_offset_bytes, total_bytes): one allocation holding
    a layer's K pool at byte 0 and its V pool at v_offset_bytes."""
    v_off, total = ctypes.c_int64(-1), ctypes.c_int64(-1)
    st = load().kap_kv_pool_layout(num_pages, Hkv, D, page_size, elem_bytes, ctypes.byref(v_off),
                                   ctypes.byref(total))
    _check(st, "kap_kv_pool_layout")
    return int(v_off.value), int(total.value)


def alloc_kv_pools(num_pages, Hkv, D, dtype=torch.bfloat16, device="cuda", zero=False):
    """A layer's K pool [num_pages][Hkv][16][D] and V pool [num_pages][Hkv][D][16]
    as views of one allocation placed by kap_kv_pool_layout."""
    eb = torch.empty((), dtype=dtype).element_size()
    v_off, total = kv_pool_layout(num_pages, Hkv, D, eb)
    buf = (torch.zeros if zero else torch.empty)(total, dtype=torch.uint8, device=device)
    n = num_pages * Hkv * 16 * D * eb
    k = buf[:n].view(dtype).view(num_pages, Hkv, 16, D)
    v = buf[v_off:v_off + n].view(dtype).view(num_pages, Hkv, D, 16)
    return k, v


def copy_kv_pools(k_pool, v_pool):
    """Copies of a layer's K and V pools in one allocation (kap_kv_pool_layout)."""
    num_pages, Hkv, ps, D = k_pool.shape
    k, v = alloc_kv_pools(num_pages, Hkv, D, k_pool.dtype, k_pool.device)
    k.copy_(k_pool)
    v.copy_(v_pool)
    return k, v


PLAN_SELECTED, PLAN_FULL_CAPACITY, PLAN_FULL_MARGIN, PLAN_FULL_BOUNDARY = 0, 1, 2, 3


def choose_plan(h, s, w_main_bytes, kv_bytes, k, budget_pages, capacity):
    """kap_choose_plan -> (choice, modeled cycle speedup Cost_base / Cost_plan)."""
    choice = ctypes.c_int32(-1)
    speedup = ctypes.c_double(0.0)
    st = load().kap_choose_plan(float(h), float(s), float(w_main_bytes), float(kv_bytes), int(k),
                                int(budget_pages), int(capacity), ctypes.byref(choice),
                                ctypes.byref(speedup))
    _check(st, "kap_choose_plan")
    return choice.value, speedup.value


def score_blocks(q, positions, summary, block_table, seq_lens, Hkv, theta=1e4, scores=None,
                 stream=None):
    """kap_score_blocks: q [B][Hq][D] -> scores [B][Hkv][max_pages] float32."""
    lib = load()
    B, Hq, D = q.shape
    max_pages = block_table.shape[1]
    if scores is None:
        scores = torch.empty((B, Hkv, max_pages), dtype=torch.float32, device=q.device)
    st = lib.kap_score_blocks(_p(q), _dt(q), _p(positions), float(theta), _p(summary),
                              _dt(summary), summary.shape[0], _p(block_table), max_pages,
                              _p(seq_lens), B, Hq, Hkv, D, 16, _p(scores), _stream(stream))
    _check(st, "kap_score_blocks")
    return scores


def score_pool_blocks(q, positions, summary, block_table, seq_lens, Hkv, theta=1e4,
                      scores=None, pooled=None, with_scores=True, stream=None):
    """kap_score_pool_blocks: per-head scores [B][Hkv][max_pages] (or None when
    with_scores is False) and the head-pooled key [B][max_pages], float32."""
    lib = load()
    B, Hq, D = q.shape
    max_pages = block_table.shape[1]
    if scores is None and with_scores:
        scores = torch.empty((B, Hkv, max_pages), dtype=torch.float32, device=q.device)
    if pooled is None:
        pooled = torch.empty((B, max_pages), dtype=torch.float32, device=q.device)
    st = lib.kap_score_pool_blocks(_p(q), _dt(q), _p(positions), float(theta), _p(summary),
                                   _dt(summary), summary.shape[0], _p(block_table), max_pages,
                                   _p(seq_lens), B, Hq, Hkv, D, 16,
                                   _p(scores), _p(pooled),
                                   _stream(stream))
    _check(st, "kap_score_pool_blocks")
    return scores, pooled


def proxy_query(hidden, w_q, q_out=None, workspace=None, stream=None):
    """kap_proxy_query: hidden [B][d_model] bf16 @ w_q [d_model][n_out] bf16 -> fp32."""
    lib = load()
    B, dm = hidden.shape
    n_out = w_q.shape[1]
    if q_out is None:
        q_out = torch.empty((B, n_out), dtype=torch.float32, device=hidden.device)
    need = proxy_workspace_bytes(B, dm, n_out)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=hidden.device)
    st = lib.kap_proxy_query(_p(hidden), _p(w_q), B, dm, n_out, _p(q_out), _p(workspace),
                             workspace.numel(), _stream(stream))
    _check(st, "kap_proxy_query")
    return q_out


def proxy_pack_weights(w_q, out=None, stream=None):
    """kap_proxy_pack_weights: the packed copy of a row-major bf16 w_q [d_model][n_out]
    (same element count, returned flat) for proxy_query_packed."""
    lib = load()
    dm, n_out = w_q.shape
    if out is None:
        out = torch.empty(dm * n_out, dtype=w_q.dtype, device=w_q.device)
    if out.numel() != dm * n_out or out.element_size() != 2:
        raise ValueError("packed output must hold d_model * n_out 16-bit values")
    st = lib.kap_proxy_pack_weights(_p(w_q), dm, n_out, _p(out), _stream(stream))
    _check(st, "kap_proxy_pack_weights")
    return out


def proxy_query_packed(hidden, w_packed, n_out, q_out=None, stream=None):
    """kap_proxy_query_packed: hidden [B][d_model] bf16 @ W_q (packed by
    proxy_pack_weights) -> fp32 [B][n_out], one launch."""
    lib = load()
    B, dm = hidden.shape
    if w_packed.numel() != dm * n_out:
        raise ValueError("packed weight size does not match d_model * n_out")
    if q_out is None:
        q_out = torch.empty((B, n_out), dtype=torch.float32, device=hidden.device)
    st = lib.kap_proxy_query_packed(_p(hidden), _p(w_packed), B, dm, n_out, _p(q_out),
                                    _stream(stream))
    _check(st, "kap_proxy_query_packed")
    return q_out


def select_topk(scores, seq_lens, anchor, recent, k_mid, max_budget, capacity, per_head=False,
                sel=None, cnt=None, stream=None):
    """kap_select_topk -> (sel [B][G][capacity] int32, cnt [B][G] int32)."""
    lib = load()
    B, Hkv, max_pages = scores.shape
    G = Hkv if per_head else 1
    if sel is None:
        sel = torch.empty((B, G, capacity), dtype=torch.int32, device=scores.device)
    if cnt is None:
        cnt = torch.empty((B, G), dtype=torch.int32, device=scores.device)
    st = lib.kap_select_topk(_p(scores), B, Hkv, max_pages, _p(seq_lens), 16, int(bool(per_head)),
                             _p(anchor), _p(recent), _p(k_mid), int(max_budget), int(capacity),
                             _p(sel), _p(cnt), _stream(stream))
    _check(st, "kap_select_topk")
    return sel, cnt


def compact_view(sel, cnt, block_table, seq_lens, positions, q_new, out=None, stream=None):
    """kap_compact_view -> (compact_bt, compact_logical, compact_len, slot_mapping)."""
    lib = load()
    B, G, cap = sel.shape
    dev = sel.device
    if out is None:
        out = (torch.empty((B, G, cap), dtype=torch.int32, device=dev),
               torch.empty((B, G, cap), dtype=torch.int32, device=dev),
               torch.empty((B, G), dtype=torch.int32, device=dev),
               torch.empty((B, max(q_new, 1)), dtype=torch.int64, device=dev))
    cbt, clog, clen, slot = out
    st = lib.kap_compact_view(_p(sel), _p(cnt), B, G, cap, _p(block_table), block_table.shape[1],
                              _p(seq_lens), 16, _p(positions), int(q_new), _p(cbt), _p(clog),
                              _p(clen), _p(slot), _stream(stream))
    _check(st, "kap_compact_view")
    return cbt, clog, clen, slot


def select_compact(scores, seq_lens, anchor, recent, k_mid, max_budget, capacity, block_table,
                   positions, q_new, per_head=False, cnt=None, out=None, stream=None):
    """kap_select_compact -> (sel_count, (compact_bt, compact_logical, compact_len,
    slot_mapping)); compact_logical is the selection list."""
    lib = load()
    B, Hkv, max_pages = scores.shape
    G = Hkv if per_head else 1
    dev = scores.device
    if cnt is None:
        cnt = torch.empty((B, G), dtype=torch.int32, device=dev)
    if out is None:
        out = (torch.empty((B, G, capacity), dtype=torch.int32, device=dev),
               torch.empty((B, G, capacity), dtype=torch.int32, device=dev),
               torch.empty((B, G), dtype=torch.int32, device=dev),
               torch.empty((B, max(q_new, 1)), dtype=torch.int64, device=dev))
    cbt, clog, clen, slot = out
    st = lib.kap_select_compact(_p(scores), B, Hkv, max_pages, _p(seq_lens), 16,
                                int(bool(per_head)), _p(anchor), _p(recent), _p(k_mid),
                                int(max_budget), int(capacity), _p(block_table), _p(positions),
                                int(q_new), _p(cnt), _p(cbt), _p(clog), _p(clen), _p(slot),
                                _stream(stream))
    _check(st, "kap_select_compact")
    return cnt, out


def _scale(D, scale):
    return 1.0 / math.sqrt(D) if scale is None else float(scale)


def decode_attn(q, positions, k_pool, v_pool, table, lens, G=1, theta=1e4, scale=None, out=None,
                lse=None, workspace=None, stream=None, logical=None):
    """kap_decode_attn: q [B][Hq][D] over a paged view table [B][G][width] with lens [B][G];
    logical [B][G][width] holds each entry's logical page (a compact view), None for a
    full block table."""
    lib = load()
    B, Hq, D = q.shape
    num_pages, Hkv = k_pool.shape[0], k_pool.shape[1]
    width = table.shape[-1]
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = torch.empty(attn_workspace_bytes(B, 1, Hq, Hkv, D), dtype=torch.uint8,
                                device=q.device)
    st = lib.kap_decode_attn(_p(q), _dt(q), _p(positions), float(theta), _scale(D, scale),
                             _p(k_pool), _p(v_pool), _dt(k_pool), num_pages, Hkv, D, 16, _p(table),
                             _p(logical), width, int(G), _p(lens), B, Hq, _p(out), _p(lse),
                             _p(workspace), workspace.numel(), _stream(stream))
    _check(st, "kap_decode_attn")
    return out


def decode_attn_noalloc(q, positions, k_pool, v_pool, table, lens, G=1, theta=1e4, scale=None,
                        out=None, lse=None, stream=None, logical=None):
    """kap_decode_attn_noalloc: kap_decode_attn without a workspace argument (the
    library's static per-GPU scratch holds the split-K partials)."""
    lib = load()
    B, Hq, D = q.shape
    num_pages, Hkv = k_pool.shape[0], k_pool.shape[1]
    if out is None:
        out = torch.empty_like(q)
    st = lib.kap_decode_attn_noalloc(_p(q), _dt(q), _p(positions), float(theta), _scale(D, scale),
                                     _p(k_pool), _p(v_pool), _dt(k_pool), num_pages, Hkv, D, 16,
                                     _p(table), _p(logical), table.shape[-1], int(G), _p(lens), B,
                                     Hq, _p(out), _p(lse), _stream(stream))
    _check(st, "kap_decode_attn_noalloc")
    return out


def verify_attn(q, start_positions, k_pool, v_pool, block_table, seq_lens, theta=1e4, scale=None,
                out=None, lse=None, workspace=None, stream=None):
    """kap_verify_attn: q [B][q_len][Hq][D] over the full table."""
    lib = load()
    B, q_len, Hq, D = q.shape
    num_pages, Hkv = k_pool.shape[0], k_pool.shape[1]
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = torch.empty(attn_workspace_bytes(B, q_len, Hq, Hkv, D), dtype=torch.uint8,
                                device=q.device)
    st = lib.kap_verify_attn(_p(q), _dt(q), _p(start_positions), q_len, float(theta),
                             _scale(D, scale), _p(k_pool), _p(v_pool), _dt(k_pool), num_pages, Hkv,
                             D, 16, _p(block_table), block_table.shape[1], _p(seq_lens), B, Hq,
                             _p(out), _p(lse), _p(workspace), workspace.numel(), _stream(stream))
    _check(st, "kap_verify_attn")
    return out


def diag_stream_read(buf, sink, stream=None):
    """kap_diag_stream_read: read every byte of `buf` (diagnostic bandwidth probe)."""
    st = load().kap_diag_stream_read(_p(buf), buf.numel() * buf.element_size(), _p(sink),
                                     _stream(stream))
    _check(st, "kap_diag_stream_read")


def build_summary(k_pool, block_table, seq_lens, summary, stream=None):
    """kap_build_summary: block-mean K of every referenced page into summary [P][Hkv][D]."""
    lib = load()
    num_pages, Hkv, ps, D = k_pool.shape
    st = lib.kap_build_summary(_p(k_pool), _dt(k_pool), num_pages, Hkv, D, ps, _p(block_table),
                               block_table.shape[1], _p(seq_lens), block_table.shape[0],
                               _p(summary), _dt(summary), _stream(stream))
    _check(st, "kap_build_summary")
    return summary


def update_summary(k_pool, block_table, seq_lens, positions, q_new, summary, stream=None):
    """kap_update_summary: recompute the summary rows of the pages holding tokens
    positions[b] .. positions[b] + q_new - 1 (seq_lens: lengths after the append)."""
    lib = load()
    num_pages, Hkv, ps, D = k_pool.shape
    st = lib.kap_update_summary(_p(k_pool), _dt(k_pool), num_pages, Hkv, D, ps, _p(block_table),
                                block_table.shape[1], _p(seq_lens), _p(positions), int(q_new),
                                block_table.shape[0], _p(summary), _dt(summary), _stream(stream))
    _check(st, "kap_update_summary")
    return summary


def append_kv(k_new, v_new, slot_mapping, k_pool, v_pool, stream=None):
    """kap_append_kv: write k_new/v_new [B][q_new][Hkv][D] into the pools at slot_mapping [B][q_new]."""
    lib = load()
    B, q_new, Hkv, D = k_new.shape
    num_pages, _, ps, _ = k_pool.shape
    if tuple(v_new.shape) != tuple(k_new.shape) or tuple(slot_mapping.shape) != (B, q_new):
        raise ValueError("k_new, v_new must be [B][q_new][Hkv][D] and slot_mapping [B][q_new]")
    if slot_mapping.dtype != torch.int64:
        raise ValueError("slot_mapping must be int64")
    if _dt(k_new) != _dt(k_pool) or _dt(v_new) != _dt(v_pool):
        raise ValueError("new K/V must have the pool's dtype")
    st = lib.kap_append_kv(_p(k_new), _p(v_new), _dt(k_pool), _p(slot_mapping), B, q_new, Hkv, D,
                           ps, num_pages, _p(k_pool), _p(v_pool), _stream(stream))
    _check(st, "kap_append_kv")
    return k_pool, v_pool


def materialize_view(k_pool, v_pool, compact_bt, k_ws=None, v_ws=None, ws_table=None, stream=None):
    """kap_materialize_view: copy the compact view's pages into a workspace of
    B*capacity pages; returns (k_ws, v_ws, ws_table)."""
    lib = load()
    num_pages, Hkv, ps, D = k_pool.shape
    B, G, cap = compact_bt.shape
    if k_ws is None:
        k_ws = torch.empty((B * cap,) + tuple(k_pool.shape[1:]), dtype=k_pool.dtype, device=k_pool.device)
        v_ws = torch.empty((B * cap,) + tuple(v_pool.shape[1:]), dtype=v_pool.dtype, device=v_pool.device)
    if ws_table is None:
        ws_table = torch.empty_like(compact_bt)
    if _dt(k_ws) != _dt(k_pool) or _dt(v_ws) != _dt(v_pool) or _dt(k_pool) != _dt(v_pool):
        raise ValueError("workspace and pool dtypes differ")
    if tuple(k_ws.shape[1:]) != tuple(k_pool.shape[1:]) or tuple(v_ws.shape[1:]) != tuple(v_pool.shape[1:]):
        raise ValueError("workspace page shape differs from the pool's")
    st = lib.kap_materialize_view(_p(k_pool), _p(v_pool), _dt(k_pool), num_pages, Hkv, D, ps,
                                  _p(compact_bt), B, G, cap, _p(k_ws), _p(v_ws), k_ws.shape[0],
                                  _p(ws_table), _stream(stream))
    _check(st, "kap_materialize_view")
    return k_ws, v_ws, ws_table


# ----------------------------------------------------------------------------- host routing
# CPU-offloaded early routing: numpy arrays in host memory, results in host
# memory (to be uploaded as page indices).  Synchronous; ctypes releases the
# GIL for the call, so a Python thread can route while the GPU works.
def _h(a, dtype):
    a = np.asarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype).name}, got {a.dtype}")
    if not a.flags.c_contiguous:
        raise ValueError("host arrays must be C-contiguous")
    return a


def _hp(a):
    return ctypes.c_void_p(a.ctypes.data)


def host_proxy_query(hidden, w_q, q_out=None, threads=0):
    """kap_host_proxy_query: hidden [B][d_model], w_q [d_model][n] bf16 bits (uint16) -> fp32 [B][n]."""
    hidden = _h(hidden, np.uint16)
    w_q = _h(w_q, np.uint16)
    B, dm = hidden.shape
    n = w_q.shape[1]
    if q_out is None:
        q_out = np.empty((B, n), np.float32)
    q_out = _h(q_out, np.float32)
    _check(load().kap_host_proxy_query(_hp(hidden), _hp(w_q), B, dm, n, _hp(q_out), threads),
           "kap_host_proxy_query")
    return q_out


def host_score_blocks(q, positions, summary, block_table, seq_lens, Hkv, theta=1e4, scores=None,
                      threads=0):
    """kap_host_score_blocks: q [B][Hq][D] fp32, summary [P][Hkv][D] bf16 bits -> [B][Hkv][max_pages]."""
    q = _h(q, np.float32)
    summary = _h(summary, np.uint16)
    block_table = _h(block_table, np.int32)
    positions = _h(positions, np.int32)
    seq_lens = _h(seq_lens, np.int32)
    B, Hq, D = q.shape
    max_pages = block_table.shape[1]
    if scores is None:
        scores = np.empty((B, Hkv, max_pages), np.float32)
    scores = _h(scores, np.float32)
    _check(load().kap_host_score_blocks(_hp(q), _hp(positions), theta, _hp(summary),
                                        summary.shape[0], _hp(block_table), max_pages,
                                        _hp(seq_lens), B, Hq, Hkv, D, 16, _hp(scores), threads),
           "kap_host_score_blocks")
    return scores


def host_select_topk(scores, seq_lens, anchor, recent, k_mid, capacity, per_head=False, sel=None,
                     cnt=None, threads=0):
    """kap_host_select_topk: same selection as select_topk, on host arrays."""
    scores = _h(scores, np.float32)
    seq_lens, anchor = _h(seq_lens, np.int32), _h(anchor, np.int32)
    recent, k_mid = _h(recent, np.int32), _h(k_mid, np.int32)
    B, Hkv, max_pages = scores.shape
    G = Hkv if per_head else 1
    if sel is None:
        sel = np.empty((B, G, capacity), np.int32)
        cnt = np.empty((B, G), np.int32)
    sel, cnt = _h(sel, np.int32), _h(cnt, np.int32)
    _check(load().kap_host_select_topk(_hp(scores), B, Hkv, max_pages, _hp(seq_lens), 16,
                                       int(per_head), _hp(anchor), _hp(recent), _hp(k_mid),
                                       capacity, _hp(sel), _hp(cnt), threads),
           "kap_host_select_topk")
    return sel, cnt
