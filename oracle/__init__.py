"""CPU oracle for selected-KV paged decode attention -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py may
import this package.  The product library (block_sparse_paged_page_amd) never
imports, links or runs anything here; the two share no code.

The arithmetic lives in kap_oracle.c (plain loops, fp64); this module only
marshals numpy arrays into it, plus the fp64 cost model of costmodel.py.
Arrays holding bf16 values are numpy uint16 bit patterns; fp32 values are
numpy float32.  See kap_oracle.c for the citation of each function.

Parity status: every function here is pinned by tests/test_oracle_*.py; none
is "parity unpinned".
"""
import ctypes
import os

import numpy as np

from . import costmodel  # noqa: F401  (re-exported)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16 = 0, 1

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_D = ctypes.c_double


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.kor_rope.argtypes = [_P, _I, _D, _D, _P]
    lib.kor_summary.argtypes = [_P, _I, _I, _P, _I, _P, _I, _I, _I, _I, _P]
    lib.kor_score.argtypes = [_P, _I, _P, _D, _P, _I, _P, _I, _P, _I, _I, _I, _I, _I, _P]
    lib.kor_proxy_query.argtypes = [_P, _I, _P, _I, _I, _I, _I, _P]
    lib.kor_select.argtypes = [_P, _I, _I, _I, _P, _I, _I, _P, _P, _P, _I, _P, _P]
    lib.kor_budget_from_ratio.argtypes = [_I, _I64, _I64, _I, _I]
    lib.kor_budget_from_ratio.restype = _I
    lib.kor_compact.argtypes = [_P, _P, _I, _I, _I, _P, _I, _P, _I, _P, _I, _P, _P, _P, _P]
    lib.kor_attend.argtypes = [_P, _I, _I, _P, _D, _D, _P, _P, _I, _I, _I, _I, _P, _I, _P, _P,
                               _I, _I, _I, _P, _P]
    lib.kor_num_threads.restype = _I
    lib.kor_append_kv.argtypes = [_P, _P, _I, _P, _I, _I, _I, _I, _I, _P, _P]
    lib.kor_materialize.argtypes = [_P, _P, _I, _I, _I, _I, _P, _I, _I, _I, _P, _P, _P]
    lib.kor_set_threads.argtypes = [_I]
    _lib = lib
    return lib


def num_threads() -> int:
    """OpenMP threads the oracle runs on."""
    return int(_load().kor_num_threads())


def set_threads(n: int) -> None:
    """Sets the OpenMP thread count of the oracle's loops (n >= 1)."""
    _load().kor_set_threads(int(n))


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle inputs are float32 or uint16 (bf16 bits), got {a.dtype}")


def _c(a, dtype=None):
    a = np.ascontiguousarray(a if dtype is None else np.asarray(a, dtype=dtype))
    return a


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def widen(a: np.ndarray) -> np.ndarray:
    """Exact fp64 value of float32 or bf16-bit (uint16) array."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def round_to_bf16(x) -> np.ndarray:
    """Round-to-nearest-even of float64/float32 values to bf16 bit patterns."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        rounded[nan] = 0x7FC0
    return rounded


# ----------------------------------------------------------------------------- O1
def rope(x, pos: float, theta: float = 1e4) -> np.ndarray:
    """Rotate one or more vectors (last axis D) at logical position pos (fp64)."""
    lib = _load()
    x = np.asarray(x, dtype=np.float64)
    flat = _c(x.reshape(-1, x.shape[-1]))
    out = np.empty_like(flat)
    D = flat.shape[1]
    for r in range(flat.shape[0]):
        lib.kor_rope(_ptr(flat[r]), D, float(pos), float(theta), _ptr(out[r]))
    return out.reshape(x.shape)


# ----------------------------------------------------------------------------- O2
def summary(K, bt, seq_lens, page_size: int = 16, out=None) -> np.ndarray:
    """Block-mean K per (page, kv head) in fp64, shape [num_pages][Hkv][D]."""
    lib = _load()
    K = _c(K)
    P, Hkv, ps, D = K.shape
    assert ps == page_size
    bt = _c(bt, np.int32)
    seq_lens = _c(seq_lens, np.int32)
    if out is None:
        out = np.zeros((P, Hkv, D), dtype=np.float64)
    lib.kor_summary(_ptr(K), _dt(K), P, _ptr(bt), bt.shape[1], _ptr(seq_lens), bt.shape[0],
                    Hkv, D, page_size, _ptr(out))
    return out


# ----------------------------------------------------------------------------- O3
def score(q, positions, summ, bt, seq_lens, Hkv: int, page_size: int = 16,
          theta: float = 1e4) -> np.ndarray:
    """fp64 page scores [B][Hkv][max_pages]; q is [B][Hq][D] (unrotated)."""
    lib = _load()
    q = _c(q)
    summ = _c(summ)
    bt = _c(bt, np.int32)
    positions = _c(positions, np.int32)
    seq_lens = _c(seq_lens, np.int32)
    B, Hq, D = q.shape
    max_pages = bt.shape[1]
    out = np.empty((B, Hkv, max_pages), dtype=np.float64)
    lib.kor_score(_ptr(q), _dt(q), _ptr(positions), float(theta), _ptr(summ), _dt(summ),
                  _ptr(bt), max_pages, _ptr(seq_lens), B, Hq, Hkv, D, page_size, _ptr(out))
    return out


def proxy_query(hidden, wq) -> np.ndarray:
    """fp64 hidden @ Wq; hidden [B][dm], Wq [dm][n] (bf16 bits or fp32)."""
    lib = _load()
    hidden = _c(hidden)
    wq = _c(wq)
    B, dm = hidden.shape
    n = wq.shape[1]
    out = np.empty((B, n), dtype=np.float64)
    lib.kor_proxy_query(_ptr(hidden), _dt(hidden), _ptr(wq), _dt(wq), B, dm, n, _ptr(out))
    return out


# ----------------------------------------------------------------------------- O4
def budget_from_ratio(N: int, s_num: int, s_den: int, a: int, r: int) -> int:
    return int(_load().kor_budget_from_ratio(int(N), int(s_num), int(s_den), int(a), int(r)))


def select(scores, seq_lens, anchor, recent, k_mid, capacity: int, per_head: bool = False,
           page_size: int = 16):
    """Top-K under A/R/K on fp32 scores [B][Hkv][max_pages].

    Returns (sel int32 [B][G][capacity] ascending, -1 padded; cnt int32 [B][G]).
    """
    lib = _load()
    scores = _c(scores, np.float32)
    B, Hkv, max_pages = scores.shape
    G = Hkv if per_head else 1
    seq_lens = _c(seq_lens, np.int32)
    a = _c(np.broadcast_to(np.asarray(anchor, dtype=np.int32), (B,)))
    r = _c(np.broadcast_to(np.asarray(recent, dtype=np.int32), (B,)))
    k = _c(np.broadcast_to(np.asarray(k_mid, dtype=np.int32), (B,)))
    sel = np.empty((B, G, capacity), dtype=np.int32)
    cnt = np.empty((B, G), dtype=np.int32)
    lib.kor_select(_ptr(scores), B, Hkv, max_pages, _ptr(seq_lens), page_size, int(per_head),
                   _ptr(a), _ptr(r), _ptr(k), capacity, _ptr(sel), _ptr(cnt))
    return sel, cnt


# ----------------------------------------------------------------------------- O5
def compact(sel, cnt, bt, seq_lens, positions, q_new: int, page_size: int = 16):
    """Returns (cbt, clog [B][G][cap], clen [B][G], slot int64 [B][q_new])."""
    lib = _load()
    sel = _c(sel, np.int32)
    cnt = _c(cnt, np.int32)
    B, G, cap = sel.shape
    bt = _c(bt, np.int32)
    seq_lens = _c(seq_lens, np.int32)
    positions = _c(positions, np.int32)
    cbt = np.empty_like(sel)
    clog = np.empty_like(sel)
    clen = np.empty((B, G), dtype=np.int32)
    slot = np.empty((B, max(q_new, 0)), dtype=np.int64)
    lib.kor_compact(_ptr(sel), _ptr(cnt), B, G, cap, _ptr(bt), bt.shape[1], _ptr(seq_lens),
                    page_size, _ptr(positions), q_new, _ptr(cbt), _ptr(clog), _ptr(clen),
                    _ptr(slot))
    return cbt, clog, clen, slot


# ----------------------------------------------------------------------------- O6/O7
def keys_full(seq_lens, G: int = 1):
    """Key lists exposing every token [0, L_b) of each request (per G-row)."""
    lists = []
    for L in seq_lens:
        for _ in range(G):
            lists.append(np.arange(int(L), dtype=np.int32))
    return lists


def keys_selected(sel, cnt, seq_lens, page_size: int = 16):
    """Key lists exposing the tokens of the selected logical pages."""
    B, G, _ = sel.shape
    lists = []
    for b in range(B):
        L = int(seq_lens[b])
        for gr in range(G):
            pages = sel[b, gr, :int(cnt[b, gr])]
            toks = [np.arange(p * page_size, min(p * page_size + page_size, L), dtype=np.int32)
                    for p in pages]
            lists.append(np.concatenate(toks) if toks else np.zeros(0, dtype=np.int32))
    return lists


def attend(q, positions, K, V, bt, key_lists, G: int, Hkv: int, page_size: int = 16,
           theta: float = 1e4, scale=None):
    """Softmax attention over explicit logical key sets.

    q [B][q_len][Hq][D]; key_lists has B*G int32 arrays (row b*G+gr).
    Returns (out fp64 [B][q_len][Hq][D], lse fp64 [B][q_len][Hq]).
    """
    lib = _load()
    q = _c(q)
    K = _c(K)
    V = _c(V)
    assert _dt(K) == _dt(V)
    B, q_len, Hq, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    bt = _c(bt, np.int32)
    positions = _c(positions, np.int32)
    assert len(key_lists) == B * G
    off = np.zeros(B * G + 1, dtype=np.int64)
    for j, kl in enumerate(key_lists):
        off[j + 1] = off[j] + len(kl)
    keys = _c(np.concatenate(key_lists) if off[-1] > 0 else np.zeros(1, np.int32), np.int32)
    out = np.empty((B, q_len, Hq, D), dtype=np.float64)
    lse = np.empty((B, q_len, Hq), dtype=np.float64)
    lib.kor_attend(_ptr(q), _dt(q), q_len, _ptr(positions), float(theta), float(scale), _ptr(K),
                   _ptr(V), _dt(K), Hkv, D, page_size, _ptr(bt), bt.shape[1], _ptr(keys),
                   _ptr(off), G, B, Hq, _ptr(out), _ptr(lse))
    return out, lse


def append_kv(k_new, v_new, slot, K, V, page_size: int = 16):
    """Write new tokens' K/V (same dtype as the pool) through a slot mapping, in place."""
    lib = _load()
    k_new = _c(k_new)
    v_new = _c(v_new)
    slot = _c(slot, np.int64)
    assert K.flags.c_contiguous and V.flags.c_contiguous
    B, q_new, Hkv, D = k_new.shape
    lib.kor_append_kv(_ptr(k_new), _ptr(v_new), _dt(K), _ptr(slot), B, q_new, Hkv, D, page_size,
                      _ptr(K), _ptr(V))


def materialize(K, V, cbt, Kws=None, Vws=None, page_size: int = 16):
    """Copy the compact view's pages into a workspace of B*cap pages (page b*cap + j,
    head slot g = head g of compact page j of row (b, g or 0)).  Returns
    (Kws, Vws, ws_table [B][G][cap])."""
    lib = _load()
    K = _c(K)
    V = _c(V)
    cbt = _c(cbt, np.int32)
    B, G, cap = cbt.shape
    P, Hkv, ps, D = K.shape
    assert ps == page_size and _dt(K) == _dt(V)
    if Kws is None:
        Kws = np.zeros((B * cap,) + K.shape[1:], dtype=K.dtype)
        Vws = np.zeros((B * cap,) + V.shape[1:], dtype=V.dtype)
    assert Kws.flags.c_contiguous and Vws.flags.c_contiguous and Kws.shape[0] >= B * cap
    table = np.empty_like(cbt)
    lib.kor_materialize(_ptr(K), _ptr(V), _dt(K), Hkv, D, page_size, _ptr(cbt), B, G, cap,
                        _ptr(Kws), _ptr(Vws), _ptr(table))
    return Kws, Vws, table
