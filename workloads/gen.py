"""Seeded generators for the five workload shapes.

Shapes follow the pages' workloads (128K-context 32B-class attention, Llama-3-8B
attention at 32K, the 40K-token early-routing setup, a mixed serving batch);
every number is drawn here from a seed and nothing comes from a dataset.

Recipe (per request b, generator default_rng(SeedSequence([seed, b])), draws in
this fixed order):
  1. decode query q[b]          [Hq][D]            N(0, sigma^2)
  2. verify queries qv[b]        [q_len][Hq][D]     N(0, sigma^2)
  3. needle pages: n distinct logical pages drawn from the middle region
     [a, N - r) without replacement
  4. keys of every allocated page, token-major      N(0, sigma^2)
  5. values of every allocated page, token-major    N(0, sigma^2)
Then, outside the per-request streams:
  6. physical placement: one permutation of the pool from
     default_rng(SeedSequence([seed, 1_000_003])); request b's logical page p
     lives at the next unused entry.
  7. (draft_kv) the verify window's new K and V rows, [q_len][Hkv][D] each,
     N(0, sigma^2), from default_rng(SeedSequence([seed, b, 2_000_029])), so
     that drawing them changes nothing above.
Needle keys: on every valid token of a needle page and every KV head g,
K += alpha * dir[b][g], alpha = needle_scale * sigma * sqrt(D).  dir is taken
from the caller when given; otherwise it is the unit vector along the sum of the
(unrotated) query heads of group g -- the literal "+1.5 q-hat" of the tiny case.
Token slots at or beyond the sequence length inside allocated pages hold NaN,
so a kernel that reads an invisible slot produces NaN and fails loudly.
bf16 values are the round-to-nearest-even of the fp32 draws, stored as uint16.

K is stored [P][Hkv][page][D] (token-major); V is stored [P][Hkv][D][page]
(dim-major), the layout the attention kernels read.  make() returns only the
allocated pages (K_pages, V_pages, in allocation order) with their pool ids
(phys) so that a 100 GB pool need not exist on the host; dense_pool() builds
the full pool arrays for small cases.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

PAGE = 16


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    seq_lens: Sequence[int]
    dtype: str = "bf16"            # "bf16" or "f32"
    seed: int = 0
    sigma: float = 1.0
    page_size: int = PAGE
    needles: Sequence[int] | int = 0  # needle pages per request
    needle_scale: float = 1.5
    anchor: Sequence[int] | int = 1
    recent: Sequence[int] | int = 2
    k_mid: Optional[Sequence[int] | int] = None        # explicit middle count
    ratio: Optional[Sequence[tuple]] = None             # per request (num, den) retention
    per_head: bool = False
    q_len: int = 4                 # verify window
    pool_pages: Optional[int] = None
    theta: float = 1e4
    hidden_dim: int = 0            # proxy-query routing (0: none)

    def per_request(self, v) -> np.ndarray:
        return np.broadcast_to(np.asarray(v, dtype=np.int32), (self.B,)).copy()

    @property
    def n_pages(self) -> np.ndarray:
        L = np.asarray(self.seq_lens, dtype=np.int64)
        return ((L + self.page_size - 1) // self.page_size).astype(np.int32)

    @property
    def alloc_pages(self) -> np.ndarray:
        """Pages allocated per request: the context plus room for q_len new tokens."""
        L = np.asarray(self.seq_lens, dtype=np.int64)
        extra = max(self.q_len, 1)
        return ((L + extra + self.page_size - 1) // self.page_size).astype(np.int32)


def _log_uniform_lengths(seed: int, B: int, lo: int, hi: int) -> list:
    rng = np.random.default_rng(np.random.SeedSequence([seed, 2_000_003]))
    u = rng.uniform(math.log(lo), math.log(hi), size=B)
    return [int(math.floor(math.exp(x))) for x in u]


def _c5_mix(seed: int, B: int):
    rng = np.random.default_rng(np.random.SeedSequence([seed, 3_000_017]))
    ratios = [(1, 100), (55, 1000), (25, 100), (1, 1)]
    splits = [(1, 2), (4, 4)]
    r_idx = rng.integers(0, len(ratios), size=B)
    s_idx = rng.integers(0, len(splits), size=B)
    return ([ratios[i] for i in r_idx], [splits[i][0] for i in s_idx],
            [splits[i][1] for i in s_idx])


def spec(name: str, **over) -> Workload:
    """Named workload shapes; keyword overrides give reduced variants for tests."""
    if name == "tiny":          # 1 request, GQA 4:1, D 64, 1024 tokens, fp32
        w = Workload(name="tiny", B=1, Hq=8, Hkv=2, D=64, seq_lens=[1024], dtype="f32", seed=1,
                     sigma=1.0 / 8.0, needles=2, needle_scale=1.5, anchor=1, recent=2, k_mid=5,
                     q_len=4, pool_pages=160)
    elif name == "llama8b_32k":  # batch 8, 32/8 heads, D 128, 32K context, s = 5.5 %
        w = Workload(name="llama8b_32k", B=8, Hq=32, Hkv=8, D=128, seq_lens=[32768] * 8,
                     dtype="bf16", seed=2, needles=20, anchor=1, recent=2, k_mid=110, q_len=4)
    elif name == "qwen32b_128k":  # batch 1-4, 64/8 heads, D 128, 128K context, s = 5.5 %
        B = over.pop("B", 4)
        w = Workload(name="qwen32b_128k", B=B, Hq=64, Hkv=8, D=128, seq_lens=[131072] * B,
                     dtype="bf16", seed=3, needles=81, anchor=1, recent=2, k_mid=448, q_len=4)
    elif name == "early_route_40k":  # 40K inputs, per-head top-8 pages, proxy query routing
        B = over.pop("B", 1)
        w = Workload(name="early_route_40k", B=B, Hq=32, Hkv=8, D=128, seq_lens=[40000] * B,
                     dtype="bf16", seed=4, needles=0, anchor=0, recent=0, k_mid=8, per_head=True,
                     q_len=1, hidden_dim=4096)
    elif name == "mixed_serving":  # 64 ragged requests 4K-128K, mixed retention and splits
        B = over.pop("B", 64)
        lo, hi = over.pop("len_range", (4096, 131072))
        seed = over.pop("seed", 5)
        lens = _log_uniform_lengths(seed, B, lo, hi)
        ratios, anchors, recents = _c5_mix(seed, B)
        needles = [max(1, int(round(0.01 * ((L + PAGE - 1) // PAGE)))) for L in lens]
        w = Workload(name="mixed_serving", B=B, Hq=32, Hkv=8, D=128, seq_lens=lens, dtype="bf16",
                     seed=seed, needles=needles, anchor=anchors, recent=recents, ratio=ratios,
                     q_len=1, pool_pages=1_525_878)
    else:
        raise KeyError(name)
    for k, v in over.items():
        if not hasattr(w, k):
            raise KeyError(k)
        setattr(w, k, v)
    return w


SPECS = ("tiny", "llama8b_32k", "qwen32b_128k", "early_route_40k", "mixed_serving")


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16 bit patterns (NaN kept quiet)."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    out = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16))
    out = out.astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return _to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def make(w: Workload, needle_dir: Optional[np.ndarray] = None, with_kv: bool = True) -> dict:
    """Draw one batch as host numpy arrays.

    needle_dir: optional [B][Hkv][D] unit directions for the needle keys.
    with_kv: False skips the K/V pages (routing-only uses); everything else,
    needle pages included, is drawn identically.
    Keys: q [B][Hq][D], qv [B][q_len][Hq][D], K_pages [T][Hkv][ps][D],
    V_pages [T][Hkv][D][ps], phys [T] (pool page of allocated page j), bt
    [B][max_alloc] pool ids (-1 unallocated), bt_local (same, indexing K_pages),
    seq_lens, positions (= seq_lens: the decode token follows the context),
    anchor, recent, k_mid or ratio, needle_pages, pool_pages.
    """
    B, Hq, Hkv, D, ps = w.B, w.Hq, w.Hkv, w.D, w.page_size
    grp = Hq // Hkv
    L = np.asarray(w.seq_lens, dtype=np.int32)
    N = w.n_pages
    NA = w.alloc_pages
    total = int(NA.sum())
    pool = int(w.pool_pages) if w.pool_pages is not None else total
    if pool < total:
        raise ValueError(f"pool of {pool} pages cannot hold {total} allocated pages")
    anchor, recent = w.per_request(w.anchor), w.per_request(w.recent)
    max_alloc = int(NA.max())

    prng = np.random.default_rng(np.random.SeedSequence([w.seed, 1_000_003]))
    phys = prng.permutation(pool)[:total].astype(np.int32)
    bt = np.full((B, max_alloc), -1, dtype=np.int32)
    bt_local = np.full((B, max_alloc), -1, dtype=np.int32)
    starts = np.concatenate([[0], np.cumsum(NA)[:-1]]).astype(np.int64)
    for b in range(B):
        bt[b, :NA[b]] = phys[starts[b]:starts[b] + NA[b]]
        bt_local[b, :NA[b]] = np.arange(starts[b], starts[b] + NA[b], dtype=np.int32)

    store_dt = np.uint16 if w.dtype == "bf16" else np.float32
    q = np.empty((B, Hq, D), dtype=store_dt)
    qv = np.empty((B, w.q_len, Hq, D), dtype=store_dt)
    K_pages = V_pages = None
    if with_kv:
        K_pages = np.empty((total, Hkv, ps, D), dtype=store_dt)
        V_pages = np.empty((total, Hkv, D, ps), dtype=store_dt)
    needle_pages = []
    alpha = w.needle_scale * w.sigma * math.sqrt(D)
    nneed = w.per_request(w.needles)
    for b in range(B):
        rng = np.random.default_rng(np.random.SeedSequence([w.seed, b]))
        qb = rng.standard_normal((Hq, D), dtype=np.float32) * np.float32(w.sigma)
        qvb = rng.standard_normal((w.q_len, Hq, D), dtype=np.float32) * np.float32(w.sigma)
        q[b] = _store(qb, w.dtype)
        qv[b] = _store(qvb, w.dtype)
        mid_lo, mid_hi = int(anchor[b]), int(N[b]) - int(recent[b])
        n_need = min(int(nneed[b]), max(mid_hi - mid_lo, 0))
        if n_need > 0:
            pages = np.sort(rng.choice(np.arange(mid_lo, mid_hi), size=n_need, replace=False))
        else:
            pages = np.zeros(0, np.int64)
        needle_pages.append(pages.astype(np.int32))
        if not with_kv:
            continue
        npg = int(NA[b])
        kb = rng.standard_normal((npg, Hkv, ps, D), dtype=np.float32) * np.float32(w.sigma)
        vb = rng.standard_normal((npg, Hkv, ps, D), dtype=np.float32) * np.float32(w.sigma)
        if n_need > 0:
            if needle_dir is not None:
                dirs = np.asarray(needle_dir[b], dtype=np.float64)
            else:
                qsum = qb.astype(np.float64).reshape(Hkv, grp, D).sum(axis=1)
                dirs = qsum / np.linalg.norm(qsum, axis=1, keepdims=True)
            bump = (alpha * dirs[:, None, :]).astype(np.float32)
            for p in pages:
                nvalid = min(ps, int(L[b]) - int(p) * ps)
                kb[p, :, :nvalid, :] += bump
        # invisible slots (at or beyond the sequence length) hold NaN
        dead = (np.arange(npg * ps).reshape(npg, ps) >= int(L[b]))
        if dead.any():
            mask = np.broadcast_to(dead[:, None, :], (npg, Hkv, ps))
            kb[mask] = np.nan
            vb[mask] = np.nan
        s0 = int(starts[b])
        K_pages[s0:s0 + npg] = _store(kb, w.dtype)
        V_pages[s0:s0 + npg] = _store(np.ascontiguousarray(vb.transpose(0, 1, 3, 2)), w.dtype)
        del kb, vb

    out = dict(q=q, qv=qv, K_pages=K_pages, V_pages=V_pages, phys=phys, bt=bt,
               bt_local=bt_local, seq_lens=L.copy(), positions=L.copy(), anchor=anchor,
               recent=recent, needle_pages=needle_pages, pool_pages=pool)
    if w.k_mid is not None:
        out["k_mid"] = w.per_request(w.k_mid)
    if w.ratio is not None:
        out["ratio"] = [tuple(r) for r in w.ratio]
    if w.hidden_dim:
        hr = np.random.default_rng(np.random.SeedSequence([w.seed, 4_000_037]))
        hidden = hr.standard_normal((B, w.hidden_dim), dtype=np.float32)
        wq = hr.standard_normal((w.hidden_dim, Hq * D), dtype=np.float32) / np.float32(
            math.sqrt(w.hidden_dim))
        out["hidden"] = _to_bf16_bits(hidden)
        out["wq"] = _to_bf16_bits(wq)
    return out


def draft_kv(w: Workload):
    """K and V rows of the q_len window tokens (appended before the causal verify):
    two [B][q_len][Hkv][D] arrays in the workload's storage type."""
    shape = (w.q_len, w.Hkv, w.D)
    ks, vs = [], []
    for b in range(w.B):
        rng = np.random.default_rng(np.random.SeedSequence([w.seed, b, 2_000_029]))
        ks.append(rng.standard_normal(shape, dtype=np.float32) * np.float32(w.sigma))
        vs.append(rng.standard_normal(shape, dtype=np.float32) * np.float32(w.sigma))
    return _store(np.stack(ks), w.dtype), _store(np.stack(vs), w.dtype)


def dense_pool(batch: dict):
    """Full pool arrays (K [pool][Hkv][ps][D], V [pool][Hkv][D][ps]); unallocated pages are 0."""
    Kp, Vp, phys, pool = batch["K_pages"], batch["V_pages"], batch["phys"], batch["pool_pages"]
    K = np.zeros((pool,) + Kp.shape[1:], dtype=Kp.dtype)
    V = np.zeros((pool,) + Vp.shape[1:], dtype=Vp.dtype)
    K[phys] = Kp
    V[phys] = Vp
    return K, V


def make_device(w: Workload, device, needle_dir: Optional[np.ndarray] = None,
                alloc_pools=None) -> dict:
    """Same recipe as make(), with the K/V pages drawn on the GPU.

    Queries, needle pages, placement and budgets come from the same numpy
    streams as make() (so they are identical); the K/V values come from
    torch's Philox generator on `device`, seeded with (seed, b), and are
    rounded to bf16 by torch (round-to-nearest-even).  Returns the make()
    dictionary without K_pages/V_pages, plus device tensors K, V (full pool,
    unallocated pages zero), and torch copies of the small arrays.
    alloc_pools(pages, Hkv, D, dtype, device), if given, returns the zeroed
    K and V pool tensors (a placement of the caller's choosing); by default
    they are two separate allocations.
    """
    import torch

    b = make(w, needle_dir=needle_dir, with_kv=False)
    B, Hq, Hkv, D, ps = w.B, w.Hq, w.Hkv, w.D, w.page_size
    grp = Hq // Hkv
    L = b["seq_lens"]
    NA = w.alloc_pages
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    pool = b["pool_pages"]
    if alloc_pools is None:
        K = torch.zeros((pool, Hkv, ps, D), dtype=tdt, device=device)
        V = torch.zeros((pool, Hkv, D, ps), dtype=tdt, device=device)
    else:
        K, V = alloc_pools(pool, Hkv, D, tdt, device)
        assert K.shape == (pool, Hkv, ps, D) and V.shape == (pool, Hkv, D, ps)
    alpha = w.needle_scale * w.sigma * math.sqrt(D)
    starts = np.concatenate([[0], np.cumsum(NA)[:-1]]).astype(np.int64)
    for bi in range(B):
        g = torch.Generator(device=device)
        g.manual_seed(int(w.seed) * 1_000_003 + bi)
        npg = int(NA[bi])
        rows = torch.from_numpy(b["phys"][starts[bi]:starts[bi] + npg].astype(np.int64)).to(device)
        kb = torch.randn((npg, Hkv, ps, D), generator=g, device=device, dtype=torch.float32)
        vb = torch.randn((npg, Hkv, ps, D), generator=g, device=device, dtype=torch.float32)
        if w.sigma != 1.0:
            kb.mul_(w.sigma)
            vb.mul_(w.sigma)
        pages = b["needle_pages"][bi]
        if len(pages):
            if needle_dir is not None:
                dirs = np.asarray(needle_dir[bi], dtype=np.float64)
            else:
                qb = b["q"][bi]
                qf = ((qb.astype(np.uint32) << 16).view(np.float32) if qb.dtype == np.uint16
                      else qb).astype(np.float64)
                qsum = qf.reshape(Hkv, grp, D).sum(axis=1)
                dirs = qsum / np.linalg.norm(qsum, axis=1, keepdims=True)
            bump = torch.from_numpy((alpha * dirs).astype(np.float32)).to(device)
            for p in pages:
                nvalid = min(ps, int(L[bi]) - int(p) * ps)
                kb[int(p), :, :nvalid, :] += bump[:, None, :]
        first_dead = int(L[bi])
        if first_dead < npg * ps:
            p0 = first_dead // ps
            for p in range(p0, npg):
                t0 = max(0, first_dead - p * ps)
                kb[p, :, t0:, :] = float("nan")
                vb[p, :, t0:, :] = float("nan")
        K[rows] = kb.to(tdt)
        V[rows] = vb.transpose(2, 3).contiguous().to(tdt)
        del kb, vb
    b["K"], b["V"] = K, V
    return b


def request_key(q: np.ndarray, position: int) -> str:
    """Identity of one request's decode query and its position (hash of the bits)."""
    import hashlib
    return hashlib.sha256(np.ascontiguousarray(q).tobytes() + int(position).to_bytes(8, "little")).hexdigest()[:16]


def aimed_dirs(w: Workload) -> np.ndarray:
    """Stored needle directions of a benchmark workload ([B][Hkv][D] float32),
    written by workloads/aim/make_aim.py (which aims them at the rotated,
    group-summed query).  Raises if the file is missing or was made from other
    query draws or positions."""
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "aim", f"{w.name}.npz")
    if not os.path.exists(path):
        raise FileNotFoundError(f"{path}: run tests/golden/make_needle_dirs.py")
    z = np.load(path, allow_pickle=False)
    dirs, keys = z["dirs"], z["keys"]
    if dirs.shape[0] < w.B or dirs.shape[1:] != (w.Hkv, w.D):
        raise ValueError(f"{path} holds {dirs.shape}, need [{w.B}][{w.Hkv}][{w.D}]")
    b = make(w, with_kv=False)
    for bi in range(w.B):
        if request_key(b["q"][bi], int(b["positions"][bi])) != str(keys[bi]):
            raise ValueError(f"{path}: request {bi} was aimed for other query draws or another "
                             "position; rerun tests/golden/make_needle_dirs.py")
    return dirs[:w.B]
