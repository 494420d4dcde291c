"""Helpers for the GPU parity tests: upload seeded inputs, run the HIP path
through the C ABI, run the oracle on the same host arrays, compare."""
import numpy as np
import torch

import block_sparse_paged_page_amd as kap
import oracle
import workloads as W

TOL = {"f32": 1e-4, "bf16": 2e-2}          # attention: max |diff| / ||ref|| per output row
LSE_TOL = {"f32": 1e-5, "bf16": 2e-2}
SCORE_TOL = 1e-5                            # |dS| <= SCORE_TOL * ||u_g|| * ||summary row||


def dev():
    return torch.device("cuda:0")


def t(a, device=None):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device or dev())


def host(x: torch.Tensor, bf16: bool):
    a = x.detach().cpu().numpy()
    if bf16:
        return oracle.widen(a.view(np.uint16))
    return a.astype(np.float64)


class Case:
    """One seeded batch on host and device, with the oracle summary."""

    def __init__(self, w, needle_dir=None, aim_needles=False):
        self.w = w
        if aim_needles and needle_dir is None:
            b0 = W.make(w, with_kv=False)
            grp = w.Hq // w.Hkv
            dirs = []
            for bi in range(w.B):
                qr = oracle.rope(oracle.widen(b0["q"][bi]) if w.dtype == "bf16"
                                 else b0["q"][bi].astype(np.float64), float(b0["positions"][bi]))
                u = qr.reshape(w.Hkv, grp, w.D).sum(axis=1)
                dirs.append(u / np.linalg.norm(u, axis=1, keepdims=True))
            needle_dir = np.stack(dirs)
        self.b = b = W.make(w, needle_dir=needle_dir)
        self.bf16 = w.dtype == "bf16"
        # oracle-side arrays: allocated pages only, tables index them directly
        self.Kl, self.Vl, self.btl = b["K_pages"], b["V_pages"], b["bt_local"]
        summ = oracle.summary(self.Kl, self.btl, b["seq_lens"])
        self.summ_l = oracle.round_to_bf16(summ) if self.bf16 else summ.astype(np.float32)
        # device: full pool with pages at their physical ids
        d = dev()
        pool = b["pool_pages"]
        phys = torch.from_numpy(b["phys"].astype(np.int64)).to(d)
        self.K = torch.zeros((pool,) + self.Kl.shape[1:], dtype=torch.int16 if self.bf16 else torch.float32, device=d)
        self.V = torch.zeros((pool,) + self.Vl.shape[1:], dtype=self.K.dtype, device=d)
        self.S = torch.zeros((pool, w.Hkv, w.D), dtype=self.K.dtype, device=d)
        self.K[phys] = t(self.Kl)
        self.V[phys] = t(self.Vl)
        self.S[phys] = t(self.summ_l)
        self.q, self.qv = t(b["q"]), t(b["qv"])
        self.bt, self.L, self.pos = t(b["bt"]), t(b["seq_lens"]), t(b["positions"])
        self.anchor, self.recent = t(b["anchor"]), t(b["recent"])
        if "k_mid" in b:
            self.k_mid_h = b["k_mid"]
        else:
            N = w.n_pages
            self.k_mid_h = np.array([
                oracle.budget_from_ratio(int(N[i]), r[0], r[1], int(b["anchor"][i]), int(b["recent"][i]))
                - int(b["anchor"][i]) - int(b["recent"][i]) for i, r in enumerate(b["ratio"])],
                dtype=np.int32)
        self.k_mid = t(self.k_mid_h)

    @property
    def max_pages(self):
        return self.b["bt"].shape[1]

    def budget(self):
        return int((self.b["anchor"] + self.b["recent"] + self.k_mid_h).max())


def row_errors(gpu, ref):
    """max |gpu - ref| / ||ref|| over the last axis; rows with ref == 0 must match exactly."""
    num = np.abs(gpu - ref).max(axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    err = np.where(den > 0, num / np.where(den > 0, den, 1.0), np.where(num == 0, 0.0, np.inf))
    return err


def u_norms(case):
    """||u_g|| per (b, g) from the oracle's rotation."""
    w, b = case.w, case.b
    grp = w.Hq // w.Hkv
    out = np.zeros((w.B, w.Hkv))
    for bi in range(w.B):
        qh = oracle.widen(b["q"][bi]) if case.bf16 else b["q"][bi].astype(np.float64)
        qr = oracle.rope(qh, float(b["positions"][bi]))
        out[bi] = np.linalg.norm(qr.reshape(w.Hkv, grp, w.D).sum(axis=1), axis=1)
    return out


def check_scores(case, s_gpu):
    """GPU scores vs the oracle's fp64 scores, within SCORE_TOL * ||u|| * ||row||."""
    w, b = case.w, case.b
    ref = oracle.score(b["q"], b["positions"], case.summ_l, case.btl, b["seq_lens"], w.Hkv)
    N = w.n_pages
    un = u_norms(case)
    worst = 0.0
    for bi in range(w.B):
        n = int(N[bi])
        assert np.all(np.isneginf(s_gpu[bi, :, n:])), "scores past the sequence must be -inf"
        rows = case.summ_l[case.btl[bi, :n]]
        rn = np.linalg.norm(oracle.widen(rows) if case.bf16 else rows.astype(np.float64), axis=-1)
        bound = SCORE_TOL * un[bi][:, None] * rn.T + 1e-30
        e = np.abs(s_gpu[bi, :, :n] - ref[bi, :, :n]) / bound
        worst = max(worst, float(e.max()) if e.size else 0.0)
    assert worst <= 1.0, f"score error {worst:.3f} x tolerance"
    return ref


def workspace(B, q_len, Hq, Hkv, D):
    return torch.empty(kap.attn_workspace_bytes(B, q_len, Hq, Hkv, D), dtype=torch.uint8, device=dev())
