"""Writes the stored needle directions of the benchmark workloads into
workloads/aim/ (test infrastructure: run it by hand after any change to the
query draws).

Needle keys are planted along the direction the page scorer sees: the unit
vector of the group-summed query heads of KV group g rotated at the request's
position, u_g / |u_g| with u_g = sum over the heads h of group g of
RoPE(q_h, P) (KRI page, KRI-Q: query . block-mean K; KAP paper, executor: the
query is rotated at its full-sequence logical position).  The rotation here is
the oracle's (oracle.rope, fp64); the queries are the generator's own draws.
The benchmark reads the resulting .npz files as plain data, so no oracle code
runs there; each file also holds, per request, a hash of the query bits and the
position it was made from, which workloads.aimed_dirs() checks.

    python tests/golden/make_needle_dirs.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
OUT = os.path.join(ROOT, "workloads", "aim")
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads as W  # noqa: E402

# the benchmark workloads with needles, at their largest batch
WORKLOADS = {"qwen32b_128k": 4, "llama8b_32k": 8, "mixed_serving": 64}


def aimed(name, B):
    """Unit directions [B][Hkv][D] (fp64) and the request keys of a workload."""
    w = W.spec(name, B=B) if name != "mixed_serving" else W.spec(name)
    b = W.make(w, with_kv=False)
    grp = w.Hq // w.Hkv
    dirs = np.zeros((w.B, w.Hkv, w.D), dtype=np.float64)
    for bi in range(w.B):
        qh = oracle.widen(b["q"][bi]) if w.dtype == "bf16" else b["q"][bi].astype(np.float64)
        u = oracle.rope(qh, float(b["positions"][bi])).reshape(w.Hkv, grp, w.D).sum(axis=1)
        dirs[bi] = u / np.linalg.norm(u, axis=1, keepdims=True)
    keys = np.array([W.request_key(b["q"][bi], int(b["positions"][bi])) for bi in range(w.B)])
    return dirs, keys


def main():
    os.makedirs(OUT, exist_ok=True)
    for name, B in WORKLOADS.items():
        dirs, keys = aimed(name, B)
        path = os.path.join(OUT, f"{name}.npz")
        np.savez_compressed(path, dirs=dirs.astype(np.float32), keys=keys)
        print(f"wrote {path}: {dirs.shape}", flush=True)


if __name__ == "__main__":
    main()
