"""Throughput of the selected-KV paged decode attention path on one MI355X.

Workload (the 128K-context, 32B-class configuration): batch B (default 4) of
131072-token requests, 64 query heads, 8 KV heads, head_dim 128, bf16 KV in
16-token pages scattered over the pool, retention s = 451/8192 pages
(A1R2K448), 1 % needle pages.  One step is one proposal-verification cycle of
one attention layer, every stage of the path:
  route   : kap_score_blocks -> kap_select_topk -> kap_compact_view
  propose : k = 4 x kap_decode_attn over the compact view (tokens at P .. P+3)
  verify  : kap_verify_attn, 4 queries at 131072..131075 over all 8192 pages
Each call reads a different layer copy of the pool (R copies, rotating), so
no call finds its bytes in the 256 MB Infinity Cache left by the previous one.

value = B * k proposal tokens per cycle / cycle time (tokens/s).  Per-call
durations come from HIP events on the launch stream inside the timed region.
The full-context decode (the same kernel over the whole table) is timed
separately for the comparison.  The CPU baseline times the oracle on request 0
of the same batch.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import block_sparse_paged_page_amd as kap  # noqa: E402
import workloads as W  # noqa: E402

METRIC = "selected-KV decode attn tokens/s + achieved HBM GB/s vs full-ctx, 128K ctx"
HBM_PEAK_GBS = 8000.0
K_PROPOSE = 4
EB = 2  # bf16


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--batch", type=int, default=4)
    ap.add_argument("--layers", type=int, default=0, help="layer copies (0: auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quiet", action="store_true")
    return ap.parse_args()


def log(msg, quiet=False):
    if not quiet:
        print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Layer:
    def __init__(self, K, V, S):
        self.K, self.V, self.S = K, V, S


def algorithmic_bytes(w, b, sel_pages):
    """Bytes each call must move (K/V of visible tokens, tables, q, out, summaries)."""
    B, Hq, Hkv, D = w.B, w.Hq, w.Hkv, w.D
    L = b["seq_lens"].astype(np.int64)
    N = (L + 15) // 16
    kv_tok = Hkv * 2 * D * EB                      # K + V bytes per token, all KV heads
    q_bytes = B * Hq * D * EB
    # selected decode: tokens of the selected pages (all pages full at 131072)
    sel_tok = 0
    for bi in range(B):
        for p in sel_pages[bi]:
            sel_tok += min(16, int(L[bi]) - 16 * int(p))
    dec_sel = sel_tok * kv_tok + 4 * sum(len(s) for s in sel_pages) + 2 * q_bytes
    dec_full = int(L.sum()) * kv_tok + 4 * int(N.sum()) + 2 * q_bytes
    verify = int(L.sum()) * kv_tok + 4 * int(N.sum()) + 2 * w.q_len * q_bytes
    max_pages = b["bt"].shape[1]
    score = int(N.sum()) * Hkv * D * EB + 4 * int(N.sum()) + B * Hkv * max_pages * 4 + q_bytes
    return dict(decode_selected=dec_sel, decode_full=dec_full, verify=verify, score=score)


def read_traffic(kernel_key):
    """HBM traffic per launch recorded from rocprofv3 PMC runs, if the kernel source still matches."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "attn_qwen32b_128k_b4_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    src = os.path.join(ROOT, "block_sparse_paged_page_amd", "csrc", "attn.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    for line in open(path):
        if line.startswith("traffic:"):
            f = dict(kv.split("=") for kv in line.split()[1:])
            if f.get("kernel") == kernel_key and f.get("attn_sha") == sha:
                return float(f["bytes_per_launch"])
    return None


def cpu_baseline(w, b, K, V, sel_budget, quiet, min_s=10.0, max_s=30.0):
    """Oracle cycles (route + 4 selected decodes + one verify) over the batch's
    requests in turn, until at least min_s seconds of CPU work have run."""
    import oracle
    T0 = time.time()
    NA = w.alloc_pages
    starts = np.concatenate([[0], np.cumsum(NA)[:-1]])
    host = []
    for bi in range(w.B):
        ph = torch.from_numpy(b["phys"][starts[bi]:starts[bi] + NA[bi]].astype(np.int64)).to(K.device)
        Kh = K[ph].view(torch.int16).cpu().numpy().view(np.uint16)
        Vh = V[ph].view(torch.int16).cpu().numpy().view(np.uint16)
        btl = np.arange(int(NA[bi]), dtype=np.int32)[None]
        Lb = b["seq_lens"][bi:bi + 1]
        summ = oracle.round_to_bf16(oracle.summary(Kh, btl, Lb))
        host.append((Kh, Vh, btl, Lb, summ))
    log(f"cpu baseline inputs ready in {time.time() - T0:.1f}s", quiet)
    threads = oracle.num_threads()
    done = 0
    t0 = time.perf_counter()
    while True:
        bi = done % w.B
        Kh, Vh, btl, Lb, summ = host[bi]
        sl = slice(bi, bi + 1)
        s = oracle.score(b["q"][sl], b["positions"][sl], summ, btl, Lb, w.Hkv)
        sel, cnt = oracle.select(s.astype(np.float32), Lb, b["anchor"][sl], b["recent"][sl],
                                 b["k_mid"][sl], sel_budget)
        oracle.compact(sel, cnt, btl, Lb, b["positions"][sl], 1)
        keys = oracle.keys_selected(sel, cnt, Lb)
        for j in range(K_PROPOSE):
            oracle.attend(b["qv"][sl, j:j + 1], b["positions"][sl] + j, Kh, Vh, btl, keys, 1, w.Hkv)
        oracle.attend(b["qv"][sl], b["positions"][sl], Kh, Vh, btl, oracle.keys_full(Lb), 1, w.Hkv)
        done += 1
        dt = time.perf_counter() - t0
        if dt >= min_s or (dt >= max_s / 2 and done >= 1):
            break
    return dict(value=round(K_PROPOSE * done / dt, 3), unit="tokens/s", cores=threads, kind="oracle",
                sample=(f"{done} request-cycles of the same batch (requests taken in turn): each "
                        "is score+select+compact over 8192 pages, 4 selected-KV decodes over 451 "
                        f"pages and one 4-query verify over 131072 tokens; {dt:.1f} s of CPU time"))


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        print("bench.py: multi-GPU runs are not part of this build (one GPU per box); "
              "see DESIGN.md for how the path would shard.", file=sys.stderr)
        sys.exit(2)
    q = args.quiet
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = W.spec("qwen32b_128k", B=args.batch)
    B, Hq, Hkv, D = w.B, w.Hq, w.Hkv, w.D
    t0 = time.time()
    b = W.make_device(w, dev)
    torch.cuda.synchronize()
    log(f"generated {w.name} B={B} on device in {time.time() - t0:.1f}s", q)

    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    bt, L, pos = to(b["bt"]), to(b["seq_lens"]), to(b["positions"])
    anchor, recent, k_mid = to(b["anchor"]), to(b["recent"]), to(b["k_mid"])
    budget = int((b["anchor"] + b["recent"] + b["k_mid"]).max())
    cap = budget
    qv = to(b["qv"].view(np.int16)).view(torch.bfloat16)                 # [B][4][Hq][D]
    q_prop = [qv[:, j].contiguous() for j in range(K_PROPOSE)]           # proposal queries
    pos_prop = [pos + j for j in range(K_PROPOSE)]
    q_route = to(b["q"].view(np.int16)).view(torch.bfloat16)
    S0 = torch.zeros((b["pool_pages"], Hkv, D), dtype=torch.bfloat16, device=dev)
    kap.build_summary(b["K"], bt, L, S0)

    layer_bytes = 2 * b["K"].numel() * EB + S0.numel() * EB
    R = args.layers or max(8, int(math.ceil(16 * 2**30 / layer_bytes)))
    layers = [Layer(b["K"], b["V"], S0)]
    for _ in range(R - 1):
        layers.append(Layer(b["K"].clone(), b["V"].clone(), S0.clone()))
    torch.cuda.synchronize()
    log(f"{R} layer copies, {R * layer_bytes / 2**30:.1f} GiB", q)

    ws = torch.empty(kap.attn_workspace_bytes(B, w.q_len, Hq, Hkv, D), dtype=torch.uint8,
                     device=dev)
    scores = torch.empty((B, Hkv, bt.shape[1]), dtype=torch.float32, device=dev)
    sel = torch.empty((B, 1, cap), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, 1), dtype=torch.int32, device=dev)
    cview = (torch.empty((B, 1, cap), dtype=torch.int32, device=dev),
             torch.empty((B, 1, cap), dtype=torch.int32, device=dev),
             torch.empty((B, 1), dtype=torch.int32, device=dev),
             torch.empty((B, 1), dtype=torch.int64, device=dev))
    dec_out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    ver_out = torch.empty((B, w.q_len, Hq, D), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    n_ev = 3 + K_PROPOSE
    state = {"layer": 0}

    def next_layer():
        lay = layers[state["layer"] % R]
        state["layer"] += 1
        return lay

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        lay = next_layer()
        kap.score_blocks(q_route, pos, lay.S, bt, L, Hkv, scores=scores)
        kap.select_topk(scores, L, anchor, recent, k_mid, budget, cap, sel=sel, cnt=cnt)
        kap.compact_view(sel, cnt, bt, L, pos, 1, out=cview)
        if ev:
            ev[1].record(stream)
        for j in range(K_PROPOSE):
            lay = next_layer()
            kap.decode_attn(q_prop[j], pos_prop[j], lay.K, lay.V, cview[0], cview[2], G=1,
                            out=dec_out, workspace=ws)
            if ev:
                ev[2 + j].record(stream)
        lay = next_layer()
        kap.verify_attn(qv, pos, lay.K, lay.V, bt, L, out=ver_out, workspace=ws)
        if ev:
            ev[2 + K_PROPOSE].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    ms_step = 1e3 * t_total / args.steps
    route_ms = np.mean([e[0].elapsed_time(e[1]) for e in evs])
    dec_ms = np.mean([e[1 + j].elapsed_time(e[2 + j]) for e in evs for j in range(K_PROPOSE)])
    ver_ms = np.mean([e[1 + K_PROPOSE].elapsed_time(e[2 + K_PROPOSE]) for e in evs])

    # selected pages (for byte accounting) -- read once after timing
    sel_h = sel.cpu().numpy()[:, 0]
    cnt_h = cnt.cpu().numpy()[:, 0]
    sel_pages = [sel_h[i, :cnt_h[i]] for i in range(B)]
    nbytes = algorithmic_bytes(w, b, sel_pages)

    # full-context decode over the same pool (comparison)
    for _ in range(3):
        lay = next_layer()
        kap.decode_attn(q_prop[0], pos, lay.K, lay.V, bt, L, G=1, out=dec_out, workspace=ws)
    e0 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    e0[0].record(stream)
    for i in range(args.steps):
        lay = next_layer()
        kap.decode_attn(q_prop[0], pos, lay.K, lay.V, bt, L, G=1, out=dec_out, workspace=ws)
        e0[i + 1].record(stream)
    torch.cuda.synchronize()
    full_ms = np.mean([e0[i].elapsed_time(e0[i + 1]) for i in range(args.steps)])

    # measured read ceiling: 16-byte-load stream over 4 GiB (median of 10)
    probe = torch.zeros(4 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(2):
        kap.diag_stream_read(probe, sink)
    pe = [torch.cuda.Event(enable_timing=True) for _ in range(11)]
    pe[0].record(stream)
    for i in range(10):
        kap.diag_stream_read(probe, sink)
        pe[i + 1].record(stream)
    torch.cuda.synchronize()
    ceil_ms = sorted(pe[i].elapsed_time(pe[i + 1]) for i in range(10))[5]
    ceiling_gbs = probe.numel() / (ceil_ms * 1e-3) / 1e9
    del probe

    gbs = lambda nb, ms: nb / (ms * 1e-3) / 1e9  # noqa: E731
    ver_gbs = gbs(nbytes["verify"], ver_ms)
    traffic = read_traffic("verify")
    roofline = {"bound": "hbm", "kernel": "kap_verify_attn (prep + MFMA split-K partial + merge)",
                "achieved": round(ver_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ver_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                "measured_read_ceiling_GBps": round(ceiling_gbs, 1),
                "frac_of_measured_ceiling": round(ver_gbs / ceiling_gbs, 4),
                "bytes_per_launch": nbytes["verify"], "avg_launch_us": round(ver_ms * 1e3, 2)}
    s_meas = nbytes["decode_selected"] / nbytes["decode_full"]
    h = 0.952  # KAP paper Table 5 at 128K: s + (h - s) = 0.055 + 0.897
    result = {
        "metric": METRIC,
        "value": round(B * K_PROPOSE / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"qwen32b_128k: B={B}, Hq={Hq}, Hkv={Hkv}, D={D}, 131072-token context, "
                         f"16-token pages, s=451/8192 (A1R2K448 pooled), step = route + "
                         f"{K_PROPOSE} selected-KV decodes + 4-query full-context verify"),
            "global_batch": B, "seq_len": int(w.seq_lens[0]), "layer_copies": R,
        },
        "roofline": roofline,
        "kernels": {
            "route_us": round(route_ms * 1e3, 2),
            "decode_selected_us": round(dec_ms * 1e3, 2),
            "decode_selected_GBps": round(gbs(nbytes["decode_selected"], dec_ms), 1),
            "decode_full_us": round(full_ms * 1e3, 2),
            "decode_full_GBps": round(gbs(nbytes["decode_full"], full_ms), 1),
            "verify_us": round(ver_ms * 1e3, 2),
            "verify_GBps": round(ver_gbs, 1),
        },
        "full_ctx": {
            "decode_tokens_per_s": round(B / (full_ms * 1e-3), 1),
            "selected_decode_tokens_per_s": round(B / (dec_ms * 1e-3), 1),
            "selected_vs_full_decode_speedup": round(full_ms / dec_ms, 3),
            "s_meas_bytes": round(s_meas, 5),
            "phase_boundary_break_even_W_over_KV": round((h - s_meas) / (1 - h), 3),
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, b, b["K"], b["V"], cap, q)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
