"""kap_decode_attn_noalloc (the allocation-free decode) against kap_decode_attn
through the C ABI: the same kernels over the same inputs, so out and lse must
match bit for bit.  Two calls in a row share the library's static scratch, the
second with a smaller input; both are also within the attention tolerance of
the oracle."""
import numpy as np
import pytest
import torch

import block_sparse_paged_page_amd as kap
import oracle
import workloads as W
from _gpu_util import LSE_TOL, TOL, Case, host, row_errors, t

pytestmark = pytest.mark.gpu


def _selected_view(c):
    cap = c.budget() + 3
    b = c.b
    s_ref = oracle.score(b["q"], b["positions"], c.summ_l, c.btl, b["seq_lens"], c.w.Hkv)
    sel, cnt = oracle.select(s_ref.astype(np.float32), b["seq_lens"], b["anchor"], b["recent"],
                             c.k_mid_h, cap, per_head=c.w.per_head)
    cbt, clog, clen, _ = kap.compact_view(t(sel), t(cnt), c.bt, c.L, c.pos, 1)
    return sel, cnt, cbt, clen, clog


def _both(c, table, lens, G, logical=None):
    w = c.w
    lse_a = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
    lse_b = torch.empty_like(lse_a)
    out_a = kap.decode_attn(c.q, c.pos, c.K, c.V, table, lens, G=G, lse=lse_a, logical=logical)
    out_b = kap.decode_attn_noalloc(c.q, c.pos, c.K, c.V, table, lens, G=G, lse=lse_b,
                                    logical=logical)
    torch.cuda.synchronize()
    assert torch.equal(out_a.view(torch.int16) if c.bf16 else out_a,
                       out_b.view(torch.int16) if c.bf16 else out_b)
    assert torch.equal(lse_a, lse_b)
    return out_b, lse_b


def _check_oracle(c, out, lse, keys, G):
    w, b = c.w, c.b
    ref, lref = oracle.attend(b["q"][:, None], b["positions"], c.Kl, c.Vl, c.btl, keys, G, w.Hkv)
    e = row_errors(host(out, c.bf16).reshape(ref[:, 0].shape), ref[:, 0])
    assert e.max() <= TOL[w.dtype], e.max()
    lg = lse.cpu().numpy()
    fin = np.isfinite(lref[:, 0])
    assert np.array_equal(np.isfinite(lg), fin)
    assert np.abs(lg[fin] - lref[:, 0][fin]).max() <= LSE_TOL[w.dtype]


def test_noalloc_decode_matches_workspace_decode_two_calls():
    # first call: Llama-shaped, three ragged requests, selected view
    print("[noalloc] call 1: llama-shaped B=3 selected view", flush=True)
    big = Case(W.spec("llama8b_32k", B=3, seq_lens=[4096, 3007, 1234]), aim_needles=True)
    sel, cnt, cbt, clen, clog = _selected_view(big)
    out, lse = _both(big, cbt, clen, 1, clog)
    _check_oracle(big, out, lse, oracle.keys_selected(sel, cnt, big.b["seq_lens"]), 1)
    # second call, smaller: one 32B-shaped request, full table
    print("[noalloc] call 2: 32B-shaped B=1 full table", flush=True)
    small = Case(W.spec("qwen32b_128k", B=1, seq_lens=[1500]))
    out, lse = _both(small, small.bt, small.L, 1)
    _check_oracle(small, out, lse, oracle.keys_full(small.b["seq_lens"]), 1)
    # and the first input once more after the smaller one
    print("[noalloc] call 3: llama-shaped again", flush=True)
    _both(big, cbt, clen, 1, clog)
