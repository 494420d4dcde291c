"""Memory-bound cost model of one proposal-verification cycle (fp64, test/bench side).

Source: the KAP tutorial page (agifrontier, "phase boundary" section) gives the
equations that the KAP paper's Section 4 names but whose text lost them:
  Cost_base = (1 + k h) (W_main + KV)
  Cost_plan = k (W_prop + s KV) + (W_main + KV)
and, with W_prop = W_main, Cost_plan < Cost_base reduces to the phase boundary
  (h - s) KV > (1 - h) W_main,
with the necessary condition h > s and the critical KV size
  KV_crit = (1 - h) W_main / (h - s).
s is the retained-KV ratio (bytes the proposal reads over the full KV bytes) and
h the proposal acceptance rate (KAP paper, Section 4 definitions).
"""


def cost_base(k: float, h: float, w_main: float, kv: float) -> float:
    """Full-context decoding spend for the 1 + k h tokens a cycle yields."""
    return (1.0 + k * h) * (w_main + kv)


def cost_plan(k: float, s: float, w_prop: float, w_main: float, kv: float) -> float:
    """k selected-KV proposal steps plus one full-context verification."""
    return k * (w_prop + s * kv) + (w_main + kv)


def phase_boundary_holds(h: float, s: float, w_main: float, kv: float) -> bool:
    """True when (h - s) KV > (1 - h) W_main (positive-speedup regime)."""
    return (h - s) * kv > (1.0 - h) * w_main


def kv_crit(h: float, s: float, w_main: float) -> float:
    """Smallest KV cost for which the plan pays off; inf when h <= s."""
    if h <= s:
        return float("inf")
    return (1.0 - h) * w_main / (h - s)


def break_even_w_over_kv(h: float, s: float) -> float:
    """Largest W_main / KV ratio that still gives a speedup: (h - s) / (1 - h)."""
    if h >= 1.0:
        return float("inf")
    return (h - s) / (1.0 - h)


def retention_ratio(proposal_bytes: float, full_bytes: float) -> float:
    """s measured as bytes a proposal step reads over bytes a full decode reads."""
    return proposal_bytes / full_bytes
