"""The page-split tag A<a>R<r>K<k> (KRI page, A<a>R<r>K<k> tag section).

A tag names a selection split: the first a pages of the sequence (anchors),
the last r pages (recents), and the k best pages of the middle [a, N - r) by
score.  k counts the middle pages only, so the total budget is a + r + k.  The
form A<a>R<r>K* leaves k open: it follows from a page budget (for instance one
derived from a retention ratio by kap_budget_from_ratio) as budget - a - r,
clamped to the middle.  Host-side configuration only: the selection itself runs
in kap_select_topk / kap_select_compact with the three numbers.
"""
import re
from typing import Optional, Tuple

_TAG = re.compile(r"A(\d+)R(\d+)K(\d+|\*)")


def parse_split_tag(tag: str) -> Tuple[int, int, Optional[int]]:
    """"A1R2K110" -> (1, 2, 110); "A4R4K*" -> (4, 4, None).  Raises ValueError
    on anything else (surrounding blanks are allowed, nothing else is)."""
    m = _TAG.fullmatch(tag.strip()) if isinstance(tag, str) else None
    if m is None:
        raise ValueError(f"not an A<a>R<r>K<k> tag: {tag!r}")
    a, r, k = m.groups()
    return int(a), int(r), None if k == "*" else int(k)


def format_split_tag(anchor: int, recent: int, k_mid: Optional[int] = None) -> str:
    """(1, 2, 110) -> "A1R2K110"; k_mid None gives the open form "A1R2K*"."""
    for name, v in (("anchor", anchor), ("recent", recent), ("k_mid", k_mid)):
        if v is not None and (not isinstance(v, (int,)) or isinstance(v, bool) or v < 0):
            raise ValueError(f"{name} must be a non-negative int, got {v!r}")
    return f"A{anchor}R{recent}K{'*' if k_mid is None else k_mid}"


def middle_count(n_pages: int, anchor: int, recent: int, k_mid: Optional[int] = None,
                 budget: Optional[int] = None) -> int:
    """Middle pages the split takes from a sequence of n_pages: k_mid, or
    budget - a - r for the open form, clamped to the middle's size (0 when the
    anchors and recents cover the sequence)."""
    if (k_mid is None) == (budget is None):
        raise ValueError("give exactly one of k_mid and budget")
    k = k_mid if k_mid is not None else budget - anchor - recent
    return max(0, min(k, n_pages - anchor - recent))
