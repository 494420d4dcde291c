"""The A<a>R<r>K<k> split tag (KRI page, A<a>R<r>K<k> tag section): parsing,
formatting, and the middle count it gives, checked against the page's worked
example and against the oracle's selection."""
import numpy as np
import pytest

import block_sparse_paged_page_amd as kap
import oracle


def test_parse_and_format_round_trip():
    for tag, want in (("A1R2K110", (1, 2, 110)), ("A1R2K448", (1, 2, 448)), ("A0R0K8", (0, 0, 8)),
                      ("A4R4K*", (4, 4, None)), (" A1R2K13 ", (1, 2, 13))):
        assert kap.parse_split_tag(tag) == want
        assert kap.parse_split_tag(kap.format_split_tag(*want)) == want
    assert kap.format_split_tag(1, 2) == "A1R2K*"


@pytest.mark.parametrize("bad", ["", "A1R2", "a1r2k3", "A1R2K-3", "A1 R2 K3", "A1R2K3x", "K3A1R2",
                                 "A1R2K3.5", None, 5])
def test_malformed_tags_are_rejected(bad):
    with pytest.raises(ValueError):
        kap.parse_split_tag(bad)


def test_format_rejects_negative_or_non_integer_counts():
    for args in ((-1, 2, 3), (1, 2.0, 3), (1, 2, -5), (True, 2, 3)):
        with pytest.raises(ValueError):
            kap.format_split_tag(*args)


def test_worked_example_of_the_tag_section():
    # 128 blocks, budget 16 as A1R2K13: anchor {0}, recents {126, 127}, best 13 of [1, 126)
    a, r, k = kap.parse_split_tag("A1R2K13")
    assert a + r + k == 16
    assert kap.middle_count(128, a, r, k_mid=k) == 13
    assert kap.middle_count(128, a, r, budget=16) == 13
    rng = np.random.default_rng(5)
    s = rng.standard_normal((1, 1, 128)).astype(np.float32)
    L = np.array([128 * 16], np.int32)
    sel, cnt = oracle.select(s, L, np.array([a], np.int32), np.array([r], np.int32),
                             np.array([k], np.int32), 16)
    got = sel[0, 0, :cnt[0, 0]]
    assert cnt[0, 0] == 16 and got[0] == 0 and list(got[-2:]) == [126, 127]
    mid = got[1:-2]
    best = 1 + np.argsort(-s[0, 0, 1:126], kind="stable")[:13]
    assert sorted(mid.tolist()) == sorted(best.tolist())


def test_middle_count_clamps():
    assert kap.middle_count(10, 4, 4, budget=64) == 2       # the middle has only 2 pages
    assert kap.middle_count(6, 4, 4, k_mid=3) == 0          # anchors and recents cover it
    assert kap.middle_count(100, 1, 2, budget=2) == 0       # budget below a + r
    with pytest.raises(ValueError):
        kap.middle_count(100, 1, 2)
    with pytest.raises(ValueError):
        kap.middle_count(100, 1, 2, k_mid=3, budget=6)
