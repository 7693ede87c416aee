"""The binding's result container for batches (CPU only)."""
import numpy as np
import pytest

from sift_descriptor_nearest_amd import MatchLists


def make():
    buf = np.arange(40, dtype=np.uint32).reshape(20, 2)
    offs = np.array([0, 5, 5, 12, 20])       # capacity of each pair, cumulated
    cnt = np.array([3, 0, 7, 2])
    return buf, MatchLists(buf, offs, cnt)


def test_items_are_views_trimmed_to_counts():
    buf, m = make()
    assert len(m) == 4
    assert m[0].tolist() == buf[0:3].tolist()
    assert m[1].shape == (0, 2)
    assert m[2].tolist() == buf[5:12].tolist()
    assert m[3].tolist() == buf[12:14].tolist()
    assert np.shares_memory(m[2], buf)
    assert m[-1].tolist() == m[3].tolist()
    assert [len(x) for x in m] == [3, 0, 7, 2]
    assert [len(x) for x in m[1:3]] == [0, 7]
    assert m[np.int64(2)].shape == (7, 2)


def test_out_of_range():
    _, m = make()
    for q in (4, -5, 100):
        with pytest.raises(IndexError):
            m[q]
