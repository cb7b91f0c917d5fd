"""Pins of the oracle's selectors (CPU only): brute force over heavy ties."""
import numpy as np
import pytest

from oracle.select import n_selected, top_n_ascending


def _brute(keys, n):
    order = sorted(range(len(keys)), key=lambda i: (-float(keys[i]), i))
    return sorted(order[:n])


@pytest.mark.parametrize("T", [1, 7, 33, 200, 1000])
def test_against_brute_force_with_ties(T):
    rng = np.random.default_rng(T)
    for trial in range(20):
        keys = rng.integers(0, 4, size=T).astype(np.float32) * np.float32(0.5)
        if trial % 3 == 0:
            keys = rng.random(T).astype(np.float32)
        for n in {1, max(1, T // 3), T}:
            got = top_n_ascending(keys, n)
            assert list(got) == _brute(keys, n)


def test_all_equal_keys_take_lowest_indices():
    np.testing.assert_array_equal(top_n_ascending(np.ones(50, np.float32), 7), np.arange(7))
    np.testing.assert_array_equal(top_n_ascending(np.zeros(9, np.float32), 9), np.arange(9))


def test_hand_example():
    keys = np.array([0.5, 2.0, 2.0, 0.1, 3.0, 2.0], np.float32)
    # order by (-key, index): 4 (3.0), 1, 2, 5 (2.0 ties by index), 0, 3
    np.testing.assert_array_equal(top_n_ascending(keys, 3), [1, 2, 4])
    np.testing.assert_array_equal(top_n_ascending(keys, 4), [1, 2, 4, 5])


def test_n_selected_rule():
    assert n_selected(0.25, 4096) == 1024      # exact product stays
    assert n_selected(0.1, 32768) == 3277      # 3276.8 rounds up
    assert n_selected(0.2, 8192) == 1639
    assert n_selected(0.5, 32) == 16
    assert n_selected(0.0, 10) == 1            # at least one row
    assert n_selected(1.0, 10) == 10
    assert n_selected(3.0, 10) == 10
    assert n_selected(0.5, 0) == 0


def test_rejects_non_finite():
    with pytest.raises(ValueError):
        top_n_ascending(np.array([1.0, np.nan], np.float32), 1)
