"""The host tier's eviction order (no GPU): least recently touched resident pages first, ties to
the lower page id (bw24 deep-dive page, section 6 item 3: LRU eviction on page access time)."""
import numpy as np

import memory_bound_autoregressive_amd as bw


def _brute(stamps, resident, n):
    cand = sorted((int(stamps[p]), p) for p in range(len(stamps)) if resident[p])
    return [p for _, p in cand[:n]]


def test_lru_order_matches_brute_force_with_ties():
    rng = np.random.default_rng(3)
    for trial in range(200):
        n_pages = int(rng.integers(0, 60))
        stamps = rng.integers(0, 6, n_pages).astype(np.uint64)  # many ties
        resident = (rng.random(n_pages) < 0.7).astype(np.uint8)
        n = int(rng.integers(0, 70))
        got = bw.bw_kv_lru_select(stamps, resident, n)
        assert got.tolist() == _brute(stamps, resident, n), trial


def test_lru_hand_case():
    # pages 0..5: page 3 untouched (not resident), pages 1 and 4 oldest (tie -> 1 first)
    stamps = np.array([5, 2, 9, 0, 2, 7], dtype=np.uint64)
    resident = np.array([1, 1, 1, 0, 1, 1], dtype=np.uint8)
    assert bw.bw_kv_lru_select(stamps, resident, 3).tolist() == [1, 4, 0]
    assert bw.bw_kv_lru_select(stamps, resident, 10).tolist() == [1, 4, 0, 5, 2]
    assert bw.bw_kv_lru_select(stamps, resident, 0).tolist() == []


def test_tier_calls_reject_null_handles_without_a_gpu():
    L = bw.lib()
    assert L.bw_kv_tier_create(None, 4, None) == bw.BW_EINVAL
    assert L.bw_kv_tier_touch(None, None, None, 1, 1, 1) == bw.BW_EINVAL
    assert L.bw_kv_tier_evict_lru(None, 1, None, None, None, None) == bw.BW_EINVAL
    assert L.bw_kv_tier_restore(None, None, None, 1, None) == bw.BW_EINVAL
    assert L.bw_kv_tier_wait(None, None) == bw.BW_EINVAL
    assert L.bw_kv_tier_free(None) == bw.BW_OK
    assert L.bw_kv_lru_select(None, None, 1, 1, None, None) == bw.BW_EINVAL
