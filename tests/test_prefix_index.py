"""The library's host-side prefix-block index (C++, CPU only) against the
oracle's PrefixCache: identical results, operation by operation, on random
and chat-shaped workloads."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_write_amd as pa


def _insert_both(idx, ref, tokens, ids):
    want = ref.insert(tokens, ids)
    if want is None:
        with pytest.raises(pa.PAError) as e:
            idx.insert(tokens, ids)
        assert e.value.status == pa.PA_ERR_INVALID_ARG
    else:
        assert idx.insert(tokens, ids) == want
    return want


def test_random_operations_match_the_oracle():
    """4000 random lookups, registrations (with reused, duplicate and
    negative ids) and removals over a small token alphabet, so that equal
    block contents recur at different positions and under different
    prefixes."""
    g = torch.Generator().manual_seed(2024)
    ri = lambda lo, hi: int(torch.randint(lo, hi, (1,), generator=g))  # noqa: E731
    idx, ref = pa.PrefixIndex(400), oracle.PrefixCache(400)
    stems = [torch.randint(0, 3, (ri(0, 120),), generator=g).tolist() for _ in range(12)]
    for step in range(4000):
        toks = stems[ri(0, len(stems))] + torch.randint(0, 3, (ri(0, 80),), generator=g).tolist()
        op = ri(0, 10)
        if op < 4:
            assert idx.match(toks) == ref.match(toks), step
        elif op < 8:
            n = len(toks) // 16 + ri(-1, 2)
            ids = torch.randint(-1 if ri(0, 8) == 0 else 0, 600, (max(n, 0),), generator=g).tolist()
            _insert_both(idx, ref, toks, ids)
        else:
            b = ri(0, 600)
            assert idx.remove(b) == ref.remove(b), step
        assert len(idx) == len(ref), step
    assert len(ref) > 50          # the run exercised a populated index


def test_capacity_limit_matches_the_oracle():
    g = torch.Generator().manual_seed(7)
    idx, ref = pa.PrefixIndex(10), oracle.PrefixCache(10)
    next_id = 0
    for _ in range(300):
        toks = torch.randint(0, 2, (int(torch.randint(16, 100, (1,), generator=g)),),
                             generator=g).tolist()
        ids = list(range(next_id, next_id + len(toks) // 16))
        next_id += len(ids)
        if torch.rand(1, generator=g).item() < 0.2 and next_id > 10:
            ids[0] = int(torch.randint(0, next_id - 1, (1,), generator=g))   # reuse an old block
        _insert_both(idx, ref, toks, ids)
        assert len(idx) == len(ref) <= 10
        assert idx.match(toks) == ref.match(toks)


def test_multi_turn_chat_hits():
    """Each turn re-sends the whole conversation: every earlier full block is
    a hit, and only the new tail registers (the warm prefix-cache pattern)."""
    g = torch.Generator().manual_seed(3)
    idx, ref = pa.PrefixIndex(100_000), oracle.PrefixCache(100_000)
    system = torch.randint(0, 50_000, (300,), generator=g).tolist()
    next_id = 0
    for user in range(8):
        conv = list(system)
        for turn in range(6):
            conv += torch.randint(0, 50_000, (int(torch.randint(20, 200, (1,), generator=g)),),
                                  generator=g).tolist()
            hit = idx.match(conv)
            assert hit == ref.match(conv)
            if turn > 0 or user > 0:
                assert len(hit) >= len(system) // 16
            nb = len(conv) // 16
            ids = hit + list(range(next_id, next_id + nb - len(hit)))
            next_id += nb - len(hit)
            assert _insert_both(idx, ref, conv, ids) == nb - len(hit)
            assert idx.match(conv) == ids
    assert len(idx) == len(ref)


def test_prefix_index_validation():
    lib = pa.load_library()
    h = ctypes.c_void_p()
    assert lib.pa_prefix_index_create(0, ctypes.byref(h)) == pa.PA_ERR_INVALID_ARG
    assert lib.pa_prefix_index_create(5, None) == pa.PA_ERR_INVALID_ARG
    assert lib.pa_prefix_index_create(5, ctypes.byref(h)) == pa.PA_OK and h.value
    n = ctypes.c_int32()
    toks = np.arange(32, dtype=np.int32)
    ids = np.array([3, 4], dtype=np.int32)
    assert lib.pa_prefix_index_match(None, toks.ctypes.data, 32, ids.ctypes.data,
                                     ctypes.byref(n)) == pa.PA_ERR_INVALID_ARG
    assert lib.pa_prefix_index_match(h, toks.ctypes.data, -1, ids.ctypes.data,
                                     ctypes.byref(n)) == pa.PA_ERR_INVALID_ARG
    assert lib.pa_prefix_index_match(h, None, 32, ids.ctypes.data,
                                     ctypes.byref(n)) == pa.PA_ERR_INVALID_ARG
    assert lib.pa_prefix_index_match(h, None, 15, None, ctypes.byref(n)) == pa.PA_OK
    assert n.value == 0
    assert lib.pa_prefix_index_insert(h, toks.ctypes.data, 32, ids.ctypes.data, -1,
                                      ctypes.byref(n)) == pa.PA_ERR_INVALID_ARG
    assert lib.pa_prefix_index_insert(h, toks.ctypes.data, 32, ids.ctypes.data, 2,
                                      None) == pa.PA_ERR_INVALID_ARG
    assert lib.pa_prefix_index_insert(h, toks.ctypes.data, 32, ids.ctypes.data, 2,
                                      ctypes.byref(n)) == pa.PA_OK and n.value == 2
    assert lib.pa_prefix_index_size(h) == 2 and lib.pa_prefix_index_size(None) == -1
    assert lib.pa_prefix_index_remove(h, 3, ctypes.byref(n)) == pa.PA_OK and n.value == 2
    assert lib.pa_prefix_index_remove(None, 3, ctypes.byref(n)) == pa.PA_ERR_INVALID_ARG
    lib.pa_prefix_index_destroy(h)
    lib.pa_prefix_index_destroy(None)
