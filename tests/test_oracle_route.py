"""Pins of the oracle's top-2 routing and expert sort (no GPU)."""
import itertools
import math

import numpy as np
import torch

from oracle import route_sort, route_top2


def _brute_top2(row):
    order = sorted(range(len(row)), key=lambda e: (-float(row[e]), e))
    return order[0], order[1]


def test_top2_brute_force_random():
    rng = np.random.default_rng(11)
    for E in (2, 3, 4, 8, 16, 64):
        l = (rng.standard_normal((50, E)) * 1.5).astype(np.float32)
        ids, w = route_top2(l)
        for t in range(50):
            assert tuple(ids[t]) == _brute_top2(l[t])


def test_top2_exhaustive_orderings_e4():
    for perm in itertools.permutations(range(4)):
        l = np.array([perm], dtype=np.float32)          # distinct values 0..3
        ids, _ = route_top2(l)
        assert ids[0, 0] == perm.index(3) and ids[0, 1] == perm.index(2)


def test_top2_ties_lower_id_first():
    l = np.array([[1.0, 2.0, 2.0, 0.5],
                  [0.0, 0.0, 0.0, 0.0],
                  [3.0, 1.0, 3.0, 3.0],
                  [-1.0, 5.0, -1.0, -1.0]], dtype=np.float32)
    ids, w = route_top2(l)
    assert ids.tolist() == [[1, 2], [0, 1], [0, 2], [1, 0]]
    assert np.allclose(w[1], [0.5, 0.5]) and np.allclose(w[2], [0.5, 0.5])


def test_weights_closed_form_and_invariants():
    rng = np.random.default_rng(12)
    l = (rng.standard_normal((200, 8)) * 1.5).astype(np.float32)
    ids, w = route_top2(l)
    l0 = l[np.arange(200), ids[:, 0]].astype(np.float64)
    l1 = l[np.arange(200), ids[:, 1]].astype(np.float64)
    w0 = np.array([1.0 / (1.0 + math.exp(b - a)) for a, b in zip(l0, l1)])
    assert np.allclose(w[:, 0], w0, rtol=0, atol=1e-15)
    assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-15)
    assert np.all(w[:, 0] >= w[:, 1])
    assert np.all(ids[:, 0] != ids[:, 1])


def test_weights_match_torch_softmax_topk():
    rng = np.random.default_rng(13)
    l = (rng.standard_normal((100, 8)) * 1.5).astype(np.float64)
    ids, w = route_top2(l.astype(np.float32))
    lt = torch.from_numpy(l.astype(np.float32).astype(np.float64))
    p = torch.softmax(lt, dim=1)
    tv, ti = torch.topk(p, 2, dim=1)
    tw = tv / tv.sum(1, keepdim=True)
    assert np.array_equal(ti.numpy(), ids)
    assert np.allclose(tw.numpy(), w, rtol=0, atol=1e-14)


def test_sort_invariants_and_brute_force():
    rng = np.random.default_rng(14)
    for T, E in ((1, 2), (16, 4), (32, 8), (257, 8), (1000, 5)):
        l = rng.standard_normal((T, E)).astype(np.float32)
        ids, _ = route_top2(l)
        counts, offsets, sp, pos = route_sort(ids, E)
        assert counts.sum() == 2 * T and offsets[0] == 0 and offsets[E] == 2 * T
        assert np.array_equal(np.diff(offsets), counts)
        assert np.array_equal(np.sort(sp), np.arange(2 * T))
        assert np.array_equal(pos[sp], np.arange(2 * T))
        # brute force: walk the experts, list their pairs in increasing pair id
        expect = []
        for e in range(E):
            for p in range(2 * T):
                if ids[p // 2, p % 2] == e:
                    expect.append(p)
        assert np.array_equal(sp, expect)
        for e in range(E):
            seg = sp[offsets[e]:offsets[e + 1]]
            assert np.all(ids.reshape(-1)[seg] == e)
            assert np.all(np.diff(seg) > 0)


def test_sort_empty_experts():
    ids = np.array([[0, 3], [3, 0], [0, 3]], dtype=np.int32)
    counts, offsets, sp, pos = route_sort(ids, 6)
    assert counts.tolist() == [3, 0, 0, 3, 0, 0]
    assert offsets.tolist() == [0, 3, 3, 3, 6, 6, 6]
    assert sp.tolist() == [0, 3, 4, 1, 2, 5]
