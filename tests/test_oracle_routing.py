"""Pins for the oracle's routing, dispatch and block table.

Each is checked against something other than itself: brute force over all
k-subsets, numpy's stable argsort and bincount, torch's fp64 softmax and
sigmoid, and the structural invariants of a bijective dispatch.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle


def _brute_topk(row, k):
    """The unique k-subset whose every member beats every non-member under
    the order (score desc, index asc), listed in that order."""
    E = len(row)

    def beats(a, b):
        return row[a] > row[b] or (row[a] == row[b] and a < b)

    found = []
    for sub in itertools.combinations(range(E), k):
        rest = [e for e in range(E) if e not in sub]
        if all(beats(a, b) for a in sub for b in rest):
            found.append(sub)
    assert len(found) == 1
    sub = list(found[0])
    sub.sort(key=lambda e: (-row[e], e))
    return sub


@pytest.mark.parametrize("E,k", [(6, 1), (6, 3), (7, 7), (8, 2)])
def test_topk_brute_force_with_ties(E, k):
    rng = np.random.default_rng(E * 10 + k)
    # few distinct values -> many exact ties; include signed zeros
    vals = np.array([-1.0, -0.0, 0.0, 0.5, 2.0], dtype=np.float32)
    scores = vals[rng.integers(0, len(vals), size=(40, E))]
    ids, _ = oracle.route(scores, k, oracle.SCORE_SOFTMAX)
    for t in range(40):
        assert list(ids[t]) == _brute_topk(scores[t].astype(np.float64), k)


def test_topk_matches_stable_argsort():
    rng = np.random.default_rng(5)
    scores = rng.standard_normal((300, 64)).astype(np.float32)
    scores[::7, 3] = scores[::7, 9]        # planted ties
    ids, _ = oracle.route(scores, 8, oracle.SCORE_SIGMOID)
    ref = np.argsort(-scores.astype(np.float64), axis=1, kind="stable")[:, :8]
    np.testing.assert_array_equal(ids, ref)


def test_softmax_weights_are_renormalised_full_softmax():
    rng = np.random.default_rng(6)
    s = rng.standard_normal((50, 16)).astype(np.float32)
    ids, w = oracle.route(s, 4, oracle.SCORE_SOFTMAX)
    full = torch.softmax(torch.from_numpy(s.astype(np.float64)), dim=1).numpy()
    sel = np.take_along_axis(full, ids.astype(np.int64), axis=1)
    np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-13, atol=0)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=1e-14)


def test_softmax_k_equals_e_is_full_softmax():
    rng = np.random.default_rng(7)
    s = rng.standard_normal((20, 8)).astype(np.float32)
    ids, w = oracle.route(s, 8, oracle.SCORE_SOFTMAX)
    full = torch.softmax(torch.from_numpy(s.astype(np.float64)), dim=1).numpy()
    np.testing.assert_allclose(w, np.take_along_axis(full, ids.astype(np.int64), 1),
                               rtol=1e-13)


def test_sigmoid_and_probs_weights():
    rng = np.random.default_rng(8)
    s = rng.standard_normal((30, 32)).astype(np.float32)
    ids, w = oracle.route(s, 8, oracle.SCORE_SIGMOID)
    sig = torch.sigmoid(torch.from_numpy(s.astype(np.float64))).numpy()
    sel = np.take_along_axis(sig, ids.astype(np.int64), 1)
    np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-13)
    p = rng.dirichlet(np.full(32, 0.1), size=30).astype(np.float32)
    ids, w = oracle.route(p, 4, oracle.SCORE_PROBS)
    sel = np.take_along_axis(p.astype(np.float64), ids.astype(np.int64), 1)
    np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-15)


def test_dispatch_against_bincount_and_stable_sort():
    rng = np.random.default_rng(9)
    T, k, E = 97, 4, 13
    s = rng.standard_normal((T, E)).astype(np.float32)
    s[:, 5] -= 50.0                          # expert 5 never chosen
    ids, _ = oracle.route(s, k, oracle.SCORE_SOFTMAX)
    counts, indptr, gather, inv = oracle.dispatch(ids, E)
    np.testing.assert_array_equal(counts, np.bincount(ids.ravel(), minlength=E))
    assert counts[5] == 0 and counts.sum() == T * k
    np.testing.assert_array_equal(indptr, np.concatenate([[0], np.cumsum(counts)]))
    np.testing.assert_array_equal(gather, np.argsort(ids.ravel(), kind="stable"))
    # bijection
    np.testing.assert_array_equal(gather[inv], np.arange(T * k))
    np.testing.assert_array_equal(np.sort(gather), np.arange(T * k))
    # each slot holds a row of its own expert
    for e in range(E):
        assert np.all(ids.ravel()[gather[indptr[e]:indptr[e + 1]]] == e)


@pytest.mark.parametrize("bm", [1, 16, 32, 128])
def test_tile_table_covers_every_row_once(bm):
    counts = np.array([0, 5, 16, 17, 0, 0, 128, 1, 300], dtype=np.int32)
    tab = oracle.tile_table(counts, bm)
    assert len(tab) == int(np.sum((counts + bm - 1) // bm))
    seen = {}
    for e, r0 in tab:
        assert counts[e] > 0 and r0 % bm == 0 and r0 < counts[e]
        for r in range(r0, min(r0 + bm, counts[e])):
            assert (e, r) not in seen
            seen[(e, r)] = 1
    assert len(seen) == counts.sum()
    # expert-major order
    assert np.all(np.diff(tab[:, 0]) >= 0)
