"""Pins for the oracle's router and permutation (CPU only)."""
import numpy as np
import pytest
from scipy.special import expit, softmax

from oracle import moe


def _bruteforce_topk(logits, k):
    out = []
    for row in logits:
        order = sorted(range(len(row)), key=lambda e: (-float(row[e]), e))
        out.append(order[:k])
    return np.array(out, dtype=np.int32)


@pytest.mark.parametrize("T,E,k", [(16, 8, 2), (33, 256, 8), (5, 64, 6), (7, 3, 3)])
def test_route_matches_sorted_bruteforce(T, E, k):
    rng = np.random.default_rng(T * 1000 + E)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[0, :] = np.float32(0.25)           # full tie row
    lg[1, 1::2] = lg[1, 0::2][: len(lg[1, 1::2])]   # pairwise ties
    idx, w = moe.route(lg, k)
    np.testing.assert_array_equal(idx, _bruteforce_topk(lg, k))
    p = softmax(lg.astype(np.float64), axis=1)      # scipy's softmax, fp64
    np.testing.assert_allclose(w, np.take_along_axis(p, idx.astype(np.int64), 1), rtol=1e-13)


def test_route_negative_zero_ties_go_to_lower_id():
    lg = np.array([[-0.0, 0.0, -1.0, 0.0]], dtype=np.float32)
    idx, _ = moe.route(lg, 3)
    np.testing.assert_array_equal(idx[0], [0, 1, 3])


def test_route_equal_logits():
    E, k = 16, 4
    idx, w = moe.route(np.zeros((3, E), np.float32), k)
    np.testing.assert_array_equal(idx, np.tile(np.arange(k), (3, 1)))
    np.testing.assert_allclose(w, 1.0 / E, rtol=0, atol=1e-16)


def test_route_k_equals_E_and_single_expert():
    rng = np.random.default_rng(1)
    lg = rng.standard_normal((4, 6)).astype(np.float32)
    idx, w = moe.route(lg, 6)
    assert sorted(idx[0].tolist()) == list(range(6))
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-14)
    idx1, w1 = moe.route(lg[:, :1], 1)
    assert np.all(idx1 == 0) and np.all(w1 == 1.0)


def test_route_two_experts_closed_form():
    lg = np.array([[0.3, -1.2], [2.0, 2.5], [0.0, 0.0]], dtype=np.float32)
    idx, w = moe.route(lg, 1)
    l64 = lg.astype(np.float64)
    want = expit(np.abs(l64[:, 0] - l64[:, 1]))     # p(top) = sigmoid(l_top - l_other)
    np.testing.assert_allclose(w[:, 0], want, rtol=1e-14)
    np.testing.assert_array_equal(idx[:, 0], [0, 1, 0])


def test_route_renorm():
    rng = np.random.default_rng(2)
    lg = rng.standard_normal((8, 32)).astype(np.float32)
    _, w = moe.route(lg, 4, renorm=True)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-14)


def _bruteforce_permute(idx, e0, n_local, shared):
    """Rows ordered by (local expert, flattened assignment index), written as a
    stable argsort rather than per-expert lists."""
    T, k = idx.shape
    g = idx.reshape(-1).astype(np.int64) - e0
    a = np.arange(T * k)
    local = (g >= 0) & (g < n_local)
    order = a[local][np.argsort(g[local], kind="stable")]
    src = order // k
    if shared:
        src = np.concatenate([src, np.arange(T)])
    counts = np.bincount(g[local], minlength=n_local)
    if shared:
        counts = np.concatenate([counts, [T]])
    return src, counts, order


@pytest.mark.parametrize("T,E,k,e0,nl,sh", [(16, 8, 2, 0, 8, False), (40, 256, 8, 0, 32, False),
                                           (40, 256, 8, 64, 32, True), (1, 256, 8, 0, 32, False),
                                           (0, 8, 2, 0, 8, True), (300, 64, 6, 0, 64, False)])
def test_permute_matches_bruteforce(T, E, k, e0, nl, sh):
    rng = np.random.default_rng(T + E + k + e0)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    idx, w = moe.route(lg, k) if T else (np.zeros((0, k), np.int32), np.zeros((0, k)))
    p = moe.permute(idx, w, e0, nl, sh)
    src, counts, order = _bruteforce_permute(idx, e0, nl, sh)
    np.testing.assert_array_equal(p.counts, counts)
    np.testing.assert_array_equal(p.row_src, src)
    assert p.offsets[0] == 0 and np.all(np.diff(p.offsets) == p.counts)
    # invariants
    n_loc = int(((idx - e0 >= 0) & (idx - e0 < nl)).sum())
    assert p.counts[:nl].sum() == n_loc
    if nl == E and e0 == 0:
        assert p.counts[:nl].sum() == T * k
    for t in range(T):
        for j in range(k + (1 if sh else 0)):
            r = p.slot_row[t, j]
            if j < k:
                g = idx[t, j] - e0
                if 0 <= g < nl:
                    assert p.offsets[g] <= r < p.offsets[g + 1] and p.row_src[r] == t
                    assert p.row_w[r] == w[t, j]
                else:
                    assert r == -1
            else:
                assert r == p.offsets[nl] + t and p.row_w[r] == 1.0
    assert len(order) == n_loc
