"""Pins of the oracle's tree attention mask, position ids and kept KV entries (the step
after the prune: one target forward over the emitted tree, RheoSampling framework
flowchart).

Each pin comes from something other than the oracle's own walk: closed forms for chain
and star trees, and on random trees the reachability of the parent graph computed as a
boolean fixed point (R = I or A R, A the child -> parent adjacency), from which the depth
is the row count minus one.
"""
import numpy as np
import pytest

from oracle import oracle as O

pytestmark = pytest.mark.filterwarnings("ignore")


def test_chain_tree_is_lower_triangular():
    n = 9
    parent = np.arange(-1, n - 1)
    mask, pos = O.tree_mask(parent)
    np.testing.assert_array_equal(mask, np.tril(np.ones((n, n), bool)))
    np.testing.assert_array_equal(pos, np.arange(n))


def test_star_tree_is_identity_plus_root_column():
    n = 7
    parent = np.array([-1] + [0] * (n - 1))
    mask, pos = O.tree_mask(parent)
    want = np.eye(n, dtype=bool)
    want[:, 0] = True
    np.testing.assert_array_equal(mask, want)
    np.testing.assert_array_equal(pos, [0] + [1] * (n - 1))


def _random_parents(rng, n):
    return np.array([-1] + [int(rng.integers(0, i)) for i in range(1, n)])


@pytest.mark.parametrize("seed", range(6))
def test_random_trees_match_reachability_fixed_point(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 70))
    parent = _random_parents(rng, n)
    mask, pos = O.tree_mask(parent)
    A = np.zeros((n, n), bool)
    for i in range(1, n):
        A[i, parent[i]] = True
    R = np.eye(n, dtype=bool)
    while True:
        nxt = np.eye(n, dtype=bool) | ((A.astype(np.int64) @ R.astype(np.int64)) > 0)
        if np.array_equal(nxt, R):
            break
        R = nxt
    np.testing.assert_array_equal(mask, R)
    np.testing.assert_array_equal(pos, R.sum(1) - 1)
    # a node attends only to nodes created before it (parents precede children)
    assert not np.triu(mask, 1).any()


def test_bad_parents_are_rejected():
    assert O.tree_mask(np.array([0, 0])) is None       # root's parent must be -1
    assert O.tree_mask(np.array([-1, 1])) is None      # a node's parent precedes it
    assert O.tree_mask(np.array([-1, 0, 5])) is None   # out of range


def test_accepted_kv_keeps_root_then_the_path():
    np.testing.assert_array_equal(O.accepted_kv(1, np.array([-1, -1])), [0])
    np.testing.assert_array_equal(O.accepted_kv(4, np.array([2, 7, 11, -1])), [0, 2, 7, 11])
