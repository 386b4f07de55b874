"""Pins of the oracle's token-tree accept (kqo_tree_accept, CPU only).

The pages' hardware-aware token tree (muser-book ch. 33, section 33.7)
scores every node of a draft tree in one pass; a round emits along the
branch the target agrees with. Pins: a chain reduces to the linear rule for
every draft and argmax vector at N = 4, k = 3; hand-built trees; and, on
random trees with distinct sibling tokens, the walk's end is the deepest
node all of whose root-path edges the target accepts (found by enumerating
every node's path, not by walking).
"""
import itertools

import numpy as np
import pytest

import oracle


def test_chain_equals_linear_rule_exhaustively():
    n, k = 4, 3
    parent = [-1, 0, 1, 2]
    for draft in itertools.product(range(n), repeat=k):
        for am in itertools.product(range(n), repeat=k + 1):
            acc, nxt, path = oracle.tree_accept(parent, [0] + list(draft), am)
            assert (acc, nxt) == oracle.accept(draft, am)
            assert path == list(range(1, acc + 1))


def test_hand_built_trees():
    # root with two branches: 1 (token 5) -> 3 (token 7); 2 (token 6) -> 4 (token 8) -> 5 (token 9)
    parent = [-1, 0, 0, 1, 2, 4]
    token = [0, 5, 6, 7, 8, 9]
    # target follows the second branch to its end: next token from node 5's row
    assert oracle.tree_accept(parent, token, [6, 0, 8, 0, 9, 42]) == (3, 42, [2, 4, 5])
    # target takes the first branch, then disagrees at node 3
    assert oracle.tree_accept(parent, token, [5, 7, 0, 11, 0, 0]) == (2, 11, [1, 3])
    # nothing matches at the root: the bonus comes from the root's own row
    assert oracle.tree_accept(parent, token, [99, 7, 8, 0, 9, 0]) == (0, 99, [])
    # a single node (no drafts) emits the root's argmax
    assert oracle.tree_accept([-1], [0], [17]) == (0, 17, [])
    # siblings repeating a token: the lower-index child is taken
    assert oracle.tree_accept([-1, 0, 0, 2], [0, 4, 4, 9], [4, 1, 9, 3]) == (1, 1, [1])


def test_invalid_trees_rejected():
    with pytest.raises(ValueError):
        oracle.tree_accept([0, 0], [0, 1], [1, 1])        # root must have parent -1
    with pytest.raises(ValueError):
        oracle.tree_accept([-1, 1], [0, 1], [1, 1])       # parent must precede the node
    with pytest.raises(ValueError):
        oracle.tree_accept([-1, 0, 3, 0], [0, 1, 2, 3], [1, 1, 1, 1])


def random_tree(rng, m, n_vocab):
    parent = [-1] + [int(rng.integers(max(0, j - 6), j)) for j in range(1, m)]
    token = [0] * m
    for j in range(1, m):
        used = {token[c] for c in range(1, j) if parent[c] == parent[j]}
        t = int(rng.integers(n_vocab))
        while t in used:
            t = int(rng.integers(n_vocab))
        token[j] = t
    return parent, token


def test_walk_end_is_the_deepest_fully_accepted_node():
    rng = np.random.default_rng(9)
    n_vocab = 6
    for trial in range(3000):
        m = int(rng.integers(1, 65))
        parent, token = random_tree(rng, m, n_vocab)
        am = [int(v) for v in rng.integers(0, n_vocab, m)]
        # bias some rows towards a child's token so deep paths occur
        for j in range(1, m):
            if rng.random() < 0.6:
                am[parent[j]] = token[j]
        acc, nxt, path = oracle.tree_accept(parent, token, am)
        best, best_chain = 0, []
        for v in range(m):
            chain, u = [], v
            while u > 0:
                chain.append(u)
                u = parent[u]
            if all(token[c] == am[parent[c]] for c in chain) and len(chain) > len(best_chain):
                best, best_chain = v, chain
        assert acc == len(best_chain) and nxt == am[best], trial
        assert path == best_chain[::-1], trial
