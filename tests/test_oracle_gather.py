"""Pins for the oracle's expert-routed matmul (metaltile PR #250, commit adding
the per-token expert-routed gather qmm: weight row = expert_ids[m]*out_dim + n
of one stacked [E*out_dim, in_dim] tensor).

Each test fails for a plausible slip in the indexing: the wrong stride between
experts, the row's own index used in place of its expert id, or experts
swapped.
"""
import numpy as np
import pytest

import oracle


def test_single_expert_is_the_plain_matmul():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 48)).astype(np.float32)
    wd = rng.standard_normal((7, 48)).astype(np.float32)
    ref, den = oracle.gather_matmul(x, wd, np.zeros(5, np.int32), 7)
    r2, d2 = oracle.matmul(x, wd)
    assert (ref == r2).all() and (den == d2).all()


def test_grouped_rows_equal_each_experts_plain_matmul():
    """Grouping the rows by expert (the schedule of the grouped GEMM) gives,
    for every expert e, the plain matmul of e's rows with e's slice of the
    stack; the experts with no rows contribute nothing."""
    rng = np.random.default_rng(3)
    E, n, k, m = 6, 5, 64, 40
    wd = rng.standard_normal((E * n, k)).astype(np.float32)
    x = rng.standard_normal((m, k)).astype(np.float32)
    ids = rng.choice([0, 2, 3, 5], m).astype(np.int32)  # experts 1 and 4 get no rows
    ref, den = oracle.gather_matmul(x, wd, ids, n)
    for e in range(E):
        rows = np.flatnonzero(ids == e)
        if rows.size == 0:
            continue
        r2, d2 = oracle.matmul(x[rows], wd[e * n:(e + 1) * n])
        assert (ref[rows] == r2).all() and (den[rows] == d2).all()


def test_constant_experts_closed_form():
    """Expert e is the constant matrix (e + 1): row i's output is
    (ids[i] + 1) * sum(x[i]) in every column."""
    E, n, k = 4, 3, 16
    wd = np.repeat(np.arange(1, E + 1, dtype=np.float32), n * k).reshape(E * n, k)
    x = (np.arange(6 * k, dtype=np.float32).reshape(6, k) % 5) - 2
    ids = np.array([3, 0, 2, 2, 1, 3], np.int32)
    ref, _ = oracle.gather_matmul(x, wd, ids, n)
    want = (ids + 1)[:, None] * x.astype(np.float64).sum(axis=1, keepdims=True)
    assert (ref == np.broadcast_to(want, (6, n))).all()


def test_expert_permutation_invariance():
    """Relabelling the experts (permuting the stack and the ids alike) leaves
    every output unchanged."""
    rng = np.random.default_rng(2)
    E, n, k, m = 5, 4, 32, 9
    wd = rng.standard_normal((E * n, k)).astype(np.float32)
    x = rng.standard_normal((m, k)).astype(np.float32)
    ids = rng.integers(0, E, m).astype(np.int32)
    perm = rng.permutation(E)  # new label of old expert e is perm[e]
    wd2 = np.empty_like(wd)
    for e in range(E):
        wd2[perm[e] * n:(perm[e] + 1) * n] = wd[e * n:(e + 1) * n]
    a = oracle.gather_matmul(x, wd, ids, n)
    b = oracle.gather_matmul(x, wd2, perm[ids].astype(np.int32), n)
    assert (a[0] == b[0]).all() and (a[1] == b[1]).all()


def test_bad_id_is_rejected():
    x = np.ones((2, 8), np.float32)
    wd = np.ones((6, 8), np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.gather_matmul(x, wd, np.array([0, 2], np.int32), 3)
