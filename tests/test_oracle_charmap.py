"""Pins of the attention-map characterization oracle (Section 3.4, Figs. 8 and 10).

* Rows of the map equal torch's softmax of the masked logits.
* Uniform attention (q = 0): every row is uniform, so the mass split has a
  closed form and both similarities are exactly 1.
* Relative-position logits (q_t . k_j a function of t - j only, built from 2D
  rotations): the diagonal score vector of query i + d is the one of query i
  scaled by a ratio of normalisers, so the diagonal similarity is 1 while the
  vertical one is below 1 (the pages' argument for the diagonal pattern).
* All mass on one decode key: the local-group boundary (the most recent 10 %
  of the decoded tokens) is pinned exactly by which group receives it.
"""
import math

import numpy as np
import pytest
import torch

from oracle import charmap


def test_rows_are_torch_softmax_of_the_causal_logits():
    rng = np.random.default_rng(0)
    T, d, L_p = 30, 16, 5
    q, kp, k = rng.normal(size=(T, d)), rng.normal(size=(L_p, d)), rng.normal(size=(T, d))
    P = charmap.attention_map(q, kp, k)
    s = torch.from_numpy(q @ np.concatenate([kp, k]).T / math.sqrt(d))
    mask = torch.ones(T, L_p + T, dtype=torch.bool)
    for t in range(T):
        mask[t, L_p + t + 1:] = False
    ref = torch.softmax(s.masked_fill(~mask, -float("inf")), dim=1).numpy()
    np.testing.assert_allclose(P, ref, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("L_p", [0, 7])
def test_uniform_attention_closed_forms(L_p):
    T, d, dmax = 40, 8, 6
    rng = np.random.default_rng(1)
    q, kp, k = np.zeros((T, d)), rng.normal(size=(L_p, d)), rng.normal(size=(T, d))
    mass, vert, diag = charmap.profile_lane(q, kp, k, dmax)
    want = np.zeros(3)
    for t in range(T):
        n = L_p + t + 1
        loc = math.ceil((t + 1) / 10)
        want += (L_p / n, loc / n, (t + 1 - loc) / n)
    np.testing.assert_allclose(mass, want / T, rtol=1e-13)
    np.testing.assert_allclose(vert, 1.0, rtol=1e-13)
    np.testing.assert_allclose(diag, 1.0, rtol=1e-13)


def rotary_relative(T, L_p, theta, seed):
    """q_t . k_j = f(t - j): 2D rotations of fixed vectors, padded with zeros."""
    rng = np.random.default_rng(seed)
    d = 8
    u, w = rng.normal(size=2), rng.normal(size=2) * 3

    def rot(a):
        return np.array([[math.cos(a), -math.sin(a)], [math.sin(a), math.cos(a)]])

    q = np.zeros((T, d))
    k = np.zeros((T, d))
    for t in range(T):
        q[t, :2] = rot(theta * t) @ w
        k[t, :2] = rot(theta * t) @ u
    kp = rng.normal(size=(L_p, d))
    return q, kp, k


@pytest.mark.parametrize("L_p,theta", [(0, 0.4), (6, 0.4), (6, 1.3)])
def test_relative_position_attention_is_exactly_diagonal(L_p, theta):
    q, kp, k = rotary_relative(48, L_p, theta, 2)
    mass, vert, diag = charmap.profile_lane(q, kp, k, 10)
    np.testing.assert_allclose(diag, 1.0, atol=1e-12)
    assert (vert < 1 - 1e-3).all()
    np.testing.assert_allclose(mass.sum(), 1.0, rtol=1e-13)


@pytest.mark.parametrize("t", [0, 8, 9, 10, 19, 20, 21, 39])
def test_local_group_boundary(t):
    """All of query t's mass on one decode key: the key at the edge of the
    local group (ceil((t + 1) / 10) most recent) counts as local, the one
    just beyond it as middle."""
    T, d, L_p = 40, 4, 3
    loc = math.ceil((t + 1) / 10)
    for j, group in ((t - loc + 1, 1), (t - loc, 2)):
        if j < 0:
            continue
        q = np.zeros((T, d))
        k = np.zeros((T, d))
        q[t, 0] = 1.0
        k[j, 0] = 200.0  # all of row t's mass on key j
        rows = charmap.mass_rows(charmap.attention_map(q, np.zeros((L_p, d)), k), L_p)
        assert rows[t, group] > 1 - 1e-12, (t, j, rows[t])


def test_local_count_is_a_tenth_rounded_up():
    assert [charmap.local_count(t) for t in (0, 9, 10, 19, 20, 575)] == [1, 1, 2, 2, 3, 58]


def test_mass_rows_sum_to_one_and_similarities_in_range():
    rng = np.random.default_rng(3)
    T, d, L_p = 36, 16, 4
    q, kp, k = rng.normal(size=(T, d)), rng.normal(size=(L_p, d)), rng.normal(size=(T, d))
    mass, vert, diag = charmap.profile_lane(q, kp, k, 8)
    np.testing.assert_allclose(mass.sum(), 1.0, rtol=1e-13)
    assert ((vert > 0) & (vert <= 1 + 1e-12)).all() and ((diag > 0) & (diag <= 1 + 1e-12)).all()
