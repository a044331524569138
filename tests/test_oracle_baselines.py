"""Pins of the baseline oracles (SlidingWindow, StreamingLLM, TOVA, H2O).

"Understanding and Exploiting Diagonal Attention Sparsity in Autoregressive
Image Generation", Section 2.3 "KV cache sparsity techniques" and Section 5.1
"Sparse KV baselines" define the four policies in words; the oracle's
readings are listed in its header.  What fixes them here, from outside the
oracle:

* outputs: torch's scaled_dot_product_attention in fp64 over the attended set;
* SlidingWindow / StreamingLLM: Algorithm 1 with N_r = N_att is the same
  policy (a different algorithm reaching the same sets), and with all-zero
  keys the output is the mean of the values over exactly the attended set;
* TOVA: closed forms for engineered logits (rising: the oldest entry always
  scores lowest, so TOVA is a sliding window; falling: the newest does, so the
  cache keeps the first N_att - 1 positions) and, on random data, the evicted
  entry's logit recomputed with numpy is the minimum;
* H2O: with all-zero keys attention is uniform and an older entry always has
  the larger accumulated score, which gives the closed form
  {0 .. h-2} + {t - r .. t} (h heavy, r recent); on random data the
  accumulated scores recomputed from numpy softmaxes match, and the evicted
  entry has the minimum among the unprotected ones.
"""
import numpy as np
import pytest

import oracle
from closed_form import monotone_inputs, sdpa_reference

TOVA, H2O = oracle.TOVA, oracle.H2O


def rand_inputs(T, d, L_p, seed):
    rng = np.random.default_rng(seed)
    return (rng.normal(size=(T, d)), rng.normal(size=(L_p, d)), rng.normal(size=(L_p, d)), rng.normal(size=(T, d)),
            rng.normal(size=(T, d)))


def mask_sets(mask):
    return [sorted(np.nonzero(row)[0].tolist()) for row in mask]


def check_outputs(res, q, kp, vp, k, v):
    for t, pos in enumerate(mask_sets(res["att_mask"])):
        np.testing.assert_allclose(res["out"][t], sdpa_reference(q[t], kp, vp, k, v, pos), rtol=1e-12, atol=1e-12)


def softmax_probs(q, kp, k, pos):
    """Probabilities of the decode rows `pos` in one softmax over prompt + pos (numpy, fp64)."""
    rows = np.concatenate([kp, k[pos]], axis=0) if len(pos) else kp
    s = rows @ q / np.sqrt(q.shape[0])
    e = np.exp(s - s.max())
    return (e / e.sum())[kp.shape[0]:]


# ------------------------------------------------------------------ SlidingWindow / StreamingLLM
@pytest.mark.parametrize("S,N_att", [(0, 1), (0, 5), (0, 13), (4, 5), (4, 9), (4, 13)])
def test_window_equals_algorithm1_with_equal_budgets(S, N_att):
    T, d, L_p = 40, 8, 3
    ins = rand_inputs(T, d, L_p, seed=N_att + S)
    w = oracle.run_window_lane(L_p, N_att, S, *ins, masks=True)
    a = oracle.run_lane(L_p, N_att, N_att, S, *ins, masks=True)
    np.testing.assert_array_equal(w["att_mask"], a["att_mask"])
    np.testing.assert_allclose(w["out"], a["out"], rtol=1e-12, atol=1e-13)
    check_outputs(w, *ins)


@pytest.mark.parametrize("S", [0, 4])
def test_window_zero_keys_average_exactly_the_window(S):
    T, d, L_p, N_att = 30, 4, 2, 9
    q = np.random.default_rng(0).normal(size=(T, d))
    k, kp = np.zeros((T, d)), np.zeros((L_p, d))
    v = np.zeros((T, d))
    v[:, 0] = np.arange(T)  # a value that names its position
    v[:, 1] = 1.0
    vp = np.zeros((L_p, d))
    vp[:, 2] = 1.0
    res = oracle.run_window_lane(L_p, N_att, S, q, kp, vp, k, v)
    for t in range(T):
        recent = list(range(max(S, t - (N_att - S) + 1), t + 1))
        pos = sorted(set(range(min(S, t + 1))) | set(recent))
        n = L_p + len(pos)
        assert res["n_dec"][t] == len(pos)
        np.testing.assert_allclose(res["out"][t, 0], sum(pos) / n, rtol=1e-13)
        np.testing.assert_allclose(res["out"][t, 1], len(pos) / n, rtol=1e-13)


def test_window_full_budget_is_dense():
    T, d, L_p = 25, 8, 4
    ins = rand_inputs(T, d, L_p, seed=3)
    res = oracle.run_window_lane(L_p, T, 0, *ins)
    q, kp, vp, k, v = ins
    for t in range(T):
        np.testing.assert_allclose(res["out"][t], sdpa_reference(q[t], kp, vp, k, v, range(t + 1)), rtol=1e-12)


# ------------------------------------------------------------------ TOVA
@pytest.mark.parametrize("N_att", [1, 2, 6, 11])
def test_tova_rising_logits_is_sliding_window(N_att):
    T = 37
    ins = monotone_inputs(T, 8, 3, +1)
    res = oracle.run_score_lane(TOVA, 3, N_att, *ins, masks=True)
    for t, pos in enumerate(mask_sets(res["att_mask"])):
        assert pos == list(range(max(0, t - N_att + 1), t + 1)), t
        want = t - N_att + 1 if t >= N_att - 1 else -1
        assert res["choice"][t] == want, t
    check_outputs(res, *ins)


@pytest.mark.parametrize("N_att", [1, 2, 6, 11])
def test_tova_falling_logits_keeps_the_first_entries(N_att):
    T = 37
    ins = monotone_inputs(T, 8, 3, -1)
    res = oracle.run_score_lane(TOVA, 3, N_att, *ins, masks=True)
    for t, pos in enumerate(mask_sets(res["att_mask"])):
        want = list(range(t + 1)) if t < N_att else list(range(N_att - 1)) + [t]
        assert pos == want, t
        assert res["choice"][t] == (t if t >= N_att - 1 else -1), t


def test_tova_all_equal_logits_evict_the_oldest():
    T, d, L_p, N_att = 30, 4, 2, 7
    q = np.random.default_rng(1).normal(size=(T, d))
    k, kp = np.zeros((T, d)), np.zeros((L_p, d))
    v, vp = np.random.default_rng(2).normal(size=(T, d)), np.zeros((L_p, d))
    res = oracle.run_score_lane(TOVA, L_p, N_att, q, kp, vp, k, v, masks=True)
    for t, pos in enumerate(mask_sets(res["att_mask"])):
        assert pos == list(range(max(0, t - N_att + 1), t + 1))


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("N_att", [1, 3, 8])
def test_tova_random_invariants(seed, N_att):
    T, d, L_p = 45, 8, 5
    ins = rand_inputs(T, d, L_p, seed)
    q, kp, vp, k, v = ins
    res = oracle.run_score_lane(TOVA, L_p, N_att, *ins, masks=True)
    sets = mask_sets(res["att_mask"])
    gone = set()
    for t, pos in enumerate(sets):
        assert len(pos) == min(t + 1, N_att) == res["n_dec"][t]
        assert t in pos and not (gone & set(pos))
        if t >= 1:  # the cache carries over: last step's set minus its eviction, plus t
            prev = set(sets[t - 1]) - {res["choice"][t - 1]}
            assert set(pos) == prev | {t}
        if t >= N_att - 1:
            logits = k[pos] @ q[t]
            j = int(np.argmin(logits))  # first minimum = lowest position among equals
            assert res["choice"][t] == pos[j]
            gone.add(pos[j])
        else:
            assert res["choice"][t] == -1
    check_outputs(res, *ins)


# ------------------------------------------------------------------ H2O
@pytest.mark.parametrize("N_att,r", [(2, 1), (4, 2), (7, 3), (7, 6), (10, 5), (10, 1)])
def test_h2o_uniform_attention_closed_form(N_att, r):
    T, d, L_p = 40, 4, 3
    h = N_att - r
    q = np.random.default_rng(5).normal(size=(T, d))
    k, kp = np.zeros((T, d)), np.zeros((L_p, d))
    v, vp = np.random.default_rng(6).normal(size=(T, d)), np.random.default_rng(7).normal(size=(L_p, d))
    res = oracle.run_score_lane(H2O, L_p, N_att, q, kp, vp, k, v, N_recent=r, masks=True)
    for t, pos in enumerate(mask_sets(res["att_mask"])):
        want = list(range(t + 1)) if t < N_att else list(range(h - 1)) + list(range(t - r, t + 1))
        assert pos == want, (t, pos, want)
        assert res["choice"][t] == (t - r if t >= N_att - 1 else -1), t


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("N_att,r", [(2, 1), (6, 3), (9, 4), (9, 8)])
def test_h2o_random_scores_and_evictions(seed, N_att, r):
    T, d, L_p = 45, 8, 4
    ins = rand_inputs(T, d, L_p, seed)
    q, kp, vp, k, v = ins
    res = oracle.run_score_lane(H2O, L_p, N_att, *ins, N_recent=r, masks=True, scores=True)
    sets = mask_sets(res["att_mask"])
    acc = {}
    for t, pos in enumerate(sets):
        assert len(pos) == min(t + 1, N_att) and t in pos
        for p, pr in zip(pos, softmax_probs(q[t], kp, k, pos)):
            acc[p] = acc.get(p, 0.0) + pr
        if t >= N_att - 1:
            cand = [p for p in pos if p <= t - r]
            keys = [acc[p] for p in cand]
            j = int(np.argmin(keys))
            assert res["choice"][t] == cand[j], t
            acc.pop(cand[j])
        else:
            assert res["choice"][t] == -1
        for p in range(T):
            np.testing.assert_allclose(res["score"][t, p], acc.get(p, 0.0), rtol=1e-12, atol=1e-15)
        if t >= 1:
            assert set(pos) == (set(sets[t - 1]) - {res["choice"][t - 1]}) | {t}
    check_outputs(res, *ins)


def test_h2o_one_heavy_slot_of_recent_only_is_sliding_window():
    T, d, L_p, N_att = 30, 8, 3, 6
    ins = rand_inputs(T, d, L_p, 9)
    res = oracle.run_score_lane(H2O, L_p, N_att, *ins, N_recent=N_att - 1, masks=True)
    for t, pos in enumerate(mask_sets(res["att_mask"])):
        assert pos == list(range(max(0, t - N_att + 1), t + 1))


# ------------------------------------------------------------------ lockstep and validation
@pytest.mark.parametrize("policy,r", [(TOVA, 0), (H2O, 3)])
def test_follow_own_choices_reproduces_run(policy, r):
    T, d, L_p, N_att = 40, 8, 3, 7
    ins = rand_inputs(T, d, L_p, 11)
    a = oracle.run_score_lane(policy, L_p, N_att, *ins, N_recent=r)
    fol = np.where(a["choice"] >= 0, a["choice"], 0)
    b = oracle.run_score_lane(policy, L_p, N_att, *ins, N_recent=r, follow=fol)
    np.testing.assert_array_equal(a["choice"], b["choice"])
    np.testing.assert_array_equal(a["out"], b["out"])
    assert not b["gap"].any()


@pytest.mark.parametrize("policy,r", [(TOVA, 0), (H2O, 3)])
def test_follow_another_candidate_changes_the_cache(policy, r):
    T, d, L_p, N_att = 30, 8, 3, 7
    ins = rand_inputs(T, d, L_p, 12)
    q, kp, vp, k, v = ins
    a = oracle.run_score_lane(policy, L_p, N_att, *ins, N_recent=r, masks=True)
    t0 = N_att - 1  # the first eviction step
    pos = mask_sets(a["att_mask"])[t0]
    other = [p for p in pos if p != a["choice"][t0] and (policy == TOVA or p <= t0 - r)][0]
    # follow the alternative at t0, then at each later step the oracle's own pick
    # under that history: run the prefix with an entry that is always a candidate
    # (TOVA: the current token; H2O: position t - r, protected until step t - 1)
    # and read the oracle's own choice at its last step
    fol = np.zeros(T, np.int32)
    fol[t0] = other
    for t in range(t0 + 1, T):
        f = fol[: t + 1].copy()
        f[t] = t if policy == TOVA else t - r
        pre = oracle.run_score_lane(policy, L_p, N_att, q[: t + 1], kp, vp, k[: t + 1], v[: t + 1], N_recent=r,
                                    follow=f)
        fol[t] = pre["choice"][t]
    b = oracle.run_score_lane(policy, L_p, N_att, *ins, N_recent=r, follow=fol, masks=True)
    assert b["gap"][t0] > 0
    assert not b["att_mask"][t0 + 1:, other].any()
    assert (b["gap"][t0 + 1:] == 0).all()
    assert (b["choice"][t0 + 1:] == fol[t0 + 1:]).all()


def test_follow_rejects_non_candidates():
    T, d, L_p, N_att = 20, 4, 2, 5
    ins = rand_inputs(T, d, L_p, 13)
    fol = np.full(T, 19, np.int32)  # a future position is never in the cache
    for policy, r in ((TOVA, 0), (H2O, 2)):
        with pytest.raises(ValueError):
            oracle.run_score_lane(policy, L_p, N_att, *ins, N_recent=r, follow=fol)
    fol = np.full(T, 0, np.int32)
    fol[N_att - 1] = N_att - 1  # H2O: a protected recent position
    with pytest.raises(ValueError):
        oracle.run_score_lane(H2O, L_p, N_att, *ins, N_recent=2, follow=fol)


def test_parameter_validation():
    ins = rand_inputs(5, 4, 2, 0)
    with pytest.raises(ValueError):
        oracle.run_window_lane(2, 4, 4, *ins)  # StreamingLLM needs N_att > 4
    with pytest.raises(ValueError):
        oracle.run_window_lane(2, 0, 0, *ins)
    with pytest.raises(ValueError):
        oracle.run_score_lane(H2O, 2, 4, *ins, N_recent=4)  # no heavy-hitter slot left
    with pytest.raises(ValueError):
        oracle.run_score_lane(H2O, 2, 4, *ins, N_recent=0)
    with pytest.raises(ValueError):
        oracle.run_score_lane(2, 2, 4, *ins)
