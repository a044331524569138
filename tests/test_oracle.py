"""Pins for the CPU oracle (no GPU): the worked example, closed forms,
exhaustive enumeration, library special cases and invariants.

Each test targets a mistake the oracle could plausibly hold: a wrong phase
boundary, a missing shift, a shift applied twice, an evicted entry still
attended, a sink that can be skipped, a wrong argmin direction or tie rule, a
wrong softmax scale, a dropped prompt row.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
import synth
from closed_form import (attended_sets, falling_expected, monotone_inputs, rising_expected, sdpa_reference,
                         selection_steps)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _sets(mask):
    return [sorted(np.nonzero(row)[0].tolist()) for row in mask]


# ---------------------------------------------------------------- worked example
def _worked_example_inputs(g):
    e = g["engineered_inputs"]
    d, L_p, T = e["d"], e["L_p"], e["T"]
    q = np.zeros((T, d))
    for t in range(T):
        q[t, {3: 0, 4: 1}.get(t, 2)] = 1.0
    k = np.zeros((T, d))
    k[:, 0], k[:, 1], k[:, 2] = e["a"], e["b"], e["c"]
    rng = np.random.default_rng(1)
    v = rng.normal(size=(T, d))
    kp = rng.normal(size=(L_p, d))
    vp = rng.normal(size=(L_p, d))
    return L_p, q, kp, vp, k, v


def test_worked_example_matches_page():
    with open(os.path.join(GOLDEN, "worked_example_nr7_natt4.json")) as f:
        g = json.load(f)
    L_p, q, kp, vp, k, v = _worked_example_inputs(g)
    r = oracle.run_lane(L_p, 7, 4, 0, q, kp, vp, k, v, masks=True)
    att = _sets(r["att_mask"])
    skip = _sets(r["skip_mask"])
    for step in g["expected"]["steps"]:
        t = step["t"]
        assert skip[t] == step["skip"], t
        assert att[t] == step["attended"], t
        assert r["choice"][t] == step["selected"], t
        assert r["evicted"][t] == step["evicted"], t
    # attended count is N_att = 4 from t = 3 on; |skip_idx| never exceeds N_r - N_att
    assert all(r["n_dec"][t] == 4 for t in range(3, 10))
    assert max(len(s) for s in skip) == 3


# ---------------------------------------------------------------- exhaustive enumeration
def _enumerate_choice_sequences(T, N_r, N_att, S):
    """Every valid sequence of argmin choices, candidates taken from the closed form."""
    sel = set(selection_steps(N_r, N_att))

    def rec(t, choices):
        if t == T:
            yield list(choices)
            return
        if t in sel:
            cands = [p for p in attended_sets(t + 1, N_r, N_att, S, choices + [-1])[t] if p >= S]
            for p in cands:
                yield from rec(t + 1, choices + [p])
        else:
            yield from rec(t + 1, choices + [-1])

    yield from rec(0, [])


CASES = [(N_r, N_att, 0) for N_r in range(1, 7) for N_att in range(1, N_r + 1)]
CASES += [(N_r, N_att, 4) for N_r in range(5, 9) for N_att in range(5, N_r + 1)]


@pytest.mark.parametrize("N_r,N_att,S", CASES)
def test_literal_matches_offset_closed_form_for_every_choice_sequence(N_r, N_att, S):
    T = N_r + 4
    d, L_p = 3, 1
    rng = np.random.default_rng(N_r * 100 + N_att * 10 + S)
    q, k, v = rng.normal(size=(T, d)), rng.normal(size=(T, d)), rng.normal(size=(T, d))
    kp, vp = rng.normal(size=(L_p, d)), rng.normal(size=(L_p, d))
    n = 0
    for choices in _enumerate_choice_sequences(T, N_r, N_att, S):
        follow = np.array([max(c, 0) for c in choices], np.int32)
        r = oracle.run_lane(L_p, N_r, N_att, S, q, kp, vp, k, v, follow=follow, masks=True)
        assert _sets(r["att_mask"]) == attended_sets(T, N_r, N_att, S, choices)
        sel = [t for t in range(T) if r["choice"][t] >= 0]
        assert sel == selection_steps(N_r, N_att)
        n += 1
    assert n >= 1


# ---------------------------------------------------------------- engineered closed forms
@pytest.mark.parametrize("S", [0, 4])
@pytest.mark.parametrize("N_r,N_att", [(12, 7), (16, 5), (9, 9), (20, 6)])
def test_rising_scores_skip_the_oldest(N_r, N_att, S):
    T = 2 * N_r + 3
    q, kp, vp, k, v = monotone_inputs(T, 8, 3, +1)
    r = oracle.run_lane(3, N_r, N_att, S, q, kp, vp, k, v, masks=True)
    att = _sets(r["att_mask"])
    for t in range(T):
        assert att[t] == rising_expected(t, N_r, N_att, S), t


@pytest.mark.parametrize("S", [0, 4])
@pytest.mark.parametrize("N_r,N_att", [(12, 7), (16, 5), (9, 9), (20, 6)])
def test_falling_scores_skip_the_newest(N_r, N_att, S):
    T = 2 * N_r + 3
    q, kp, vp, k, v = monotone_inputs(T, 8, 3, -1)
    r = oracle.run_lane(3, N_r, N_att, S, q, kp, vp, k, v, masks=True)
    att = _sets(r["att_mask"])
    for t in range(T):
        assert att[t] == falling_expected(t, N_r, N_att, S), t


@pytest.mark.parametrize("S", [0, 4])
def test_all_equal_scores_tie_to_oldest_and_average_values(S):
    """K = 0: every logit is 0, so ties everywhere: the oldest candidate must be
    chosen (same sets as rising scores), and the output is the plain mean of V
    over exactly the attended rows (uniform softmax)."""
    N_r, N_att, T, d, L_p = 14, 8, 33, 4, 2
    rng = np.random.default_rng(5)
    q = rng.normal(size=(T, d))
    k = np.zeros((T, d))
    kp = np.zeros((L_p, d))
    v = np.zeros((T, d))
    v[:, 0] = np.arange(T)          # V encodes the position
    v[:, 1] = 1.0
    vp = np.zeros((L_p, d))
    vp[:, 0] = -100.0
    vp[:, 1] = 1.0
    r = oracle.run_lane(L_p, N_r, N_att, S, q, kp, vp, k, v, masks=True)
    att = _sets(r["att_mask"])
    for t in range(T):
        assert att[t] == rising_expected(t, N_r, N_att, S), t
        rows = [-100.0] * L_p + att[t]
        assert r["out"][t, 0] == pytest.approx(np.mean(rows), abs=1e-12)
        assert r["out"][t, 1] == pytest.approx(1.0, abs=1e-12)


# ---------------------------------------------------------------- library special cases
def _tiny():
    return synth.WORKLOADS["tiny_fp32"]


@pytest.mark.parametrize("h", range(4))
def test_full_budget_equals_dense_attention(h):
    """N_att = N_r >= L_dec: nothing is ever skipped or evicted, so Algorithm 1
    is dense decode attention; checked against torch SDPA and the dense oracle."""
    w = _tiny()
    q, kp, vp, k, v = oracle.lane_inputs(w, 0, 0, h)
    T = w.L_dec
    r = oracle.run_lane(w.L_p, T, T, 0, q, kp, vp, k, v)
    dense = oracle.run_dense_lane(w.L_p, q, kp, vp, k, v)
    assert (r["choice"] == -1).all() and (r["evicted"] == -1).all()
    for t in range(T):
        ref = sdpa_reference(q[t], kp, vp, k, v, range(t + 1))
        np.testing.assert_allclose(r["out"][t], ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(dense[t], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("S", [0, 4])
def test_equal_budgets_below_length_is_sliding_window_or_streaming(S):
    """N_att = N_r < L_dec: SlidingWindow (S = 0: prompt + the last N_r tokens) or
    StreamingLLM (S = 4: prompt + 4 sinks + the last N_r - 4 tokens)."""
    w = _tiny()
    q, kp, vp, k, v = oracle.lane_inputs(w, 0, 0, 1)
    T, N = w.L_dec, 32
    r = oracle.run_lane(w.L_p, N, N, S, q, kp, vp, k, v, masks=True)
    att = _sets(r["att_mask"])
    for t in range(T):
        recent = list(range(max(S, t - (N - S) + 1), t + 1))
        want = sorted(set(range(min(S, t + 1))) | set(recent))
        assert att[t] == want, t
        ref = sdpa_reference(q[t], kp, vp, k, v, want)
        np.testing.assert_allclose(r["out"][t], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("S", [0, 4])
def test_output_is_softmax_attention_over_the_attended_set(S):
    """On generator data with the tiny workload's budgets, every step's output
    equals torch SDPA over prompt + the oracle's own attended set."""
    w = _tiny()
    q, kp, vp, k, v = oracle.lane_inputs(w, 0, 0, 2)
    r = oracle.run_lane(w.L_p, w.N_r, w.N_att, S, q, kp, vp, k, v, masks=True)
    att = _sets(r["att_mask"])
    for t in range(w.L_dec):
        ref = sdpa_reference(q[t], kp, vp, k, v, att[t])
        np.testing.assert_allclose(r["out"][t], ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("S,N_att", [(0, 8), (0, 1), (0, 31), (4, 8), (4, 5)])
def test_invariants_on_generator_data(S, N_att):
    w = _tiny()
    N_r = w.N_r
    q, kp, vp, k, v = oracle.lane_inputs(w, 0, 0, 3)
    T = w.L_dec
    r = oracle.run_lane(w.L_p, N_r, N_att, S, q, kp, vp, k, v, masks=True)
    att, skip = r["att_mask"], r["skip_mask"]
    live = np.zeros(T, bool)
    for t in range(T):
        # attended decode count = min(t + 1, N_att): phase 1 grows, then fixed
        assert r["n_dec"][t] == min(t + 1, N_att)
        # selections exactly at t in [N_att - 1, N_r - 2]
        assert (r["choice"][t] >= 0) == (N_att - 1 <= t <= N_r - 2)
        # eviction of t - (N_r - S) from t = N_r on; live decode KV <= N_r
        assert r["evicted"][t] == (t - (N_r - S) if t >= N_r else -1)
        live[t] = True
        if r["evicted"][t] >= 0:
            live[r["evicted"][t]] = False
        assert live.sum() <= N_r
        assert not (att[t] & ~live).any()
        # skip and attended are disjoint; sinks are never skipped
        assert not (att[t] & skip[t]).any()
        assert not skip[t][:S].any()
        # skip positions advance by one per step; one new entry per selection
        if t + 1 < T:
            moved = np.zeros(T, bool)
            moved[1:] = skip[t][:-1]
            if r["choice"][t] >= 0:
                moved[r["choice"][t] + 1] = True
            assert (skip[t + 1] == moved).all(), t
        # the choice is the lowest raw logit among attended non-sink positions,
        # the oldest among equals (brute force with numpy)
        if r["choice"][t] >= 0:
            cands = [p for p in np.nonzero(att[t])[0] if p >= S]
            logits = [float(np.dot(q[t], k[p])) for p in cands]
            best = min(range(len(cands)), key=lambda i: (logits[i], cands[i]))
            assert r["choice"][t] == cands[best]


def test_follow_rejects_non_candidates():
    w = _tiny()
    q, kp, vp, k, v = oracle.lane_inputs(w, 0, 0, 0)
    follow = np.zeros(w.L_dec, np.int32)
    follow[w.N_att - 1] = w.N_att + 3       # a future position, not a candidate
    with pytest.raises(ValueError):
        oracle.run_lane(w.L_p, w.N_r, w.N_att, 0, q, kp, vp, k, v, follow=follow)


def test_follow_own_choices_reproduces_run_and_zero_gaps():
    w = _tiny()
    q, kp, vp, k, v = oracle.lane_inputs(w, 0, 0, 1)
    a = oracle.run_lane(w.L_p, w.N_r, w.N_att, 0, q, kp, vp, k, v)
    follow = np.maximum(a["choice"], 0)
    b = oracle.run_lane(w.L_p, w.N_r, w.N_att, 0, q, kp, vp, k, v, follow=follow)
    assert (a["choice"] == b["choice"]).all()
    assert (b["gap"] == 0).all()
    np.testing.assert_array_equal(a["out"], b["out"])


@pytest.mark.parametrize("S", [0, 4])
def test_gap_of_forced_choices_matches_numpy(S):
    """The lockstep gap (Section 4, Algorithm 1, phase 2 selection; the near-tie
    reading) is (s[follow] - s[own choice]) / max(|s[follow]|, |s[own choice]|)
    on the raw logits.  Forcing the highest-logit candidate at every selection
    step (candidates from the offset closed form, not from the oracle) makes
    every gap positive and large; numpy recomputes both logits.  A flipped
    sign, a min in the denominator or a gap taken against the wrong entry fails."""
    w = _tiny()
    q, kp, vp, k, v = oracle.lane_inputs(w, 0, 0, 2)
    T = w.L_dec
    sel = set(selection_steps(w.N_r, w.N_att))
    follow = np.full(T, -1, np.int32)
    own = {}
    for t in range(T):
        if t in sel:
            cands = [p for p in attended_sets(t + 1, w.N_r, w.N_att, S, list(follow[:t]) + [-1])[t] if p >= S]
            logits = [float(np.dot(q[t], k[p])) for p in cands]
            follow[t] = cands[int(np.argmax(logits))]
            own[t] = min(zip(logits, cands))[1]
    r = oracle.run_lane(w.L_p, w.N_r, w.N_att, S, q, kp, vp, k, v, follow=np.maximum(follow, 0))
    for t in range(T):
        if t not in sel:
            assert r["gap"][t] == 0.0 and r["choice"][t] == -1
            continue
        assert r["choice"][t] == own[t], t
        a, b = float(np.dot(q[t], k[follow[t]])), float(np.dot(q[t], k[own[t]]))
        want = (a - b) / max(abs(a), abs(b))
        assert want > 1e-3, t
        assert r["gap"][t] == pytest.approx(want, rel=1e-9), t


def test_parameter_validation():
    z = np.zeros((4, 4))
    zp = np.zeros((1, 4))
    for N_r, N_att, S in [(4, 0, 0), (3, 4, 0), (8, 4, 4), (8, 6, 2)]:
        with pytest.raises(ValueError):
            oracle.run_lane(1, N_r, N_att, S, z, zp, zp, z, z)
