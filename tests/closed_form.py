"""Test-side formulations that pin the oracle from outside it.

* ``attended_sets`` restates the selection rule in query-relative offsets.  A
  skip entry chosen at step s at position p sits at p + (t - s) at every later
  step t, because every step adds +1 to it (Algorithm 1, the two shift lines
  of phases 2 and 3).  Its offset d = t - position = s - p therefore never
  changes, and the attended decode set of step t is
  {t - d : 0 <= d <= min(t - S, N_r - S - 1), d not in D_t} plus the sinks,
  with D_t the offsets chosen before t.  No list, no shift, no eviction: a
  different route to the same sets than the oracle's literal transcription.
* ``sdpa_reference`` is torch's scaled_dot_product_attention in fp64 with a
  boolean mask: the textbook softmax attention the pages' Attn(.) names.
"""
from __future__ import annotations

import numpy as np


def attended_sets(T, N_r, N_att, S, choices):
    """Attended decode positions per step from the offset closed form.

    choices[t] is the position selected at step t (or -1).  Returns a list of
    sorted position lists, one per step.
    """
    D = set()
    out = []
    Nr_w = N_r - S
    for t in range(T):
        sinks = list(range(min(t + 1, S)))
        tw = t - S  # time inside the non-sink sub-sequence
        win = []
        if tw >= 0:
            for d in range(0, min(tw, Nr_w - 1) + 1):
                if d not in D:
                    win.append(t - d)
        out.append(sorted(sinks + win))
        if choices[t] >= 0:
            D.add(t - choices[t])
    return out


def selection_steps(N_r, N_att):
    """Steps that select a new skip entry: t in [N_att - 1, N_r - 2]."""
    return list(range(N_att - 1, N_r - 1))


def sdpa_reference(q, kp, vp, k, v, positions):
    """fp64 softmax attention of q over prompt rows plus decode ``positions`` (torch SDPA)."""
    import torch

    rows_k = np.concatenate([kp, k[list(positions)]], axis=0) if len(positions) else kp
    rows_v = np.concatenate([vp, v[list(positions)]], axis=0) if len(positions) else vp
    Q = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float64)).view(1, 1, 1, -1)
    Kt = torch.from_numpy(np.ascontiguousarray(rows_k, dtype=np.float64)).view(1, 1, rows_k.shape[0], -1)
    Vt = torch.from_numpy(np.ascontiguousarray(rows_v, dtype=np.float64)).view(1, 1, rows_v.shape[0], -1)
    o = torch.nn.functional.scaled_dot_product_attention(Q, Kt, Vt)
    return o.view(-1).numpy()


def monotone_inputs(T, d, L_p, direction, seed=0):
    """q = e0 for every step, key of position p = direction * 0.01 * (p + 1) * e0.

    direction +1: logits rise with position, so the oldest candidate is always
    the lowest; -1: they fall, so the newest is.
    """
    rng = np.random.default_rng(seed)
    q = np.zeros((T, d))
    q[:, 0] = 1.0
    k = rng.normal(size=(T, d)) * 0.0
    k[:, 0] = direction * 0.01 * (np.arange(T) + 1)
    v = rng.normal(size=(T, d))
    kp = np.zeros((L_p, d))
    kp[:, 0] = 5.0
    vp = rng.normal(size=(L_p, d))
    return q, kp, vp, k, v


def rising_expected(t, N_r, N_att, S):
    """Attended positions when the oldest candidate always loses (closed form)."""
    sinks = list(range(min(t + 1, S)))
    Nr_w, Na_w = N_r - S, N_att - S
    if t < S:
        return sinks
    if t < N_att - 1:
        return sinks + list(range(S, t + 1))
    if t < N_r:
        # offsets {0 .. Na_w - 2} plus the oldest position S
        return sinks + [S] + list(range(t - Na_w + 2, t + 1))
    return sinks + [t - Nr_w + 1] + list(range(t - Na_w + 2, t + 1))


def falling_expected(t, N_r, N_att, S):
    """Attended positions when the newest candidate always loses (closed form)."""
    sinks = list(range(min(t + 1, S)))
    Nr_w, Na_w = N_r - S, N_att - S
    if t < S:
        return sinks
    if t < N_att - 1:
        return sinks + list(range(S, t + 1))
    if t < N_r:
        return sinks + list(range(S, S + Na_w))
    return sinks + list(range(t - Nr_w + 1, t - Nr_w + 1 + Na_w))
