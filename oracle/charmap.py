"""CPU oracle for the attention-map characterization (fp64, numpy).

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the GPU library.

"Understanding and Exploiting Diagonal Attention Sparsity in Autoregressive
Image Generation", Section 3.4:
  * Fig. 8, "Skewed attention toward prompt and local tokens": the attention
    mass of a decode query split over three key groups, the prompt tokens, the
    local tokens (the most recent 10 % of the decoded tokens) and the middle
    tokens (the other decoded tokens);
  * Fig. 10, "Diagonal attention sparsity pattern": the cosine similarity of
    the attention score vectors of queries i and i + d, vertical (both over
    keys [0, i]) and diagonal (query i over keys [0, i], query i + d over keys
    [d, i + d]), averaged over queries (and, by the caller, over heads and
    layers).

Readings taken where the pages leave a step open:
  * the attention map is the dense decode map: query t attends the prompt and
    decode positions 0..t, one softmax with scale 1 / sqrt(d);
  * "score vectors" are the probabilities of the decode keys (the prompt
    columns are left out, the comparison is about the decode region);
  * at query t the decoded tokens are positions 0..t, and the local group is
    the ceil(0.1 (t + 1)) most recent of them (the current token included);
  * per lane, the mass split is the mean over queries of each group's mass,
    and the similarity at distance d the mean over i in [0, T - d) of the
    cosine; lanes are averaged by the caller.
"""
from __future__ import annotations

import math

import numpy as np


def attention_map(q, kp, k):
    """Dense decode attention probabilities: P [T][L_p + T], row t over the
    prompt columns then decode positions 0..t (zero beyond t)."""
    T, d = q.shape
    L_p = kp.shape[0]
    keys = np.concatenate([kp, k], axis=0) if L_p else k
    s = (q @ keys.T) / math.sqrt(d)
    P = np.zeros_like(s)
    for t in range(T):
        row = s[t, : L_p + t + 1]
        e = np.exp(row - row.max())
        P[t, : L_p + t + 1] = e / e.sum()
    return P


def local_count(t):
    """Decoded tokens in the local group of query t: the most recent 10 % of
    the t + 1 decoded tokens, rounded up (ceil((t + 1) / 10))."""
    return (t + 10) // 10


def mass_rows(P, L_p):
    """(prompt, local, middle) attention mass of every query: [T][3]."""
    T = P.shape[0]
    out = np.zeros((T, 3))
    for t in range(T):
        n_loc = local_count(t)
        out[t] = (P[t, :L_p].sum(), P[t, L_p + t + 1 - n_loc: L_p + t + 1].sum(),
                  P[t, L_p: L_p + t + 1 - n_loc].sum())
    return out


def mass_split(P, L_p):
    """Mean over queries of the (prompt, local, middle) attention mass."""
    return mass_rows(P, L_p).mean(axis=0)


def similarities(P, L_p, max_dist):
    """Mean vertical and diagonal cosine similarity for query distances 1..max_dist."""
    T = P.shape[0]
    A = P[:, L_p:]  # decode columns
    vert = np.zeros(max_dist)
    diag = np.zeros(max_dist)
    for dd in range(1, max_dist + 1):
        n = T - dd
        if n <= 0:
            vert[dd - 1] = diag[dd - 1] = np.nan
            continue
        sv = sd = 0.0
        for i in range(n):
            a = A[i, : i + 1]
            b = A[i + dd, : i + 1]
            c = A[i + dd, dd: i + dd + 1]
            sv += a @ b / math.sqrt((a @ a) * (b @ b))
            sd += a @ c / math.sqrt((a @ a) * (c @ c))
        vert[dd - 1] = sv / n
        diag[dd - 1] = sd / n
    return vert, diag


def profile_lane(q, kp, k, max_dist):
    """(mass [3], vertical [max_dist], diagonal [max_dist]) of one lane."""
    P = attention_map(q, kp, k)
    return mass_split(P, kp.shape[0]), *similarities(P, kp.shape[0], max_dist)
