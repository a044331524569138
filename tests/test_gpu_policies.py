"""GPU parity of the baseline policies (SlidingWindow, StreamingLLM, TOVA, H2O)
through the C ABI against the CPU oracle.

SlidingWindow / StreamingLLM have no data-dependent choice: outputs within the
dtype's tolerance, every attended set equal to the oracle's.  TOVA and H2O run
in lockstep: the oracle follows the GPU's evictions and reports its own; they
must agree except at near-ties (relative gap of the ranking key below 1e-6 for
TOVA's fp64 logits, 1e-9 for H2O's fp64 accumulated scores), which are
counted and printed.
"""
import sys

import numpy as np
import pytest
import torch

import autoregressive_image_generation_amd as dsa
import oracle
import synth
from closed_form import monotone_inputs
from gpu_util import device_inputs, lane_inputs_from, run_sparse, to_dev, tol

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
NEAR_TIE = {dsa.DSA_POLICY_TOVA: 1e-6, dsa.DSA_POLICY_H2O: 1e-9}
NAMES = {dsa.DSA_POLICY_SLIDING_WINDOW: "window", dsa.DSA_POLICY_STREAMING_LLM: "streamingllm",
         dsa.DSA_POLICY_TOVA: "tova", dsa.DSA_POLICY_H2O: "h2o"}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def tiny(**kw):
    return synth.WORKLOADS["tiny_fp32"].with_(**kw)


def n_r_for(policy, w):
    """N_r argument of each policy: the cache size, or H2O's protected recent count."""
    return w.N_att - w.N_att // 2 if policy == dsa.DSA_POLICY_H2O else w.N_att


def offsets_of(mask_row, t_next):
    return sorted(t_next - p for p in np.nonzero(mask_row)[0])


def check_policy(policy, w, lanes=None, waves=0, read_every=0, layer=0, T=None, fill=None, splits=0):
    T = w.L_dec if T is None else T
    n_r = n_r_for(policy, w)
    say("policy %s %s T=%d N_att=%d N_r=%d waves=%d fill=%s splits=%d" % (NAMES[policy], w.name, T, w.N_att, n_r,
                                                                          waves, fill, splits))
    ins = device_inputs(w, layer, T, DEV)
    out, trace, reads = run_sparse(w, ins, T, DEV, waves=waves, read_every=read_every, policy=policy, N_r=n_r,
                                   fill=fill, splits=splits)
    lanes = lanes or [(b, h) for b in range(w.batch) for h in range(w.heads)]
    stats = {"near_ties": 0, "choices": 0, "max_err": 0.0}
    for (b, h) in lanes:
        li = lane_inputs_from(w, layer, b, h, T)
        tr = trace[:, b, h, :]
        if policy in (dsa.DSA_POLICY_SLIDING_WINDOW, dsa.DSA_POLICY_STREAMING_LLM):
            S = 4 if policy == dsa.DSA_POLICY_STREAMING_LLM else 0
            ref = oracle.run_window_lane(w.L_p, w.N_att, S, *li, masks=True)
            assert (tr[:, 0] == -1).all()
            steps = np.arange(T)
            np.testing.assert_array_equal(tr[:, 1], np.where(steps >= w.N_att, steps - (w.N_att - S), -1))
            sink_cut = S  # dsa_read_state lists window entries only
        else:
            gpu = tr[:, 0].astype(np.int32)
            assert (tr[:, 1] == -1).all()
            fol = np.where(gpu >= 0, gpu, 0).astype(np.int32)
            ref = oracle.run_score_lane(0 if policy == dsa.DSA_POLICY_TOVA else 1, w.L_p, w.N_att, *li,
                                        N_recent=n_r, follow=fol, masks=True)
            np.testing.assert_array_equal(gpu >= 0, ref["choice"] >= 0)
            for t in np.nonzero(gpu != ref["choice"])[0]:
                g = abs(float(ref["gap"][t]))
                assert g < NEAR_TIE[policy], "step %d: GPU evicted %d, oracle %d, gap %.3g" % (
                    t, gpu[t], ref["choice"][t], g)
                stats["near_ties"] += 1
            stats["choices"] += int((gpu >= 0).sum())
            sink_cut = 0
        err = float(np.abs(out[:, b, h, :].cpu().numpy().astype(np.float64) - ref["out"]).max())
        stats["max_err"] = max(stats["max_err"], err)
        assert err <= tol(w), "max |out - oracle| = %.3g" % err
        lane = b * w.heads + h
        for t, (offs, cnt) in reads.items():
            if t + 1 >= T:
                continue
            got = sorted(int(x) for x in offs[lane][: cnt[lane]])
            mask = ref["att_mask"][t + 1].copy()
            mask[:sink_cut] = False
            assert got == offsets_of(mask, t + 1), (t, got)
    say("  lanes=%d choices=%d near_ties=%d max_err=%.3g" % (len(lanes), stats["choices"], stats["near_ties"],
                                                            stats["max_err"]))
    return trace, stats


ALL = [dsa.DSA_POLICY_SLIDING_WINDOW, dsa.DSA_POLICY_STREAMING_LLM, dsa.DSA_POLICY_TOVA, dsa.DSA_POLICY_H2O]


@pytest.mark.parametrize("policy", ALL)
def test_tiny_fp32_every_step(policy):
    check_policy(policy, tiny(), read_every=1)


@pytest.mark.parametrize("policy", ALL)
@pytest.mark.parametrize("dt,D", [(synth.BF16, 64), (synth.BF16, 128), (synth.F32, 128)])
def test_dtypes_and_head_dims(policy, dt, D):
    check_policy(policy, tiny(dtype=dt, head_dim=D, batch=3, heads=5), read_every=5)


@pytest.mark.parametrize("policy", [dsa.DSA_POLICY_TOVA, dsa.DSA_POLICY_H2O])
@pytest.mark.parametrize("waves", [1, 2, 4, 8, 16])
def test_every_workgroup_size(policy, waves):
    check_policy(policy, tiny(), waves=waves)


@pytest.mark.parametrize("policy,kw", [
    (dsa.DSA_POLICY_TOVA, dict(N_att=1)),             # the cache holds the current token only
    (dsa.DSA_POLICY_TOVA, dict(L_p=0)),
    (dsa.DSA_POLICY_TOVA, dict(N_att=64)),            # never full before the last step
    (dsa.DSA_POLICY_H2O, dict(N_att=2)),              # one heavy slot, one recent
    (dsa.DSA_POLICY_H2O, dict(L_p=0, N_att=13)),
    (dsa.DSA_POLICY_H2O, dict(batch=7, heads=3, L_p=5)),
    (dsa.DSA_POLICY_SLIDING_WINDOW, dict(N_att=1)),
    (dsa.DSA_POLICY_STREAMING_LLM, dict(N_att=5)),
    (dsa.DSA_POLICY_STREAMING_LLM, dict(L_p=0, N_att=64)),
])
def test_edge_cases(policy, kw):
    check_policy(policy, tiny(**kw), read_every=3)


def _engineered(policy, q, kp, vp, k, v, N_att, n_r):
    T, d = q.shape
    D = 64

    def pad(x):
        y = np.zeros((x.shape[0], D), np.float32)
        y[:, :d] = x
        return y

    w = tiny(batch=1, heads=1, L_p=kp.shape[0], L_dec=T, N_r=N_att, N_att=N_att)
    ins = (to_dev(pad(q)[:, None, None, :], DEV), to_dev(pad(k)[:, None, None, :], DEV),
           to_dev(pad(v)[:, None, None, :], DEV), to_dev(pad(kp)[None, :, None, :], DEV),
           to_dev(pad(vp)[None, :, None, :], DEV))
    out, trace, reads = run_sparse(w, ins, T, DEV, read_every=1, policy=policy, N_r=n_r)
    return trace[:, 0, 0, :], reads


@pytest.mark.parametrize("direction", [+1, -1])
def test_tova_monotone_logits_on_gpu(direction):
    T, N_att = 47, 9
    trace, reads = _engineered(dsa.DSA_POLICY_TOVA, *monotone_inputs(T, 8, 3, direction), N_att, N_att)
    for t in range(T):
        want = -1 if t < N_att - 1 else (t - N_att + 1 if direction > 0 else t)
        assert trace[t, 0] == want, t


@pytest.mark.parametrize("N_att,r", [(2, 1), (7, 3), (10, 5), (10, 9)])
def test_h2o_uniform_attention_on_gpu(N_att, r):
    # all-zero keys: every probability is exactly 1/n on both sides, so the
    # accumulated scores and every eviction follow the closed form exactly
    T, d, L_p = 40, 8, 3
    rng = np.random.default_rng(5)
    q = rng.normal(size=(T, d)).astype(np.float32)
    k, kp = np.zeros((T, d)), np.zeros((L_p, d))
    v, vp = rng.normal(size=(T, d)), rng.normal(size=(L_p, d))
    trace, reads = _engineered(dsa.DSA_POLICY_H2O, q, kp, vp, k, v, N_att, r)
    h = N_att - r
    for t in range(T):
        assert trace[t, 0] == (t - r if t >= N_att - 1 else -1), t
        if t + 1 < T:
            offs, cnt = reads[t]
            tn = t + 1
            want = list(range(tn + 1)) if tn < N_att else list(range(h - 1)) + list(range(tn - r, tn + 1))
            assert sorted(tn - int(x) for x in offs[0][: cnt[0]]) == want, tn


# ------------------------------------------------------------------ launches of 2048 wavefronts and more
@pytest.mark.parametrize("policy", ALL)
@pytest.mark.parametrize("dt", [synth.F32, synth.BF16, synth.MXFP8])
def test_big_launches(policy, dt):
    """512 lanes x 4 wavefronts: a launch the library runs with its shallow
    row pipeline (depth 2); sampled lanes in lockstep with the oracle."""
    w = tiny(batch=32, heads=16, head_dim=128, dtype=dt)
    check_policy(policy, w, lanes=_sample_lanes(w, 12, 11), waves=4, read_every=9)


# ------------------------------------------------------------------ the Janus-Pro-7B shape (one layer)
def _sample_lanes(w, n, seed):
    rng = np.random.default_rng(seed)
    lanes = {(0, 0), (w.batch - 1, w.heads - 1)}
    while len(lanes) < n:
        lanes.add((int(rng.integers(w.batch)), int(rng.integers(w.heads))))
    return sorted(lanes)


@pytest.mark.parametrize("policy", ALL)
def test_janus_pro_7b_shape_sampled_lanes(policy):
    w = synth.WORKLOADS["janus_pro_7b"]
    trace, stats = check_policy(policy, w, lanes=_sample_lanes(w, 4, 3), layer=w.layers - 1)
    T = w.L_dec
    steps = np.arange(T)[:, None, None]
    ch = trace[:, :, :, 0]
    if policy in (dsa.DSA_POLICY_TOVA, dsa.DSA_POLICY_H2O):
        # every lane evicts exactly once per step from t = N_att - 1 on, a position it holds
        assert ((ch >= 0) == (steps >= w.N_att - 1)).all()
        hi = steps - (n_r_for(policy, w) if policy == dsa.DSA_POLICY_H2O else 0)
        assert ((ch < 0) | ((ch >= 0) & (ch <= hi))).all()
        # a position leaves once: no lane evicts the same position twice
        flat = ch.reshape(T, -1)
        for lane in range(0, flat.shape[1], 97):
            col = flat[:, lane]
            col = col[col >= 0]
            assert len(np.unique(col)) == len(col)


def test_h2o_largest_cache():
    """L_p + N_att = DSA_MAX_H2O_ROWS (4096 fp64 logits of a lane in LDS): the
    cache fills, then evicts on every step, in lockstep with the oracle."""
    w = synth.WORKLOADS["tiny_fp32"].with_(batch=1, heads=2, L_p=96, N_att=4000, N_r=2000, L_dec=4010)
    _, stats = check_policy(dsa.DSA_POLICY_H2O, w)
    assert stats["choices"] == 2 * 11
