"""The allocation-free characterization entry point (dsa_attention_profile_static)
against the workspace one (dsa_attention_profile), through the C ABI.

Both run the same three kernels on the same inputs; the static one takes its
scratch from the library's own device array.  Two calls in a row, the second
on a smaller profile (the array keeps the first call's contents, which must
not reach the second's results), each compared with the workspace entry
point (to 1e-12: the only difference allowed is the order of the per-tile
double additions in LDS) and with the fp64 oracle at the profile's bar (1e-4).
"""
import sys

import numpy as np
import pytest
import torch

import autoregressive_image_generation_amd as dsa
import oracle
import synth
from gpu_util import device_inputs
from oracle import charmap

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = 1e-4


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _outputs(lanes, max_dist):
    return (torch.full((lanes, 3), float("nan"), dtype=torch.float64, device=DEV),
            torch.full((lanes, max_dist), float("nan"), dtype=torch.float64, device=DEV),
            torch.full((lanes, max_dist), float("nan"), dtype=torch.float64, device=DEV))


def _both(w, max_dist, oracle_lanes):
    T, B, H, D, L = w.L_dec, w.batch, w.heads, w.head_dim, w.L_p
    need = dsa.dsa_profile_workspace_bytes(B, H, L, T, max_dist)
    say("static profile %s B=%d H=%d T=%d max_dist=%d: %d scratch bytes of %d" % (
        w.name, B, H, T, max_dist, need, dsa.DSA_PROFILE_STATIC_SCRATCH_BYTES))
    assert need <= dsa.DSA_PROFILE_STATIC_SCRATCH_BYTES
    q, k, v, kp, vp = device_inputs(w, 0, T, DEV)
    stream = torch.cuda.current_stream(DEV)
    ms, vs, ds = _outputs(B * H, max_dist)
    dsa.dsa_attention_profile_static(q, k, kp if L else None, B, H, D, L, T, w.dtype, max_dist, ms, vs, ds, stream)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    mw, vw, dw = _outputs(B * H, max_dist)
    dsa.dsa_attention_profile(q, k, kp if L else None, B, H, D, L, T, w.dtype, max_dist, ws, need, mw, vw, dw,
                              stream)
    torch.cuda.synchronize(DEV)
    for a, b in ((ms, mw), (vs, vw), (ds, dw)):
        a, b = a.cpu().numpy(), b.cpu().numpy()
        assert np.isfinite(a).all()
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)
    mass, vert, diag = ms.cpu().numpy(), vs.cpu().numpy(), ds.cpu().numpy()
    worst = 0.0
    for (b, h) in oracle_lanes:
        lq, lkp, lvp, lk, lv = oracle.lane_inputs(w, 0, b, h, T)
        rm, rv, rd = charmap.profile_lane(lq, lkp, lk, max_dist)
        lane = b * H + h
        err = max(np.abs(mass[lane] - rm).max(), np.abs(vert[lane] - rv).max(), np.abs(diag[lane] - rd).max())
        worst = max(worst, err)
        assert err <= TOL, (b, h, err)
    say("  matches the workspace entry point; oracle max_err=%.3g over %d lanes" % (worst, len(oracle_lanes)))


def test_static_scratch_two_calls_second_smaller():
    big = synth.WORKLOADS["janus_pro_7b"].with_(batch=1)        # 32 lanes x 576 steps: most of the array
    _both(big, 48, [(0, 0), (0, 17), (0, 31)])
    small = synth.WORKLOADS["tiny_fp32"].with_(dtype=synth.BF16, head_dim=128, batch=3, heads=5, L_p=5, L_dec=37)
    _both(small, 12, [(b, h) for b in range(3) for h in range(5)])


def test_static_scratch_repeated_on_one_stream():
    w = synth.WORKLOADS["tiny_fp32"]
    for _ in range(3):
        _both(w, 20, [(0, h) for h in range(w.heads)])
