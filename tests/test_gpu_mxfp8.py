"""GPU parity of the MXFP8 KV cache (OCP MX E4M3, E8M0 scale per 32 values).

* Bit-exact: every code and scale byte the library writes into the cache
  (prompt rows and appended rows) equals the oracle's quantisation of the same
  bf16 inputs; the workspace layout is the one the library documents (prompt
  region [lanes][L_p] rows at every lane count for MXFP8 states, ring region
  [N_r][lanes] rows, a row = K codes
  then V codes; the rows' 8-byte scale words in a region of their own,
  [lanes][L_p + N_r] words).
* Lockstep: choices and evictions exactly as the oracle run on the quantised
  K / V (near-ties counted), outputs within 1e-3 (both sides attend the same
  dequantised values; the 2e-2 bf16 bound is the stated one, 1e-3 catches a
  stray code).
"""
import sys

import numpy as np
import pytest
import torch

import autoregressive_image_generation_amd as dsa
import oracle
import synth
from gpu_util import check_lane, check_steps, device_inputs, lane_inputs_from, run_dense, run_sparse

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
MX_TOL = 1e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def tiny(**kw):
    base = dict(dtype=synth.MXFP8, head_dim=64)
    base.update(kw)
    return synth.WORKLOADS["tiny_fp32"].with_(**base)


def bf16(x):
    return oracle.widen(x, synth.BF16)


def _parity(w, waves=0, read_every=0, layer=0, lanes=None, fill=None):
    say("mxfp8 parity %s T=%d N_r=%d N_att=%d sink=%d d=%d waves=%d fill=%s" % (
        w.name, w.L_dec, w.N_r, w.N_att, w.sink, w.head_dim, waves, fill))
    T = w.L_dec
    ins = device_inputs(w, layer, T, DEV)
    out, trace, reads = run_sparse(w, ins, T, DEV, waves=waves, read_every=read_every, fill=fill,
                                   read_at=check_steps(w, T))
    lanes = lanes or [(b, h) for b in range(w.batch) for h in range(w.heads)]
    stats = {}
    for (b, h) in lanes:
        li = lane_inputs_from(w, layer, b, h, T)
        check_lane(w, li, out[:, b, h, :].cpu().numpy(), trace[:, b, h, :], stats, reads=reads,
                   lane=b * w.heads + h)
    say("  lanes=%d selections=%d near_ties=%d max_err=%.3g" % (len(lanes), stats["selections"],
                                                              stats["near_ties"], stats["max_err"]))
    assert stats["max_err"] <= MX_TOL
    return stats


def _quantised_rows(x):
    """(codes, scales) of rows [..., d]: a row's K or V codes, and the 4 scale bytes of that half."""
    return oracle.quantize_mxfp8(bf16(x))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("S", [0, 4])
def test_cache_bytes_equal_the_oracle_quantisation(D, S):
    w = tiny(head_dim=D, batch=2, heads=3, sink=S, L_dec=24, N_r=32, N_att=8)
    T, B, H, L = w.L_dec, w.batch, w.heads, w.L_p
    ins = device_inputs(w, 0, T, DEV)
    q, k, v, kp, vp = ins
    nbytes = dsa.dsa_state_workspace_bytes(B, L, w.N_r, w.N_att, H, D, S, w.dtype)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    st = dsa.dsa_state_init(B, L, w.N_r, w.N_att, H, D, S, w.dtype, ws, nbytes, torch.cuda.current_stream(DEV))
    dsa.dsa_append_prompt(st, kp, vp)
    out = torch.empty((B, H, D), dtype=torch.float32, device=DEV)
    for t in range(T):
        dsa.dsa_append_decode_step(st, k[t], v[t], q[t], out)
    torch.cuda.synchronize(DEV)
    dsa.dsa_state_destroy(st)
    raw = ws.cpu().numpy()
    RB = 2 * D                              # a row's codes: K then V
    lanes = B * H
    nb = D // 32
    host = {n: x.cpu().numpy().view(np.uint16) for n, x in zip(("q", "k", "v", "kp", "vp"), ins)}
    # prompt region: [lanes][L_p] rows
    prompt = raw[: lanes * L * RB].reshape(lanes, L, RB)
    # ring region: [N_r][lanes] rows; decode position p (< N_r here) sits at ring index p
    ring = raw[lanes * L * RB: lanes * (L + w.N_r) * RB].reshape(w.N_r, lanes, RB)
    # scale words after the 256-byte aligned cache rows: [lanes][L_p + N_r] words of 8 bytes
    # (byte 4 half + b: block b of K (half 0) or V (half 1)); row L_p + i is ring index i
    off = (lanes * (L + w.N_r) * RB + 255) // 256 * 256
    words = raw[off: off + lanes * (L + w.N_r) * 8].reshape(lanes, L + w.N_r, 8)
    for b in range(B):
        for h in range(H):
            lane = b * H + h
            for half, name in ((0, "kp"), (1, "vp")):
                c, s = _quantised_rows(host[name][b, :, h, :])
                np.testing.assert_array_equal(prompt[lane, :, half * D:(half + 1) * D], c)
                np.testing.assert_array_equal(words[lane, :L, 4 * half: 4 * half + nb], s)
            for half, name in ((0, "k"), (1, "v")):
                c, s = _quantised_rows(host[name][:, b, h, :])
                np.testing.assert_array_equal(ring[:T, lane, half * D:(half + 1) * D], c)
                np.testing.assert_array_equal(words[lane, L:L + T, 4 * half: 4 * half + nb], s)


def test_tiny_all_phases():
    _parity(tiny(), read_every=1)


@pytest.mark.parametrize("D", [64, 128])
def test_sink4_and_head_dims(D):
    _parity(tiny(head_dim=D, sink=4, batch=3, heads=5))


def test_big_launch_sampled_lanes():
    """512 lanes x 4 wavefronts (the shallow row pipeline), sink-free and sink4."""
    rng = np.random.default_rng(5)
    for sink in (0, 4):
        w = tiny(batch=32, heads=16, head_dim=128, sink=sink)
        lanes = sorted({(0, 0), (31, 15)} | {(int(rng.integers(32)), int(rng.integers(16))) for _ in range(10)})
        _parity(w, waves=4, lanes=lanes)


@pytest.mark.parametrize("waves", [1, 2, 4, 8, 16])
def test_every_workgroup_size(waves):
    _parity(tiny(head_dim=128), waves=waves)


@pytest.mark.parametrize("kw", [
    dict(L_p=0),
    dict(N_att=1),
    dict(N_att=2, N_r=3),
    dict(N_att=5, N_r=6, sink=4),
    dict(N_r=64, N_att=64),   # dense through the sparse kernel
    dict(batch=7, heads=3, L_p=5),
])
def test_edge_cases(kw):
    _parity(tiny(**kw))


@pytest.mark.parametrize("kw", [dict(), dict(sink=4, head_dim=128), dict(N_r=64, N_att=64)])
def test_workspace_garbage_never_reaches_the_attention(kw):
    """The workspace starts as 0xFF bytes (NaN codes, an infinite scale byte):
    the cache clear at init keeps every row the kernel reads finite, also the
    rows no token has reached and the current token's own slot."""
    _parity(tiny(**kw), fill=0xFF)


@pytest.mark.parametrize("fill", [None, 0xFF])
def test_dense_matches_oracle_on_quantised_kv(fill):
    w = tiny(head_dim=128, batch=2)
    T = w.L_dec
    ins = device_inputs(w, 0, T, DEV)
    out = run_dense(w, ins, T, DEV, fill=fill).cpu().numpy()
    err = 0.0
    for b in range(w.batch):
        for h in range(w.heads):
            ref = oracle.run_dense_lane(w.L_p, *lane_inputs_from(w, 0, b, h, T))
            err = max(err, float(np.abs(out[:, b, h, :] - ref).max()))
    assert err <= MX_TOL, err


@pytest.mark.parametrize("policy", [dsa.DSA_POLICY_SLIDING_WINDOW, dsa.DSA_POLICY_STREAMING_LLM,
                                    dsa.DSA_POLICY_TOVA, dsa.DSA_POLICY_H2O])
@pytest.mark.parametrize("fill", [None, 0xFF])
def test_policies_on_quantised_kv(policy, fill):
    from test_gpu_policies import check_policy

    _, stats = check_policy(policy, tiny(head_dim=128, batch=2), read_every=4, fill=fill)
    assert stats["max_err"] <= MX_TOL


def test_janus_pro_7b_shape_sampled_lanes():
    w = synth.WORKLOADS["janus_pro_7b"].with_(dtype=synth.MXFP8)
    rng = np.random.default_rng(5)
    lanes = sorted({(0, 0), (w.batch - 1, w.heads - 1)} | {(int(rng.integers(w.batch)), int(rng.integers(w.heads)))
                                                           for _ in range(2)})
    _parity(w, layer=w.layers - 1, lanes=lanes)
