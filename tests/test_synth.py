"""The synthetic input generator (synth/), shared by the oracle and the GPU
tests: deterministic, independent of the thread count and of how a request is
cut into blocks, and its bf16 values are the round-to-nearest-even of its fp32
values."""
import numpy as np
import pytest

import synth


def tiny(**kw):
    return synth.WORKLOADS["tiny_fp32"].with_(**kw)


@pytest.mark.parametrize("stream", [synth.Q, synth.K, synth.V])
def test_deterministic_and_thread_count_independent(stream):
    w = tiny(batch=3, heads=5)
    a = w.decode(0, stream, threads=1)
    b = w.decode(0, stream, threads=8)
    c = w.decode(0, stream)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(a, c)


def test_blocks_equal_slices_of_the_whole():
    w = tiny(batch=3, heads=5, L_dec=40)
    full = w.decode(2, synth.K)
    np.testing.assert_array_equal(w.decode(2, synth.K, tok0=7, ntok=11), full[7:18])
    for b, h in ((0, 0), (2, 4), (1, 3)):
        np.testing.assert_array_equal(w.lane(2, b, h, synth.K), full[:, b, h, :])
        np.testing.assert_array_equal(w.lane(2, b, h, synth.V, tok0=5, ntok=9), w.decode(2, synth.V)[5:14, b, h, :])
    prompt = w.prompt(2, synth.KP)
    np.testing.assert_array_equal(w.lane(2, 1, 3, synth.KP), prompt[1, :, 3, :])


def test_streams_layers_and_seeds_differ():
    w = tiny(batch=2, heads=2)
    base = w.decode(0, synth.Q)
    assert not np.array_equal(base, w.decode(0, synth.K))
    assert not np.array_equal(base, w.decode(1, synth.Q))
    assert not np.array_equal(base, w.with_(seed=1).decode(0, synth.Q))


def test_bf16_values_are_rne_of_fp32():
    w32 = tiny(batch=2, heads=3, head_dim=128, dtype=synth.F32)
    w16 = w32.with_(dtype=synth.BF16)
    for stream in (synth.Q, synth.V):
        f = w32.decode(0, stream).view(np.uint32).astype(np.uint64)
        want = ((f + 0x7FFF + ((f >> 16) & 1)) >> 16).astype(np.uint16)  # round to nearest, ties to even
        np.testing.assert_array_equal(w16.decode(0, stream), want)


def test_queries_and_keys_share_a_relative_position_structure():
    """q and k of a head rotate one base vector by the token's grid position,
    so q_t . k_j depends (up to the 0.1 noise) on the offset between the
    tokens: same-offset pairs agree far better than arbitrary pairs."""
    w = tiny(batch=1, heads=1, head_dim=64, L_dec=64)
    q = w.decode(0, synth.Q)[:, 0, 0, :].astype(np.float64)
    k = w.decode(0, synth.K)[:, 0, 0, :].astype(np.float64)
    s = q @ k.T
    W = w.grid_w
    same = [s[t, t - 1] for t in range(1, 64) if t % W]           # left neighbour on the grid row
    spread_same = np.std(same)
    spread_all = np.std(s[np.tril_indices(64, -1)])
    assert spread_same < 0.4 * spread_all, (spread_same, spread_all)  # 1.12 vs 3.88 at seed 0
