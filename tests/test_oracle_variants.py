"""Pins of the oracle's variant patches (codernav.top article, section on
linear layers, last paragraph; xix.ai article, end of the paragraph on linear
layers): the rotary re-rotation of a cached pair and the short causal
convolution whose taps the seam warm-up feeds.

Each function is held to something other than itself: hand-worked values
(tests/golden/variant_cases.json), group laws of rotations, the definition of
the pair for keys rotated at absolute positions, and numpy's own convolution.
"""
import json
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
G = json.load(open(os.path.join(HERE, "golden", "variant_cases.json")))


def test_rope_matrix_hand_values_and_group_laws():
    r = G["rope"]
    R = oracle.rope_matrix(r["d"], r["p"], r["base"])
    np.testing.assert_allclose(R[:, 0], r["R_e0"], atol=1e-15)
    np.testing.assert_allclose(R[:, 1], r["R_e1"], atol=1e-15)
    rng = np.random.default_rng(1)
    for d in (4, 16, 64):
        a, b = rng.uniform(0, 5000, 2)
        Ra, Rb = oracle.rope_matrix(d, a), oracle.rope_matrix(d, b)
        np.testing.assert_allclose(Ra @ Ra.T, np.eye(d), atol=1e-12)
        np.testing.assert_allclose(Ra @ Rb, oracle.rope_matrix(d, a + b), atol=1e-9)
        np.testing.assert_allclose(oracle.rope_matrix(d, 0.0), np.eye(d), atol=0)
        # channel i pairs with i + d/2 only
        assert np.count_nonzero(np.abs(Ra) > 0) == 2 * d


def _keys(n, d, seed):
    rng = np.random.default_rng(seed)
    k = rng.normal(size=(n, d))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    return k, rng.normal(size=(n, d)), rng


def _rotated(k, p0, base=10000.0):
    """Token t of k at position p0 + t."""
    return np.stack([oracle.rope_matrix(k.shape[1], p0 + t, base) @ k[t] for t in range(len(k))])


@pytest.mark.parametrize("fam", ["linear", "retnet", "mamba2", "deltanet", "gdn"])
def test_rerotate_equals_pair_of_absolutely_rotated_keys(fam):
    """A segment's pair with keys at positions P + t equals the pair at local
    positions t, re-rotated by P: (R T R^T, R S)."""
    n, d, P = 23, 8, 1234.0
    k, v, rng = _keys(n, d, 3)
    g = -np.abs(rng.normal(0.05, 0.02, n)) if fam in ("mamba2", "gdn") else None
    beta = rng.uniform(0.2, 0.9, n) if fam in ("deltanet", "gdn") else None
    gamma = 0.97
    T_loc, S_loc = oracle.pair(fam, _rotated(k, 0.0), v, g, beta, gamma)
    T_abs, S_abs = oracle.pair(fam, _rotated(k, P), v, g, beta, gamma)
    T_rr, S_rr = oracle.rerotate(T_loc, S_loc, P)
    np.testing.assert_allclose(T_rr, T_abs, atol=1e-12)
    np.testing.assert_allclose(S_rr, S_abs, atol=1e-12)
    if fam in ("deltanet", "gdn"):
        # the rotation matters: without it the pair is wrong
        assert np.linalg.norm(S_loc - S_abs) > 1e-3 * np.linalg.norm(S_abs)


@pytest.mark.parametrize("fam", ["gla", "kda"])
def test_rerotate_per_channel_gates_only_with_paired_gates(fam):
    """With a per-channel decay the law holds only when the two channels of
    each rotation pair decay alike (the library refuses these families)."""
    n, d, P = 17, 8, 321.0
    k, v, rng = _keys(n, d, 4)
    beta = rng.uniform(0.2, 0.9, n) if fam == "kda" else None
    g_free = -np.abs(rng.normal(0.1, 0.05, (n, d)))
    g_pair = np.concatenate([g_free[:, : d // 2], g_free[:, : d // 2]], axis=1)
    for g, holds in ((g_pair, True), (g_free, False)):
        T_loc, S_loc = oracle.pair(fam, _rotated(k, 0.0), v, g, beta)
        T_abs, S_abs = oracle.pair(fam, _rotated(k, P), v, g, beta)
        T_rr, S_rr = oracle.rerotate(T_loc, S_loc, P)
        err = oracle.rel_fro(S_rr, S_abs) + oracle.rel_fro(T_rr, T_abs)
        assert (err < 1e-12) if holds else (err > 1e-3), (fam, holds, err)


def test_conv_hand_values_numpy_and_silu():
    c = G["conv"]
    y = oracle.conv(np.array(c["x"], float), np.array(c["w"], float))
    np.testing.assert_array_equal(y, c["y"])
    assert abs(oracle.conv(np.ones((1, 1)), np.ones((1, 1)), act=1)[0, 0] - c["silu_at_1"]) < 1e-15
    rng = np.random.default_rng(9)
    x, w = rng.normal(size=(40, 5)), rng.normal(size=(5, 4))
    y = oracle.conv(x, w)
    for ch in range(5):
        ref = np.convolve(x[:, ch], w[ch][::-1])[:40]   # numpy's full convolution, causal part
        np.testing.assert_allclose(y[:, ch], ref, atol=1e-12)
    ys = oracle.conv(x, w, act=1)
    np.testing.assert_allclose(ys, y / (1 + np.exp(-y)), atol=1e-15)


def test_conv_warm_up_is_the_whole_sequence_convolution():
    """A seam window's outputs with the previous segment's last K-1 raw
    inputs as history are the whole sequence's outputs there; with a cold
    (zero) history its first K-1 tokens differ."""
    rng = np.random.default_rng(10)
    K, w, s = 4, 8, 50
    x, taps = rng.normal(size=(90, 6)), rng.normal(size=(6, K))
    full = oracle.conv(x, taps, act=1)
    warm = oracle.conv(x[s - K + 1: s + w], taps, act=1)[K - 1:]
    np.testing.assert_allclose(warm, full[s: s + w], atol=1e-14)
    cold = oracle.conv(x[s: s + w], taps, act=1)
    assert np.abs(cold[: K - 1] - full[s: s + K - 1]).max() > 1e-3
    np.testing.assert_allclose(cold[K - 1:], full[s + K - 1: s + w], atol=1e-14)
