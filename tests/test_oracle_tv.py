"""Pins of the oracle's total-variation distance between the translated map and a
receiver's own map (oracle.mapflow_oracle.tv_distance): closed forms when the
receiver is the sender itself, a target with no sources, bounds for convex
mixtures, and a pure-Python brute force on tiny inputs.
"""
import numpy as np

from oracle import bruteforce as bf
from oracle import mapflow_oracle as orc

BIAS = dict(sink_n=4, sink_bias=4.0, local_w=12, local_bias=2.0)


def _inputs(rng, H, lens, d):
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    q = rng.normal(size=(H, T, d))
    k = rng.normal(size=(H, T, d))
    return q, k, cu


def test_tv_of_the_sender_itself_is_one_minus_kept_mass():
    """Receiver = sender and W = I: the renormalised kept row differs from the full
    row by (1/kmass - 1) A on kept blocks and A on dropped ones, so TV = 1 - kmass;
    without renormalisation only the dropped mass counts, TV = (1 - kmass) / 2."""
    rng = np.random.default_rng(3)
    H, B = 3, 16
    q, k, cu = _inputs(rng, H, [90, 37], 8)
    for p in (0.6, 0.9):
        res = orc.compress(q, k, cu, B, p, BIAS)
        W = np.eye(H)
        tv = orc.tv_distance(res, W, q, k, cu, B, BIAS)
        tv_raw = orc.tv_distance(res, W, q, k, cu, B, BIAS, renorm=False)
        assert len(tv) == H * len(orc.block_rows(cu, B))
        for (t, s, I), v in tv.items():
            km = res[(t, s, I)].kmass
            assert np.allclose(v, 1.0 - km, atol=1e-12, rtol=0)
            assert np.allclose(tv_raw[(t, s, I)], 0.5 * (1.0 - km), atol=1e-12, rtol=0)
        assert max(float(v.max()) for v in tv.values()) > 0.01
    res = orc.compress(q, k, cu, B, 1.0, BIAS)
    tv = orc.tv_distance(res, np.eye(H), q, k, cu, B, BIAS)
    assert max(float(v.max()) for v in tv.values()) < 1e-12


def test_tv_of_a_target_without_sources_is_one_half():
    rng = np.random.default_rng(4)
    H, B = 2, 16
    q, k, cu = _inputs(rng, H, [70], 8)
    res = orc.compress(q, k, cu, B, 0.9, BIAS)
    W = np.array([[0.0, 0.0], [0.3, 0.7]])
    tv = orc.tv_distance(res, W, q, k, cu, B, BIAS, targets=[0])
    for v in tv.values():
        assert np.allclose(v, 0.5, atol=1e-12, rtol=0)


def test_tv_of_convex_mixtures_lies_in_unit_interval():
    """A simplex row of W mixes renormalised rows (each a distribution), so both
    maps are distributions and TV is in [0, 1]; with an unrelated receiver it is
    far from both ends."""
    rng = np.random.default_rng(5)
    Hs, Ht, B = 4, 5, 16
    q, k, cu = _inputs(rng, Hs, [120, 64], 8)
    qr, kr, _ = _inputs(rng, Ht, [120, 64], 8)
    res = orc.compress(q, k, cu, B, 0.85, BIAS)
    W = rng.dirichlet(np.ones(Hs), size=Ht)
    W[:, 0] = 0.0
    W /= W.sum(axis=1, keepdims=True)
    tv = orc.tv_distance(res, W, qr, kr[:Ht], cu, B, BIAS)
    vals = np.concatenate(list(tv.values()))
    assert vals.min() >= 0.0 and vals.max() <= 1.0 + 1e-12
    assert 0.05 < vals.mean() < 0.95


def test_tv_matches_bruteforce_on_tiny_inputs():
    rng = np.random.default_rng(6)
    Hs, Ht, Hkr, B, d, L = 2, 4, 2, 8, 4, 29
    q, k, cu = _inputs(rng, Hs, [L], d)
    qr = rng.normal(size=(Ht, L, d))
    kr = rng.normal(size=(Hkr, L, d))
    W = rng.normal(size=(Ht, Hs))
    W[1, 0] = 0.0
    res = orc.compress(q, k, cu, B, 0.8, BIAS)
    per_src = {h: bf.bf_compress(q[h].tolist(), k[h].tolist(), B, 0.8, BIAS) for h in range(Hs)}
    for renorm in (True, False):
        tv = orc.tv_distance(res, W, qr, kr, cu, B, BIAS, renorm=renorm)
        for t in range(Ht):
            g = orc.v_head(t, Ht, Hkr)
            A_r = bf.bf_map(qr[t].tolist(), kr[g].tolist(), BIAS)
            ref = bf.bf_tv(per_src, W.tolist(), t, A_r, B, renorm)
            got = np.concatenate([tv[(t, 0, I)] for I in range((L + B - 1) // B)])
            assert np.allclose(got, ref, atol=1e-12, rtol=0)
