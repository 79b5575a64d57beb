"""Pins of the oracle's fp8 tile codec (oracle/mx_codec.py) against what the E4M3
and block-scale definitions fix: landmark values of the format, nearest-even
rounding by brute force over all codes, the scale rule, the error bound, and
the codec inside translated retrieval.
"""
import math

import numpy as np
import pytest

from oracle import mx_codec as mx
from oracle import mapflow_oracle as orc

FINITE = [c for c in range(256) if not math.isnan(mx.e4m3_value(c))]
NONNEG = [c for c in range(0x7F)]  # 0x00 .. 0x7E: every finite value >= 0


def test_e4m3_landmarks():
    """Values fixed by the OCP E4M3 layout (bias 7, 3 mantissa bits, no inf)."""
    v = mx.e4m3_value
    assert v(0x00) == 0.0 and math.copysign(1.0, v(0x80)) == -1.0 and v(0x80) == 0.0
    assert v(0x01) == 2.0 ** -9          # smallest subnormal
    assert v(0x07) == 7 * 2.0 ** -9      # largest subnormal
    assert v(0x08) == 2.0 ** -6          # smallest normal
    assert v(0x38) == 1.0
    assert v(0x39) == 1.125
    assert v(0x70) == 128.0
    assert v(0x78) == 256.0
    assert v(0x7E) == 448.0              # largest finite
    assert math.isnan(v(0x7F)) and math.isnan(v(0xFF))
    assert v(0xB8) == -1.0
    assert len(FINITE) == 254


def test_e4m3_values_increase_with_code():
    vals = [mx.e4m3_value(c) for c in NONNEG]
    assert all(a < b for a, b in zip(vals, vals[1:]))


def _nearest_even_bruteforce(x: float) -> int:
    best, bd = None, None
    for c in NONNEG:
        d = abs(mx.e4m3_value(c) - x)
        if bd is None or d < bd or (d == bd and (c & 1) == 0):
            best, bd = c, d
    return best


def test_encode_is_nearest_even_bruteforce():
    rng = np.random.default_rng(11)
    xs = list(rng.uniform(0, 448, 300)) + list(2.0 ** rng.uniform(-12, 8.8, 600))
    # exact values, midpoints (ties) and quarter points between neighbours
    for c in range(0x7E):
        a, b = mx.e4m3_value(c), mx.e4m3_value(c + 1)
        xs += [a, (a + b) / 2, 0.75 * a + 0.25 * b, 0.25 * a + 0.75 * b]
    xs = [x for x in xs if 0.0 <= x <= 448.0]
    for x in xs:
        assert mx.e4m3_code(x) == _nearest_even_bruteforce(x), x
    assert np.array_equal(mx.e4m3_codes(np.array(xs)), [mx.e4m3_code(x) for x in xs])


def test_encode_ties_go_to_even_mantissa():
    assert mx.e4m3_code(1.0625) == 0x38      # between 1.0 (m=0) and 1.125 (m=1)
    assert mx.e4m3_code(1.1875) == 0x3A      # between 1.125 (m=1) and 1.25 (m=2)
    assert mx.e4m3_code(1.5 * 2.0 ** -9) == 0x02  # subnormal tie 1.5 -> 2
    assert mx.e4m3_code(0.5 * 2.0 ** -9) == 0x00  # half the smallest subnormal -> 0
    assert mx.e4m3_code(248.0) == 0x78       # between 240 (m=7) and 256 (m=0) -> 256


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        mx.e4m3_code(449.0)
    with pytest.raises(ValueError):
        mx.e4m3_codes(np.array([1.0, -1.0]))


def test_block_scale_rule():
    for k in range(-30, 1):
        for f in (1.0, 1.3, 1.999):
            a = f * 2.0 ** k
            e = mx.block_scale_exponent(a)
            assert e == k - 7
            assert 128.0 <= a * 2.0 ** -e < 256.0
    assert mx.block_scale_exponent(0.0) == -126
    assert mx.block_scale_exponent(2.0 ** -125) == -126   # clamped
    P = np.zeros((2, 64))
    P[0, 5] = 1.0
    P[1, 40] = 0.3
    codes, scales = mx.encode_tile(P)
    assert scales.shape == (2, 2)
    assert scales[0, 0] == 120 and scales[0, 1] == 1      # 2^-7 ; all-zero block
    assert scales[1, 0] == 1 and scales[1, 1] == 127 - 2 - 7
    assert codes[0, 5] == 0x70                            # 1.0 * 2^7 = 128


def test_scale_is_shared_by_32_keys():
    """Small values next to a large one in the same 32-key block flush to zero;
    in the next block they keep their own scale."""
    P = np.zeros((1, 64))
    P[0, 0:16] = 2.0 ** -20
    P[0, 16] = 1.0
    P[0, 32:48] = 2.0 ** -20
    q = mx.quantize(P)
    assert np.all(q[0, 0:16] == 0.0)
    assert q[0, 16] == 1.0
    assert np.all(q[0, 32:48] == 2.0 ** -20)


def test_quantize_within_bound_and_exact_on_grid():
    rng = np.random.default_rng(5)
    s = rng.normal(0, 2.5, (64, 256))
    P = np.exp(s - s.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    P[:, 200:] = 0.0
    q = mx.quantize(P)
    assert np.all(np.abs(q - P) <= mx.error_bound(P))
    assert np.all(q >= 0)
    codes, scales = mx.encode_tile(P)
    assert np.array_equal(mx.decode_tile(codes, scales), q)
    # values on the grid of their block round-trip exactly, wherever the block
    # keeps its scale (a maximum that rounds up to the next power of two moves
    # the block to a coarser grid)
    _, s2 = mx.encode_tile(q)
    same = np.repeat(s2 == scales, mx.MX_BLOCK, axis=1)
    assert same.mean() > 0.5
    assert np.array_equal(mx.quantize(q)[same], q[same])
    # relative error of the larger elements is at most 2^-4
    big = P > 2.0 ** -6 * P.max(axis=1, keepdims=True)
    assert np.all(np.abs(q - P)[big] <= 2.0 ** -4 * P[big])


def _grid_rowresult(rng, B, I, L):
    """A RowResult whose kept tiles are already exact codec values."""
    rows = np.arange(I * B, min((I + 1) * B, L))
    ncols = min((I + 1) * B, L)
    P = np.zeros((len(rows), ncols))
    for J in range(I + 1):
        t = np.zeros((B, B))
        blk = rng.random((len(rows), min(B, ncols - J * B))) ** 6 / (I + 1)
        t[:blk.shape[0], :blk.shape[1]] = blk
        # twice: a block whose maximum rounds up to a power of two settles on
        # the coarser grid in the second pass
        t = mx.quantize(mx.quantize(t))
        assert np.array_equal(mx.quantize(t), t)
        P[:, J * B:J * B + blk.shape[1]] = t[:blk.shape[0], :blk.shape[1]]
    M = orc.block_masses(P, B, I + 1)
    sel = orc.topp_select(M, 0.9)
    kmass = sum(P[:, J * B:(J + 1) * B].sum(axis=1) for J in sel.kept)
    return orc.RowResult(rows, M, sel, P, np.zeros(len(rows)), kmass, set())


def test_apply_row_codec_exact_on_grid_and_bounded():
    rng = np.random.default_rng(9)
    B, d = 32, 16
    W = rng.normal(size=(2, 3))
    for L in (128, 100):   # a full block-row of 32 rows, and a ragged one
        src = {h: _grid_rowresult(rng, B, 3, L) for h in range(3)}
        v = rng.normal(size=(L, d))
        a = orc.apply_row(src, W, 1, v, B)
        b = orc.apply_row(src, W, 1, v, B, codec="mxfp8")
        assert np.array_equal(a, b)
    # real softmax rows: |O_q - O| <= sum_h |W| / kmass * sum_j bound_j |v_j|
    q = rng.normal(size=(L, d))
    k = rng.normal(size=(L, d))
    bias = dict(sink_n=4, sink_bias=4.0, local_w=16, local_bias=2.0)
    src = {h: orc.compress_row(q, k, 3, B, 0.9, bias) for h in range(3)}
    a = orc.apply_row(src, W, 0, v, B)
    b = orc.apply_row(src, W, 0, v, B, codec="mxfp8")
    bound = np.zeros_like(a)
    for h, rr in src.items():
        for J in rr.kept:
            eb = mx.error_bound(rr.tile(J, B))[:len(rr.rows), :]
            vj = np.zeros((B, d))
            vj[:min(B, L - J * B)] = v[J * B:min((J + 1) * B, L)]
            bound += (abs(W[0, h]) / rr.kmass)[:, None] * (eb @ np.abs(vj))
    assert np.all(np.abs(b - a) <= bound * (1 + 1e-9) + 1e-15)
    assert np.linalg.norm(b - a) > 0


def test_apply_rejects_unknown_codec():
    with pytest.raises(ValueError):
        orc.apply_row({}, np.zeros((1, 1)), 0, np.zeros((4, 2)), 32, codec="int4")


def _grid_from_bits():
    """All finite non-negative E4M3 values, decoded here from the bit layout
    (exponent field f, mantissa m: f = 0 -> m/8 * 2^-6, else (1 + m/8) * 2^(f-7);
    0x7F is NaN), independently of mx.e4m3_value."""
    vals = []
    for code in range(0x7F):
        f, m = code >> 3, code & 7
        vals.append(m / 8.0 * 2.0 ** -6 if f == 0 else (1.0 + m / 8.0) * 2.0 ** (f - 7))
    return np.array(sorted(vals))


@pytest.mark.parametrize("E", [7, 0, -5, -30])
def test_error_bound_is_the_grid_half_spacing(E):
    """error_bound pinned against the E4M3 grid by brute force: in a block whose
    maximum lies in [2^E, 2^(E+1)) (scale e = E - 7), every element p = y 2^e
    rounds to within half the local grid spacing of y; the worst case is the
    midpoint of two neighbours.  At every midpoint the bound must cover that
    half spacing (validity), and it must not be loose: it is attained exactly on
    the subnormal part of the grid and within a factor 1 + 1/16 at the bottom of
    every normal binade (tightness), so a looser or tighter formula fails."""
    g = _grid_from_bits()
    assert len(g) == 127 and g[0] == 0.0 and g[-1] == 448.0
    e = E - 7
    # scaled values of such a block lie in [0, 256): neighbours up to 256
    g = g[g <= 256.0]
    lo, hi = g[:-1], g[1:]
    mid = (lo + hi) / 2
    half = (hi - lo) / 2
    # one block per midpoint: the midpoint and a maximum 1.5 * 2^E that fixes the scale
    P = np.zeros((len(mid), 32))
    P[:, 0] = mid * 2.0 ** e
    P[:, 1] = 1.5 * 2.0 ** E
    assert all(mx.block_scale_exponent(a) == e for a in P.max(axis=1))
    bound = mx.error_bound(P)[:, 0]
    worst = half * 2.0 ** e
    assert np.all(worst <= bound), "the bound misses the rounding error at a midpoint"
    ratio = worst / bound
    sub = hi <= 2.0 ** -6                       # both neighbours on the subnormal spacing
    assert np.allclose(ratio[sub], 1.0)
    assert ratio[~sub].max() == pytest.approx(1.0 / (1.0 + 1.0 / 16), rel=1e-12)
    # the codec really reaches the half spacing there (ties round to even)
    q = mx.quantize(P)[:, 0]
    assert np.allclose(np.abs(q - P[:, 0]), worst)
