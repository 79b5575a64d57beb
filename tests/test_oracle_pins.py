"""Pins of the fp64 oracle against things other than itself: closed forms, library
routines (torch's scaled_dot_product_attention and matmul in float64 on the CPU),
brute force and invariants.

Each test names the mistake it would catch. Method references: MapFlow
("Accelerating Cross-Model LLM Inference via Attention Map Reuse") §3.3, §4,
§5.2, §5.4; AttnCache guide ("AttnCache Guide: Reusing Attention Maps in LLM
Prefill"), "The Quadratic Self-Attention Cost" and its PyTorch prototype.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import mapflow_oracle as orc
from oracle import bruteforce as bf
from cross_model_sparse_amd import workloads as wlmod

NOBIAS = dict(sink_n=4, sink_bias=0.0, local_w=64, local_bias=0.0)
BIAS = dict(sink_n=4, sink_bias=4.0, local_w=64, local_bias=2.0)


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def test_uniform_map_closed_form():
    """q = 0 and no bias: every causal logit equal, P[i, j] = 1 / (i + 1).
    Catches a wrong causal direction, a missing mask or an off-by-one diagonal."""
    L, d = 37, 8
    q = np.zeros((L, d))
    k = rand((L, d), 1)
    A = orc.attention_map(q, k, NOBIAS)
    i, j = np.meshgrid(np.arange(L), np.arange(L), indexing="ij")
    expect = np.where(j <= i, 1.0 / (i + 1), 0.0)
    np.testing.assert_allclose(A, expect, rtol=0, atol=1e-15)


def test_sink_and_local_closed_form():
    """q = 0: the logit of (i, j) is only the bias, so P has a closed form.
    sink: +b_s on j < 4; local: +b_l on 0 <= i - j < w. Catches a bias on the wrong
    axis, a wrong window edge or natural-log / log2 confusion."""
    L, d, w = 40, 4, 6
    bias = dict(sink_n=4, sink_bias=4.0, local_w=w, local_bias=2.0)
    A = orc.attention_map(np.zeros((L, d)), rand((L, d), 2), bias)
    for i in range(L):
        logit = [(4.0 if j < 4 else 0.0) + (2.0 if 0 <= i - j < w else 0.0) for j in range(i + 1)]
        z = sum(math.exp(x) for x in logit)
        for j in range(L):
            e = math.exp(logit[j]) / z if j <= i else 0.0
            assert abs(A[i, j] - e) < 1e-15


def test_uniform_block_masses_fractions():
    """q = 0, no bias: M[I, J] = sum_{i in I} |J cap [0, i]| / (i + 1), exact rationals."""
    L, B, d = 22, 4, 3
    q = np.zeros((L, d))
    k = rand((L, d), 3)
    for I in range(orc.nblocks(L, B)):
        r = orc.compress_row(q, k, I, B, 0.9, NOBIAS)
        for J in range(I + 1):
            f = Fraction(0)
            for i in range(I * B, min((I + 1) * B, L)):
                cnt = max(0, min(i, (J + 1) * B - 1) - J * B + 1)
                f += Fraction(cnt, i + 1)
            assert abs(r.M[J] - float(f)) < 1e-14


def test_tie_break_lower_block_first():
    """q = 0, no bias: blocks J < I of a row carry exactly equal masses (identical
    probabilities), so the cut must prefer the lower key-block index.
    Row I = 3, B = 4: M0 = M1 = M2 = 4 * (1/13 + 1/14 + 1/15 + 1/16), M3 smaller.
    p = 0.5 needs two blocks -> {0, 1}. Catches a reversed tie rule."""
    L, B = 16, 4
    q = np.zeros((L, 2))
    k = rand((L, 2), 4)
    r = orc.compress_row(q, k, 3, B, 0.5, NOBIAS)
    assert r.M[0] == r.M[1] == r.M[2] > r.M[3]
    assert r.kept == [0, 1]
    # p -> 0+: exactly the argmax, lowest index among the tied maxima
    assert orc.compress_row(q, k, 3, B, 1e-9, NOBIAS).kept == [0]
    # one block short of the total: three blocks, the tied ones
    m = [Fraction(4, 13) + Fraction(4, 14) + Fraction(4, 15) + Fraction(4, 16)] * 3
    m.append(Fraction(1, 13) + Fraction(2, 14) + Fraction(3, 15) + Fraction(4, 16))
    assert sum(m) == 4
    p = float((m[0] * 2 + m[0] / 2) / 4)  # needs a third block
    assert orc.compress_row(q, k, 3, B, p, NOBIAS).kept == [0, 1, 2]


def test_key_shift_invariance():
    """Adding one vector u to every key adds q_i . u to a whole row: P is unchanged.
    Catches a per-column normalisation or a softmax over the wrong axis."""
    L, d = 50, 16
    q, k = rand((L, d), 5), rand((L, d), 6)
    u = rand((1, d), 7) * 3
    np.testing.assert_allclose(orc.attention_map(q, k, BIAS), orc.attention_map(q, k + u, BIAS),
                               rtol=1e-12, atol=1e-14)


def test_gqa_constant_values():
    """V head g constant c_g: renormalised rows sum to 1, so O_t = c_g(t) * sum_h W[t,h]
    on every row. Pins g(t) = floor(t * Hkv / Ht) and the renormalisation."""
    wl = wlmod.make_workload(wlmod.Spec("gqa", (100,), 3, 8, 2, 16, 16, 0.8, "fp32", 8,
                                        "gauss", w_var=1.0, seed=11))
    v = np.zeros((2, 100, 16))
    v[0] += 1.5
    v[1] -= 0.25
    res = orc.compress(wl.q, wl.k, wl.cu_seqlens, 16, 0.8, wl.bias())
    out = orc.apply(res, wl.W, v, wl.cu_seqlens, 16, 2)
    O = orc.assemble(out, 8, wl.cu_seqlens, 16, 16)
    for t in range(8):
        c = 1.5 if t < 4 else -0.25
        np.testing.assert_allclose(O[t], c * wl.W[t].astype(np.float64).sum(), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# library routines
# ---------------------------------------------------------------------------

def sdpa_reference(q, k, v, bias):
    """torch scaled_dot_product_attention (float64, CPU) with an explicit additive mask."""
    L = q.shape[0]
    i = torch.arange(L)[:, None]
    j = torch.arange(L)[None, :]
    mask = torch.zeros(L, L, dtype=torch.float64)
    mask += bias["sink_bias"] * (j < bias["sink_n"])
    mask += bias["local_bias"] * ((i - j >= 0) & (i - j < bias["local_w"]))
    mask = mask.masked_fill(j > i, float("-inf"))
    t = lambda a: torch.as_tensor(np.asarray(a, dtype=np.float64))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=mask)[0, 0].numpy()


@pytest.mark.parametrize("lens,B", [([96], 32), ([70, 33, 1], 16), ([128], 64)])
def test_p1_identity_is_dense_attention(lens, B):
    """p = 1 and W = I: the translated retrieval is exactly dense causal attention.
    Compared with torch's SDPA (its own 1/sqrt(d) scaling). Catches a dropped scale,
    transposed operands, a wrong V head or a missing block."""
    H, d = 3, 16
    spec = wlmod.Spec("p1", tuple(lens), H, H, H, d, B, 1.0, "fp32", 24, "gauss", w_var=1.0, seed=21)
    wl = wlmod.make_workload(spec, W=np.eye(H, dtype=np.float32))
    res = orc.compress(wl.q, wl.k, wl.cu_seqlens, B, 1.0, wl.bias())
    O = orc.assemble(orc.apply(res, wl.W, wl.v, wl.cu_seqlens, B, H), H, wl.cu_seqlens, B, d)
    D = orc.dense_attention(wl.q, wl.k, wl.v, wl.cu_seqlens, wl.bias())
    for h in range(H):
        for s, (a, L) in enumerate(orc.seqs(wl.cu_seqlens)):
            ref = sdpa_reference(wl.q[h, a:a + L], wl.k[h, a:a + L], wl.v[h, a:a + L], wl.bias())
            np.testing.assert_allclose(O[h, a:a + L], ref, rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(D[(h, s)], ref, rtol=1e-10, atol=1e-12)


def test_dense_gqa_matches_sdpa():
    """Dense attention with Hq = 4, Hkv = 2: head h reads K/V head floor(h * Hkv / Hq)."""
    Hq, Hkv, L, d = 4, 2, 45, 8
    q, k, v = rand((Hq, L, d), 31), rand((Hkv, L, d), 32), rand((Hkv, L, d), 33)
    cu = np.array([0, L], dtype=np.int32)
    D = orc.dense_attention(q, k, v, cu, BIAS)
    for h in range(Hq):
        g = h // 2
        np.testing.assert_allclose(D[(h, 0)], sdpa_reference(q[h], k[g], v[g], BIAS), rtol=1e-10, atol=1e-12)


def test_dense_row_ranges_match_sdpa_rows():
    """Dense attention restricted to a row window per sequence (the sampled
    full-length check uses this) equals the same rows of torch's
    scaled_dot_product_attention over the whole sequence, GQA included; an
    empty window gives no rows."""
    Hq, Hkv, d = 4, 2, 8
    lens = [70, 33, 5]
    cu = np.array([0, 70, 103, 108], dtype=np.int32)
    T = int(cu[-1])
    q, k, v = rand((Hq, T, d), 41), rand((Hkv, T, d), 42), rand((Hkv, T, d), 43)
    ranges = {0: (17, 51), 1: (0, 33), 2: (3, 3)}
    D = orc.dense_attention(q, k, v, cu, BIAS, row_ranges=ranges)
    for h in range(Hq):
        g = h // 2
        for s, (a, L) in enumerate(orc.seqs(cu)):
            r0, r1 = ranges[s]
            ref = sdpa_reference(q[h, a:a + L], k[g, a:a + L], v[g, a:a + L], BIAS)[r0:r1]
            assert D[(h, s)].shape == (r1 - r0, d)
            np.testing.assert_allclose(D[(h, s)], ref, rtol=1e-10, atol=1e-12)


def test_identity_w_is_per_head_reuse():
    """W = I: O_h = renorm(A_hat_h) V_h, the cached-map reuse path. The reference here
    builds the dense sparsified map from SDPA-style softmax (torch), zeroes dropped
    blocks, divides rows by their sums and multiplies by V with torch.matmul."""
    H, L, d, B, p = 2, 90, 8, 16, 0.7
    spec = wlmod.Spec("wI", (L,), H, H, H, d, B, p, "fp32", 10, "gauss", w_var=1.0, seed=41)
    wl = wlmod.make_workload(spec, W=np.eye(H, dtype=np.float32))
    res = orc.compress(wl.q, wl.k, wl.cu_seqlens, B, p, wl.bias())
    O = orc.assemble(orc.apply(res, wl.W, wl.v, wl.cu_seqlens, B, H), H, wl.cu_seqlens, B, d)
    for h in range(H):
        q = torch.as_tensor(wl.q[h], dtype=torch.float64)
        k = torch.as_tensor(wl.k[h], dtype=torch.float64)
        i = torch.arange(L)[:, None]
        j = torch.arange(L)[None, :]
        s = q @ k.T / math.sqrt(d) + 4.0 * (j < 4) + 2.0 * ((i - j >= 0) & (i - j < 10))
        A = torch.softmax(s.masked_fill(j > i, float("-inf")), dim=1)
        keep = torch.zeros(L, L, dtype=torch.bool)
        for I in range(orc.nblocks(L, B)):
            for J in res[(h, 0, I)].kept:
                keep[I * B:(I + 1) * B, J * B:(J + 1) * B] = True
        Ak = A * keep
        Ak = Ak / Ak.sum(dim=1, keepdim=True)
        ref = (Ak @ torch.as_tensor(wl.v[h], dtype=torch.float64)).numpy()
        np.testing.assert_allclose(O[h], ref, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------------------
# brute force
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("L,B,p,seed", [(1, 8, 0.9, 1), (7, 8, 0.5, 2), (33, 8, 0.9, 3),
                                        (64, 16, 0.6, 4), (40, 8, 0.95, 5), (24, 4, 0.3, 6),
                                        (30, 8, 1.0, 7)])
def test_bruteforce_pipeline(L, B, p, seed):
    """Pure-Python map, masses, exhaustive subset selection, kept mass and translated
    output agree with the numpy oracle on tiny inputs."""
    Hs, Ht, d = 2, 3, 4
    rng = np.random.default_rng(seed)
    q, k, v = rng.standard_normal((Hs, L, d)), rng.standard_normal((Hs, L, d)), rng.standard_normal((1, L, d))
    W = rng.standard_normal((Ht, Hs))
    bias = dict(sink_n=4, sink_bias=4.0, local_w=5, local_bias=2.0)
    cu = np.array([0, L], dtype=np.int32)
    res = orc.compress(q, k, cu, B, p, bias)
    per_src = {}
    for h in range(Hs):
        per_src[h] = bf.bf_compress(q[h].tolist(), k[h].tolist(), B, p, bias)
        for I in range(orc.nblocks(L, B)):
            r, b = res[(h, 0, I)], per_src[h][I]
            np.testing.assert_allclose(r.M, b["M"], rtol=1e-12, atol=1e-14)
            assert r.kept == b["kept"]
            np.testing.assert_allclose(r.kmass, b["kmass"], rtol=1e-12, atol=1e-14)
    O = orc.assemble(orc.apply(res, W, v, cu, B, 1), Ht, cu, B, d)
    for t in range(Ht):
        ref = bf.bf_apply(per_src, W.tolist(), t, v[0].tolist(), B)
        np.testing.assert_allclose(O[t], np.array(ref), rtol=1e-11, atol=1e-12)


def test_bruteforce_workload1():
    """Workload 1 itself (L = 256, B = 32: 8 candidate blocks, 256 subsets per row),
    first source head: masses and kept sets from exhaustive search."""
    wl = wlmod.make_config(1)
    b = bf.bf_compress(wl.q[0].tolist(), wl.k[0].tolist(), 32, 0.9, wl.bias())
    res = orc.compress(wl.q, wl.k, wl.cu_seqlens, 32, 0.9, wl.bias(), heads=[0])
    for I in range(8):
        np.testing.assert_allclose(res[(0, 0, I)].M, b[I]["M"], rtol=1e-12)
        assert res[(0, 0, I)].kept == b[I]["kept"]


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def small_multi():
    wl = wlmod.small_variant(5, [200, 130, 77, 300], Hs=4, Ht=5, Hkv=5)
    B = 32
    res = orc.compress(wl.q, wl.k, wl.cu_seqlens, B, 0.9, wl.bias())
    return wl, B, res


def test_mass_rows_and_selection_invariants(small_multi):
    """Row masses sum to the number of valid rows; masses >= 0; the kept set reaches
    p of the total and is minimal; kept masses dominate dropped ones; renormalised
    kept rows sum to 1; kept mass summed over the rows equals the kept block masses."""
    wl, B, res = small_multi
    p = 0.9
    for (h, s, I), r in res.items():
        assert abs(r.M.sum() - len(r.rows)) < 1e-12 * max(1, len(r.rows))
        assert (r.M >= 0).all()
        kept = r.kept
        ksum = sum(r.M[J] for J in kept)
        assert ksum >= p * r.M.sum() * (1 - 1e-15)
        assert ksum - min(r.M[J] for J in kept) < p * r.M.sum()
        dropped = [J for J in range(len(r.M)) if J not in kept]
        if dropped:
            assert min(r.M[J] for J in kept) >= max(r.M[J] for J in dropped)
        assert kept == sorted(kept)
        rowsum = sum(r.P[:, J * B:(J + 1) * B].sum(axis=1) for J in kept) / r.kmass
        np.testing.assert_allclose(rowsum, 1.0, rtol=1e-13)
        assert abs(r.kmass.sum() - ksum) < 1e-12 * len(r.rows)


def test_bsr_layout(small_multi):
    wl, B, res = small_multi
    rp, ci = orc.bsr_layout(res, 4, wl.cu_seqlens, B)
    assert rp[0] == 0 and (np.diff(rp) >= 1).all() and rp[-1] == len(ci)
    br = orc.block_rows(wl.cu_seqlens, B)
    for h in range(4):
        for g, (s, I) in enumerate(br):
            r = h * len(br) + g
            assert list(ci[rp[r]:rp[r + 1]]) == res[(h, s, I)].kept


def test_linear_in_w_and_source_permutation(small_multi):
    """O is linear in W, and permuting the sources together with W's columns leaves
    it unchanged. Catches a mix-up between W's row and column axes."""
    wl, B, res = small_multi
    cu = wl.cu_seqlens
    rng = np.random.default_rng(9)
    W1, W2 = rng.standard_normal((5, 4)), rng.standard_normal((5, 4))
    O = lambda W, r=res: orc.assemble(orc.apply(r, W, wl.v, cu, B, 5), 5, cu, B, 128)
    np.testing.assert_allclose(O(W1 + 2 * W2), O(W1) + 2 * O(W2), rtol=1e-10, atol=1e-12)
    perm = [2, 0, 3, 1]
    res_p = {(perm.index(h), s, I): r for (h, s, I), r in res.items()}
    np.testing.assert_allclose(O(W1[:, perm], res_p), O(W1), rtol=1e-12, atol=1e-13)
    # a single nonzero W[t, h] isolates one pair: O_t = W[t,h] * renorm(A_h) V_t
    E = np.zeros((5, 4))
    E[3, 1] = 1.0
    Oe = O(E)
    assert np.abs(Oe[[0, 1, 2, 4]]).max() == 0.0
    O2 = O(2.5 * E)
    np.testing.assert_allclose(O2[3], 2.5 * Oe[3], rtol=1e-12, atol=1e-14)


def test_multiturn_prefix_rows_repeat(small_multi):
    """Rows wholly inside a sequence's copy of sequence 0's head have the same kept
    sets, masses and kept mass as sequence 0 (causal rows only see the prefix)."""
    wl, B, res = small_multi
    n = 0
    for s in range(1, 4):
        P = wl.prefix[s]
        for I in range(P // B):
            for h in range(4):
                a, b0 = res[(h, s, I)], res[(h, 0, I)]
                assert a.kept == b0.kept
                np.testing.assert_allclose(a.M, b0.M, rtol=1e-13)
                np.testing.assert_allclose(a.kmass, b0.kmass, rtol=1e-13)
                n += 1
    assert n > 0


def test_ambiguity_band():
    """Constructed masses: the cut block within 1e-5 of the threshold, and two masses
    within 1e-5 of each other at the cut, are flagged; clear cases are not."""
    M = np.array([0.5, 0.3, 0.2])
    sel = orc.topp_select(M, 0.8)
    assert sel.kept == [0, 1]
    assert orc.ambiguous_blocks(M, sel) == {1, 2}  # prefix 0.8 sits on the threshold
    sel = orc.topp_select(M, 0.7)
    assert sel.kept == [0, 1] and orc.ambiguous_blocks(M, sel) == set()
    M = np.array([0.4, 0.3, 0.3 * (1 + 5e-6)])
    sel = orc.topp_select(M, 0.65)
    assert sel.kept == [0, 2]
    assert orc.ambiguous_blocks(M, sel) == {1, 2}
    assert orc.ambiguous_blocks(M, orc.topp_select(M, 1.0)) == set()


def test_workload_generator():
    """Seeded determinism, bf16 round-to-nearest-even, multi-turn structure."""
    a, b = wlmod.make_workload(wlmod.SPECS[2], lens=[64]), wlmod.make_workload(wlmod.SPECS[2], lens=[64])
    assert np.array_equal(a.q, b.q) and np.array_equal(a.W, b.W)
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.0 - 2 ** -7 - 2 ** -9],
                 dtype=np.float32)
    back = wlmod.bf16_bits_to_f32(wlmod.f32_to_bf16_bits(x))
    assert list(back) == [1.0, 1.0, 1.0 + 4 * 2 ** -8, 1.0, -2.0 - 2 ** -6]
    w5 = wlmod.make_config(5)
    lens = w5.lens
    assert len(lens) == 16 and min(lens) >= 1024 and max(lens) <= 8192
    for s in range(1, 16):
        P = min(lens[s] // 2, lens[0])
        a0, a1 = int(w5.cu_seqlens[0]), int(w5.cu_seqlens[s])
        assert np.array_equal(w5.q[:, a1:a1 + P], w5.q[:, a0:a0 + P])
        assert not np.array_equal(w5.k[:, a1 + P:a1 + P + 8], w5.k[:, a0 + P:a0 + P + 8])
    w4W = wlmod.make_workload(wlmod.SPECS[4], lens=[128]).W
    assert ((w4W != 0).sum(axis=1) == 4).all() and np.allclose(w4W.sum(axis=1), 1.0, atol=1e-6)
    assert (w4W >= 0).all()


# ---------------------------------------------------------------------------
# shared prefixes (MapFlow §5.3, §2.3)
# ---------------------------------------------------------------------------

def test_prefix_alias_matches_planted_prefixes():
    """The multi-turn generator copies the first P_s = min(L_s // 2, L_0) tokens of
    sequence 0 into sequence s (q, k, v, every head); the rest is fresh noise. So
    exactly the full block-rows (I + 1) * B <= P_s of s > 0 share sequence 0's
    block-row I. Catches: comparing the wrong token range, aliasing partial blocks,
    aliasing across different block indices, or picking a later sequence."""
    wl = wlmod.small_variant(5, [300, 520, 64, 130, 700, 300], Hs=3, Ht=3, Hkv=3)
    B = 32
    cu, lens = wl.cu_seqlens, wl.lens
    rows = orc.block_rows(cu, B)
    first = np.concatenate([[0], np.cumsum([orc.nblocks(L, B) for L in lens])])
    expect = np.arange(len(rows))
    for g, (s, I) in enumerate(rows):
        if s > 0 and (I + 1) * B <= wl.prefix[s]:
            expect[g] = first[0] + I
    got = orc.prefix_alias(wl.q, wl.k, cu, B)
    assert got.tolist() == expect.tolist()
    # sequence 5 repeats sequence 0's length and prefix rule; still sequence 0 first
    assert any(got[first[5] + I] == I for I in range(3))


def _bf_alias(q, k, cu, B):
    """Pure-Python brute force: compare the token lists of every prefix directly."""
    rows = orc.block_rows(cu, B)
    idx = {r: g for g, r in enumerate(rows)}
    out = []
    for g, (s, I) in enumerate(rows):
        a, L = int(cu[s]), int(cu[s + 1] - cu[s])
        n = (I + 1) * B
        hit = g
        if n <= L:
            mine = [(q[h][a + t].tolist(), k[h][a + t].tolist()) for h in range(q.shape[0]) for t in range(n)]
            for s2 in range(s):
                a2, L2 = int(cu[s2]), int(cu[s2 + 1] - cu[s2])
                if n > L2:
                    continue
                other = [(q[h][a2 + t].tolist(), k[h][a2 + t].tolist()) for h in range(q.shape[0]) for t in range(n)]
                if mine == other:
                    hit = idx[(s2, I)]
                    break
        out.append(hit)
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_prefix_alias_bruteforce(seed):
    """Tiny random packs with planted repeats: a sequence that repeats another's
    prefix exactly, one that differs in a single element of one head (q or k), one
    whose repeated part ends inside a block, and a sequence repeated whole. Catches:
    ignoring k, ignoring a head, off-by-one block coverage."""
    rng = np.random.default_rng(seed)
    B, Hs, d = 4, 2, 3
    lens = [13, 13, 11, 9, 16, 13]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q = rng.standard_normal((Hs, T, d)).astype(np.float32)
    k = rng.standard_normal((Hs, T, d)).astype(np.float32)
    def copy(dst, src, n):
        for x in (q, k):
            x[:, cu[dst]:cu[dst] + n] = x[:, cu[src]:cu[src] + n]
    copy(1, 0, 13)          # whole repeat of sequence 0
    copy(2, 0, 10)          # repeat ends inside block 2 (tokens 8..11)
    copy(3, 0, 9)
    k[1, cu[3] + 5, 2] += 1.0  # one element of one head's k differs inside block 1
    copy(4, 0, 12)
    copy(5, 4, 13)          # repeats sequence 4, whose first 12 tokens repeat 0
    got = orc.prefix_alias(q, k, cu, B).tolist()
    assert got == _bf_alias(q, k, cu, B)
    assert got != list(range(len(got)))  # something is shared


def test_row_subsets_match_the_full_computation():
    """compress(rows=...) and apply(rows=...), which the chunked-prefill and
    sampled checks use, return exactly the full computation's results on the
    requested (sequence, block-row) pairs, and nothing else."""
    wl = wlmod.small_variant(5, [200, 96, 33], Hs=2, Ht=3, Hkv=3)
    B = 32
    full = orc.compress(wl.q, wl.k, wl.cu_seqlens, B, 0.9, wl.bias())
    allrows = orc.block_rows(wl.cu_seqlens, B)
    pick = [allrows[i] for i in (0, 3, len(allrows) - 1, 7)]
    sub = orc.compress(wl.q, wl.k, wl.cu_seqlens, B, 0.9, wl.bias(), rows=pick)
    assert set(sub) == {(h, s, I) for h in range(2) for (s, I) in pick}
    for key, rr in sub.items():
        assert rr.kept == full[key].kept
        assert np.array_equal(rr.P, full[key].P) and np.array_equal(rr.kmass, full[key].kmass)
    out_full = orc.apply(full, wl.W, wl.v, wl.cu_seqlens, B, wl.spec.Hkv)
    out_sub = orc.apply(full, wl.W, wl.v, wl.cu_seqlens, B, wl.spec.Hkv, rows=pick)
    assert set(out_sub) == {(t, s, I) for t in range(3) for (s, I) in pick}
    for key, o in out_sub.items():
        assert np.array_equal(o, out_full[key])


def test_shared_block_rows_compress_identically():
    """The reason sharing is allowed: a full block-row with the same prefix as an
    earlier one has the same masses, kept set, probabilities and kept mass (the
    offsets are measured from each sequence start). Catches: a bias or causal mask
    that depends on absolute token positions."""
    wl = wlmod.small_variant(5, [300, 520, 130], Hs=2, Ht=2, Hkv=2)
    B = 32
    alias = orc.prefix_alias(wl.q, wl.k, wl.cu_seqlens, B)
    rows = orc.block_rows(wl.cu_seqlens, B)
    pairs = [(rows[g], rows[int(a)]) for g, a in enumerate(alias) if a != g]
    assert pairs
    res = orc.compress(wl.q, wl.k, wl.cu_seqlens, B, 0.9, wl.bias(),
                       rows=sorted({r for pr in pairs for r in pr}))
    for (s, I), (s2, I2) in pairs:
        for h in range(2):
            a, b = res[(h, s, I)], res[(h, s2, I2)]
            assert a.kept == b.kept
            assert np.array_equal(a.P, b.P) and np.array_equal(a.kmass, b.kmass)
