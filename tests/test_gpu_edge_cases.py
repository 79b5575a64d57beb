"""GPU pins of the cases the method defines exactly (MapFlow page, §5.2 block-level
top-p and §3.3 translated retrieval), through the C ABI against the fp64 oracle:

  exact ties      q = 0 and no bias make every logit 0, so all key blocks below
                  the diagonal carry bit-identical masses on both sides; the
                  kept set must be exactly the lowest block indices (ties go to
                  the lower key-block index), with no cut-band allowance;
  a real flip     two key blocks whose masses differ by ~1e-9 relative (below
                  fp32 resolution, so the GPU sees a tie and keeps the lower
                  index, while fp64 ranks the higher one first): the row's kept
                  set differs from the oracle's, and the row is graded on the
                  GPU's own kept set and kept mass;
  kept mass 0     rows whose kept mass is 0 contribute nothing: every source at
                  0 gives an exactly zero output row; one source at 0 drops that
                  source's term.
"""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import mapflow_oracle as orc
from cross_model_sparse_amd import mapflow as mf
from cross_model_sparse_amd import workloads as wlmod
from parity_util import (HostMap, check_apply, check_rows, gpu_compress, global_row, regrade,
                         rel_frob, say, to_dev_v)

pytestmark = pytest.mark.gpu


def with_qk(wl, q: np.ndarray, k: np.ndarray):
    """The workload with q, k replaced (values exactly representable in its dtype)."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    if wl.spec.qk_dtype == "bf16":
        qb, kb = wlmod.f32_to_bf16_bits(q), wlmod.f32_to_bf16_bits(k)
        assert np.array_equal(q.view(np.uint32) >> 16, qb) and np.array_equal(k.view(np.uint32) >> 16, kb)
        return dataclasses.replace(wl, q=q, k=k, q_bits=qb, k_bits=kb)
    return dataclasses.replace(wl, q=q, k=k)


def no_bias_spec(name, lens, Hs, Ht, Hkv, d, B, p, dt, seed):
    return wlmod.Spec(name, tuple(lens), Hs, Ht, Hkv, d, B, p, dt, 0, "gauss", w_var=1.0, sink_n=0,
                      sink_bias=0.0, local_bias=0.0, seed=seed)


@pytest.mark.parametrize("B,dt,p", [(64, "bf16", 0.5), (128, "bf16", 0.37), (32, "fp32", 0.45)])
def test_exact_ties_keep_lowest_blocks(gpu, B, dt, p):
    spec = no_bias_spec(f"ties B={B}", [8 * B + 5], 2, 2, 2, 64, B, p, dt, 300 + B)
    wl = wlmod.make_workload(spec)
    wl = with_qk(wl, np.zeros_like(wl.q), wl.k)
    m, st, nnz = gpu_compress(wl, gpu)
    assert st == mf.MF_OK
    res = orc.compress(wl.q, wl.k, wl.cu_seqlens, B, p, wl.bias())
    hm = HostMap(m)
    n_tied = 0
    for (h, s, I), rr in res.items():
        cols = [int(c) for c in hm.row(h * hm.NBR + global_row(wl.cu_seqlens, B, s, I))[0]]
        below = rr.M[:I]
        if I >= 2:
            # the oracle's masses of the blocks below the diagonal are bit-identical
            assert np.all(below == below[0])
        kept = sorted(rr.kept)
        assert cols == kept, f"row {(h, s, I)}: GPU kept {cols}, ties must keep {kept}"
        tied_kept = [J for J in kept if J < I]
        assert tied_kept == list(range(len(tied_kept))), f"row {(h, s, I)} kept {kept}"
        if 0 < len(tied_kept) < I:
            n_tied += 1
    say(f"ties B={B} {dt} p={p}: {len(res)} rows, {n_tied} cut inside a run of tied blocks")
    assert n_tied >= 4


def test_near_tie_really_flips_and_is_graded_on_gpu_set(gpu):
    """Blocks 0 and 1 of block-rows 2 and 3 hold almost all the mass, equally in
    fp32; fp64 puts block 1 ahead by ~9e-10 relative.  p = 0.3 keeps one block:
    the oracle keeps {1}, the GPU (ties to the lower index) {0}."""
    B, d, L = 64, 64, 4 * 64
    spec = no_bias_spec("near tie", [L], 1, 1, 1, d, B, 0.3, "bf16", 321)
    wl = wlmod.make_workload(spec)
    q = np.zeros((1, L, d), np.float32)
    k = np.zeros((1, L, d), np.float32)
    q[0, :, 0] = 4.0
    q[0, :, 1] = 2.0 ** -20
    k[0, :2 * B, 0] = 16.0          # logit 8 for keys of blocks 0 and 1
    k[0, :B, 1] = 1.0
    k[0, B:2 * B, 1] = 1.0 + 2.0 ** -7   # one bf16 step more: +2^-30 in the fp64 logit
    wl = dataclasses.replace(with_qk(wl, q, k), W=np.ones((1, 1), np.float32))
    m, st, nnz = gpu_compress(wl, gpu)
    assert st == mf.MF_OK
    res = orc.compress(wl.q, wl.k, wl.cu_seqlens, B, 0.3, wl.bias())
    for I in (2, 3):
        rr = res[(0, 0, I)]
        assert rr.kept == [1] and {0, 1} <= rr.ambiguous and 0 < rr.M[1] / rr.M[0] - 1 < 1e-8
    hm = HostMap(m)
    stats = check_rows(hm, res, wl.cu_seqlens, wl.T)
    for I in (2, 3):
        assert [int(c) for c in hm.row(I)[0]] == [0], "the GPU keeps the lower of two tied blocks"
    assert stats["ambiguous_rows"] == 2 and set(stats["overrides"]) == {(0, 0, 2), (0, 0, 3)}
    O = mf.mf_apply_translated(m, torch.from_numpy(wl.W).to(gpu), to_dev_v(wl, gpu), wl.cu_seqlens)
    out = orc.apply(regrade(res, stats["overrides"]), wl.W, wl.v, wl.cu_seqlens, B, 1)
    err = check_apply(O.cpu().numpy(), out, wl.cu_seqlens, B)
    # the regraded rows read V of block 0, the oracle's own set V of block 1
    own = orc.apply(res, wl.W, wl.v, wl.cu_seqlens, B, 1)
    rows3 = slice(3 * B, 4 * B)
    assert np.abs(O.cpu().numpy()[0, rows3] - own[(0, 0, 3)]).max() > 0.1
    say(f"near tie: flips={stats['ambiguous_rows']} graded on the GPU's sets, out_err={err:.2e}")


@pytest.mark.parametrize("idx,kw,W_kind,fmt", [
    (4, dict(Hs=8, Ht=8, Hkv=8), "four", "bf16"),      # pair kernel
    (2, dict(Hs=6, Ht=4, Hkv=2), "dense", "bf16"),     # dense mixing
    (4, dict(Hs=8, Ht=8, Hkv=4), "four", "mxfp8"),     # fp8 tiles
])
def test_zero_kept_mass_rows(gpu, idx, kw, W_kind, fmt):
    wl = wlmod.small_variant(idx, [700, 300], **kw)
    B, Hs = wl.spec.B, wl.spec.Hs
    m, st, nnz = gpu_compress(wl, gpu, tile_format=fmt)
    assert st == mf.MF_OK
    res = orc.compress(wl.q, wl.k, wl.cu_seqlens, B, wl.spec.p, wl.bias())
    stats = check_rows(HostMap(m), res, wl.cu_seqlens, wl.T)
    rng = np.random.default_rng(9)
    T = wl.T
    all_zero = np.sort(rng.choice(T, 40, replace=False))            # every source at 0
    one_zero = np.setdiff1d(np.sort(rng.choice(T, 60, replace=False)), all_zero)
    h1 = 1
    km = m.kept_mass.clone()
    km[:, torch.from_numpy(all_zero).to(gpu)] = 0.0
    km[h1, torch.from_numpy(one_zero).to(gpu)] = 0.0
    m.kept_mass.copy_(km)
    O = mf.mf_apply_translated(m, torch.from_numpy(wl.W).to(gpu), to_dev_v(wl, gpu),
                               wl.cu_seqlens).cpu().numpy()
    assert np.all(O[:, all_zero] == 0.0), "a row with kept mass 0 everywhere must give a zero output row"
    # oracle with the same kept masses set to 0
    kmh = km.cpu().numpy()
    ov = dict(stats["overrides"])
    for (h, s, I), rr in res.items():
        a = int(wl.cu_seqlens[s]) + I * B
        kept = ov[(h, s, I)][0] if (h, s, I) in ov else rr.kept
        base = ov[(h, s, I)][1] if (h, s, I) in ov else rr.kmass
        ov[(h, s, I)] = (kept, np.where(kmh[h, a:a + len(rr.rows)] == 0.0, 0.0, base))
    out = orc.apply(regrade(res, ov), wl.W, wl.v, wl.cu_seqlens, B, wl.spec.Hkv,
                    codec="mxfp8" if fmt == "mxfp8" else None)
    err = check_apply(O, out, wl.cu_seqlens, B)
    say(f"kept mass 0: {len(all_zero)} rows all sources, {len(one_zero)} rows source {h1}; "
        f"{W_kind} W {fmt}: out_err={err:.2e}")


def _bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest-even bf16 value, as float64."""
    b = wlmod.f32_to_bf16_bits(np.asarray(x, dtype=np.float32)).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def _retrieval_model(res, W, v, cu, B, Hkv, codec=None, coef_bf16=False):
    """The oracle's retrieval step on the tile values the map stores (bf16 of the
    probabilities, or the fp8 codec's values) with fp64 coefficients
    W[t,h] / kmass_h[i], or (coef_bf16) with each coefficient formed in fp32 and
    rounded to bf16.  A model used only to size roundings, not a reference."""
    from oracle import mx_codec
    Ht = W.shape[0]
    out = {}
    for t in range(Ht):
        g = orc.v_head(t, Ht, Hkv)
        for (h, s, I), rr in res.items():
            if W[t, h] == 0.0:
                continue
            a, L = orc.seqs(cu)[s]
            vs = np.asarray(v[g, a:a + L], dtype=np.float64)
            if coef_bf16:
                inv = np.where(rr.kmass > 0, np.float32(1.0) / rr.kmass.astype(np.float32), np.float32(0.0))
                c = _bf16_round(np.float32(W[t, h]) * inv.astype(np.float32))
            else:
                km = np.asarray(rr.kmass, dtype=np.float64)
                c = float(W[t, h]) * np.where(km > 0, 1.0 / np.where(km > 0, km, 1.0), 0.0)
            acc = out.setdefault((t, s, I), np.zeros((len(rr.rows), vs.shape[1])))
            for J in rr.kept:
                blk = rr.P[:, J * B:(J + 1) * B]
                if codec == "mxfp8":
                    blk = mx_codec.quantize(rr.tile(J, B))[:blk.shape[0], :blk.shape[1]]
                else:
                    blk = _bf16_round(blk.astype(np.float32))
                acc += c[:, None] * (blk @ vs[J * B:J * B + blk.shape[1]])
    return out


def _worst_rel_frob(O, out, cu, B):
    """Largest relative Frobenius distance per (sequence, target) between a full
    [Ht][T][d] array and block-row results (no tolerance applied)."""
    per = {}
    for (t, s, I), blk in out.items():
        a = int(cu[s]) + I * B
        per.setdefault((t, s), []).append((O[t][a:a + blk.shape[0]], blk))
    worst = 0.0
    for pairs in per.values():
        g = np.concatenate([x for x, _ in pairs])
        o = np.concatenate([y for _, y in pairs])
        worst = max(worst, rel_frob(g, o))
    return worst


@pytest.mark.parametrize("idx,lens,kw,fmt", [
    (2, [900, 130], dict(Hs=12, Ht=8, Hkv=8), "bf16"),
    (3, [1000], dict(Hs=12, Ht=16, Hkv=4), "bf16"),
    (5, [600, 640, 65], dict(Hs=16, Ht=16, Hkv=16), "bf16"),
    (5, [600, 640, 65], dict(Hs=16, Ht=16, Hkv=16), "mxfp8"),
    (5, [300, 520, 64, 1, 129, 0, 700], dict(Hs=8, Ht=8, Hkv=8), "bf16"),
])
def test_dense_mixing_exact_coefficients(gpu, idx, lens, kw, fmt):
    """Dense mixing (more than four sources per target, mixed-sign Gaussian W,
    where the mixed value can be much smaller than its terms) keeps each
    coefficient W[t,h] / kmass_h[i] in fp32.  Against the retrieval on the stored
    tile values with exact coefficients, the GPU differs by the translated tile's
    own rounding to bf16 (2^-9 per element, which the sum over keys can grow
    where its mixed-sign terms cancel; 1.8e-3 to 3.3e-3 on these cases, held
    under 2^-8), and it must be closer to that retrieval than a bf16 rounding of
    the coefficients alone would put it."""
    wl = wlmod.small_variant(idx, lens, **kw)
    B = wl.spec.B
    assert (np.count_nonzero(wl.W, axis=1) > 4).all()
    m, st, nnz = gpu_compress(wl, gpu, tile_format=fmt)
    assert st == mf.MF_OK
    res = orc.compress(wl.q, wl.k, wl.cu_seqlens, B, wl.spec.p, wl.bias())
    stats = check_rows(HostMap(m), res, wl.cu_seqlens, wl.T)
    res = regrade(res, stats["overrides"])
    codec = "mxfp8" if fmt == "mxfp8" else None
    O = mf.mf_apply_translated(m, torch.from_numpy(wl.W).to(gpu), to_dev_v(wl, gpu),
                               wl.cu_seqlens).cpu().numpy()
    exact = orc.apply(res, wl.W, wl.v, wl.cu_seqlens, B, wl.spec.Hkv, codec=codec)
    tiles = _retrieval_model(res, wl.W, wl.v, wl.cu_seqlens, B, wl.spec.Hkv, codec)
    rounded = _retrieval_model(res, wl.W, wl.v, wl.cu_seqlens, B, wl.spec.Hkv, codec, coef_bf16=True)
    Or = np.zeros_like(O)
    for (t, s, I), blk in rounded.items():
        a = int(wl.cu_seqlens[s]) + I * B
        Or[t, a:a + blk.shape[0]] = blk
    e_gpu = check_apply(O, exact, wl.cu_seqlens, B)
    e_tiles = _worst_rel_frob(O, tiles, wl.cu_seqlens, B)
    e_coef = _worst_rel_frob(Or, tiles, wl.cu_seqlens, B)
    say(f"dense mixing {wl.spec.name[:20]} {fmt}: GPU vs exact {e_gpu:.2e}; GPU vs stored-tile "
        f"retrieval {e_tiles:.2e}; bf16 coefficients alone would put {e_coef:.2e}")
    assert e_tiles <= 2.0 ** -8
    assert e_tiles < e_coef
