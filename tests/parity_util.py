"""Shared helpers of the GPU parity tests: move seeded inputs to the device, run
the HIP path through the binding, and compare against the fp64 oracle.

Comparison rules (floating point decides the kept sets, so they are compared up
to the cut band; everything else to fixed tolerances):
  kept sets   equal to the oracle's except blocks the oracle flags as
              cut-ambiguous (mass within 1e-5 relative of the cut); a row whose
              set differs there ("flip") is then graded on the GPU's own set:
              its kept mass against the fp64 sum over that set, its outputs
              against the oracle's retrieval step evaluated with the GPU's
              kept set and kept mass;
  tiles       |bf16 tile - P| <= 2e-3 on every block the GPU kept (bf16 rounding
              of a probability <= 1 is at most 2^-9 ~ 1.95e-3 with nearest-even);
  fp8 tiles   (block-scaled E4M3 maps) scale bytes and codes equal the oracle
              codec's applied to the fp64 probabilities, except where the fp64
              value sits within FP8_EPS (relative) of a decision boundary (a
              power of two for a block maximum, a rounding midpoint for a code):
              there the kernel's fp32 probability may fall on either side;
              decoded values within the codec's bound max(2^-4 p, 2^(e-10));
  kept mass   1e-4 relative where the sets agree (fp32 sums of fp32 exponentials);
  outputs     relative Frobenius error <= 1e-2 per (sequence, target head), over
              the rows compared (bf16 tiles and bf16 mixed tiles feeding fp32
              accumulation: per-element rounding 2^-9, averaged over a row); for
              fp8 maps against the oracle reading its own codec's tiles.
"""
from __future__ import annotations

import sys
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np
import torch

import oracle_pool
from oracle import mapflow_oracle as orc
from oracle import mx_codec as mx
from cross_model_sparse_amd import mapflow as mf

TILE_ATOL = 2e-3
FP8_EPS = 3e-5      # relative distance of an fp64 value to an fp8 decision boundary
KMASS_RTOL = 1e-4
OUT_RFROB = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev_qk(wl, dev):
    if wl.spec.qk_dtype == "bf16":
        q = torch.from_numpy(wl.q_bits.view(np.int16)).to(dev).view(torch.bfloat16)
        k = torch.from_numpy(wl.k_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        q = torch.from_numpy(np.ascontiguousarray(wl.q)).to(dev)
        k = torch.from_numpy(np.ascontiguousarray(wl.k)).to(dev)
    return q, k


def to_dev_v(wl, dev):
    return torch.from_numpy(wl.v_bits.view(np.int16)).to(dev).view(torch.bfloat16)


def gpu_compress(wl, dev, p=None, capacity=None, tile_format="bf16"):
    q, k = to_dev_qk(wl, dev)
    m = mf.mf_compress_topp(q, k, wl.cu_seqlens, wl.spec.B, wl.spec.p if p is None else p,
                            wl.bias(), capacity=capacity, tile_format=tile_format)
    st, nnz = mf.mf_read_status(m)
    return m, st, nnz


def tiles_to_rowmajor(t: np.ndarray) -> np.ndarray:
    """[n, B, B] tiles as stored (fragment order, see include/mapflow.h) -> row-major."""
    n, B = t.shape[0], t.shape[1]
    KC = B // 32
    flat = t.reshape(n, -1)
    i = np.arange(B)[:, None]
    j = np.arange(B)[None, :]
    off = (((i // 16) * KC + j // 32) * 64 + ((j % 32) // 8) * 16 + i % 16) * 8 + j % 8
    return flat[:, off]


def fp8_tiles_unpack(raw: np.ndarray, B: int) -> Tuple[np.ndarray, np.ndarray]:
    """[n, B*B + B*B/32] bytes as stored (layout in include/mapflow.h) ->
    (codes [n, B, B] row-major, scale bytes [n, B, B/32])."""
    n = raw.shape[0]
    NP = 2 if B >= 64 else 1
    i = np.arange(B)[:, None]
    j = np.arange(B)[None, :]
    off = ((((i // 16) * (B // (32 * NP)) + j // (32 * NP)) * 64 + ((j % 32) // 8) * 16 + i % 16) * 8 * NP
           + ((j % (32 * NP)) // 32) * 8 + j % 8)
    codes = raw[:, :B * B][:, off]
    scales = raw[:, B * B:].reshape(n, B, B // 32)
    return codes, scales


def check_fp8_tile(codes: np.ndarray, scales: np.ndarray, P: np.ndarray, key) -> int:
    """One fp8 tile against the oracle codec (module doc); returns the number of
    codes that differ from the codec's at a rounding midpoint."""
    B = P.shape[0]
    G = B // 32
    c_orc, s_orc = mx.encode_tile(P)
    amax = P.reshape(B, G, 32).max(axis=2)
    with np.errstate(divide="ignore"):
        near_pow2 = (amax > 0) & (np.abs(amax / np.exp2(np.round(np.log2(np.where(amax > 0, amax, 1.0)))) - 1.0)
                                  <= FP8_EPS)
    bad = (scales != s_orc) & ~near_pow2
    assert not bad.any(), f"tile {key}: scale bytes differ at {np.argwhere(bad)[:4].tolist()}"
    e = scales.astype(np.int64) - mx.SCALE_BIAS
    y = np.ldexp(P.reshape(B, G, 32), -e[:, :, None]).reshape(B, B)
    assert y.max() < 448.0, f"tile {key}: a value does not fit the kernel's scale"
    c_ref = mx.e4m3_codes(y)
    mism = codes != c_ref
    if mism.any():
        vg, vr = mx.E4M3_TABLE[codes[mism]], mx.E4M3_TABLE[c_ref[mism]]
        ym = y[mism]
        ok = np.abs(vg - ym) - np.abs(vr - ym) <= 2 * FP8_EPS * ym
        assert ok.all(), (f"tile {key}: codes {codes[mism][~ok][:4]} vs {c_ref[mism][~ok][:4]} "
                          f"for scaled values {ym[~ok][:4]}")
    dec = mx.decode_tile(codes, scales)
    lim = mx.error_bound(P) * (1 + 2 * FP8_EPS) + 2 * FP8_EPS * P + 1e-30
    assert np.all(np.abs(dec - P) <= lim), f"tile {key}: decoded value outside the codec bound"
    return int(mism.sum())


class HostMap:
    """CPU copy of the parts of a device map the checks need (selected rows only)."""

    def __init__(self, m: "mf.BsrMap", rows: Optional[Sequence[int]] = None):
        self.B = m.block
        self.fmt = m.tile_format
        self.NBR = m.num_block_rows
        self.row_ptr = m.row_ptr.cpu().numpy()
        nnz = int(self.row_ptr[-1])
        self.kept_mass = m.kept_mass.cpu().numpy()
        if rows is None:
            self.col_idx = m.col_idx[:nnz].cpu().numpy()
            self.tiles = self._host_tiles(m.tiles[:nnz])
            self.tile_base = 0
            self.rows = None
        else:
            # gather only the requested BSR rows
            idx = np.concatenate([np.arange(self.row_ptr[r], self.row_ptr[r + 1]) for r in rows])
            it = torch.from_numpy(idx).to(m.col_idx.device)
            self.sel_col = m.col_idx[it].cpu().numpy()
            self.sel_tiles = self._host_tiles(m.tiles[it])
            self.sel_pos = {}
            o = 0
            for r in rows:
                n = int(self.row_ptr[r + 1] - self.row_ptr[r])
                self.sel_pos[r] = (o, n)
                o += n
            self.rows = set(rows)

    def _host_tiles(self, t: torch.Tensor):
        """bf16: row-major float tiles; fp8: (codes, scale bytes) row-major."""
        if self.fmt == "bf16":
            return tiles_to_rowmajor(t.float().cpu().numpy())
        codes, scales = fp8_tiles_unpack(t.cpu().numpy(), self.B)
        return list(zip(codes, scales))

    def row(self, r: int) -> Tuple[np.ndarray, np.ndarray]:
        """(col_idx, tiles) of BSR row r."""
        if self.rows is None:
            a, b = self.row_ptr[r], self.row_ptr[r + 1]
            return self.col_idx[a:b], self.tiles[a:b]
        o, n = self.sel_pos[r]
        return self.sel_col[o:o + n], self.sel_tiles[o:o + n]


def global_row(cu, B, s, I) -> int:
    nb = [(int(cu[t + 1] - cu[t]) + B - 1) // B for t in range(len(cu) - 1)]
    return sum(nb[:s]) + I


def check_rows(hm: HostMap, res: Dict[Tuple[int, int, int], "orc.RowResult"], cu, T) -> dict:
    """Compare kept sets, tiles and kept mass of every oracle row in `res`."""
    B = hm.B
    stats = dict(rows=0, ambiguous_rows=0, tile_err=0.0, kmass_err=0.0, flips=[], fp8_mid=0,
                 fp8_codes=0, overrides={}, tiles=0)
    for (h, s, I), rr in res.items():
        gr = global_row(cu, B, s, I)
        r = h * hm.NBR + gr
        cols, tiles = hm.row(r)
        gset, oset = [int(c) for c in cols], rr.kept
        assert gset == sorted(gset), f"row {(h, s, I)} col_idx not ascending"
        diff = set(gset) ^ set(oset)
        assert diff <= rr.ambiguous, (f"row {(h, s, I)}: kept {gset} vs oracle {oset}, "
                                      f"ambiguous {sorted(rr.ambiguous)}")
        if diff:
            stats["ambiguous_rows"] += 1
            stats["flips"].append((h, s, I))
        for c, J in enumerate(gset):
            assert 0 <= J <= I, f"row {(h, s, I)} keeps block {J} past its diagonal"
            if True:  # P covers every block J <= I, kept by the oracle or not
                if hm.fmt == "bf16":
                    e = float(np.max(np.abs(tiles[c] - rr.tile(J, B))))
                    stats["tile_err"] = max(stats["tile_err"], e)
                    assert e <= TILE_ATOL, f"tile {(h, s, I, J)} max error {e}"
                else:
                    codes, scales = tiles[c]
                    P = rr.tile(J, B)
                    stats["fp8_mid"] += check_fp8_tile(codes, scales, P, (h, s, I, J))
                    stats["fp8_codes"] += codes.size
                    e = float(np.max(np.abs(mx.decode_tile(codes, scales) - P)))
                    stats["tile_err"] = max(stats["tile_err"], e)
        a = int(cu[s]) + I * B
        km = hm.kept_mass[h, a:a + len(rr.rows)]
        if diff:
            # graded on the GPU's own set: the fp64 kept mass of that set
            ref = np.zeros(len(rr.rows))
            for J in gset:
                ref += rr.P[:, J * B:(J + 1) * B].sum(axis=1)
            stats["overrides"][(h, s, I)] = (gset, km.astype(np.float64))
        else:
            ref = rr.kmass
        e = float(np.max(np.abs(km - ref) / ref))
        stats["kmass_err"] = max(stats["kmass_err"], e)
        assert e <= KMASS_RTOL, f"kept mass {(h, s, I)} rel error {e}"
        stats["rows"] += 1
        stats["tiles"] += len(gset)
    return stats


def regrade(res: Dict[Tuple[int, int, int], "orc.RowResult"], overrides) -> Dict:
    """Oracle rows with the GPU's kept set and kept mass on flipped rows."""
    out = dict(res)
    for key, (kept, km) in overrides.items():
        out[key] = oracle_pool.regraded(res[key], kept, km)
    return out


def map_invariants(m: "mf.BsrMap", cu, p: float, nnz: int) -> dict:
    """Whole-map checks on the device map (every head and block-row):
    row_ptr starts at 0, is non-decreasing and ends at nnz; col_idx is strictly
    ascending inside each row and never past the row's diagonal block; per
    block-row the kept mass sums to at least p * rows (1 - 1e-6); and (bf16
    tiles) every row's tile sums over its kept blocks equal its kept mass within
    bf16 rounding (at most 2^-8 relative per value, all values >= 0)."""
    dev = m.row_ptr.device
    B, NBR, Hs = m.block, m.num_block_rows, m.num_heads
    rp = m.row_ptr
    assert int(rp[0]) == 0 and int(rp[-1]) == nnz
    cnt = rp[1:] - rp[:-1]
    assert bool((cnt >= 0).all()), "row_ptr decreases"
    cuh = np.asarray(cu, dtype=np.int64)
    # block-row table: global token start, valid rows, diagonal block index
    starts, lens, diag = [], [], []
    for s in range(len(cuh) - 1):
        L = int(cuh[s + 1] - cuh[s])
        for I in range((L + B - 1) // B):
            starts.append(int(cuh[s]) + I * B)
            lens.append(min(B, L - I * B))
            diag.append(I)
    assert len(starts) == NBR
    starts_d = torch.tensor(starts, device=dev, dtype=torch.int64)
    lens_d = torch.tensor(lens, device=dev, dtype=torch.int64)
    diag_d = torch.tensor(diag, device=dev, dtype=torch.int64)
    row_of = torch.repeat_interleave(torch.arange(Hs * NBR, device=dev), cnt)   # BSR row per tile
    col = m.col_idx[:nnz].to(torch.int64)
    assert bool((col >= 0).all()) and bool((col <= diag_d[row_of % NBR]).all()), "col_idx past the diagonal"
    same = row_of[1:] == row_of[:-1]
    assert bool((col[1:][same] > col[:-1][same]).all()), "col_idx not strictly ascending in a row"
    # kept mass per block-row
    km = m.kept_mass.to(torch.float64)                       # [Hs, T]
    T = km.shape[1]
    csum = torch.zeros((Hs, T + 1), dtype=torch.float64, device=dev)
    csum[:, 1:] = torch.cumsum(km, dim=1)
    blk = csum[:, starts_d + lens_d] - csum[:, starts_d]     # [Hs, NBR]
    need = p * lens_d.to(torch.float64) * (1 - 1e-6)
    short = blk < need[None, :]
    assert not bool(short.any()), f"{int(short.sum())} block-rows keep less than p of their mass"
    out = dict(tile_rows=0, max_rowsum_err=0.0)
    if m.tile_format == "bf16" and nnz > 0:
        i = np.arange(B)[:, None]
        j = np.arange(B)[None, :]
        KC = B // 32
        perm = torch.from_numpy((((i // 16) * KC + j // 32) * 64 + ((j % 32) // 8) * 16 + i % 16) * 8
                                + j % 8).reshape(-1).to(dev)
        rows_sum = torch.zeros(Hs * T + B, dtype=torch.float64, device=dev)
        step = 8192
        for c0 in range(0, nnz, step):
            c1 = min(nnz, c0 + step)
            t = m.tiles[c0:c1].reshape(c1 - c0, B * B)[:, perm].reshape(c1 - c0, B, B)
            rs = t.to(torch.float64).sum(dim=2)              # [n, B] row sums
            r = row_of[c0:c1]
            base = (r // NBR) * T + starts_d[r % NBR]        # flat index of the tile's first row
            idx = (base[:, None] + torch.arange(B, device=dev)[None, :]).reshape(-1)
            valid = (torch.arange(B, device=dev)[None, :] < lens_d[r % NBR][:, None]).reshape(-1)
            rows_sum.index_add_(0, idx[valid], rs.reshape(-1)[valid])
        rs = rows_sum[:Hs * T].reshape(Hs, T)
        err = (rs - km).abs()
        # nearest-even bf16 is off by at most half an ulp, 2^-8 of the value at the
        # bottom of a binade; all values are >= 0, so a row sum is off by at most
        # 2^-8 of the kept mass
        lim = 2.0 ** -8 * km * (1 + 1e-3) + 1e-6
        bad = err > lim
        assert not bool(bad.any()), (f"{int(bad.sum())} rows: tile sums differ from kept mass, worst "
                                     f"{float(err.max())}")
        out["tile_rows"] = int(Hs * T)
        out["max_rowsum_err"] = float((err / km.clamp_min(1e-30)).max())
    return out


def rel_frob(a: np.ndarray, b: np.ndarray) -> float:
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def check_apply(O_gpu: np.ndarray, out: Dict[Tuple[int, int, int], np.ndarray], cu, B) -> float:
    """Relative Frobenius error per (sequence, target) over the compared block-rows.
    O_gpu: [Ht][T][d] host array, or {t: [T][d]}.  Rows that flipped at an
    ambiguous cut are in `out` as the oracle evaluated them on the GPU's kept
    set (see regrade), so every block-row of `out` is compared."""
    per = {}
    for (t, s, I), blk in out.items():
        a = int(cu[s]) + I * B
        g = O_gpu[t][a:a + blk.shape[0]]
        per.setdefault((t, s), []).append((g, blk))
    worst = 0.0
    for key, pairs in per.items():
        g = np.concatenate([x for x, _ in pairs])
        o = np.concatenate([y for _, y in pairs])
        e = rel_frob(g, o)
        worst = max(worst, e)
        assert e <= OUT_RFROB, f"output {key}: relative Frobenius error {e}"
    return worst
