"""Plain, slow fp64 CPU oracle for block top-p attention-map compression and
translated retrieval.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline import this module. It shares no code with the HIP library: it takes
plain numpy arrays and does every step in float64 with numpy primitives, one
sequence, head and block-row at a time, in the order the method states.

What it computes, and where that is stated:

* Attention map.  A_h = softmax(Q_h K_h^T / sqrt(d) + bias) per head, causal
  (decoder-only models).  MapFlow, "Accelerating Cross-Model LLM Inference via
  Attention Map Reuse", §2.1 (scaled dot-product attention, the map holds
  token-to-token weights); the AttnCache guide ("AttnCache Guide: Reusing
  Attention Maps in LLM Prefill"), section "The Quadratic Self-Attention Cost",
  gives Softmax(Q K^T / sqrt(d_k)) V.  The logit offsets (a sink on the first
  key positions of each sequence, a local window) are the synthetic workloads'
  stand-ins for the head patterns in the AttnCache guide, section "1. The
  Attention Map Redundancy Discovery".
* Block top-p compression into BSR.  MapFlow §4 (top-p compression stores the
  maps in Block Sparse Row form) and §5.2 (block-level top-p sparsity, retained
  blocks stored in BSR).  Reading taken here: a block's mass is the sum of its
  probabilities; each query-block row keeps the shortest prefix of its causal
  blocks, sorted by mass (descending, lower key-block index first on ties),
  whose cumulative mass reaches p times the row's total; p == 1 keeps every
  causal block; kept blocks are stored in ascending key-block order with the
  raw (not renormalised) probabilities, and each token row records its kept
  mass.
* Translated retrieval.  MapFlow §3.3 (a receiver head is a linear mix of
  sender heads), §4 (linear head mapping) and §5.4 (the receiver attention is
  rebuilt from the sparse sender maps and the mapping weights, then applied to
  the receiver's values):  O_t = sum_h W[t, h] * renorm(A_hat_h) V_g(t), where
  renorm divides each kept row by its kept mass and g(t) = floor(t * Hkv / Ht)
  picks the V head of target t.  With W = I this is the AttnCache reuse path
  (cached map times V; AttnCache guide, PyTorch prototype).
* fp8 tiles (optional).  MapFlow §9 names quantised sparse maps as the way to
  shrink them further; `codec="mxfp8"` in apply reads every kept tile through
  the block-scaled E4M3 codec of oracle/mx_codec.py.
* Recompute-boundary profiling (MapFlow §3.3: the receiver layers to
  recompute are chosen offline from layer-wise total-variation distance between
  the translated map and the receiver's own map).  Reading taken here: per query
  row, TV_t[i] = 1/2 sum_j |A~_t[i,j] - A_t[i,j]|, where A~_t is the translated
  map exactly as retrieval uses it (sum_h W[t,h] renorm(A_hat_h), zero outside
  the kept blocks) and A_t the receiver's causal softmax map from its own q and
  k (K head g(t) as for V); a layer's score is the mean over rows.
* Dense attention for recomputed heads (MapFlow §4: the receiver computes its
  first r layers normally): O_h = A_h V_g(h).

Parity pins (tests/test_oracle_*.py) tie every function here to closed forms,
library routines, brute force and invariants.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from oracle import mx_codec

AMBIGUITY_REL = 1e-5  # relative band around the top-p cut treated as a tie


# ----------------------------------------------------------------------------
# Attention map (one sequence, one head)
# ----------------------------------------------------------------------------

def logits(q: np.ndarray, k: np.ndarray, rows: np.ndarray, ncols: int, bias: dict) -> np.ndarray:
    """s[i, j] = q_i . k_j / sqrt(d) + sink + local for j <= i; -inf above the diagonal.

    q, k: [L, d] of one sequence and head (any float dtype, used as float64).
    rows: positions i inside the sequence; columns are j = 0 .. ncols-1.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    d = q.shape[1]
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(ncols, dtype=np.int64)[None, :]
    s = (q[rows] @ k[:ncols].T) / np.sqrt(d)
    s = s + bias["sink_bias"] * (j < bias["sink_n"])
    diff = i - j
    s = s + bias["local_bias"] * ((diff >= 0) & (diff < bias["local_w"]))
    return np.where(j <= i, s, -np.inf)


def softmax_rows(s: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Row softmax with the max subtracted; returns (P, lse) with lse = log sum exp s."""
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    z = np.sum(e, axis=1, keepdims=True)
    lse = m + np.log(z)
    return np.exp(s - lse), lse[:, 0]


def attention_map(q: np.ndarray, k: np.ndarray, bias: dict) -> np.ndarray:
    """Dense causal map A [L, L] of one sequence and head (small L only)."""
    L = q.shape[0]
    P, _ = softmax_rows(logits(q, k, np.arange(L), L, bias))
    return P


# ----------------------------------------------------------------------------
# Block top-p selection
# ----------------------------------------------------------------------------

def block_masses(P: np.ndarray, B: int, nblocks: int) -> np.ndarray:
    """M[J] = sum over the given rows and the columns of key block J of P."""
    M = np.zeros(nblocks, dtype=np.float64)
    for J in range(nblocks):
        M[J] = np.sum(P[:, J * B:(J + 1) * B])
    return M


def sort_order(M: np.ndarray) -> np.ndarray:
    """Key blocks ordered by mass descending, lower block index first on equal mass."""
    idx = np.arange(len(M))
    return np.array(sorted(idx, key=lambda J: (-M[J], J)), dtype=np.int64)


@dataclasses.dataclass
class Selection:
    kept: List[int]          # ascending key-block indices
    order: np.ndarray        # sorted order used for the cut
    prefix: np.ndarray       # cumulative masses in that order
    kstar: int               # number kept
    total: float             # T_I = sum of the row's block masses
    target: float            # p * T_I
    keep_all: bool           # p == 1: every causal block kept without a cut


def topp_select(M: np.ndarray, p: float) -> Selection:
    """Shortest mass-sorted prefix whose cumulative mass reaches p * sum(M)."""
    n = len(M)
    total = float(np.sum(M))
    order = sort_order(M)
    prefix = np.cumsum(M[order])
    target = p * total
    if p >= 1.0:
        kstar = n
    else:
        kstar = n
        for r in range(n):
            if prefix[r] >= target:
                kstar = r + 1
                break
    kept = sorted(int(J) for J in order[:kstar])
    return Selection(kept, order, prefix, kstar, total, target, p >= 1.0)


def ambiguous_blocks(M: np.ndarray, sel: Selection, rel: float = AMBIGUITY_REL) -> set:
    """Blocks whose membership could flip under a relative perturbation `rel` of the
    masses near the cut:
      (a) order: a kept block whose mass is within rel of the largest dropped mass,
          or a dropped block within rel of the smallest kept mass (the two could
          swap places in the sorted order);
      (b) threshold: the last kept and the first dropped block when a prefix sum
          next to the cut lies within rel of p times the row total."""
    n = len(M)
    k = sel.kstar
    if n == 0 or sel.keep_all:
        return set()  # p == 1 keeps everything without comparing masses
    out = set()
    kept = set(sel.kept)
    m_last = M[sel.order[k - 1]]
    m_next = M[sel.order[k]] if k < n else None
    for J in range(n):
        if J in kept:
            if m_next is not None and M[J] - m_next <= rel * M[J]:
                out.add(J)
        elif m_last - M[J] <= rel * m_last:
            out.add(J)
    c_before = sel.prefix[k - 2] if k >= 2 else 0.0
    c_at = sel.prefix[k - 1]
    if abs(c_before - sel.target) <= rel * sel.target or abs(c_at - sel.target) <= rel * sel.target:
        out.add(int(sel.order[k - 1]))
        if k < n:
            out.add(int(sel.order[k]))
    return out


# ----------------------------------------------------------------------------
# Compression of one block-row
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class RowResult:
    rows: np.ndarray         # positions i of the block-row inside the sequence
    M: np.ndarray            # masses of key blocks 0..I
    sel: Selection
    P: np.ndarray            # probabilities [len(rows), min((I+1)B, L)]
    lse: np.ndarray          # natural-log normaliser per row
    kmass: np.ndarray        # kept mass per row (sum of P over kept blocks)
    ambiguous: set

    @property
    def kept(self) -> List[int]:
        return self.sel.kept

    def tile(self, J: int, B: int) -> np.ndarray:
        """Full B x B tile of key block J: zeros above the diagonal and outside the sequence."""
        t = np.zeros((B, B), dtype=np.float64)
        blk = self.P[:, J * B:(J + 1) * B]
        t[:blk.shape[0], :blk.shape[1]] = blk
        return t


def compress_row(q: np.ndarray, k: np.ndarray, I: int, B: int, p: float, bias: dict) -> RowResult:
    """Block-row I of one sequence and head: logits, softmax, block masses, top-p cut,
    kept mass per row."""
    L = q.shape[0]
    rows = np.arange(I * B, min((I + 1) * B, L))
    ncols = min((I + 1) * B, L)
    P, lse = softmax_rows(logits(q, k, rows, ncols, bias))
    M = block_masses(P, B, I + 1)
    sel = topp_select(M, p)
    kmass = np.zeros(len(rows), dtype=np.float64)
    for J in sel.kept:
        kmass += np.sum(P[:, J * B:(J + 1) * B], axis=1)
    return RowResult(rows, M, sel, P, lse, kmass, ambiguous_blocks(M, sel))


def nblocks(L: int, B: int) -> int:
    return (L + B - 1) // B


def seqs(cu: np.ndarray) -> List[Tuple[int, int]]:
    """(start, length) of every packed sequence."""
    return [(int(cu[s]), int(cu[s + 1] - cu[s])) for s in range(len(cu) - 1)]


def block_rows(cu: np.ndarray, B: int) -> List[Tuple[int, int]]:
    """Global block-row order: sequence-major, block-row ascending -> (s, I)."""
    out = []
    for s, (_, L) in enumerate(seqs(cu)):
        out += [(s, I) for I in range(nblocks(L, B))]
    return out


def prefix_alias(q: np.ndarray, k: np.ndarray, cu: np.ndarray, B: int) -> np.ndarray:
    """Shared block-rows (MapFlow §5.3: compressed blocks indexed by their prefix;
    §2.3: prefix caching).

    Block-row (s, I) is full when (I + 1) * B <= L_s.  Its compressed rows depend
    only on q and k of the sequence's tokens 0 .. (I + 1) * B - 1 (causal rows,
    offsets measured from the sequence start), so a full block-row whose prefix
    equals, bit for bit over every head, that of an earlier sequence s' whose
    block-row I is also full shares that block-row.  Returns, per global
    block-row, the global index of the first such (s', I), or its own index.

    Decided by direct comparison of the arrays (no hashing): for each pair of
    sequences, the length of their common prefix."""
    rows = block_rows(cu, B)
    first = {}
    g = 0
    for s, (_, L) in enumerate(seqs(cu)):
        first[s] = g
        g += nblocks(L, B)
    sq = seqs(cu)
    qb = q.view(np.uint32) if q.dtype == np.float32 else q
    kb = k.view(np.uint32) if k.dtype == np.float32 else k

    def common(s: int, s2: int) -> int:
        (a, L), (a2, L2) = sq[s], sq[s2]
        n = min(L, L2)
        if n == 0:
            return 0
        diff = (np.any(qb[:, a:a + n] != qb[:, a2:a2 + n], axis=(0, 2)) |
                np.any(kb[:, a:a + n] != kb[:, a2:a2 + n], axis=(0, 2)))
        idx = np.flatnonzero(diff)
        return int(idx[0]) if len(idx) else n

    alias = np.arange(len(rows), dtype=np.int32)
    memo = {}
    for gr, (s, I) in enumerate(rows):
        need = (I + 1) * B
        if need > sq[s][1]:
            continue
        for s2 in range(s):
            if need > sq[s2][1]:
                continue
            if (s, s2) not in memo:
                memo[(s, s2)] = common(s, s2)
            if memo[(s, s2)] >= need:
                alias[gr] = first[s2] + I
                break
    return alias


def compress(q: np.ndarray, k: np.ndarray, cu: np.ndarray, B: int, p: float, bias: dict,
             heads: Optional[Sequence[int]] = None,
             rows: Optional[Sequence[Tuple[int, int]]] = None) -> Dict[Tuple[int, int, int], RowResult]:
    """Compress the given (head, (seq, block-row)) pairs; all of them by default.

    q, k: [Hs][T][d] packed along T. Returns {(h, s, I): RowResult}."""
    heads = range(q.shape[0]) if heads is None else heads
    rows = block_rows(cu, B) if rows is None else rows
    out = {}
    sq = seqs(cu)
    for h in heads:
        for (s, I) in rows:
            a, L = sq[s]
            out[(h, s, I)] = compress_row(q[h, a:a + L], k[h, a:a + L], I, B, p, bias)
    return out


def bsr_layout(res: Dict[Tuple[int, int, int], RowResult], Hs: int, cu: np.ndarray,
               B: int) -> Tuple[np.ndarray, np.ndarray]:
    """row_ptr (exclusive prefix of kept counts over rows r = h * NBR + global block-row)
    and col_idx (ascending within a row), from a complete compress() result."""
    br = block_rows(cu, B)
    counts = [len(res[(h, s, I)].kept) for h in range(Hs) for (s, I) in br]
    row_ptr = np.zeros(len(counts) + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)
    cols = [J for h in range(Hs) for (s, I) in br for J in res[(h, s, I)].kept]
    return row_ptr, np.asarray(cols, dtype=np.int32)


# ----------------------------------------------------------------------------
# Translated retrieval
# ----------------------------------------------------------------------------

def v_head(t: int, Ht: int, Hkv: int) -> int:
    """V head read by target head t: contiguous groups of Ht / Hkv targets."""
    return (t * Hkv) // Ht


def apply_row(src_rows: Dict[int, RowResult], W: np.ndarray, t: int, v_seq: np.ndarray,
              B: int, renorm: bool = True, codec: Optional[str] = None) -> np.ndarray:
    """O_t for one block-row: sum_h W[t,h] * sum_{J kept by h} (P^h / kmass^h) V[J].

    src_rows: {h: RowResult of that source's block-row}; v_seq: [L, d] of V head g(t).
    codec "mxfp8": each kept B x B tile is first replaced by what the block-scaled
    E4M3 tile codec (oracle.mx_codec) reads back; the kept mass stays that of the
    unquantised probabilities."""
    if codec not in (None, "mxfp8"):
        raise ValueError(f"unknown tile codec {codec!r}")
    v = np.asarray(v_seq, dtype=np.float64)
    any_row = next(iter(src_rows.values()))
    out = np.zeros((len(any_row.rows), v.shape[1]), dtype=np.float64)
    for h, rr in src_rows.items():
        w = float(W[t, h])
        if w == 0.0:
            continue
        if renorm:
            with np.errstate(divide="ignore", invalid="ignore"):
                scale = np.where(rr.kmass > 0, w / rr.kmass, 0.0)
        else:
            scale = np.full(len(rr.rows), w)
        for J in rr.kept:
            blk = rr.P[:, J * B:(J + 1) * B]
            if codec == "mxfp8":
                blk = mx_codec.quantize(rr.tile(J, B))[:blk.shape[0], :blk.shape[1]]
            out += scale[:, None] * (blk @ v[J * B:J * B + blk.shape[1]])
    return out


def apply(res: Dict[Tuple[int, int, int], RowResult], W: np.ndarray, v: np.ndarray,
          cu: np.ndarray, B: int, Hkv: int, renorm: bool = True,
          targets: Optional[Sequence[int]] = None,
          rows: Optional[Sequence[Tuple[int, int]]] = None,
          codec: Optional[str] = None) -> Dict[Tuple[int, int, int], np.ndarray]:
    """Translated retrieval for the given (target, (seq, block-row)) pairs.

    res must hold every source with a nonzero weight for those rows. v: [Hkv][T][d].
    Returns {(t, s, I): O rows [len(rows), d]}."""
    Ht, Hs = W.shape
    targets = range(Ht) if targets is None else targets
    rows = block_rows(cu, B) if rows is None else rows
    sq = seqs(cu)
    out = {}
    for t in targets:
        g = v_head(t, Ht, Hkv)
        for (s, I) in rows:
            a, L = sq[s]
            src = {h: res[(h, s, I)] for h in range(Hs) if W[t, h] != 0.0}
            if not src:
                n = len(range(I * B, min((I + 1) * B, L)))
                out[(t, s, I)] = np.zeros((n, v.shape[2]))
                continue
            out[(t, s, I)] = apply_row(src, W, t, v[g, a:a + L], B, renorm, codec)
    return out


def translated_map_row(src_rows: Dict[int, RowResult], W: np.ndarray, t: int, B: int,
                       renorm: bool = True, codec: Optional[str] = None) -> np.ndarray:
    """A~_t for one block-row: sum_h W[t,h] * (P^h / kmass^h) on h's kept blocks, 0 elsewhere."""
    any_row = next(iter(src_rows.values()))
    out = np.zeros_like(any_row.P)
    for h, rr in src_rows.items():
        w = float(W[t, h])
        if w == 0.0:
            continue
        if renorm:
            with np.errstate(divide="ignore", invalid="ignore"):
                scale = np.where(rr.kmass > 0, w / rr.kmass, 0.0)
        else:
            scale = np.full(len(rr.rows), w)
        for J in rr.kept:
            blk = rr.P[:, J * B:(J + 1) * B]
            if codec == "mxfp8":
                blk = mx_codec.quantize(rr.tile(J, B))[:blk.shape[0], :blk.shape[1]]
            out[:, J * B:J * B + blk.shape[1]] += scale[:, None] * blk
    return out


def tv_distance(res: Dict[Tuple[int, int, int], RowResult], W: np.ndarray, q_r: np.ndarray,
                k_r: np.ndarray, cu: np.ndarray, B: int, bias: dict, renorm: bool = True,
                targets: Optional[Sequence[int]] = None,
                rows: Optional[Sequence[Tuple[int, int]]] = None,
                codec: Optional[str] = None) -> Dict[Tuple[int, int, int], np.ndarray]:
    """TV_t[i] = 1/2 sum_j |A~_t[i,j] - A_t[i,j]| for the given (target, (seq, block-row)).

    res must hold every source with a nonzero weight for those rows; q_r [Ht][T][d]
    and k_r [Hkr][T][d] are the receiver's; query head t reads K head g(t).
    Returns {(t, s, I): TV per row of the block-row}."""
    Ht, Hs = W.shape
    Hkr = k_r.shape[0]
    targets = range(Ht) if targets is None else targets
    rows = block_rows(cu, B) if rows is None else rows
    sq = seqs(cu)
    out = {}
    for t in targets:
        g = v_head(t, Ht, Hkr)
        for (s, I) in rows:
            a, L = sq[s]
            r = np.arange(I * B, min((I + 1) * B, L))
            ncols = min((I + 1) * B, L)
            A, _ = softmax_rows(logits(q_r[t, a:a + L], k_r[g, a:a + L], r, ncols, bias))
            src = {h: res[(h, s, I)] for h in range(Hs) if W[t, h] != 0.0}
            At = translated_map_row(src, W, t, B, renorm, codec) if src else np.zeros_like(A)
            out[(t, s, I)] = 0.5 * np.sum(np.abs(At - A), axis=1)
    return out


def assemble(rows_out: Dict[Tuple[int, int, int], np.ndarray], n_heads: int, cu: np.ndarray,
             B: int, d: int) -> np.ndarray:
    """Pack per-(head, seq, block-row) outputs into [H][T][d]."""
    O = np.zeros((n_heads, int(cu[-1]), d), dtype=np.float64)
    sq = seqs(cu)
    for (h, s, I), blk in rows_out.items():
        a = sq[s][0] + I * B
        O[h, a:a + blk.shape[0]] = blk
    return O


# ----------------------------------------------------------------------------
# Dense causal attention (recomputed heads)
# ----------------------------------------------------------------------------

def dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu: np.ndarray, bias: dict,
                    heads: Optional[Sequence[int]] = None,
                    row_ranges: Optional[Dict[int, Tuple[int, int]]] = None) -> Dict[Tuple[int, int], np.ndarray]:
    """O_h = softmax(Q_h K_g^T / sqrt(d) + bias) V_g, causal per sequence, g = v_head(h).

    q: [Hq][T][d]; k, v: [Hkv][T][d]. row_ranges optionally restricts rows per sequence
    to [r0, r1). Returns {(h, s): O rows}."""
    Hq, Hkv = q.shape[0], k.shape[0]
    heads = range(Hq) if heads is None else heads
    out = {}
    for h in heads:
        g = v_head(h, Hq, Hkv)
        for s, (a, L) in enumerate(seqs(cu)):
            r0, r1 = (0, L) if row_ranges is None or s not in row_ranges else row_ranges[s]
            rws = np.arange(r0, r1)
            ncols = r1 if r1 > 0 else 0
            if len(rws) == 0:
                out[(h, s)] = np.zeros((0, v.shape[2]))
                continue
            P, _ = softmax_rows(logits(q[h, a:a + L], k[g, a:a + L], rws, ncols, bias))
            out[(h, s)] = P @ np.asarray(v[g, a:a + ncols], dtype=np.float64)
    return out
