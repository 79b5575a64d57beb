"""Pure-Python brute force for tiny inputs (no numpy in the arithmetic).

TEST INFRASTRUCTURE: only the tests import this. It recomputes the attention
map, the block masses, the top-p kept sets and the translated retrieval with
math.fsum (correctly rounded sums) and, for the selection, an exhaustive search
over subsets instead of sorting. It serves as an independent pin of the fp64
oracle in oracle/mapflow_oracle.py on inputs small enough to enumerate.

Definitions followed: MapFlow ("Accelerating Cross-Model LLM Inference via
Attention Map Reuse") §4 and §5.2 for block top-p retention in BSR form, §3.3
and §5.4 for the linear head mix applied to the receiver's values; the
AttnCache guide ("AttnCache Guide: Reusing Attention Maps in LLM Prefill"),
section "The Quadratic Self-Attention Cost", for the softmax attention map;
MapFlow §3.3 for the total-variation distance used to pick recomputed layers.
The subset rule (smallest subset reaching p of the row mass, largest mass
among those, lowest indices among equal masses) is the reading of "top-p
blocks" taken in the oracle's header.
"""
from __future__ import annotations

import itertools
import math
from typing import Dict, List, Sequence, Tuple


def bf_map(q: Sequence[Sequence[float]], k: Sequence[Sequence[float]], bias: dict) -> List[List[float]]:
    """Dense causal probabilities of one sequence and head, element by element."""
    L = len(q)
    d = len(q[0])
    rt = math.sqrt(d)
    out = []
    for i in range(L):
        s = []
        for j in range(i + 1):
            x = math.fsum(float(q[i][c]) * float(k[j][c]) for c in range(d)) / rt
            if j < bias["sink_n"]:
                x += bias["sink_bias"]
            if 0 <= i - j < bias["local_w"]:
                x += bias["local_bias"]
            s.append(x)
        m = max(s)
        z = math.fsum(math.exp(x - m) for x in s)
        row = [math.exp(x - m) / z for x in s] + [0.0] * (L - i - 1)
        out.append(row)
    return out


def bf_masses(A: List[List[float]], B: int, I: int) -> List[float]:
    L = len(A)
    rows = range(I * B, min((I + 1) * B, L))
    return [math.fsum(A[i][j] for i in rows for j in range(J * B, min((J + 1) * B, L)))
            for J in range(I + 1)]


def bf_select(M: List[float], p: float) -> List[int]:
    """Exhaustive search: among subsets reaching p * sum(M), the smallest ones; among
    those the largest mass; among equal masses the lexicographically smallest."""
    n = len(M)
    if p >= 1.0:
        return list(range(n))
    target = p * math.fsum(M)
    for size in range(1, n + 1):
        best = None
        best_mass = -1.0
        for sub in itertools.combinations(range(n), size):
            m = math.fsum(M[J] for J in sub)
            if m >= target and (m > best_mass or (m == best_mass and sub < best)):
                best, best_mass = sub, m
        if best is not None:
            return list(best)
    return list(range(n))


def bf_compress(q, k, B: int, p: float, bias: dict) -> Dict[int, dict]:
    """{I: {"M", "kept", "kmass", "A"}} for one sequence and head."""
    A = bf_map(q, k, bias)
    L = len(A)
    nb = (L + B - 1) // B
    out = {}
    for I in range(nb):
        M = bf_masses(A, B, I)
        kept = bf_select(M, p)
        rows = range(I * B, min((I + 1) * B, L))
        kmass = [math.fsum(A[i][j] for J in kept for j in range(J * B, min((J + 1) * B, L)))
                 for i in rows]
        out[I] = {"M": M, "kept": kept, "kmass": kmass, "A": A}
    return out


def bf_apply(per_src: Dict[int, Dict[int, dict]], W: Sequence[Sequence[float]], t: int,
             v: Sequence[Sequence[float]], B: int, renorm: bool = True) -> List[List[float]]:
    """O_t [L][d] = sum_h W[t][h] sum_{J kept} (A_h[i][j] / kmass) v[j], elementwise fsum."""
    L = len(v)
    d = len(v[0])
    out = [[0.0] * d for _ in range(L)]
    for i in range(L):
        I = i // B
        terms = [[] for _ in range(d)]
        for h, rows in per_src.items():
            w = float(W[t][h])
            if w == 0.0:
                continue
            r = rows[I]
            km = r["kmass"][i - I * B]
            scale = (w / km if km > 0 else 0.0) if renorm else w
            for J in r["kept"]:
                for j in range(J * B, min((J + 1) * B, L)):
                    a = r["A"][i][j]
                    for c in range(d):
                        terms[c].append(scale * a * float(v[j][c]))
        out[i] = [math.fsum(x) for x in terms]
    return out


def bf_tv(per_src: Dict[int, Dict[int, dict]], W: Sequence[Sequence[float]], t: int,
          A_r: List[List[float]], B: int, renorm: bool = True) -> List[float]:
    """TV_t[i] = 1/2 sum_j |A~_t[i][j] - A_r[i][j]|, A~ built element by element."""
    L = len(A_r)
    out = []
    for i in range(L):
        I = i // B
        mix = [[] for _ in range(L)]
        for h, rows in per_src.items():
            w = float(W[t][h])
            if w == 0.0:
                continue
            r = rows[I]
            km = r["kmass"][i - I * B]
            scale = (w / km if km > 0 else 0.0) if renorm else w
            for J in r["kept"]:
                for j in range(J * B, min((J + 1) * B, L)):
                    mix[j].append(scale * r["A"][i][j])
        out.append(0.5 * math.fsum(abs(math.fsum(mix[j]) - A_r[i][j]) for j in range(L)))
    return out
