"""Seeded synthetic inputs for attention-map compression and translated retrieval.

This module only draws numbers; it holds none of the method's arithmetic. Both
the fp64 oracle (through the tests and the benchmark) and the HIP library are
fed from here.

The five workloads stand in for the long-context, multi-turn and heterogeneous
model-pair settings of MapFlow ("Accelerating Cross-Model LLM Inference via
Attention Map Reuse", §7.3 long context, §7.4 multi-turn conversation, §3.2 /
§4 heterogeneous head counts), whose real models and datasets are not used.
The sink and local-window logit offsets imitate the head patterns listed in
the AttnCache guide ("AttnCache Guide: Reusing Attention Maps in LLM Prefill",
section "1. The Attention Map Redundancy Discovery": attention sinks on the
first tokens and local sliding windows).

Recipe (fixed, seed = workload index unless overridden):
  rng = numpy.random.default_rng(seed)
  draw order: sequence lengths (multi-turn only), Q [Hs][T][d], K [Hs][T][d],
  V [Hkv][T][d], then W [Ht][Hs];
  Q, K, V are float32 N(0, 1); for bf16 workloads they are rounded to bf16
  with round-to-nearest-even and the rounded values are what both sides see;
  W is float32: N(0, var) dense, or per target row 4 distinct sources drawn
  without replacement with Dirichlet(1, 1, 1, 1) weights.
  Multi-turn: 16 lengths uniform on [1024, 8192]; sequence s > 0 copies the
  first min(L_s // 2, L_0) rows of Q, K and V (every head) from sequence 0.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Spec:
    """Shape and distribution of one synthetic workload."""
    name: str
    lens: Optional[tuple]       # fixed sequence lengths, or None for the multi-turn draw
    Hs: int                     # source (sender) heads: Q and K heads of the map
    Ht: int                     # target (receiver) heads
    Hkv: int                    # receiver V heads (Ht % Hkv == 0)
    d: int                      # head dimension
    B: int                      # block size of the BSR map
    p: float                    # top-p threshold
    qk_dtype: str               # "fp32" or "bf16"
    local_w: int                # local window: bias where 0 <= i - j < local_w
    w_kind: str                 # "gauss" or "dirichlet4"
    w_var: float = 0.0          # variance of the Gaussian W
    sink_n: int = 4             # sink: bias on key positions [0, sink_n) of each sequence
    sink_bias: float = 4.0
    local_bias: float = 2.0
    nseq_multi: int = 0         # multi-turn: number of sequences
    len_lo: int = 0
    len_hi: int = 0
    seed: int = 0


SPECS = {
    1: Spec("tiny L=256 Hs=2 Ht=2 d=64 B=32 p=0.9 fp32", (256,), 2, 2, 2, 64, 32, 0.9,
            "fp32", 64, "gauss", w_var=0.5, seed=1),
    2: Spec("L=4096 Hs=32 Ht=32 d=128 B=64 p=0.95 bf16", (4096,), 32, 32, 32, 128, 64, 0.95,
            "bf16", 256, "gauss", w_var=1.0 / 32, seed=2),
    3: Spec("heterogeneous L=16384 Hs=24 Ht=32 Hkv=8 d=128 B=64 p=0.9 bf16", (16384,), 24, 32, 8,
            128, 64, 0.9, "bf16", 256, "gauss", w_var=1.0 / 24, seed=3),
    4: Spec("long context L=32768 Hs=32 Ht=64 d=128 B=128 p=0.95 bf16", (32768,), 32, 64, 64,
            128, 128, 0.95, "bf16", 512, "dirichlet4", seed=4),
    5: Spec("multi-turn 16 seqs L~U[1024,8192] Hs=32 Ht=32 d=128 B=64 p=0.9 bf16", None, 32, 32,
            32, 128, 64, 0.9, "bf16", 256, "gauss", w_var=1.0 / 32, nseq_multi=16,
            len_lo=1024, len_hi=8192, seed=5),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Workload:
    """One seeded instance. Float arrays are float32 holding exactly the values both
    sides use (already bf16-rounded for bf16 workloads); *_bits hold the bf16 patterns."""
    spec: Spec
    cu_seqlens: np.ndarray      # int32 [nseq + 1]
    q: np.ndarray               # float32 [Hs][T][d]
    k: np.ndarray               # float32 [Hs][T][d]
    v: np.ndarray               # float32 [Hkv][T][d]
    W: np.ndarray               # float32 [Ht][Hs]
    q_bits: Optional[np.ndarray] = None
    k_bits: Optional[np.ndarray] = None
    v_bits: np.ndarray = None   # V is always handed to the GPU as bf16
    prefix: Optional[List[int]] = None  # multi-turn: rows copied from sequence 0

    @property
    def lens(self) -> List[int]:
        return [int(b - a) for a, b in zip(self.cu_seqlens[:-1], self.cu_seqlens[1:])]

    @property
    def T(self) -> int:
        return int(self.cu_seqlens[-1])

    def bias(self) -> dict:
        s = self.spec
        return dict(sink_n=s.sink_n, sink_bias=s.sink_bias, local_w=s.local_w,
                    local_bias=s.local_bias)


def _normal(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def make_workload(spec: Spec, seed: Optional[int] = None, lens: Optional[List[int]] = None,
                  W: Optional[np.ndarray] = None) -> Workload:
    """Draw one instance of `spec`. `lens` overrides the sequence lengths (used for
    small parity cases with the same distributions); `W` overrides the mixing matrix."""
    rng = np.random.default_rng(spec.seed if seed is None else seed)
    prefix = None
    if lens is None:
        if spec.lens is None:
            lens = [int(x) for x in rng.integers(spec.len_lo, spec.len_hi + 1, spec.nseq_multi)]
        else:
            lens = list(spec.lens)
    lens = [int(x) for x in lens]
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    T = int(cu[-1])
    q = _normal(rng, (spec.Hs, T, spec.d))
    k = _normal(rng, (spec.Hs, T, spec.d))
    v = _normal(rng, (spec.Hkv, T, spec.d))
    if W is None:
        if spec.w_kind == "gauss":
            W = (rng.standard_normal((spec.Ht, spec.Hs)) * np.sqrt(spec.w_var)).astype(np.float32)
        elif spec.w_kind == "dirichlet4":
            W = np.zeros((spec.Ht, spec.Hs), dtype=np.float32)
            for t in range(spec.Ht):
                src = rng.choice(spec.Hs, size=4, replace=False)
                W[t, src] = rng.dirichlet(np.ones(4)).astype(np.float32)
        else:
            raise ValueError(spec.w_kind)
    W = np.ascontiguousarray(W, dtype=np.float32)
    if spec.lens is None and len(lens) > 1:
        # multi-turn: later sequences repeat the head of the first one
        prefix = [0]
        for s in range(1, len(lens)):
            P = min(lens[s] // 2, lens[0])
            prefix.append(P)
            a0, a = int(cu[0]), int(cu[s])
            q[:, a:a + P] = q[:, a0:a0 + P]
            k[:, a:a + P] = k[:, a0:a0 + P]
            v[:, a:a + P] = v[:, a0:a0 + P]
    wl = Workload(spec, cu, q, k, v, W, prefix=prefix)
    if spec.qk_dtype == "bf16":
        wl.q_bits = f32_to_bf16_bits(q)
        wl.k_bits = f32_to_bf16_bits(k)
        wl.q = bf16_bits_to_f32(wl.q_bits)
        wl.k = bf16_bits_to_f32(wl.k_bits)
        wl.v_bits = f32_to_bf16_bits(v)
        wl.v = bf16_bits_to_f32(wl.v_bits)
    else:
        # fp32 Q/K; V goes to the GPU as bf16 and the oracle keeps the fp32 V
        wl.v_bits = f32_to_bf16_bits(v)
    return wl


def make_config(index: int, seed: Optional[int] = None) -> Workload:
    return make_workload(SPECS[index], seed=seed)


def small_variant(index: int, lens: List[int], seed: Optional[int] = None,
                  Hs: Optional[int] = None, Ht: Optional[int] = None,
                  Hkv: Optional[int] = None) -> Workload:
    """Same generator as workload `index`, with shorter sequences (and optionally fewer
    heads) so the oracle finishes in seconds. W keeps the workload's distribution."""
    s = SPECS[index]
    kw = {}
    if Hs is not None:
        kw["Hs"] = Hs
    if Ht is not None:
        kw["Ht"] = Ht
    if Hkv is not None:
        kw["Hkv"] = Hkv
    if kw:
        if "Hs" in kw and s.w_kind == "gauss":
            kw["w_var"] = 1.0 / kw["Hs"]
        s = dataclasses.replace(s, **kw)
    return make_workload(s, seed=seed, lens=lens)


def receiver_qk(wl: Workload, Hkr: Optional[int] = None, alpha: float = 0.9,
                seed: Optional[int] = None):
    """A receiver model's queries [Ht][T][d] and keys [Hkr][T][d] for map-distance
    profiling: each receiver head leans on the sender head with the largest weight in
    its row of W (alpha times that head's q or k plus sqrt(1 - alpha^2) times fresh
    N(0,1) noise), so the two models' maps are related but not equal.  Rounded to bf16
    for bf16 workloads.  Returns (q, k, q_bits, k_bits); the bits are None for fp32."""
    s = wl.spec
    Ht = wl.W.shape[0]
    Hkr = Ht if Hkr is None else Hkr
    rng = np.random.default_rng((s.seed if seed is None else seed) + 7919)
    top = np.argmax(np.abs(wl.W), axis=1)
    beta = np.float32(np.sqrt(1.0 - alpha * alpha))
    q = np.empty((Ht, wl.T, s.d), dtype=np.float32)
    k = np.empty((Hkr, wl.T, s.d), dtype=np.float32)
    for t in range(Ht):
        q[t] = np.float32(alpha) * wl.q[top[t]] + beta * _normal(rng, (wl.T, s.d))
    for g in range(Hkr):
        k[g] = np.float32(alpha) * wl.k[top[g * (Ht // Hkr)]] + beta * _normal(rng, (wl.T, s.d))
    if s.qk_dtype == "bf16":
        qb, kb = f32_to_bf16_bits(q), f32_to_bf16_bits(k)
        return bf16_bits_to_f32(qb), bf16_bits_to_f32(kb), qb, kb
    return q, k, None, None


def paged_v(v_bits: np.ndarray, cu: np.ndarray, page_size: int, seed: int = 0, spare: int = 3):
    """V [Hkv][T][d] (bf16 bits) laid out in a paged pool for retrieval with a page
    table: every sequence's pages go to seeded random physical slots of a pool
    [num_pages][Hkv][page_size][d] with `spare` unused pages; slots past a
    sequence's end hold random bits.  Returns (pool, block_table [nseq][max_pages])."""
    rng = np.random.default_rng(seed + 104729)
    Hkv, T, d = v_bits.shape
    lens = [int(b - a) for a, b in zip(cu[:-1], cu[1:])]
    npg = [(L + page_size - 1) // page_size for L in lens]
    maxp = max(npg + [1])
    total = sum(npg) + spare
    perm = rng.permutation(total)
    pool = rng.integers(0, 1 << 16, size=(total, Hkv, page_size, d), dtype=np.uint16)
    table = np.full((len(lens), maxp), -1, dtype=np.int32)
    k = 0
    for s, (a, L) in enumerate(zip(cu[:-1], lens)):
        for p in range(npg[s]):
            phys = int(perm[k])
            k += 1
            table[s, p] = phys
            n = min(page_size, L - p * page_size)
            pool[phys, :, :n, :] = v_bits[:, a + p * page_size:a + p * page_size + n, :]
    return pool, table
