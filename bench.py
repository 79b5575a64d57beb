"""Benchmark: compressed-map prefill throughput on one MI355X.

One step = one pass of the whole hot path over one batch: block top-p
compression of every source head's causal attention map into BSR tiles
(mf_compress_topp) followed by translated retrieval for every target head
(mf_apply_translated).  Inputs are seeded synthetic tensors already resident in
device memory; the map, workspaces and output are preallocated.

Prints one JSON line (rank 0).  The default workload is the long-context one:
one sequence of 32768 tokens, 32 source heads -> 64 target heads, d = 128,
B = 128, p = 0.95, bf16 Q/K/V, each target mixing 4 sources (Dirichlet weights).

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
                  [--config N] [--dedupe] [--tile-format bf16|mxfp8]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # dense bf16 MFMA


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# sources each recorded launch sequence is built from (relative to the repository root)
KERNEL_SOURCES = {
    "mf_apply_translated": ("cross_model_sparse_amd/csrc/mf_apply.hip", "cross_model_sparse_amd/csrc/mf_rows.hip",
                            "cross_model_sparse_amd/csrc/mf_common.hpp", "cross_model_sparse_amd/csrc/mf_host.hpp",
                            "include/mapflow.h"),
    "mf_compress_topp": ("cross_model_sparse_amd/csrc/mf_compress.hip", "cross_model_sparse_amd/csrc/mf_qk.hpp",
                         "cross_model_sparse_amd/csrc/mf_rows.hip", "cross_model_sparse_amd/csrc/mf_common.hpp",
                         "cross_model_sparse_amd/csrc/mf_host.hpp", "include/mapflow.h"),
}


def source_hash(kernel: str) -> str:
    """Hash of the sources a recorded kernel sequence is built from: a traffic record
    taken with other sources does not describe the kernel that runs now."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_record(kernel: str, workload: str):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE for this
    kernel, if recorded for the current kernel sources (else None)."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p))
    except (OSError, ValueError):
        return None
    r = rec.get(kernel, {}).get(workload)
    if not r or r.get("source_hash") != source_hash(kernel):
        return None
    return r.get("bytes_per_launch")


def algorithmic_bytes(wl, nnz: int, tile_format: str = "bf16") -> dict:
    s = wl.spec
    T, NBR = wl.T, sum((L + s.B - 1) // s.B for L in wl.lens)
    e_qk = 4 if s.qk_dtype == "fp32" else 2
    meta = (s.Hs * NBR + 1) * 8 + s.Hs * T * 4          # row_ptr + kept mass
    tile = s.B * s.B * 2 if tile_format == "bf16" else s.B * s.B + s.B * (s.B // 32)
    tiles = nnz * (tile + 4)                             # tiles + col_idx
    compress = 2 * s.Hs * T * s.d * e_qk + tiles + meta
    apply = tiles + meta + s.Hkv * T * s.d * 2 + s.Ht * s.Hs * 4 + s.Ht * T * s.d * 4
    return dict(compress=compress, apply=apply)


def mfma_flops(torch, wl, m, W, nnz: int) -> dict:
    """Algorithmic MFMA work: compress = one QK^T over every causal tile of every
    source head; apply = one (B x B) x (B x d) product per target, query block and
    key block in the union of the target's sources' kept blocks."""
    s = wl.spec
    NBR = m.num_block_rows
    nbs = [(L + s.B - 1) // s.B for L in wl.lens]
    tri = sum(n * (n + 1) // 2 for n in nbs)
    compress = 2.0 * s.d * s.B * s.B * s.Hs * tri
    dev = m.row_ptr.device
    rp = m.row_ptr
    rows = torch.repeat_interleave(torch.arange(s.Hs * NBR, device=dev), rp[1:] - rp[:-1])
    kept = torch.zeros((s.Hs, NBR, max(nbs)), dtype=torch.bool, device=dev)
    kept[rows // NBR, rows % NBR, m.col_idx[:nnz].long()] = True
    if m.row_alias is not None:
        kept = kept[:, m.row_alias.long()]
    nz = (W != 0)
    blocks = sum(int(kept[nz[t]].any(dim=0).sum()) for t in range(W.shape[0]))
    return dict(compress=compress, apply=2.0 * s.B * s.B * s.d * blocks)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, rows, target_stride: int = 2):
    """The fp64 oracle on a bounded sample: block-rows `rows` compressed for every
    source head, retrieved for every `target_stride`-th target head; each part
    scaled to the whole workload (compress by the share of causal key blocks the
    sampled rows cover, retrieval also by the share of targets)."""
    from threadpoolctl import threadpool_info
    from oracle import mapflow_oracle as orc
    s = wl.spec
    targets = list(range(0, s.Ht, target_stride))
    t0 = time.perf_counter()
    res = orc.compress(wl.q, wl.k, wl.cu_seqlens, s.B, s.p, wl.bias(), rows=rows)
    t1 = time.perf_counter()
    orc.apply(res, wl.W, wl.v, wl.cu_seqlens, s.B, s.Hkv, rows=rows, targets=targets)
    t2 = time.perf_counter()
    blocks_sample = sum(I + 1 for (_, I) in rows)
    blocks_total = sum(n * (n + 1) // 2 for n in ((L + s.B - 1) // s.B for L in wl.lens))
    full = ((t1 - t0) + (t2 - t1) * s.Ht / len(targets)) * blocks_total / blocks_sample
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return dict(value=wl.T / full, unit="tokens/s", cores=int(threads), kind="oracle",
                cpu=cpu_model(),
                sample=(f"fp64 numpy oracle: compress of block-rows {[I for _, I in rows]} (all {s.Hs} "
                        f"source heads, {t1 - t0:.1f} s) and retrieval of them for {len(targets)} of "
                        f"{s.Ht} target heads ({t2 - t1:.1f} s), scaled by {s.Ht}/{len(targets)} targets "
                        f"and {blocks_total}/{blocks_sample} causal key blocks to the whole workload; "
                        f"BLAS uses up to {threads} threads, numpy's elementwise exp and sums one"))


def copy_calibration(torch, nbytes: int = 1 << 30, reps: int = 3):
    """A plain copy of known size: under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE its
    counters give the scale between the counters and bytes actually moved."""
    dev = torch.device("cuda:0")
    a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)


def tv_bench(torch, mf, wlmod, wl, m, W, cu, cu_dev, args):
    """Times mf_tv_distance over the whole workload (every target head and row)."""
    s = wl.spec
    dev = W.device
    rq, rk, rqb, rkb = wlmod.receiver_qk(wl)
    if rqb is not None:
        qr = torch.from_numpy(rqb.view(np.int16)).to(dev).view(torch.bfloat16)
        kr = torch.from_numpy(rkb.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        qr, kr = torch.from_numpy(rq).to(dev), torch.from_numpy(rk).to(dev)
    del rq, rk, rqb, rkb
    out = torch.empty((W.shape[0], wl.T), dtype=torch.float32, device=dev)
    ws = torch.empty(mf.load().mf_tv_distance_workspace_bytes(mf._cu_ptr(mf._cu_host(cu)), len(cu) - 1, s.B),
                     dtype=torch.uint8, device=dev)
    for _ in range(max(args.warmup, 1)):
        mf.mf_tv_distance(m, W, qr, kr, cu, wl.bias(), out=out, workspace=ws, cu_dev=cu_dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        mf.mf_tv_distance(m, W, qr, kr, cu, wl.bias(), out=out, workspace=ws, cu_dev=cu_dev)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ms_ev = e0.elapsed_time(e1) / args.steps
    nbs = [(L + s.B - 1) // s.B for L in wl.lens]
    tri = sum(n * (n + 1) // 2 for n in nbs)
    flops = 2 * 2.0 * s.d * s.B * s.B * W.shape[0] * tri     # two Q K^T passes per target
    log(f"tv: {ms_ev:.3f} ms per call, mean tv {float(out.mean()):.4f}")
    line = {
        "metric": "map TV-distance profiling tokens/s (all target heads)",
        "value": round(wl.T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if s.qk_dtype == "bf16" else "fp32", "data": "synthetic",
        "config": {"workload": s.name, "tokens": wl.T, "target_heads": int(W.shape[0]),
                   "tile_format": args.tile_format, "parallelism": "none (1 GPU)"},
        "roofline": {"kernel": "mf_tv_distance", "bound": "mfma",
                     "achieved": round(flops / (ms_ev * 1e-3) / 1e12, 1), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(flops / (ms_ev * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "ms_per_launch": round(ms_ev, 4)},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def dense_bench(torch, mf, wlmod, wl, v, cu, cu_dev, args):
    """Times mf_dense_ref_attention for a receiver layer recomputed in full: the
    receiver's Ht query heads against the workload's Hkv key/value heads, every
    causal row (MFMA work 4 d sum_s L_s (L_s + 1) / 2 per query head)."""
    s = wl.spec
    dev = v.device
    Ht = int(wl.W.shape[0])
    rq, rk, rqb, rkb = wlmod.receiver_qk(wl, Hkr=s.Hkv)
    if rqb is not None:
        qr = torch.from_numpy(rqb.view(np.int16)).to(dev).view(torch.bfloat16)
        kr = torch.from_numpy(rkb.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        qr, kr = torch.from_numpy(rq).to(dev), torch.from_numpy(rk).to(dev)
    del rq, rk, rqb, rkb
    out = torch.empty((Ht, wl.T, s.d), dtype=torch.float32, device=dev)
    ws = torch.empty(mf.mf_dense_workspace_bytes(s.Hkv, cu, s.d), dtype=torch.uint8, device=dev)
    for _ in range(max(args.warmup, 1)):
        mf.mf_dense_ref_attention(qr, kr, v, cu, wl.bias(), out=out, workspace=ws, cu_dev=cu_dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        mf.mf_dense_ref_attention(qr, kr, v, cu, wl.bias(), out=out, workspace=ws, cu_dev=cu_dev)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ms_ev = e0.elapsed_time(e1) / args.steps
    causal = sum(L * (L + 1) // 2 for L in wl.lens)
    flops = 4.0 * s.d * causal * Ht
    log(f"dense: {ms_ev:.3f} ms per call ({Ht} query heads, {s.Hkv} kv heads)")
    line = {
        "metric": "dense causal attention tokens/s (recomputed receiver layer, all heads)",
        "value": round(wl.T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if s.qk_dtype == "bf16" else "fp32", "data": "synthetic",
        "config": {"workload": s.name, "tokens": wl.T, "query_heads": Ht, "kv_heads": int(s.Hkv),
                   "parallelism": "none (1 GPU)"},
        "roofline": {"kernel": "mf_dense_ref_attention", "bound": "mfma",
                     "achieved": round(flops / (ms_ev * 1e-3) / 1e12, 1), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(flops / (ms_ev * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "ms_per_launch": round(ms_ev, 4)},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=4, help="workload index (4: long context)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dedupe", action="store_true",
                    help="share block-rows whose q/k prefix repeats an earlier sequence's "
                         "(mf_prefix_dedupe inside every step; multi-turn workload 5)")
    ap.add_argument("--tile-format", choices=("bf16", "mxfp8"), default="bf16",
                    help="map tiles: bf16, or block-scaled E4M3 (half the tile bytes)")
    ap.add_argument("--tv", action="store_true",
                    help="time mf_tv_distance (translated map vs a synthetic receiver's own map) "
                         "on the compressed map instead of the compress + apply step")
    ap.add_argument("--dense", action="store_true",
                    help="time mf_dense_ref_attention (a receiver layer recomputed in full) "
                         "instead of the compress + apply step")
    ap.add_argument("--paged", type=int, default=0, metavar="P",
                    help="V in a paged pool of P-token pages (mf_apply_translated_paged)")
    ap.add_argument("--chunks", type=int, default=1,
                    help="with --paged: prefill in this many query chunks per step")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (HBM counter scale)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only: the hot path is measured on a single MI355X "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}); multi-GPU sharding is not built.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        copy_calibration(torch)
        return
    from cross_model_sparse_amd import mapflow as mf
    from cross_model_sparse_amd import workloads as wlmod

    mf.load()
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    wl = wlmod.make_config(args.config)
    s = wl.spec
    log(f"workload {args.config}: {s.name}; T={wl.T} generated in {time.perf_counter() - t0:.1f}s")

    if s.qk_dtype == "bf16":
        q = torch.from_numpy(wl.q_bits.view(np.int16)).to(dev).view(torch.bfloat16)
        k = torch.from_numpy(wl.k_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        q = torch.from_numpy(wl.q).to(dev)
        k = torch.from_numpy(wl.k).to(dev)
    v = torch.from_numpy(wl.v_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    W = torch.from_numpy(wl.W).to(dev)
    cu = wl.cu_seqlens
    cu_dev = torch.from_numpy(cu).to(dev)
    m = mf.alloc_map(s.Hs, cu, s.B, dev, tile_format=args.tile_format)
    ws_c = torch.empty(mf.mf_compress_workspace_bytes(s.Hs, cu, s.B, s.d), dtype=torch.uint8, device=dev)
    ws_a = torch.empty(mf.mf_apply_workspace_bytes(s.Hkv, cu, s.B, s.d), dtype=torch.uint8, device=dev)
    O = torch.empty((s.Ht, wl.T, s.d), dtype=torch.float32, device=dev)
    bias = wl.bias()
    alias_buf = ws_d = None
    if args.dedupe:
        alias_buf = torch.empty(max(m.num_block_rows, 1), dtype=torch.int32, device=dev)
        ws_d = torch.empty(mf.mf_prefix_dedupe_workspace_bytes(cu, s.B), dtype=torch.uint8, device=dev)

    def compress():
        ra = None
        if args.dedupe:
            ra = mf.mf_prefix_dedupe(q, k, cu, s.B, out=alias_buf, workspace=ws_d, cu_dev=cu_dev)
        mf.mf_compress_topp(q, k, cu, s.B, s.p, bias, out=m, workspace=ws_c, cu_dev=cu_dev,
                            row_alias=ra)

    windows = None
    if args.paged:
        pool_np, table_np = wlmod.paged_v(wl.v_bits, cu, args.paged)
        pool = torch.from_numpy(pool_np.view(np.int16)).to(dev).view(torch.bfloat16)
        table = torch.from_numpy(table_np).to(dev)
        del pool_np
        nbmax = max((L + s.B - 1) // s.B for L in wl.lens)
        per = (nbmax + args.chunks - 1) // args.chunks
        windows = []
        for c in range(args.chunks):
            w = [[min(c * per * s.B, L), min((c + 1) * per * s.B, L)] for L in wl.lens]
            windows.append((w, torch.from_numpy(np.asarray(w, dtype=np.int32).reshape(-1)).to(dev)))

    def apply():
        if args.paged:
            for w, wd in windows:
                mf.mf_apply_translated_paged(m, W, pool, table, cu, window=w if args.chunks > 1 else None,
                                             out=O, workspace=ws_a, cu_dev=cu_dev,
                                             window_dev=wd if args.chunks > 1 else None)
        else:
            mf.mf_apply_translated(m, W, v, cu, out=O, workspace=ws_a, cu_dev=cu_dev)

    def step():
        compress()
        apply()

    if args.dense:
        dense_bench(torch, mf, wlmod, wl, v, cu, cu_dev, args)
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    nnz = None
    if args.warmup > 0:
        st, nnz = mf.mf_read_status(m)
        if st != mf.MF_OK:
            raise SystemExit(f"compression status {st}")
        log(f"warmup done: nnz={nnz} tiles ({nnz / m.capacity:.3f} of causal)")

    if args.tv:
        if args.warmup == 0:
            step()
        tv_bench(torch, mf, wlmod, wl, m, W, cu, cu_dev, args)
        return

    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        compress()
        ev[i][1].record(stream)
        apply()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    st2, nnz2 = mf.mf_read_status(m)
    if st2 != mf.MF_OK or (nnz is not None and nnz2 != nnz):
        raise SystemExit(f"compression status {st2}, kept tiles {nnz2} (warmup {nnz})")
    nnz = nnz2
    ms_step = (t1 - t0) * 1e3 / args.steps
    t_comp = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    t_apply = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    log(f"ms/step {ms_step:.3f}  compress {t_comp:.3f} ms  apply {t_apply:.3f} ms")

    ab = algorithmic_bytes(wl, nnz, args.tile_format)
    fl = mfma_flops(torch, wl, m, W, nnz)
    workload = f"workload{args.config}" + ("" if args.tile_format == "bf16" else f"_{args.tile_format}")
    if args.paged:
        workload += f"_paged{args.paged}x{args.chunks}"
    achieved = ab["apply"] / (t_apply * 1e-3) / 1e9
    traffic = traffic_record("mf_apply_translated", workload)
    roof = dict(kernel="mf_apply_translated (fused retrieval)", bound="hbm", achieved=round(achieved, 1),
                peak=HBM_PEAK_GBS, unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic,
                algorithmic_bytes=int(ab["apply"]), ms_per_launch=round(t_apply, 4),
                mfma_tflops=round(fl["apply"] / (t_apply * 1e-3) / 1e12, 1),
                mfma_frac=round(fl["apply"] / (t_apply * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                compress_ms=round(t_comp, 4),
                compress_gbs=round(ab["compress"] / (t_comp * 1e-3) / 1e9, 1),
                compress_mfma_tflops=round(fl["compress"] / (t_comp * 1e-3) / 1e12, 1),
                compress_mfma_frac=round(fl["compress"] / (t_comp * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4))

    cpu = None
    if not args.no_cpu_baseline:
        # 8 block-rows at the centres of 8 equal bands of the longest sequence
        sq = int(np.argmax(wl.lens))
        nb = (wl.lens[sq] + s.B - 1) // s.B
        rows = sorted({(sq, min(nb - 1, int((2 * b + 1) * nb // 16))) for b in range(8)})
        log(f"cpu baseline on block-rows {rows} ...")
        cpu = cpu_baseline(wl, rows)
        log(f"cpu baseline {cpu['value']:.1f} tokens/s")

    if args.dedupe:
        a = alias_buf[:m.num_block_rows].cpu().numpy()
        shared = int((a != np.arange(len(a))).sum())
        log(f"dedupe: {shared} of {len(a)} block-rows share an earlier one")
    line = {
        "metric": ("compressed-map prefill tokens/s at L=32K (compress+apply)"
                   if args.config == 4 and args.tile_format == "bf16" and not args.paged
                   else "compressed-map prefill tokens/s (compress+apply)"),
        "value": round(wl.T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if s.qk_dtype == "bf16" else "fp32",
        "data": "synthetic",
        "config": {"workload": s.name, "tokens": wl.T, "source_heads": s.Hs, "target_heads": s.Ht,
                   "v_heads": s.Hkv, "head_dim": s.d, "block": s.B, "top_p": s.p,
                   "kept_tiles": nnz, "tile_format": args.tile_format,
                   "v_pages": args.paged or None, "prefill_chunks": args.chunks if args.paged else 1,
                   "prefix_dedupe": bool(args.dedupe),
                   "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
