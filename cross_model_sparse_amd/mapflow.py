"""Python binding of libmapflow.so (ctypes).

Argument marshalling only: every step of compression, retrieval and dense
attention runs in the HIP kernels behind the C ABI declared in
include/mapflow.h.  torch provides device memory and the current stream.  If
the library has not been built, load() raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Sequence

import numpy as np
import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmapflow.so")

MF_OK, MF_ERR_INVALID_ARG, MF_ERR_UNSUPPORTED, MF_ERR_CAPACITY, MF_ERR_HIP, MF_ERR_WORKSPACE = range(6)
MF_BF16, MF_FP32 = 0, 1
MF_TILE_BF16, MF_TILE_MXFP8 = 0, 1
TILE_FORMATS = {"bf16": MF_TILE_BF16, "mxfp8": MF_TILE_MXFP8}

EXPORTS = ("mf_num_block_rows", "mf_compress_max_tiles", "mf_compress_workspace_bytes",
           "mf_compress_topp", "mf_apply_workspace_bytes", "mf_apply_translated",
           "mf_dense_workspace_bytes", "mf_dense_ref_attention", "mf_read_status",
           "mf_status_string", "mf_prefix_dedupe_workspace_bytes", "mf_prefix_dedupe",
           "mf_tile_bytes", "mf_tv_distance_workspace_bytes", "mf_tv_distance",
           "mf_apply_translated_paged", "mf_apply_translated_noalloc")

# Bytes of the fixed per-GPU scratch of mf_apply_translated_noalloc
# (MF_APPLY_NOALLOC_SCRATCH_BYTES in include/mapflow.h).
APPLY_NOALLOC_SCRATCH_BYTES = 128 << 20


class MfLogitBias(ctypes.Structure):
    _fields_ = [("sink_n", ctypes.c_int32), ("sink_bias", ctypes.c_float),
                ("local_w", ctypes.c_int32), ("local_bias", ctypes.c_float)]


class MfBsrMap(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("block", ctypes.c_int32),
                ("num_block_rows", ctypes.c_int32), ("total_tokens", ctypes.c_int32),
                ("capacity_tiles", ctypes.c_int64), ("row_ptr", ctypes.c_void_p),
                ("col_idx", ctypes.c_void_p), ("tiles", ctypes.c_void_p),
                ("kept_mass", ctypes.c_void_p), ("nnz", ctypes.c_void_p),
                ("status", ctypes.c_void_p), ("row_alias", ctypes.c_void_p),
                ("tile_format", ctypes.c_int32)]


class MfPagedV(ctypes.Structure):
    _fields_ = [("pages", ctypes.c_void_p), ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("block_table", ctypes.c_void_p), ("max_pages_per_seq", ctypes.c_int32)]


class MapflowError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn}: {text} (status {status})")
        self.status = status


_lib = None


def load():
    """Load the native library (once). Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run cross_model_sparse_amd.build.build()")
    lib = ctypes.CDLL(LIB_PATH)
    i32, i64, sz, vp, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_double
    pcu = ctypes.POINTER(ctypes.c_int32)
    sig = {
        "mf_num_block_rows": (i32, [pcu, i32, i32]),
        "mf_compress_max_tiles": (i64, [i32, pcu, i32, i32]),
        "mf_compress_workspace_bytes": (sz, [i32, pcu, i32, i32, i32]),
        "mf_compress_topp": (i32, [vp, vp, vp, i32, pcu, vp, i32, i32, i32, i32, f64,
                                   ctypes.POINTER(MfLogitBias), ctypes.POINTER(MfBsrMap), vp, sz]),
        "mf_apply_workspace_bytes": (sz, [i32, pcu, i32, i32, i32]),
        "mf_apply_translated": (i32, [vp, ctypes.POINTER(MfBsrMap), vp, i32, vp, i32, i32, pcu, vp,
                                      i32, i32, vp, vp, sz]),
        "mf_dense_workspace_bytes": (sz, [i32, pcu, i32, i32]),
        "mf_dense_ref_attention": (i32, [vp, vp, vp, vp, i32, i32, i32, i32, pcu, vp, i32,
                                         ctypes.POINTER(MfLogitBias), vp, vp, sz]),
        "mf_read_status": (i32, [vp, ctypes.POINTER(MfBsrMap), ctypes.POINTER(i64)]),
        "mf_status_string": (ctypes.c_char_p, [i32]),
        "mf_prefix_dedupe_workspace_bytes": (sz, [pcu, i32, i32]),
        "mf_prefix_dedupe": (i32, [vp, vp, vp, i32, pcu, vp, i32, i32, i32, i32, vp, vp, sz]),
        "mf_tile_bytes": (i64, [i32, i32]),
        "mf_apply_translated_noalloc": (i32, [vp, ctypes.POINTER(MfBsrMap), vp, i32, vp, i32, i32, pcu,
                                              vp, i32, i32, vp]),
        "mf_apply_translated_paged": (i32, [vp, ctypes.POINTER(MfBsrMap), vp, i32, ctypes.POINTER(MfPagedV),
                                            i32, i32, pcu, vp, i32, pcu, vp, i32, vp, vp, sz]),
        "mf_tv_distance_workspace_bytes": (sz, [pcu, i32, i32]),
        "mf_tv_distance": (i32, [vp, ctypes.POINTER(MfBsrMap), vp, i32, vp, vp, i32, i32, i32, pcu,
                                 vp, i32, ctypes.POINTER(MfLogitBias), i32, vp, vp, sz]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(fn: str, st: int):
    if st != MF_OK:
        raise MapflowError(fn, st, load().mf_status_string(st).decode())


def _cu_host(cu) -> np.ndarray:
    if isinstance(cu, torch.Tensor):
        cu = cu.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(cu, dtype=np.int32))


def _cu_ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _bias(bias: Optional[dict]):
    if bias is None:
        return None
    return ctypes.byref(MfLogitBias(int(bias["sink_n"]), float(bias["sink_bias"]),
                                    int(bias["local_w"]), float(bias["local_bias"])))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MF_BF16
    if t.dtype == torch.float32:
        return MF_FP32
    raise TypeError(f"Q/K must be bfloat16 or float32, got {t.dtype}")


def _dev_cu(cu_host: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(cu_host).to(device)


def _check_tokens(what: str, t: torch.Tensor, cu: np.ndarray):
    """The kernels use cu_seqlens[-1] as the token count of every [H, T, d]
    tensor (its head stride); a tensor of another length would be read or
    written at the wrong offsets."""
    if len(cu) == 0:
        raise ValueError("cu_seqlens must have at least one entry")
    if t.dim() != 3 or int(t.shape[1]) != int(cu[-1]):
        raise ValueError(f"{what} must be [H, T, d] with T = cu_seqlens[-1] = {int(cu[-1])}, "
                         f"got {tuple(t.shape)}")


def _check_out(out: torch.Tensor, shape, dtype=torch.float32):
    if out.dtype != dtype or tuple(out.shape) != tuple(shape) or not out.is_contiguous():
        raise ValueError(f"out must be contiguous {dtype} {tuple(shape)}, got {out.dtype} "
                         f"{tuple(out.shape)}")


# ---------------------------------------------------------------------------
# size queries
# ---------------------------------------------------------------------------

def mf_num_block_rows(cu_seqlens, B: int) -> int:
    cu = _cu_host(cu_seqlens)
    return load().mf_num_block_rows(_cu_ptr(cu), len(cu) - 1, B)


def mf_compress_max_tiles(Hs: int, cu_seqlens, B: int) -> int:
    cu = _cu_host(cu_seqlens)
    return load().mf_compress_max_tiles(Hs, _cu_ptr(cu), len(cu) - 1, B)


def mf_compress_workspace_bytes(Hs: int, cu_seqlens, B: int, d: int) -> int:
    cu = _cu_host(cu_seqlens)
    return load().mf_compress_workspace_bytes(Hs, _cu_ptr(cu), len(cu) - 1, B, d)


def mf_apply_workspace_bytes(Hkv: int, cu_seqlens, B: int, d: int) -> int:
    cu = _cu_host(cu_seqlens)
    return load().mf_apply_workspace_bytes(Hkv, _cu_ptr(cu), len(cu) - 1, B, d)


def mf_dense_workspace_bytes(Hkv: int, cu_seqlens, d: int) -> int:
    cu = _cu_host(cu_seqlens)
    return load().mf_dense_workspace_bytes(Hkv, _cu_ptr(cu), len(cu) - 1, d)


# ---------------------------------------------------------------------------
# compressed map
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class BsrMap:
    """Device arrays of one compressed map (see mf_bsr_map in include/mapflow.h)."""
    num_heads: int
    block: int
    num_block_rows: int
    total_tokens: int
    row_ptr: torch.Tensor      # int64 [Hs * NBR + 1]
    col_idx: torch.Tensor      # int32 [capacity]
    tiles: torch.Tensor        # bfloat16 [capacity, B, B], or uint8 [capacity, B*B + B*B/32] (mxfp8)
    kept_mass: torch.Tensor    # float32 [Hs, T]
    nnz: torch.Tensor          # int64 [1]
    status: torch.Tensor       # int32 [1]
    row_alias: Optional[torch.Tensor] = None  # int32 [NBR] from mf_prefix_dedupe, or None
    tile_format: str = "bf16"  # "bf16" or "mxfp8"

    @property
    def capacity(self) -> int:
        return int(self.col_idx.shape[0])

    def cstruct(self) -> MfBsrMap:
        return MfBsrMap(self.num_heads, self.block, self.num_block_rows, self.total_tokens,
                        self.capacity, self.row_ptr.data_ptr(), self.col_idx.data_ptr(),
                        self.tiles.data_ptr(), self.kept_mass.data_ptr(), self.nnz.data_ptr(),
                        self.status.data_ptr(),
                        self.row_alias.data_ptr() if self.row_alias is not None else None,
                        TILE_FORMATS[self.tile_format])


def mf_tile_bytes(B: int, tile_format: str = "bf16") -> int:
    return int(load().mf_tile_bytes(B, TILE_FORMATS[tile_format]))


def alloc_map(Hs: int, cu_seqlens, B: int, device, capacity: Optional[int] = None,
              tile_format: str = "bf16") -> BsrMap:
    if tile_format not in TILE_FORMATS:
        raise ValueError(f"tile_format must be one of {sorted(TILE_FORMATS)}")
    cu = _cu_host(cu_seqlens)
    nbr = mf_num_block_rows(cu, B)
    if nbr < 0:
        raise ValueError("invalid sequence offsets or block size")
    if capacity is None:
        capacity = mf_compress_max_tiles(Hs, cu, B)
    T = int(cu[-1])
    return BsrMap(Hs, B, nbr, T,
                  torch.zeros(Hs * nbr + 1, dtype=torch.int64, device=device),
                  torch.zeros(max(capacity, 0), dtype=torch.int32, device=device),
                  (torch.empty((max(capacity, 0), B, B), dtype=torch.bfloat16, device=device)
                   if tile_format == "bf16" else
                   torch.empty((max(capacity, 0), mf_tile_bytes(B, tile_format)), dtype=torch.uint8,
                               device=device)),
                  torch.zeros((Hs, T), dtype=torch.float32, device=device),
                  torch.zeros(1, dtype=torch.int64, device=device),
                  torch.zeros(1, dtype=torch.int32, device=device),
                  tile_format=tile_format)


def mf_prefix_dedupe_workspace_bytes(cu_seqlens, B: int) -> int:
    cu = _cu_host(cu_seqlens)
    return load().mf_prefix_dedupe_workspace_bytes(_cu_ptr(cu), len(cu) - 1, B)


def mf_prefix_dedupe(q: torch.Tensor, k: torch.Tensor, cu_seqlens, B: int,
                     out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                     cu_dev: Optional[torch.Tensor] = None) -> torch.Tensor:
    """int32 [NBR]: for every global block-row, the first block-row with the same
    q/k prefix (itself when unique); pass it to mf_compress_topp as row_alias."""
    lib = load()
    cu = _cu_host(cu_seqlens)
    Hs, T, d = q.shape
    if k.shape != q.shape or k.dtype != q.dtype or not (q.is_contiguous() and k.is_contiguous()):
        raise ValueError("q and k must be contiguous, of the same shape and dtype")
    _check_tokens("q", q, cu)
    dev = q.device
    nbr = mf_num_block_rows(cu, B)
    if nbr < 0:
        raise ValueError("invalid sequence offsets or block size")
    if out is None:
        out = torch.empty(max(nbr, 1), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = torch.empty(mf_prefix_dedupe_workspace_bytes(cu, B), dtype=torch.uint8, device=dev)
    if cu_dev is None:
        cu_dev = _dev_cu(cu, dev)
    st = lib.mf_prefix_dedupe(_stream(), q.data_ptr(), k.data_ptr(), _dtype_code(q), _cu_ptr(cu),
                              cu_dev.data_ptr(), len(cu) - 1, Hs, d, B, out.data_ptr(),
                              workspace.data_ptr(), workspace.numel())
    _check("mf_prefix_dedupe", st)
    return out[:nbr]


def mf_compress_topp(q: torch.Tensor, k: torch.Tensor, cu_seqlens, B: int, p: float,
                     bias: Optional[dict] = None, out: Optional[BsrMap] = None,
                     capacity: Optional[int] = None, workspace: Optional[torch.Tensor] = None,
                     cu_dev: Optional[torch.Tensor] = None,
                     row_alias: Optional[torch.Tensor] = None,
                     tile_format: str = "bf16") -> BsrMap:
    """Block top-p compression of the causal maps of all heads of q, k ([Hs, T, d]).
    With row_alias (from mf_prefix_dedupe), block-rows that share an earlier one
    are not computed; the map keeps the alias for retrieval.  tile_format
    "mxfp8" stores block-scaled E4M3 tiles (ignored when `out` is given: the
    map's own format is used)."""
    lib = load()
    cu = _cu_host(cu_seqlens)
    Hs, T, d = q.shape
    if k.shape != q.shape or k.dtype != q.dtype:
        raise ValueError("q and k must have the same shape and dtype")
    if not (q.is_contiguous() and k.is_contiguous()):
        raise ValueError("q and k must be contiguous")
    _check_tokens("q", q, cu)
    dev = q.device
    m = out if out is not None else alloc_map(Hs, cu, B, dev, capacity, tile_format)
    if row_alias is not None and (row_alias.dtype != torch.int32 or not row_alias.is_contiguous()):
        raise ValueError("row_alias must be contiguous int32")
    m.row_alias = row_alias
    if workspace is None:
        workspace = torch.empty(mf_compress_workspace_bytes(Hs, cu, B, d), dtype=torch.uint8, device=dev)
    if cu_dev is None:
        cu_dev = _dev_cu(cu, dev)
    cs = m.cstruct()
    st = lib.mf_compress_topp(_stream(), q.data_ptr(), k.data_ptr(), _dtype_code(q), _cu_ptr(cu),
                              cu_dev.data_ptr(), len(cu) - 1, Hs, d, B, float(p), _bias(bias),
                              ctypes.byref(cs), workspace.data_ptr(), workspace.numel())
    _check("mf_compress_topp", st)
    m.num_heads, m.block, m.num_block_rows, m.total_tokens = cs.num_heads, cs.block, cs.num_block_rows, cs.total_tokens
    return m


def mf_read_status(m: BsrMap):
    """(status, nnz); synchronises the current stream."""
    nnz = ctypes.c_int64(0)
    cs = m.cstruct()
    st = load().mf_read_status(_stream(), ctypes.byref(cs), ctypes.byref(nnz))
    return int(st), int(nnz.value)


def mf_apply_translated(m: BsrMap, W: torch.Tensor, v: torch.Tensor, cu_seqlens, renorm: bool = True,
                        out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                        cu_dev: Optional[torch.Tensor] = None) -> torch.Tensor:
    """O_t = sum_h W[t,h] renorm(A_hat_h) V_g(t) for all targets; v is [Hkv, T, d] bf16."""
    lib = load()
    cu = _cu_host(cu_seqlens)
    Ht = W.shape[0]
    Hkv, T, d = v.shape
    if v.dtype != torch.bfloat16 or not v.is_contiguous():
        raise ValueError("v must be contiguous bfloat16")
    if W.dtype != torch.float32 or not W.is_contiguous() or W.dim() != 2 or W.shape[1] != m.num_heads:
        raise ValueError("W must be contiguous float32 [Ht, Hs]")
    _check_tokens("v", v, cu)
    dev = v.device
    if out is None:
        out = torch.empty((Ht, T, d), dtype=torch.float32, device=dev)
    else:
        _check_out(out, (Ht, T, d))
    if workspace is None:
        workspace = torch.empty(mf_apply_workspace_bytes(Hkv, cu, m.block, d), dtype=torch.uint8, device=dev)
    if cu_dev is None:
        cu_dev = _dev_cu(cu, dev)
    cs = m.cstruct()
    st = lib.mf_apply_translated(_stream(), ctypes.byref(cs), W.data_ptr(), Ht, v.data_ptr(), Hkv, d,
                                 _cu_ptr(cu), cu_dev.data_ptr(), len(cu) - 1, int(bool(renorm)),
                                 out.data_ptr(), workspace.data_ptr(), workspace.numel())
    _check("mf_apply_translated", st)
    return out


def mf_apply_translated_noalloc(m: BsrMap, W: torch.Tensor, v: torch.Tensor, cu_seqlens,
                                renorm: bool = True, out: Optional[torch.Tensor] = None,
                                cu_dev: Optional[torch.Tensor] = None) -> torch.Tensor:
    """mf_apply_translated with the library's fixed per-GPU scratch in place of a
    workspace: the native call allocates nothing.  Pass `out` and `cu_dev` to
    keep the binding from allocating them.  Calls that overlap on one GPU race."""
    lib = load()
    cu = _cu_host(cu_seqlens)
    Ht = W.shape[0]
    Hkv, T, d = v.shape
    if v.dtype != torch.bfloat16 or not v.is_contiguous():
        raise ValueError("v must be contiguous bfloat16")
    if W.dtype != torch.float32 or not W.is_contiguous() or W.dim() != 2 or W.shape[1] != m.num_heads:
        raise ValueError("W must be contiguous float32 [Ht, Hs]")
    _check_tokens("v", v, cu)
    dev = v.device
    if out is None:
        out = torch.empty((Ht, T, d), dtype=torch.float32, device=dev)
    else:
        _check_out(out, (Ht, T, d))
    if cu_dev is None:
        cu_dev = _dev_cu(cu, dev)
    cs = m.cstruct()
    st = lib.mf_apply_translated_noalloc(_stream(), ctypes.byref(cs), W.data_ptr(), Ht, v.data_ptr(), Hkv,
                                         d, _cu_ptr(cu), cu_dev.data_ptr(), len(cu) - 1,
                                         int(bool(renorm)), out.data_ptr())
    _check("mf_apply_translated_noalloc", st)
    return out


def mf_apply_translated_paged(m: BsrMap, W: torch.Tensor, pages: torch.Tensor, block_table: torch.Tensor,
                              cu_seqlens, window=None, renorm: bool = True,
                              out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                              cu_dev: Optional[torch.Tensor] = None,
                              window_dev: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Translated retrieval with V in a paged pool pages [num_pages, Hkv, page_size, d]
    (bf16) addressed through block_table [nseq, max_pages] (int32), optionally only
    for the query-token windows `window` ([nseq][2], a prefill chunk per sequence);
    rows outside the windows of `out` are left as they are."""
    lib = load()
    cu = _cu_host(cu_seqlens)
    Ht = W.shape[0]
    npages, Hkv, P, d = pages.shape
    if pages.dtype != torch.bfloat16 or not pages.is_contiguous():
        raise ValueError("pages must be contiguous bfloat16 [num_pages, Hkv, page_size, d]")
    if block_table.dtype != torch.int32 or not block_table.is_contiguous() or block_table.dim() != 2:
        raise ValueError("block_table must be contiguous int32 [nseq, max_pages]")
    if W.dtype != torch.float32 or not W.is_contiguous() or W.dim() != 2 or W.shape[1] != m.num_heads:
        raise ValueError("W must be contiguous float32 [Ht, Hs]")
    dev = pages.device
    T = int(cu[-1])
    if out is None:
        out = torch.zeros((Ht, T, d), dtype=torch.float32, device=dev)
    else:
        _check_out(out, (Ht, T, d))
    if workspace is None:
        workspace = torch.empty(mf_apply_workspace_bytes(Hkv, cu, m.block, d), dtype=torch.uint8, device=dev)
    if cu_dev is None:
        cu_dev = _dev_cu(cu, dev)
    wh = wd = None
    if window is not None:
        wh = np.ascontiguousarray(np.asarray(window, dtype=np.int32).reshape(-1))
        wd = window_dev if window_dev is not None else torch.from_numpy(wh).to(dev)
    pv = MfPagedV(pages.data_ptr(), P, npages, block_table.data_ptr(), int(block_table.shape[1]))
    cs = m.cstruct()
    st = lib.mf_apply_translated_paged(_stream(), ctypes.byref(cs), W.data_ptr(), Ht, ctypes.byref(pv),
                                       Hkv, d, _cu_ptr(cu), cu_dev.data_ptr(), len(cu) - 1,
                                       _cu_ptr(wh) if wh is not None else None,
                                       wd.data_ptr() if wd is not None else None, int(bool(renorm)),
                                       out.data_ptr(), workspace.data_ptr(), workspace.numel())
    _check("mf_apply_translated_paged", st)
    return out


def mf_tv_distance(m: BsrMap, W: torch.Tensor, q: torch.Tensor, k: torch.Tensor, cu_seqlens,
                   bias: Optional[dict] = None, renorm: bool = True,
                   out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                   cu_dev: Optional[torch.Tensor] = None) -> torch.Tensor:
    """[Ht, T] fp32: 1/2 sum_j |translated - receiver| per query row; q [Ht, T, d] and
    k [Hkr, T, d] are the receiver's."""
    lib = load()
    cu = _cu_host(cu_seqlens)
    Ht, T, d = q.shape
    Hkr = k.shape[0]
    if k.dtype != q.dtype or k.shape[1:] != q.shape[1:] or not (q.is_contiguous() and k.is_contiguous()):
        raise ValueError("q and k must be contiguous, of one dtype, [H, T, d]")
    if W.dtype != torch.float32 or not W.is_contiguous() or tuple(W.shape) != (Ht, m.num_heads):
        raise ValueError("W must be contiguous float32 [Ht, Hs]")
    _check_tokens("q", q, cu)
    dev = q.device
    if out is None:
        out = torch.empty((Ht, T), dtype=torch.float32, device=dev)
    else:
        _check_out(out, (Ht, T))
    if workspace is None:
        workspace = torch.empty(lib.mf_tv_distance_workspace_bytes(_cu_ptr(cu), len(cu) - 1, m.block),
                                dtype=torch.uint8, device=dev)
    if cu_dev is None:
        cu_dev = _dev_cu(cu, dev)
    cs = m.cstruct()
    st = lib.mf_tv_distance(_stream(), ctypes.byref(cs), W.data_ptr(), Ht, q.data_ptr(), k.data_ptr(),
                            _dtype_code(q), Hkr, d, _cu_ptr(cu), cu_dev.data_ptr(), len(cu) - 1,
                            _bias(bias), int(bool(renorm)), out.data_ptr(), workspace.data_ptr(),
                            workspace.numel())
    _check("mf_tv_distance", st)
    return out


def mf_dense_ref_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens,
                           bias: Optional[dict] = None, out: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None,
                           cu_dev: Optional[torch.Tensor] = None) -> torch.Tensor:
    """softmax(Q K^T / sqrt(d) + bias) V, causal, GQA; q [Hq,T,d], k [Hkv,T,d], v bf16 [Hkv,T,d]."""
    lib = load()
    cu = _cu_host(cu_seqlens)
    Hq, T, d = q.shape
    Hkv = k.shape[0]
    if k.dtype != q.dtype or v.dtype != torch.bfloat16:
        raise ValueError("k must match q's dtype; v must be bfloat16")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k and v must be contiguous")
    if k.dim() != 3 or tuple(k.shape[1:]) != (T, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [Hkv, T, d] with q's T and d")
    _check_tokens("q", q, cu)
    dev = q.device
    if out is None:
        out = torch.empty((Hq, T, d), dtype=torch.float32, device=dev)
    else:
        _check_out(out, (Hq, T, d))
    if workspace is None:
        workspace = torch.empty(mf_dense_workspace_bytes(Hkv, cu, d), dtype=torch.uint8, device=dev)
    if cu_dev is None:
        cu_dev = _dev_cu(cu, dev)
    st = lib.mf_dense_ref_attention(_stream(), q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q),
                                    Hq, Hkv, d, _cu_ptr(cu), cu_dev.data_ptr(), len(cu) - 1, _bias(bias),
                                    out.data_ptr(), workspace.data_ptr(), workspace.numel())
    _check("mf_dense_ref_attention", st)
    return out
