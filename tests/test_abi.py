"""C-ABI boundary on the CPU: the library loads, exports every entry point that
include/mapflow.h declares, answers size queries, and rejects invalid arguments
before touching the GPU (no device calls are made here)."""
import ctypes
import os
import re

import numpy as np
import pytest

from cross_model_sparse_amd import mapflow as mf
from cross_model_sparse_amd import workloads as wlmod

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mf.LIB_PATH):
        from cross_model_sparse_amd import build
        build.build()
    return mf.load()


def header_functions():
    text = open(os.path.join(ROOT, "include", "mapflow.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mf_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert len(names) == 17
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(mf.EXPORTS) == names


def cu(lens):
    c = np.zeros(len(lens) + 1, dtype=np.int32)
    c[1:] = np.cumsum(lens)
    return c


def test_size_queries(lib):
    lens = [300, 0, 1, 129, 4096]
    c = cu(lens)
    nb = [(L + 63) // 64 for L in lens]
    assert mf.mf_num_block_rows(c, 64) == sum(nb)
    assert mf.mf_compress_max_tiles(5, c, 64) == 5 * sum(n * (n + 1) // 2 for n in nb)
    ws = mf.mf_compress_workspace_bytes(5, c, 64, 128)
    # partials alone: 4 bytes per (row, causal block) and head
    assert ws >= 5 * 64 * sum(n * (n + 1) // 2 for n in nb) * 4
    assert mf.mf_apply_workspace_bytes(2, c, 64, 128) >= 2 * 128 * sum(nb) * 64 * 2
    assert mf.mf_dense_workspace_bytes(2, c, 64) > 0
    # invalid geometry
    assert mf.mf_num_block_rows(c, 48) == -1
    assert mf.mf_num_block_rows(np.array([0, 5, 3], dtype=np.int32), 64) == -1
    assert mf.mf_num_block_rows(np.array([1, 5], dtype=np.int32), 64) == -1
    assert mf.mf_compress_max_tiles(0, c, 64) == -1
    assert mf.mf_compress_workspace_bytes(5, c, 64, 96) == 0
    # more than 1024 key blocks in one sequence
    assert mf.mf_num_block_rows(cu([32 * 1024 + 1]), 32) == -1


def _compress(lib, c, Hs=2, d=64, B=32, p=0.9, dtype=0, mp=True, ws=1 << 40, bias=None):
    m = mf.MfBsrMap(0, 0, 0, 0, 10, 8, 8, 8, 8, 8, 8)
    fake = ctypes.c_void_p(16)
    return lib.mf_compress_topp(None, fake, fake, dtype, c.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                fake, len(c) - 1, Hs, d, B, p, bias,
                                ctypes.byref(m) if mp else None, fake, ws)


def test_compress_rejects_bad_arguments(lib):
    c = cu([100, 50])
    assert _compress(lib, c, mp=False) == mf.MF_ERR_INVALID_ARG
    assert _compress(lib, c, B=48) == mf.MF_ERR_UNSUPPORTED
    assert _compress(lib, c, d=96) == mf.MF_ERR_UNSUPPORTED
    assert _compress(lib, c, dtype=7) == mf.MF_ERR_UNSUPPORTED
    for p in (0.0, -0.5, 1.0000001, float("nan")):
        assert _compress(lib, c, p=p) == mf.MF_ERR_INVALID_ARG
    assert _compress(lib, c, Hs=0) == mf.MF_ERR_INVALID_ARG
    assert _compress(lib, np.array([0, 10, 5], dtype=np.int32)) == mf.MF_ERR_INVALID_ARG
    assert _compress(lib, c, ws=100) == mf.MF_ERR_WORKSPACE
    bad = mf.MfLogitBias(4, float("inf"), 8, 1.0)
    assert _compress(lib, c, bias=ctypes.byref(bad)) == mf.MF_ERR_INVALID_ARG


def test_apply_and_dense_reject_bad_arguments(lib):
    c = cu([100])
    fake = ctypes.c_void_p(16)
    pc = c.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    m = mf.MfBsrMap(2, 32, 4, 100, 10, 8, 8, 8, 8, 8, 8, None)
    f = lib.mf_apply_translated
    assert f(None, ctypes.byref(m), fake, 4, fake, 3, 64, pc, fake, 1, 1, fake, fake, 1 << 40) == mf.MF_ERR_INVALID_ARG
    assert f(None, ctypes.byref(m), fake, 4, fake, 2, 80, pc, fake, 1, 1, fake, fake, 1 << 40) == mf.MF_ERR_UNSUPPORTED
    m.num_block_rows = 5  # does not match the offsets
    assert f(None, ctypes.byref(m), fake, 4, fake, 2, 64, pc, fake, 1, 1, fake, fake, 1 << 40) == mf.MF_ERR_INVALID_ARG
    m.num_block_rows = 4
    assert f(None, ctypes.byref(m), fake, 4, fake, 2, 64, pc, fake, 1, 1, fake, fake, 10) == mf.MF_ERR_WORKSPACE
    g = lib.mf_dense_ref_attention
    assert g(None, fake, fake, fake, 0, 6, 4, 64, pc, fake, 1, None, fake, fake, 1 << 40) == mf.MF_ERR_INVALID_ARG
    assert g(None, fake, fake, fake, 0, 4, 4, 64, pc, fake, 1, None, fake, fake, 10) == mf.MF_ERR_WORKSPACE
    assert lib.mf_read_status(None, None, None) == mf.MF_ERR_INVALID_ARG


def test_prefix_dedupe_rejects_bad_arguments(lib):
    c = cu([100, 60])
    fake = ctypes.c_void_p(16)
    pc = c.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    need = lib.mf_prefix_dedupe_workspace_bytes(pc, 2, 32)
    assert need > 0
    assert lib.mf_prefix_dedupe_workspace_bytes(pc, 2, 48) == 0
    f = lib.mf_prefix_dedupe
    assert f(None, fake, fake, 0, None, fake, 2, 4, 64, 32, fake, fake, need) == mf.MF_ERR_INVALID_ARG
    assert f(None, fake, fake, 0, pc, fake, 2, 0, 64, 32, fake, fake, need) == mf.MF_ERR_INVALID_ARG
    assert f(None, fake, fake, 7, pc, fake, 2, 4, 64, 32, fake, fake, need) == mf.MF_ERR_UNSUPPORTED
    assert f(None, fake, fake, 0, pc, fake, 2, 4, 96, 32, fake, fake, need) == mf.MF_ERR_UNSUPPORTED
    assert f(None, fake, fake, 0, pc, fake, 2, 4, 64, 32, None, fake, need) == mf.MF_ERR_INVALID_ARG
    assert f(None, fake, fake, 0, pc, fake, 2, 4, 64, 32, fake, fake, need - 1) == mf.MF_ERR_WORKSPACE


def test_tile_bytes(lib):
    for B in (32, 64, 128):
        assert lib.mf_tile_bytes(B, mf.MF_TILE_BF16) == B * B * 2
        assert lib.mf_tile_bytes(B, mf.MF_TILE_MXFP8) == B * B + B * (B // 32)
    assert lib.mf_tile_bytes(48, mf.MF_TILE_BF16) == 0
    assert lib.mf_tile_bytes(64, 2) == 0
    assert lib.mf_tile_bytes(64, -1) == 0


def test_unknown_tile_format_rejected(lib):
    c = cu([100])
    fake = ctypes.c_void_p(16)
    pc = c.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    m = mf.MfBsrMap(0, 0, 0, 0, 10, 8, 8, 8, 8, 8, 8, None, 2)
    assert lib.mf_compress_topp(None, fake, fake, 0, pc, fake, 1, 2, 64, 32, 0.9, None,
                                ctypes.byref(m), fake, 1 << 40) == mf.MF_ERR_INVALID_ARG
    m = mf.MfBsrMap(2, 32, 4, 100, 10, 8, 8, 8, 8, 8, 8, None, 5)
    assert lib.mf_apply_translated(None, ctypes.byref(m), fake, 4, fake, 2, 64, pc, fake, 1, 1,
                                   fake, fake, 1 << 40) == mf.MF_ERR_INVALID_ARG


def test_tv_distance_rejects_bad_arguments(lib):
    c = cu([100])
    fake = ctypes.c_void_p(16)
    pc = c.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    need = lib.mf_tv_distance_workspace_bytes(pc, 1, 32)
    assert need > 0 and lib.mf_tv_distance_workspace_bytes(pc, 1, 48) == 0
    m = mf.MfBsrMap(2, 32, 4, 100, 10, 8, 8, 8, 8, 8, 8, None, 0)
    f = lib.mf_tv_distance
    args = lambda Ht=4, Hkr=2, dt=0, d=64, ws=need: (None, ctypes.byref(m), fake, Ht, fake, fake, dt, Hkr, d,
                                                      pc, fake, 1, None, 1, fake, fake, ws)
    assert f(*args(Hkr=3)) == mf.MF_ERR_INVALID_ARG
    assert f(*args(d=80)) == mf.MF_ERR_UNSUPPORTED
    assert f(*args(dt=5)) == mf.MF_ERR_UNSUPPORTED
    assert f(*args(ws=need - 1)) == mf.MF_ERR_WORKSPACE
    m.num_block_rows = 5
    assert f(*args()) == mf.MF_ERR_INVALID_ARG


def test_paged_v_layout_round_trip():
    """The paged pool holds every token of every sequence at the slot its table says."""
    rng = np.random.default_rng(1)
    lens = [37, 0, 100, 16]
    c = cu(lens)
    v = rng.integers(0, 1 << 16, size=(3, int(c[-1]), 8), dtype=np.uint16)
    for P in (1, 7, 16, 64):
        pool, table = wlmod.paged_v(v, c, P, seed=P)
        for s, L in enumerate(lens):
            for j in range(L):
                pg = table[s, j // P]
                assert np.array_equal(pool[pg, :, j % P, :], v[:, c[s] + j, :])
        used = table[table >= 0]
        assert len(set(used.tolist())) == len(used) and used.max() < pool.shape[0]


def test_apply_paged_rejects_bad_arguments(lib):
    c = cu([100, 60])
    fake = ctypes.c_void_p(16)
    pc = c.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    m = mf.MfBsrMap(2, 32, 6, 160, 10, 8, 8, 8, 8, 8, 8, None, 0)
    f = lib.mf_apply_translated_paged
    ws = 1 << 40

    def call(pv, win=None, wdev=fake):
        wp = None
        if win is not None:
            arr = np.asarray(win, dtype=np.int32)
            call.keep = arr
            wp = arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        else:
            wdev = None
        return f(None, ctypes.byref(m), fake, 4, ctypes.byref(pv) if pv is not None else None, 2, 64, pc,
                 fake, 2, wp, wdev, 1, fake, fake, ws)

    good = mf.MfPagedV(16, 16, 20, 16, 8)
    assert call(None) == mf.MF_ERR_INVALID_ARG
    assert call(mf.MfPagedV(None, 16, 20, 16, 8)) == mf.MF_ERR_INVALID_ARG
    assert call(mf.MfPagedV(16, 0, 20, 16, 8)) == mf.MF_ERR_INVALID_ARG
    assert call(mf.MfPagedV(16, 16, 20, 16, 6)) == mf.MF_ERR_INVALID_ARG   # 100 > 6 * 16
    assert call(mf.MfPagedV(16, 16, 20, None, 8)) == mf.MF_ERR_INVALID_ARG
    assert call(good, [[0, 64], [32, 60]], None) == mf.MF_ERR_INVALID_ARG  # host without device copy
    assert call(good, [[16, 64], [0, 60]]) == mf.MF_ERR_INVALID_ARG         # begin not block-aligned
    assert call(good, [[0, 50], [0, 60]]) == mf.MF_ERR_INVALID_ARG          # end mid-block, not L
    assert call(good, [[0, 128], [0, 60]]) == mf.MF_ERR_INVALID_ARG         # end past L
    assert call(good, [[64, 32], [0, 60]]) == mf.MF_ERR_INVALID_ARG         # end before begin


def test_status_strings(lib):
    for s in range(6):
        assert lib.mf_status_string(s).decode() not in ("", "unknown status")
    assert lib.mf_status_string(99).decode() == "unknown status"


def test_apply_noalloc_rejects_before_touching_the_device(lib):
    """Invalid arguments and inputs whose workspace would exceed the fixed scratch
    are refused on the host (no device call is made on these paths)."""
    fake = ctypes.c_void_p(16)
    f = lib.mf_apply_translated_noalloc
    c = cu([100])
    pc = c.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    m = mf.MfBsrMap(2, 32, 4, 100, 10, 8, 8, 8, 8, 8, 8, None, 0)
    assert f(None, ctypes.byref(m), fake, 4, fake, 3, 64, pc, fake, 1, 1, fake) == mf.MF_ERR_INVALID_ARG
    assert f(None, ctypes.byref(m), fake, 4, fake, 2, 80, pc, fake, 1, 1, fake) == mf.MF_ERR_UNSUPPORTED
    assert f(None, None, fake, 4, fake, 2, 64, pc, fake, 1, 1, fake) == mf.MF_ERR_INVALID_ARG
    # the workspace of Hkv = 8, d = 128, B = 128 outgrows the scratch past 65408 tokens
    lim = mf.APPLY_NOALLOC_SCRATCH_BYTES
    for L, fits in ((65408, True), (65409, False), (32768 * 4, False)):
        c = cu([L])
        pc = c.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        assert (0 < mf.mf_apply_workspace_bytes(8, c, 128, 128) <= lim) == fits
        if not fits:
            m = mf.MfBsrMap(8, 128, (L + 127) // 128, L, 10, 8, 8, 8, 8, 8, 8, None, 0)
            assert f(None, ctypes.byref(m), fake, 8, fake, 8, 128, pc, fake, 1, 1, fake) == mf.MF_ERR_WORKSPACE
