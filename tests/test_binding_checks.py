"""The Python binding rejects tensors whose shapes disagree with cu_seqlens or
with each other before any native call is made: every kernel takes
cu_seqlens[-1] as the token count (and head stride) of its [H, T, d] tensors,
so a mismatch would otherwise read or write at the wrong offsets.  CPU tensors
suffice: the checks run before the first device call."""
import numpy as np
import pytest
import torch

from cross_model_sparse_amd import mapflow as mf


@pytest.fixture(scope="module", autouse=True)
def lib():
    import os
    if not os.path.exists(mf.LIB_PATH):
        from cross_model_sparse_amd import build
        build.build()
    return mf.load()


def cu(lens):
    c = np.zeros(len(lens) + 1, dtype=np.int32)
    c[1:] = np.cumsum(lens)
    return c


C = cu([100, 60])  # T = 160
B = 32


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def test_compress_token_axis():
    with pytest.raises(ValueError, match="cu_seqlens"):
        mf.mf_compress_topp(bf(2, 150, 64), bf(2, 150, 64), C, B, 0.9)
    with pytest.raises(ValueError):
        mf.mf_compress_topp(bf(2, 160, 64), bf(2, 161, 64), C, B, 0.9)
    with pytest.raises(ValueError):
        mf.mf_compress_topp(bf(160, 64), bf(160, 64), C, B, 0.9)


def test_prefix_dedupe_token_axis():
    with pytest.raises(ValueError, match="cu_seqlens"):
        mf.mf_prefix_dedupe(bf(2, 170, 64), bf(2, 170, 64), C, B)


def test_apply_shapes():
    m = mf.alloc_map(2, C, B, "cpu", capacity=8)
    W = f32(4, 2)
    with pytest.raises(ValueError, match="cu_seqlens"):
        mf.mf_apply_translated(m, W, bf(2, 159, 64), C)
    with pytest.raises(ValueError, match="out must be"):
        mf.mf_apply_translated(m, W, bf(2, 160, 64), C, out=f32(4, 160, 32))
    with pytest.raises(ValueError, match="out must be"):
        mf.mf_apply_translated(m, W, bf(2, 160, 64), C, out=f32(3, 160, 64))
    with pytest.raises(ValueError, match="out must be"):
        mf.mf_apply_translated(m, W, bf(2, 160, 64), C, out=bf(4, 160, 64))
    with pytest.raises(ValueError, match="out must be"):
        mf.mf_apply_translated(m, W, bf(2, 160, 64), C, out=f32(4, 64, 160).transpose(1, 2))
    with pytest.raises(ValueError, match="W must be"):
        mf.mf_apply_translated(m, f32(4, 3), bf(2, 160, 64), C)
    with pytest.raises(ValueError, match="W must be"):
        mf.mf_apply_translated(m, f32(4, 2, 1), bf(2, 160, 64), C)


def test_apply_paged_out_shape():
    m = mf.alloc_map(2, C, B, "cpu", capacity=8)
    pages = bf(20, 2, 16, 64)
    table = torch.zeros((2, 8), dtype=torch.int32)
    with pytest.raises(ValueError, match="out must be"):
        mf.mf_apply_translated_paged(m, f32(4, 2), pages, table, C, out=f32(4, 150, 64))


def test_tv_distance_shapes():
    m = mf.alloc_map(2, C, B, "cpu", capacity=8)
    with pytest.raises(ValueError, match="cu_seqlens"):
        mf.mf_tv_distance(m, f32(4, 2), bf(4, 150, 64), bf(2, 150, 64), C)
    with pytest.raises(ValueError, match="out must be"):
        mf.mf_tv_distance(m, f32(4, 2), bf(4, 160, 64), bf(2, 160, 64), C, out=f32(4, 161))


def test_dense_shapes():
    with pytest.raises(ValueError, match="cu_seqlens"):
        mf.mf_dense_ref_attention(bf(4, 150, 64), bf(2, 150, 64), bf(2, 150, 64), C)
    with pytest.raises(ValueError, match="k and v"):
        mf.mf_dense_ref_attention(bf(4, 160, 64), bf(2, 160, 64), bf(2, 159, 64), C)
    with pytest.raises(ValueError, match="out must be"):
        mf.mf_dense_ref_attention(bf(4, 160, 64), bf(2, 160, 64), bf(2, 160, 64), C, out=f32(2, 160, 64))
