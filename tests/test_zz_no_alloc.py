"""mf_apply_translated_noalloc (fixed per-GPU scratch, no allocation) against
mf_apply_translated (caller's workspace) through the C ABI: two calls in a
row, the second on a smaller input, so that scratch contents left by the first
call must not leak into the second.  Both run the same kernels on the same
inputs, so the outputs must agree bit for bit."""
import pytest
import torch

from cross_model_sparse_amd import mapflow as mf
from cross_model_sparse_amd import workloads as wlmod
from parity_util import gpu_compress, say, to_dev_v

pytestmark = pytest.mark.gpu


def _one(wl, dev, fmt):
    m, st, nnz = gpu_compress(wl, dev, tile_format=fmt)
    assert st == mf.MF_OK
    W = torch.from_numpy(wl.W).to(dev)
    v = to_dev_v(wl, dev)
    ref = mf.mf_apply_translated(m, W, v, wl.cu_seqlens)
    out = torch.full_like(ref, float("nan"))
    cu_dev = torch.from_numpy(wl.cu_seqlens).to(dev)
    got = mf.mf_apply_translated_noalloc(m, W, v, wl.cu_seqlens, out=out, cu_dev=cu_dev)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    need = mf.mf_apply_workspace_bytes(wl.spec.Hkv, wl.cu_seqlens, wl.spec.B, wl.spec.d)
    say(f"noalloc {wl.spec.name} lens={wl.lens} tiles={fmt} nnz={nnz} workspace={need} "
        f"of {mf.APPLY_NOALLOC_SCRATCH_BYTES}")
    assert torch.equal(got, ref)
    return need


@pytest.mark.parametrize("idx,big,small,kw,fmt", [
    (4, [2500, 900], [700, 130, 1], dict(Hs=8, Ht=16, Hkv=16), "bf16"),
    (3, [3000], [333, 0, 64], dict(Hs=6, Ht=8, Hkv=2), "bf16"),
    (5, [1500, 64, 900], [200, 65], dict(Hs=4, Ht=4, Hkv=4), "mxfp8"),
])
def test_noalloc_equals_workspace_entry_twice(gpu, idx, big, small, kw, fmt):
    n1 = _one(wlmod.small_variant(idx, big, **kw), gpu, fmt)
    n2 = _one(wlmod.small_variant(idx, small, **kw), gpu, fmt)
    assert n2 < n1


def test_noalloc_rejects_oversized_input(gpu):
    """A workspace beyond the fixed scratch is refused before any launch."""
    L = 65409
    m = mf.alloc_map(8, [0, L], 128, gpu, capacity=1)
    W = torch.zeros((8, 8), dtype=torch.float32, device=gpu)
    v = torch.zeros((8, L, 128), dtype=torch.bfloat16, device=gpu)
    with pytest.raises(mf.MapflowError) as e:
        mf.mf_apply_translated_noalloc(m, W, v, [0, L])
    assert e.value.status == mf.MF_ERR_WORKSPACE
