"""Attention-map reuse on MI355X: block top-p compression of attention maps into
BSR tiles and fused translated retrieval, as hand-written HIP kernels behind a
C ABI (include/mapflow.h).

Submodules:
  mapflow    ctypes binding of libmapflow.so (mf_compress_topp, mf_apply_translated,
             mf_dense_ref_attention, size queries, status)
  workloads  seeded synthetic inputs
  build      hipcc build of libmapflow.so

Importing the package loads nothing; the binding loads the library on first use.
"""
