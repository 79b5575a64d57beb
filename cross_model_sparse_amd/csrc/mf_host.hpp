// Host-side helpers shared by the entry points: argument checks, sequence
// geometry, workspace layouts and the block-row table launch.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "mf_common.hpp"

namespace mf {

struct SeqGeom {
  int32_t nseq = 0;
  int64_t T = 0;        // total tokens
  int32_t NBR = 0;      // global block-rows
  int32_t maxnb = 0;    // most key blocks in one sequence
  int64_t tri = 0;      // sum_s nb_s (nb_s + 1) / 2  (causal blocks of one head)
};

inline bool valid_block(int32_t B) { return B == 32 || B == 64 || B == 128; }
inline bool valid_dim(int32_t d) { return d == 64 || d == 128; }
inline bool valid_tile_format(int32_t f) { return f == MF_TILE_BF16 || f == MF_TILE_MXFP8; }

// Bytes of one stored tile (codes, then one scale byte per 32 keys of a row, for
// the block-scaled fp8 format).
constexpr int64_t tile_bytes(int B, int fmt) {
  return fmt == MF_TILE_MXFP8 ? (int64_t)B * B + (int64_t)B * (B / 32) : (int64_t)B * B * 2;
}

// Validates host offsets and fills the geometry for blocks of B tokens (any
// B > 0; the caller checks that B suits its kernels). MF_ERR_UNSUPPORTED for
// too many blocks in one sequence.
inline mf_status seq_geom_blocks(const int32_t *cu, int32_t nseq, int32_t B, SeqGeom *g) {
  if (nseq < 0 || !cu || B <= 0) return MF_ERR_INVALID_ARG;
  if (cu[0] != 0) return MF_ERR_INVALID_ARG;
  SeqGeom r;
  r.nseq = nseq;
  int64_t nbr = 0;
  for (int32_t s = 0; s < nseq; ++s) {
    int64_t L = (int64_t)cu[s + 1] - (int64_t)cu[s];
    if (L < 0) return MF_ERR_INVALID_ARG;
    int64_t nb = (L + B - 1) / B;
    if (nb > kMaxNB) return MF_ERR_UNSUPPORTED;
    nbr += nb;
    r.tri += nb * (nb + 1) / 2;
    if (nb > r.maxnb) r.maxnb = (int32_t)nb;
  }
  if (nbr > INT32_MAX / 2) return MF_ERR_UNSUPPORTED;
  r.NBR = (int32_t)nbr;
  r.T = cu[nseq];
  *g = r;
  return MF_OK;
}

// The same for a map's block size B (32, 64 or 128).
inline mf_status seq_geom(const int32_t *cu, int32_t nseq, int32_t B, SeqGeom *g) {
  if (nseq < 0 || !cu) return MF_ERR_INVALID_ARG;
  if (!valid_block(B)) return MF_ERR_UNSUPPORTED;
  return seq_geom_blocks(cu, nseq, B, g);
}

struct BiasArgs {
  int32_t sink_n;
  float sink2;     // sink offset in log2 units
  int32_t local_w;
  float local2;    // local offset in log2 units
};

inline BiasArgs bias_args(const mf_logit_bias *b) {
  BiasArgs a{0, 0.f, 0, 0.f};
  if (b) {
    a.sink_n = b->sink_n > 0 ? b->sink_n : 0;
    a.sink2 = b->sink_bias * kLog2e;
    a.local_w = b->local_w > 0 ? b->local_w : 0;
    a.local2 = b->local_bias * kLog2e;
  }
  return a;
}

inline bool bias_ok(const mf_logit_bias *b) {
  if (!b) return true;
  return isfinite(b->sink_bias) && isfinite(b->local_bias) && b->sink_n >= 0 && b->local_w >= 0;
}

// Block-row table in the workspace (built on the device from cu_seqlens_dev).
struct RowTable {
  size_t rows, sched, pbase, nbcum;
};

inline RowTable carve_rows(Carve &c, const SeqGeom &g) {
  RowTable t;
  t.rows = c.take<RowInfo>(g.NBR > 0 ? g.NBR : 1);
  t.sched = c.take<int32_t>(g.NBR > 0 ? g.NBR : 1);
  t.pbase = c.take<int64_t>(g.NBR > 0 ? g.NBR : 1);
  t.nbcum = c.take<int32_t>(g.nseq + 1);
  return t;
}

// Compress workspace layout.
struct CompressWs {
  RowTable rt;
  size_t lse2, partials, counts, bitmaps;
  int32_t nbw;
  size_t total;
};

inline CompressWs compress_ws(const SeqGeom &g, int32_t Hs, int32_t B) {
  Carve c;
  CompressWs w;
  w.rt = carve_rows(c, g);
  w.lse2 = c.take<float>((size_t)Hs * (g.T > 0 ? g.T : 1));
  w.partials = c.take<float>((size_t)Hs * (size_t)B * (size_t)(g.tri > 0 ? g.tri : 1));
  w.counts = c.take<int32_t>((size_t)Hs * (g.NBR > 0 ? g.NBR : 1));
  w.nbw = (g.maxnb + 31) / 32;
  if (w.nbw < 1) w.nbw = 1;
  w.bitmaps = c.take<uint32_t>((size_t)Hs * (g.NBR > 0 ? g.NBR : 1) * w.nbw);
  w.total = c.off + 256;
  return w;
}

// Apply / dense workspace: row table + transposed, block-padded V + the
// schedule of a query window.
struct VtWs {
  RowTable rt;
  size_t vt, wsched, gtab, psched, vzero;
  size_t total;
};

// Zero block of the apply workspace: at least one tile of the largest format
// (B = 128 bf16) and one V row.
constexpr int kZeroBytes = 32 * 1024;

// Target-group table of the apply path: a count, then up to 1024 groups of at
// most 4 targets.
constexpr int kGroupTableInts = 1 + 4 * 1024;

inline VtWs vt_ws(const SeqGeom &g, int32_t Hkv, int32_t B, int32_t d) {
  Carve c;
  VtWs w;
  w.rt = carve_rows(c, g);
  w.vt = c.take<uint16_t>((size_t)Hkv * d * (size_t)(g.NBR > 0 ? g.NBR : 1) * B);
  w.wsched = c.take<int32_t>(g.NBR > 0 ? g.NBR : 1);
  w.gtab = c.take<int32_t>(kGroupTableInts);
  w.psched = c.take<int32_t>(2 * (size_t)(g.NBR > 0 ? g.NBR : 1));
  w.vzero = c.take<char>(kZeroBytes);  // zeros: a V row past a sequence's end, a missing tile
  w.total = c.off + 256;
  return w;
}

template <typename T>
inline T *at(void *base, size_t off) {
  return reinterpret_cast<T *>(static_cast<char *>(base) + off);
}

inline mf_status hip_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? MF_OK : MF_ERR_HIP;
}

// Launches the block-row table build (defined in mf_rows.hip).
mf_status launch_rowtable(hipStream_t s, const int32_t *cu_dev, const SeqGeom &g, int32_t B,
                          void *ws, const RowTable &rt);

}  // namespace mf
