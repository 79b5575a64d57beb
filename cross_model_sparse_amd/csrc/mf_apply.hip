// Receiver-side fused retrieval with linear head translation (MapFlow,
// "Accelerating Cross-Model LLM Inference via Attention Map Reuse", §3.3 linear
// head mapping, §5.4 attention retrieval with a fused kernel):
//
//   O_t[i,:] = sum_h W[t,h] sum_{J kept by h} sum_{j in J} (A_h[i,j] / kmass_h[i]) V_g(t)[j,:]
//
// One work-group per (target head, query block); one wave per 32 query rows.
// Per key block J in the union of the sources' kept sets, each lane rebuilds its
// row of the translated tile  A~_t[i, J] = sum_h c_h[i] A_h[i, J]  in fp32
// registers straight from the bf16 tiles (c_h[i] = W[t,h] / kmass_h[i]),
// rounds it to bf16 and feeds it as the A operand of a 32x32x16 MFMA against
// V_g(t)[J] staged in LDS.  The translated map never leaves registers; nothing
// of size L x L is written.
//
// V is first copied into a transposed, block-padded layout Vt[g][d][NBR * B]
// (k_vtranspose) so that the MFMA B operand (8 consecutive keys of one value
// column) is one 16-byte read.  Padding columns are zero.
//
// Work-group order: the hardware hands consecutive work-groups to the 8 XCDs in
// turn; the id is decoded so that all targets of one query block run on one XCD
// and reuse its L2 copy of the source tiles, while the 8 XCDs work on 8 query
// blocks at once and share V through the memory-side cache.
#include "mf_host.hpp"

namespace mf {

constexpr int kXcds = 8;

// ---------------------------------------------------------------------------
// V [Hkv][T][D] -> Vt [Hkv][D][NBR * B], zero past each sequence end
// ---------------------------------------------------------------------------
template <int B, int D>
__global__ __launch_bounds__(256) void k_vtranspose(const uint16_t *__restrict__ v, int64_t T,
                                                    const RowInfo *__restrict__ rows, int32_t NBR,
                                                    uint16_t *__restrict__ vt) {
  constexpr int P = B + 8;  // LDS row pitch in elements
  __shared__ __attribute__((aligned(16))) uint16_t t[D * P];
  const int gr = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const RowInfo ri = rows[gr];
  const int nval = min(B, ri.len - ri.blk * B);
  const int64_t tok0 = (int64_t)ri.start + (int64_t)ri.blk * B;
  const uint16_t *src = v + ((int64_t)g * T + tok0) * D;
  for (int idx = tid; idx < B * D / 8; idx += 256) {
    const int j = idx / (D / 8), c = idx % (D / 8);
    u32x4 x = u32x4{0u, 0u, 0u, 0u};
    if (j < nval) x = *reinterpret_cast<const u32x4 *>(src + (int64_t)j * D + c * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      t[(c * 8 + 2 * e) * P + j] = (uint16_t)(x[e] & 0xffffu);
      t[(c * 8 + 2 * e + 1) * P + j] = (uint16_t)(x[e] >> 16);
    }
  }
  __syncthreads();
  const int64_t tpad = (int64_t)NBR * B;
  uint16_t *dst = vt + (int64_t)g * D * tpad + (int64_t)gr * B;
  for (int idx = tid; idx < D * B / 8; idx += 256) {
    const int d = idx / (B / 8), c = idx % (B / 8);
    *reinterpret_cast<u32x4 *>(dst + (int64_t)d * tpad + c * 8) =
        *reinterpret_cast<const u32x4 *>(&t[d * P + c * 8]);
  }
}

// ---------------------------------------------------------------------------
// k_apply
// ---------------------------------------------------------------------------
template <int B, int D>
struct ApplyCfg {
  static constexpr int NW = B / 32;
  static constexpr int NT = B * 2;
  static constexpr int VPITCH = B * 2 + kLdsPad;  // bytes per Vt row (one value column)
  static constexpr int VBYTES = D * VPITCH;
  static constexpr int CPR = B * 2 / 16;
  static constexpr int NCH = D * CPR / NT;
  static_assert(NCH * NT == D * CPR, "V tile chunks must divide evenly");
};

// LDS after the V tile: src[Hs] int, wt[Hs] float, rbase[Hs] int64, bm[Hs][nbw],
// pc[Hs][nbw], uni[nbw], coef[Hs][B], nsrc.
inline size_t apply_smem(int B, int D, int Hs, int nbw) {
  size_t s = (size_t)D * (B * 2 + kLdsPad);
  s += (size_t)Hs * (4 + 4 + 8);
  s += (size_t)Hs * nbw * 8 + (size_t)nbw * 4;
  s += (size_t)Hs * B * 4;
  s += 64;
  return s;
}

template <int B, int D>
__global__ __launch_bounds__(B * 2) void k_apply(
    const int64_t *__restrict__ row_ptr, const int32_t *__restrict__ col_idx,
    const uint16_t *__restrict__ tiles, const float *__restrict__ kept_mass, int32_t Hs,
    int32_t NBR, int64_t T, const float *__restrict__ W, int32_t Ht, int32_t grp,
    const uint16_t *__restrict__ vt, const RowInfo *__restrict__ rows,
    const int32_t *__restrict__ sched, int32_t nbw, int64_t capacity, int32_t renorm,
    float *__restrict__ o) {
  using C = ApplyCfg<B, D>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char *vlds = smem;
  int32_t *src = reinterpret_cast<int32_t *>(smem + C::VBYTES);
  float *wt = reinterpret_cast<float *>(src + Hs);
  int64_t *rbase = reinterpret_cast<int64_t *>(
      (reinterpret_cast<uintptr_t>(wt + Hs) + 7) & ~uintptr_t(7));
  uint32_t *bm = reinterpret_cast<uint32_t *>(rbase + Hs);
  int32_t *pc = reinterpret_cast<int32_t *>(bm + Hs * nbw);
  uint32_t *uni = reinterpret_cast<uint32_t *>(pc + Hs * nbw);
  float *coef = reinterpret_cast<float *>(uni + nbw);
  int32_t *nsrc_p = reinterpret_cast<int32_t *>(coef + Hs * B);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 31, hl = lane >> 5;
  const int x = blockIdx.x % kXcds, kx = blockIdx.x / kXcds;
  const int pos = (kx / Ht) * kXcds + x, t = kx % Ht;
  if (pos >= NBR) return;
  const int gr = sched[pos];
  const RowInfo ri = rows[gr];
  const int I = ri.blk, L = ri.len;
  const int n = I + 1;
  const int nw_row = (n + 31) / 32;
  const int g = t / grp;
  const int64_t tok0 = (int64_t)ri.start;
  const int64_t tpad = (int64_t)NBR * B;

  // sources with a nonzero weight, in head order
  if (tid == 0) {
    int ns = 0;
    for (int h = 0; h < Hs; ++h) {
      const float w = W[(int64_t)t * Hs + h];
      if (w != 0.f) {
        src[ns] = h;
        wt[ns] = w;
        rbase[ns] = row_ptr[(int64_t)h * NBR + gr];
        ++ns;
      }
    }
    *nsrc_p = ns;
  }
  for (int i = tid; i < Hs * nbw; i += C::NT) bm[i] = 0u;
  __syncthreads();
  const int ns = *nsrc_p;
  for (int q = 0; q < ns; ++q) {
    // entries past the capacity of an overflowed map are treated as missing
    const int64_t b = rbase[q], e = min(row_ptr[(int64_t)src[q] * NBR + gr + 1], capacity);
    for (int64_t idx = b + tid; idx < e; idx += C::NT) {
      const int J = col_idx[idx];
      atomicOr(&bm[q * nbw + (J >> 5)], 1u << (J & 31));
    }
  }
  for (int idx = tid; idx < ns * B; idx += C::NT) {
    const int q = idx / B, il = idx % B;
    const int ip = I * B + il;
    float c = 0.f;
    if (ip < L) {
      if (renorm) {
        const float km = kept_mass[(int64_t)src[q] * T + tok0 + ip];
        c = km > 0.f ? wt[q] / km : 0.f;
      } else {
        c = wt[q];
      }
    }
    coef[q * B + il] = c;
  }
  __syncthreads();
  for (int q = tid; q < ns; q += C::NT) {
    int run = 0;
    for (int w = 0; w < nw_row; ++w) {
      pc[q * nbw + w] = run;
      run += __popc(bm[q * nbw + w]);
    }
  }
  if (tid < nw_row) {
    uint32_t u = 0u;
    for (int q = 0; q < ns; ++q) u |= bm[q * nbw + tid];
    uni[tid] = u;
  }
  __syncthreads();

  // first key block of the union (uniform scan)
  auto next_J = [&](int from) -> int {
    for (int w = from >> 5; w < nw_row; ++w) {
      uint32_t bits = uni[w];
      if (w == (from >> 5)) bits &= ~((1u << (from & 31)) - 1u);
      if (bits) return w * 32 + __ffs(bits) - 1;
    }
    return -1;
  };

  const int i_loc = wave * 32 + m;
  f32x16 acc[D / 32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) acc[nb] = zero16();

  const uint16_t *vtg = vt + (int64_t)g * D * tpad;
  auto gload_v = [&](u32x4 (&stg)[C::NCH], int J) {
    const int64_t col0 = (int64_t)(gr - I + J) * B;  // block J of this sequence
#pragma unroll
    for (int c = 0; c < C::NCH; ++c) {
      const int idx = tid + c * C::NT;
      const int d = idx / C::CPR, cc = idx % C::CPR;
      stg[c] = *reinterpret_cast<const u32x4 *>(vtg + (int64_t)d * tpad + col0 + cc * 8);
    }
  };
  auto lstore_v = [&](const u32x4 (&stg)[C::NCH]) {
#pragma unroll
    for (int c = 0; c < C::NCH; ++c) {
      const int idx = tid + c * C::NT;
      const int d = idx / C::CPR, cc = idx % C::CPR;
      *reinterpret_cast<u32x4 *>(vlds + d * C::VPITCH + cc * 16) = stg[c];
    }
  };

  int J = next_J(0);
  u32x4 stg[C::NCH];
  if (J >= 0) {
    gload_v(stg, J);
    lstore_v(stg);
  }
  __syncthreads();
  while (J >= 0) {
    const int Jn = (J + 1 < n) ? next_J(J + 1) : -1;
    if (Jn >= 0) gload_v(stg, Jn);

    float mix[B / 2];
#pragma unroll
    for (int e = 0; e < B / 2; ++e) mix[e] = 0.f;
    const int jw = J >> 5;
    const uint32_t below = (1u << (J & 31)) - 1u;
    for (int q = 0; q < ns; ++q) {
      const uint32_t word = bm[q * nbw + jw];
      if (!((word >> (J & 31)) & 1u)) continue;
      const int64_t tix = rbase[q] + pc[q * nbw + jw] + __popc(word & below);
      if (tix >= capacity) continue;
      const uint16_t *tp = tiles + tix * (int64_t)(B * B) + (int64_t)i_loc * B + 16 * hl;
      const float c = coef[q * B + i_loc];
#pragma unroll
      for (int kc = 0; kc < B / 32; ++kc) {
        const u32x4 v0 = *reinterpret_cast<const u32x4 *>(tp + kc * 32);
        const u32x4 v1 = *reinterpret_cast<const u32x4 *>(tp + kc * 32 + 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          mix[kc * 16 + 2 * e] += c * bf16lo(v0[e]);
          mix[kc * 16 + 2 * e + 1] += c * bf16hi(v0[e]);
          mix[kc * 16 + 8 + 2 * e] += c * bf16lo(v1[e]);
          mix[kc * 16 + 8 + 2 * e + 1] += c * bf16hi(v1[e]);
        }
      }
    }
#pragma unroll
    for (int kc = 0; kc < B / 32; ++kc) {
      u32x4 a0, a1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a0[e] = pack_bf16x2(mix[kc * 16 + 2 * e], mix[kc * 16 + 2 * e + 1]);
        a1[e] = pack_bf16x2(mix[kc * 16 + 8 + 2 * e], mix[kc * 16 + 8 + 2 * e + 1]);
      }
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb) {
        const char *vp = vlds + (nb * 32 + m) * C::VPITCH + (kc * 32 + 16 * hl) * 2;
        const u32x4 b0 = *reinterpret_cast<const u32x4 *>(vp);
        const u32x4 b1 = *reinterpret_cast<const u32x4 *>(vp + 16);
        acc[nb] = mfma_bf16(as_bf16x8(a0), as_bf16x8(b0), acc[nb]);
        acc[nb] = mfma_bf16(as_bf16x8(a1), as_bf16x8(b1), acc[nb]);
      }
    }
    __syncthreads();
    if (Jn >= 0) lstore_v(stg);
    __syncthreads();
    J = Jn;
  }

  float *ot = o + (int64_t)t * T * D;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int il = wave * 32 + acc_row(r, lane);
    const int ip = I * B + il;
    if (ip < L) {
      float *dst = ot + (tok0 + ip) * D + m;
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb) dst[nb * 32] = acc[nb][r];
    }
  }
}

template <int B, int D>
static mf_status launch_apply(hipStream_t s, const mf_bsr_map *map, const float *W, int32_t Ht,
                              const void *v, int32_t Hkv, const SeqGeom &g, int32_t renorm,
                              float *o, void *ws, const VtWs &w) {
  const int nbw = (g.maxnb + 31) / 32 > 0 ? (g.maxnb + 31) / 32 : 1;
  const size_t smem = apply_smem(B, D, map->num_heads, nbw);
  if (smem > 160 * 1024) return MF_ERR_UNSUPPORTED;
  hipLaunchKernelGGL((k_vtranspose<B, D>), dim3(g.NBR, Hkv), dim3(256), 0, s,
                     reinterpret_cast<const uint16_t *>(v), g.T, at<RowInfo>(ws, w.rt.rows), g.NBR,
                     at<uint16_t>(ws, w.vt));
  if (hip_status() != MF_OK) return MF_ERR_HIP;
  if (smem > 64 * 1024)
    hipFuncSetAttribute(reinterpret_cast<const void *>(&k_apply<B, D>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  const int64_t npos = ((int64_t)g.NBR + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL((k_apply<B, D>), dim3((unsigned)(npos * Ht)), dim3(B * 2), smem, s,
                     map->row_ptr, map->col_idx, map->tiles, map->kept_mass, map->num_heads,
                     g.NBR, g.T, W, Ht, Ht / Hkv, at<uint16_t>(ws, w.vt),
                     at<RowInfo>(ws, w.rt.rows), at<int32_t>(ws, w.rt.sched), nbw, map->capacity_tiles, renorm, o);
  return hip_status();
}

}  // namespace mf

using namespace mf;

extern "C" size_t mf_apply_workspace_bytes(int32_t Hkv, const int32_t *cu, int32_t nseq, int32_t B,
                                           int32_t d) {
  SeqGeom g;
  if (Hkv <= 0 || !valid_dim(d) || seq_geom(cu, nseq, B, &g) != MF_OK) return 0;
  return vt_ws(g, Hkv, B, d).total;
}

extern "C" mf_status mf_apply_translated(void *stream, const mf_bsr_map *map, const float *W,
                                         int32_t Ht, const void *v, int32_t Hkv, int32_t d,
                                         const int32_t *cu_host, const int32_t *cu_dev,
                                         int32_t nseq, int32_t renorm, float *o, void *ws,
                                         size_t ws_bytes) {
  if (!map || !cu_host || !cu_dev || Ht <= 0 || Hkv <= 0 || Ht % Hkv != 0)
    return MF_ERR_INVALID_ARG;
  if (!valid_block(map->block)) return MF_ERR_INVALID_ARG;
  if (!valid_dim(d)) return MF_ERR_UNSUPPORTED;
  if (map->num_heads <= 0 || !W) return MF_ERR_INVALID_ARG;
  SeqGeom g;
  mf_status st = seq_geom(cu_host, nseq, map->block, &g);
  if (st != MF_OK) return st;
  if (g.NBR != map->num_block_rows || g.T != map->total_tokens) return MF_ERR_INVALID_ARG;
  if ((int64_t)g.NBR * Ht > INT32_MAX / 2) return MF_ERR_UNSUPPORTED;
  if (g.T > 0 && (!v || !o || !map->row_ptr || !map->col_idx || !map->tiles || !map->kept_mass))
    return MF_ERR_INVALID_ARG;
  const VtWs w = vt_ws(g, Hkv, map->block, d);
  if (!ws || ws_bytes < w.total) return MF_ERR_WORKSPACE;
  if (g.NBR == 0) return MF_OK;
  void *wsa = reinterpret_cast<void *>((reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if ((st = launch_rowtable(s, cu_dev, g, map->block, wsa, w.rt)) != MF_OK) return st;
  const int B = map->block;
  if (B == 32)
    return d == 64 ? launch_apply<32, 64>(s, map, W, Ht, v, Hkv, g, renorm, o, wsa, w)
                   : launch_apply<32, 128>(s, map, W, Ht, v, Hkv, g, renorm, o, wsa, w);
  if (B == 64)
    return d == 64 ? launch_apply<64, 64>(s, map, W, Ht, v, Hkv, g, renorm, o, wsa, w)
                   : launch_apply<64, 128>(s, map, W, Ht, v, Hkv, g, renorm, o, wsa, w);
  return d == 64 ? launch_apply<128, 64>(s, map, W, Ht, v, Hkv, g, renorm, o, wsa, w)
                 : launch_apply<128, 128>(s, map, W, Ht, v, Hkv, g, renorm, o, wsa, w);
}
