// Sender-side block top-p compression into BSR (MapFlow, "Accelerating
// Cross-Model LLM Inference via Attention Map Reuse", §4 top-p compression into
// Block Sparse Row form, §5.2 Attention State Compressor).
//
// Three kernels per call (after the block-row table):
//   k_select   one work-group per (source head, query block): streams the key
//              blocks of the causal row through LDS, computes S^T tiles on
//              MFMA, and stores per (query row, key block) the block-local
//              log2-sum-exp.  From those partials it forms the row normaliser,
//              every block's probability mass, sorts the masses (descending,
//              lower block first on ties), cuts at p of the row total with fp64
//              prefix sums, and writes the kept bitmap, kept count and each
//              row's kept mass.  One pass over Q K^T instead of separate
//              normaliser and mass passes.
//   k_offsets  exclusive scan of kept counts -> row_ptr, nnz, capacity status.
//   k_tiles    one work-group per (source head, query block): recomputes only
//              the kept tiles, rounds exp2(x - lse2) to bf16 (nearest even),
//              reorders them through LDS into fragment order (see mf_bsr_map)
//              and writes each tile with coalesced 16-byte stores, plus col_idx.
#include <type_traits>

#include "mf_host.hpp"
#include "mf_qk.hpp"

namespace mf {

// ---------------------------------------------------------------------------
// k_select
// ---------------------------------------------------------------------------
template <int B, int D, bool F32>
struct SelectCfg {
  using C = QKCfg<B, D, F32>;
  // epilogue arrays reuse the K staging buffer once the key loop is done
  static constexpr int OFF_KEYS = C::NW * kMaxNB * 4;        // after msum[NW][kMaxNB]
  static constexpr int OFF_TSUM = OFF_KEYS + kMaxNB * 8;     // keys[kMaxNB]
  static constexpr int OFF_BM = OFF_TSUM + (C::NT + 1) * 8;  // tsum[NT + 1]
  static constexpr int OFF_KC = OFF_BM + 32 * 4;             // bm[32]
  static constexpr int EPI = OFF_KC + 16;
  static constexpr int SMEM = C::KBYTES > EPI ? C::KBYTES : EPI;
};

template <int B, int D, bool F32>
__global__ __launch_bounds__(B * 2) __attribute__((amdgpu_waves_per_eu(F32 ? 1 : 2))) void k_select(
    const void *__restrict__ qv, const void *__restrict__ kv, int64_t T, int32_t Hs, int32_t NBR,
    const RowInfo *__restrict__ rows, const int32_t *__restrict__ sched,
    const int64_t *__restrict__ pbase, int64_t ptot, float scale2, BiasArgs bias, double p,
    float *__restrict__ lse2_out, float *__restrict__ partials, int32_t *__restrict__ counts,
    uint32_t *__restrict__ bitmaps, int32_t nbw, float *__restrict__ kept_mass) {
  using C = QKCfg<B, D, F32>;
  using E = std::conditional_t<F32, float, uint16_t>;
  __shared__ __attribute__((aligned(16))) char smem[SelectCfg<B, D, F32>::SMEM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 31, hl = lane >> 5;
  const int pos = blockIdx.x / Hs, h = blockIdx.x % Hs;
  const int gr = sched[pos];
  const RowInfo ri = rows[gr];
  const int I = ri.blk, L = ri.len;
  const int i_loc = wave * 32 + m;
  const int i_pos = I * B + i_loc;
  const bool rvalid = i_pos < L;
  const int64_t tok0 = (int64_t)ri.start;

  const E *qh = reinterpret_cast<const E *>(qv) + (int64_t)h * T * D;
  const char *kh = reinterpret_cast<const char *>(kv) + (int64_t)h * T * D * C::ESZ;
  float *part = partials + (int64_t)h * ptot + pbase[gr];

  QOp<D, F32> qo;
  load_q<D>(qo, rvalid ? qh + (tok0 + i_pos) * D : nullptr, hl);

  u32x4 stg[C::NCH];
  gload_tile<B, D, F32>(stg, kh, tok0, min(B, L), tid);
  lstore_tile<B, D, F32>(smem, stg, tid);
  __syncthreads();

  float m_run = -INFINITY;
  for (int J = 0; J <= I; ++J) {
    if (J < I) gload_tile<B, D, F32>(stg, kh, tok0 + (int64_t)(J + 1) * B, min(B, L - (J + 1) * B), tid);
    f32x16 acc[B / 32];
    st_tile<B, D>(acc, smem, qo, lane);
    const bool plain = plain_tile(I, J, B, bias.sink_n, bias.sink2, bias.local_w, bias.local2);
    float mx = logits_inplace<B>(acc, plain, rvalid, i_pos, J * B, scale2, bias.sink_n,
                                 bias.sink2, bias.local_w, bias.local2, lane);
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    float sum = 0.f;
    if (mx != -INFINITY) sum = lane_expsum<B>(acc, mx);
    sum += __shfl_xor(sum, 32, kWave);
    const float lse = (mx == -INFINITY) ? -INFINITY : mx + fast_log2(sum);
    if (hl == 0) part[(int64_t)J * B + i_loc] = lse;
    m_run = fmaxf(m_run, lse);
    __syncthreads();
    if (J < I) lstore_tile<B, D, F32>(smem, stg, tid);
    __syncthreads();
  }

  // ---- epilogue: row normaliser, block masses, top-p cut, kept mass --------
  using SC = SelectCfg<B, D, F32>;
  float *msum = reinterpret_cast<float *>(smem);
  uint64_t *keys = reinterpret_cast<uint64_t *>(smem + SC::OFF_KEYS);
  double *tsum = reinterpret_cast<double *>(smem + SC::OFF_TSUM);
  uint32_t *bm = reinterpret_cast<uint32_t *>(smem + SC::OFF_BM);
  int *kcount = reinterpret_cast<int *>(smem + SC::OFF_KC);
  const int n = I + 1;

  // row normaliser lse2_i = m_run + log2(sum_J exp2(part - m_run)), fp64 sum
  double zs = 0.0;
  if (rvalid)
    for (int J = hl; J < n; J += 2) zs += (double)fast_exp2(part[(int64_t)J * B + i_loc] - m_run);
  zs += __shfl_xor(zs, 32, kWave);
  const float lse2 = rvalid ? m_run + fast_log2((float)zs) : 0.f;

  // block masses: per wave over its 32 rows, two key blocks at a time
  for (int J0 = 0; J0 < n; J0 += 2) {
    const int J = J0 + hl;
    float v = 0.f;
    if (rvalid && J < n) v = fast_exp2(part[(int64_t)J * B + i_loc] - lse2);
    v = half_sum(v);
    if (m == 0 && J < n) msum[wave * kMaxNB + J] = v;
  }
  if (tid < 32) bm[tid] = 0u;
  if (tid == 0) *kcount = 0;
  __syncthreads();

  int N = 1;
  while (N < n) N <<= 1;
  for (int J = tid; J < N; J += C::NT) {
    uint64_t key = 0;
    if (J < n) {
      float M = msum[J];
#pragma unroll
      for (int w = 1; w < C::NW; ++w) M += msum[w * kMaxNB + J];
      key = ((uint64_t)__float_as_uint(M) << 32) | (uint64_t)(0xffffffffu - (uint32_t)J);
    }
    keys[J] = key;
  }
  __syncthreads();
  // bitonic sort, descending by (mass, -index)
  for (int kk = 2; kk <= N; kk <<= 1) {
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      for (int idx = tid; idx < N; idx += C::NT) {
        const int ixj = idx ^ jj;
        if (ixj > idx) {
          const uint64_t a = keys[idx], b = keys[ixj];
          const bool desc = (idx & kk) == 0;
          if (desc ? (a < b) : (a > b)) {
            keys[idx] = b;
            keys[ixj] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  // fp64 prefix sums in sorted order; count prefixes below the threshold
  const int per = (n + C::NT - 1) / C::NT;
  const int c0 = min(n, tid * per), c1 = min(n, c0 + per);
  double loc = 0.0;
  for (int c = c0; c < c1; ++c) loc += (double)__uint_as_float((uint32_t)(keys[c] >> 32));
  tsum[tid] = loc;
  __syncthreads();
  if (tid == 0) {
    double run = 0.0;
    for (int t = 0; t < C::NT; ++t) {
      const double x = tsum[t];
      tsum[t] = run;
      run += x;
    }
    tsum[C::NT] = run;
  }
  __syncthreads();
  const double total = tsum[C::NT];
  const double target = p * total;
  int below = 0;
  double run = tsum[tid];
  for (int c = c0; c < c1; ++c) {
    run += (double)__uint_as_float((uint32_t)(keys[c] >> 32));
    below += (run < target) ? 1 : 0;
  }
  if (below) atomicAdd(kcount, below);
  __syncthreads();
  const int kstar = (p >= 1.0) ? n : min(n, *kcount + 1);
  for (int c = tid; c < kstar; c += C::NT) {
    const uint32_t J = 0xffffffffu - (uint32_t)(keys[c] & 0xffffffffu);
    atomicOr(&bm[J >> 5], 1u << (J & 31));
  }
  __syncthreads();
  const int64_t r = (int64_t)h * NBR + gr;
  for (int w = tid; w < nbw; w += C::NT) bitmaps[r * nbw + w] = (w < 32) ? bm[w] : 0u;
  if (tid == 0) counts[r] = kstar;

  // kept mass per row, fp64 over kept blocks in ascending order per lane half
  double ks = 0.0;
  if (rvalid)
    for (int J = hl; J < n; J += 2)
      if ((bm[J >> 5] >> (J & 31)) & 1u) ks += (double)fast_exp2(part[(int64_t)J * B + i_loc] - lse2);
  ks += __shfl_xor(ks, 32, kWave);
  if (rvalid && hl == 0) {
    kept_mass[(int64_t)h * T + tok0 + i_pos] = (float)ks;
    lse2_out[(int64_t)h * T + tok0 + i_pos] = lse2;
  }
}

// ---------------------------------------------------------------------------
// k_offsets: row_ptr = exclusive scan of counts, nnz, status
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_offsets(const int32_t *__restrict__ counts, int64_t R,
                                                  int64_t capacity, int64_t *__restrict__ row_ptr,
                                                  int64_t *__restrict__ nnz,
                                                  int32_t *__restrict__ status) {
  __shared__ int64_t ts[1024];
  const int tid = threadIdx.x, nt = blockDim.x;
  const int64_t per = (R + nt - 1) / nt;
  const int64_t a = min(R, (int64_t)tid * per), b = min(R, a + per);
  int64_t s = 0;
  for (int64_t i = a; i < b; ++i) s += counts[i];
  ts[tid] = s;
  __syncthreads();
  if (tid == 0) {
    int64_t run = 0;
    for (int i = 0; i < nt; ++i) {
      const int64_t x = ts[i];
      ts[i] = run;
      run += x;
    }
    row_ptr[R] = run;
    *nnz = run;
    *status = run > capacity ? (int32_t)MF_ERR_CAPACITY : (int32_t)MF_OK;
  }
  __syncthreads();
  int64_t run = ts[tid];
  for (int64_t i = a; i < b; ++i) {
    row_ptr[i] = run;
    run += counts[i];
  }
}

// ---------------------------------------------------------------------------
// k_tiles
// ---------------------------------------------------------------------------
template <int B, int D, bool F32>
struct TilesCfg {
  using C = QKCfg<B, D, F32>;
  static constexpr int TPITCH = B * 2 + kLdsPad;   // bf16 tile row pitch in LDS
  static constexpr int TBYTES = B * TPITCH;
  static constexpr int LIST = kMaxNB * 4 + 64 * 4;
  static constexpr int SMEM = C::KBYTES + TBYTES + LIST;
  static constexpr int TCH = B * B * 2 / 16 / C::NT;  // 16-byte tile chunks per thread
};

template <int B, int D, bool F32>
__global__ __launch_bounds__(B * 2) __attribute__((amdgpu_waves_per_eu(F32 ? 1 : 2))) void k_tiles(
    const void *__restrict__ qv, const void *__restrict__ kv, int64_t T, int32_t Hs, int32_t NBR,
    const RowInfo *__restrict__ rows, const int32_t *__restrict__ sched, float scale2,
    BiasArgs bias, const float *__restrict__ lse2_in, const uint32_t *__restrict__ bitmaps,
    int32_t nbw, const int64_t *__restrict__ row_ptr, int64_t capacity,
    int32_t *__restrict__ col_idx, uint16_t *__restrict__ tiles) {
  using C = QKCfg<B, D, F32>;
  using TC = TilesCfg<B, D, F32>;
  using E = std::conditional_t<F32, float, uint16_t>;
  __shared__ __attribute__((aligned(16))) char smem[TC::SMEM];
  char *klds = smem;
  char *tlds = smem + C::KBYTES;
  int32_t *list = reinterpret_cast<int32_t *>(smem + C::KBYTES + TC::TBYTES);
  int32_t *woff = list + kMaxNB;  // [33] word offsets

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 31, hl = lane >> 5;
  const int pos = blockIdx.x / Hs, h = blockIdx.x % Hs;
  const int gr = sched[pos];
  const RowInfo ri = rows[gr];
  const int I = ri.blk, L = ri.len;
  const int n = I + 1;
  const int i_loc = wave * 32 + m;
  const int i_pos = I * B + i_loc;
  const bool rvalid = i_pos < L;
  const int64_t tok0 = (int64_t)ri.start;
  const int64_t r = (int64_t)h * NBR + gr;
  const int nw_row = (n + 31) / 32;

  // kept list, ascending
  if (tid == 0) {
    int run = 0;
    for (int w = 0; w < nw_row; ++w) {
      woff[w] = run;
      run += __popc(bitmaps[r * nbw + w]);
    }
    woff[nw_row] = run;
  }
  __syncthreads();
  for (int w = tid; w < nw_row; w += C::NT) {
    uint32_t bits = bitmaps[r * nbw + w];
    int o = woff[w];
    while (bits) {
      const int b = __ffs(bits) - 1;
      list[o++] = w * 32 + b;
      bits &= bits - 1;
    }
  }
  __syncthreads();
  const int cnt = woff[nw_row];
  const int64_t base = row_ptr[r];
  for (int c = tid; c < cnt; c += C::NT)
    if (base + c < capacity) col_idx[base + c] = list[c];
  if (cnt == 0) return;

  const E *qh = reinterpret_cast<const E *>(qv) + (int64_t)h * T * D;
  const char *kh = reinterpret_cast<const char *>(kv) + (int64_t)h * T * D * C::ESZ;
  QOp<D, F32> qo;
  load_q<D>(qo, rvalid ? qh + (tok0 + i_pos) * D : nullptr, hl);
  const float lse2 = rvalid ? lse2_in[(int64_t)h * T + tok0 + i_pos] : 0.f;

  u32x4 stg[C::NCH];
  {
    const int J = list[0];
    gload_tile<B, D, F32>(stg, kh, tok0 + (int64_t)J * B, min(B, L - J * B), tid);
    lstore_tile<B, D, F32>(klds, stg, tid);
  }
  __syncthreads();
  for (int c = 0; c < cnt; ++c) {
    const int J = list[c];
    if (c + 1 < cnt) {
      const int Jn = list[c + 1];
      gload_tile<B, D, F32>(stg, kh, tok0 + (int64_t)Jn * B, min(B, L - Jn * B), tid);
    }
    f32x16 acc[B / 32];
    st_tile<B, D>(acc, klds, qo, lane);
    const bool plain = plain_tile(I, J, B, bias.sink_n, bias.sink2, bias.local_w, bias.local2);
    logits_inplace<B>(acc, plain, rvalid, i_pos, J * B, scale2, bias.sink_n, bias.sink2,
                      bias.local_w, bias.local2, lane);
    // probabilities -> bf16, written transposed into the LDS tile [i][j]
#pragma unroll
    for (int mb = 0; mb < B / 32; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float pv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pv[e] = rvalid ? fast_exp2(acc[mb][4 * g + e] - lse2) : 0.f;
        uint2 w;
        w.x = pack_bf16x2(pv[0], pv[1]);
        w.y = pack_bf16x2(pv[2], pv[3]);
        const int j_loc = mb * 32 + 8 * g + 4 * hl;
        *reinterpret_cast<uint2 *>(tlds + i_loc * TC::TPITCH + j_loc * 2) = w;
      }
    __syncthreads();
    if (c + 1 < cnt) lstore_tile<B, D, F32>(klds, stg, tid);
    if (base + c < capacity) {
      char *dst = reinterpret_cast<char *>(tiles + (base + c) * (int64_t)B * B);
#pragma unroll
      for (int k = 0; k < TC::TCH; ++k) {
        // fragment order: 16-byte chunk q = (row group * KC + key chunk) * 64 + f
        // holds row 16 * group + f % 16, keys 32 * chunk + 8 * (f / 16) .. + 8
        const int q = tid + k * C::NT;
        const int blk = q >> 6, f = q & 63;
        const int rr = (blk / (B / 32)) * 16 + (f & 15);
        const int c0 = (blk % (B / 32)) * 32 + 8 * (f >> 4);
        *reinterpret_cast<u32x4 *>(dst + q * 16) =
            *reinterpret_cast<const u32x4 *>(tlds + rr * TC::TPITCH + c0 * 2);
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// host dispatch
// ---------------------------------------------------------------------------
template <int B, int D, bool F32>
static mf_status launch_compress(hipStream_t s, const void *q, const void *k, const SeqGeom &g,
                                 int32_t Hs, double p, const BiasArgs &ba, mf_bsr_map *map,
                                 void *ws, const CompressWs &w) {
  const float scale2 = kLog2e / sqrtf((float)D);
  const int64_t ptot = (int64_t)B * g.tri;
  const dim3 grid((unsigned)((int64_t)g.NBR * Hs));
  hipLaunchKernelGGL((k_select<B, D, F32>), grid, dim3(B * 2), 0, s, q, k, g.T, Hs, g.NBR,
                     at<RowInfo>(ws, w.rt.rows), at<int32_t>(ws, w.rt.sched),
                     at<int64_t>(ws, w.rt.pbase), ptot, scale2, ba, p, at<float>(ws, w.lse2),
                     at<float>(ws, w.partials), at<int32_t>(ws, w.counts),
                     at<uint32_t>(ws, w.bitmaps), w.nbw, map->kept_mass);
  if (hip_status() != MF_OK) return MF_ERR_HIP;
  hipLaunchKernelGGL(k_offsets, dim3(1), dim3(1024), 0, s, at<int32_t>(ws, w.counts),
                     (int64_t)Hs * g.NBR, map->capacity_tiles, map->row_ptr, map->nnz,
                     map->status);
  if (hip_status() != MF_OK) return MF_ERR_HIP;
  hipLaunchKernelGGL((k_tiles<B, D, F32>), grid, dim3(B * 2), 0, s, q, k, g.T, Hs, g.NBR,
                     at<RowInfo>(ws, w.rt.rows), at<int32_t>(ws, w.rt.sched), scale2, ba,
                     at<float>(ws, w.lse2), at<uint32_t>(ws, w.bitmaps), w.nbw, map->row_ptr,
                     map->capacity_tiles, map->col_idx, map->tiles);
  return hip_status();
}

template <int B>
static mf_status dispatch_d(int32_t d, bool f32, hipStream_t s, const void *q, const void *k,
                            const SeqGeom &g, int32_t Hs, double p, const BiasArgs &ba,
                            mf_bsr_map *map, void *ws, const CompressWs &w) {
  if (d == 64)
    return f32 ? launch_compress<B, 64, true>(s, q, k, g, Hs, p, ba, map, ws, w)
               : launch_compress<B, 64, false>(s, q, k, g, Hs, p, ba, map, ws, w);
  return f32 ? launch_compress<B, 128, true>(s, q, k, g, Hs, p, ba, map, ws, w)
             : launch_compress<B, 128, false>(s, q, k, g, Hs, p, ba, map, ws, w);
}

}  // namespace mf

using namespace mf;

extern "C" int32_t mf_num_block_rows(const int32_t *cu, int32_t nseq, int32_t B) {
  SeqGeom g;
  if (seq_geom(cu, nseq, B, &g) != MF_OK) return -1;
  return g.NBR;
}

extern "C" int64_t mf_compress_max_tiles(int32_t Hs, const int32_t *cu, int32_t nseq, int32_t B) {
  SeqGeom g;
  if (Hs <= 0 || seq_geom(cu, nseq, B, &g) != MF_OK) return -1;
  return (int64_t)Hs * g.tri;
}

extern "C" size_t mf_compress_workspace_bytes(int32_t Hs, const int32_t *cu, int32_t nseq,
                                              int32_t B, int32_t d) {
  SeqGeom g;
  if (Hs <= 0 || !valid_dim(d) || seq_geom(cu, nseq, B, &g) != MF_OK) return 0;
  return compress_ws(g, Hs, B).total;
}

extern "C" mf_status mf_compress_topp(void *stream, const void *q, const void *k,
                                      mf_dtype qk_dtype, const int32_t *cu_host,
                                      const int32_t *cu_dev, int32_t nseq, int32_t Hs, int32_t d,
                                      int32_t B, double p, const mf_logit_bias *bias,
                                      mf_bsr_map *map, void *ws, size_t ws_bytes) {
  if (!map || !cu_host || !cu_dev || Hs <= 0 || !(p > 0.0 && p <= 1.0) || !bias_ok(bias))
    return MF_ERR_INVALID_ARG;
  if (qk_dtype != MF_BF16 && qk_dtype != MF_FP32) return MF_ERR_UNSUPPORTED;
  if (!valid_dim(d)) return MF_ERR_UNSUPPORTED;
  SeqGeom g;
  mf_status st = seq_geom(cu_host, nseq, B, &g);
  if (st != MF_OK) return st;
  if ((int64_t)Hs * g.NBR > INT32_MAX) return MF_ERR_UNSUPPORTED;
  if (map->capacity_tiles < 0 || !map->row_ptr || !map->nnz || !map->status) return MF_ERR_INVALID_ARG;
  if (g.T > 0 && (!q || !k || !map->kept_mass)) return MF_ERR_INVALID_ARG;
  if (map->capacity_tiles > 0 && (!map->col_idx || !map->tiles)) return MF_ERR_INVALID_ARG;
  const CompressWs w = compress_ws(g, Hs, B);
  if (!ws || ws_bytes < w.total) return MF_ERR_WORKSPACE;
  void *wsa = reinterpret_cast<void *>((reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255));
  map->num_heads = Hs;
  map->block = B;
  map->num_block_rows = g.NBR;
  map->total_tokens = (int32_t)g.T;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if ((st = launch_rowtable(s, cu_dev, g, B, wsa, w.rt)) != MF_OK) return st;
  if (g.NBR == 0) {
    hipLaunchKernelGGL(k_offsets, dim3(1), dim3(1024), 0, s, at<int32_t>(wsa, w.counts),
                       (int64_t)0, map->capacity_tiles, map->row_ptr, map->nnz, map->status);
    return hip_status();
  }
  const BiasArgs ba = bias_args(bias);
  const bool f32 = qk_dtype == MF_FP32;
  switch (B) {
    case 32: return dispatch_d<32>(d, f32, s, q, k, g, Hs, p, ba, map, wsa, w);
    case 64: return dispatch_d<64>(d, f32, s, q, k, g, Hs, p, ba, map, wsa, w);
    default: return dispatch_d<128>(d, f32, s, q, k, g, Hs, p, ba, map, wsa, w);
  }
}
