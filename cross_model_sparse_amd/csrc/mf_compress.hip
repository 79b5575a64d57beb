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
//              the kept tiles, rounds exp2(x - lse2) to bf16 (nearest even) or
//              encodes it as block-scaled E4M3, exchanges lane halves with
//              v_permlane32_swap into fragment order (see mf_bsr_map) and
//              writes each tile with coalesced 16-byte stores, plus col_idx.
#include <type_traits>

#include "mf_host.hpp"
#include "mf_qk.hpp"

namespace mf {

// Work-group id -> (schedule position, source head) of both passes.
// Position-major by default: the work-groups in flight on one XCD are a run of
// consecutive schedule positions for Hs / 8 heads, which in a single sequence
// are neighbouring block-rows reading the same K rows.  Head-major (several
// sequences, heads splitting evenly over the XCDs): each XCD takes its heads
// one at a time, every position of a head before its next head, so that the
// positions in flight, which the longest-first schedule draws from different
// sequences, at least share one head's K rows in the XCD's L2.
__device__ __forceinline__ void compress_slot(int b, int Hs, int NBR, int head_major, int &pos, int &h) {
  if (head_major) {
    const int x = b % kQkXcds, k = b / kQkXcds;
    pos = k % NBR;
    h = x + kQkXcds * (k / NBR);
  } else {
    pos = b / Hs;
    h = b % Hs;
  }
}

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
  // K tile buffers: one for bf16 Q/K with B <= 64, so that a work-group takes a
  // third of a CU and three waves share each SIMD (two barriers per block);
  // else two (one barrier per block) and two waves per SIMD
  static constexpr int NKB = (!F32 && B <= 64) ? 1 : 2;
  static constexpr int WAVES = F32 ? 1 : (NKB == 1 ? 3 : 2);
  static constexpr int SMEM = NKB * C::KBYTES > EPI ? NKB * C::KBYTES : EPI;
};

template <int B, int D, bool F32>
__global__ __launch_bounds__(B * 2) __attribute__((amdgpu_waves_per_eu(SelectCfg<B, D, F32>::WAVES))) void k_select(
    const void *__restrict__ qv, const void *__restrict__ kv, int64_t T, int32_t Hs, int32_t NBR,
    const RowInfo *__restrict__ rows, const int32_t *__restrict__ sched,
    const int64_t *__restrict__ pbase, int64_t ptot, float scale2, BiasArgs bias, double p,
    float *__restrict__ lse2_out, float *__restrict__ partials, int32_t *__restrict__ counts,
    uint32_t *__restrict__ bitmaps, int32_t nbw, float *__restrict__ kept_mass,
    const int32_t *__restrict__ row_alias, int32_t head_major) {
  using C = QKCfg<B, D, F32>;
  using E = std::conditional_t<F32, float, uint16_t>;
  __shared__ __attribute__((aligned(16))) char smem[SelectCfg<B, D, F32>::SMEM];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int m = lane & 31, hl = lane >> 5;
  int pos, h;
  compress_slot(blockIdx.x, Hs, NBR, head_major, pos, h);
  const int gr = sched[pos];
  if (row_alias && row_alias[gr] != gr && row_alias[gr] >= 0 && row_alias[gr] < NBR) {
    // shares an earlier block-row: no tiles of its own (kept mass is copied
    // once the first copy is done)
    const int64_t r = (int64_t)h * NBR + gr;
    for (int w = tid; w < nbw; w += C::NT) bitmaps[r * nbw + w] = 0u;
    if (tid == 0) counts[r] = 0;
    return;
  }
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

  // Block J + 1 of K loads into registers while block J is multiplied.  Two
  // buffers: it is stored into the other buffer, one barrier per block.  One
  // buffer: stored after a barrier (every wave's reads of block J done), and
  // the barrier that ends the step makes it visible.
  constexpr int NKB = SelectCfg<B, D, F32>::NKB;
  u32x4 stg[C::NCH];
  gload_tile<B, D, F32>(stg, kh, tok0, min(B, L), tid);
  lstore_tile<B, D, F32>(smem, stg, tid);
  __syncthreads();

  float m_run = -INFINITY;
  for (int J = 0; J <= I; ++J) {
    const char *kcur = smem + (NKB == 2 ? (J & 1) * C::KBYTES : 0);
    char *knext = smem + (NKB == 2 ? ((J + 1) & 1) * C::KBYTES : 0);
    if (J < I) gload_tile<B, D, F32>(stg, kh, tok0 + (int64_t)(J + 1) * B, min(B, L - (J + 1) * B), tid);
    f32x16 acc[B / 32];
    st_tile<B, D>(acc, kcur, qo, lane);
    if (NKB == 1 && J < I) {
      __syncthreads();
      lstore_tile<B, D, F32>(knext, stg, tid);
    }
    float lse, off;
    if (uniform_tile(I, J, B, bias.sink_n, bias.sink2, bias.local_w, bias.local2, off)) {
      // the scale is positive: the largest scaled logit is the image of the
      // largest raw score, and the offset cancels inside the sum
      const float mr = pair_max(lane_rawmax<B>(acc));
      const float sum = pair_sum(lane_expsum_fma<B>(acc, scale2, -mr * scale2));
      lse = rvalid ? fmaf(mr, scale2, off) + fast_log2(sum) : -INFINITY;
    } else {
      float mx = logits_inplace<B>(acc, false, rvalid, i_pos, J * B, scale2, bias.sink_n,
                                   bias.sink2, bias.local_w, bias.local2, lane);
      mx = pair_max(mx);
      float sum = 0.f;
      if (mx != -INFINITY) sum = lane_expsum<B>(acc, mx);
      sum = pair_sum(sum);
      lse = (mx == -INFINITY) ? -INFINITY : mx + fast_log2(sum);
    }
    if (hl == 0) part[(int64_t)J * B + i_loc] = lse;
    m_run = fmaxf(m_run, lse);
    // the other buffer held block J - 1, whose readers all passed the last barrier
    if (NKB == 2 && J < I) lstore_tile<B, D, F32>(knext, stg, tid);
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
  // thread prefixes: a shuffle scan inside each wave, then the wave totals
  double incl = loc;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const double u = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += u;
  }
  double excl = __shfl_up(incl, 1, kWave);
  if (lane == 0) excl = 0.0;
  if (lane == kWave - 1) tsum[wave] = incl;
  __syncthreads();
  double total = 0.0;
#pragma unroll
  for (int w = 0; w < C::NW; ++w) {
    const double x = tsum[w];
    if (w < wave) excl += x;
    total += x;
  }
  const double target = p * total;
  int below = 0;
  double run = excl;
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
// k_alias_kmass: block-rows that share an earlier one take its kept masses
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_alias_kmass(const RowInfo *__restrict__ rows,
                                                     const int32_t *__restrict__ row_alias,
                                                     int32_t NBR, int32_t Hs, int64_t T, int32_t B,
                                                     float *__restrict__ kept_mass) {
  const int gr = blockIdx.x;
  const int src = row_alias[gr];
  if (src == gr || src < 0 || src >= NBR) return;
  const RowInfo a = rows[gr], b = rows[src];
  // rows valid in both block-rows (all B for the full block-rows sharing is set on)
  const int nv = min(B, min(a.len - a.blk * B, b.len - b.blk * B));
  const int64_t t_dst = (int64_t)a.start + (int64_t)a.blk * B;
  const int64_t t_src = (int64_t)b.start + (int64_t)b.blk * B;
  for (int idx = threadIdx.x; idx < Hs * nv; idx += blockDim.x) {
    const int h = idx / nv, i = idx % nv;
    kept_mass[(int64_t)h * T + t_dst + i] = kept_mass[(int64_t)h * T + t_src + i];
  }
}

// ---------------------------------------------------------------------------
// k_offsets: row_ptr = exclusive scan of counts, nnz, status
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_offsets(const int32_t *__restrict__ counts, int64_t R,
                                                  int64_t capacity, int64_t *__restrict__ row_ptr,
                                                  int64_t *__restrict__ nnz,
                                                  int32_t *__restrict__ status) {
  __shared__ int64_t wsum[16];
  const int tid = threadIdx.x, nt = blockDim.x;  // nt == 1024
  const int64_t per = (R + nt - 1) / nt;
  const int64_t a = min(R, (int64_t)tid * per), b = min(R, a + per);
  int64_t s = 0;
  for (int64_t i = a; i < b; ++i) s += counts[i];
  const int64_t incl = block_scan_incl(s, wsum);
  if (tid == nt - 1) {
    row_ptr[R] = incl;
    *nnz = incl;
    *status = incl > capacity ? (int32_t)MF_ERR_CAPACITY : (int32_t)MF_OK;
  }
  int64_t run = incl - s;
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
  static constexpr int LIST = kMaxNB * 4 + 64 * 4;
  static constexpr int SMEM = 2 * C::KBYTES + LIST;   // two K tiles + kept list
};

// Probabilities of one lane's 4 consecutive keys (fp32) -> two bf16 pairs, RNE.
__device__ __forceinline__ uint2 pack4(float p0, float p1, float p2, float p3) {
  uint2 w;
  w.x = pack_bf16x2(p0, p1);
  w.y = pack_bf16x2(p2, p3);
  return w;
}

// One wave's 32 rows of a kept tile, from the S^T accumulators to the map in
// fragment order.  Lane (m, hl) holds row m and, per 32-key group and 8-key
// run q, keys 8q + 4hl .. + 3.  One v_permlane32_swap per word pair hands lanes
// 0-31 the full 8-key run q = 2p and lanes 32-63 the run q = 2p + 1, which is
// one 16-byte chunk of the fragment-ordered tile: row group i / 16, key chunk
// mb, position (q * 16 + i % 16).
template <int B>
__device__ __forceinline__ void store_tile_rows(char *dst, const uint2 (&w)[B / 32][4], int wave,
                                                int lane) {
  const int m = lane & 31, hl = lane >> 5;
  const int i_loc = wave * 32 + m;
#pragma unroll
  for (int mb = 0; mb < B / 32; ++mb)
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      const auto s0 = __builtin_amdgcn_permlane32_swap(w[mb][2 * pr].x, w[mb][2 * pr + 1].x, false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(w[mb][2 * pr].y, w[mb][2 * pr + 1].y, false, false);
      const u32x4 chunk = u32x4{s0[0], s1[0], s0[1], s1[1]};
      const int q = 2 * pr + hl;
      const int off = (((i_loc >> 4) * (B / 32) + mb) * 64 + q * 16 + (i_loc & 15)) * 16;
      // streaming store: the map is not read again by this pass, and letting
      // it allocate in L2 would evict the K rows other work-groups still read
      __builtin_nontemporal_store(chunk, reinterpret_cast<u32x4 *>(dst + off));
    }
}

// Block-scaled E4M3 form of one wave's 32 rows of a kept tile (format in
// mf_bsr_map).  Per 32-key block of row m, the lane's 16 probabilities and its
// partner's (lane ^ 32) give the block maximum a; its scale exponent is
// e = max(floor(log2 a) - 7, -126), read off the fp32 exponent field (0 for
// a = 0 or a denormal a, giving -126).  p * 2^-e is exact (a power-of-two
// scale, at most 2^126) and below 256, and v_cvt_pk_fp8_f32 rounds it to the
// nearest-even E4M3 code.  After the same v_permlane32_swap as the bf16 path,
// lanes 0-31 hold 8-key run 2p and lanes 32-63 run 2p + 1 of both chunks of a
// 64-key piece (one chunk for B = 32), which is one 16-byte (8-byte) piece.
template <int B>
__device__ __forceinline__ void store_tile_fp8(char *dst, const f32x16 (&pv)[B / 32], int wave,
                                               int lane) {
  constexpr int NP = B >= 64 ? 2 : 1;
  const int m = lane & 31, hl = lane >> 5;
  const int i_loc = wave * 32 + m;
  uint32_t d[B / 32][4];
  uint32_t sbytes = 0u;
#pragma unroll
  for (int mb = 0; mb < B / 32; ++mb) {
    float a = 0.f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) a = max3(a, pv[mb][r], pv[mb][r + 1]);
    a = pair_max(a);
    const int E = (int)(__float_as_uint(a) >> 23) - 127;
    const int e = E - 7 > -126 ? E - 7 : -126;
    const float up = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e
    sbytes |= (uint32_t)(e + 127) << (8 * mb);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(pv[mb][4 * g + 0] * up, pv[mb][4 * g + 1] * up, 0u, false);
      d[mb][g] = __builtin_amdgcn_cvt_pk_fp8_f32(pv[mb][4 * g + 2] * up, pv[mb][4 * g + 3] * up, w, true);
    }
  }
#pragma unroll
  for (int cp = 0; cp < B / 32 / NP; ++cp)
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      const int q = 2 * pr + hl;
      const int piece = (i_loc >> 4) * (B / 32 / NP) + cp;
      const auto s0 = __builtin_amdgcn_permlane32_swap(d[NP * cp][2 * pr], d[NP * cp][2 * pr + 1], false, false);
      if constexpr (NP == 2) {
        const auto s1 = __builtin_amdgcn_permlane32_swap(d[2 * cp + 1][2 * pr], d[2 * cp + 1][2 * pr + 1], false, false);
        const u32x4 chunk = u32x4{s0[0], s0[1], s1[0], s1[1]};
        __builtin_nontemporal_store(chunk, reinterpret_cast<u32x4 *>(dst + (piece * 64 + q * 16 + (i_loc & 15)) * 16));
      } else {
        const u32x2 chunk = u32x2{s0[0], s0[1]};
        __builtin_nontemporal_store(chunk, reinterpret_cast<u32x2 *>(dst + (piece * 64 + q * 16 + (i_loc & 15)) * 8));
      }
    }
  // scale bytes of row i_loc, written by the lower lane half
  char *sdst = dst + B * B + i_loc * (B / 32);
  if (hl == 0) {
    if constexpr (B == 128)
      __builtin_nontemporal_store(sbytes, reinterpret_cast<uint32_t *>(sdst));
    else if constexpr (B == 64)
      __builtin_nontemporal_store((uint16_t)sbytes, reinterpret_cast<uint16_t *>(sdst));
    else
      __builtin_nontemporal_store((uint8_t)sbytes, reinterpret_cast<uint8_t *>(sdst));
  }
}

template <int B, int D, bool F32, int FMT>
__global__ __launch_bounds__(B * 2) __attribute__((amdgpu_waves_per_eu(F32 ? 1 : 2))) void k_tiles(
    const void *__restrict__ qv, const void *__restrict__ kv, int64_t T, int32_t Hs, int32_t NBR,
    const RowInfo *__restrict__ rows, const int32_t *__restrict__ sched, float scale2,
    BiasArgs bias, const float *__restrict__ lse2_in, const uint32_t *__restrict__ bitmaps,
    int32_t nbw, const int64_t *__restrict__ row_ptr, int64_t capacity,
    int32_t *__restrict__ col_idx, char *__restrict__ tiles, int32_t head_major) {
  using C = QKCfg<B, D, F32>;
  using TC = TilesCfg<B, D, F32>;
  using E = std::conditional_t<F32, float, uint16_t>;
  __shared__ __attribute__((aligned(16))) char smem[TC::SMEM];
  int32_t *list = reinterpret_cast<int32_t *>(smem + 2 * C::KBYTES);
  int32_t *woff = list + kMaxNB;  // [33] word offsets

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int m = lane & 31, hl = lane >> 5;
  int pos, h;
  compress_slot(blockIdx.x, Hs, NBR, head_major, pos, h);
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
  // rows past the sequence end: -lse = -inf makes every probability exactly 0
  const float nlse2 = rvalid ? -lse2_in[(int64_t)h * T + tok0 + i_pos] : -INFINITY;

  // K tiles alternate between two LDS buffers: tile c is read from buffer c & 1
  // while tile c + 1 is written to the other one, one barrier per tile.
  u32x4 stg[C::NCH];
  {
    const int J = list[0];
    gload_tile<B, D, F32>(stg, kh, tok0 + (int64_t)J * B, min(B, L - J * B), tid);
    lstore_tile<B, D, F32>(smem, stg, tid);
  }
  __syncthreads();
  for (int c = 0; c < cnt; ++c) {
    const int J = list[c];
    const char *kcur = smem + (c & 1) * C::KBYTES;
    char *knext = smem + ((c + 1) & 1) * C::KBYTES;
    if (c + 1 < cnt) {
      const int Jn = list[c + 1];
      gload_tile<B, D, F32>(stg, kh, tok0 + (int64_t)Jn * B, min(B, L - Jn * B), tid);
    }
    f32x16 acc[B / 32];
    st_tile<B, D>(acc, kcur, qo, lane);
    // probabilities, in place
    float off;
    if (uniform_tile(I, J, B, bias.sink_n, bias.sink2, bias.local_w, bias.local2, off)) {
      const float c0 = nlse2 + off;
#pragma unroll
      for (int mb = 0; mb < B / 32; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mb][r] = fast_exp2(fmaf(acc[mb][r], scale2, c0));
    } else {
      logits_inplace<B>(acc, false, rvalid, i_pos, J * B, scale2, bias.sink_n, bias.sink2,
                        bias.local_w, bias.local2, lane);
#pragma unroll
      for (int mb = 0; mb < B / 32; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mb][r] = fast_exp2(acc[mb][r] + nlse2);
    }
    if (base + c < capacity) {
      char *dst = tiles + (base + c) * tile_bytes(B, FMT);
      if constexpr (FMT == MF_TILE_MXFP8) {
        store_tile_fp8<B>(dst, acc, wave, lane);
      } else {
        uint2 w[B / 32][4];
#pragma unroll
        for (int mb = 0; mb < B / 32; ++mb)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            w[mb][g] = pack4(acc[mb][4 * g + 0], acc[mb][4 * g + 1], acc[mb][4 * g + 2],
                             acc[mb][4 * g + 3]);
        store_tile_rows<B>(dst, w, wave, lane);
      }
    }
    // the other buffer held tile c - 1, whose readers all passed the last barrier
    if (c + 1 < cnt) lstore_tile<B, D, F32>(knext, stg, tid);
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
  const int32_t head_major = (Hs % kQkXcds == 0 && g.nseq > 1) ? 1 : 0;
  const dim3 grid((unsigned)((int64_t)g.NBR * Hs));
  hipLaunchKernelGGL((k_select<B, D, F32>), grid, dim3(B * 2), 0, s, q, k, g.T, Hs, g.NBR,
                     at<RowInfo>(ws, w.rt.rows), at<int32_t>(ws, w.rt.sched),
                     at<int64_t>(ws, w.rt.pbase), ptot, scale2, ba, p, at<float>(ws, w.lse2),
                     at<float>(ws, w.partials), at<int32_t>(ws, w.counts),
                     at<uint32_t>(ws, w.bitmaps), w.nbw, map->kept_mass, map->row_alias, head_major);
  if (hip_status() != MF_OK) return MF_ERR_HIP;
  if (map->row_alias) {
    hipLaunchKernelGGL(k_alias_kmass, dim3(g.NBR), dim3(256), 0, s, at<RowInfo>(ws, w.rt.rows),
                       map->row_alias, g.NBR, Hs, g.T, B, map->kept_mass);
    if (hip_status() != MF_OK) return MF_ERR_HIP;
  }
  hipLaunchKernelGGL(k_offsets, dim3(1), dim3(1024), 0, s, at<int32_t>(ws, w.counts),
                     (int64_t)Hs * g.NBR, map->capacity_tiles, map->row_ptr, map->nnz,
                     map->status);
  if (hip_status() != MF_OK) return MF_ERR_HIP;
  char *tiles = static_cast<char *>(map->tiles);
  if (map->tile_format == MF_TILE_MXFP8)
    hipLaunchKernelGGL((k_tiles<B, D, F32, MF_TILE_MXFP8>), grid, dim3(B * 2), 0, s, q, k, g.T,
                       Hs, g.NBR, at<RowInfo>(ws, w.rt.rows), at<int32_t>(ws, w.rt.sched),
                       scale2, ba, at<float>(ws, w.lse2), at<uint32_t>(ws, w.bitmaps), w.nbw,
                       map->row_ptr, map->capacity_tiles, map->col_idx, tiles, head_major);
  else
    hipLaunchKernelGGL((k_tiles<B, D, F32, MF_TILE_BF16>), grid, dim3(B * 2), 0, s, q, k, g.T,
                       Hs, g.NBR, at<RowInfo>(ws, w.rt.rows), at<int32_t>(ws, w.rt.sched),
                       scale2, ba, at<float>(ws, w.lse2), at<uint32_t>(ws, w.bitmaps), w.nbw,
                       map->row_ptr, map->capacity_tiles, map->col_idx, tiles, head_major);
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

extern "C" int64_t mf_tile_bytes(int32_t B, int32_t tile_format) {
  if (!valid_block(B) || !valid_tile_format(tile_format)) return 0;
  return tile_bytes(B, tile_format);
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
  if (!valid_tile_format(map->tile_format)) return MF_ERR_INVALID_ARG;
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
