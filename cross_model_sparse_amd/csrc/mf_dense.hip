// Dense causal attention for recomputed heads (MapFlow, "Accelerating
// Cross-Model LLM Inference via Attention Map Reuse", §4: the receiver computes
// its first layers normally) and the exact path a cache miss falls back to
// (AttnCache guide, "AttnCache Guide: Reusing Attention Maps in LLM Prefill":
// threshold-gated fallback to standard attention).
//
//   O_h = softmax(Q_h K_g^T / sqrt(d) + bias) V_g,  g = h / (Hq / Hkv), causal.
//
// One work-group per (query head, 256-row query block), one wave per 32 rows.
// 64-key blocks of K, and of V transposed and block-padded per sequence, stream
// through two LDS buffer sets (one barrier per block).  S^T tiles on MFMA leave
// each lane holding one query row, so the running max and sum (online softmax)
// stay in the lane.  A row's running max moves only when a block's maximum
// exceeds it by more than 8 (log2 units): the accumulated rows are rescaled
// rarely, and P stays below 2^8 in the exact form (below 2^16 in the short
// form below).  P, rounded to bf16, is already in the A-operand layout of the
// P V product, which runs on MFMA against the transposed V tile.  No map is
// stored.
//
// With bf16 inputs, Q is scaled by log2(e)/sqrt(d) once (one more bf16
// rounding per element).  Blocks with one offset for all of their pairs, and
// blocks where only the local window's edge varies (its bias added per
// element), then take a short form: the Q K^T accumulators start from
// (offset - running max) of the lane's row, so they leave the MFMA as
// exponents; P = exp2 of them, with no per-block maximum, and the row sum is
// taken from the bf16 P.  A block whose row sum passes 2^16 is redone in the
// exact form.
#include <type_traits>

#include "mf_host.hpp"
#include "mf_qk.hpp"

namespace mf {

constexpr int kDenseQB = 256;  // query rows per work-group; row table and V staging block
constexpr int kDenseKB = 64;   // keys per block

template <int D, bool F32>
struct DenseCfg {
  static constexpr int QB = kDenseQB, KB = kDenseKB;
  static constexpr int NT = QB * 2;                 // eight waves
  using C = QKCfg<KB, D, F32>;                      // K tile geometry in LDS
  static constexpr int KCH = KB * C::CPR / NT;      // 16-byte K chunks per thread
  static constexpr int VPITCH = KB * 2 + kLdsPad;   // LDS row (one value column) of V^T
  static constexpr int VBYTES = D * VPITCH;
  static constexpr int VCPR = KB * 2 / 16;
  static constexpr int VCH = D * VCPR / NT;         // 16-byte V chunks per thread
  static constexpr int SET = C::KBYTES + VBYTES;    // one K + V buffer set
  static constexpr int SMEM = 2 * SET;
  static_assert(KCH * NT == KB * C::CPR && VCH * NT == D * VCPR, "tiles must split evenly");
};

// Whether the 32 query rows [r0, r0 + 32) against the keys [k0, k0 + kb) see
// every key (no causal mask) with one common offset `off` (log2 units): no sink
// column, and the local window covers all of the pairs or none of them.
__device__ __forceinline__ bool dense_uniform(int r0, int k0, int kb, const BiasArgs &b, float &off) {
  off = 0.f;
  if (k0 + kb - 1 > r0) return false;
  if (b.sink2 != 0.f && k0 < b.sink_n) return false;
  if (b.local2 != 0.f) {
    const int dmin = r0 - (k0 + kb - 1), dmax = r0 + 31 - k0;
    if (dmax < b.local_w)
      off = b.local2;
    else if (dmin < b.local_w)
      return false;
  }
  return true;
}

// Whether the rows [r0, r0 + 32) against the keys [k0, k0 + kb) see every key
// with no sink column, while the local window covers only part of the pairs:
// the one bias left is the window's, element by element.
__device__ __forceinline__ bool dense_window_edge(int r0, int k0, int kb, const BiasArgs &b) {
  if (k0 + kb - 1 > r0 || b.local2 == 0.f) return false;
  if (b.sink2 != 0.f && k0 < b.sink_n) return false;
  const int dmin = r0 - (k0 + kb - 1), dmax = r0 + 31 - k0;
  return dmin < b.local_w && b.local_w <= dmax;
}

// Multiplies every bf16 element of the lane's Q half-row by `s` (RNE).
template <int D>
__device__ __forceinline__ void scale_q(QOp<D, false> &qo, float s) {
#pragma unroll
  for (int c = 0; c < D / 16; ++c)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t x = qo.v[c][w];
      qo.v[c][w] = pack_bf16x2(__uint_as_float(x << 16) * s, __uint_as_float(x & 0xffff0000u) * s);
    }
}

// S^T tile for the wave's 32 query rows against the B staged keys, as
// st_tile, with every accumulator starting from `seed` instead of 0.
template <int B, int D>
__device__ __forceinline__ void st_tile_seeded(f32x16 (&acc)[B / 32], const char *klds,
                                               const QOp<D, false> &qo, int lane,
                                               const f32x16 &seed) {
  using C = QKCfg<B, D, false>;
  const int m = lane & 31, hl = lane >> 5;
  const char *rowp = klds + m * C::PITCH + hl * D;
#pragma unroll
  for (int mb = 0; mb < B / 32; ++mb) acc[mb] = seed;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
    for (int mb = 0; mb < B / 32; ++mb) {
      u32x4 a = *reinterpret_cast<const u32x4 *>(rowp + mb * 32 * C::PITCH + ks * 16);
      acc[mb] = mfma_bf16(as_bf16x8(a), as_bf16x8(qo.v[ks]), acc[mb]);
    }
}

// acc + lo + hi of a packed bf16 pair (one dot2 against [1, 1]).
__device__ __forceinline__ float add_bf16x2(uint32_t w, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                         __builtin_bit_cast(bf16x2, 0x3f803f80u), acc, false);
}

template <int D, bool F32>
__global__ __launch_bounds__(kDenseQB * 2) __attribute__((amdgpu_waves_per_eu(2))) void k_dense(
    const void *__restrict__ qv, const void *__restrict__ kv, const uint16_t *__restrict__ vt,
    int64_t T, int32_t Hq, int32_t grp, int32_t NBR, const RowInfo *__restrict__ rows,
    const int32_t *__restrict__ sched, float scale2, BiasArgs bias, float *__restrict__ o,
    int32_t kv_major) {
  using DC = DenseCfg<D, F32>;
  using C = typename DC::C;
  constexpr int QB = DC::QB, KB = DC::KB, NT = DC::NT;
  using E = std::conditional_t<F32, float, uint16_t>;
  __shared__ __attribute__((aligned(16))) char smem[DC::SMEM];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int m = lane & 31, hl = lane >> 5;
  int pos, h;
  kv_major_slot(blockIdx.x, Hq, grp, NBR, kv_major, pos, h);
  const int g = h / grp;
  const int gr = sched[pos];
  const RowInfo ri = rows[gr];
  const int I = ri.blk, L = ri.len;
  const int r0 = I * QB + wave * 32;  // the wave's first query row in the sequence
  const int i_pos = r0 + m;
  const bool rvalid = i_pos < L;
  const int64_t tok0 = (int64_t)ri.start;
  const int64_t tpad = (int64_t)NBR * QB;
  // key blocks up to the work-group's last row, and up to this wave's (0 when
  // the wave has no row inside the sequence)
  const int nkb = (min(I * QB + QB, L) - 1) / KB + 1;
  const int wkb = r0 < L ? min(r0 + 31, L - 1) / KB + 1 : 0;

  const E *qh = reinterpret_cast<const E *>(qv) + (int64_t)h * T * D;
  const char *kh = reinterpret_cast<const char *>(kv) + ((int64_t)g * T + tok0) * C::ROWB;
  const uint16_t *vtg = vt + (int64_t)g * D * tpad + (int64_t)(gr - I) * QB;
  QOp<D, F32> qo;
  load_q<D>(qo, rvalid ? qh + (tok0 + i_pos) * D : nullptr, hl);
  if constexpr (!F32) scale_q<D>(qo, scale2);
  const float sc = F32 ? scale2 : 1.f;  // scale still due on the MFMA's scores

  // key block J: K rows (zeros past the sequence end) and V^T columns into
  // registers, then into a buffer set
  u32x4 kst[DC::KCH], vst[DC::VCH];
  auto gload = [&](int J) {
    const int nval = min(KB, L - J * KB);
#pragma unroll
    for (int c = 0; c < DC::KCH; ++c) {
      const int idx = tid + c * NT;
      const int r = idx / C::CPR, col = idx % C::CPR;
      kst[c] = r < nval ? *reinterpret_cast<const u32x4 *>(kh + (int64_t)(J * KB + r) * C::ROWB + col * 16)
                        : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int c = 0; c < DC::VCH; ++c) {
      const int idx = tid + c * NT;
      const int d = idx / DC::VCPR, cc = idx % DC::VCPR;
      vst[c] = *reinterpret_cast<const u32x4 *>(vtg + (int64_t)d * tpad + J * KB + cc * 8);
    }
  };
  auto lstore = [&](char *set) {
#pragma unroll
    for (int c = 0; c < DC::KCH; ++c) {
      const int idx = tid + c * NT;
      const int r = idx / C::CPR, col = idx % C::CPR;
      *reinterpret_cast<u32x4 *>(set + r * C::PITCH + col * 16) = kst[c];
    }
#pragma unroll
    for (int c = 0; c < DC::VCH; ++c) {
      const int idx = tid + c * NT;
      const int d = idx / DC::VCPR, cc = idx % DC::VCPR;
      *reinterpret_cast<u32x4 *>(set + C::KBYTES + d * DC::VPITCH + cc * 16) = vst[c];
    }
  };

  gload(0);
  lstore(smem);
  __syncthreads();

  f32x16 oacc[D / 32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) oacc[nb] = zero16();
  float m_run = -INFINITY, l_run = 0.f;
  // accumulator seed of the short form: offset - m_run of the lane's row
  float seedv = -INFINITY;
  f32x16 seed = zero16();

  for (int J = 0; J < nkb; ++J) {
    const char *cur = smem + (J & 1) * DC::SET;
    char *nxt = smem + ((J + 1) & 1) * DC::SET;
    if (J + 1 < nkb) gload(J + 1);
    if (J < wkb) {
      f32x16 acc[KB / 32];
      u32x4 pa[KB / 32][2];  // P in bf16: the lane's A operands of P V
      const int k0 = J * KB;
      float off;
      const bool uni = dense_uniform(r0, k0, KB, bias, off);
      // window-edge blocks take the short form too (off = 0), plus the window
      // bias element by element
      const bool edge = !uni && dense_window_edge(r0, k0, KB, bias);
      bool done = false;
      if constexpr (!F32) {
        if ((uni || edge) && !wave_ballot(m_run == -INFINITY)) {
          const float want = off - m_run;
          if (wave_ballot(want != seedv)) {
            // rare (a moved max or a new offset): kept as a branch, not selects
            asm volatile("" ::: "memory");
            seedv = want;
#pragma unroll
            for (int r = 0; r < 16; ++r) seed[r] = seedv;
          }
          st_tile_seeded<KB, D>(acc, cur, qo, lane, seed);
          if (edge) {
            // key k0 + mb * 32 + acc_row(r) is inside the window (i - j < w)
            // when mb * 32 + 8 (r / 4) + r % 4 > i - w - k0 - 4 hl
            const int t = i_pos - bias.local_w - k0 - 4 * hl;
#pragma unroll
            for (int mb = 0; mb < KB / 32; ++mb)
#pragma unroll
              for (int r = 0; r < 16; ++r)
                acc[mb][r] += (mb * 32 + 8 * (r >> 2) + (r & 3) > t) ? bias.local2 : 0.f;
          }
          float rs = 0.f;
#pragma unroll
          for (int mb = 0; mb < KB / 32; ++mb)
#pragma unroll
            for (int e2 = 0; e2 < 2; ++e2)
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                pa[mb][e2][k] = pack_bf16x2(fast_exp2(acc[mb][8 * e2 + 2 * k]),
                                            fast_exp2(acc[mb][8 * e2 + 2 * k + 1]));
                rs = add_bf16x2(pa[mb][e2][k], rs);
              }
          rs = pair_sum(rs);
          // P below 2^16 in every row (inf and NaN fail the test): the block stands
          if (!wave_ballot(!(rs <= 65536.f))) {
            l_run += rs;
            done = true;
          }
        }
      }
      if (!done) {
        st_tile<KB, D>(acc, cur, qo, lane);
        float mx;
        if (uni) {
          // the scale is positive: the largest logit is the image of the largest score
          mx = fmaf(pair_max(lane_rawmax<KB>(acc)), sc, off);
        } else {
          mx = pair_max(logits_inplace<KB>(acc, false, rvalid, i_pos, k0, sc, bias.sink_n,
                                           bias.sink2, bias.local_w, bias.local2, lane));
        }
        const float m_new = (mx > m_run + 8.f) ? mx : m_run;
        const float msafe = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - msafe);
        float rs = 0.f;
        if (uni) {
          const float c0 = off - msafe;
#pragma unroll
          for (int mb = 0; mb < KB / 32; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float pv = fast_exp2(fmaf(acc[mb][r], sc, c0));
              acc[mb][r] = pv;
              rs += pv;
            }
        } else {
#pragma unroll
          for (int mb = 0; mb < KB / 32; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float pv = rvalid ? fast_exp2(acc[mb][r] - msafe) : 0.f;
              acc[mb][r] = pv;
              rs += pv;
            }
        }
        l_run = fmaf(l_run, alpha, pair_sum(rs));
        m_run = m_new;
        // rescale the accumulated rows whose max moved (row acc_row(r) of this
        // wave belongs to that lane)
        if (wave_ballot(alpha != 1.f)) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float f = __shfl(alpha, acc_row(r, lane), kWave);
#pragma unroll
            for (int nb = 0; nb < D / 32; ++nb) oacc[nb][r] *= f;
          }
        }
#pragma unroll
        for (int mb = 0; mb < KB / 32; ++mb)
#pragma unroll
          for (int e2 = 0; e2 < 2; ++e2)
#pragma unroll
            for (int k = 0; k < 4; ++k)
              pa[mb][e2][k] = pack_bf16x2(acc[mb][8 * e2 + 2 * k], acc[mb][8 * e2 + 2 * k + 1]);
      }
      // P (bf16, A operand) x V tile (LDS, B operand)
      const char *vlds = cur + C::KBYTES;
#pragma unroll
      for (int mb = 0; mb < KB / 32; ++mb)
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
          // the lane's keys 16 e2 + 4 hl + {0..3, 8..11} of chunk mb: 8
          // consecutive columns of the quad-swapped V^T rows
          const int c0 = mb * 32 + 16 * e2 + 8 * hl;
#pragma unroll
          for (int nb = 0; nb < D / 32; ++nb) {
            const u32x4 b =
                *reinterpret_cast<const u32x4 *>(vlds + (nb * 32 + m) * DC::VPITCH + c0 * 2);
            oacc[nb] = mfma_bf16(as_bf16x8(pa[mb][e2]), as_bf16x8(b), oacc[nb]);
          }
        }
    }
    // the other set held block J - 1, whose readers all passed the last barrier
    if (J + 1 < nkb) lstore(nxt);
    __syncthreads();
  }

  float *oh = o + (int64_t)h * T * D;
  const float inv = (l_run > 0.f) ? 1.f / l_run : 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = acc_row(r, lane);
    const float f = __shfl(inv, row, kWave);
    const int ip = r0 + row;
    if (ip < L) {
      float *dst = oh + (tok0 + ip) * D + m;
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb) dst[nb * 32] = oacc[nb][r] * f;
    }
  }
}

// V [Hkv][T][D] -> Vt[g][d][NBR * QB]: per sequence block-padded to QB columns,
// zeros past the sequence end.  Within every 16 keys the middle two groups of
// four trade places (keys 4-7 in columns 8-11 and back), so the 8 keys one lane
// feeds a P V MFMA (4 hl + {0..3, 8..11}) are 8 consecutive columns.
__device__ __forceinline__ int quad_swap16(int j) { return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1); }

template <int D>
__global__ __launch_bounds__(256) void k_vtranspose_dense(const uint16_t *__restrict__ v, int64_t T,
                                                          const RowInfo *__restrict__ rows,
                                                          int32_t NBR, uint16_t *__restrict__ vt) {
  constexpr int B = kDenseQB, P = B + 8;
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
      t[(c * 8 + 2 * e) * P + quad_swap16(j)] = (uint16_t)(x[e] & 0xffffu);
      t[(c * 8 + 2 * e + 1) * P + quad_swap16(j)] = (uint16_t)(x[e] >> 16);
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

template <int D, bool F32>
static mf_status launch_dense(hipStream_t s, const void *q, const void *k, const void *v,
                              int32_t Hq, int32_t Hkv, const SeqGeom &g, const BiasArgs &ba,
                              float *o, void *ws, const VtWs &w) {
  hipLaunchKernelGGL((k_vtranspose_dense<D>), dim3(g.NBR, Hkv), dim3(256), 0, s,
                     reinterpret_cast<const uint16_t *>(v), g.T, at<RowInfo>(ws, w.rt.rows), g.NBR,
                     at<uint16_t>(ws, w.vt));
  if (hip_status() != MF_OK) return MF_ERR_HIP;
  const float scale2 = kLog2e / sqrtf((float)D);
  if (DenseCfg<D, F32>::SMEM > 160 * 1024) return MF_ERR_UNSUPPORTED;
  hipLaunchKernelGGL((k_dense<D, F32>), dim3((unsigned)((int64_t)g.NBR * Hq)), dim3(kDenseQB * 2),
                     0, s, q, k, at<uint16_t>(ws, w.vt), g.T, Hq, Hq / Hkv, g.NBR,
                     at<RowInfo>(ws, w.rt.rows), at<int32_t>(ws, w.rt.sched), scale2, ba, o,
                     (int32_t)(Hkv % kQkXcds == 0));
  return hip_status();
}

}  // namespace mf

using namespace mf;

extern "C" size_t mf_dense_workspace_bytes(int32_t Hkv, const int32_t *cu, int32_t nseq,
                                           int32_t d) {
  SeqGeom g;
  if (Hkv <= 0 || !valid_dim(d) || seq_geom_blocks(cu, nseq, kDenseQB, &g) != MF_OK) return 0;
  return vt_ws(g, Hkv, kDenseQB, d).total;
}

extern "C" mf_status mf_dense_ref_attention(void *stream, const void *q, const void *k,
                                            const void *v, mf_dtype qk_dtype, int32_t Hq,
                                            int32_t Hkv, int32_t d, const int32_t *cu_host,
                                            const int32_t *cu_dev, int32_t nseq,
                                            const mf_logit_bias *bias, float *o, void *ws,
                                            size_t ws_bytes) {
  if (!cu_host || !cu_dev || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || !bias_ok(bias))
    return MF_ERR_INVALID_ARG;
  if (qk_dtype != MF_BF16 && qk_dtype != MF_FP32) return MF_ERR_UNSUPPORTED;
  if (!valid_dim(d)) return MF_ERR_UNSUPPORTED;
  SeqGeom g;
  mf_status st = seq_geom_blocks(cu_host, nseq, kDenseQB, &g);
  if (st != MF_OK) return st;
  if ((int64_t)g.NBR * Hq > INT32_MAX / 2) return MF_ERR_UNSUPPORTED;
  if (g.T > 0 && (!q || !k || !v || !o)) return MF_ERR_INVALID_ARG;
  const VtWs w = vt_ws(g, Hkv, kDenseQB, d);
  if (!ws || ws_bytes < w.total) return MF_ERR_WORKSPACE;
  if (g.NBR == 0) return MF_OK;
  void *wsa = reinterpret_cast<void *>((reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if ((st = launch_rowtable(s, cu_dev, g, kDenseQB, wsa, w.rt)) != MF_OK) return st;
  const BiasArgs ba = bias_args(bias);
  const bool f32 = qk_dtype == MF_FP32;
  if (d == 64)
    return f32 ? launch_dense<64, true>(s, q, k, v, Hq, Hkv, g, ba, o, wsa, w)
               : launch_dense<64, false>(s, q, k, v, Hq, Hkv, g, ba, o, wsa, w);
  return f32 ? launch_dense<128, true>(s, q, k, v, Hq, Hkv, g, ba, o, wsa, w)
             : launch_dense<128, false>(s, q, k, v, Hq, Hkv, g, ba, o, wsa, w);
}
