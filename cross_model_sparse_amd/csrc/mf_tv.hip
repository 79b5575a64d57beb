// Total-variation distance between the translated map and a receiver's own map
// (MapFlow, "Accelerating Cross-Model LLM Inference via Attention Map Reuse",
// §3.3: the receiver layers to recompute are chosen offline from layer-wise TV
// distance between the two maps):
//
//   TV_t[i] = 1/2 sum_j | A~_t[i,j] - A_t[i,j] |
//   A~_t[i,j] = sum_h W[t,h] A_hat_h[i,j] / kmass_h[i]   (0 outside h's kept blocks)
//   A_t       = causal softmax(q_t k_g(t)^T / sqrt(d) + bias), the receiver's map
//
// Neither map is materialised.  One work-group per (query block, target head),
// one wave per 32 query rows, S^T tiles on MFMA as in the compressor (lane l
// holds query row l % 32 and 16 keys of every 32-key group):
//   pass 1  streams the receiver's key blocks and forms each row's log2-sum-exp
//           with a running (max, sum) pair;
//   pass 2  streams them again; per key block it rebuilds the lane's 64
//           receiver probabilities and, from the BSR tiles of every source that
//           kept the block, the lane's 64 translated values (fp32 coefficients
//           W[t,h] / kmass_h[i], bf16 or block-scaled E4M3 tiles), and adds the
//           absolute differences.  Blocks no source kept add the receiver's mass.
#include <type_traits>

#include "mf_host.hpp"
#include "mf_qk.hpp"

namespace mf {

// Dynamic LDS (byte offsets): rbase[Hs] int64, src[Hs] int32, bm[Hs][nbw],
// pc[Hs][nbw], coef[Hs][B] fp32, ns.
inline size_t tv_smem(int B, int Hs, int nbw) {
  return (size_t)Hs * (8 + 4) + (size_t)Hs * nbw * 8 + (size_t)Hs * B * 4 + 64;
}

// Occupancy.  With bf16 Q/K a work-group fits half a CU: one K tile buffer (two
// barriers per block) and 256 VGPRs, so two waves share each SIMD and hide each
// other's load latency; the sources' tile values load after the block's
// probabilities, two sources at a time at B = 128 (four would need 128
// registers of tile values).  With fp32 Q/K one wave per SIMD holds the whole
// register file: two K tile buffers (one barrier per block), and the first four
// sources' tile values load before the QK^T tile, so their latency hides behind
// the MFMAs.  Either way the translated values are subtracted from the
// receiver's probabilities in place.
template <int B, int D, bool F32>
constexpr bool tv_two_waves() { return !F32; }

template <int B, int D, bool F32, int FMT>
__global__ __launch_bounds__(B * 2)
__attribute__((amdgpu_waves_per_eu(tv_two_waves<B, D, F32>() ? 2 : 1))) void k_tv(
    const int64_t *__restrict__ row_ptr, const int32_t *__restrict__ col_idx,
    const char *__restrict__ tiles, const float *__restrict__ kept_mass, int32_t Hs, int32_t NBR,
    int64_t T, const float *__restrict__ W, int32_t Ht, int32_t grp, const void *__restrict__ qv,
    const void *__restrict__ kv, const RowInfo *__restrict__ rows,
    const int32_t *__restrict__ sched, float scale2, BiasArgs bias, int32_t nbw, int64_t capacity,
    int32_t renorm, const int32_t *__restrict__ row_alias, float *__restrict__ tv_out) {
  using C = QKCfg<B, D, F32>;
  using E = std::conditional_t<F32, float, uint16_t>;
  constexpr bool FP8 = FMT == MF_TILE_MXFP8;
  constexpr int NP = (FP8 && B >= 64) ? 2 : 1;
  constexpr int64_t TBYTES = tile_bytes(B, FMT);
  constexpr bool TW = tv_two_waves<B, D, F32>();
  constexpr int NKB = TW ? 1 : 2;  // K tile buffers
  __shared__ __attribute__((aligned(16))) char kbuf[NKB * C::KBYTES];
  extern __shared__ __attribute__((aligned(16))) char smem[];
  int64_t *rbase = reinterpret_cast<int64_t *>(smem);
  int32_t *src = reinterpret_cast<int32_t *>(smem + Hs * 8);
  uint32_t *bm = reinterpret_cast<uint32_t *>(smem + Hs * 12);
  int32_t *pc = reinterpret_cast<int32_t *>(smem + Hs * 12 + Hs * nbw * 4);
  float *coef = reinterpret_cast<float *>(smem + Hs * 12 + Hs * nbw * 8);
  int32_t *nsrc = reinterpret_cast<int32_t *>(smem + Hs * 12 + Hs * nbw * 8 + Hs * B * 4);

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int m = lane & 31, hl = lane >> 5;
  const int pos = blockIdx.x / Ht, t = blockIdx.x % Ht;
  const int gr = sched[pos];
  const RowInfo ri = rows[gr];
  const int I = ri.blk, L = ri.len;
  const int n = I + 1;
  const int i_loc = wave * 32 + m;
  const int i_pos = I * B + i_loc;
  const bool rvalid = i_pos < L;
  const int64_t tok0 = (int64_t)ri.start;
  const int ga = row_alias ? row_alias[gr] : gr;
  const int grm = (ga >= 0 && ga < NBR) ? ga : gr;  // BSR row (shared block-rows)

  // ---- sources of t (ballot compaction), kept bitmaps, coefficients ---------
  if (tid < 64) {
    int ns = 0;
    for (int h0 = 0; h0 < Hs; h0 += 64) {
      const int h = h0 + tid;
      const float w = h < Hs ? W[(int64_t)t * Hs + h] : 0.f;
      const uint64_t mask = wave_ballot(w != 0.f);
      if (w != 0.f) {
        const int q = ns + lanes_below(mask);
        src[q] = h;
        rbase[q] = row_ptr[(int64_t)h * NBR + grm];
      }
      ns += __popcll(mask);
    }
    if (tid == 0) *nsrc = ns;
  }
  for (int i = tid; i < Hs * nbw; i += C::NT) bm[i] = 0u;
  __syncthreads();
  const int ns = __builtin_amdgcn_readfirstlane(*nsrc);
  for (int q = 0; q < ns; ++q) {
    // entries past the capacity of an overflowed map are treated as missing
    const int64_t b0 = rbase[q], e0 = min(row_ptr[(int64_t)src[q] * NBR + grm + 1], capacity);
    for (int64_t idx = b0 + tid; idx < e0; idx += C::NT) {
      const int J = col_idx[idx];
      atomicOr(&bm[q * nbw + (J >> 5)], 1u << (J & 31));
    }
  }
  for (int idx = tid; idx < ns * B; idx += C::NT) {
    const int q = idx / B, il = idx % B;
    const int ip = I * B + il;
    const float w = W[(int64_t)t * Hs + src[q]];
    float c = 0.f;
    if (ip < L) {
      if (renorm) {
        const float km = kept_mass[(int64_t)src[q] * T + tok0 + ip];
        c = km > 0.f ? w / km : 0.f;
      } else {
        c = w;
      }
    }
    coef[q * B + il] = c;
  }
  __syncthreads();
  const int nw_row = (n + 31) / 32;
  for (int q = tid; q < ns; q += C::NT) {
    int run = 0;
    for (int w = 0; w < nw_row; ++w) {
      pc[q * nbw + w] = run;
      run += __popc(bm[q * nbw + w]);
    }
  }
  __syncthreads();

  const E *qh = reinterpret_cast<const E *>(qv) + (int64_t)t * T * D;
  const char *kh = reinterpret_cast<const char *>(kv) + (int64_t)(t / grp) * T * D * C::ESZ;
  QOp<D, F32> qo;
  load_q<D>(qo, rvalid ? qh + (tok0 + i_pos) * D : nullptr, hl);

  // Block J + 1 of K loads into registers while block J is multiplied.  Two
  // buffers: it is stored into the other buffer, and one barrier per block
  // makes it visible.  One buffer: a barrier (every wave's reads of block J
  // done) comes first, and the barrier that ends the step makes it visible.
  u32x4 stg[C::NCH];
  auto kcur_of = [&](int J) -> const char * { return kbuf + (NKB == 2 ? (J & 1) * C::KBYTES : 0); };
  auto knext_of = [&](int J) -> char * { return kbuf + (NKB == 2 ? ((J + 1) & 1) * C::KBYTES : 0); };
  auto stage_first = [&]() {
    gload_tile<B, D, F32>(stg, kh, tok0, min(B, L), tid);
    lstore_tile<B, D, F32>(kbuf, stg, tid);
    __syncthreads();
  };

  // ---- pass 1: row log2-sum-exp -------------------------------------------
  float lse_run = -INFINITY;
  stage_first();
  for (int J = 0; J <= I; ++J) {
    if (J < I) gload_tile<B, D, F32>(stg, kh, tok0 + (int64_t)(J + 1) * B, min(B, L - (J + 1) * B), tid);
    f32x16 acc[B / 32];
    st_tile<B, D>(acc, kcur_of(J), qo, lane);
    if (NKB == 1 && J < I) {
      __syncthreads();
      lstore_tile<B, D, F32>(knext_of(J), stg, tid);
    }
    float lse_t, off;
    if (uniform_tile(I, J, B, bias.sink_n, bias.sink2, bias.local_w, bias.local2, off)) {
      const float mr = pair_max(lane_rawmax<B>(acc));
      const float sum = pair_sum(lane_expsum_fma<B>(acc, scale2, -mr * scale2));
      lse_t = fmaf(mr, scale2, off) + fast_log2(sum);
    } else {
      float mx = logits_inplace<B>(acc, false, rvalid, i_pos, J * B, scale2, bias.sink_n,
                                   bias.sink2, bias.local_w, bias.local2, lane);
      mx = pair_max(mx);
      float sum = 0.f;
      if (mx != -INFINITY) sum = lane_expsum<B>(acc, mx);
      sum = pair_sum(sum);
      lse_t = (mx == -INFINITY) ? -INFINITY : mx + fast_log2(sum);
    }
    if (lse_t != -INFINITY) {
      const float mm = fmaxf(lse_run, lse_t);
      lse_run = mm + fast_log2(fast_exp2(lse_run - mm) + fast_exp2(lse_t - mm));
    }
    if (NKB == 2 && J < I) lstore_tile<B, D, F32>(knext_of(J), stg, tid);
    // also after the last block: its reads done before pass 2 restages block 0
    __syncthreads();
  }
  // rows past the sequence end: -lse = -inf makes every probability exactly 0
  const float nlse2 = rvalid ? -lse_run : -INFINITY;

  // ---- pass 2: |translated - receiver| summed over the causal row ---------
  // Lane values of up to four sources' tiles at key block J: per 32-key chunk mb
  // and 8-key run g, keys 8 g + 4 hl .. + 3 of the lane's row (bf16: 8 bytes of
  // the 16-byte fragment piece; fp8: 4 code bytes and the chunk's scale byte).
  using Raw = std::conditional_t<FP8, uint32_t, uint2>;
  // sources per group: two in the two-wave form at B = 128 (their values are
  // 64 registers), else four
  constexpr int GS = (TW && B == 128) ? 2 : 4;
  Raw raw[GS][B / 32][4];
  uint32_t raw_scale[GS];
  float cq[GS];
  const int voff = FP8 ? ((i_loc >> 4) * (B / (32 * NP)) * 64 + (i_loc & 15)) * 8 * NP + 4 * hl
                       : ((i_loc >> 4) * (B / 32) * 64 + (i_loc & 15)) * 16 + 8 * hl;
  auto load_group = [&](int q0, int J) {
#pragma unroll
    for (int u = 0; u < GS; ++u) {
      const int q = q0 + u;
      int64_t ti = -1;
      if (q < ns) {
        const uint32_t word = __builtin_amdgcn_readfirstlane(bm[q * nbw + (J >> 5)]);
        if ((word >> (J & 31)) & 1u) {
          const int64_t x = rbase[q] + pc[q * nbw + (J >> 5)] + __popc(word & ((1u << (J & 31)) - 1u));
          if (x < capacity) ti = x;
        }
      }
      // one descriptor per source, zero-length without a tile: absent tiles
      // read as zeros with no branch and no 64-bit lane addresses
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          (void *)(tiles + (ti >= 0 ? ti : 0) * TBYTES), 0, ti >= 0 ? (int)TBYTES : 0, 0x00020000);
      cq[u] = ti >= 0 ? coef[q * B + i_loc] : 0.f;
      // per-lane part of the offset in one register, the (mb, g) part a
      // constant scalar offset, so one lane offset serves all 16 loads
#pragma unroll
      for (int mb = 0; mb < B / 32; ++mb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          if constexpr (!FP8) {
            const auto w2 = __builtin_amdgcn_raw_buffer_load_b64(r, voff, (mb * 64 + g * 16) * 16, 0);
            raw[u][mb][g] = uint2{w2[0], w2[1]};
          } else {
            raw[u][mb][g] = __builtin_amdgcn_raw_buffer_load_b32(
                r, voff, ((mb / NP) * 64 + g * 16) * 8 * NP + (mb % NP) * 8, 0);
          }
        }
      if constexpr (FP8) {
        // the row's B/32 scale bytes in one word
        if constexpr (B == 128) raw_scale[u] = __builtin_amdgcn_raw_buffer_load_b32(r, i_loc * 4, B * B, 0);
        else if constexpr (B == 64) raw_scale[u] = __builtin_amdgcn_raw_buffer_load_b16(r, i_loc * 2, B * B, 0);
        else raw_scale[u] = __builtin_amdgcn_raw_buffer_load_b8(r, i_loc, B * B, 0);
      }
    }
  };
  // the group's translated values, subtracted from the receiver's probabilities
  auto sub_group = [&](f32x16 (&d)[B / 32]) {
#pragma unroll
    for (int u = 0; u < GS; ++u) {
#pragma unroll
      for (int mb = 0; mb < B / 32; ++mb) {
        if constexpr (!FP8) {
          const float c = -cq[u];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const uint2 w2 = raw[u][mb][g];
            d[mb][4 * g + 0] = fmaf(c, bf16lo(w2.x), d[mb][4 * g + 0]);
            d[mb][4 * g + 1] = fmaf(c, bf16hi(w2.x), d[mb][4 * g + 1]);
            d[mb][4 * g + 2] = fmaf(c, bf16lo(w2.y), d[mb][4 * g + 2]);
            d[mb][4 * g + 3] = fmaf(c, bf16hi(w2.y), d[mb][4 * g + 3]);
          }
        } else {
          const int sb = (int)((raw_scale[u] >> (8 * mb)) & 0xffu);
          const float cs = -__builtin_amdgcn_ldexpf(cq[u], sb - 127);
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(raw[u][mb][g], false);
            const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(raw[u][mb][g], true);
            d[mb][4 * g + 0] = fmaf(cs, lo[0], d[mb][4 * g + 0]);
            d[mb][4 * g + 1] = fmaf(cs, lo[1], d[mb][4 * g + 1]);
            d[mb][4 * g + 2] = fmaf(cs, hi[0], d[mb][4 * g + 2]);
            d[mb][4 * g + 3] = fmaf(cs, hi[1], d[mb][4 * g + 3]);
          }
        }
      }
    }
  };
  float tvl = 0.f;
  stage_first();
  for (int J = 0; J <= I; ++J) {
    if (J < I) gload_tile<B, D, F32>(stg, kh, tok0 + (int64_t)(J + 1) * B, min(B, L - (J + 1) * B), tid);
    if (!TW) load_group(0, J);
    f32x16 acc[B / 32];
    st_tile<B, D>(acc, kcur_of(J), qo, lane);
    if (NKB == 1 && J < I) {
      __syncthreads();
      lstore_tile<B, D, F32>(knext_of(J), stg, tid);
    }
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
    // receiver minus translated values of the lane's 64 elements, sources four
    // at a time
    for (int q0 = 0; q0 < ns; q0 += GS) {
      if (TW || q0 > 0) load_group(q0, J);
      sub_group(acc);
    }
#pragma unroll
    for (int mb = 0; mb < B / 32; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) tvl += fabsf(acc[mb][r]);
    if (NKB == 2 && J < I) lstore_tile<B, D, F32>(knext_of(J), stg, tid);
    if (J < I) __syncthreads();
  }
  const float tv = 0.5f * pair_sum(tvl);
  if (rvalid && hl == 0) tv_out[(int64_t)t * T + tok0 + i_pos] = tv;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
template <int B, int D, bool F32, int FMT>
static mf_status launch_tv(hipStream_t s, const mf_bsr_map *map, const float *W, int32_t Ht,
                           const void *q, const void *k, int32_t Hkr, const SeqGeom &g,
                           const BiasArgs &ba, int32_t renorm, float *tv, void *ws,
                           const RowTable &rt) {
  const int nbw = (g.maxnb + 31) / 32 > 0 ? (g.maxnb + 31) / 32 : 1;
  const size_t smem = tv_smem(B, map->num_heads, nbw);
  // the static K tile buffers
  const size_t kb = (tv_two_waves<B, D, F32>() ? 1 : 2) * (size_t)QKCfg<B, D, F32>::KBYTES;
  if (smem + kb > 160 * 1024) return MF_ERR_UNSUPPORTED;
  if (smem + kb > 64 * 1024 &&
      hipFuncSetAttribute(reinterpret_cast<const void *>(&k_tv<B, D, F32, FMT>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem) != hipSuccess)
    return MF_ERR_HIP;
  const float scale2 = kLog2e / sqrtf((float)D);
  hipLaunchKernelGGL((k_tv<B, D, F32, FMT>), dim3((unsigned)((int64_t)g.NBR * Ht)), dim3(B * 2),
                     smem, s, map->row_ptr, map->col_idx, static_cast<const char *>(map->tiles),
                     map->kept_mass, map->num_heads, g.NBR, g.T, W, Ht, Ht / Hkr, q, k,
                     at<RowInfo>(ws, rt.rows), at<int32_t>(ws, rt.sched), scale2, ba, nbw,
                     map->capacity_tiles, renorm, map->row_alias, tv);
  return hip_status();
}

template <int B>
static mf_status dispatch_tv(int32_t d, bool f32, int fmt, hipStream_t s, const mf_bsr_map *map,
                             const float *W, int32_t Ht, const void *q, const void *k, int32_t Hkr,
                             const SeqGeom &g, const BiasArgs &ba, int32_t renorm, float *tv,
                             void *ws, const RowTable &rt) {
#define MF_TV(DD, FF, FM) launch_tv<B, DD, FF, FM>(s, map, W, Ht, q, k, Hkr, g, ba, renorm, tv, ws, rt)
  if (fmt == MF_TILE_MXFP8) {
    if (d == 64) return f32 ? MF_TV(64, true, MF_TILE_MXFP8) : MF_TV(64, false, MF_TILE_MXFP8);
    return f32 ? MF_TV(128, true, MF_TILE_MXFP8) : MF_TV(128, false, MF_TILE_MXFP8);
  }
  if (d == 64) return f32 ? MF_TV(64, true, MF_TILE_BF16) : MF_TV(64, false, MF_TILE_BF16);
  return f32 ? MF_TV(128, true, MF_TILE_BF16) : MF_TV(128, false, MF_TILE_BF16);
#undef MF_TV
}

struct TvWs {
  RowTable rt;
  size_t total;
};

inline TvWs tv_ws(const SeqGeom &g) {
  Carve c;
  TvWs w;
  w.rt = carve_rows(c, g);
  w.total = c.off + 256;
  return w;
}

}  // namespace mf

using namespace mf;

extern "C" size_t mf_tv_distance_workspace_bytes(const int32_t *cu, int32_t nseq, int32_t B) {
  SeqGeom g;
  if (seq_geom(cu, nseq, B, &g) != MF_OK) return 0;
  return tv_ws(g).total;
}

extern "C" mf_status mf_tv_distance(void *stream, const mf_bsr_map *map, const float *W,
                                    int32_t Ht, const void *q, const void *k, mf_dtype qk_dtype,
                                    int32_t Hkr, int32_t d, const int32_t *cu_host,
                                    const int32_t *cu_dev, int32_t nseq,
                                    const mf_logit_bias *bias, int32_t renorm, float *tv, void *ws,
                                    size_t ws_bytes) {
  if (!map || !cu_host || !cu_dev || Ht <= 0 || Hkr <= 0 || Ht % Hkr != 0 || !bias_ok(bias))
    return MF_ERR_INVALID_ARG;
  if (!valid_block(map->block) || map->num_heads <= 0 || !W || !valid_tile_format(map->tile_format))
    return MF_ERR_INVALID_ARG;
  if (qk_dtype != MF_BF16 && qk_dtype != MF_FP32) return MF_ERR_UNSUPPORTED;
  if (!valid_dim(d)) return MF_ERR_UNSUPPORTED;
  if (map->num_heads > 1024) return MF_ERR_UNSUPPORTED;
  SeqGeom g;
  mf_status st = seq_geom(cu_host, nseq, map->block, &g);
  if (st != MF_OK) return st;
  if (g.NBR != map->num_block_rows || g.T != map->total_tokens) return MF_ERR_INVALID_ARG;
  if ((int64_t)g.NBR * Ht > INT32_MAX / 2) return MF_ERR_UNSUPPORTED;
  if (g.T > 0 && (!q || !k || !tv || !map->row_ptr || !map->col_idx || !map->tiles ||
                  !map->kept_mass))
    return MF_ERR_INVALID_ARG;
  const TvWs w = tv_ws(g);
  if (!ws || ws_bytes < w.total) return MF_ERR_WORKSPACE;
  if (g.NBR == 0) return MF_OK;
  void *wsa = reinterpret_cast<void *>((reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if ((st = launch_rowtable(s, cu_dev, g, map->block, wsa, w.rt)) != MF_OK) return st;
  const BiasArgs ba = bias_args(bias);
  const bool f32 = qk_dtype == MF_FP32;
  const int fmt = map->tile_format;
  switch (map->block) {
    case 32: return dispatch_tv<32>(d, f32, fmt, s, map, W, Ht, q, k, Hkr, g, ba, renorm, tv, wsa, w.rt);
    case 64: return dispatch_tv<64>(d, f32, fmt, s, map, W, Ht, q, k, Hkr, g, ba, renorm, tv, wsa, w.rt);
    default: return dispatch_tv<128>(d, f32, fmt, s, map, W, Ht, q, k, Hkr, g, ba, renorm, tv, wsa, w.rt);
  }
}
