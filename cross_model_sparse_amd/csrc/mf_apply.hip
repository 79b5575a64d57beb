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
constexpr int kBufferFlags = 0x00020000;  // buffer descriptor word 3 for raw dword loads

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
  static constexpr int NW = B / 16;                // waves per work-group, 16 rows each
  static constexpr int NT = NW * 64;
  static constexpr int KC = B / 32;                // 32-key chunks per key block
  static constexpr int CPR = B * 2 / 16;           // 16-byte chunks per Vt row
  static constexpr int VPITCH = B * 2;             // Vt row pitch in LDS (XOR-swizzled, no pad)
  static constexpr int VBYTES = D * VPITCH;
  static constexpr int VINST = VBYTES / 1024 / NW; // 1 KB direct loads per wave per tile
  static_assert(VINST * 1024 * NW == VBYTES, "V tile must split into 1 KB wave loads");
};

// Dynamic LDS (byte offsets; the two V buffers are static): rbase[Hs] int64,
// src[Hs], wt[Hs], bm[Hs][nbw], pc[Hs][nbw], uni[nbw], coef[Hs][B] (bf16 bits), nsrc.
inline size_t apply_smem(int B, int D, int Hs, int nbw) {
  (void)B;
  (void)D;
  size_t s = (size_t)Hs * (8 + 4 + 4);
  s += (size_t)Hs * nbw * 8 + (size_t)nbw * 4;
  s += (size_t)Hs * B * 2;
  s += 64;
  return s;
}

// acc += c * (bf16 pair) for both halves of a packed word, one dot2 each:
// dot2([lo, hi], [c, 0]) = c * lo and dot2([lo, hi], [0, c]) = c * hi, fp32
// accumulate; the coefficient is held in bf16.
__device__ __forceinline__ void mix_word(float &even, float &odd, uint32_t w, uint32_t c_lo,
                                         uint32_t c_hi) {
  even = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                         __builtin_bit_cast(bf16x2, c_lo), even, false);
  odd = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                        __builtin_bit_cast(bf16x2, c_hi), odd, false);
}

typedef __attribute__((address_space(3))) void lds_void;

template <int B, int D, bool MANY>
__global__ __launch_bounds__(B * 4) __attribute__((amdgpu_waves_per_eu(4))) void k_apply(
    const int64_t *__restrict__ row_ptr, const int32_t *__restrict__ col_idx,
    const uint16_t *__restrict__ tiles, const float *__restrict__ kept_mass, int32_t Hs,
    int32_t NBR, int64_t T, const float *__restrict__ W, int32_t Ht, int32_t grp,
    const uint16_t *__restrict__ vt, const RowInfo *__restrict__ rows,
    const int32_t *__restrict__ sched, int32_t nbw, int64_t capacity, int32_t renorm,
    float *__restrict__ o) {
  using C = ApplyCfg<B, D>;
  constexpr int KC = C::KC;
  // The two V buffers are separate arrays so the compiler can tell that the
  // direct loads into one never alias reads of the other (otherwise every LDS
  // read waits for all outstanding direct loads).
  __shared__ __attribute__((aligned(16))) char vA[C::VBYTES];
  __shared__ __attribute__((aligned(16))) char vB[C::VBYTES];
  extern __shared__ __attribute__((aligned(16))) char smem[];
  // byte offsets, kept relative to smem so every access stays an LDS access
  const int o_rbase = 0;
  const int o_src = o_rbase + Hs * 8;
  const int o_wt = o_src + Hs * 4;
  const int o_bm = o_wt + Hs * 4;
  const int o_pc = o_bm + Hs * nbw * 4;
  const int o_uni = o_pc + Hs * nbw * 4;
  const int o_coef = o_uni + nbw * 4;
  const int o_ns = (o_coef + Hs * B * 2 + 3) & ~3;
  int64_t *rbase = reinterpret_cast<int64_t *>(smem + o_rbase);
  int32_t *src = reinterpret_cast<int32_t *>(smem + o_src);
  float *wt = reinterpret_cast<float *>(smem + o_wt);
  uint32_t *bm = reinterpret_cast<uint32_t *>(smem + o_bm);
  int32_t *pc = reinterpret_cast<int32_t *>(smem + o_pc);
  uint32_t *uni = reinterpret_cast<uint32_t *>(smem + o_uni);
  uint16_t *coef = reinterpret_cast<uint16_t *>(smem + o_coef);  // bf16 bits
  int32_t *nsrc_p = reinterpret_cast<int32_t *>(smem + o_ns);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m16 = lane & 15, kg = lane >> 4;
  // work-group id -> (query block, target): consecutive ids land on XCDs in
  // turn; XCD x takes every eighth query block of the longest-first order, all
  // targets of one block before the next, zig-zagging between rounds so the
  // XCDs stay in step and share V through the memory-side cache.
  const int x = blockIdx.x % kXcds, kx = blockIdx.x / kXcds;
  const int round = kx / Ht, t = kx % Ht;
  const int pos = round * kXcds + ((round & 1) ? (kXcds - 1 - x) : x);
  if (pos >= NBR) return;
  const int gr = sched[pos];
  const RowInfo ri = rows[gr];
  const int I = ri.blk, L = ri.len;
  const int n = I + 1;
  const int nw_row = (n + 31) / 32;
  const int g = t / grp;
  const int64_t tok0 = (int64_t)ri.start;
  const int64_t tpad = (int64_t)NBR * B;

  // ---- per-row setup: sources, kept bitmaps, ranks, coefficients ----------
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
  const int ns = __builtin_amdgcn_readfirstlane(*nsrc_p);
  // targets with at most four sources run in the <false> instance, the rest in <true>
  if (MANY != (ns > 4)) return;
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
    coef[q * B + il] = (uint16_t)pack_bf16x2(c, 0.f);
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

  // next key block of the union at or after `from` (uniform), -1 if none
  auto next_J = [&](int from) -> int {
    if (from >= n) return -1;
    for (int w = from >> 5; w < nw_row; ++w) {
      uint32_t bits = __builtin_amdgcn_readfirstlane(uni[w]);
      if (w == (from >> 5)) bits &= ~((1u << (from & 31)) - 1u);
      if (bits) return w * 32 + __ffs(bits) - 1;
    }
    return -1;
  };
  // tile index of source q at key block J, or -1 (uniform)
  auto tile_of = [&](int q, int J) -> int64_t {
    const uint32_t word = __builtin_amdgcn_readfirstlane(bm[q * nbw + (J >> 5)]);
    if (!((word >> (J & 31)) & 1u)) return -1;
    const int rank = __builtin_amdgcn_readfirstlane(pc[q * nbw + (J >> 5)]) +
                     __popc(word & ((1u << (J & 31)) - 1u));
    const int64_t rb = rbase[q];
    const int64_t ti = (int64_t)__builtin_amdgcn_readfirstlane((int)(rb & 0xffffffff)) +
                       ((int64_t)__builtin_amdgcn_readfirstlane((int)(rb >> 32)) << 32) + rank;
    return ti < capacity ? ti : -1;
  };

  // V tile of key block J -> LDS buffer with direct buffer->LDS loads (the same
  // load class as the tile reads, so the compiler's wait counts stay exact);
  // chunk c of row d is stored at chunk position c ^ (d % CPR).
  const uint16_t *vtg = vt + (int64_t)g * D * tpad;
  auto dma_v = [&](char *dstbuf, int J) {
    const int64_t col0 = (int64_t)(gr - I + J) * B;
#pragma unroll
    for (int i = 0; i < C::VINST; ++i) {
      const int blk = wave * C::VINST + i;        // 1 KB block of the tile
      const int d0 = blk * 64 / C::CPR;           // first row of the block
      const int k = blk * 64 + lane;              // 16-byte chunk index
      const int d = k / C::CPR, pp = k % C::CPR;
      const int c = pp ^ (d % C::CPR);
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          (void *)(vtg + (int64_t)d0 * tpad + col0), 0, 0x7fffffff, kBufferFlags);
      const int off = (int)(((int64_t)(d - d0) * tpad + c * 8) * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(dstbuf + blk * 1024), 16, off, 0, 0, 0);
    }
  };
  auto vread = [&](const char *vl, int d, int c) -> u32x4 {
    return *reinterpret_cast<const u32x4 *>(vl + d * C::VPITCH + ((c ^ (d % C::CPR)) << 4));
  };

  // lane row: wave * 16 + m16; keys of chunk kc: kc * 32 + 8 * kg + e
  const int r0 = wave * 16 + m16;
  // Tiles are stored in fragment order: the wave's 16 rows x 32 keys of chunk kc
  // are one contiguous 1 KB block, lane l's 16 bytes at l * 16.
  const int loff = wave * KC * 512 + lane * 8;  // lane offset inside a tile (elements)
  const uint16_t *rowbase = tiles + loff;
  f32x4 acc[D / 16];
#pragma unroll
  for (int nb = 0; nb < D / 16; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // translated row chunk (bf16) times the staged V tile
  auto finish_chunk = [&](float (&mix)[8], const char *vl, int kc) {
    u32x4 a;
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] = pack_bf16x2(mix[2 * e], mix[2 * e + 1]);
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) {
      const u32x4 b = vread(vl, nb * 16 + m16, kc * 4 + kg);
      acc[nb] = mfma16_bf16(as_bf16x8(a), as_bf16x8(b), acc[nb]);
    }
  };
  auto mix_src = [&](float (&mix)[8], const u32x4 &v, uint32_t c) {
    const uint32_t c_lo = c, c_hi = c << 16;
#pragma unroll
    for (int e = 0; e < 4; ++e) mix_word(mix[2 * e], mix[2 * e + 1], v[e], c_lo, c_hi);
  };

  // tile pointers and coefficients of the first four sources at key block J
  // Tile reads go through buffer descriptors (uniform base in scalar registers,
  // one shared lane offset).  A source without a tile at this key block gets a
  // zero-length descriptor: its loads return zeros without touching memory.
  const int voff = loff * 2;  // bytes
  struct Src4 {
    __amdgpu_buffer_rsrc_t r[4];
    uint32_t c[4];
  };
  auto src4 = [&](Src4 &S, int J) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int64_t ti = -1;
      if (J >= 0 && u < ns) ti = tile_of(u, J);
      S.r[u] = __builtin_amdgcn_make_buffer_rsrc(
          (void *)(tiles + (ti >= 0 ? ti : 0) * (int64_t)(B * B)), 0, ti >= 0 ? B * B * 2 : 0,
          kBufferFlags);
      S.c[u] = ti >= 0 ? (uint32_t)coef[u * B + r0] : 0u;
    }
  };
  auto load4 = [&](u32x4 (&dst)[4], const Src4 &S, int kc) {
#pragma unroll
    for (int u = 0; u < 4; ++u) dst[u] = __builtin_amdgcn_raw_buffer_load_b128(S.r[u], voff, kc * 1024, 0);
  };

  int J = (ns > 0) ? next_J(0) : -1;
  if (J >= 0) dma_v(vA, J);
  if constexpr (!MANY) {
    // at most four sources: one chunk of loads in flight ahead of the one
    // being mixed, across key-block boundaries
    Src4 Sc, Sn;
    src4(Sc, J);
    u32x4 ta[2][4];
    load4(ta[0], Sc, 0);  // zero-length descriptors when J < 0
    // one key block: mix + multiply from vl while V of the next block loads into vnext
    auto block = [&](int Jc, int Jn, const char *vl, char *vnext) {
      src4(Sn, Jn);
      // Own V loads for this block have landed (vector-memory loads retire in
      // issue order and only the four loads of the prefetched chunk are
      // younger) and own LDS reads are done; then the work-group barrier.  No
      // full fence here: it would also drain the prefetched chunk.
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0x0074);  // vmcnt(4) lgkmcnt(0)
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      dma_v(vnext, Jn >= 0 ? Jn : Jc);  // unconditional (keeps wait counts static)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        // (unconditional: a missing next block has zero-length descriptors, so
        // the wait counts stay static)
        if (kc + 1 < KC)
          load4(ta[(kc + 1) & 1], Sc, kc + 1);
        else
          load4(ta[KC & 1], Sn, 0);
        // keep the prefetch ahead of this chunk's work (the scheduler would
        // otherwise sink it next to its first use)
        __builtin_amdgcn_sched_barrier(0);
        float mix[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) mix[e] = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) mix_src(mix, ta[kc & 1][u], Sc.c[u]);
        finish_chunk(mix, vl, kc);
      }
      if constexpr (KC & 1) {
        // odd chunk count: the next block's first chunk went to buffer 1
#pragma unroll
        for (int u = 0; u < 4; ++u) ta[0][u] = ta[1][u];
      }
      Sc = Sn;
    };
    // two blocks per trip so each one's V buffers are fixed arrays
    while (J >= 0) {
      int Jn = next_J(J + 1);
      block(J, Jn, vA, vB);
      J = Jn;
      if (J < 0) break;
      Jn = next_J(J + 1);
      block(J, Jn, vB, vA);
      J = Jn;
    }
  } else {
    int buf = 0;
    while (J >= 0) {
      const int Jn = next_J(J + 1);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (Jn >= 0) dma_v(buf ? vA : vB, Jn);
      const char *vl = buf ? vB : vA;
      // many sources: chunk by chunk, four sources at a time
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        float mix[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) mix[e] = 0.f;
        for (int q0 = 0; q0 < ns; q0 += 4) {
          u32x4 va[4];
          uint32_t cl[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            cl[u] = 0u;
            const int q = q0 + u;
            if (q >= ns) continue;
            const int64_t ti = tile_of(q, J);
            if (ti < 0) continue;
            va[u] = *reinterpret_cast<const u32x4 *>(rowbase + ti * (int64_t)(B * B) + kc * 512);
            cl[u] = (uint32_t)coef[q * B + r0];
          }
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (cl[u] != 0u) mix_src(mix, va[u], cl[u]);
        }
        finish_chunk(mix, vl, kc);
      }
      buf ^= 1;
      J = Jn;
    }
  }

  float *ot = o + (int64_t)t * T * D;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int ip = I * B + wave * 16 + 4 * kg + r;
    if (ip < L) {
      float *dst = ot + (tok0 + ip) * D + m16;
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb) dst[nb * 16] = acc[nb][r];
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
  if (smem > 64 * 1024) {
    hipFuncSetAttribute(reinterpret_cast<const void *>(&k_apply<B, D, false>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    hipFuncSetAttribute(reinterpret_cast<const void *>(&k_apply<B, D, true>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  }
  const int64_t npos = ((int64_t)g.NBR + kXcds - 1) / kXcds * kXcds;
  // one launch per source-count class; a work-group whose target is of the other
  // class returns right after reading its weight row
  hipLaunchKernelGGL((k_apply<B, D, false>), dim3((unsigned)(npos * Ht)), dim3(B * 4), smem, s,
                     map->row_ptr, map->col_idx, map->tiles, map->kept_mass, map->num_heads,
                     g.NBR, g.T, W, Ht, Ht / Hkv, at<uint16_t>(ws, w.vt),
                     at<RowInfo>(ws, w.rt.rows), at<int32_t>(ws, w.rt.sched), nbw, map->capacity_tiles, renorm, o);
  if (hip_status() != MF_OK) return MF_ERR_HIP;
  hipLaunchKernelGGL((k_apply<B, D, true>), dim3((unsigned)(npos * Ht)), dim3(B * 4), smem, s,
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
