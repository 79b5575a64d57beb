// Receiver-side fused retrieval with linear head translation (MapFlow,
// "Accelerating Cross-Model LLM Inference via Attention Map Reuse", §3.3 linear
// head mapping, §5.4 attention retrieval with a fused kernel):
//
//   O_t[i,:] = sum_h W[t,h] sum_{J kept by h} sum_{j in J} (A_h[i,j] / kmass_h[i]) V_g(t)[j,:]
//
// Per (target head, query block) and key block J in the union of the sources'
// kept sets, each lane rebuilds its row of the translated tile
// A~_t[i, J] = sum_h c_h[i] A_h[i, J] in fp32 registers straight from the bf16
// tiles (c_h[i] = W[t,h] / kmass_h[i]), rounds it to bf16 and feeds it as the A
// operand of 16x16x32 MFMAs against V_g(t)[J] staged in LDS.  The translated
// map never leaves registers; nothing of size L x L is written.  k_apply4 takes
// targets with at most four sources, k_apply_mix the others.
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
// V -> Vt [Hkv][D][NBR * B], zero past each sequence end.
//
// V is either contiguous [Hkv][T][D] or paged: token j of sequence s lives in
// page block_table[s][j / P] of a pool [pages][Hkv][P][D] at slot j % P (page
// indices outside the pool read as zeros).  With query windows (chunked prefill)
// only key blocks below the window's end are staged: no other block is read.
// ---------------------------------------------------------------------------
struct VSrc {
  const uint16_t *v;          // contiguous V, or null
  const uint16_t *pages;      // paged pool, or null
  const int32_t *table;       // [nseq][max_pages]
  int32_t page_size, max_pages, num_pages, Hkv;
  const int32_t *window;      // [nseq][2] query tokens [begin, end), or null
};

template <int B, int D>
__global__ __launch_bounds__(256) void k_vtranspose(VSrc vs, int64_t T,
                                                    const RowInfo *__restrict__ rows, int32_t NBR,
                                                    uint16_t *__restrict__ vt) {
  constexpr int P = B + 8;  // LDS row pitch in elements
  __shared__ __attribute__((aligned(16))) uint16_t t[D * P];
  const int gr = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const RowInfo ri = rows[gr];
  if (vs.window && ri.blk * B >= vs.window[2 * ri.seq + 1]) return;  // not a key of the window
  const int nval = min(B, ri.len - ri.blk * B);
  const int64_t tok0 = (int64_t)ri.start + (int64_t)ri.blk * B;
  for (int idx = tid; idx < B * D / 8; idx += 256) {
    const int j = idx / (D / 8), c = idx % (D / 8);
    u32x4 x = u32x4{0u, 0u, 0u, 0u};
    if (j < nval) {
      const uint16_t *row = nullptr;
      if (vs.pages) {
        const int js = ri.blk * B + j;  // token index inside the sequence
        const int pg = vs.table[(int64_t)ri.seq * vs.max_pages + js / vs.page_size];
        if (pg >= 0 && pg < vs.num_pages)
          row = vs.pages + (((int64_t)pg * vs.Hkv + g) * vs.page_size + js % vs.page_size) * D;
      } else {
        row = vs.v + ((int64_t)g * T + tok0 + j) * D;
      }
      if (row) x = *reinterpret_cast<const u32x4 *>(row + c * 8);
    }
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

// Schedule of the block-rows inside the query windows, in the longest-first
// order of the full schedule (stable compaction, one work-group).
__global__ __launch_bounds__(1024) void k_window_sched(const RowInfo *__restrict__ rows,
                                                       const int32_t *__restrict__ sched,
                                                       int32_t NBR, int32_t B,
                                                       const int32_t *__restrict__ window,
                                                       int32_t *__restrict__ wsched) {
  __shared__ int32_t wsum[16];
  __shared__ int32_t base;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) base = 0;
  __syncthreads();
  for (int p0 = 0; p0 < NBR; p0 += 1024) {
    const int p = p0 + tid;
    int gr = -1;
    bool keep = false;
    if (p < NBR) {
      gr = sched[p];
      const RowInfo ri = rows[gr];
      const int a = ri.blk * B;
      keep = a >= window[2 * ri.seq] && a < window[2 * ri.seq + 1];
    }
    const uint64_t mask = wave_ballot(keep);
    if (lane == 0) wsum[wave] = __popcll(mask);
    __syncthreads();
    int off = base;
    for (int w = 0; w < wave; ++w) off += wsum[w];
    if (keep) wsched[off + lanes_below(mask)] = gr;
    __syncthreads();
    if (tid == 0) {
      int tot = 0;
      for (int w = 0; w < 16; ++w) tot += wsum[w];
      base += tot;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// per (target, query block) set-up shared by both apply kernels
// ---------------------------------------------------------------------------
// Dynamic LDS (byte offsets; the V buffers are static): rbase[Hs] int64,
// src[Hs], wt[Hs], bm[Hs][nbw], pc[Hs][nbw], uni[nbw], coef[Hs][B] (bf16 bits), nsrc.
// k_apply4 appends the union's key-block list: blist[nbw * 32] int32 and
// tix[nbw * 32][4] int32 (tile index of each of up to four sources, -1 if none).
inline size_t apply_smem(int B, int Hs, int nbw) {
  size_t s = (size_t)Hs * (8 + 4 + 4);
  s += (size_t)Hs * nbw * 8 + (size_t)nbw * 4;
  s += (size_t)Hs * B * 2;
  s += 64;
  s += (size_t)nbw * 32 * 5 * 4;
  return s;
}

// LDS views of one (target, query block)'s source maps
struct RowMaps {
  int64_t *rbase;   // first tile of each source's block-row
  int32_t *src;     // source heads with a nonzero weight
  float *wt;        // their weights
  uint32_t *bm;     // kept bitmaps [source][nbw]
  int32_t *pc;      // exclusive popcount prefix of bm (tile rank of each word)
  uint32_t *uni;    // union of the kept bitmaps
  uint16_t *coef;   // [source][B] row coefficients W[t,h] / kmass_h[i], bf16 bits
  int32_t *nsrc;
  int32_t *tix;     // [k][4] tile index of source u at the k-th union block, -1 if none
  int32_t *blist;   // [k] the k-th key block of the union, ascending
  int nbw;
};

// byte offsets, kept relative to smem so every access stays an LDS access
__device__ __forceinline__ RowMaps row_maps(char *smem, int Hs, int nbw, int B) {
  const int o_rbase = 0;
  const int o_src = o_rbase + Hs * 8;
  const int o_wt = o_src + Hs * 4;
  const int o_bm = o_wt + Hs * 4;
  const int o_pc = o_bm + Hs * nbw * 4;
  const int o_uni = o_pc + Hs * nbw * 4;
  const int o_coef = o_uni + nbw * 4;
  const int o_ns = (o_coef + Hs * B * 2 + 3) & ~3;
  const int o_tix = (o_ns + 4 + 15) & ~15;
  const int o_blist = o_tix + nbw * 32 * 16;
  RowMaps m;
  m.rbase = reinterpret_cast<int64_t *>(smem + o_rbase);
  m.src = reinterpret_cast<int32_t *>(smem + o_src);
  m.wt = reinterpret_cast<float *>(smem + o_wt);
  m.bm = reinterpret_cast<uint32_t *>(smem + o_bm);
  m.pc = reinterpret_cast<int32_t *>(smem + o_pc);
  m.uni = reinterpret_cast<uint32_t *>(smem + o_uni);
  m.coef = reinterpret_cast<uint16_t *>(smem + o_coef);
  m.nsrc = reinterpret_cast<int32_t *>(smem + o_ns);
  m.tix = reinterpret_cast<int32_t *>(smem + o_tix);
  m.blist = reinterpret_cast<int32_t *>(smem + o_blist);
  m.nbw = nbw;
  return m;
}

// Sources of target t (nonzero weights, ascending head order) and the start of
// their tile runs at block-row gr; clears the bitmaps.  Returns the source count
// (uniform).
template <int NT>
__device__ int row_sources(const RowMaps &m, const float *__restrict__ W, int t, int Hs,
                           const int64_t *__restrict__ row_ptr, int NBR, int gr, int tid) {
  if (tid < 64) {
    // wave 0 scans the weight row 64 heads at a time, compacting by ballot
    int ns = 0;
    for (int h0 = 0; h0 < Hs; h0 += 64) {
      const int h = h0 + tid;
      const float w = h < Hs ? W[(int64_t)t * Hs + h] : 0.f;
      const uint64_t mask = wave_ballot(w != 0.f);
      if (w != 0.f) {
        const int q = ns + lanes_below(mask);
        m.src[q] = h;
        m.wt[q] = w;
        m.rbase[q] = row_ptr[(int64_t)h * NBR + gr];
      }
      ns += __popcll(mask);
    }
    if (tid == 0) *m.nsrc = ns;
  }
  for (int i = tid; i < Hs * m.nbw; i += NT) m.bm[i] = 0u;
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*m.nsrc);
}

// Kept bitmaps of the ns sources at block-row gr, their tile ranks, the union
// bitmap and the per-row coefficients (bf16): W[t,h] / kmass_h[i] when
// renormalising (0 where the kept mass is 0), else W[t,h]; rows past the
// sequence end get 0.
template <int B, int NT>
__device__ void row_maps_fill(const RowMaps &m, int ns, const int64_t *__restrict__ row_ptr,
                              const int32_t *__restrict__ col_idx, int64_t capacity,
                              const float *__restrict__ kept_mass, int64_t T, int NBR, int gr,
                              int64_t tok0, int I, int L, int nw_row, int renorm, int tid) {
  for (int q = 0; q < ns; ++q) {
    // entries past the capacity of an overflowed map are treated as missing
    const int64_t b = m.rbase[q], e = min(row_ptr[(int64_t)m.src[q] * NBR + gr + 1], capacity);
    for (int64_t idx = b + tid; idx < e; idx += NT) {
      const int J = col_idx[idx];
      atomicOr(&m.bm[q * m.nbw + (J >> 5)], 1u << (J & 31));
    }
  }
  for (int idx = tid; idx < ns * B; idx += NT) {
    const int q = idx / B, il = idx % B;
    const int ip = I * B + il;
    float c = 0.f;
    if (ip < L) {
      if (renorm) {
        const float km = kept_mass[(int64_t)m.src[q] * T + tok0 + ip];
        c = km > 0.f ? m.wt[q] / km : 0.f;
      } else {
        c = m.wt[q];
      }
    }
    m.coef[q * B + il] = (uint16_t)pack_bf16x2(c, 0.f);
  }
  __syncthreads();
  for (int q = tid; q < ns; q += NT) {
    int run = 0;
    for (int w = 0; w < nw_row; ++w) {
      m.pc[q * m.nbw + w] = run;
      run += __popc(m.bm[q * m.nbw + w]);
    }
  }
  if (tid < nw_row) {
    uint32_t u = 0u;
    for (int q = 0; q < ns; ++q) u |= m.bm[q * m.nbw + tid];
    m.uni[tid] = u;
  }
  __syncthreads();
}

// next key block of the union at or after `from` (uniform), -1 if none
__device__ __forceinline__ int union_next(const RowMaps &m, int n, int from) {
  if (from < 0 || from >= n) return -1;
  const int nw_row = (n + 31) / 32;
  for (int w = from >> 5; w < nw_row; ++w) {
    uint32_t bits = __builtin_amdgcn_readfirstlane(m.uni[w]);
    if (w == (from >> 5)) bits &= ~((1u << (from & 31)) - 1u);
    if (bits) return w * 32 + __ffs(bits) - 1;
  }
  return -1;
}

// tile index of source q at key block J, or -1 (uniform)
__device__ __forceinline__ int64_t tile_index(const RowMaps &m, int q, int J, int64_t capacity) {
  const uint32_t word = __builtin_amdgcn_readfirstlane(m.bm[q * m.nbw + (J >> 5)]);
  if (!((word >> (J & 31)) & 1u)) return -1;
  const int rank = __builtin_amdgcn_readfirstlane(m.pc[q * m.nbw + (J >> 5)]) +
                   __popc(word & ((1u << (J & 31)) - 1u));
  const int64_t rb = m.rbase[q];
  const int64_t ti = (int64_t)__builtin_amdgcn_readfirstlane((int)(rb & 0xffffffff)) +
                     ((int64_t)__builtin_amdgcn_readfirstlane((int)(rb >> 32)) << 32) + rank;
  return ti < capacity ? ti : -1;
}

// The union's key blocks in ascending order with the tile index of each of the
// (at most four) sources at each block; returns the number of blocks (uniform).
template <int NT>
__device__ int build_block_list(const RowMaps &m, int ns, int n, int64_t capacity, int tid) {
  const int nw_row = (n + 31) / 32;
  for (int J = tid; J < n; J += NT) {
    const uint32_t w = m.uni[J >> 5];
    if (!((w >> (J & 31)) & 1u)) continue;
    int k = __popc(w & ((1u << (J & 31)) - 1u));
    for (int i = 0; i < (J >> 5); ++i) k += __popc(m.uni[i]);
    m.blist[k] = J;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int32_t ti = -1;
      if (u < ns) {
        const uint32_t word = m.bm[u * m.nbw + (J >> 5)];
        if ((word >> (J & 31)) & 1u) {
          const int64_t x = m.rbase[u] + m.pc[u * m.nbw + (J >> 5)] +
                            __popc(word & ((1u << (J & 31)) - 1u));
          if (x < capacity) ti = (int32_t)x;
        }
      }
      m.tix[k * 4 + u] = ti;
    }
  }
  int total = 0;
  for (int i = 0; i < nw_row; ++i) total += __popc(m.uni[i]);
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(total);
}

// work-group id -> (schedule position, target): consecutive ids land on XCDs in
// turn; XCD x takes every eighth query block of the longest-first order, all
// targets of one block before the next, zig-zagging between rounds so the XCDs
// stay in step and share V through the memory-side cache.
__device__ __forceinline__ void xcd_map(int Ht, int &pos, int &t) {
  const int x = blockIdx.x % kXcds, kx = blockIdx.x / kXcds;
  const int round = kx / Ht;
  t = kx % Ht;
  pos = round * kXcds + ((round & 1) ? (kXcds - 1 - x) : x);
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

// V tile of key block J -> LDS buffer with direct buffer->LDS loads (the same
// load class as the tile reads, so the compiler's wait counts stay exact); the
// wave moves VINST 1 KB blocks.  16-byte chunk c of row d is stored at chunk
// position c ^ (d % CPR), so the MFMA B-operand reads below are conflict-free.
template <int B, int D, int VINST>
__device__ __forceinline__ void dma_v_tile(char *dstbuf, const uint16_t *vtg, int64_t tpad,
                                           int64_t col0, int wave, int lane) {
  constexpr int CPR = B * 2 / 16;   // 16-byte chunks per row
  constexpr int RPB = 64 / CPR;     // rows per 1 KB block
  // the swizzle of a block's rows repeats every PER blocks: the lane part of
  // the offset takes PER values, the row part d0 * tpad * 2 is uniform
  constexpr int PER = CPR * CPR / 64 > 1 ? CPR * CPR / 64 : 1;
  // one descriptor per tile; byte offsets d * tpad * 2 stay below 2^31 (checked
  // by the host)
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void *)(vtg + col0), 0, 0x7fffffff, kBufferFlags);
  const int dl = lane / CPR, pp = lane % CPR;
#pragma unroll
  for (int i = 0; i < VINST; ++i) {
    const int blk = wave * VINST + i;        // 1 KB block of the tile
    const int d0 = blk * RPB;                // its first row
    const int c = pp ^ ((d0 + dl) % CPR);    // swizzled chunk position
    (void)PER;
    const int voff = (dl * (int)tpad + c * 8) * 2;
    const int soff = d0 * (int)tpad * 2;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(dstbuf + blk * 1024), 16, voff, soff, 0, 0);
  }
}

template <int B>
__device__ __forceinline__ u32x4 v_frag(const char *vl, int d, int c) {
  constexpr int CPR = B * 2 / 16;
  return *reinterpret_cast<const u32x4 *>(vl + d * (B * 2) + ((c ^ (d % CPR)) << 4));
}

// ---------------------------------------------------------------------------
// k_apply4: targets with at most four sources (the translated map of a
// head-mapping row).  One work-group per (target, query block), one wave per
// RG 16-row MFMA groups.  The union's key blocks and each source's tile index
// there are listed once in LDS, so stepping to the next block is one broadcast
// read.
//
// Tile chunks (32 keys x 16 rows, 1 KB, fragment order) stream through a
// register ring of NR chunk slots, NR - 1 chunks ahead of the one being mixed,
// across key-block boundaries; V tiles go straight to a double LDS buffer one
// key block ahead.  Loads of sources without a tile at a key block (and past
// the last block) use zero-length descriptors: they return zeros without
// touching memory and keep the number of loads in flight static.
// ---------------------------------------------------------------------------
constexpr int cgcd(int a, int b) { return b == 0 ? a : cgcd(b, a % b); }

template <int B, int D, int FMT>
struct Apply4Cfg {
  static constexpr int RG = 1;                       // 16-row MFMA groups per wave
  static constexpr int NW = B / (16 * RG);           // waves
  static constexpr int NT = NW * 64;
  static constexpr int KC = B / 32;                  // 32-key chunks per key block
  // a ring unit is one load per source: a 32-key chunk of bf16 (16 bytes per
  // lane), or NP chunks of E4M3 codes (8 NP bytes per lane)
  static constexpr int NP = (FMT == MF_TILE_MXFP8 && B >= 64) ? 2 : 1;
  static constexpr int KU = KC / NP;                 // units per key block
  static constexpr int64_t TBYTES = tile_bytes(B, FMT);
  static constexpr int VBYTES = D * B * 2;
  static constexpr int VINST = VBYTES / 1024 / NW;   // 1 KB direct loads per wave per V tile
  // Ring slots (chunks).  Two, i.e. one chunk ahead.  About eight work-groups
  // of one query block read every source tile, and they hit in the XCD's L2
  // only while its recent tiles still fit there; deeper prefetch lowers that
  // hit rate (measured at L = 32K: 54% with two slots, 12% with four, and
  // twice the fabric traffic); 32-row waves with more slots lose the same way.
  static constexpr int NR = 2;
  // loads per unit: row groups x 4 sources, plus 4 scale loads with a block's first unit
  static constexpr int LPC = 4 * RG + (FMT == MF_TILE_MXFP8 ? 4 : 0);
  // key blocks per unrolled trip: ring slots and V buffers both return to their start
  static constexpr int TB = (NR * 2 * KU / cgcd(NR, 2 * KU)) / KU;
  // descriptor queue depth: blocks from the current one to the farthest prefetched
  static constexpr int DQ = (KU - 1 + NR - 1) / KU + 1;
  static_assert(VINST * 1024 * NW == VBYTES, "V tile must split into 1 KB wave loads");
  static_assert(TB % 2 == 0 && (TB * KU) % NR == 0, "trip must close the ring and V buffers");
  static_assert((NR - 1) * LPC + VINST <= 63, "vmcnt range");
  static_assert(FMT == MF_TILE_BF16 || RG == 1, "fp8 tiles take one row group per wave");
};


template <int B, int D, int FMT>
__global__ __launch_bounds__(B * 4) __attribute__((amdgpu_waves_per_eu(4))) void k_apply4(
    const int64_t *__restrict__ row_ptr, const int32_t *__restrict__ col_idx,
    const char *__restrict__ tiles, const float *__restrict__ kept_mass, int32_t Hs,
    int32_t NBR, int64_t T, const float *__restrict__ W, int32_t Ht, int32_t grp,
    const uint16_t *__restrict__ vt, const RowInfo *__restrict__ rows,
    const int32_t *__restrict__ sched, int32_t nrows, int32_t nbw, int64_t capacity,
    int32_t renorm, float *__restrict__ o, const int32_t *__restrict__ row_alias) {
  using C = Apply4Cfg<B, D, FMT>;
  constexpr int KU = C::KU, NP = C::NP, NR = C::NR, TB = C::TB, DQ = C::DQ;
  constexpr bool FP8 = FMT == MF_TILE_MXFP8;
  // separate arrays, so the compiler can tell that direct loads into one never
  // alias reads of the other
  __shared__ __attribute__((aligned(16))) char vA[C::VBYTES];
  __shared__ __attribute__((aligned(16))) char vB[C::VBYTES];
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const RowMaps mp = row_maps(smem, Hs, nbw, B);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m16 = lane & 15, kg = lane >> 4;
  int pos, t;
  xcd_map(Ht, pos, t);
  if (pos >= nrows) return;
  const int gr = sched[pos];
  const RowInfo ri = rows[gr];
  const int I = ri.blk, L = ri.len;
  const int n = I + 1;
  const int g = t / grp;
  const int64_t tok0 = (int64_t)ri.start;
  const int64_t tpad = (int64_t)NBR * B;

  // BSR row of this block-row: its own, or that of the earlier block-row it
  // shares (tiles and kept masses are equal; V and O stay this row's own)
  const int ga = row_alias ? row_alias[gr] : gr;
  const int grm = (ga >= 0 && ga < NBR) ? ga : gr;
  const int ns = row_sources<C::NT>(mp, W, t, Hs, row_ptr, NBR, grm, tid);
  if (ns > 4) return;  // handled by k_apply_mix
  row_maps_fill<B, C::NT>(mp, ns, row_ptr, col_idx, capacity, kept_mass, T, NBR, grm, tok0, I, L,
                          (n + 31) / 32, renorm, tid);

  // coefficients of this lane's two rows, [c, 0] and [0, c] bf16 pairs (zero
  // for missing sources)
  constexpr int RG = C::RG;
  uint32_t clo[RG][4];
#pragma unroll
  for (int h = 0; h < RG; ++h)
#pragma unroll
    for (int u = 0; u < 4; ++u)
      clo[h][u] = u < ns ? (uint32_t)mp.coef[u * B + wave * 16 * RG + 16 * h + m16] : 0u;

  const int nblk = build_block_list<C::NT>(mp, ns, n, capacity, tid);

  // k-th block of the union (uniform), -1 past the end
  auto blk_J = [&](int k) -> int {
    return k < nblk ? __builtin_amdgcn_readfirstlane(mp.blist[k]) : -1;
  };
  // tile descriptors of the k-th union block; zero-length for a source without
  // a tile there and past the last block
  struct Src4 {
    __amdgpu_buffer_rsrc_t r[4];
  };
  auto src4 = [&](Src4 &S, int k) {
    u32x4 ti4 = u32x4{~0u, ~0u, ~0u, ~0u};
    if (k < nblk) ti4 = *reinterpret_cast<const u32x4 *>(mp.tix + k * 4);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ti = __builtin_amdgcn_readfirstlane((int)ti4[u]);
      S.r[u] = __builtin_amdgcn_make_buffer_rsrc(
          (void *)(tiles + (int64_t)(ti >= 0 ? ti : 0) * C::TBYTES), 0,
          ti >= 0 ? (int)C::TBYTES : 0, kBufferFlags);
    }
  };
  // unit ku of the wave's row groups: bf16, the 1 KB fragment block (row group,
  // chunk ku), lane l's 16 bytes at l * 16; fp8, the (row group, piece ku)
  // block of 512 NP bytes, lane l's 8 NP bytes at l * 8 NP
  const int voff = FP8 ? (wave * KU * 64 + lane) * 8 * NP : (RG * wave * KU * 64 + lane) * 16;
  auto load_chunk = [&](u32x4 (&dst)[RG][4], const Src4 &S, int ku) {
#pragma unroll
    for (int h = 0; h < RG; ++h)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if constexpr (!FP8) {
          dst[h][u] = __builtin_amdgcn_raw_buffer_load_b128(S.r[u], voff, (h * KU + ku) * 1024, 0);
        } else if constexpr (NP == 2) {
          dst[h][u] = __builtin_amdgcn_raw_buffer_load_b128(S.r[u], voff, ku * 1024, 0);
        } else {
          const auto d2 = __builtin_amdgcn_raw_buffer_load_b64(S.r[u], voff, ku * 512, 0);
          dst[h][u] = u32x4{d2[0], d2[1], 0u, 0u};
        }
      }
  };
  // scale bytes of the lane's row (B/32 of them, one per chunk), fp8 only
  const int soff_lane = (wave * 16 + m16) * (B / 32);
  auto load_scales = [&](uint32_t (&sc)[4], const Src4 &S) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if constexpr (B == 128)
        sc[u] = __builtin_amdgcn_raw_buffer_load_b32(S.r[u], soff_lane, B * B, 0);
      else if constexpr (B == 64)
        sc[u] = __builtin_amdgcn_raw_buffer_load_b16(S.r[u], soff_lane, B * B, 0);
      else
        sc[u] = __builtin_amdgcn_raw_buffer_load_b8(S.r[u], soff_lane, B * B, 0);
    }
  };

  const uint16_t *vtg = vt + (int64_t)g * D * tpad;
  auto dma_v = [&](char *dstbuf, int J) {
    dma_v_tile<B, D, C::VINST>(dstbuf, vtg, tpad, (int64_t)(gr - I + J) * B, wave, lane);
  };

  f32x4 acc[RG][D / 16];
#pragma unroll
  for (int h = 0; h < RG; ++h)
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) acc[h][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fp8: coefficients as fp32, scaled per chunk by the tile's block scale
  float cf[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) cf[u] = __uint_as_float(clo[0][u] << 16);

  if (nblk > 0) {
    // queue of tile descriptors: S[k] for the (cur + k)-th union block
    Src4 S[DQ];
#pragma unroll
    for (int k = 0; k < DQ; ++k) src4(S[k], k);
    u32x4 ring[NR][RG][4];
    uint32_t sc[2][4];  // fp8 scale words of blocks with even / odd trip position
    // prologue: the first V tile and units 0 .. NR-2
    dma_v(vA, blk_J(0));
#pragma unroll
    for (int p = 0; p < NR - 1; ++p) {
      load_chunk(ring[p], S[p / KU], p % KU);
      if constexpr (FP8)
        if (p % KU == 0) load_scales(sc[(p / KU) & 1], S[p / KU]);
    }
    int cur = 0;  // list position of the block being multiplied
    bool done = false;
    while (!done) {
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        if (done) break;
        const char *vcur = (tb & 1) ? vB : vA;
        char *vnxt = (tb & 1) ? vA : vB;
        const int Jc = blk_J(cur), Jn = blk_J(cur + 1);
        // block start: this wave's part of V(Jc) has landed and its LDS reads of
        // the previous block are done; then the work-group barrier.  The wait
        // is a full drain: direct-to-LDS loads are not ordered with loads into
        // registers, so no partial count proves that V has landed.  Besides V
        // only this block's first chunk is in flight, and it is needed next.
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        dma_v(vnxt, Jn >= 0 ? Jn : Jc);  // unconditional: static wait counts
#pragma unroll
        for (int ku = 0; ku < KU; ++ku) {
          const int pc = tb * KU + ku;          // unit position in the trip
          const int pf = ku + NR - 1;           // prefetched unit, relative to this block
          load_chunk(ring[(pc + NR - 1) % NR], S[pf / KU], pf % KU);
          if constexpr (FP8)
            if (pf % KU == 0) load_scales(sc[(tb + pf / KU) & 1], S[pf / KU]);
          // keep the prefetch ahead of this unit's work (the scheduler would
          // otherwise sink it next to its first use)
          __builtin_amdgcn_sched_barrier(0);
          const u32x4(&cr)[RG][4] = ring[pc % NR];
#pragma unroll
          for (int sub = 0; sub < NP; ++sub) {
            const int kc = ku * NP + sub;       // 32-key chunk of the block
            u32x4 a[RG];
#pragma unroll
            for (int h = 0; h < RG; ++h) {
              float mx[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) mx[e] = 0.f;
              if constexpr (!FP8) {
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                  for (int e = 0; e < 4; ++e)
                    mix_word(mx[2 * e], mx[2 * e + 1], cr[h][u][e], clo[h][u], clo[h][u] << 16);
              } else {
                // code_value * 2^(scale byte - 127), the scale folded into c
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                  const int sb = (int)((sc[tb & 1][u] >> (8 * kc)) & 0xffu);
                  const float c = __builtin_amdgcn_ldexpf(cf[u], sb - 127);
#pragma unroll
                  for (int w = 0; w < 2; ++w) {
                    const uint32_t codes = cr[h][u][2 * sub + w];
                    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(codes, false);
                    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(codes, true);
                    mx[4 * w + 0] = fmaf(c, lo[0], mx[4 * w + 0]);
                    mx[4 * w + 1] = fmaf(c, lo[1], mx[4 * w + 1]);
                    mx[4 * w + 2] = fmaf(c, hi[0], mx[4 * w + 2]);
                    mx[4 * w + 3] = fmaf(c, hi[1], mx[4 * w + 3]);
                  }
                }
              }
#pragma unroll
              for (int e = 0; e < 4; ++e) a[h][e] = pack_bf16x2(mx[2 * e], mx[2 * e + 1]);
            }
#pragma unroll
            for (int nb = 0; nb < D / 16; ++nb) {
              const u32x4 bv = v_frag<B>(vcur, nb * 16 + m16, kc * 4 + kg);
#pragma unroll
              for (int h = 0; h < RG; ++h)
                acc[h][nb] = mfma16_bf16(as_bf16x8(a[h]), as_bf16x8(bv), acc[h][nb]);
            }
          }
        }
        // advance the queue
#pragma unroll
        for (int k = 0; k + 1 < DQ; ++k) S[k] = S[k + 1];
        src4(S[DQ - 1], cur + DQ);
        ++cur;
        done = cur >= nblk;
      }
    }
    // drain the prefetches of blocks that do not exist before the wave ends
    __builtin_amdgcn_s_waitcnt(0);
  }

  float *ot = o + (int64_t)t * T * D;
#pragma unroll
  for (int h = 0; h < RG; ++h)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ip = I * B + wave * 16 * RG + 16 * h + 4 * kg + r;
      if (ip < L) {
        float *dst = ot + (tok0 + ip) * D + m16;
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb) __builtin_nontemporal_store(acc[h][nb][r], dst + nb * 16);
      }
    }
}

// ---------------------------------------------------------------------------
// k_apply_mix: targets with more than four sources (dense head mixing).
//
// One work-group per (query block, group of G consecutive targets); one wave
// per 16 query rows, for all G targets.  Every source tile chunk (16 rows x 32
// keys, one 1 KB fragment block) is loaded once per work-group and mixed into
// the G translated rows.  Sources go two at a time: v_perm_b32 pairs their e-th
// elements into one bf16 pair [P1[e], P2[e]], and one v_dot2 with the
// coefficient pair [c1, c2] adds both products, so every instruction does two
// multiply-adds and the pairing is shared by the G targets.  The coefficients
// are c = W[t,h] / kmass_h[i] (bf16).
//
// Per key block of the union, the block's V tiles (one per distinct V head of
// the group) load into LDS while the first 32-key chunk is mixed; then a full
// drain and a barrier; then each chunk's bf16 mix is multiplied with V on MFMA
// right after it is built; a barrier frees the V buffer for the next block.
// Within a chunk, the next batch of source chunks loads while the current one
// is mixed.
// ---------------------------------------------------------------------------
template <int B, int D, int FMT>
struct ApplyMixCfg {
  static constexpr int G = (4 * D * B * 2 <= 64 * 1024) ? 4 : 2;  // targets per work-group
  static constexpr int NW = B / 16;                 // waves, 16 rows each
  static constexpr int NT = NW * 64;
  static constexpr int KC = B / 32;                 // 32-key chunks per key block
  static constexpr int VBYTES = D * B * 2;
  static constexpr int VINST = VBYTES / 1024 / NW;  // 1 KB direct loads per wave per V tile
  static constexpr int SB = 4;                      // sources per load batch (two pairs)
  static constexpr int NP = (FMT == MF_TILE_MXFP8 && B >= 64) ? 2 : 1;  // fp8 chunks per piece
  static constexpr int64_t TBYTES = tile_bytes(B, FMT);
  static_assert(VINST * 1024 * NW == VBYTES, "V tile must split into 1 KB wave loads");
  static_assert(G * VBYTES <= 64 * 1024, "V buffers must stay in the first 64 KB of LDS");
};
constexpr int kMixMaxSources = 128;

// Dynamic LDS of k_apply_mix (byte offsets): src[Hs] int32, rbase[Hs] int64,
// wtab[Hs][4] fp32 (weight of each source for each target of the group),
// bm[Hs][nbw], pc[Hs][nbw], uni[nbw], rtab[Hs][B] fp32 (1 / kept mass of each
// row, 0 where none), blist[nbw * 32], counters.
inline size_t mix_smem(int B, int Hs, int nbw) {
  size_t s = (size_t)Hs * (4 + 8 + 16);
  s += (size_t)Hs * nbw * 8 + (size_t)nbw * 4;
  s += (size_t)Hs * B * 4;
  s += (size_t)nbw * 32 * 4;
  s += 64 + 64;
  return s;
}

template <int B, int D, int FMT>
__global__ __launch_bounds__(B * 4) __attribute__((amdgpu_waves_per_eu(2))) void k_apply_mix(
    const int64_t *__restrict__ row_ptr, const int32_t *__restrict__ col_idx,
    const char *__restrict__ tiles, const float *__restrict__ kept_mass, int32_t Hs,
    int32_t NBR, int64_t T, const float *__restrict__ W, int32_t Ht, int32_t grp,
    const uint16_t *__restrict__ vt, const RowInfo *__restrict__ rows,
    const int32_t *__restrict__ sched, int32_t nrows, int32_t nbw, int64_t capacity,
    int32_t renorm, float *__restrict__ o, const int32_t *__restrict__ row_alias) {
  using C = ApplyMixCfg<B, D, FMT>;
  constexpr int G = C::G, KC = C::KC, SB = C::SB, NP = C::NP;
  constexpr bool FP8 = FMT == MF_TILE_MXFP8;
  __shared__ __attribute__((aligned(16))) char vbuf[G * C::VBYTES];
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int o_src = 0;
  const int o_rbase = (o_src + Hs * 4 + 7) & ~7;
  const int o_wt = o_rbase + Hs * 8;
  const int o_bm = o_wt + Hs * 16;
  const int o_pc = o_bm + Hs * nbw * 4;
  const int o_uni = o_pc + Hs * nbw * 4;
  const int o_rt = o_uni + nbw * 4;
  const int o_bl = o_rt + Hs * B * 4;
  const int o_misc = o_bl + nbw * 32 * 4;
  int32_t *src = reinterpret_cast<int32_t *>(smem + o_src);
  int64_t *rbase = reinterpret_cast<int64_t *>(smem + o_rbase);
  float *wtab = reinterpret_cast<float *>(smem + o_wt);
  uint32_t *bm = reinterpret_cast<uint32_t *>(smem + o_bm);
  int32_t *pc = reinterpret_cast<int32_t *>(smem + o_pc);
  uint32_t *uni = reinterpret_cast<uint32_t *>(smem + o_uni);
  float *rtab = reinterpret_cast<float *>(smem + o_rt);
  int32_t *blist = reinterpret_cast<int32_t *>(smem + o_bl);
  int32_t *misc = reinterpret_cast<int32_t *>(smem + o_misc);  // [0] ns, [1..G] active

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m16 = lane & 15, kg = lane >> 4;
  const int ngrp = (Ht + G - 1) / G;
  // work-group id -> (schedule position, target group), XCD-aware as in k_apply4
  const int x = blockIdx.x % kXcds, kx = blockIdx.x / kXcds;
  const int round = kx / ngrp, tg = kx % ngrp;
  const int pos = round * kXcds + ((round & 1) ? (kXcds - 1 - x) : x);
  if (pos >= nrows) return;
  const int gr = sched[pos];
  const RowInfo ri = rows[gr];
  const int I = ri.blk, L = ri.len;
  const int n = I + 1;
  const int64_t tok0 = (int64_t)ri.start;
  const int64_t tpad = (int64_t)NBR * B;
  const int ga = row_alias ? row_alias[gr] : gr;
  const int grm = (ga >= 0 && ga < NBR) ? ga : gr;  // BSR row (shared block-rows)
  const int t0 = tg * G;

  // ---- set-up: active targets, source union, weights, kept bitmaps ---------
  if (tid < 64) {
    // wave 0, 64 heads at a time: source counts of the G targets (those with at
    // most four sources are k_apply4's), then the union of the active targets'
    // sources compacted by ballot in ascending head order
    bool act[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      int cnt = 0;
      if (t0 + g < Ht)
        for (int h0 = 0; h0 < Hs; h0 += 64) {
          const int h = h0 + tid;
          cnt += __popcll(wave_ballot(h < Hs && W[(int64_t)(t0 + g) * Hs + h] != 0.f));
        }
      act[g] = cnt > 4;
    }
    int ns = 0;
    for (int h0 = 0; h0 < Hs; h0 += 64) {
      const int h = h0 + tid;
      float w[G];
      bool any = false;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        w[g] = (act[g] && h < Hs) ? W[(int64_t)(t0 + g) * Hs + h] : 0.f;
        any |= w[g] != 0.f;
      }
      const uint64_t mask = wave_ballot(any);
      if (any) {
        const int q = ns + lanes_below(mask);
        src[q] = h;
        rbase[q] = row_ptr[(int64_t)h * NBR + grm];
#pragma unroll
        for (int g = 0; g < G; ++g) wtab[q * 4 + g] = w[g];
#pragma unroll
        for (int g = G; g < 4; ++g) wtab[q * 4 + g] = 0.f;
      }
      ns += __popcll(mask);
    }
    if (tid == 0) {
      misc[0] = ns;
#pragma unroll
      for (int g = 0; g < G; ++g) misc[1 + g] = act[g];
    }
  }
  for (int i = tid; i < Hs * nbw; i += C::NT) bm[i] = 0u;
  __syncthreads();
  const int ns = __builtin_amdgcn_readfirstlane(misc[0]);
  if (ns == 0) return;
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
    float r = 0.f;
    if (ip < L) {
      if (renorm) {
        const float km = kept_mass[(int64_t)src[q] * T + tok0 + ip];
        r = km > 0.f ? 1.f / km : 0.f;
      } else {
        r = 1.f;
      }
    }
    rtab[q * B + il] = r;
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
  if (tid < nw_row) {
    uint32_t u = 0u;
    for (int q = 0; q < ns; ++q) u |= bm[q * nbw + tid];
    uni[tid] = u;
  }
  __syncthreads();
  // union block list
  for (int J = tid; J < n; J += C::NT) {
    const uint32_t w = uni[J >> 5];
    if (!((w >> (J & 31)) & 1u)) continue;
    int k = __popc(w & ((1u << (J & 31)) - 1u));
    for (int i = 0; i < (J >> 5); ++i) k += __popc(uni[i]);
    blist[k] = J;
  }
  int nblk = 0;
  for (int i = 0; i < nw_row; ++i) nblk += __popc(uni[i]);
  __syncthreads();
  nblk = __builtin_amdgcn_readfirstlane(nblk);

  bool act[G];
#pragma unroll
  for (int g = 0; g < G; ++g) act[g] = misc[1 + g] != 0;
  const int gv0 = t0 / grp;                       // V head of the group's first target
  int nvh = 0;                                    // distinct V heads of the group
#pragma unroll
  for (int g = 0; g < G; ++g)
    if (t0 + g < Ht) nvh = (t0 + g) / grp - gv0 + 1;

  const int r0 = wave * 16 + m16;                 // lane row inside the block
  // lane's bytes of chunk kc: bf16 16 bytes at loff + kc * 1024; fp8 8 bytes at
  // loff + (kc / NP) * 512 NP + (kc % NP) * 8, and its row's scale byte
  const int loff = FP8 ? (wave * (KC / NP) * 64 + lane) * 8 * NP : (wave * KC * 64 + lane) * 16;
  const int soff = B * B + r0 * (B / 32);
  f32x4 acc[G][D / 16];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) acc[g][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int kb = 0; kb < nblk; ++kb) {
    const int J = __builtin_amdgcn_readfirstlane(blist[kb]);
    // tile index of every source at J, lane u holding sources u and u + 64
    int ti[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int u = lane + 64 * hh;
      int v = -1;
      if (u < ns) {
        const uint32_t word = bm[u * nbw + (J >> 5)];
        if ((word >> (J & 31)) & 1u) {
          const int64_t tix = rbase[u] + pc[u * nbw + (J >> 5)] + __popc(word & ((1u << (J & 31)) - 1u));
          if (tix < capacity) v = (int)tix;
        }
      }
      ti[hh] = v;
    }
    auto tile_at = [&](int u) -> int {  // uniform
      if (u >= ns) return -1;
      return u < 64 ? __builtin_amdgcn_readlane(ti[0], u) : __builtin_amdgcn_readlane(ti[1], u - 64);
    };
    // V tiles of this block for every distinct V head of the group
    const int64_t col0 = (int64_t)(gr - I + J) * B;
    for (int vh = 0; vh < nvh; ++vh)
      dma_v_tile<B, D, C::VINST>(vbuf + vh * C::VBYTES, vt + (int64_t)(gv0 + vh) * D * tpad, tpad,
                                 col0, wave, lane);

    u32x4 amix[G];
    // Buffer loads through one descriptor per source (wave-uniform base, 32-bit
    // lane offsets), zero-length for a source without a tile at this block, so
    // missing tiles read as zeros with no branch and no 64-bit lane addresses.
    auto load_batch = [&](u32x4 (&d)[SB], uint32_t (&sb)[SB], int kc, int u0) {
#pragma unroll
      for (int e = 0; e < SB; ++e) {
        const int t_ = tile_at(u0 + e);
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(tiles + (int64_t)(t_ >= 0 ? t_ : 0) * C::TBYTES), 0,
            t_ >= 0 ? (int)C::TBYTES : 0, kBufferFlags);
        if constexpr (!FP8) {
          d[e] = __builtin_amdgcn_raw_buffer_load_b128(r, loff, kc * 1024, 0);
          sb[e] = 0u;
        } else {
          const auto c2 = __builtin_amdgcn_raw_buffer_load_b64(r, loff, (kc / NP) * 512 * NP + (kc % NP) * 8, 0);
          d[e] = u32x4{c2[0], c2[1], 0u, 0u};
          sb[e] = __builtin_amdgcn_raw_buffer_load_b8(r, soff, kc, 0);
        }
      }
    };
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      float mx[G][8];
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) mx[g][e] = 0.f;
      u32x4 cur[SB], nxt[SB];
      uint32_t scur[SB], snxt[SB];
      load_batch(cur, scur, kc, 0);
      for (int u0 = 0; u0 < ns; u0 += SB) {
        if (u0 + SB < ns) load_batch(nxt, snxt, kc, u0 + SB);
#pragma unroll
        for (int pr = 0; pr < SB / 2; ++pr) {
          const int u1 = u0 + 2 * pr, u2 = u1 + 1;
          float ra = u1 < ns ? rtab[u1 * B + r0] : 0.f;
          float rb = u2 < ns ? rtab[u2 * B + r0] : 0.f;
          if constexpr (FP8) {
            // the block scales 2^(byte - 127) folded into the coefficients
            ra = __builtin_amdgcn_ldexpf(ra, (int)scur[2 * pr] - 127);
            rb = __builtin_amdgcn_ldexpf(rb, (int)scur[2 * pr + 1] - 127);
          }
          uint32_t cp[G];
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float wa = u1 < ns ? wtab[u1 * 4 + g] : 0.f;
            const float wb = u2 < ns ? wtab[u2 * 4 + g] : 0.f;
            cp[g] = pack_bf16x2(wa * ra, wb * rb);
          }
          if constexpr (!FP8) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t lo = __builtin_amdgcn_perm(cur[2 * pr + 1][e], cur[2 * pr][e], 0x05040100u);
              const uint32_t hi = __builtin_amdgcn_perm(cur[2 * pr + 1][e], cur[2 * pr][e], 0x07060302u);
#pragma unroll
              for (int g = 0; g < G; ++g) {
                mx[g][2 * e] = __builtin_amdgcn_fdot2_f32_bf16(
                    __builtin_bit_cast(bf16x2, lo), __builtin_bit_cast(bf16x2, cp[g]), mx[g][2 * e], false);
                mx[g][2 * e + 1] = __builtin_amdgcn_fdot2_f32_bf16(
                    __builtin_bit_cast(bf16x2, hi), __builtin_bit_cast(bf16x2, cp[g]), mx[g][2 * e + 1], false);
              }
            }
          } else {
            // byte pairs [P1[e], P2[e]] of the two sources' codes, then E4M3 ->
            // bf16 (exact: 3 mantissa bits, and the scale 1 changes nothing)
#pragma unroll
            for (int w = 0; w < 2; ++w)
#pragma unroll
              for (int hw = 0; hw < 2; ++hw) {
                const uint32_t pairs = __builtin_amdgcn_perm(
                    cur[2 * pr + 1][w], cur[2 * pr][w], hw ? 0x07030602u : 0x05010400u);
                const bf16x2 pv[2] = {__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(pairs, 1.0f, false),
                                      __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(pairs, 1.0f, true)};
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                  const int e = 4 * w + 2 * hw + k;
#pragma unroll
                  for (int g = 0; g < G; ++g)
                    mx[g][e] = __builtin_amdgcn_fdot2_f32_bf16(pv[k], __builtin_bit_cast(bf16x2, cp[g]),
                                                               mx[g][e], false);
                }
              }
          }
        }
#pragma unroll
        for (int e = 0; e < SB; ++e) {
          cur[e] = nxt[e];
          scur[e] = snxt[e];
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) amix[g][e] = pack_bf16x2(mx[g][2 * e], mx[g][2 * e + 1]);
      if (kc == 0) {
        // V tiles landed (direct-to-LDS loads: full drain) in every wave
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb)
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const int vh = (t0 + g < Ht) ? (t0 + g) / grp - gv0 : 0;
          const u32x4 bv = v_frag<B>(vbuf + vh * C::VBYTES, nb * 16 + m16, kc * 4 + kg);
          acc[g][nb] = mfma16_bf16(as_bf16x8(amix[g]), as_bf16x8(bv), acc[g][nb]);
        }
    }
    // every wave's reads of V done before the next block's loads overwrite it
    __syncthreads();
  }

#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (!act[g]) continue;
    float *ot = o + (int64_t)(t0 + g) * T * D;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ip = I * B + wave * 16 + 4 * kg + r;
      if (ip < L) {
        float *dst = ot + (tok0 + ip) * D + m16;
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb) __builtin_nontemporal_store(acc[g][nb][r], dst + nb * 16);
      }
    }
  }
}

// The two apply kernels for one tile format, over `nrows` block-rows of `sched`.
template <int B, int D, int FMT>
static mf_status launch_apply_fmt(hipStream_t s, const mf_bsr_map *map, const float *W, int32_t Ht,
                                  int32_t Hkv, const SeqGeom &g, int32_t renorm, float *o,
                                  void *ws, const VtWs &w, const int32_t *sched, int32_t nrows,
                                  int nbw, size_t smem, size_t smem_mix, size_t vbufs,
                                  size_t vbufs_mix) {
  using CM = ApplyMixCfg<B, D, FMT>;
  if (smem + vbufs > 64 * 1024 &&
      hipFuncSetAttribute(reinterpret_cast<const void *>(&k_apply4<B, D, FMT>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem) != hipSuccess)
    return MF_ERR_HIP;
  if (smem_mix + vbufs_mix > 64 * 1024 &&
      hipFuncSetAttribute(reinterpret_cast<const void *>(&k_apply_mix<B, D, FMT>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem_mix) != hipSuccess)
    return MF_ERR_HIP;
  const char *tiles = static_cast<const char *>(map->tiles);
  const int64_t npos = ((int64_t)nrows + kXcds - 1) / kXcds * kXcds;
  // one launch per source-count class; a work-group whose targets are all of
  // the other class returns right after reading their weight rows
  hipLaunchKernelGGL((k_apply4<B, D, FMT>), dim3((unsigned)(npos * Ht)),
                     dim3(Apply4Cfg<B, D, FMT>::NT), smem, s, map->row_ptr, map->col_idx, tiles,
                     map->kept_mass, map->num_heads, g.NBR, g.T, W, Ht, Ht / Hkv,
                     at<uint16_t>(ws, w.vt), at<RowInfo>(ws, w.rt.rows), sched, nrows, nbw,
                     map->capacity_tiles, renorm, o, map->row_alias);
  if (hip_status() != MF_OK) return MF_ERR_HIP;
  const int64_t ngrp = (Ht + CM::G - 1) / CM::G;
  hipLaunchKernelGGL((k_apply_mix<B, D, FMT>), dim3((unsigned)(npos * ngrp)), dim3(CM::NT),
                     smem_mix, s, map->row_ptr, map->col_idx, tiles, map->kept_mass,
                     map->num_heads, g.NBR, g.T, W, Ht, Ht / Hkv, at<uint16_t>(ws, w.vt),
                     at<RowInfo>(ws, w.rt.rows), sched, nrows, nbw, map->capacity_tiles, renorm,
                     o, map->row_alias);
  return hip_status();
}

// V staging, the window schedule (if any), then both apply kernels.
template <int B, int D>
static mf_status launch_apply(hipStream_t s, const mf_bsr_map *map, const float *W, int32_t Ht,
                              const VSrc &vs, const SeqGeom &g, int32_t nrows, int32_t renorm,
                              float *o, void *ws, const VtWs &w) {
  const int nbw = (g.maxnb + 31) / 32 > 0 ? (g.maxnb + 31) / 32 : 1;
  const size_t smem = apply_smem(B, map->num_heads, nbw);
  const size_t smem_mix = mix_smem(B, map->num_heads, nbw);
  // tile indices are held in int32; V rows are addressed with 32-bit byte
  // offsets d * NBR * B * 2
  if (map->capacity_tiles > INT32_MAX) return MF_ERR_UNSUPPORTED;
  if ((int64_t)D * g.NBR * B * 2 >= ((int64_t)1 << 31)) return MF_ERR_UNSUPPORTED;
  if (map->num_heads > kMixMaxSources) return MF_ERR_UNSUPPORTED;
  const size_t vbufs = 2 * (size_t)B * D * 2;  // the two static V tile buffers of k_apply4
  const size_t vbufs_mix = (size_t)ApplyMixCfg<B, D, MF_TILE_BF16>::G * B * D * 2;
  if (smem + vbufs > 160 * 1024 || smem_mix + vbufs_mix > 160 * 1024) return MF_ERR_UNSUPPORTED;
  hipLaunchKernelGGL((k_vtranspose<B, D>), dim3(g.NBR, vs.Hkv), dim3(256), 0, s, vs, g.T,
                     at<RowInfo>(ws, w.rt.rows), g.NBR, at<uint16_t>(ws, w.vt));
  if (hip_status() != MF_OK) return MF_ERR_HIP;
  const int32_t *sched = at<int32_t>(ws, w.rt.sched);
  if (vs.window) {
    if (nrows == 0) return MF_OK;
    hipLaunchKernelGGL(k_window_sched, dim3(1), dim3(1024), 0, s, at<RowInfo>(ws, w.rt.rows),
                       sched, g.NBR, B, vs.window, at<int32_t>(ws, w.wsched));
    if (hip_status() != MF_OK) return MF_ERR_HIP;
    sched = at<int32_t>(ws, w.wsched);
  }
  if (map->tile_format == MF_TILE_MXFP8)
    return launch_apply_fmt<B, D, MF_TILE_MXFP8>(s, map, W, Ht, vs.Hkv, g, renorm, o, ws, w, sched,
                                                 nrows, nbw, smem, smem_mix, vbufs, vbufs_mix);
  return launch_apply_fmt<B, D, MF_TILE_BF16>(s, map, W, Ht, vs.Hkv, g, renorm, o, ws, w, sched,
                                              nrows, nbw, smem, smem_mix, vbufs, vbufs_mix);
}

// Shared argument checks and dispatch of both apply entry points.
static mf_status apply_common(void *stream, const mf_bsr_map *map, const float *W, int32_t Ht,
                              VSrc vs, int32_t d, const int32_t *cu_host, const int32_t *cu_dev,
                              int32_t nseq, const int32_t *window_host, int32_t renorm, float *o,
                              void *ws, size_t ws_bytes) {
  const int32_t Hkv = vs.Hkv;
  if (!map || !cu_host || !cu_dev || Ht <= 0 || Hkv <= 0 || Ht % Hkv != 0)
    return MF_ERR_INVALID_ARG;
  if (!valid_block(map->block)) return MF_ERR_INVALID_ARG;
  if (!valid_dim(d)) return MF_ERR_UNSUPPORTED;
  if (map->num_heads <= 0 || !W || !valid_tile_format(map->tile_format)) return MF_ERR_INVALID_ARG;
  SeqGeom g;
  mf_status st = seq_geom(cu_host, nseq, map->block, &g);
  if (st != MF_OK) return st;
  if (g.NBR != map->num_block_rows || g.T != map->total_tokens) return MF_ERR_INVALID_ARG;
  if ((int64_t)g.NBR * Ht > INT32_MAX / 2) return MF_ERR_UNSUPPORTED;
  if (g.T > 0 && (!(vs.v || vs.pages) || !o || !map->row_ptr || !map->col_idx || !map->tiles ||
                  !map->kept_mass))
    return MF_ERR_INVALID_ARG;
  const int B = map->block;
  int64_t nrows = g.NBR;
  if (vs.pages) {
    if (vs.page_size <= 0 || vs.num_pages <= 0 || vs.max_pages <= 0 || !vs.table)
      return MF_ERR_INVALID_ARG;
    for (int32_t s = 0; s < nseq; ++s)
      if ((int64_t)cu_host[s + 1] - cu_host[s] > (int64_t)vs.max_pages * vs.page_size)
        return MF_ERR_INVALID_ARG;  // the table cannot cover the sequence
  }
  if (vs.window) {
    if (!window_host) return MF_ERR_INVALID_ARG;
    nrows = 0;
    for (int32_t s = 0; s < nseq; ++s) {
      const int32_t L = cu_host[s + 1] - cu_host[s];
      const int32_t a = window_host[2 * s], b = window_host[2 * s + 1];
      if (a < 0 || b < a || b > L) return MF_ERR_INVALID_ARG;
      if (a == b) continue;  // nothing of this sequence in the chunk
      if (a % B != 0 || (b % B != 0 && b != L)) return MF_ERR_INVALID_ARG;
      nrows += ((int64_t)b + B - 1) / B - a / B;
    }
  }
  const VtWs w = vt_ws(g, Hkv, B, d);
  if (!ws || ws_bytes < w.total) return MF_ERR_WORKSPACE;
  if (g.NBR == 0) return MF_OK;
  void *wsa = reinterpret_cast<void *>((reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if ((st = launch_rowtable(s, cu_dev, g, B, wsa, w.rt)) != MF_OK) return st;
  const int32_t nr = (int32_t)nrows;
  if (B == 32)
    return d == 64 ? launch_apply<32, 64>(s, map, W, Ht, vs, g, nr, renorm, o, wsa, w)
                   : launch_apply<32, 128>(s, map, W, Ht, vs, g, nr, renorm, o, wsa, w);
  if (B == 64)
    return d == 64 ? launch_apply<64, 64>(s, map, W, Ht, vs, g, nr, renorm, o, wsa, w)
                   : launch_apply<64, 128>(s, map, W, Ht, vs, g, nr, renorm, o, wsa, w);
  return d == 64 ? launch_apply<128, 64>(s, map, W, Ht, vs, g, nr, renorm, o, wsa, w)
                 : launch_apply<128, 128>(s, map, W, Ht, vs, g, nr, renorm, o, wsa, w);
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
  VSrc vs{static_cast<const uint16_t *>(v), nullptr, nullptr, 0, 0, 0, Hkv, nullptr};
  return apply_common(stream, map, W, Ht, vs, d, cu_host, cu_dev, nseq, nullptr, renorm, o, ws,
                      ws_bytes);
}

extern "C" mf_status mf_apply_translated_paged(void *stream, const mf_bsr_map *map,
                                               const float *W, int32_t Ht, const mf_paged_v *pv,
                                               int32_t Hkv, int32_t d, const int32_t *cu_host,
                                               const int32_t *cu_dev, int32_t nseq,
                                               const int32_t *window_host,
                                               const int32_t *window_dev, int32_t renorm,
                                               float *o, void *ws, size_t ws_bytes) {
  if (!pv || !pv->pages) return MF_ERR_INVALID_ARG;
  if ((window_host == nullptr) != (window_dev == nullptr)) return MF_ERR_INVALID_ARG;
  VSrc vs{nullptr, static_cast<const uint16_t *>(pv->pages), pv->block_table, pv->page_size,
          pv->max_pages_per_seq, pv->num_pages, Hkv, window_dev};
  return apply_common(stream, map, W, Ht, vs, d, cu_host, cu_dev, nseq, window_host, renorm, o,
                      ws, ws_bytes);
}
