// Block-row table: global block-row -> (sequence, block index), partial-buffer
// offsets, and a longest-first schedule.  One work-group, built on the device
// from the device copy of the sequence offsets so no host-to-device copy is
// needed.
#include "mf_host.hpp"

namespace mf {

__global__ __launch_bounds__(1024) void k_rowtable(const int32_t *__restrict__ cu, int32_t nseq,
                                                   int32_t B, int32_t maxnb,
                                                   RowInfo *__restrict__ rows,
                                                   int32_t *__restrict__ sched,
                                                   int64_t *__restrict__ pbase,
                                                   int32_t *__restrict__ nbcum) {
  __shared__ int64_t wsum[16];
  __shared__ int32_t hist[kMaxNB + 1];
  __shared__ int32_t startI[kMaxNB];
  __shared__ int32_t fillI[kMaxNB];
  const int tid = threadIdx.x, nt = blockDim.x;  // nt == 1024
  const int per = (nseq + nt - 1) / nt;
  const int s0 = min(nseq, tid * per), s1 = min(nseq, s0 + per);
  for (int i = tid; i <= kMaxNB; i += nt) hist[i] = 0;
  for (int i = tid; i < kMaxNB; i += nt) fillI[i] = 0;
  __syncthreads();
  // this thread's sequences: block-rows, causal blocks, lengths histogram
  int64_t a = 0, b = 0;
  for (int s = s0; s < s1; ++s) {
    int64_t nb = ((int64_t)(cu[s + 1] - cu[s]) + B - 1) / B;
    a += nb;
    b += nb * (nb + 1) / 2;
    atomicAdd(&hist[nb], 1);
  }
  const int64_t ia = block_scan_incl(a, wsum), ib = block_scan_incl(b, wsum);
  int64_t gr = ia - a, tri = ib - b;  // first block-row and partial offset of s0
  if (tid == nt - 1) nbcum[nseq] = (int32_t)ia;
  // schedule: slots by I descending, the sequences with more than I blocks at
  // each I.  Thread t takes I = maxnb - 1 - t: above = sequences with nb > I
  // (a running count of the histogram from the top), startI = the slots of all
  // larger I before it.
  const int It = maxnb - 1 - tid;
  const int64_t hv = (It >= 0) ? hist[It + 1] : 0;
  const int64_t above = block_scan_incl(hv, wsum);
  const int64_t run = block_scan_incl(above, wsum) - above;
  if (It >= 0) startI[It] = (int32_t)run;
  // first block-row and partial offset of every sequence
  for (int s = s0; s < s1; ++s) {
    const int32_t nb = (cu[s + 1] - cu[s] + B - 1) / B;
    nbcum[s] = (int32_t)gr;
    if (nb > 0) pbase[gr] = (int64_t)B * tri;
    gr += nb;
    tri += (int64_t)nb * (nb + 1) / 2;
  }
  __syncthreads();  // nbcum, pbase of first rows and startI visible to the block
  // every block-row, spread over the threads: its sequence is the last one
  // whose first block-row is at or before it (empty sequences share their
  // successor's first row and are passed over)
  const int64_t NBR = nbcum[nseq];
  for (int64_t g = tid; g < NBR; g += nt) {
    int lo = 0, hi = nseq - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (nbcum[mid] <= g) lo = mid;
      else hi = mid - 1;
    }
    const int s = lo;
    const int32_t g0 = nbcum[s];
    const int32_t I = (int32_t)(g - g0);
    const int32_t st = cu[s], L = cu[s + 1] - cu[s];
    rows[g] = RowInfo{s, I, st, L};
    if (I > 0) pbase[g] = pbase[g0] + (int64_t)B * ((int64_t)I * (I + 1) / 2);
    // order inside one I does not affect results, only which group runs it
    const int32_t pos = startI[I] + atomicAdd(&fillI[I], 1);
    sched[pos] = (int32_t)g;
  }
}

mf_status launch_rowtable(hipStream_t s, const int32_t *cu_dev, const SeqGeom &g, int32_t B,
                          void *ws, const RowTable &rt) {
  hipLaunchKernelGGL(k_rowtable, dim3(1), dim3(1024), 0, s, cu_dev, g.nseq, B, g.maxnb,
                     at<RowInfo>(ws, rt.rows), at<int32_t>(ws, rt.sched),
                     at<int64_t>(ws, rt.pbase), at<int32_t>(ws, rt.nbcum));
  return hip_status();
}

}  // namespace mf
