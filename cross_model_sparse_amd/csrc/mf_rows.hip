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
  __shared__ int64_t t_nb[1024];
  __shared__ int64_t t_tri[1024];
  __shared__ int32_t hist[kMaxNB + 1];
  __shared__ int32_t startI[kMaxNB];
  __shared__ int32_t fillI[kMaxNB];
  const int tid = threadIdx.x, nt = blockDim.x;
  const int per = (nseq + nt - 1) / nt;
  const int s0 = min(nseq, tid * per), s1 = min(nseq, s0 + per);
  for (int i = tid; i <= kMaxNB; i += nt) hist[i] = 0;
  for (int i = tid; i < kMaxNB; i += nt) fillI[i] = 0;
  __syncthreads();
  int64_t a = 0, b = 0;
  for (int s = s0; s < s1; ++s) {
    int64_t nb = ((int64_t)(cu[s + 1] - cu[s]) + B - 1) / B;
    a += nb;
    b += nb * (nb + 1) / 2;
    atomicAdd(&hist[nb], 1);
  }
  t_nb[tid] = a;
  t_tri[tid] = b;
  __syncthreads();
  if (tid == 0) {
    int64_t ra = 0, rb = 0;
    for (int i = 0; i < nt; ++i) {
      int64_t x = t_nb[i], y = t_tri[i];
      t_nb[i] = ra;
      t_tri[i] = rb;
      ra += x;
      rb += y;
    }
    nbcum[nseq] = (int32_t)ra;
    // sequences with more than I blocks, then schedule slots by I descending
    int32_t above = 0;  // sequences with nb > I
    int32_t run = 0;
    for (int I = maxnb - 1; I >= 0; --I) {
      above += hist[I + 1];
      startI[I] = run;
      run += above;
    }
  }
  __syncthreads();
  int64_t gr = t_nb[tid], tri = t_tri[tid];
  for (int s = s0; s < s1; ++s) {
    const int32_t st = cu[s], L = cu[s + 1] - cu[s];
    const int32_t nb = (L + B - 1) / B;
    nbcum[s] = (int32_t)gr;
    for (int32_t I = 0; I < nb; ++I) {
      rows[gr + I] = RowInfo{s, I, st, L};
      pbase[gr + I] = (int64_t)B * (tri + (int64_t)I * (I + 1) / 2);
      // order inside one I does not affect results, only which group runs it
      int32_t pos = startI[I] + atomicAdd(&fillI[I], 1);
      sched[pos] = (int32_t)(gr + I);
    }
    gr += nb;
    tri += (int64_t)nb * (nb + 1) / 2;
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
