// Status read-back and status strings.
#include "mf_host.hpp"

extern "C" mf_status mf_read_status(void *stream, const mf_bsr_map *map, int64_t *nnz_out) {
  if (!map || !map->status || !map->nnz) return MF_ERR_INVALID_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int32_t st = 0;
  int64_t nnz = 0;
  if (hipMemcpyAsync(&st, map->status, sizeof(st), hipMemcpyDeviceToHost, s) != hipSuccess)
    return MF_ERR_HIP;
  if (hipMemcpyAsync(&nnz, map->nnz, sizeof(nnz), hipMemcpyDeviceToHost, s) != hipSuccess)
    return MF_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return MF_ERR_HIP;
  if (nnz_out) *nnz_out = nnz;
  return (mf_status)st;
}

extern "C" const char *mf_status_string(mf_status status) {
  switch (status) {
    case MF_OK: return "ok";
    case MF_ERR_INVALID_ARG: return "invalid argument";
    case MF_ERR_UNSUPPORTED: return "unsupported block size, head dimension, dtype or size";
    case MF_ERR_CAPACITY: return "more kept tiles than the map's capacity";
    case MF_ERR_HIP: return "HIP runtime or launch error";
    case MF_ERR_WORKSPACE: return "workspace missing or too small";
  }
  return "unknown status";
}
