// Utility entry points of libse: status word readback, error strings, version.
#include "common.hpp"

extern "C" int32_t se_status_read(int32_t *status, int32_t *host_value, int32_t reset, se_stream_t stream) {
  if (!status || !host_value) return SE_ERR_NULL;
  hipStream_t st = (hipStream_t)stream;
  if (hipMemcpyAsync(host_value, status, sizeof(int32_t), hipMemcpyDeviceToHost, st) != hipSuccess) return SE_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return SE_ERR_HIP;
  if (reset) {
    const int32_t zero = 0;
    if (hipMemcpyAsync(status, &zero, sizeof(int32_t), hipMemcpyHostToDevice, st) != hipSuccess) return SE_ERR_HIP;
    if (hipStreamSynchronize(st) != hipSuccess) return SE_ERR_HIP;
  }
  return SE_OK;
}

extern "C" const char *se_error_string(int32_t code) {
  switch (code) {
    case SE_OK: return "ok";
    case SE_ERR_NULL: return "a required pointer is NULL";
    case SE_ERR_SHAPE: return "sizes or strides do not fit together";
    case SE_ERR_DTYPE: return "unsupported element type or head dimension";
    case SE_ERR_PARAM: return "parameter outside its domain";
    case SE_ERR_WORKSPACE: return "workspace missing or too small";
    case SE_ERR_UNSUPPORTED: return "combination not implemented";
    case SE_ERR_HIP: return "HIP runtime error";
    case SE_ERR_SCRATCH_LIMIT: return "needs more scratch than the allocation-free entry point holds";
    default: break;
  }
  if (code & SE_DEV_INDEX) return "device: index list entry out of range, unsorted, duplicated or not resident";
  if (code & SE_DEV_CAPACITY) return "device: free block stack, slot stack or slot range exhausted";
  return "unknown status";
}

extern "C" const char *se_version(void) { return "libse 0.1 (gfx950)"; }
