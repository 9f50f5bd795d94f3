// Host-side argument checks shared by the libmx entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/mx.h"

namespace mxk {

inline bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// CUs of the current device (cached per device; 0 if the query fails).
inline int64_t device_cus() {
  static int64_t cache[64] = {};
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 0;
    cache[dev] = cus;
  }
  return cache[dev];
}

inline mx_status_t check_common_quant(mx_dtype_t in, int64_t rows, int64_t cols, int block, mx_elem_t fmt,
                                      mx_scale_rule_t rule) {
  if (in != MX_F32 && in != MX_BF16 && in != MX_F16) return MX_ERR_UNSUPPORTED;
  if (fmt != MX_E4M3 && fmt != MX_E5M2 && fmt != MX_E2M1) return MX_ERR_UNSUPPORTED;
  if (rule != MX_SCALE_FLOOR && rule != MX_SCALE_CEIL) return MX_ERR_UNSUPPORTED;
  if (block != 32) return MX_ERR_UNSUPPORTED;
  if (rows < 0 || cols < 0) return MX_ERR_SHAPE;
  // element indices and grid sizes are kept within 2^31 workgroups / 2^62 elements
  if (rows > (int64_t(1) << 31) || cols > (int64_t(1) << 31)) return MX_ERR_SHAPE;
  return MX_OK;
}

// Row-wise MXFP6 quantization (quantize_fp6.hip), reached from mx_quantize.
mx_status_t fp6_quantize(const void* x, mx_dtype_t in, int64_t rows, int64_t cols, int block, mx_elem_t fmt,
                         mx_scale_rule_t rule, mx_orient_t orient, int hadamard, uint8_t* q, uint8_t* scales,
                         float* amax_out, hipStream_t stream);
// Dual (row-wise + column-wise) MXFP6 quantization (quantize_fp6.hip), reached from mx_quantize_dual.
mx_status_t fp6_quantize_dual(const void* x, mx_dtype_t in, int64_t rows, int64_t cols, int block, mx_elem_t fmt,
                              mx_scale_rule_t rule, uint8_t* q_row, uint8_t* s_row, uint8_t* q_colT,
                              uint8_t* s_colT, float* amax_out, hipStream_t stream);

}  // namespace mxk
