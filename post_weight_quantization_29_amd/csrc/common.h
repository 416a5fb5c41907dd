// Shared device helpers for the gfx950 GPTQ kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>
#include <algorithm>
#include <cmath>

#include "../../include/gptq.h"

#define GPTQ_DEV __device__ __forceinline__

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

namespace gptq {

// hipError_t -> status (no error state is kept between calls)
#define GPTQ_HIP_TRY(expr)                                  \
  do {                                                      \
    hipError_t e_ = (expr);                                 \
    if (e_ != hipSuccess) return GPTQ_ERR_HIP;              \
  } while (0)

#define GPTQ_LAUNCH_CHECK()                                 \
  do {                                                      \
    hipError_t e_ = hipGetLastError();                      \
    if (e_ != hipSuccess) return GPTQ_ERR_HIP;              \
  } while (0)

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }

// Output layout of v_mfma_f32_32x32x{2f32,16bf16,16f16} (checked on gfx950):
// lane l, accumulator register r holds C[row][col] with
//   row = 8*(r/4) + 4*(l/32) + (r%4),  col = l%32.
// Operand A: lane l supplies A[l%32][k-slot group l/32]; operand B: B[k][l%32].
GPTQ_DEV int mfma32_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }
GPTQ_DEV int mfma32_col(int lane) { return lane & 31; }

GPTQ_DEV float load_as_float(const void* p, gptq_dtype t, size_t i) {
  if (t == GPTQ_F32) return static_cast<const float*>(p)[i];
  if (t == GPTQ_F16) return (float)static_cast<const _Float16*>(p)[i];
  uint32_t b = (uint32_t)static_cast<const uint16_t*>(p)[i] << 16;
  return __builtin_bit_cast(float, b);
}

}  // namespace gptq
