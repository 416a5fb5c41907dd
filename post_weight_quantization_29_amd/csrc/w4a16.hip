// y = x W^T on the packed 4-bit layer (GPTQ practice page m.lqnn.cn/news/117696,
// section 4.3: at inference the 4-bit weights are dequantized to a 16-bit type
// and then multiplied; what the 4 bits save is the bytes moved, so at small
// batch this product is bound by HBM).
//
// One wave per output row r: each lane streams words of the row's packed codes
// (8 codes per word, the gptq_pack_int4 layout), forms each weight as the fp32
// product scale * (code - zero) rounded to the activation's 16-bit type, and
// multiplies it with up to 8 activation rows at a time, accumulating in fp32;
// a wave reduction finishes each dot product.
#include "common.h"

namespace gptq {

constexpr int kWRows = 8;   // activation rows per pass over the weights

template <typename T> struct Act;
template <> struct Act<__bf16> {
  static GPTQ_DEV float to_f(uint32_t h) { return __builtin_bit_cast(float, h << 16); }
  static GPTQ_DEV float round16(float x) {     // ties to even
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    u = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
    return __builtin_bit_cast(float, u);
  }
};
template <> struct Act<_Float16> {
  static GPTQ_DEV float to_f(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }
  static GPTQ_DEV float round16(float x) { return (float)(_Float16)x; }
};

template <typename TY> GPTQ_DEV TY out_cast(float v);
template <> GPTQ_DEV float out_cast<float>(float v) { return v; }
template <> GPTQ_DEV __bf16 out_cast<__bf16>(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, Act<__bf16>::round16(v));
  return __builtin_bit_cast(__bf16, (uint16_t)(u >> 16));
}
template <> GPTQ_DEV _Float16 out_cast<_Float16>(float v) { return (_Float16)v; }

// NATURAL: column c is in group c / G (G a multiple of 8, so a word's eight
// codes share a group); otherwise group g_idx[c], clamped to [0, ng).
template <typename T, typename TY, bool NATURAL>
__global__ __launch_bounds__(256) void w4a16_kernel(const uint16_t* __restrict__ X, int64_t m, int d_in,
                                                    const uint32_t* __restrict__ packed,
                                                    const float* __restrict__ scales,
                                                    const int32_t* __restrict__ zeros,
                                                    const int32_t* __restrict__ g_idx, int G, int ng,
                                                    int d_out, TY* __restrict__ Y) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = blockIdx.x * 4 + wave;
  if (r >= d_out) return;
  const int nw = d_in >> 3;
  const uint32_t* prow = packed + (size_t)r * nw;
  const float* srow = scales + (size_t)r * ng;
  const int32_t* zrow = zeros + (size_t)r * ng;
  const float invG = 1.0f / (float)G;
  for (int64_t m0 = 0; m0 < m; m0 += kWRows) {
    const int mc = (int)min<int64_t>(kWRows, m - m0);
    const uint16_t* xb = X + m0 * d_in;
    float acc[kWRows];
#pragma unroll
    for (int i = 0; i < kWRows; ++i) acc[i] = 0.0f;
#pragma unroll 4
    for (int q = lane; q < nw; q += 64) {
      const uint32_t p = prow[q];
      const int c0 = q * 8;
      float w[8];
      if (NATURAL) {
        int g = (int)((float)c0 * invG);          // exact quotient after one correction
        if (g * G > c0) --g;
        if ((g + 1) * G <= c0) ++g;
        const float s = srow[g], z = (float)zrow[g];
#pragma unroll
        for (int k = 0; k < 8; ++k) w[k] = Act<T>::round16(s * ((float)((p >> (4 * k)) & 15u) - z));
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int g = min(max(g_idx[c0 + k], 0), ng - 1);
          w[k] = Act<T>::round16(srow[g] * ((float)((p >> (4 * k)) & 15u) - (float)zrow[g]));
        }
      }
#pragma unroll
      for (int i = 0; i < kWRows; ++i) {
        if (i < mc) {
          const uint4 xv = *reinterpret_cast<const uint4*>(xb + (size_t)i * d_in + c0);
          const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w};
          float a = acc[i];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            a = fmaf(Act<T>::to_f(xs[k] & 0xFFFFu), w[2 * k], a);
            a = fmaf(Act<T>::to_f(xs[k] >> 16), w[2 * k + 1], a);
          }
          acc[i] = a;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kWRows; ++i) {
      float v = acc[i];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
      if (lane == 0 && i < mc) Y[(size_t)(m0 + i) * d_out + r] = out_cast<TY>(v);
    }
  }
}

template <typename T, typename TY>
static void launch_w4a16(const void* X, int64_t m, int d_in, const uint32_t* packed, const float* scales,
                         const int32_t* zeros, const int32_t* g_idx, int G, int ng, int d_out, void* Y,
                         hipStream_t s) {
  const unsigned grid = (unsigned)((d_out + 3) / 4);
  const uint16_t* x = static_cast<const uint16_t*>(X);
  if (g_idx)
    w4a16_kernel<T, TY, false><<<grid, 256, 0, s>>>(x, m, d_in, packed, scales, zeros, g_idx, G, ng, d_out,
                                                    static_cast<TY*>(Y));
  else
    w4a16_kernel<T, TY, true><<<grid, 256, 0, s>>>(x, m, d_in, packed, scales, zeros, nullptr, G, ng, d_out,
                                                   static_cast<TY*>(Y));
}

}  // namespace gptq

using namespace gptq;

extern "C" int gptq_w4a16_gemm(const void* X, gptq_dtype x_dtype, int64_t m, int32_t d_in,
                               const uint32_t* packed, const float* scales, const int32_t* zeros,
                               const int32_t* g_idx, int32_t group_size, int32_t n_groups,
                               int32_t d_out, void* Y, gptq_dtype y_dtype, hipStream_t s) {
  if (!X || !packed || !scales || !zeros || !Y) return GPTQ_ERR_INVALID_ARG;
  if (m < 0 || d_in <= 0 || d_out <= 0 || (d_in % 8) != 0 || n_groups <= 0) return GPTQ_ERR_INVALID_ARG;
  if (x_dtype != GPTQ_F16 && x_dtype != GPTQ_BF16) return GPTQ_ERR_INVALID_ARG;
  if (y_dtype != GPTQ_F32 && y_dtype != GPTQ_F16 && y_dtype != GPTQ_BF16) return GPTQ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(X) & 15) != 0) return GPTQ_ERR_INVALID_ARG;
  int G = group_size;
  if (!g_idx) {
    if (G == -1) G = d_in;
    if (G <= 0 || (G % 8) != 0) return GPTQ_ERR_INVALID_ARG;
    if (n_groups != (d_in + G - 1) / G) return GPTQ_ERR_INVALID_ARG;
  } else {
    G = 1;
  }
  if (m == 0) return GPTQ_OK;
  const uint32_t* pk = packed;
  if (x_dtype == GPTQ_BF16) {
    if (y_dtype == GPTQ_F32) launch_w4a16<__bf16, float>(X, m, d_in, pk, scales, zeros, g_idx, G, n_groups, d_out, Y, s);
    else if (y_dtype == GPTQ_BF16) launch_w4a16<__bf16, __bf16>(X, m, d_in, pk, scales, zeros, g_idx, G, n_groups, d_out, Y, s);
    else launch_w4a16<__bf16, _Float16>(X, m, d_in, pk, scales, zeros, g_idx, G, n_groups, d_out, Y, s);
  } else {
    if (y_dtype == GPTQ_F32) launch_w4a16<_Float16, float>(X, m, d_in, pk, scales, zeros, g_idx, G, n_groups, d_out, Y, s);
    else if (y_dtype == GPTQ_BF16) launch_w4a16<_Float16, __bf16>(X, m, d_in, pk, scales, zeros, g_idx, G, n_groups, d_out, Y, s);
    else launch_w4a16<_Float16, _Float16>(X, m, d_in, pk, scales, zeros, g_idx, G, n_groups, d_out, Y, s);
  }
  GPTQ_LAUNCH_CHECK();
  return GPTQ_OK;
}
