// Activation-aware weight quantization (AWQ) of one linear layer, the second
// method the pages set beside GPTQ.  Steps, after "GPTQ/AWQ量化导出：让大模型在
// 消费级显卡上跑起来" (the AWQ list: per-channel RMS of the calibration
// activations, the top 5 % of channels, a larger factor for them, the factor
// undone at inference) and "大模型压缩量化技术：GPTQ 与 AWQ 原理详解 + Python
// 实战教程" section 四 (weights of the large-activation channels times s > 1,
// quantize, activations divided by s; the best factor is chosen; no Hessian):
//
//   gptq_awq_act_sumsq  a_j += sum_t x_tj^2 (the RMS squared times N), fp64
//   gptq_awq_search     salient set = top-k channels by a_j; for every
//                       candidate sigma: the group grid of fp32(w * s_j),
//                       s_j = sigma on salient channels and 1 elsewhere, and
//                       E(sigma) = sum_j a_j sum_i (w_ij - Qhat_ij)^2 with
//                       Qhat = scale * (code - zero) / s_j; the smallest E wins
//   gptq_awq_quantize   the group grid of fp32(w * s_j) for given factors
//
// The grid is the asymmetric min-max grid of the GPTQ path (zero point not
// clamped; a constant group a uses [min(a,0), max(a,0)]; all zero: scale 1),
// here with correctly rounded fp32 divisions for the scale, the zero point and
// each code.
#include "common.h"

namespace gptq {

constexpr int kAwqMaxGrid = 32;    // candidates per search
constexpr int kAwqBatch = 8;       // candidates per pass over a group in the search
constexpr int kSqCh = 8;           // channels per thread in the statistics pass
constexpr int kSqBlockCh = 256 * kSqCh;
constexpr int kSqTok = 8;          // tokens loaded together per thread

template <int DT>
GPTQ_DEV float ld(const void* p, size_t i) {
  if constexpr (DT == GPTQ_F32) return static_cast<const float*>(p)[i];
  else if constexpr (DT == GPTQ_F16) return (float)static_cast<const _Float16*>(p)[i];
  else return __builtin_bit_cast(float, (uint32_t)static_cast<const uint16_t*>(p)[i] << 16);
}

// Eight consecutive values of X starting at element i (16-bit types: one
// 16-byte load; fp32: two).  VEC: i is a multiple of 8 and rows are aligned.
template <int DT, bool VEC>
GPTQ_DEV void ld8(const void* p, size_t i, int nvalid, float (&v)[kSqCh]) {
  if constexpr (VEC) {
    if constexpr (DT == GPTQ_F32) {
      const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
      const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
      const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + i);
      const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if constexpr (DT == GPTQ_F16) {
          v[2 * k] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u[k] & 0xFFFFu));
          v[2 * k + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u[k] >> 16));
        } else {
          v[2 * k] = __builtin_bit_cast(float, u[k] << 16);
          v[2 * k + 1] = __builtin_bit_cast(float, u[k] & 0xFFFF0000u);
        }
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < kSqCh; ++k) v[k] = (k < nvalid) ? ld<DT>(p, i + k) : 0.0f;
  }
}

// Split s of the tokens, 2048 channels per block: each thread sums the exact
// fp64 squares of its eight channels over the split's tokens in token order.
template <int DT, bool VEC>
__global__ __launch_bounds__(256) void sumsq_kernel(const void* __restrict__ X, int64_t n, int d,
                                                    int64_t per_split, double* __restrict__ part) {
  const int c0 = (blockIdx.x * 256 + threadIdx.x) * kSqCh;
  if (c0 >= d) return;
  const int nvalid = min(kSqCh, d - c0);
  const int64_t t0 = (int64_t)blockIdx.y * per_split;
  const int64_t t1 = min(n, t0 + per_split);
  double acc[kSqCh];
#pragma unroll
  for (int k = 0; k < kSqCh; ++k) acc[k] = 0.0;
  // eight tokens' loads in flight, then their squares in token order
  int64_t t = t0;
  for (; t + kSqTok <= t1; t += kSqTok) {
    float v[kSqTok][kSqCh];
#pragma unroll
    for (int i = 0; i < kSqTok; ++i) ld8<DT, VEC>(X, (size_t)(t + i) * d + c0, nvalid, v[i]);
#pragma unroll
    for (int i = 0; i < kSqTok; ++i)
#pragma unroll
      for (int k = 0; k < kSqCh; ++k) {
        const double x = (double)v[i][k];
        acc[k] += x * x;
      }
  }
  for (; t < t1; ++t) {
    float v[kSqCh];
    ld8<DT, VEC>(X, (size_t)t * d + c0, nvalid, v);
#pragma unroll
    for (int k = 0; k < kSqCh; ++k) {
      const double x = (double)v[k];
      acc[k] += x * x;
    }
  }
  double* out = part + (size_t)blockIdx.y * d + c0;
#pragma unroll
  for (int k = 0; k < kSqCh; ++k)
    if (k < nvalid) out[k] = acc[k];
}

// a_j += the splits' partial sums, added in split order.
__global__ __launch_bounds__(256) void sumsq_reduce_kernel(const double* __restrict__ part, int splits, int d,
                                                           double* __restrict__ a) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= d) return;
  double s = 0.0;
  for (int p = 0; p < splits; ++p) s += part[(size_t)p * d + j];
  a[j] += s;
}

// above_j = the number of channels ranking above j (a larger a, or an equal a
// at a lower index), counted over channel chunks of kRankChunk (grid.y) and
// added with integer atomics (exact in any order); then mask_j = 1 when
// above_j < ktop: the top-ktop channels, ties to the lower index.
constexpr int kRankChunk = 256;
__global__ __launch_bounds__(256) void rank_count_kernel(const double* __restrict__ a, int d,
                                                         int* __restrict__ above) {
  __shared__ double sa[kRankChunk];
  const int j = blockIdx.x * 256 + threadIdx.x;
  const int k0 = blockIdx.y * kRankChunk;
  const double aj = (j < d) ? a[j] : 0.0;
  sa[threadIdx.x] = (k0 + (int)threadIdx.x < d) ? a[k0 + threadIdx.x] : 0.0;
  __syncthreads();
  const int kn = min(kRankChunk, d - k0);
  int cnt = 0;
  for (int u = 0; u < kn; ++u) {
    const double ak = sa[u];
    cnt += (ak > aj) || (ak == aj && k0 + u < j);
  }
  if (j < d && cnt) atomicAdd(above + j, cnt);
}

__global__ __launch_bounds__(256) void rank_mask_kernel(int* __restrict__ above, int d, int ktop,
                                                        uint8_t* __restrict__ mask) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j < d) mask[j] = (above[j] < ktop) ? 1 : 0;
}

__global__ __launch_bounds__(256) void zero_int_kernel(int* __restrict__ p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

// The asymmetric min-max grid of [mn, mx] with correctly rounded divisions.
GPTQ_DEV void awq_grid(float mn, float mx, float maxq, float& scale, float& zero) {
  if (mx == mn) {
    mn = fminf(mn, 0.0f);
    mx = fmaxf(mx, 0.0f);
  }
  const float rng = (mx == mn) ? maxq : mx - mn;
  scale = __fdiv_rn(rng, maxq);
  zero = rintf(__fdiv_rn(-mn, scale));
}

GPTQ_DEV float wave_min(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o));
  return v;
}
GPTQ_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

struct AwqGrid {
  float v[kAwqMaxGrid];      // the candidate factors
  double r[kAwqMaxGrid];     // their correctly rounded fp64 reciprocals
};

// rint(RN(x / y)) with y > 0 and ry = RN(1/y), without a division in almost
// every case: t = RN(x * ry) is within 2^-23 |t| of the real quotient and the
// correctly rounded quotient within 2^-24 of it, so unless a half-integer
// lies within 4e-7 |t| + 1e-6 of t (then the correctly rounded quotient is
// formed and decides) both round to the same integer.  For |t| >= 1.25e6 the
// division is always taken.
GPTQ_DEV float rint_quot(float x, float y, float ry) {
  const float t = x * ry;
  const float r = rintf(t);
  if (fabsf(fabsf(t - r) - 0.5f) <= 4e-7f * fabsf(t) + 1e-6f) return rintf(__fdiv_rn(x, y));
  return r;
}

// RN(a / b) for b a float32 value > 0 (as a double) and rb = RN(1/b): the
// quotient of the reciprocal, corrected once with the exact remainder
// (Markstein's correction; it rounds correctly unless b's 53-bit significand
// is all ones, which a float32 value cannot have).
GPTQ_DEV double quot64(double a, double b, double rb) {
  const double q0 = a * rb;
  const double rem = __builtin_fma(-q0, b, a);
  return __builtin_fma(rem, rb, q0);
}

// Lanes are weight rows: wave w of block (rb, gb, kb) takes rows 64 rb .. +63,
// group 4 gb + w and candidates 8 kb .. 8 kb + 7, so every column's statistic
// and salient flag are the same for the whole wave.  Per lane: the extremes of the salient and of the
// other weights of its row's group (w -> fp32(w * sigma) is monotone, so the
// scaled group's extremes follow from them for every sigma), the grid of
// its candidates, then one pass over the group's columns, eight at a time,
// accumulating each candidate's weighted squared error in fp64.  The wave's
// sums per candidate go to part[(rb * ng + g) * 32 + k].  VEC: 16-byte loads
// (groups and rows start at multiples of 8 columns, W 16-byte aligned).
template <int DT, bool VEC>
__global__ __launch_bounds__(256) void awq_search_kernel(const void* __restrict__ W, int d_out, int d,
                                                         const double* __restrict__ a,
                                                         const uint8_t* __restrict__ mask, AwqGrid grid,
                                                         int n_grid, int G, int ng, float maxq,
                                                         double* __restrict__ part) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  const int g = __builtin_amdgcn_readfirstlane(blockIdx.y * 4 + (threadIdx.x >> 6));
  if (g >= ng) return;
  const int row = blockIdx.x * 64 + lane;
  const bool live = row < d_out;
  const size_t rb = (size_t)min(row, d_out - 1) * d;
  const int c0 = g * G, c1 = min(d, c0 + G);

  auto load8 = [&](int cc, int nv, float (&wv)[8]) {
    if constexpr (VEC) {
      ld8<DT, true>(W, rb + cc, 8, wv);
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) wv[u] = (u < nv) ? ld<DT>(W, rb + cc + u) : 0.0f;
    }
  };

  float mn0 = INFINITY, mx0 = -INFINITY, mns = INFINITY, mxs = -INFINITY;
  for (int cc = c0; cc < c1; cc += 8) {
    const int nv = min(8, c1 - cc);
    float wv[8];
    load8(cc, nv, wv);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (u < nv) {
        if (mask[cc + u]) {
          mns = fminf(mns, wv[u]);
          mxs = fmaxf(mxs, wv[u]);
        } else {
          mn0 = fminf(mn0, wv[u]);
          mx0 = fmaxf(mx0, wv[u]);
        }
      }
    }
  }
  // candidates k0 .. k0 + kAwqBatch - 1 (blockIdx.z = batch), their grids and
  // sums in registers
  double* out = part + ((size_t)blockIdx.x * ng + g) * kAwqMaxGrid;
  {
    const int k0 = blockIdx.z * kAwqBatch;
    float scl[kAwqBatch], zer[kAwqBatch], rsc[kAwqBatch], sgv[kAwqBatch];
    double acc[kAwqBatch], rsg[kAwqBatch];
#pragma unroll
    for (int kk = 0; kk < kAwqBatch; ++kk) {
      acc[kk] = 0.0;
      scl[kk] = 1.0f;
      zer[kk] = 0.0f;
      rsc[kk] = 1.0f;
      sgv[kk] = 1.0f;
      rsg[kk] = 1.0;
      if (k0 + kk < n_grid) {
        sgv[kk] = grid.v[k0 + kk];
        rsg[kk] = grid.r[k0 + kk];
        // fp32(mns * sg) is +inf when the group has no salient channel
        awq_grid(fminf(mn0, mns * sgv[kk]), fmaxf(mx0, mxs * sgv[kk]), maxq, scl[kk], zer[kk]);
        rsc[kk] = __fdiv_rn(1.0f, scl[kk]);
      }
    }
    for (int cc = c0; cc < c1; cc += 8) {
      const int nv = min(8, c1 - cc);
      float wv[8];
      load8(cc, nv, wv);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (u < nv) {
          const int c = cc + u;
          const double ac = a[c];
          const double wd = (double)wv[u];
          if (mask[c]) {
#pragma unroll
            for (int kk = 0; kk < kAwqBatch; ++kk) {
              if (k0 + kk < n_grid) {
                const float code =
                    fminf(fmaxf(rint_quot(wv[u] * sgv[kk], scl[kk], rsc[kk]) + zer[kk], 0.0f), maxq);
                const double qh =
                    quot64((double)scl[kk] * ((double)code - (double)zer[kk]), (double)sgv[kk], rsg[kk]);
                const double df = wd - qh;
                acc[kk] = acc[kk] + (ac * df) * df;
              }
            }
          } else {
#pragma unroll
            for (int kk = 0; kk < kAwqBatch; ++kk) {
              if (k0 + kk < n_grid) {
                const float code = fminf(fmaxf(rint_quot(wv[u], scl[kk], rsc[kk]) + zer[kk], 0.0f), maxq);
                const double df = wd - (double)scl[kk] * ((double)code - (double)zer[kk]);
                acc[kk] = acc[kk] + (ac * df) * df;
              }
            }
          }
        }
      }
    }
#pragma unroll
    for (int kk = 0; kk < kAwqBatch; ++kk) {
      if (k0 + kk < n_grid) {
        double v = live ? acc[kk] : 0.0;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) v = v + __shfl_xor(v, o);
        if (lane == 0) out[k0 + kk] = v;
      }
    }
  }
}

// scores[k] = sum over the n_part (row block, group) partials part[p][k], in
// a fixed order.
__global__ __launch_bounds__(256) void awq_score_kernel(const double* __restrict__ part, int n_part,
                                                        double* __restrict__ scores) {
  __shared__ double red[256];
  const int k = blockIdx.x;
  double s = 0.0;
  for (int r = threadIdx.x; r < n_part; r += 256) s += part[(size_t)r * kAwqMaxGrid + k];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) scores[k] = red[0];
}

// The first candidate with the smallest score; s_j = its sigma on salient
// channels, 1 elsewhere.
__global__ __launch_bounds__(256) void awq_select_kernel(const double* __restrict__ scores, int n_grid,
                                                         AwqGrid grid, const uint8_t* __restrict__ mask,
                                                         int d, float* __restrict__ s_out,
                                                         int32_t* __restrict__ best) {
  int bi = 0;
  for (int k = 1; k < n_grid; ++k)
    if (scores[k] < scores[bi]) bi = k;
  const float sg = grid.v[bi];
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j < d) s_out[j] = mask[j] ? sg : 1.0f;
  if (j == 0 && best) *best = bi;
}

// One wave per row: per group the grid of fp32(w * s_j), codes, and the
// effective weights scale * (code - zero) / s_j.
template <int DT>
__global__ __launch_bounds__(256) void awq_quant_kernel(const void* __restrict__ W, int d_out, int d,
                                                        const float* __restrict__ s, int G, int ng, float maxq,
                                                        uint8_t* __restrict__ codes, float* __restrict__ scales,
                                                        int32_t* __restrict__ zeros, float* __restrict__ Qhat) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= d_out) return;
  const size_t rb = (size_t)row * d;
  for (int c0 = 0, g = 0; c0 < d; c0 += G, ++g) {
    const int c1 = min(d, c0 + G);
    float mn = INFINITY, mx = -INFINITY;
    for (int c = c0 + lane; c < c1; c += 64) {
      const float ws = ld<DT>(W, rb + c) * s[c];
      mn = fminf(mn, ws);
      mx = fmaxf(mx, ws);
    }
    mn = wave_min(mn);
    mx = wave_max(mx);
    float scale, zero;
    awq_grid(mn, mx, maxq, scale, zero);
    if (lane == 0) {
      scales[(size_t)row * ng + g] = scale;
      zeros[(size_t)row * ng + g] = (int32_t)zero;
    }
    for (int c = c0 + lane; c < c1; c += 64) {
      const float sc = s[c];
      const float ws = ld<DT>(W, rb + c) * sc;
      const float code = fminf(fmaxf(rintf(__fdiv_rn(ws, scale)) + zero, 0.0f), maxq);
      codes[rb + c] = (uint8_t)code;
      if (Qhat) Qhat[rb + c] = (float)(((double)scale * ((double)code - (double)zero)) / (double)sc);
    }
  }
}

struct SumsqShape {
  int cblocks;
  int splits;
  int64_t per_split;
};

static SumsqShape sumsq_shape(int64_t n, int d) {
  SumsqShape sh;
  sh.cblocks = (d + kSqBlockCh - 1) / kSqBlockCh;
  const int64_t max_splits = std::max<int64_t>(1, (n + 63) / 64);       // at least 64 tokens a split
  sh.splits = (int)std::max<int64_t>(1, std::min<int64_t>(512 / sh.cblocks, max_splits));
  sh.per_split = (n + sh.splits - 1) / sh.splits;
  sh.splits = (int)std::max<int64_t>(1, (n + sh.per_split - 1) / sh.per_split);
  return sh;
}

struct SearchLayout {
  size_t off_mask, off_above, off_part, total;
};

// partials: one per (64-row block, group)
static SearchLayout search_layout(int d_out, int d, int G) {
  SearchLayout L;
  L.off_mask = 0;
  L.off_above = align_up((size_t)d);
  L.off_part = align_up(L.off_above + (size_t)d * sizeof(int));
  const size_t nparts = (size_t)((d_out + 63) / 64) * ((d + G - 1) / G);
  L.total = align_up(L.off_part + nparts * kAwqMaxGrid * sizeof(double));
  return L;
}

}  // namespace gptq

using namespace gptq;

extern "C" size_t gptq_awq_sumsq_workspace_size(int64_t n_tokens, int32_t d_in) {
  if (n_tokens <= 0 || d_in <= 0) return 0;
  const SumsqShape sh = sumsq_shape(n_tokens, d_in);
  return align_up((size_t)sh.splits * d_in * sizeof(double));
}

extern "C" int gptq_awq_act_sumsq(double* sumsq, const void* X, gptq_dtype x_dtype, int64_t n_tokens,
                                  int32_t d_in, void* ws, size_t ws_bytes, hipStream_t s) {
  if (!sumsq || d_in <= 0 || n_tokens < 0) return GPTQ_ERR_INVALID_ARG;
  if (x_dtype != GPTQ_F32 && x_dtype != GPTQ_F16 && x_dtype != GPTQ_BF16) return GPTQ_ERR_INVALID_ARG;
  if (n_tokens == 0) return GPTQ_OK;
  if (!X) return GPTQ_ERR_INVALID_ARG;
  const SumsqShape sh = sumsq_shape(n_tokens, d_in);
  if (!ws || ws_bytes < (size_t)sh.splits * d_in * sizeof(double)) return GPTQ_ERR_WORKSPACE;
  double* part = static_cast<double*>(ws);
  const bool aligned = (reinterpret_cast<uintptr_t>(X) & 15) == 0;
  const bool vec = aligned && (x_dtype == GPTQ_F32 ? (d_in % 4 == 0) : (d_in % 8 == 0));
  const dim3 grid(sh.cblocks, sh.splits);
#define GPTQ_SUMSQ(DT)                                                                             \
  (vec ? sumsq_kernel<DT, true><<<grid, 256, 0, s>>>(X, n_tokens, d_in, sh.per_split, part)         \
       : sumsq_kernel<DT, false><<<grid, 256, 0, s>>>(X, n_tokens, d_in, sh.per_split, part))
  if (x_dtype == GPTQ_F32) GPTQ_SUMSQ(GPTQ_F32);
  else if (x_dtype == GPTQ_F16) GPTQ_SUMSQ(GPTQ_F16);
  else GPTQ_SUMSQ(GPTQ_BF16);
#undef GPTQ_SUMSQ
  GPTQ_LAUNCH_CHECK();
  sumsq_reduce_kernel<<<(d_in + 255) / 256, 256, 0, s>>>(part, sh.splits, d_in, sumsq);
  GPTQ_LAUNCH_CHECK();
  return GPTQ_OK;
}

extern "C" size_t gptq_awq_search_workspace_size(int32_t d_out, int32_t d_in, int32_t group_size) {
  if (d_out <= 0 || d_in <= 0 || group_size == 0 || group_size < -1) return 0;
  return search_layout(d_out, d_in, group_size == -1 ? d_in : group_size).total;
}

static int awq_common_checks(const void* W, gptq_dtype w_dtype, int32_t d_out, int32_t d_in, int32_t bits,
                             int32_t group_size) {
  if (!W || d_out <= 0 || d_in <= 0) return GPTQ_ERR_INVALID_ARG;
  if (w_dtype != GPTQ_F32 && w_dtype != GPTQ_F16 && w_dtype != GPTQ_BF16) return GPTQ_ERR_INVALID_ARG;
  if (bits < 2 || bits > 8) return GPTQ_ERR_INVALID_ARG;
  if (group_size != -1 && group_size <= 0) return GPTQ_ERR_INVALID_ARG;
  return GPTQ_OK;
}

extern "C" int gptq_awq_search(const void* W, gptq_dtype w_dtype, int32_t d_out, int32_t d_in,
                               const double* sumsq, int32_t bits, int32_t group_size, float top_frac,
                               const float* grid, int32_t n_grid, float* s_out, double* scores,
                               int32_t* best, void* ws, size_t ws_bytes, hipStream_t s) {
  const int st = awq_common_checks(W, w_dtype, d_out, d_in, bits, group_size);
  if (st != GPTQ_OK) return st;
  if (!sumsq || !grid || !s_out || !scores) return GPTQ_ERR_INVALID_ARG;
  if (n_grid < 1 || n_grid > kAwqMaxGrid) return GPTQ_ERR_INVALID_ARG;
  if (!(top_frac >= 0.0f && top_frac <= 1.0f)) return GPTQ_ERR_INVALID_ARG;
  AwqGrid gv{};
  for (int k = 0; k < n_grid; ++k) {
    if (!(grid[k] > 0.0f) || !std::isfinite(grid[k])) return GPTQ_ERR_INVALID_ARG;
    gv.v[k] = grid[k];
    gv.r[k] = 1.0 / (double)grid[k];
  }
  const int G = (group_size == -1) ? d_in : group_size;
  const SearchLayout L = search_layout(d_out, d_in, G);
  if (!ws || ws_bytes < L.total) return GPTQ_ERR_WORKSPACE;
  uint8_t* mask = static_cast<uint8_t*>(ws) + L.off_mask;
  double* part = reinterpret_cast<double*>(static_cast<char*>(ws) + L.off_part);
  const float maxq = (float)((1 << bits) - 1);
  // k = top_frac * d_in rounded to nearest, halves up, in double
  const int ktop = (int)std::min<double>(d_in, std::floor((double)top_frac * d_in + 0.5));

  int* above = reinterpret_cast<int*>(static_cast<char*>(ws) + L.off_above);
  zero_int_kernel<<<(d_in + 255) / 256, 256, 0, s>>>(above, d_in);
  rank_count_kernel<<<dim3((d_in + 255) / 256, (d_in + kRankChunk - 1) / kRankChunk), 256, 0, s>>>(sumsq, d_in,
                                                                                                 above);
  rank_mask_kernel<<<(d_in + 255) / 256, 256, 0, s>>>(above, d_in, ktop, mask);
  GPTQ_LAUNCH_CHECK();
  const int ng = (d_in + G - 1) / G;
  const dim3 sgrid((unsigned)((d_out + 63) / 64), (unsigned)((ng + 3) / 4),
                   (unsigned)((n_grid + kAwqBatch - 1) / kAwqBatch));
  const bool vec = (G % 8 == 0) && (d_in % 8 == 0) && (reinterpret_cast<uintptr_t>(W) & 15) == 0;
#define GPTQ_SEARCH(DT)                                                                                      \
  (vec ? awq_search_kernel<DT, true><<<sgrid, 256, 0, s>>>(W, d_out, d_in, sumsq, mask, gv, n_grid, G, ng,   \
                                                           maxq, part)                                       \
       : awq_search_kernel<DT, false><<<sgrid, 256, 0, s>>>(W, d_out, d_in, sumsq, mask, gv, n_grid, G, ng,  \
                                                            maxq, part))
  if (w_dtype == GPTQ_F32) GPTQ_SEARCH(GPTQ_F32);
  else if (w_dtype == GPTQ_F16) GPTQ_SEARCH(GPTQ_F16);
  else GPTQ_SEARCH(GPTQ_BF16);
#undef GPTQ_SEARCH
  GPTQ_LAUNCH_CHECK();
  awq_score_kernel<<<n_grid, 256, 0, s>>>(part, (int)(sgrid.x * ng), scores);
  GPTQ_LAUNCH_CHECK();
  awq_select_kernel<<<(d_in + 255) / 256, 256, 0, s>>>(scores, n_grid, gv, mask, d_in, s_out, best);
  GPTQ_LAUNCH_CHECK();
  return GPTQ_OK;
}

extern "C" int gptq_awq_quantize(const void* W, gptq_dtype w_dtype, int32_t d_out, int32_t d_in,
                                 const float* s_in, int32_t bits, int32_t group_size, uint8_t* codes,
                                 float* scales, int32_t* zeros, float* Qhat, hipStream_t s) {
  const int st = awq_common_checks(W, w_dtype, d_out, d_in, bits, group_size);
  if (st != GPTQ_OK) return st;
  if (!s_in || !codes || !scales || !zeros) return GPTQ_ERR_INVALID_ARG;
  const int G = (group_size == -1) ? d_in : group_size;
  const int ng = (d_in + G - 1) / G;
  const float maxq = (float)((1 << bits) - 1);
  const unsigned rows_grid = (unsigned)((d_out + 3) / 4);
  if (w_dtype == GPTQ_F32)
    awq_quant_kernel<GPTQ_F32><<<rows_grid, 256, 0, s>>>(W, d_out, d_in, s_in, G, ng, maxq, codes, scales, zeros, Qhat);
  else if (w_dtype == GPTQ_F16)
    awq_quant_kernel<GPTQ_F16><<<rows_grid, 256, 0, s>>>(W, d_out, d_in, s_in, G, ng, maxq, codes, scales, zeros, Qhat);
  else
    awq_quant_kernel<GPTQ_BF16><<<rows_grid, 256, 0, s>>>(W, d_out, d_in, s_in, G, ng, maxq, codes, scales, zeros, Qhat);
  GPTQ_LAUNCH_CHECK();
  return GPTQ_OK;
}
