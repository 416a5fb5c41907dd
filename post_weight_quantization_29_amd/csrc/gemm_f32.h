// fp32 MFMA GEMM (v_mfma_f32_32x32x2f32) shared by the inverse-Hessian
// factorization, the lazy-batch trailing update and the layer error.
//
//   C[M x N] = alpha * Aop * Bop + beta * C          (epilogue kStore)
//   out[tile] = sum_{m,n} (Aop * Bop)[m][n] * D[m][n] (epilogue kDot, fp64)
//
// Aop(m, k) = A[k*lda + m] ("k-major", A_KMAJOR) or A[m*lda + k];
// Bop(k, n) = B[k*ldb + n] always.  Tiles are 128x128, four waves (2x2) of
// 64x64, 16 values of k per LDS stage, double-buffered.  Several independent
// problems of one shape class (a "group") run in one launch; each workgroup
// finds its problem from the tile prefix sums passed by value.
//
// Optional triangular structure, decided per tile:
//   kloFromM: the contraction starts at k = m0 (Aop upper triangular),
//   khiFromN: it stops at k = n0 + 128 (Bop upper triangular),
//   upperOnly: tiles strictly below the diagonal are skipped (symmetric update).
#pragma once
#include "common.h"

namespace gptq {

constexpr int kGT = 128;          // tile edge
constexpr int kGK = 16;           // k per stage
constexpr int kGP = kGT + 32;     // LDS pitch (floats): the two half-waves of an
                                  // operand read sit 32 banks apart
constexpr int kGemmMaxGroup = 32;

struct GemmProblem {
  const float* A;
  const float* B;
  float* C;          // kStore: output; kDot: unused
  const float* D;    // kDot: the matrix the product is dotted with (ld = ldc)
  int lda, ldb, ldc;
  int M, N, K;
};

struct GemmGroup {
  GemmProblem p[kGemmMaxGroup];
  int tile_start[kGemmMaxGroup + 1];   // prefix sums of tiles per problem
  int count;
};

enum GemmEpilogue { kStore = 0, kDot = 1 };

template <bool A_KMAJOR, int EPI>
__global__ __launch_bounds__(256, 2) void gemm_f32_kernel(GemmGroup grp, float alpha, float beta,
                                                          int kloFromM, int khiFromN, int upperOnly,
                                                          double* __restrict__ dot_out) {
  __shared__ __attribute__((aligned(16))) float sA[2][kGK * kGP];
  __shared__ __attribute__((aligned(16))) float sB[2][kGK * kGP];
  __shared__ double sRed[4];

  const int wg = blockIdx.x;
  int pi = 0;
  while (pi + 1 < grp.count && grp.tile_start[pi + 1] <= wg) ++pi;
  const GemmProblem& P = grp.p[pi];
  const int local = wg - grp.tile_start[pi];
  const int tn = (P.N + kGT - 1) / kGT;
  const int m0 = (local / tn) * kGT, n0 = (local % tn) * kGT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const bool skip = upperOnly && (n0 + kGT <= m0);
  int klo = kloFromM ? m0 : 0;
  int khi = khiFromN ? min(P.K, n0 + kGT) : P.K;
  if (khi < klo) khi = klo;

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  if (!skip && klo < khi) {
    float ra[8], rb[8];
    // B (and k-major A): 16 rows of 128 -> thread owns column c = tid%128, rows r0+2i
    // m-major A: 128 rows of 16 -> thread owns k = tid%16, rows tid/16 + 16i
    auto gload = [&](int k0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int kr = (tid >> 7) + 2 * i, c = tid & 127;
        const int k = k0 + kr, n = n0 + c;
        rb[i] = (k < khi && n < P.N) ? P.B[(size_t)k * P.ldb + n] : 0.0f;
        if (A_KMAJOR) {
          const int m = m0 + c;
          ra[i] = (k < khi && m < P.M) ? P.A[(size_t)k * P.lda + m] : 0.0f;
        } else {
          const int kk = k0 + (tid & 15), mr = (tid >> 4) + 16 * i, m = m0 + mr;
          ra[i] = (kk < khi && m < P.M) ? P.A[(size_t)m * P.lda + kk] : 0.0f;
        }
      }
    };
    auto lstore = [&](int buf) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int kr = (tid >> 7) + 2 * i, c = tid & 127;
        sB[buf][kr * kGP + c] = rb[i];
        if (A_KMAJOR) {
          sA[buf][kr * kGP + c] = ra[i];
        } else {
          sA[buf][(tid & 15) * kGP + (tid >> 4) + 16 * i] = ra[i];
        }
      }
    };
    const int kbeg = klo - (klo % kGK);
    gload(kbeg);
    lstore(0);
    __syncthreads();
    int buf = 0;
    for (int k0 = kbeg; k0 < khi; k0 += kGK) {
      const bool more = k0 + kGK < khi;
      if (more) gload(k0 + kGK);
      const float* a_s = sA[buf];
      const float* b_s = sB[buf];
#pragma unroll
      for (int k2 = 0; k2 < kGK; k2 += 2) {
        const int row = (k2 + (lane >> 5)) * kGP + (lane & 31);
        const float a0 = a_s[row + wm * 64], a1 = a_s[row + wm * 64 + 32];
        const float b0 = b_s[row + wn * 64], b1 = b_s[row + wn * 64 + 32];
        acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
        acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
        acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
        acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
      }
      if (more) lstore(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
  }

  if (EPI == kStore) {
    if (skip) return;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + wm * 64 + i * 32 + mfma32_row(r, lane);
          const int n = n0 + wn * 64 + j * 32 + mfma32_col(lane);
          if (m < P.M && n < P.N) {
            float* c = P.C + (size_t)m * P.ldc + n;
            float v = alpha * acc[i][j][r];
            if (beta != 0.0f) v += beta * *c;
            *c = v;
          }
        }
  } else {
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + wm * 64 + i * 32 + mfma32_row(r, lane);
          const int n = n0 + wn * 64 + j * 32 + mfma32_col(lane);
          if (m < P.M && n < P.N) s += (double)acc[i][j][r] * (double)P.D[(size_t)m * P.ldc + n];
        }
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) sRed[wave] = s;
    __syncthreads();
    if (tid == 0) dot_out[wg] = ((sRed[0] + sRed[1]) + (sRed[2] + sRed[3]));
  }
}

inline int gemm_tiles(int M, int N) { return ((M + kGT - 1) / kGT) * ((N + kGT - 1) / kGT); }

// Launch one group (count <= kGemmMaxGroup).  Returns the total tile count.
template <bool A_KMAJOR, int EPI>
inline int launch_gemm_group(GemmGroup& g, float alpha, float beta, int kloFromM, int khiFromN,
                             int upperOnly, double* dot_out, hipStream_t s) {
  int t = 0;
  for (int i = 0; i < g.count; ++i) {
    g.tile_start[i] = t;
    t += gemm_tiles(g.p[i].M, g.p[i].N);
  }
  g.tile_start[g.count] = t;
  if (t > 0)
    gemm_f32_kernel<A_KMAJOR, EPI><<<t, 256, 0, s>>>(g, alpha, beta, kloFromM, khiFromN, upperOnly,
                                                    dot_out);
  return t;
}

template <bool A_KMAJOR>
inline void gemm_f32(const float* A, int lda, const float* B, int ldb, float* C, int ldc, int M,
                     int N, int K, float alpha, float beta, int kloFromM, int khiFromN, int upperOnly,
                     hipStream_t s) {
  if (M <= 0 || N <= 0) return;
  GemmGroup g;
  g.count = 1;
  g.p[0] = GemmProblem{A, B, C, nullptr, lda, ldb, ldc, M, N, K};
  launch_gemm_group<A_KMAJOR, kStore>(g, alpha, beta, kloFromM, khiFromN, upperOnly, nullptr, s);
}

}  // namespace gptq
