// fp32 MFMA GEMM (v_mfma_f32_32x32x2f32) shared by the inverse-Hessian
// factorization, the lazy-batch trailing update and the layer error.
//
//   C[M x N] = alpha * Aop * Bop + beta * C          (epilogue kStore)
//   out[tile] = sum_{m,n} (Aop * Bop)[m][n] * D[m][n] (epilogue kDot, fp64)
//
// Aop(m, k) = A[k*lda + m] ("k-major", A_KMAJOR) or A[m*lda + k];
// Bop(k, n) = B[k*ldb + n] always.  Tiles are 128x128, four waves (2x2) of
// 64x64; k runs in chunks of 32, each loaded into registers (float4 when the
// leading dimensions allow) while the previous chunk is multiplied out of
// LDS, so global latency hides behind a chunk of MFMA work.  Several independent
// problems of one shape class (a "group") run in one launch; each workgroup
// finds its problem from the tile prefix sums passed by value.
//
// Optional triangular structure, decided per tile:
//   kloFromM: the contraction starts at k = m0 (Aop upper triangular),
//   khiFromN: it stops at k = n0 + 128 (Bop upper triangular),
//   upperOnly: only tiles on or right of the diagonal are launched (symmetric
//              update); the grid holds no idle workgroups, which would
//              otherwise skew how the dispatcher spreads the real ones over CUs.
#pragma once
#include "common.h"

namespace gptq {

constexpr int kGT = 128;          // tile edge
constexpr int kGK = 32;           // k per chunk: loaded into registers one chunk ahead
constexpr int kGP = kGT + 4;      // LDS pitch (floats)
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
  int ndesc;   // set by the launchers: tiles run by column from the last one
};

// Origin of tile `local` of a problem: row by row, or (ndesc) column by column
// from the last column, so that with khiFromN the tiles with the longest
// contraction are dispatched first and the short ones fill in behind them.
GPTQ_DEV void tile_origin(const GemmProblem& P, int local, int ndesc, int& m0, int& n0) {
  if (ndesc) {
    const int tm = (P.M + kGT - 1) / kGT, tn = (P.N + kGT - 1) / kGT;
    m0 = (local % tm) * kGT;
    n0 = (tn - 1 - local / tm) * kGT;
  } else {
    const int tn = (P.N + kGT - 1) / kGT;
    m0 = (local / tn) * kGT;
    n0 = (local % tn) * kGT;
  }
}

enum GemmEpilogue { kStore = 0, kDot = 1, kPartial = 2 };

// 4 consecutive floats p[0..3], the ones at index >= lim read as 0.  VEC: the
// address is 16-byte aligned whenever lim >= 4.
template <bool VEC>
GPTQ_DEV float4 load4(const float* p, int lim) {
  if (VEC && lim >= 4) return *reinterpret_cast<const float4*>(p);
  float4 r;
  r.x = lim > 0 ? p[0] : 0.0f;
  r.y = lim > 1 ? p[1] : 0.0f;
  r.z = lim > 2 ? p[2] : 0.0f;
  r.w = lim > 3 ? p[3] : 0.0f;
  return r;
}

// One chunk of kGK = 32 k: A chunk 128 (m) x 32 (k), B chunk 32 (k) x 128 (n);
// each thread holds 4 float4 of each.
constexpr int kGL = kGK * kGT / 1024;   // float4 per thread per operand chunk
template <bool A_KMAJOR, bool VEC>
GPTQ_DEV void gemm_gload(const GemmProblem& P, int m0, int n0, int k0, int khi, int tid,
                         float4 (&ra)[kGL], float4 (&rb)[kGL]) {
  // B (and k-major A): row k = k0 + tid/32 + 8i, columns c = 4*(tid%32) .. +3
  const int c4 = 4 * (tid & 31);
  if (VEC && A_KMAJOR && m0 + kGT <= P.M && n0 + kGT <= P.N && k0 + kGK <= khi) {
    // a chunk inside every bound (the common case; the test is uniform over
    // the workgroup): no per-lane limits, so no branches around the loads
#pragma unroll
    for (int i = 0; i < kGL; ++i) {
      const int k = k0 + (tid >> 5) + 8 * i;
      rb[i] = *reinterpret_cast<const float4*>(P.B + (size_t)k * P.ldb + n0 + c4);
      ra[i] = *reinterpret_cast<const float4*>(P.A + (size_t)k * P.lda + m0 + c4);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < kGL; ++i) {
    const int k = k0 + (tid >> 5) + 8 * i;
    const bool kv = k < khi;
    rb[i] = kv ? load4<VEC>(P.B + (size_t)k * P.ldb + n0 + c4, P.N - n0 - c4)
               : make_float4(0.f, 0.f, 0.f, 0.f);
    if (A_KMAJOR)
      ra[i] = kv ? load4<VEC>(P.A + (size_t)k * P.lda + m0 + c4, P.M - m0 - c4)
                 : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (!A_KMAJOR) {
    // m-major A: row m = m0 + tid/8 + 32i, k = k0 + 4*(tid%8) .. +3
    const int kq = k0 + 4 * (tid & 7);
#pragma unroll
    for (int i = 0; i < kGL; ++i) {
      const int m = m0 + (tid >> 3) + 32 * i;
      ra[i] = (m < P.M) ? load4<VEC>(P.A + (size_t)m * P.lda + kq, khi - kq)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
}

template <bool A_KMAJOR>
GPTQ_DEV void gemm_lstore(float* sA, float* sB, int tid, const float4 (&ra)[kGL], const float4 (&rb)[kGL]) {
  const int c4 = 4 * (tid & 31);
#pragma unroll
  for (int i = 0; i < kGL; ++i) {
    const int kr = (tid >> 5) + 8 * i;
    *reinterpret_cast<float4*>(sB + kr * kGP + c4) = rb[i];
    if (A_KMAJOR) *reinterpret_cast<float4*>(sA + kr * kGP + c4) = ra[i];
  }
  if (!A_KMAJOR) {
    const int kq = 4 * (tid & 7);
#pragma unroll
    for (int i = 0; i < kGL; ++i) {
      const int mr = (tid >> 3) + 32 * i;
      sA[(kq + 0) * kGP + mr] = ra[i].x;
      sA[(kq + 1) * kGP + mr] = ra[i].y;
      sA[(kq + 2) * kGP + mr] = ra[i].z;
      sA[(kq + 3) * kGP + mr] = ra[i].w;
    }
  }
}

// One 128x128 tile, four waves (2x2) of 64x64: acc += Aop[m0.., klo:khi] * Bop[klo:khi, n0..],
// k in chunks of kGK staged through sA, sB (kGK x kGP floats each); the next
// chunk is loaded into registers while the current one is multiplied.
template <bool A_KMAJOR, bool VEC>
GPTQ_DEV void gemm_tile_contract(const GemmProblem& P, int m0, int n0, int klo, int khi, float* sA, float* sB,
                                 f32x16_t (&acc)[2][2]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  if (klo >= khi) return;
  float4 ra[kGL], rb[kGL];
  gemm_gload<A_KMAJOR, VEC>(P, m0, n0, klo, khi, tid, ra, rb);
  for (int k0 = klo; k0 < khi; k0 += kGK) {
    __syncthreads();                         // the previous chunk is consumed
    gemm_lstore<A_KMAJOR>(sA, sB, tid, ra, rb);
    __syncthreads();
    if (k0 + kGK < khi) gemm_gload<A_KMAJOR, VEC>(P, m0, n0, k0 + kGK, khi, tid, ra, rb);
    const int kn = min(kGK, khi - k0);       // zero-filled beyond khi: keep even steps
#pragma unroll 4
    for (int k2 = 0; k2 < kn; k2 += 2) {
      const int row = (k2 + (lane >> 5)) * kGP + (lane & 31);
      const float a0 = sA[row + wm * 64], a1 = sA[row + wm * 64 + 32];
      const float b0 = sB[row + wn * 64], b1 = sB[row + wn * 64 + 32];
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
    }
  }
}

// C = alpha * acc + beta * C over the tile (beta == 0: alpha * acc, C not
// read), after the contraction: the old values of one half of a wave's
// 64 x 64 block (32 per thread) are read in one batch, then that half is
// written.  Holding C through the contraction cost registers (the tile runs
// three workgroups per CU), and its loads queued ahead of the first
// operand chunk's; the other workgroups on the CU cover this batch's latency.
GPTQ_DEV void gemm_tile_update(const GemmProblem& P, int m0, int n0, float alpha, float beta,
                               f32x16_t (&acc)[2][2]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    float cold[2][16];
    if (beta != 0.0f) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + wm * 64 + i * 32 + mfma32_row(r, lane);
          const int n = n0 + wn * 64 + j * 32 + mfma32_col(lane);
          cold[j][r] = (m < P.M && n < P.N) ? P.C[(size_t)m * P.ldc + n] : 0.0f;
        }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + i * 32 + mfma32_row(r, lane);
        const int n = n0 + wn * 64 + j * 32 + mfma32_col(lane);
        const float v = (beta != 0.0f) ? alpha * acc[i][j][r] + beta * cold[j][r] : alpha * acc[i][j][r];
        if (m < P.M && n < P.N) P.C[(size_t)m * P.ldc + n] = v;
      }
  }
}

// kPartial (split-K): workgroup w takes part w % parts of tile w / parts, i.e.
// the part's share of the tile's contraction range (cut in multiples of kGK),
// and writes its raw 128x128 sum to partial (float*) in MFMA register order,
// [tile*parts + part][wave 4][block 4][reg 16][lane 64]; gemm_splitk_reduce
// adds the parts in order.
template <bool A_KMAJOR, int EPI, bool VEC>
__global__ __launch_bounds__(256, 3) void gemm_f32_kernel(GemmGroup grp, float alpha, float beta,
                                                          int kloFromM, int khiFromN, int upperOnly,
                                                          double* __restrict__ dot_out, int parts = 1) {
  __shared__ __attribute__((aligned(16))) float sA[kGK * kGP];
  __shared__ __attribute__((aligned(16))) float sB[kGK * kGP];
  __shared__ double sRed[4];

  const int wg = (EPI == kPartial) ? (int)blockIdx.x / parts : (int)blockIdx.x;
  const int part = (EPI == kPartial) ? (int)blockIdx.x % parts : 0;
  int pi = 0;
  while (pi + 1 < grp.count && grp.tile_start[pi + 1] <= wg) ++pi;
  const GemmProblem P = grp.p[pi];          // fields held in registers from here on
  const int local = wg - grp.tile_start[pi];
  const int tn = (P.N + kGT - 1) / kGT;
  int m0, n0;
  if (upperOnly) {
    // only the tiles on or right of the diagonal are launched, row by row
    int r = 0, rem = local;
    while (rem >= tn - r) { rem -= tn - r; ++r; }
    m0 = r * kGT;
    n0 = (r + rem) * kGT;
  } else {
    tile_origin(P, local, grp.ndesc, m0, n0);
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const bool skip = upperOnly && (n0 + kGT <= m0);
  int klo = kloFromM ? m0 : 0;
  int khi = khiFromN ? min(P.K, n0 + kGT) : P.K;
  if (khi < klo) khi = klo;
  if (EPI == kPartial) {
    const int per = ((khi - klo + parts - 1) / parts + kGK - 1) / kGK * kGK;
    const int b = min(khi, klo + part * per);
    khi = min(khi, b + per);
    klo = b;
  }

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  if (!skip) gemm_tile_contract<A_KMAJOR, VEC>(P, m0, n0, klo, khi, sA, sB, acc);

  if (EPI == kPartial) {
    float* out = reinterpret_cast<float*>(dot_out) + ((size_t)blockIdx.x * 4 + wave) * (4 * 16 * 64);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) out[((i * 2 + j) * 16 + r) * 64 + lane] = acc[i][j][r];
    return;
  }
  if (EPI == kStore) {
    if (skip) return;
    gemm_tile_update(P, m0, n0, alpha, beta, acc);
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

// C = alpha * sum_p partial[tile][p] + beta * C, parts added in order.
// kRedSlices workgroups per tile (so that launches of a few tiles still spread
// over the chip); thread t of slice s handles elements s*1024 + t + 256u,
// u = 0..3, of the tile's 16384 in partial order (reads fully coalesced).
constexpr int kRedSlices = 16;
[[maybe_unused]] static __global__ __launch_bounds__(256) void gemm_splitk_reduce(GemmGroup grp, const float* __restrict__ partial,
                                                          int parts, float alpha, float beta) {
  const int wg = blockIdx.x / kRedSlices, slice = blockIdx.x % kRedSlices;
  int pi = 0;
  while (pi + 1 < grp.count && grp.tile_start[pi + 1] <= wg) ++pi;
  const GemmProblem P = grp.p[pi];
  int m0, n0;
  tile_origin(P, wg - grp.tile_start[pi], grp.ndesc, m0, n0);
  const float* src = partial + (size_t)wg * parts * 16384 + slice * 1024;
  float sum[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) sum[u] = 0.0f;
  for (int p = 0; p < parts; ++p) {
#pragma unroll
    for (int u = 0; u < 4; ++u) sum[u] += src[(size_t)p * 16384 + threadIdx.x + 256 * u];
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = slice * 1024 + threadIdx.x + 256 * u;
    const int w = e >> 12, blk = (e >> 10) & 3, r = (e >> 6) & 15, lane = e & 63;
    const int m = m0 + (w >> 1) * 64 + (blk >> 1) * 32 + mfma32_row(r, lane);
    const int n = n0 + (w & 1) * 64 + (blk & 1) * 32 + mfma32_col(lane);
    if (m < P.M && n < P.N) {
      const size_t off = (size_t)m * P.ldc + n;
      P.C[off] = (beta != 0.0f) ? alpha * sum[u] + beta * P.C[off] : alpha * sum[u];
    }
  }
}

// ---------------------------------------------------------------- small tiles
// The same product in 64x64 tiles (four waves of 32x32, one MFMA accumulator
// each), for launches of a few 128x128 tiles per CU or fewer: four times the
// workgroups, a quarter of the work each.  Every element takes the same MFMA
// steps in the same k order as in the 128x128 kernel, so the results are
// identical.  upperOnly works at 128-block granularity, like the large kernel
// (the diagonal 128-blocks are computed whole).
constexpr int kST = 64;            // small tile edge
constexpr int kSP = kST + 4;       // LDS pitch (floats)
constexpr int kSK = 64;            // k per chunk

template <bool A_KMAJOR, bool VEC>
__global__ __launch_bounds__(256) void gemm_f32_small_kernel(GemmGroup grp, float alpha, float beta,
                                                             int kloFromM, int khiFromN, int upperOnly) {
  __shared__ __attribute__((aligned(16))) float sA[kSK * kSP];
  __shared__ __attribute__((aligned(16))) float sB[kSK * kSP];
  const int wg = (int)blockIdx.x;
  int pi = 0;
  while (pi + 1 < grp.count && grp.tile_start[pi + 1] <= wg) ++pi;
  const GemmProblem P = grp.p[pi];
  const int local = wg - grp.tile_start[pi];
  const int tm = (P.M + kST - 1) / kST, tn = (P.N + kST - 1) / kST;
  int m0, n0;
  if (upperOnly) {
    // only the tiles of 128-blocks on or right of the diagonal are launched:
    // tile row r starts at tile column 2*(r/2)
    int r = 0, rem = local;
    while (rem >= tn - 2 * (r / 2)) { rem -= tn - 2 * (r / 2); ++r; }
    m0 = r * kST;
    n0 = (2 * (r / 2) + rem) * kST;
  } else if (grp.ndesc) {
    m0 = (local % tm) * kST;
    n0 = (tn - 1 - local / tm) * kST;
  } else {
    m0 = (local / tn) * kST;
    n0 = (local % tn) * kST;
  }
  if (upperOnly && (n0 / kGT) < (m0 / kGT)) return;
  // the contraction bounds of the 128x128 tile this tile lies in
  const int klo = kloFromM ? (m0 / kGT) * kGT : 0;
  int khi = khiFromN ? min(P.K, (n0 / kGT) * kGT + kGT) : P.K;
  if (khi < klo) khi = klo;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  f32x16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
  float cold[16];
  if (beta != 0.0f) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + wm * 32 + mfma32_row(r, lane), n = n0 + wn * 32 + mfma32_col(lane);
      cold[r] = (m < P.M && n < P.N) ? P.C[(size_t)m * P.ldc + n] : 0.0f;
    }
  }
  // chunk loads: B (and k-major A) rows k = tid/16 + 16i, columns 4(tid%16) .. +3;
  // m-major A rows m = tid/16 + 16i, k = 4(tid%16) .. +3
  auto gload = [&](int k0, float4 (&ra)[4], float4 (&rb)[4]) {
    const int c4 = 4 * (tid & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = k0 + (tid >> 4) + 16 * i;
      const bool kv = k < khi;
      rb[i] = kv ? load4<VEC>(P.B + (size_t)k * P.ldb + n0 + c4, P.N - n0 - c4) : make_float4(0.f, 0.f, 0.f, 0.f);
      if (A_KMAJOR)
        ra[i] = kv ? load4<VEC>(P.A + (size_t)k * P.lda + m0 + c4, P.M - m0 - c4) : make_float4(0.f, 0.f, 0.f, 0.f);
      else {
        const int m = m0 + (tid >> 4) + 16 * i, kq = k0 + c4;
        ra[i] = (m < P.M) ? load4<VEC>(P.A + (size_t)m * P.lda + kq, khi - kq) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  };
  if (klo < khi) {
    float4 ra[4], rb[4];
    gload(klo, ra, rb);
    for (int k0 = klo; k0 < khi; k0 += kSK) {
      __syncthreads();
      {
        const int c4 = 4 * (tid & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kr = (tid >> 4) + 16 * i;
          *reinterpret_cast<float4*>(sB + kr * kSP + c4) = rb[i];
          if (A_KMAJOR) {
            *reinterpret_cast<float4*>(sA + kr * kSP + c4) = ra[i];
          } else {
            sA[(c4 + 0) * kSP + kr] = ra[i].x;
            sA[(c4 + 1) * kSP + kr] = ra[i].y;
            sA[(c4 + 2) * kSP + kr] = ra[i].z;
            sA[(c4 + 3) * kSP + kr] = ra[i].w;
          }
        }
      }
      __syncthreads();
      if (k0 + kSK < khi) gload(k0 + kSK, ra, rb);
      const int kn = min(kSK, khi - k0);       // zero-filled beyond khi: keep even steps
#pragma unroll 4
      for (int k2 = 0; k2 < kn; k2 += 2) {
        const int row = (k2 + (lane >> 5)) * kSP + (lane & 31);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(sA[row + wm * 32], sB[row + wn * 32], acc, 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = m0 + wm * 32 + mfma32_row(r, lane), n = n0 + wn * 32 + mfma32_col(lane);
    if (m < P.M && n < P.N) P.C[(size_t)m * P.ldc + n] = (beta != 0.0f) ? alpha * acc[r] + beta * cold[r] : alpha * acc[r];
  }
}

// 64x64 tiles of a problem (upperOnly: those of 128-blocks on or right of the diagonal)
inline int gemm_small_tiles(int M, int N, int upperOnly) {
  const int sm = (M + kST - 1) / kST, sn = (N + kST - 1) / kST;
  if (!upperOnly) return sm * sn;
  int t = 0;
  for (int r = 0; r < sm; ++r) t += std::max(0, sn - 2 * (r / 2));
  return t;
}

// Launch one group in 64x64 tiles (kStore semantics, same results as the
// 128x128 kernel).
template <bool A_KMAJOR>
inline void launch_gemm_group_small(GemmGroup& g, float alpha, float beta, int kloFromM, int khiFromN,
                                    int upperOnly, hipStream_t s) {
  int t = 0;
  bool vec = true;
  for (int i = 0; i < g.count; ++i) {
    g.tile_start[i] = t;
    t += gemm_small_tiles(g.p[i].M, g.p[i].N, upperOnly);
    const GemmProblem& p = g.p[i];
    vec = vec && (p.lda % 4 == 0) && (p.ldb % 4 == 0) &&
          ((reinterpret_cast<uintptr_t>(p.A) | reinterpret_cast<uintptr_t>(p.B)) & 15) == 0;
  }
  g.tile_start[g.count] = t;
  g.ndesc = (khiFromN && !upperOnly) ? 1 : 0;
  if (t == 0) return;
  if (vec)
    gemm_f32_small_kernel<A_KMAJOR, true><<<t, 256, 0, s>>>(g, alpha, beta, kloFromM, khiFromN, upperOnly);
  else
    gemm_f32_small_kernel<A_KMAJOR, false><<<t, 256, 0, s>>>(g, alpha, beta, kloFromM, khiFromN, upperOnly);
}

inline int gemm_tiles(int M, int N) { return ((M + kGT - 1) / kGT) * ((N + kGT - 1) / kGT); }

// 128-tiles on or right of the diagonal (what an upperOnly launch runs)
inline int gemm_upper_tiles(int M, int N) {
  const int tm = (M + kGT - 1) / kGT, tn = (N + kGT - 1) / kGT;
  int t = 0;
  for (int r = 0; r < tm; ++r) t += std::max(0, tn - r);
  return t;
}

// Parts per tile for a launch of `tiles` tiles whose longest contraction is
// kmax: enough workgroups to fill the chip twice over (two resident per CU),
// each part at least 128 deep, at most 8 parts.
inline int splitk_parts(int tiles, int kmax) {
  if (tiles <= 0) return 1;
  int p = 1024 / tiles;
  p = std::min(p, kmax / 128);
  return std::max(1, std::min(8, p));
}

// Launch one group (count <= kGemmMaxGroup).  Returns the total tile count.
// float4 global loads are used when every leading dimension is a multiple of 4
// and every base pointer is 16-byte aligned (tile origins are multiples of 128).
template <bool A_KMAJOR, int EPI>
inline int launch_gemm_group(GemmGroup& g, float alpha, float beta, int kloFromM, int khiFromN,
                             int upperOnly, double* dot_out, hipStream_t s) {
  int t = 0;
  bool vec = true;
  for (int i = 0; i < g.count; ++i) {
    g.tile_start[i] = t;
    t += upperOnly ? gemm_upper_tiles(g.p[i].M, g.p[i].N) : gemm_tiles(g.p[i].M, g.p[i].N);
    const GemmProblem& p = g.p[i];
    vec = vec && (p.lda % 4 == 0) && (p.ldb % 4 == 0) &&
          ((reinterpret_cast<uintptr_t>(p.A) | reinterpret_cast<uintptr_t>(p.B)) & 15) == 0;
  }
  g.tile_start[g.count] = t;
  g.ndesc = (khiFromN && !upperOnly) ? 1 : 0;
  if (t > 0) {
    if (vec)
      gemm_f32_kernel<A_KMAJOR, EPI, true><<<t, 256, 0, s>>>(g, alpha, beta, kloFromM, khiFromN,
                                                           upperOnly, dot_out);
    else
      gemm_f32_kernel<A_KMAJOR, EPI, false><<<t, 256, 0, s>>>(g, alpha, beta, kloFromM, khiFromN,
                                                            upperOnly, dot_out);
  }
  return t;
}

// Split-K launch of a group (kStore semantics): each tile's contraction range
// is cut into `parts`, the partial tiles go to `partial` (tiles * parts * 64 KB)
// and are added in a fixed order by a second kernel.
template <bool A_KMAJOR>
inline void launch_gemm_group_splitk(GemmGroup& g, int parts, float alpha, float beta, int kloFromM,
                                     int khiFromN, float* partial, hipStream_t s) {
  int t = 0;
  bool vec = true;
  for (int i = 0; i < g.count; ++i) {
    g.tile_start[i] = t;
    t += gemm_tiles(g.p[i].M, g.p[i].N);
    const GemmProblem& p = g.p[i];
    vec = vec && (p.lda % 4 == 0) && (p.ldb % 4 == 0) &&
          ((reinterpret_cast<uintptr_t>(p.A) | reinterpret_cast<uintptr_t>(p.B)) & 15) == 0;
  }
  g.tile_start[g.count] = t;
  g.ndesc = khiFromN ? 1 : 0;
  if (t == 0) return;
  double* pp = reinterpret_cast<double*>(partial);
  if (vec)
    gemm_f32_kernel<A_KMAJOR, kPartial, true><<<t * parts, 256, 0, s>>>(g, alpha, beta, kloFromM, khiFromN,
                                                                        0, pp, parts);
  else
    gemm_f32_kernel<A_KMAJOR, kPartial, false><<<t * parts, 256, 0, s>>>(g, alpha, beta, kloFromM, khiFromN,
                                                                         0, pp, parts);
  gemm_splitk_reduce<<<t * kRedSlices, 256, 0, s>>>(g, partial, parts, alpha, beta);
}

template <bool A_KMAJOR>
inline void gemm_f32(const float* A, int lda, const float* B, int ldb, float* C, int ldc, int M,
                     int N, int K, float alpha, float beta, int kloFromM, int khiFromN, int upperOnly,
                     hipStream_t s) {
  if (M <= 0 || N <= 0) return;
  // launches of few large tiles (counting only those upperOnly keeps) take 64x64
  // tiles; with a short contraction (the rank-128 updates) up to ~3.5 tiles per CU
  GemmGroup g;
  g.count = 1;
  g.p[0] = GemmProblem{A, B, C, nullptr, lda, ldb, ldc, M, N, K};
  if (!kloFromM && !khiFromN) {
    const int t128 = upperOnly ? gemm_upper_tiles(M, N) : gemm_tiles(M, N);
    if (t128 < (K <= 256 ? 448 : 192)) {
      launch_gemm_group_small<A_KMAJOR>(g, alpha, beta, 0, 0, upperOnly, s);
      return;
    }
  }
  launch_gemm_group<A_KMAJOR, kStore>(g, alpha, beta, kloFromM, khiFromN, upperOnly, nullptr, s);
}

}  // namespace gptq
