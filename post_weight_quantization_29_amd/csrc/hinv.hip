// Damping, desc_act column order and the triangular factor of the inverse
// Hessian (GPTQ practice page m.lqnn.cn/news/117696: section 2.2 "first"
// (fixed order by the Hessian diagonal), section 2.2 "third" (Cholesky factor
// of H^-1 instead of repeated inverse updates), section 3.3 (damp_percent,
// desc_act)).
//
// Target: U upper triangular with U^T U = Hd^-1, Hd = H[perm][:,perm] + lambda I.
// With J the order-reversing permutation and A = J Hd J = R^T R (R upper, the
// ordinary Cholesky factor of the flipped matrix), Hd^-1 = (J R^-1 J)(J R^-1 J)^T
// and J R^-1 J is lower triangular, so U = (J R^-1 J)^T, i.e.
// U[a][b] = R^-1[n-1-b][n-1-a].  This costs one Cholesky (n^3/3) and one
// triangular inverse (n^3/3); the flip rides on the permuting gather.
//
// Steps (all on stream s):
//   1. lambda = damp * mean(diag H)             (one workgroup, fp64 sum)
//   2. perm: identity or stable descending rank of diag(H)
//   3. A[a][b] = H[perm[n-1-a]][perm[n-1-b]] + lambda*[a==b], padded with I
//   4. blocked right-looking upper Cholesky, 128-row blocks:
//        block kernel: every workgroup factors A_kk; workgroup 0 forms
//                      R_kk^-1, the others the panel R_k,rest = R_kk^-T A_k,rest
//                      (in place); PD flag on a bad pivot
//        update GEMM:  A_rest -= R_k,rest^T R_k,rest    (upper tiles only)
//   5. triangular inverse by a binary tree over the 128-blocks: for a node
//      [a, mid) + [mid, b) with both halves already inverted,
//      X12 = -X11 * R12 * X22 (two grouped GEMMs per tree level)
//   6. U[a][b] = X[n-1-b][n-1-a] for b >= a, 0 below.
#include "gemm_f32.h"
#include "split3.h"

#include <vector>

namespace gptq {

constexpr int kNB = 128;   // factorization block

// ---------------------------------------------------------------- 1. lambda
// The diagonal comes from hdiag (fp64 sums kept by the Hessian call) when given,
// else from H itself.
GPTQ_DEV double diag_key(const float* H, const double* hdiag, int n, int i) {
  return hdiag ? hdiag[i] : (double)H[(size_t)i * n + i];
}

__global__ __launch_bounds__(1024) void damp_lambda_kernel(const float* __restrict__ H,
                                                           const double* __restrict__ hdiag, int n,
                                                           float damp, double* __restrict__ lam_out,
                                                           int* __restrict__ flag) {
  __shared__ double red[1024];
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += 1024) s += diag_key(H, hdiag, n, i);
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    lam_out[0] = (double)damp * (red[0] / (double)n);
    flag[0] = 0;
  }
}

// ---------------------------------------------------------------- 2. order
// rank[i] = #{j : key_j > key_i} + #{j < i : key_j == key_i}; perm[rank[i]] = i.
// NaN keys compare as smaller than every number (they sort last, by index).
GPTQ_DEV bool key_before(double kj, int j, double ki, int i) {
  const bool nj = kj != kj, ni = ki != ki;
  if (nj || ni) return (!nj && ni) || (nj && ni && j < i);
  return kj > ki || (kj == ki && j < i);
}

__global__ __launch_bounds__(256) void act_order_kernel(const float* __restrict__ H,
                                                        const double* __restrict__ hdiag, int n,
                                                        int desc, int* __restrict__ perm) {
  __shared__ double keys[256];
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (!desc) {
    if (i < n) perm[i] = i;
    return;
  }
  const double ki = (i < n) ? diag_key(H, hdiag, n, i) : 0.0;
  int rank = 0;
  for (int base = 0; base < n; base += 256) {
    const int j = base + threadIdx.x;
    __syncthreads();
    keys[threadIdx.x] = (j < n) ? diag_key(H, hdiag, n, j) : 0.0;
    __syncthreads();
    const int lim = min(256, n - base);
    for (int t = 0; t < lim; ++t) rank += key_before(keys[t], base + t, ki, i) ? 1 : 0;
  }
  if (i < n) perm[rank] = i;
}

// The same rank, with the chip filled: a workgroup takes 64 keys i (one per
// lane) and its 16 waves split the keys j into 16 contiguous slices; a wave
// reads 64 keys j at a time (one per lane) and hands them to every lane with
// v_readlane, so each comparison costs no memory access.  The 16 partial
// counts of key i are added in slice order.
constexpr int kRankSlices = 16;
__global__ __launch_bounds__(1024) void act_rank_kernel(const float* __restrict__ H,
                                                        const double* __restrict__ hdiag, int n,
                                                        int* __restrict__ perm) {
  __shared__ int part[kRankSlices][64];
  const int lane = threadIdx.x & 63;
  const int q = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int i = blockIdx.x * 64 + lane;
  const double ki = (i < n) ? diag_key(H, hdiag, n, i) : 0.0;
  const int j0 = (int)((int64_t)n * q / kRankSlices), j1 = (int)((int64_t)n * (q + 1) / kRankSlices);
  int rank = 0;
  for (int jb = j0; jb < j1; jb += 64) {
    const int jl = jb + lane;
    const double kl = (jl < j1) ? diag_key(H, hdiag, n, jl) : 0.0;
    const int lo = __double2loint(kl), hi = __double2hiint(kl);
    const int cnt = min(64, j1 - jb);
#pragma unroll
    for (int u = 0; u < 64; ++u) {
      if (u < cnt) {
        const double kj = __hiloint2double(__builtin_amdgcn_readlane(hi, u), __builtin_amdgcn_readlane(lo, u));
        rank += key_before(kj, jb + u, ki, i) ? 1 : 0;
      }
    }
  }
  part[q][lane] = rank;
  __syncthreads();
  if (q == 0 && i < n) {
    int r = 0;
#pragma unroll
    for (int t = 0; t < kRankSlices; ++t) r += part[t][lane];
    perm[r] = i;
  }
}

// ---------------------------------------------------------------- 3. gather
// Output row a reads source row perm[n-1-a] of H at the columns
// perm[n-1-b]: the row is first copied to LDS with coalesced loads and the
// column gather then reads LDS (a direct gather from memory touches a new
// cache line for almost every element).  Rows up to kGatherRow floats.
constexpr int kGatherRow = 32768;
__global__ __launch_bounds__(1024) void gather_flip_row_kernel(const float* __restrict__ H, int n, int np,
                                                              const int* __restrict__ perm,
                                                              const double* __restrict__ lam,
                                                              float* __restrict__ A, int vec) {
  __shared__ float row[kGatherRow];
  const int a = blockIdx.x;
  float* out = A + (size_t)a * np;
  if (a >= n) {                        // padding rows: identity
    for (int b = threadIdx.x; b < np; b += 1024) out[b] = (a == b) ? 1.0f : 0.0f;
    return;
  }
  const float* src = H + (size_t)perm[n - 1 - a] * n;
  const float l = (float)lam[0];
  if (vec) {
    // 16-byte loads and stores, every one of a thread's loads issued at once
    // (vec: n is a multiple of 4 and H and perm are 16-byte aligned, so every
    // row and every group of four perm entries is; np is a multiple of 128)
    constexpr int kU = kGatherRow / 4 / 1024;
    float4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int c = 4 * (threadIdx.x + 1024 * u);
      if (c < n) v[u] = *reinterpret_cast<const float4*>(src + c);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int c = 4 * (threadIdx.x + 1024 * u);
      if (c < n) *reinterpret_cast<float4*>(row + c) = v[u];
    }
    __syncthreads();
    for (int b = 4 * threadIdx.x; b < np; b += 4096) {
      float4 o;
      if (b < n) {
        // perm[n-1-b-3 .. n-1-b]: one aligned 16-byte load, in reverse order
        const int4 q = *reinterpret_cast<const int4*>(perm + (n - 4 - b));
        o = make_float4(row[q.w], row[q.z], row[q.y], row[q.x]);
        if (a >= b && a < b + 4) (&o.x)[a - b] += l;
      } else {
        o = make_float4(a == b ? 1.0f : 0.0f, a == b + 1 ? 1.0f : 0.0f, a == b + 2 ? 1.0f : 0.0f,
                        a == b + 3 ? 1.0f : 0.0f);
      }
      *reinterpret_cast<float4*>(out + b) = o;
    }
    return;
  }
  for (int c = threadIdx.x; c < n; c += 1024) row[c] = src[c];
  __syncthreads();
  for (int b = threadIdx.x; b < np; b += 1024) {
    float v;
    if (b < n) {
      v = row[perm[n - 1 - b]];
      if (a == b) v += l;
    } else {
      v = (a == b) ? 1.0f : 0.0f;
    }
    out[b] = v;
  }
}

__global__ __launch_bounds__(256) void gather_flip_kernel(const float* __restrict__ H, int n, int np,
                                                          const int* __restrict__ perm,
                                                          const double* __restrict__ lam,
                                                          float* __restrict__ A) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  const int a = blockIdx.y;
  if (b >= np) return;
  float v;
  if (a < n && b < n) {
    v = H[(size_t)perm[n - 1 - a] * n + perm[n - 1 - b]];
    if (a == b) v += (float)lam[0];
  } else {
    v = (a == b) ? 1.0f : 0.0f;
  }
  A[(size_t)a * np + b] = v;
}

// ---------------------------------------------------------------- 4. block step
// One launch per 128-block k: every workgroup factors the diagonal block
// A_kk = L L^T itself (L = R_kk^T) and then applies L^-1 to a 128-column
// tile T: workgroup 0 to the identity, which yields L^-1 = R_kk^-T (stored
// transposed, as R_kk^-1, in Dinv), workgroup t >= 1 to the tile A_k,(k+t),
// which yields the panel R_k,(k+t) = R_kk^-T A_k,(k+t) in place.  The
// factorization is repeated per workgroup (the workgroups would otherwise
// wait for one another), so the launch has no inter-workgroup dependency.
//
// Inside a workgroup (4 waves, all data in LDS):
//   for each 32-column sub-block b: one wave factors and inverts the 32x32
//   diagonal sub-block (two columns per step: the pivots through readlane,
//   the scaled columns through LDS); then the sub-blocks below are scaled,
//   M_ab <- M_ab L_bb^-T, and the trailing lower sub-blocks updated,
//   M_ac -= M_ab M_cb^T, with v_mfma_f32_32x32x2f32;
//   then each wave solves L X = T for 32 of the tile's columns, sub-block row
//   by sub-block row: X_a = L_aa^-1 (T_a - sum_{m<a} L_am X_m).
constexpr int kLP = kNB + 1;      // LDS pitch of the 128x128 tiles (odd: column walks hit distinct banks)
constexpr int kVP = 33;           // LDS pitch of the 32x32 sub-block inverses

// acc(m, n) += sum_{k < 32} A(m, k) B(k, n), A(m, k) = sa * pa[m*lda + k];
// B(k, n) = pb[n*ldb + k] (B_NMAJOR) or pb[k*ldb + n].  Lane l supplies
// A(l%32, 2s + l/32) and B(2s + l/32, l%32) to step s.
template <bool B_NMAJOR>
GPTQ_DEV void mm32(f32x16_t& acc, const float* pa, int lda, float sa, const float* pb, int ldb, int lane) {
  const int m = lane & 31, kh = lane >> 5;
#pragma unroll
  for (int st = 0; st < 16; ++st) {
    const int k = 2 * st + kh;
    const float av = sa * pa[m * lda + k];
    const float bv = B_NMAJOR ? pb[m * ldb + k] : pb[k * ldb + m];
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
  }
}
GPTQ_DEV void load32(f32x16_t& acc, const float* p, int ld, int lane) {
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = p[mfma32_row(r, lane) * ld + mfma32_col(lane)];
}
GPTQ_DEV void store32(const f32x16_t& acc, float* p, int ld, int lane) {
#pragma unroll
  for (int r = 0; r < 16; ++r) p[mfma32_row(r, lane) * ld + mfma32_col(lane)] = acc[r];
}

// Cholesky and inverse of the 32x32 sub-block at Mb (pitch kLP), split over
// two waves that run one step apart.  Two columns J, J+1 per step.
//
// Factor wave (leaf_factor): lane l holds row l%32 of the block, columns
// 16(l/32) .. +15 (v).  Per step its pivots come through readlane; the two
// finished L columns go to the step's slot of the LDS ring (ring[step][64],
// pivots in rs[step][4]), a flag releases the step to the inverse wave, and
// every lane reads the columns back for its rank-2 update.  Mb keeps L on and
// below the diagonal (the upper triangle is left undefined).
//
// Inverse wave (leaf_inverse): lane l holds column l%32 of the inverse, rows
// 16(l/32) .. +15 (y, starting from I).  Per step it waits for the factor
// wave's flag, takes the same row operations (so y ends as L^-1), and
// exchanges its two finished inverse rows between its halves through yx.  Vb
// (pitch kVP) receives L^-1 with zeros above.
//
// Every value takes the same operations in the same order as when one wave
// did both.  epoch makes each leaf's flags distinct (they are never cleared);
// bad is set on a pivot that is not > 0, and on a wait that does not end
// within its bound (which would mean the factor wave stopped).
constexpr int kLeafSteps = 16;

GPTQ_DEV float leaf_rsq(float p) {
  // 1/sqrt(p): hardware estimate refined by one Newton step
  const float dd = __builtin_amdgcn_rsqf(p);
  return dd * fmaf(-0.5f * p * dd, dd, 1.5f);
}

// Factor-wave step order.  A step's rank-2 update of the trailing columns is
// split: the two columns the next step pivots on (J+2, J+3, when they lie in
// the same half) are updated at once, with the four L values they need taken
// by readlane; the rest of the update reads its L columns from the ring and is
// applied at the start of the following step's update, after that step's
// pivots.  So the LDS round trip overlaps the next pivot chain.  Every column
// still takes its updates in step order, with the same operations.
constexpr bool leaf_ahead(int J2) {
  return (2 * J2 + 3 <= 31) && (((2 * J2 + 2) >> 4) == ((2 * J2) >> 4));
}
constexpr bool leaf_deferred(int J2) { return leaf_ahead(J2) && J2 + 1 < kLeafSteps; }

GPTQ_DEV void leaf_factor(float* Mb, float (*ring)[64], float (*rs)[4], int* flags, int epoch, int lane,
                          int& bad) {
  int i = lane & 31, h = lane >> 5;
  // opaque per call: keeps the compiler from hoisting the per-step lane masks
  // out of the caller's loop (they would spill)
  asm volatile("" : "+v"(i), "+v"(h));
  float v[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) v[r] = Mb[i * kLP + 16 * h + r];
  auto rl = [](float x, int ln) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), ln));
  };
  // v(i, c) -= li0 lc0[r] + li1 lc1[r] for the lane's columns c = 16h + r > cmin
  auto rank2 = [&]<int CMIN>(float li0, float li1, const float (&lc0)[16], const float (&lc1)[16]) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float nv = fmaf(-li1, lc1[r], fmaf(-li0, lc0[r], v[r]));
      if (r > CMIN) {
        v[r] = nv;                    // both halves: columns r and 16 + r exceed CMIN
      } else if (16 + r > CMIN) {
        v[r] = h ? nv : v[r];         // only the upper half's column 16 + r
      }
    }
  };
  // the previous step's deferred update: its L columns and the lane's L values
  float plc0[16], plc1[16], pli0 = 0.0f, pli1 = 0.0f;
  auto step = [&]<int J2>() {
    constexpr int J = 2 * J2, hj = J >> 4, r0 = J & 15, r1 = r0 + 1;
    const float p0 = rl(v[r0], hj * 32 + J);          // A[J][J]
    const float a10 = rl(v[r0], hj * 32 + J + 1);     // A[J+1][J]
    const float p1r = rl(v[r1], hj * 32 + J + 1);     // A[J+1][J+1]
    const float d0 = leaf_rsq(p0);
    const float l10 = a10 * d0;
    const float p1 = fmaf(-l10, l10, p1r);
    const float d1 = leaf_rsq(p1);
    if (!(p0 > 0.0f) || !(p1 > 0.0f)) bad = 1;
    float* cb = ring[J2];
    const float c0 = (i == J) ? p0 * d0 : v[r0] * d0;                       // L[i][J]
    const float c1 = (i == J + 1) ? p1 * d1 : fmaf(-c0, l10, v[r1]) * d1;   // L[i][J+1]
    if (h == hj) {
      if (i >= J) v[r0] = c0;
      if (i >= J + 1) v[r1] = c1;
      cb[i] = c0;
      cb[32 + i] = c1;
    }
    if (lane == 0) {
      rs[J2][0] = d0;
      rs[J2][1] = l10;
      rs[J2][2] = d1;
    }
    // the step's slot is written: release it to the inverse wave
    if (lane == 0) __hip_atomic_store(&flags[J2], epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    asm volatile("" ::: "memory");
    // the previous step's update of the columns beyond this step's two
    if constexpr (J2 > 0 && leaf_deferred(J2 - 1)) rank2.template operator()<J + 1>(pli0, pli1, plc0, plc1);
    if constexpr (leaf_ahead(J2)) {
      // this step's update of the next step's two columns (lanes of half hj
      // hold them; their own c0, c1 are L[i][J], L[i][J+1])
      constexpr int rn0 = (J + 2) & 15, rn1 = rn0 + 1;
      const float l20 = rl(c0, hj * 32 + J + 2), l21 = rl(c1, hj * 32 + J + 2);
      const float l30 = rl(c0, hj * 32 + J + 3), l31 = rl(c1, hj * 32 + J + 3);
      const float n0 = fmaf(-c1, l21, fmaf(-c0, l20, v[rn0]));
      const float n1 = fmaf(-c1, l31, fmaf(-c0, l30, v[rn1]));
      v[rn0] = (h == hj) ? n0 : v[rn0];
      v[rn1] = (h == hj) ? n1 : v[rn1];
    }
    const float li0 = cb[i], li1 = cb[32 + i];
    float lc0[16], lc1[16];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const float4 q0 = reinterpret_cast<const float4*>(cb + 16 * h)[r4];
      const float4 q1 = reinterpret_cast<const float4*>(cb + 32 + 16 * h)[r4];
      lc0[4 * r4 + 0] = q0.x; lc0[4 * r4 + 1] = q0.y; lc0[4 * r4 + 2] = q0.z; lc0[4 * r4 + 3] = q0.w;
      lc1[4 * r4 + 0] = q1.x; lc1[4 * r4 + 1] = q1.y; lc1[4 * r4 + 2] = q1.z; lc1[4 * r4 + 3] = q1.w;
    }
    if constexpr (leaf_deferred(J2)) {
      // applied after the next step's pivots (columns J+2, J+3 are done)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        plc0[r] = lc0[r];
        plc1[r] = lc1[r];
      }
      pli0 = li0;
      pli1 = li1;
    } else {
      rank2.template operator()<J + 1>(li0, li1, lc0, lc1);
    }
    asm volatile("" ::: "memory");
  };
  [&]<int... Js>(std::integer_sequence<int, Js...>) {
    (step.template operator()<Js>(), ...);
  }(std::make_integer_sequence<int, kLeafSteps>{});
#pragma unroll
  for (int r = 0; r < 16; ++r) Mb[i * kLP + 16 * h + r] = v[r];
}

GPTQ_DEV void leaf_inverse(float* Vb, float (*ring)[64], float (*rs)[4], const int* flags, float* yx,
                           int epoch, int lane, int& bad) {
  int i = lane & 31, h = lane >> 5;
  asm volatile("" : "+v"(i), "+v"(h));
  float y[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) y[r] = (16 * h + r == i) ? 1.0f : 0.0f;
  auto step = [&]<int J2>() {
    constexpr int J = 2 * J2, hj = J >> 4, r0 = J & 15, r1 = r0 + 1;
    // the factor wave never waits for this one, so the flag comes; the bound
    // only turns a broken invariant into an error instead of a hang
    int spins = 0;
    while (__hip_atomic_load(&flags[J2], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != epoch) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > (1 << 22)) {
        bad = 1;
        break;
      }
    }
    const float* cb = ring[J2];
    const float d0 = rs[J2][0], l10 = rs[J2][1], d1 = rs[J2][2];
    if (h == hj) {
      // inverse rows J, J+1 of this lane's column i
      const float yj = y[r0] * d0;
      const float yj1 = fmaf(-l10, yj, y[r1]) * d1;
      y[r0] = yj;
      y[r1] = yj1;
      yx[i] = yj;
      yx[32 + i] = yj1;
    }
    asm volatile("" ::: "memory");
    const float yJ = yx[i], yJ1 = yx[32 + i];
    float lc0[16], lc1[16];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const float4 q0 = reinterpret_cast<const float4*>(cb + 16 * h)[r4];
      const float4 q1 = reinterpret_cast<const float4*>(cb + 32 + 16 * h)[r4];
      lc0[4 * r4 + 0] = q0.x; lc0[4 * r4 + 1] = q0.y; lc0[4 * r4 + 2] = q0.z; lc0[4 * r4 + 3] = q0.w;
      lc1[4 * r4 + 0] = q1.x; lc1[4 * r4 + 1] = q1.y; lc1[4 * r4 + 2] = q1.z; lc1[4 * r4 + 3] = q1.w;
    }
    // rows 16h + r > J + 1 take the same rank-2 operation:
    // y(row, i) -= L[row][J] Y[J][i] + L[row][J+1] Y[J+1][i]
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float ny = fmaf(-lc1[r], yJ1, fmaf(-lc0[r], yJ, y[r]));
      if (J + 1 < 16) {
        if (r > J + 1) y[r] = ny;
        else y[r] = h ? ny : y[r];
      } else if (r > J + 1 - 16) {
        y[r] = h ? ny : y[r];
      }
    }
    asm volatile("" ::: "memory");
  };
  [&]<int... Js>(std::integer_sequence<int, Js...>) {
    (step.template operator()<Js>(), ...);
  }(std::make_integer_sequence<int, kLeafSteps>{});
#pragma unroll
  for (int r = 0; r < 16; ++r) Vb[(16 * h + r) * kVP + i] = y[r];
}

// The part of an update that rides with the factor of row block k: factor
// rows [k0, k0 + K) (already factored R row blocks) times themselves over the
// columns after row block k, subtracted from rows [(k + 1)*128, + rows) and
// every column after row block k (upper tiles only).
struct TrailArgs {
  int k0;     // first factor row of the contraction
  int K;      // contraction length (128 per factored block)
  int rows;   // rows of A updated, from row (k + 1) * 128
};

// Trailing workgroups of the factor launch for block k: workgroup `local` of
// the update owed by the rows after row block k (set up by the previous
// factor; the upper 128 x 128 tiles of A[(k+1)*128 : (k+1)*128 + t.rows,
// (k+1)*128 :], row by row), with the same tile contraction as a separate
// trailing-update launch.  They run on the CUs the factor leaves idle and
// stage their operands in its LDS arrays.
GPTQ_DEV void trail_tile(float* A, int np, int k, const TrailArgs& t, int local, float* sA, float* sB) {
  const int c0 = (k + 1) * kNB, rest = np - c0;
  const float* Arow = A + (size_t)t.k0 * np + c0;
  const GemmProblem P{Arow, Arow, A + (size_t)c0 * np + c0, nullptr, np, np, np, t.rows, rest, t.K};
  const int tn = rest / kGT;
  int r = 0, rem = local;
  while (rem >= tn - r) { rem -= tn - r; ++r; }
  const int m0 = r * kGT, n0 = (r + rem) * kGT;
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
  gemm_tile_contract<true, true>(P, m0, n0, 0, t.K, sA, sB, acc);
  gemm_tile_update(P, m0, n0, -1.0f, 1.0f, acc);
}

__global__ __launch_bounds__(256) void chol_panel_kernel(float* __restrict__ A, int np, int k,
                                                         float* __restrict__ Dinv, int* __restrict__ flag,
                                                         int ntrail, TrailArgs trail) {
  __shared__ __attribute__((aligned(16))) float M[kNB * kLP];
  __shared__ __attribute__((aligned(16))) float T[kNB * kLP];
  __shared__ __attribute__((aligned(16))) float V[4][32 * kVP];
  __shared__ __attribute__((aligned(16))) float ring[kLeafSteps][64];
  __shared__ __attribute__((aligned(16))) float rs[kLeafSteps][4];
  __shared__ __attribute__((aligned(16))) float yx[64];
  __shared__ int flags[kLeafSteps];

  if ((int)blockIdx.x >= (int)gridDim.x - ntrail) {
    trail_tile(A, np, k, trail, (int)blockIdx.x - ((int)gridDim.x - ntrail), M, T);
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile = blockIdx.x;                     // 0: identity, t >= 1: column block k + t
  const float* Akk = A + (size_t)k * kNB * np + (size_t)k * kNB;
  float* At = A + (size_t)k * kNB * np + (size_t)(k + tile) * kNB;

  // load the diagonal block and the tile (16 float4 per thread each)
  {
    float4 va[16], vt[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = u * 256 + tid, r = e >> 5, c4 = 4 * (e & 31);
      va[u] = *reinterpret_cast<const float4*>(Akk + (size_t)r * np + c4);
      if (tile > 0) vt[u] = *reinterpret_cast<const float4*>(At + (size_t)r * np + c4);
      else vt[u] = make_float4(r == c4 ? 1.f : 0.f, r == c4 + 1 ? 1.f : 0.f, r == c4 + 2 ? 1.f : 0.f,
                               r == c4 + 3 ? 1.f : 0.f);
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = u * 256 + tid, r = e >> 5, c4 = 4 * (e & 31);
      float* pm = M + r * kLP + c4;
      pm[0] = va[u].x; pm[1] = va[u].y; pm[2] = va[u].z; pm[3] = va[u].w;
      float* pt = T + r * kLP + c4;
      pt[0] = vt[u].x; pt[1] = vt[u].y; pt[2] = vt[u].z; pt[3] = vt[u].w;
    }
  }
  if (tid < kLeafSteps) flags[tid] = 0;     // leaf epochs start at 1
  __syncthreads();

  int bad = 0;
#pragma unroll 1
  for (int b = 0; b < 4; ++b) {
    const int o = 32 * b;
    if (wave == 0) leaf_factor(M + o * kLP + o, ring, rs, flags, b + 1, lane, bad);
    else if (wave == 1) leaf_inverse(V[b], ring, rs, flags, yx, b + 1, lane, bad);
    __syncthreads();
    // sub-blocks below: M_ab <- M_ab L_bb^-T   (wave w: a = b + 1 + w)
    if (wave < 3 - b) {
      const int a = b + 1 + wave;
      f32x16_t acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
      mm32<true>(acc, M + (32 * a) * kLP + o, kLP, 1.0f, V[b], kVP, lane);
      asm volatile("" ::: "memory");
      store32(acc, M + (32 * a) * kLP + o, kLP, lane);
    }
    __syncthreads();
    // trailing lower sub-blocks: M_ac -= M_ab M_cb^T, a >= c > b
    {
      int q = 0;
      for (int a = b + 1; a < 4; ++a) {
        for (int c = b + 1; c <= a; ++c, ++q) {
          if ((q & 3) != wave) continue;
          f32x16_t acc;
          load32(acc, M + (32 * a) * kLP + 32 * c, kLP, lane);
          mm32<true>(acc, M + (32 * a) * kLP + o, kLP, -1.0f, M + (32 * c) * kLP + o, kLP, lane);
          store32(acc, M + (32 * a) * kLP + 32 * c, kLP, lane);
        }
      }
    }
    __syncthreads();
  }
  if (bad) flag[0] = 1;

  // forward substitution on this wave's 32 columns of T
  {
    float* Tw = T + 32 * wave;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      f32x16_t acc;
      load32(acc, Tw + (32 * a) * kLP, kLP, lane);
#pragma unroll
      for (int m = 0; m < a; ++m)
        mm32<false>(acc, M + (32 * a) * kLP + 32 * m, kLP, -1.0f, Tw + (32 * m) * kLP, kLP, lane);
      store32(acc, Tw + (32 * a) * kLP, kLP, lane);
      asm volatile("" ::: "memory");
      f32x16_t x;
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = 0.0f;
      mm32<false>(x, V[a], kVP, 1.0f, Tw + (32 * a) * kLP, kLP, lane);
      asm volatile("" ::: "memory");
      store32(x, Tw + (32 * a) * kLP, kLP, lane);
      asm volatile("" ::: "memory");
    }
  }
  __syncthreads();

  if (tile == 0) {
    // R_kk^-1 = (L^-1)^T: Dinv[r][c] = T[c][r] for c >= r, 0 below the diagonal
    float* D = Dinv + (size_t)k * kNB * kNB;
    for (int e = tid; e < kNB * kNB; e += 256) {
      const int r = e >> 7, c = e & 127;
      D[e] = (c >= r) ? T[c * kLP + r] : 0.0f;
    }
  } else {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = u * 256 + tid, r = e >> 5, c4 = 4 * (e & 31);
      const float* pt = T + r * kLP + c4;
      *reinterpret_cast<float4*>(At + (size_t)r * np + c4) = make_float4(pt[0], pt[1], pt[2], pt[3]);
    }
  }
}

// diagonal blocks of R^-1 into A, where the triangular inverse starts from them
__global__ __launch_bounds__(256) void dinv_scatter_kernel(const float* __restrict__ Dinv, float* __restrict__ A,
                                                           int np) {
  const int k = blockIdx.x;
  const float* D = Dinv + (size_t)k * kNB * kNB;
  float* blk = A + (size_t)k * kNB * np + (size_t)k * kNB;
  for (int e = threadIdx.x; e < kNB * kNB / 4; e += 256) {
    const int r = e >> 5, c4 = 4 * (e & 31);
    *reinterpret_cast<float4*>(blk + (size_t)r * np + c4) = *reinterpret_cast<const float4*>(D + (size_t)r * kNB + c4);
  }
}

// ---------------------------------------------------------------- 6. anti-transpose
__global__ __launch_bounds__(256) void flip_out_kernel(const float* __restrict__ X, int np, int n,
                                                       float* __restrict__ U) {
  // U[a][b] = X[n-1-b][n-1-a] for b >= a, 0 below the diagonal; 64 x 64 tiles
  // of U, staged through LDS.  Tiles wholly inside U with n a multiple of 4 move
  // 16 bytes per access (the source columns of four consecutive a are four
  // consecutive, reversed floats); edge tiles go element by element.
  __shared__ float tile[64][65];
  const int a0 = blockIdx.y * 64, b0 = blockIdx.x * 64;
  const int tid = threadIdx.x;
  const bool full = (a0 + 64 <= n) && (b0 + 64 <= n) && (n % 4 == 0);
  if (full && b0 + 63 < a0) {
    // wholly below the diagonal
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = k * 256 + tid, ya = e >> 4, x4 = 4 * (e & 15);
      *reinterpret_cast<float4*>(U + (size_t)(a0 + ya) * n + b0 + x4) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    return;
  }
  if (full) {
    // tile[yb][xa] = X[n-1-(b0+yb)][n-1-(a0+xa)]: a float4 at source column
    // n-1-(a0+x4+3) holds xa = x4+3, x4+2, x4+1, x4
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = k * 256 + tid, yb = e >> 4, x4 = 4 * (e & 15);
      const int b = b0 + yb;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (b >= a0 + x4)   // some a of the four has b >= a
        v = *reinterpret_cast<const float4*>(X + (size_t)(n - 1 - b) * np + (n - 4 - a0 - x4));
      tile[yb][x4 + 3] = (b >= a0 + x4 + 3) ? v.x : 0.0f;
      tile[yb][x4 + 2] = (b >= a0 + x4 + 2) ? v.y : 0.0f;
      tile[yb][x4 + 1] = (b >= a0 + x4 + 1) ? v.z : 0.0f;
      tile[yb][x4 + 0] = v.w;   // b >= a0 + x4 here, or v is zero
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = k * 256 + tid, ya = e >> 4, x4 = 4 * (e & 15);
      *reinterpret_cast<float4*>(U + (size_t)(a0 + ya) * n + b0 + x4) =
          make_float4(tile[x4][ya], tile[x4 + 1][ya], tile[x4 + 2][ya], tile[x4 + 3][ya]);
    }
    return;
  }
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;   // 64 x 4
  for (int yy = ty; yy < 64; yy += 4) {
    const int b = b0 + yy, a = a0 + tx;
    float v = 0.0f;
    if (a < n && b < n && b >= a) v = X[(size_t)(n - 1 - b) * np + (n - 1 - a)];
    tile[yy][tx] = v;
  }
  __syncthreads();
  for (int yy = ty; yy < 64; yy += 4) {
    const int a = a0 + yy, b = b0 + tx;
    if (a < n && b < n) U[(size_t)a * n + b] = tile[tx][yy];
  }
}

// ---------------------------------------------------------------- planning
struct HinvLayout {
  int n, np, nblk, ldz;
  size_t off_A, off_Z, off_sk, off_planes, off_lam, off_flag, total;
};

struct TreeNode { int a, mid, b; };

// tree launches of fewer 128x128 tiles than this run in 64x64 tiles
constexpr int kTreeSmallTiles = 128;

static void build_levels(int lo, int hi, int depth, std::vector<std::vector<TreeNode>>& lv) {
  if (hi - lo <= 1) return;
  const int mid = lo + (hi - lo) / 2;
  if ((int)lv.size() <= depth) lv.resize(depth + 1);
  lv[depth].push_back(TreeNode{lo, mid, hi});
  build_levels(lo, mid, depth + 1, lv);
  build_levels(mid, hi, depth + 1, lv);
}

// tiles and longest contraction of one launch of tree nodes [c0, c0 + cnt)
static void tree_launch_shape(const std::vector<TreeNode>& nodes, size_t c0, int cnt, int& tiles, int& kmax) {
  tiles = 0;
  kmax = 0;
  for (int i = 0; i < cnt; ++i) {
    const TreeNode& t = nodes[c0 + i];
    const int M = (t.mid - t.a) * kNB, N = (t.b - t.mid) * kNB;
    tiles += gemm_tiles(M, N);
    kmax = std::max(kmax, std::max(M, N));
  }
}

// Blocks per super-block of the factor's trailing updates: 8 once the padded
// matrix exceeds the 256 MB last-level cache (the rank-128 updates are then
// bound by its read-modify-write from HBM), else 1.
static int hinv_super_blocks(int np) {
  return ((size_t)np * np * sizeof(float) > (size_t(256) << 20)) ? 8 : 1;
}

// a tree node [a, mid) + [mid, b) takes its two products in the split fp16
// form when both have enough tiles (Z = X11 R12 and X12 = -Z X22 are M x N)
static bool tree_split3(int M, int N) { return split3_gemm_shape_ok(M, M, N) && split3_gemm_shape_ok(N, M, N); }

static HinvLayout hinv_layout(int n) {
  HinvLayout L;
  L.n = n;
  L.nblk = (n + kNB - 1) / kNB;
  L.np = L.nblk * kNB;
  L.ldz = ((L.nblk + 1) / 2) * kNB;
  size_t off = 0;
  L.off_A = off;
  off = align_up(off + (size_t)L.np * L.np * sizeof(float));
  L.off_Z = off;
  off = align_up(off + (size_t)L.np * L.ldz * sizeof(float));
  // split-K partial tiles of the tree levels that have few tiles
  size_t sk = 0;
  {
    std::vector<std::vector<TreeNode>> levels;
    build_levels(0, L.nblk, 0, levels);
    for (const auto& nodes : levels)
      for (size_t c0 = 0; c0 < nodes.size(); c0 += kGemmMaxGroup) {
        const int cnt = (int)std::min<size_t>(kGemmMaxGroup, nodes.size() - c0);
        int tiles, kmax;
        tree_launch_shape(nodes, c0, cnt, tiles, kmax);
        const int parts = splitk_parts(tiles, kmax);
        if (parts > 1) sk = std::max(sk, (size_t)tiles * parts * kGT * kGT * sizeof(float));
      }
  }
  L.off_sk = off;
  off = align_up(off + sk);
  // fp16 pieces of a super-block's rows for the split trailing updates,
  // and of the operands of the tree nodes whose products take the split form
  // (the factor and the tree run one after the other: one region serves both)
  const int gb = hinv_super_blocks(L.np);
  size_t planes = (gb > 1) ? split3_planes_bytes(gb * kNB, L.np - gb * kNB) : 0;
  {
    std::vector<std::vector<TreeNode>> levels;
    build_levels(0, L.nblk, 0, levels);
    for (const auto& nodes : levels)
      for (const TreeNode& t : nodes) {
        const int M = (t.mid - t.a) * kNB, N = (t.b - t.mid) * kNB;
        if (tree_split3(M, N)) planes = std::max(planes, split3_gemm_planes_bytes(std::max(M, N), M, N));
      }
  }
  L.off_planes = off;
  off = align_up(off + planes);
  L.off_lam = off;
  off = align_up(off + sizeof(double));
  L.off_flag = off;
  off = align_up(off + sizeof(int));
  L.total = off;
  return L;
}

}  // namespace gptq

using namespace gptq;

extern "C" size_t gptq_prepare_hinv_workspace_size(int32_t d_in) {
  if (d_in <= 0) return 0;
  return hinv_layout(d_in).total;
}

extern "C" int gptq_prepare_hinv(const float* H, const double* hdiag, int32_t d_in, float damp_percent,
                                 int32_t desc_act, float* U, int32_t* perm, void* ws, size_t ws_bytes,
                                 hipStream_t s) {
  if (!H || !U || !perm || d_in <= 0 || d_in > 65536) return GPTQ_ERR_INVALID_ARG;
  if (!(damp_percent >= 0.0f) || !(damp_percent < 1e30f)) return GPTQ_ERR_INVALID_ARG;
  if (desc_act != 0 && desc_act != 1) return GPTQ_ERR_INVALID_ARG;
  const HinvLayout L = hinv_layout(d_in);
  if (!ws || ws_bytes < L.total) return GPTQ_ERR_WORKSPACE;
  char* base = static_cast<char*>(ws);
  float* A = reinterpret_cast<float*>(base + L.off_A);
  float* Z = reinterpret_cast<float*>(base + L.off_Z);
  float* SK = reinterpret_cast<float*>(base + L.off_sk);
  void* planes = base + L.off_planes;
  double* lam = reinterpret_cast<double*>(base + L.off_lam);
  int* flag = reinterpret_cast<int*>(base + L.off_flag);
  const int n = L.n, np = L.np, nb = L.nblk;

  damp_lambda_kernel<<<1, 1024, 0, s>>>(H, hdiag, n, damp_percent, lam, flag);
  GPTQ_LAUNCH_CHECK();
  if (desc_act)
    act_rank_kernel<<<(n + 63) / 64, 1024, 0, s>>>(H, hdiag, n, perm);
  else
    act_order_kernel<<<(n + 255) / 256, 256, 0, s>>>(H, hdiag, n, desc_act, perm);
  GPTQ_LAUNCH_CHECK();
  if (n <= kGatherRow)
    gather_flip_row_kernel<<<np, 1024, 0, s>>>(H, n, np, perm, lam, A,
                                               (n % 4 == 0) && (reinterpret_cast<uintptr_t>(H) % 16 == 0) &&
                                                   (reinterpret_cast<uintptr_t>(perm) % 16 == 0));
  else
    gather_flip_kernel<<<dim3((np + 255) / 256, np), 256, 0, s>>>(H, n, np, perm, lam, A);
  GPTQ_LAUNCH_CHECK();

  // 4. Cholesky A = R^T R: per block, diagonal factor + panel in one launch,
  //    then the trailing update, split so that only its first row block sits
  //    between two factors (lookahead); R_kk^-1 goes to Dinv (in Z's space,
  //    which the triangular inverse only uses later) and then onto A's
  //    diagonal blocks.  Blocks form super-blocks of gb: inside a super-block
  //    a factored row block updates only the rows of the super-block's later
  //    blocks; at its end the whole super-block's rows update every later row
  //    in one product of K = 128 gb (the same sums regrouped; the trailing
  //    matrix is read and written gb times less often).
  const int gb = hinv_super_blocks(np);
  float* Dinv = Z;
  bool ride = false;   // the previous update's rows after row block k ride with factor k
  TrailArgs trail{0, 0, 0};
  for (int k = 0; k < nb; ++k) {
    const int rest = np - (k + 1) * kNB;
    // the previous update's rows after row block k ride along with block k's
    // factor (other CUs; they touch neither row block k nor Dinv) ...
    const int ntr = (ride && rest > 0 && trail.rows > 0) ? gemm_upper_tiles(trail.rows, rest) : 0;
    chol_panel_kernel<<<1 + rest / kNB + ntr, 256, 0, s>>>(A, np, k, Dinv, flag, ntr, trail);
    GPTQ_LAUNCH_CHECK();
    if (rest <= 0) continue;
    // the update this factor owes: factor rows [k0, (k+1)*128) subtracted
    // from rows [(k+1)*128, row_end) and every column after row block k
    const bool s_end = (k + 1) % gb == 0;
    const int k0 = (s_end ? (k / gb) * gb : k) * kNB;
    const int Kk = (k + 1) * kNB - k0;
    const int row_end = s_end ? np : std::min(np, (k / gb + 1) * gb * kNB);
    const int urows = row_end - (k + 1) * kNB;
    float* Arow = A + (size_t)k0 * np + (size_t)(k + 1) * kNB;
    float* Atrail = A + (size_t)(k + 1) * kNB * np + (size_t)(k + 1) * kNB;
    // ... and the update of row block k + 1 alone runs before block k+1's
    // factor.  Every element gets the same tile contraction as one upper-tile
    // update of those rows would give.  Riding tiles run one workgroup per CU
    // (the factor's LDS); when they would need more than two rounds of the CUs
    // the next factor leaves free, the whole update runs on its own instead
    // (two workgroups per CU).
    const int ride_rows = urows - kNB;
    const int next_tiles = ride_rows > 0 ? gemm_upper_tiles(ride_rows, rest - kNB) : 0;
    const int free_cus = 256 - (1 + (rest - kNB) / kNB);
    ride = next_tiles <= 2 * free_cus;
    trail = TrailArgs{k0, Kk, ride ? std::max(0, ride_rows) : 0};
    if (gb > 1 && s_end && !ride && split3_pays(rest)) {
      // a super-block's whole update on fp16 MFMA through the split pieces
      const int st = split3_update(Arow, np, Kk, rest, Atrail, np, planes, s);
      if (st != GPTQ_OK) return st;
      continue;
    }
    gemm_f32<true>(Arow, np, Arow, np, Atrail, np, ride ? kNB : urows, rest, Kk, -1.0f, 1.0f, 0, 0,
                   ride ? 0 : 1, s);
    GPTQ_LAUNCH_CHECK();
  }
  dinv_scatter_kernel<<<nb, 256, 0, s>>>(Dinv, A, np);
  GPTQ_LAUNCH_CHECK();

  // 5. triangular inverse, deepest tree level first
  std::vector<std::vector<TreeNode>> levels;
  build_levels(0, nb, 0, levels);
  for (int lv = (int)levels.size() - 1; lv >= 0; --lv) {
    // nodes large enough run their two products in the split fp16 form, one
    // node at a time: Z = X11 R12 (X11 upper triangular: tile row I contracts
    // from 256 I), then X12 = -Z X22 (X22 upper triangular: tile column J
    // contracts up to 256 (J + 1)); the entries below the two diagonals are
    // read as zero.  The rest go to the grouped fp32 launches.
    std::vector<TreeNode> nodes;
    for (const TreeNode& t : levels[lv]) {
      const int r0 = t.a * kNB, r1 = t.mid * kNB, r2 = t.b * kNB;
      const int M = r1 - r0, N = r2 - r1;
      float* Zn = Z + (size_t)r0 * L.ldz;
      const float* X11 = A + (size_t)r0 * np + r0;
      const float* R12 = A + (size_t)r0 * np + r1;
      const float* X22 = A + (size_t)r1 * np + r1;
      if (!tree_split3(M, N) || !split3_gemm_applies(X11, np, true, R12, np, M, M, N) ||
          !split3_gemm_applies(Zn, L.ldz, true, X22, np, N, M, N)) {
        nodes.push_back(t);
        continue;
      }
      int st = split3_gemm(X11, np, true, R12, np, M, M, N, Zn, L.ldz, false, false, 1, planes, s);
      if (st != GPTQ_OK) return st;
      st = split3_gemm(Zn, L.ldz, true, X22, np, N, M, N, A + (size_t)r0 * np + r1, np, true, false, 2, planes, s);
      if (st != GPTQ_OK) return st;
    }
    for (size_t c0 = 0; c0 < nodes.size(); c0 += kGemmMaxGroup) {
      const int cnt = (int)std::min<size_t>(kGemmMaxGroup, nodes.size() - c0);
      GemmGroup g1, g2;
      g1.count = g2.count = cnt;
      for (int i = 0; i < cnt; ++i) {
        const TreeNode& t = nodes[c0 + i];
        const int r0 = t.a * kNB, r1 = t.mid * kNB, r2 = t.b * kNB;
        const int M = r1 - r0, N = r2 - r1;
        float* Zn = Z + (size_t)r0 * L.ldz;
        // Z = X11 * R12, X11 upper triangular (contraction from k = m0)
        g1.p[i] = GemmProblem{A + (size_t)r0 * np + r0, A + (size_t)r0 * np + r1, Zn, nullptr,
                              np, np, L.ldz, M, N, M};
        // X12 = -Z * X22, X22 upper triangular (contraction up to k = n0 + 128)
        g2.p[i] = GemmProblem{Zn, A + (size_t)r1 * np + r1, A + (size_t)r0 * np + r1, nullptr,
                              L.ldz, np, np, M, N, N};
      }
      int tiles, kmax;
      tree_launch_shape(nodes, c0, cnt, tiles, kmax);
      const int parts = splitk_parts(tiles, kmax);
      if (tiles < kTreeSmallTiles) {
        // the deep levels: 64x64 tiles, four workgroups per 128-tile, no split
        launch_gemm_group_small<false>(g1, 1.0f, 0.0f, 1, 0, 0, s);
        GPTQ_LAUNCH_CHECK();
        launch_gemm_group_small<false>(g2, -1.0f, 0.0f, 0, 1, 0, s);
        GPTQ_LAUNCH_CHECK();
      } else if (parts > 1) {
        // few tiles with long contractions: split them (partials in SK)
        launch_gemm_group_splitk<false>(g1, parts, 1.0f, 0.0f, 1, 0, SK, s);
        GPTQ_LAUNCH_CHECK();
        launch_gemm_group_splitk<false>(g2, parts, -1.0f, 0.0f, 0, 1, SK, s);
        GPTQ_LAUNCH_CHECK();
      } else {
        launch_gemm_group<false, kStore>(g1, 1.0f, 0.0f, 1, 0, 0, nullptr, s);
        GPTQ_LAUNCH_CHECK();
        launch_gemm_group<false, kStore>(g2, -1.0f, 0.0f, 0, 1, 0, nullptr, s);
        GPTQ_LAUNCH_CHECK();
      }
    }
  }

  // 6. U
  flip_out_kernel<<<dim3((n + 63) / 64, (n + 63) / 64), 256, 0, s>>>(A, np, n, U);
  GPTQ_LAUNCH_CHECK();

  int hflag = 0;
  GPTQ_HIP_TRY(hipMemcpyAsync(&hflag, flag, sizeof(int), hipMemcpyDeviceToHost, s));
  GPTQ_HIP_TRY(hipStreamSynchronize(s));
  return hflag ? GPTQ_ERR_NOT_PD : GPTQ_OK;
}
