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
//        diag kernel: R_kk and R_kk^-1 from the block (one workgroup, LDS),
//                     R_kk^-1 stored in place, PD flag on a bad pivot
//        panel GEMM:  R_k,rest = R_kk^-T A_k,rest      (in place)
//        update GEMM: A_rest -= R_k,rest^T R_k,rest    (upper tiles only)
//   5. triangular inverse by a binary tree over the 128-blocks: for a node
//      [a, mid) + [mid, b) with both halves already inverted,
//      X12 = -X11 * R12 * X22 (two grouped GEMMs per tree level)
//   6. U[a][b] = X[n-1-b][n-1-a] for b >= a, 0 below.
#include "gemm_f32.h"

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

// ---------------------------------------------------------------- 3. gather
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

// ---------------------------------------------------------------- 4a. diagonal block
// In-place elimination on the augmented block [A_kk | I]: at step j the pivot
// row is scaled by 1/sqrt(pivot) and subtracted from the rows below, on both
// halves.  Column j of the left half is retired at that step, so it stores the
// new column j of the right half.  The finished block holds R^-T (lower incl.
// diagonal) and R (strict upper).  Thread t owns column t%128 and rows
// 16*(t/128) .. +15 in registers (a wave's rows are uniform); pivot rows go
// through LDS.  The step loop is unrolled by 16 so that register indices and
// the "row below the pivot" tests are compile-time.
__global__ __launch_bounds__(1024) void chol_diag_kernel(float* __restrict__ A, int np, int k,
                                                         int* __restrict__ flag) {
  __shared__ __attribute__((aligned(16))) float rowbuf[2][kNB];
  const int t = threadIdx.x;
  const int x = t & (kNB - 1), g = t >> 7;
  float* blk = A + (size_t)k * kNB * np + (size_t)k * kNB;
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = blk[(size_t)(16 * g + i) * np + x];

#pragma unroll 1
  for (int jb = 0; jb < kNB / 16; ++jb) {
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const int j = 16 * jb + jj;
      float* rb = rowbuf[jj & 1];
      if (g == jb) rb[x] = v[jj];
      __syncthreads();
      if (g < jb) continue;                 // rows already final
      const float p = rb[j];
      if (g == jb && x == j && !(p > 0.0f)) flag[0] = 1;   // an active lane reports the pivot
      // 1/sqrt(p): hardware estimate refined by one Newton step
      float sc = __builtin_amdgcn_rsqf(p);
      sc = sc * fmaf(-0.5f * p * sc, sc, 1.5f);
      const bool isj = (x == j);
      const float rjx = isj ? sc : rb[x] * sc;
      const float keep = isj ? 0.0f : 1.0f;
      const float cmul = sc * rjx;          // row i: v -= rb[i] * sc * rjx
      const float4* r4 = reinterpret_cast<const float4*>(rb + 16 * g);
      float m[16];
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const float4 u = r4[i4];
        m[4 * i4 + 0] = u.x; m[4 * i4 + 1] = u.y; m[4 * i4 + 2] = u.z; m[4 * i4 + 3] = u.w;
      }
      if (g > jb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = fmaf(-m[i], cmul, v[i] * keep);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if (i == jj) v[i] = rjx;
          else if (i > jj) v[i] = fmaf(-m[i], cmul, v[i] * keep);
        }
      }
    }
  }
  // store R_kk^-1 = (R^-T)^T in place: blk[x][row] = v(row, x) for row >= x, 0 below
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = 16 * g + i;
    blk[(size_t)x * np + row] = (row >= x) ? v[i] : 0.0f;
  }
}

// ---------------------------------------------------------------- 6. anti-transpose
__global__ __launch_bounds__(256) void flip_out_kernel(const float* __restrict__ X, int np, int n,
                                                       float* __restrict__ U) {
  __shared__ float tile[32][33];
  const int a0 = blockIdx.y * 32, b0 = blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8
  // U[a][b] = X[n-1-b][n-1-a]; read rows r = n-1-b (b in tile), cols c = n-1-a
  for (int yy = ty; yy < 32; yy += 8) {
    const int b = b0 + yy, a = a0 + tx;
    float v = 0.0f;
    if (a < n && b < n && b >= a) v = X[(size_t)(n - 1 - b) * np + (n - 1 - a)];
    tile[yy][tx] = v;
  }
  __syncthreads();
  for (int yy = ty; yy < 32; yy += 8) {
    const int a = a0 + yy, b = b0 + tx;
    if (a < n && b < n) U[(size_t)a * n + b] = tile[tx][yy];
  }
}

// ---------------------------------------------------------------- planning
struct HinvLayout {
  int n, np, nblk, ldz;
  size_t off_A, off_Z, off_lam, off_flag, total;
};

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
  L.off_lam = off;
  off = align_up(off + sizeof(double));
  L.off_flag = off;
  off = align_up(off + sizeof(int));
  L.total = off;
  return L;
}

struct TreeNode { int a, mid, b; };

static void build_levels(int lo, int hi, int depth, std::vector<std::vector<TreeNode>>& lv) {
  if (hi - lo <= 1) return;
  const int mid = lo + (hi - lo) / 2;
  if ((int)lv.size() <= depth) lv.resize(depth + 1);
  lv[depth].push_back(TreeNode{lo, mid, hi});
  build_levels(lo, mid, depth + 1, lv);
  build_levels(mid, hi, depth + 1, lv);
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
  double* lam = reinterpret_cast<double*>(base + L.off_lam);
  int* flag = reinterpret_cast<int*>(base + L.off_flag);
  const int n = L.n, np = L.np, nb = L.nblk;

  damp_lambda_kernel<<<1, 1024, 0, s>>>(H, hdiag, n, damp_percent, lam, flag);
  GPTQ_LAUNCH_CHECK();
  act_order_kernel<<<(n + 255) / 256, 256, 0, s>>>(H, hdiag, n, desc_act, perm);
  GPTQ_LAUNCH_CHECK();
  gather_flip_kernel<<<dim3((np + 255) / 256, np), 256, 0, s>>>(H, n, np, perm, lam, A);
  GPTQ_LAUNCH_CHECK();

  // 4. Cholesky A = R^T R, storing R_kk^-1 on the diagonal blocks
  for (int k = 0; k < nb; ++k) {
    chol_diag_kernel<<<1, 1024, 0, s>>>(A, np, k, flag);
    GPTQ_LAUNCH_CHECK();
    const int rest = np - (k + 1) * kNB;
    if (rest <= 0) continue;
    float* Akk = A + (size_t)k * kNB * np + (size_t)k * kNB;
    float* Arow = Akk + kNB;                                  // A[k-block rows][after]
    float* Atrail = A + (size_t)(k + 1) * kNB * np + (size_t)(k + 1) * kNB;
    // R_k,rest = R_kk^-T A_k,rest : Aop(i,j) = Rinv[j][i] (k-major), in place
    gemm_f32<true>(Akk, np, Arow, np, Arow, np, kNB, rest, kNB, 1.0f, 0.0f, 0, 0, 0, s);
    GPTQ_LAUNCH_CHECK();
    // A_rest -= R_k,rest^T R_k,rest (upper tiles)
    gemm_f32<true>(Arow, np, Arow, np, Atrail, np, rest, rest, kNB, -1.0f, 1.0f, 0, 0, 1, s);
    GPTQ_LAUNCH_CHECK();
  }

  // 5. triangular inverse, deepest tree level first
  std::vector<std::vector<TreeNode>> levels;
  build_levels(0, nb, 0, levels);
  for (int lv = (int)levels.size() - 1; lv >= 0; --lv) {
    const std::vector<TreeNode>& nodes = levels[lv];
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
      launch_gemm_group<false, kStore>(g1, 1.0f, 0.0f, 1, 0, 0, nullptr, s);
      GPTQ_LAUNCH_CHECK();
      launch_gemm_group<false, kStore>(g2, -1.0f, 0.0f, 0, 1, 0, nullptr, s);
      GPTQ_LAUNCH_CHECK();
    }
  }

  // 6. U
  flip_out_kernel<<<dim3((n + 31) / 32, (n + 31) / 32), 256, 0, s>>>(A, np, n, U);
  GPTQ_LAUNCH_CHECK();

  int hflag = 0;
  GPTQ_HIP_TRY(hipMemcpyAsync(&hflag, flag, sizeof(int), hipMemcpyDeviceToHost, s));
  GPTQ_HIP_TRY(hipStreamSynchronize(s));
  return hflag ? GPTQ_ERR_NOT_PD : GPTQ_OK;
}
