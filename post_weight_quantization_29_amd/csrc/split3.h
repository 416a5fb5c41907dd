// Products of fp32 operands on the 16-bit MFMA tile loop (csrc/hessian.hip):
// each operand is scaled by a power of two per output row or column (exact)
// and split into two fp16 pieces h + l, and the three piece products lh, hl,
// hh carry the product to within 3 2^-22 of it, below what the contraction's
// fp32 accumulation carries; so each fp32 product costs three fp16 MFMA
// products.  Symmetric rank-K updates (the factor's super-block updates) and
// general products (the tree inverse's large nodes, the column loop's
// super-block tails).
#pragma once
#include "common.h"

namespace gptq {

// true when an n-wide update has enough 256 x 256 tiles to fill the chip
// (below that the fp32 tiles are as fast)
bool split3_pays(int n);

// bytes of the planes of a K x n panel (h, l) and of its columns' scales
size_t split3_planes_bytes(int K, int n);

// C[r][c] -= sum_k P[k][r] P[k][c] for r <= c (r, c < n; the strictly lower
// 128-blocks of C are not touched; the lower halves of the diagonal 128-blocks
// are written too).  P: K x n fp32, row pitch ldp; C: n x n fp32, row pitch
// ldc; K a multiple of 32, n a multiple of 128, ldp a multiple of 4, P 16-byte
// aligned; planes: split3_planes_bytes(K, n) bytes of device scratch, 16-byte
// aligned.  Asynchronous on s.
int split3_update(const float* P, int ldp, int K, int n, float* C, int ldc, void* planes, hipStream_t s);

// General product on the same tile loop: C = beta C + alpha A^T B with
// alpha = -1 (neg) or +1 and beta = 1 or 0, for A: K x m fp32 k-major (row
// pitch lda), or, with a_rows, m x K row-major (transposed while it is
// split), and B: K x n fp32 k-major (row pitch ldb); C: m x n fp32, row pitch
// ldc.  tri = 1: A is upper triangular (a_rows; A[i][k] = 0 for k < i, tile
// row I contracts k >= 256 I); tri = 2: B is upper triangular (B[k][j] = 0
// for k > j, tile column J contracts k < 256 (J + 1)); entries below those
// diagonals are not read as stored.  The pieces h, l of A and of B are
// formed first (2 K (m + n) fp16 and m + n scales in planes, 16-byte
// aligned: split3_gemm_planes_bytes(K, m, n)).  Applies when
// m, n are multiples of 8, K of 32, lda and ldb of 4, A and B 16-byte
// aligned, and C has at least 128 tiles of 256 x 256; callers use the fp32
// tiles otherwise.  Asynchronous on s.
bool split3_gemm_shape_ok(int K, int m, int n);
bool split3_gemm_applies(const float* A, int lda, bool a_rows, const float* B, int ldb, int K, int m, int n);
size_t split3_gemm_planes_bytes(int K, int m, int n);
int split3_gemm(const float* A, int lda, bool a_rows, const float* B, int ldb, int K, int m, int n, float* C,
                int ldc, bool neg, bool beta, int tri, void* planes, hipStream_t s);

}  // namespace gptq
