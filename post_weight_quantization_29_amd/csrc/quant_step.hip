// Fused block step of the GPTQ column loop (GPTQ practice page m.lqnn.cn/news/117696,
// section 2.2 "second": a block of columns is quantized, then everything after
// it is updated with one matrix product).
//
// The per-block order is: column loop of block b, then W[:, after b] -= Err_b *
// U[b, after b], then the column loop of block b + 1.  Block b + 1's loop only
// needs block b's update of its own columns, and each row needs only its own
// part of it, so one launch holds two kinds of workgroups:
//   * column-loop workgroups (16 rows each): the 16 x 128 product
//     Err_b[rows] * U[b, b+1] with v_mfma_f32_32x32x2f32 (rows 16..31 of the
//     32-row operand are zero), the same MFMA steps in the same k order as the
//     trailing GEMM's tile, kept in LDS; then the column loop of block b + 1
//     starting from the work copy minus that product;
//   * trailing-GEMM workgroups: W[:, after b + 1] -= Err_b * U[b, after b + 1],
//     128 x 128 tiles.
// Neither reads what the other writes, so there are no waits between them, and
// every value equals what the per-block launches compute.
#include "gemm_f32.h"
#include "panel.h"

namespace gptq {

constexpr int kPreP = kQB + 4;                             // pitch of the product rows (floats)
constexpr size_t kStepU = (size_t)kQB * kQB * 4;           // U tile / sU4 (64 KB)
constexpr size_t kStepInv = kStepU;                        // sInv: kQB doubles
constexpr size_t kStepPerm = kStepInv + kQB * 8;           // sPerm: kQB ints
constexpr size_t kStepE = kStepPerm + kQB * 4;             // Err rows [kQB][16], later the products [16][kPreP]
constexpr size_t kStepLds = kStepE + (size_t)kQRows * kPreP * 4;
static_assert((size_t)kQB * kQRows * 4 <= (size_t)kQRows * kPreP * 4, "Err rows fit the product area");
static_assert(kStepLds >= 2 * (size_t)kGK * kGP * 4, "the GEMM tile's staging fits");
static_assert(2 * kStepLds <= 160 * 1024, "two workgroups per CU");

// products P[r][c] = sum_k Err_b[k][row0 + r] * U[b0 + k][b1 + c], r < 16, c < 128
GPTQ_DEV void step_products(const StepArgs& f, int row0, char* lds) {
  const PanelArgs& a = f.pa;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float* sE = reinterpret_cast<float*>(lds + kStepE);      // [k][16]
  float* sUb = reinterpret_cast<float*>(lds);              // [k][kQB]
  // Err rows: k = tid/16 + 16u, row row0 + tid%16 (16 consecutive floats per k)
  {
    const int i = tid & 15, r = row0 + i;
    float e[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k = (tid >> 4) + 16 * u;
      e[u] = (r < a.d_out) ? f.Eprev[(size_t)k * a.d_out + r] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) sE[((tid >> 4) + 16 * u) * kQRows + i] = e[u];
  }
  // U tile: rows k of block b, columns c < bw of block b + 1 (zero beyond)
  {
    float4 v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = u * 256 + tid, k = e >> 5, c = 4 * (e & 31);
      v[u] = (c + 3 < a.bw) ? *reinterpret_cast<const float4*>(f.Uprev + (size_t)k * a.d + c)
                            : make_float4(c + 0 < a.bw ? f.Uprev[(size_t)k * a.d + c + 0] : 0.0f,
                                          c + 1 < a.bw ? f.Uprev[(size_t)k * a.d + c + 1] : 0.0f,
                                          c + 2 < a.bw ? f.Uprev[(size_t)k * a.d + c + 2] : 0.0f, 0.0f);
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = u * 256 + tid;
      reinterpret_cast<float4*>(sUb)[e] = v[u];
    }
  }
  __syncthreads();
  // wave w: rows 0..31 (16..31 zero) x columns 32w .. 32w+31, k in pairs
  f32x16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
  const int m = lane & 31, kh = lane >> 5;
#pragma unroll 8
  for (int k2 = 0; k2 < kQB; k2 += 2) {
    const float av = (m < kQRows) ? sE[(k2 + kh) * kQRows + m] : 0.0f;
    const float bv = sUb[(k2 + kh) * kQB + 32 * wave + m];
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
  }
  __syncthreads();                                         // sE and sUb are read
  float* sPre = reinterpret_cast<float*>(lds + kStepE);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int rr = mfma32_row(r, lane);
    if (rr < kQRows) sPre[rr * kPreP + 32 * wave + mfma32_col(lane)] = acc[r];
  }
  // the column loop's first barrier orders these stores before their reads
}

template <int GT>
__global__ __launch_bounds__(256, 2) void quant_step_kernel(StepArgs f) {
  __shared__ __attribute__((aligned(16))) char lds[kStepLds];
  const int npanel = (f.pa.d_out + kQRows - 1) / kQRows;
  const int wg = (int)blockIdx.x;
  if (wg < npanel) {
    step_products(f, wg * kQRows, lds);
    panel_rows<GT, true>(f.pa, wg, reinterpret_cast<float4 (*)[kQS / 4][kQL]>(lds),
                         reinterpret_cast<double*>(lds + kStepInv), reinterpret_cast<int*>(lds + kStepPerm),
                         reinterpret_cast<const float*>(lds + kStepE));
    return;
  }
  // trailing tile: rows 128*(t / tn), columns 128*(t % tn) of the columns after block b + 1
  const GemmProblem P{f.Eprev, f.Urest, f.Wrest, nullptr, f.pa.d_out, f.pa.d, f.pa.d, f.pa.d_out, f.rest, f.kprev};
  int m0, n0;
  tile_origin(P, wg - npanel, 0, m0, n0);
  float* sA = reinterpret_cast<float*>(lds);
  float* sB = sA + kGK * kGP;
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  float cold[2][2][16];
  gemm_tile_load_c(P, m0, n0, cold);
  gemm_tile_contract<true, true>(P, m0, n0, 0, P.K, sA, sB, acc);
  gemm_tile_store(P, m0, n0, -1.0f, 1.0f, acc, cold);
}

void launch_quant_step(const StepArgs& f, int gt, hipStream_t s) {
  const int npanel = (f.pa.d_out + kQRows - 1) / kQRows;
  const int grid = npanel + (f.rest > 0 ? gemm_tiles(f.pa.d_out, f.rest) : 0);
  switch (gt) {
    case 4: quant_step_kernel<4><<<grid, 256, 0, s>>>(f); break;
    case 8: quant_step_kernel<8><<<grid, 256, 0, s>>>(f); break;
    case 16: quant_step_kernel<16><<<grid, 256, 0, s>>>(f); break;
    case 32: quant_step_kernel<32><<<grid, 256, 0, s>>>(f); break;
    case 64: quant_step_kernel<64><<<grid, 256, 0, s>>>(f); break;
    default: quant_step_kernel<128><<<grid, 256, 0, s>>>(f); break;
  }
}

}  // namespace gptq
