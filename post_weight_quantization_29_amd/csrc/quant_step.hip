// Fused block step of the GPTQ column loop (GPTQ practice page m.lqnn.cn/news/117696,
// section 2.2 "second": a block of columns is quantized, then everything after
// it is updated with one matrix product).
//
// Blocks are grouped into super-blocks of gb consecutive blocks.  The
// per-block order is: column loop of block b, then its lazy update of the
// later columns of its super-block, W[:, b+1 .. end of S] -= Err_b U[b, ...];
// at the super-block's end, one update of every column after it by the whole
// super-block, W[:, after S] -= Err_S U[S, after S] (K = 128 gb).  Deferring
// the far columns' updates to one product of K = 128 gb is exact in exact
// arithmetic (the sums are only regrouped) and reads and writes the work copy
// gb times less often.  Block b + 1's loop only needs the update it still
// owes (block b's, or at a super-block's end the whole super-block's) for its
// own columns, and each row needs only its own part of it, so one launch
// holds two kinds of workgroups:
//   * column-loop workgroups (16 rows each): the 16 x 128 product of the owed
//     Err rows and U rows with v_mfma_f32_32x32x2f32 (rows 16..31 of the
//     32-row operand are zero), the same MFMA steps in the same k order as the
//     trailing GEMM's tile, kept in LDS; then the column loop of block b + 1
//     starting from the work copy minus that product;
//   * trailing-GEMM workgroups: the same Err rows' update of the columns after
//     block b + 1 (to the super-block's end, or to the last column), 128 x 128
//     tiles.
// Neither reads what the other writes, so there are no waits between them, and
// every value equals what the per-block launches compute.
#include "gemm_f32.h"
#include "panel.h"

namespace gptq {

constexpr int kPreP = kQB + 4;                             // pitch of the product rows (floats)
constexpr int kPK = 64;                                    // k per staged chunk of the products
// LDS: [0, kStepU) the packed U block of the column loop; before it, the
// products' staging (a U chunk [kPK][kQB] and Err rows [kPK][16]) and then
// the products themselves [16][kPreP], read before the U block is written
constexpr size_t kStepU = (size_t)kUPacked * 16;           // 48 KB
constexpr size_t kStepStageE = (size_t)kPK * kQB * 4;      // Err rows after the U chunk
constexpr size_t kStepInv = kStepU;                        // sInv: kQB doubles
constexpr size_t kStepPerm = kStepInv + kQB * 8;           // sPerm: kQB ints
constexpr size_t kStepLds = kStepPerm + kQB * 4;
static_assert(kStepStageE + (size_t)kPK * kQRows * 4 <= kStepU, "the products' staging fits the U area");
static_assert((size_t)kQRows * kPreP * 4 <= kStepU, "the products fit the U area");
static_assert(kStepLds >= 2 * (size_t)kGK * kGP * 4, "the GEMM tile's staging fits");
static_assert(3 * kStepLds <= 160 * 1024, "three workgroups per CU");

// products P[r][c] = sum_k Eprev[k][row0 + r] * Uprev[k][c], r < 16, c < 128,
// k < kprev (128 per block whose update is still owed), in chunks of kPK k
// staged through LDS; the k order is the trailing GEMM tile's
GPTQ_DEV void step_products(const StepArgs& f, int row0, char* lds) {
  const PanelArgs& a = f.pa;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float* sE = reinterpret_cast<float*>(lds + kStepStageE);  // [k][16]
  float* sUb = reinterpret_cast<float*>(lds);              // [k][kQB]
  f32x16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
  const int m = lane & 31, kh = lane >> 5;
  for (int kc = 0; kc < f.kprev; kc += kPK) {
    const float* E = f.Eprev + (size_t)kc * a.d_out;
    const float* Ub = f.Uprev + (size_t)kc * a.d;
    // Err rows: k = tid/16 + 16u, row row0 + tid%16 (16 consecutive floats per k)
    {
      const int i = tid & 15, r = row0 + i;
      float e[kPK / 16];
#pragma unroll
      for (int u = 0; u < kPK / 16; ++u) {
        const int k = (tid >> 4) + 16 * u;
        e[u] = (r < a.d_out) ? E[(size_t)k * a.d_out + r] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < kPK / 16; ++u) sE[((tid >> 4) + 16 * u) * kQRows + i] = e[u];
    }
    // U chunk: rows kc + k of the owed blocks, columns c < bw of this block (zero beyond)
    {
      constexpr int NU = kPK * kQB / 4 / 256;
      float4 v[NU];
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int e = u * 256 + tid, k = e >> 5, c = 4 * (e & 31);
        v[u] = (c + 3 < a.bw) ? *reinterpret_cast<const float4*>(Ub + (size_t)k * a.d + c)
                              : make_float4(c + 0 < a.bw ? Ub[(size_t)k * a.d + c + 0] : 0.0f,
                                            c + 1 < a.bw ? Ub[(size_t)k * a.d + c + 1] : 0.0f,
                                            c + 2 < a.bw ? Ub[(size_t)k * a.d + c + 2] : 0.0f, 0.0f);
      }
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int e = u * 256 + tid;
        reinterpret_cast<float4*>(sUb)[e] = v[u];
      }
    }
    __syncthreads();
    // wave w: rows 0..31 (16..31 zero) x columns 32w .. 32w+31, k in pairs
#pragma unroll 8
    for (int k2 = 0; k2 < kPK; k2 += 2) {
      const float av = (m < kQRows) ? sE[(k2 + kh) * kQRows + m] : 0.0f;
      const float bv = sUb[(k2 + kh) * kQB + 32 * wave + m];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
    }
    __syncthreads();                                       // sE and sUb are read
  }
  float* sPre = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int rr = mfma32_row(r, lane);
    if (rr < kQRows) sPre[rr * kPreP + 32 * wave + mfma32_col(lane)] = acc[r];
  }
  __syncthreads();                                         // the products are complete
}

template <int GT>
__global__ __launch_bounds__(256, 3) void quant_step_kernel(StepArgs f) {
  __shared__ __attribute__((aligned(16))) char lds[kStepLds];
  const int npanel = (f.pa.d_out + kQRows - 1) / kQRows;
  const int wg = (int)blockIdx.x;
  if (wg < npanel) {
    step_products(f, wg * kQRows, lds);
    panel_rows<GT, true>(f.pa, wg, reinterpret_cast<float4*>(lds),
                         reinterpret_cast<double*>(lds + kStepInv), reinterpret_cast<int*>(lds + kStepPerm),
                         reinterpret_cast<const float*>(lds));
    return;
  }
  // trailing tile: rows 128*(t / tn), columns 128*(t % tn) of the update's columns
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
  gemm_tile_contract<true, true>(P, m0, n0, 0, P.K, sA, sB, acc);
  gemm_tile_update(P, m0, n0, -1.0f, 1.0f, acc);
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
