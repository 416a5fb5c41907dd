// GPTQ column loop and INT4 packing.
//
// Sources: GPTQ practice page m.lqnn.cn/news/117696, section 2.1 (quantize one
// weight, move the not-yet-quantized ones along the inverse-Hessian column),
// section 2.2 "second" (quantize a 128-column block, then update everything
// after it with one matrix product), section 3.3 (group_size consecutive
// columns share a scale and zero point); tutorial page "大模型压缩量化技术：GPTQ
// 与 AWQ 原理详解 + Python 实战教程", section 二 (min-max uniform grid).
//
// Per 128-column block b (processing order):
//   panel_kernel:   rows in parallel, 16 lanes per row (lane q holds the
//                   block's columns 16t+q, t = 0..7), 4 rows per wave, 4 waves
//                   per workgroup; U's diagonal block in LDS; column j's
//                   weight is broadcast across the row's lanes with DPP,
//                   quantized, its scaled error e = (w - q)/U[j][j] pushed onto
//                   the later columns of the block (w -= e*U[j][.], in fp64)
//                   and kept in ErrT.
//   trailing GEMM:  W[:, b1:] -= Err * U[b0:b1, b1:] (fp32 MFMA).
#include "gemm_f32.h"
#include "lookahead.h"
#include "panel.h"

#include <cstdlib>
#include <cstring>
#include <utility>

namespace gptq {

// ---------------------------------------------------------------- W gather
__global__ __launch_bounds__(256) void gather_w_kernel(const void* __restrict__ W, gptq_dtype wt,
                                                       int d_out, int d, const int* __restrict__ perm,
                                                       int G, float* __restrict__ Wp,
                                                       int* __restrict__ g_idx) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= d) return;
  const int src = perm[j];
  if (blockIdx.y == 0) g_idx[src] = j / G;
  for (int r = blockIdx.y; r < d_out; r += gridDim.y)
    Wp[(size_t)r * d + j] = load_as_float(W, wt, (size_t)r * d + src);
}

// ---------------------------------------------------------------- pack
// packed word m = sum_k (codes[8m+k] & 15) << 4k over the flat code array
// (cols % 8 == 0, so no word straddles two rows).
__global__ __launch_bounds__(256) void pack_int4_kernel(const uint8_t* __restrict__ codes,
                                                        int64_t nwords, uint32_t* __restrict__ out) {
  const int64_t nq = nwords / 4;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nq; i += stride) {
    const uint4 a = reinterpret_cast<const uint4*>(codes)[2 * i];
    const uint4 b = reinterpret_cast<const uint4*>(codes)[2 * i + 1];
    auto pk = [](uint32_t lo, uint32_t hi) -> uint32_t {
      uint32_t r = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) r |= ((lo >> (8 * k)) & 0xFu) << (4 * k);
#pragma unroll
      for (int k = 0; k < 4; ++k) r |= ((hi >> (8 * k)) & 0xFu) << (16 + 4 * k);
      return r;
    };
    uint4 o;
    o.x = pk(a.x, a.y);
    o.y = pk(a.z, a.w);
    o.z = pk(b.x, b.y);
    o.w = pk(b.z, b.w);
    reinterpret_cast<uint4*>(out)[i] = o;
  }
  // tail words (nwords % 4), one thread each
  const int64_t tail0 = nq * 4;
  const int64_t ti = tail0 + (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (blockIdx.x == 0 && ti < nwords) {
    uint32_t r = 0;
    for (int k = 0; k < 8; ++k) r |= ((uint32_t)codes[8 * ti + k] & 0xFu) << (4 * k);
    out[ti] = r;
  }
}

// dense packing: one thread per output word; word w of a row holds bits
// [32w, 32w + 32) of the row's stream, i.e. codes floor(32w/bits) ..
// floor((32w + 31)/bits), the first and last possibly in part.
__global__ __launch_bounds__(256) void pack_dense_kernel(const uint8_t* __restrict__ codes, int64_t rows,
                                                         int64_t cols, int bits, int64_t nw,
                                                         uint32_t* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows * nw) return;
  const int64_t r = idx / nw, w = idx - r * nw;
  const uint8_t* row = codes + r * cols;
  const int64_t bit0 = 32 * w;
  const int64_t k0 = bit0 / bits, k1 = (bit0 + 31) / bits;
  const uint32_t mask = (1u << bits) - 1u;
  uint64_t acc = 0;
  for (int64_t k = k0; k <= k1; ++k) {
    const uint64_t v = (uint64_t)(row[k] & mask);
    const int64_t pos = k * bits - bit0;         // -bits < pos < 32
    acc |= (pos >= 0) ? (v << pos) : (v >> (-pos));
  }
  out[idx] = (uint32_t)acc;
}

// ---------------------------------------------------------------- planning
struct QuantLayout {
  size_t off_wp, off_err, total;
};

static QuantLayout quant_layout(int d_out, int d) {
  QuantLayout L;
  size_t off = 0;
  L.off_wp = off;
  off = align_up(off + (size_t)d_out * d * sizeof(float));
  L.off_err = off;   // two buffers: panel b+1 writes one while block b's update reads the other
  off = align_up(off + 2 * (size_t)kQB * d_out * sizeof(float));
  L.total = off;
  return L;
}

static int check_config(const gptq_config* c, int d) {
  if (!c) return GPTQ_ERR_INVALID_ARG;
  if (c->bits < 2 || c->bits > 8) return GPTQ_ERR_INVALID_ARG;
  if (c->desc_act != 0 && c->desc_act != 1) return GPTQ_ERR_INVALID_ARG;
  if (c->block_size <= 0 || c->sym < 0 || c->sym > 1) return GPTQ_ERR_INVALID_ARG;
  const int G = c->group_size;
  if (G != -1 && G <= 0) return GPTQ_ERR_INVALID_ARG;
  if (c->block_size != kQB) return GPTQ_ERR_UNSUPPORTED;
  if (G != -1) {
    const bool inside = (kQB % G == 0) && (G % 4 == 0);
    const bool spans = (G % kQB == 0);
    if (!inside && !spans) {
      // G and the block size neither divide one another: lazy batching would
      // no longer equal the column-by-column method
      if ((kQB % G != 0) && (G % kQB != 0)) return GPTQ_ERR_INVALID_ARG;
      return GPTQ_ERR_UNSUPPORTED;
    }
  }
  (void)d;
  return GPTQ_OK;
}

}  // namespace gptq

using namespace gptq;

extern "C" size_t gptq_quantize_workspace_size(int32_t d_out, int32_t d_in, const gptq_config* cfg) {
  (void)cfg;
  if (d_out <= 0 || d_in <= 0) return 0;
  return quant_layout(d_out, d_in).total;
}

extern "C" int gptq_quantize_layer(const void* W, gptq_dtype w_dtype, int32_t d_out, int32_t d_in,
                                   const float* U, const int32_t* perm, const gptq_config* cfg,
                                   uint8_t* codes, float* scales, int32_t* zeros, int32_t* g_idx,
                                   float* Q, void* ws, size_t ws_bytes, hipStream_t s) {
  if (!W || !U || !perm || !codes || !scales || !zeros || !g_idx) return GPTQ_ERR_INVALID_ARG;
  if (d_out <= 0 || d_in <= 0) return GPTQ_ERR_INVALID_ARG;
  if (w_dtype != GPTQ_F32 && w_dtype != GPTQ_F16 && w_dtype != GPTQ_BF16) return GPTQ_ERR_INVALID_ARG;
  const int st = check_config(cfg, d_in);
  if (st != GPTQ_OK) return st;
  const QuantLayout L = quant_layout(d_out, d_in);
  if (!ws || ws_bytes < L.total) return GPTQ_ERR_WORKSPACE;
  char* base = static_cast<char*>(ws);
  float* Wp = reinterpret_cast<float*>(base + L.off_wp);
  float* ErrT = reinterpret_cast<float*>(base + L.off_err);
  const int d = d_in;
  const int G = (cfg->group_size == -1) ? d : cfg->group_size;
  const int ng = (d + G - 1) / G;

  gather_w_kernel<<<dim3((d + 255) / 256, std::min(d_out, 1024)), 256, 0, s>>>(W, w_dtype, d_out, d,
                                                                              perm, G, Wp, g_idx);
  GPTQ_LAUNCH_CHECK();

  PanelArgs pa;
  pa.Wp = Wp; pa.U = U; pa.perm = perm; pa.codes = codes; pa.Q = Q;
  pa.scales = scales; pa.zeros = zeros; pa.ErrT = ErrT;
  pa.d_out = d_out; pa.d = d; pa.G = G; pa.ng = ng;
  pa.maxq = (float)((1 << cfg->bits) - 1);
  pa.sym = cfg->sym;
  const int nrow_blocks = (d_out + kQRows - 1) / kQRows;
  // in-block group sizes are compile-time; wider groups (or one per row) use 0
  const int gt = (G <= kQB && kQB % G == 0 && G % 4 == 0) ? G : 0;

  // Fused block steps (groups inside the block, operands the 16-byte loads
  // take): block 0's column loop, then one launch per later block holding its
  // column loop (which first applies the previous block's update to its own
  // rows) beside the previous block's trailing update of the columns after
  // it.  Same operations, same results as the per-block launches below.
  const char* fused_env = std::getenv("GPTQ_FUSED_STEP");
  const bool fused_on = !(fused_env && std::strcmp(fused_env, "0") == 0);
  if (fused_on && quant_step_applies(d_out, d, U, gt)) {
    pa.b0 = 0;
    pa.bw = std::min(kQB, d);
    pa.ErrT = ErrT;
    switch (gt) {
      case 4: panel_kernel<4><<<nrow_blocks, 256, 0, s>>>(pa); break;
      case 8: panel_kernel<8><<<nrow_blocks, 256, 0, s>>>(pa); break;
      case 16: panel_kernel<16><<<nrow_blocks, 256, 0, s>>>(pa); break;
      case 32: panel_kernel<32><<<nrow_blocks, 256, 0, s>>>(pa); break;
      case 64: panel_kernel<64><<<nrow_blocks, 256, 0, s>>>(pa); break;
      default: panel_kernel<128><<<nrow_blocks, 256, 0, s>>>(pa); break;
    }
    GPTQ_LAUNCH_CHECK();
    for (int b0 = 0, blk = 0; b0 + kQB < d; b0 += kQB, ++blk) {
      const int b1 = b0 + kQB, bw1 = std::min(kQB, d - b1);
      StepArgs st;
      st.pa = pa;
      st.pa.b0 = b1;
      st.pa.bw = bw1;
      st.pa.ErrT = ErrT + (size_t)((blk + 1) & 1) * kQB * d_out;
      st.Eprev = ErrT + (size_t)(blk & 1) * kQB * d_out;
      st.Uprev = U + (size_t)b0 * d + b1;
      st.Wrest = Wp + b1 + bw1;
      st.Urest = U + (size_t)b0 * d + b1 + bw1;
      st.rest = d - b1 - bw1;
      st.kprev = kQB;
      launch_quant_step(st, gt, s);
      GPTQ_LAUNCH_CHECK();
    }
    return GPTQ_OK;
  }
  // Lookahead: block b's update of the next block's columns runs on the
  // caller's stream, the rest of the trailing columns on the side stream, so
  // panel b+1 overlaps it.  Panels alternate between two ErrT buffers; an
  // update of columns c waits for the side stream's previous update, which
  // also wrote columns c.  Each element gets the same tile, contraction and
  // order of updates as with one stream.  Each cross-stream wait costs a few
  // microseconds, so only layers of 2^25 weights or more (where the trailing
  // updates are long) take this path: measured 3-8 % faster there, 11 %
  // slower at 4096 x 4096.
  Lookahead* la = ((int64_t)d_out * d >= (int64_t(1) << 25)) ? lookahead_for_current_device() : nullptr;
  std::unique_lock<std::mutex> lk;
  if (la) lk = std::unique_lock<std::mutex>(la->mu);
  bool side_pending = false;
  for (int b0 = 0, blk = 0; b0 < d; b0 += kQB, ++blk) {
    const int bw = std::min(kQB, d - b0);
    float* Eb = ErrT + (size_t)(blk & 1) * kQB * d_out;
    pa.b0 = b0;
    pa.bw = bw;
    pa.ErrT = Eb;
    // a group wider than the block takes its grid at its first column from
    // every column of the group, so its panel waits for the side stream too
    if (side_pending && gt == 0 && b0 % G == 0 && b0 + bw < d) {
      GPTQ_HIP_TRY(hipStreamWaitEvent(s, la->trail_done, 0));
      side_pending = false;
    }
    switch (gt) {
      case 4: panel_kernel<4><<<nrow_blocks, 256, 0, s>>>(pa); break;
      case 8: panel_kernel<8><<<nrow_blocks, 256, 0, s>>>(pa); break;
      case 16: panel_kernel<16><<<nrow_blocks, 256, 0, s>>>(pa); break;
      case 32: panel_kernel<32><<<nrow_blocks, 256, 0, s>>>(pa); break;
      case 64: panel_kernel<64><<<nrow_blocks, 256, 0, s>>>(pa); break;
      case 128: panel_kernel<128><<<nrow_blocks, 256, 0, s>>>(pa); break;
      default: panel_kernel<0><<<nrow_blocks, 256, 0, s>>>(pa); break;
    }
    GPTQ_LAUNCH_CHECK();
    const int b1 = b0 + bw;
    if (b1 >= d) continue;
    const int rest = d - b1;
    // W[:, b1:] -= Err * U[b0:b1, b1:]  with Aop(m, k) = ErrT[k][m]
    if (!la || rest <= kQB) {
      if (side_pending) GPTQ_HIP_TRY(hipStreamWaitEvent(s, la->trail_done, 0));
      side_pending = false;
      gemm_f32<true>(Eb, d_out, U + (size_t)b0 * d + b1, d, Wp + b1, d, d_out, rest, bw, -1.0f, 1.0f,
                     0, 0, 0, s);
      GPTQ_LAUNCH_CHECK();
      continue;
    }
    GPTQ_HIP_TRY(hipEventRecord(la->panel_done, s));
    if (side_pending) GPTQ_HIP_TRY(hipStreamWaitEvent(s, la->trail_done, 0));
    gemm_f32<true>(Eb, d_out, U + (size_t)b0 * d + b1, d, Wp + b1, d, d_out, kQB, bw, -1.0f, 1.0f, 0,
                   0, 0, s);
    GPTQ_LAUNCH_CHECK();
    GPTQ_HIP_TRY(hipStreamWaitEvent(la->side, la->panel_done, 0));
    gemm_f32<true>(Eb, d_out, U + (size_t)b0 * d + b1 + kQB, d, Wp + b1 + kQB, d, d_out, rest - kQB, bw,
                   -1.0f, 1.0f, 0, 0, 0, la->side);
    GPTQ_LAUNCH_CHECK();
    GPTQ_HIP_TRY(hipEventRecord(la->trail_done, la->side));
    side_pending = true;
  }
  if (side_pending) GPTQ_HIP_TRY(hipStreamWaitEvent(s, la->trail_done, 0));
  return GPTQ_OK;
}

extern "C" int gptq_pack_int4(const uint8_t* codes, int64_t rows, int64_t cols, uint32_t* packed,
                              hipStream_t s) {
  if (!codes || !packed || rows < 0 || cols < 0 || (cols % 8) != 0) return GPTQ_ERR_INVALID_ARG;
  const int64_t nwords = rows * cols / 8;
  if (nwords == 0) return GPTQ_OK;
  if ((reinterpret_cast<uintptr_t>(codes) & 15) || (reinterpret_cast<uintptr_t>(packed) & 15))
    return GPTQ_ERR_INVALID_ARG;
  const int64_t nq = std::max<int64_t>(1, nwords / 4);
  const int blocks = (int)std::min<int64_t>((nq + 255) / 256, 8192);
  pack_int4_kernel<<<blocks, 256, 0, s>>>(codes, nwords, packed);
  GPTQ_LAUNCH_CHECK();
  return GPTQ_OK;
}

extern "C" int gptq_pack_dense(const uint8_t* codes, int64_t rows, int64_t cols, int32_t bits,
                               uint32_t* packed, hipStream_t s) {
  if (!codes || !packed || rows < 0 || cols < 0) return GPTQ_ERR_INVALID_ARG;
  if (bits != 2 && bits != 3 && bits != 4 && bits != 8) return GPTQ_ERR_INVALID_ARG;
  if ((cols * bits) % 32 != 0) return GPTQ_ERR_INVALID_ARG;
  const int64_t nw = cols * bits / 32;
  const int64_t total = rows * nw;
  if (total == 0) return GPTQ_OK;
  const int64_t blocks = (total + 255) / 256;
  if (blocks > 0x7fffffff) return GPTQ_ERR_INVALID_ARG;
  pack_dense_kernel<<<(unsigned)blocks, 256, 0, s>>>(codes, rows, cols, bits, nw, packed);
  GPTQ_LAUNCH_CHECK();
  return GPTQ_OK;
}
