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
#include "split3.h"
#include "panel.h"

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

// The same gather with row r staged in LDS first (coalesced loads; the
// permuted reads then hit LDS instead of a new cache line per element); one
// workgroup per row, rows up to kGatherW elements.
constexpr int kGatherW = 32768;
__global__ __launch_bounds__(1024) void gather_w_row_kernel(const void* __restrict__ W, gptq_dtype wt,
                                                           int d_out, int d, const int* __restrict__ perm,
                                                           int G, float* __restrict__ Wp,
                                                           int* __restrict__ g_idx, int vec) {
  __shared__ float row[kGatherW];
  const int r = blockIdx.x;
  if (vec) {
    // 16-byte accesses (vec: d % 8 == 0 and W, perm 16-byte aligned), 8
    // elements per load, every one of a thread's loads issued at once
    constexpr int kU = kGatherW / 8 / 1024;
    uint4 v[kU];
    const char* wr = static_cast<const char*>(W) + (size_t)r * d * (wt == GPTQ_F32 ? 4 : 2);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int c = 8 * (threadIdx.x + 1024 * u);
      if (c < d) {
        if (wt == GPTQ_F32) {
          v[u] = *reinterpret_cast<const uint4*>(wr + 4 * (size_t)c);       // elements c .. c+3
        } else {
          v[u] = *reinterpret_cast<const uint4*>(wr + 2 * (size_t)c);       // elements c .. c+7
        }
      }
    }
    if (wt == GPTQ_F32) {
      // the fp32 row needs twice the loads: the second half of each 8-element chunk
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int c = 8 * (threadIdx.x + 1024 * u);
        if (c < d) {
          const uint4 w2 = *reinterpret_cast<const uint4*>(wr + 4 * (size_t)(c + 4));
          *reinterpret_cast<uint4*>(row + c) = v[u];
          *reinterpret_cast<uint4*>(row + c + 4) = w2;
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int c = 8 * (threadIdx.x + 1024 * u);
        if (c < d) {
          const uint32_t q[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
          float f[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint16_t h = (uint16_t)((e & 1) ? (q[e >> 1] >> 16) : (q[e >> 1] & 0xFFFFu));
            f[e] = (wt == GPTQ_F16) ? (float)__builtin_bit_cast(_Float16, h)
                                    : __builtin_bit_cast(float, (uint32_t)h << 16);
          }
          *reinterpret_cast<float4*>(row + c) = make_float4(f[0], f[1], f[2], f[3]);
          *reinterpret_cast<float4*>(row + c + 4) = make_float4(f[4], f[5], f[6], f[7]);
        }
      }
    }
    __syncthreads();
    for (int j = 4 * threadIdx.x; j < d; j += 4096) {
      const int4 q = *reinterpret_cast<const int4*>(perm + j);
      if (r == 0) {
        g_idx[q.x] = j / G;
        g_idx[q.y] = (j + 1) / G;
        g_idx[q.z] = (j + 2) / G;
        g_idx[q.w] = (j + 3) / G;
      }
      *reinterpret_cast<float4*>(Wp + (size_t)r * d + j) = make_float4(row[q.x], row[q.y], row[q.z], row[q.w]);
    }
    return;
  }
  for (int c = threadIdx.x; c < d; c += 1024) row[c] = load_as_float(W, wt, (size_t)r * d + c);
  __syncthreads();
  for (int j = threadIdx.x; j < d; j += 1024) {
    const int src = perm[j];
    if (r == 0) g_idx[src] = j / G;
    Wp[(size_t)r * d + j] = row[src];
  }
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
  size_t off_wp, off_err, off_gscale, off_planes, total;
};

// Blocks per super-block (the lazy updates of the columns after a super-block
// are one product of K = 128 * gb).  Layers whose fp32 work copy exceeds the
// 256 MB last-level cache take 16: their per-block updates are bound by the
// copy's read-modify-write from HBM, and a longer contraction amortizes the
// tiles' read-modify-write of C (8192 x 28672: 68.5 ms with 8, 65.4 with 16).
// Groups wider than the block read the rest of the group from the work copy at
// its first column, so they keep 1.
constexpr size_t kSuperMinBytes = size_t(256) << 20;
static int super_blocks(int d_out, int d, int gt) {
  if (gt == 0) return 1;
  return ((size_t)d_out * d * sizeof(float) > kSuperMinBytes) ? 16 : 1;
}

static int in_block_group(int G) { return (G <= kQB && kQB % G == 0 && G % 4 == 0) ? G : 0; }

static QuantLayout quant_layout(int d_out, int d, int gb) {
  QuantLayout L;
  size_t off = 0;
  L.off_wp = off;
  off = align_up(off + (size_t)d_out * d * sizeof(float));
  // Err rows of two super-blocks: the next block's column loop writes one
  // while the current super-block's update reads the other
  L.off_err = off;
  off = align_up(off + 2 * (size_t)gb * kQB * d_out * sizeof(float));
  L.off_gscale = off;   // fp64 scale of each row's group in progress (groups wider than the block)
  off = align_up(off + (size_t)d_out * sizeof(double));
  // fp16 pieces of a super-block's Err rows and U rows for the split
  // update of the columns after the next super-block
  L.off_planes = off;
  if (gb > 1) off = align_up(off + split3_gemm_planes_bytes(gb * kQB, d_out, d));
  L.total = off;
  return L;
}

static int check_config(const gptq_config* c, int d) {
  if (!c) return GPTQ_ERR_INVALID_ARG;
  if (c->bits < 2 || c->bits > 8) return GPTQ_ERR_INVALID_ARG;
  if (c->desc_act != 0 && c->desc_act != 1) return GPTQ_ERR_INVALID_ARG;
  if (c->block_size <= 0 || c->sym < 0 || c->sym > 1) return GPTQ_ERR_INVALID_ARG;
  if (c->per_block_steps != 0 && c->per_block_steps != 1) return GPTQ_ERR_INVALID_ARG;
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

static int config_super_blocks(int d_out, int d, const gptq_config* cfg) {
  if (!cfg) return super_blocks(d_out, d, 1);   // the largest layout any configuration needs
  const int G = (cfg->group_size == -1) ? d : cfg->group_size;
  return super_blocks(d_out, d, G > 0 ? in_block_group(G) : 0);
}

extern "C" size_t gptq_quantize_workspace_size(int32_t d_out, int32_t d_in, const gptq_config* cfg) {
  if (d_out <= 0 || d_in <= 0) return 0;
  return quant_layout(d_out, d_in, config_super_blocks(d_out, d_in, cfg)).total;
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
  const int d = d_in;
  const int G = (cfg->group_size == -1) ? d : cfg->group_size;
  const int ng = (d + G - 1) / G;
  // in-block group sizes are compile-time; wider groups (or one per row) use 0
  const int gt = in_block_group(G);
  const int gb = super_blocks(d_out, d, gt);
  const QuantLayout L = quant_layout(d_out, d_in, gb);
  if (!ws || ws_bytes < L.total) return GPTQ_ERR_WORKSPACE;
  char* base = static_cast<char*>(ws);
  float* Wp = reinterpret_cast<float*>(base + L.off_wp);
  float* ErrT = reinterpret_cast<float*>(base + L.off_err);
  double* gscale = reinterpret_cast<double*>(base + L.off_gscale);
  void* planes = base + L.off_planes;

  if (d <= kGatherW)
    gather_w_row_kernel<<<d_out, 1024, 0, s>>>(W, w_dtype, d_out, d, perm, G, Wp, g_idx,
                                               (d % 8 == 0) && (reinterpret_cast<uintptr_t>(W) % 16 == 0) &&
                                                   (reinterpret_cast<uintptr_t>(perm) % 16 == 0));
  else
    gather_w_kernel<<<dim3((d + 255) / 256, std::min(d_out, 1024)), 256, 0, s>>>(W, w_dtype, d_out, d,
                                                                                perm, G, Wp, g_idx);
  GPTQ_LAUNCH_CHECK();

  PanelArgs pa;
  pa.Wp = Wp; pa.U = U; pa.perm = perm; pa.codes = codes; pa.Q = Q;
  pa.scales = scales; pa.zeros = zeros; pa.ErrT = ErrT; pa.gscale = gscale;
  pa.d_out = d_out; pa.d = d; pa.G = G; pa.ng = ng;
  pa.maxq = (float)((1 << cfg->bits) - 1);
  pa.sym = cfg->sym;
  const int nrow_blocks = (d_out + kQRows - 1) / kQRows;
  const int nb = (d + kQB - 1) / kQB;
  // Err rows of block b: super-block b / gb's buffer, slot b % gb
  auto err_of = [&](int b) { return ErrT + ((size_t)((b / gb) & 1) * gb + b % gb) * kQB * d_out; };
  // first column after block b's super-block
  auto super_end = [&](int b) { return std::min(d, (b / gb + 1) * gb * kQB); };
  // At the end of super-block S (block b its last, gb > 1) every later column
  // takes S's update (K = 128 gb) as one split fp16 product when it applies
  // (the next block's column loop then owes nothing); else the columns after
  // the next block; else those after the next super-block; else none (d).
  // Both schedules take the same choice, so their bits agree.
  auto split_start = [&](int b) {
    const int b1 = (b + 1) * kQB, k0 = (b / gb) * gb * kQB;
    const float* E = err_of(b - b % gb);
    const int c_next = b1 + std::min(kQB, d - b1);
    for (const int c : {b1, c_next, std::max(super_end(b + 1), c_next)})
      if (c < d && split3_gemm_applies(E, d_out, false, U + (size_t)k0 * d + c, d, b1 - k0, d_out, d - c)) return c;
    return d;
  };

  // Fused block steps (groups inside the block, operands the 16-byte loads
  // take): block 0's column loop, then one launch per later block holding its
  // column loop (which first applies the previous block's update to its own
  // rows) beside the previous block's trailing update of the columns after
  // it.  Same operations, same results as the per-block launches below
  // (cfg->per_block_steps = 1 selects those).
  if (!cfg->per_block_steps && quant_step_applies(d_out, d, U, gt)) {
    pa.b0 = 0;
    pa.bw = std::min(kQB, d);
    pa.ErrT = err_of(0);
    switch (gt) {
      case 4: panel_kernel<4><<<nrow_blocks, 256, 0, s>>>(pa); break;
      case 8: panel_kernel<8><<<nrow_blocks, 256, 0, s>>>(pa); break;
      case 16: panel_kernel<16><<<nrow_blocks, 256, 0, s>>>(pa); break;
      case 32: panel_kernel<32><<<nrow_blocks, 256, 0, s>>>(pa); break;
      case 64: panel_kernel<64><<<nrow_blocks, 256, 0, s>>>(pa); break;
      default: panel_kernel<128><<<nrow_blocks, 256, 0, s>>>(pa); break;
    }
    GPTQ_LAUNCH_CHECK();
    for (int b = 0; b + 1 < nb; ++b) {
      const int b0 = b * kQB, b1 = b0 + kQB, bw1 = std::min(kQB, d - b1);
      // the Err rows block b + 1 still owes: block b's inside a super-block,
      // the whole super-block's at its end (then every later column takes them)
      const bool s_end = (b + 1) % gb == 0;
      const int k0 = s_end ? (b / gb) * gb * kQB : b0;
      StepArgs st;
      st.pa = pa;
      st.pa.b0 = b1;
      st.pa.bw = bw1;
      st.pa.ErrT = err_of(b + 1);
      st.Eprev = s_end ? err_of(b - b % gb) : err_of(b);
      st.kprev = b1 - k0;
      st.Uprev = U + (size_t)k0 * d + b1;
      st.Wrest = Wp + b1 + bw1;
      st.Urest = U + (size_t)k0 * d + b1 + bw1;
      st.rest = std::max(0, (s_end ? d : super_end(b)) - (b1 + bw1));
      // At a super-block's end (gb > 1) the update of the columns after the
      // next block (K = 128 gb) runs as a launch of its own: the split fp16
      // product from split_start(b) on, the fp32 tiles (four per CU instead of
      // the fused kernel's two) for the columns after the next super-block
      // when the split does not apply.
      int tail = 0;
      if (s_end && gb > 1) {
        const int c_s = split_start(b);
        if (c_s == b1) {
          // the whole update, the next block's columns included, first; the
          // next block's column loop then starts from the work copy as it is
          const int e = split3_gemm(st.Eprev, d_out, false, st.Uprev, d, st.kprev, d_out, d - b1, Wp + b1, d, true,
                                    true, 0, planes, s);
          if (e != GPTQ_OK) return e;
          st.kprev = 0;
          st.rest = 0;
        } else {
          tail = (c_s < d) ? d - c_s : std::max(0, d - std::max(super_end(b + 1), b1 + bw1));
          st.rest = std::max(0, st.rest - tail);
        }
      }
      launch_quant_step(st, gt, s);
      GPTQ_LAUNCH_CHECK();
      if (tail > 0) {
        const int c = d - tail;
        const float* Uc = U + (size_t)k0 * d + c;
        if (split3_gemm_applies(st.Eprev, d_out, false, Uc, d, st.kprev, d_out, tail)) {
          // on fp16 MFMA through split fp32 operands (about an fp32 product's error)
          const int e = split3_gemm(st.Eprev, d_out, false, Uc, d, st.kprev, d_out, tail, Wp + c, d, true, true, 0, planes, s);
          if (e != GPTQ_OK) return e;
        } else {
          gemm_f32<true>(st.Eprev, d_out, Uc, d, Wp + c, d, d_out, tail, st.kprev, -1.0f, 1.0f, 0, 0, 0, s);
          GPTQ_LAUNCH_CHECK();
        }
      }
    }
    return GPTQ_OK;
  }
  // One launch per step: block b's column loop, then its lazy update: of the
  // later columns of its super-block, or, at the super-block's end, the whole
  // super-block's update of every later column; W[:, c] -= Err * U[rows, c]
  // with Aop(m, k) = ErrT[k][m].
  for (int b = 0; b < nb; ++b) {
    const int b0 = b * kQB, bw = std::min(kQB, d - b0);
    pa.b0 = b0;
    pa.bw = bw;
    pa.ErrT = err_of(b);
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
    if (b1 >= d) break;
    const bool s_end = (b + 1) % gb == 0;
    const int k0 = s_end ? (b / gb) * gb * kQB : b0;
    const int c1 = s_end ? d : super_end(b);
    const float* E = s_end ? err_of(b - b % gb) : err_of(b);
    // at a super-block's end the columns from split_start(b) on take the
    // split fp16 product, as in the fused steps
    const int c_s = (s_end && gb > 1) ? split_start(b) : c1;
    gemm_f32<true>(E, d_out, U + (size_t)k0 * d + b1, d, Wp + b1, d, d_out, c_s - b1, b1 - k0, -1.0f, 1.0f, 0, 0,
                   0, s);
    GPTQ_LAUNCH_CHECK();
    if (c_s < c1) {
      const int e = split3_gemm(E, d_out, false, U + (size_t)k0 * d + c_s, d, b1 - k0, d_out, c1 - c_s, Wp + c_s, d,
                                true, true, 0, planes, s);
      if (e != GPTQ_OK) return e;
    }
  }
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
