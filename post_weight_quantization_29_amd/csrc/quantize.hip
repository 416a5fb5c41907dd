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

#include <utility>

namespace gptq {

constexpr int kQB = 128;          // block width (lazy batch)
constexpr int kQL = 16;           // lanes per row
constexpr int kQS = kQB / kQL;    // columns (slots) per lane
constexpr int kQRows = 16;        // rows per workgroup (4 waves x 4 rows)

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

// ---------------------------------------------------------------- helpers
// DPP on 16-lane rows.  dpp control: quad_perm 0x00-0xFF, row_ror:r = 0x120+r;
// bank k = lanes 4k..4k+3 of a row; lanes of banks left out of bank_mask keep
// `old`.
template <int CTRL, int BANKS>
GPTQ_DEV int dpp_upd(int old, int src) {
  return __builtin_amdgcn_update_dpp(old, src, CTRL, 0xF, BANKS, false);
}
template <int CTRL>
GPTQ_DEV float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// every lane of a 16-lane row reads lane P of that row: broadcast inside the
// quads, then copy bank P/4 to the opposite bank (rotate by 8) and those two
// to the remaining two (rotate by 4); either rotation direction maps the banks
// the same way
template <int P>
GPTQ_DEV float row_bcast16(float v) {
  constexpr int p = P & 3, B0 = P >> 2;
  int x = __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), p | (p << 2) | (p << 4) | (p << 6),
                                   0xF, 0xF, false);
  x = dpp_upd<0x128, (1 << (B0 ^ 2))>(x, x);
  x = dpp_upd<0x124, (1 << (B0 ^ 1)) | (1 << (B0 ^ 3))>(x, x);
  return __builtin_bit_cast(float, x);
}
template <int P>
GPTQ_DEV double row_bcast16d(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_bit_cast(uint32_t, row_bcast16<P>(__builtin_bit_cast(float, (uint32_t)b)));
  const uint32_t hi = __builtin_bit_cast(uint32_t, row_bcast16<P>(__builtin_bit_cast(float, (uint32_t)(b >> 32))));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
GPTQ_DEV float row_min16(float v) {
  v = fminf(v, dpp_f<0xB1>(v));
  v = fminf(v, dpp_f<0x4E>(v));
  v = fminf(v, dpp_f<0x124>(v));
  v = fminf(v, dpp_f<0x128>(v));
  return v;
}
GPTQ_DEV float row_max16(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x124>(v));
  v = fmaxf(v, dpp_f<0x128>(v));
  return v;
}

// min-max grid of one group: scale = (max - min)/maxq, zero = rint(-min/scale);
// a constant group a uses the range [min(a,0), max(a,0)]; all-zero -> (1, 0).
GPTQ_DEV void grid_params(float xmin, float xmax, float maxq, float& scale, float& zero) {
  if (xmax == xmin) {
    xmin = fminf(xmin, 0.0f);
    xmax = fmaxf(xmax, 0.0f);
  }
  if (xmax == xmin) {
    scale = 1.0f;
    zero = 0.0f;
    return;
  }
  scale = (xmax - xmin) / maxq;
  zero = rintf(-xmin / scale);
}

// ---------------------------------------------------------------- panel
struct PanelArgs {
  float* Wp;            // [d_out x d] fp32 work copy, processing order
  const float* U;       // [d x d]
  const int* perm;
  uint8_t* codes;       // [d_out x d], original order
  float* Q;             // nullable
  float* scales;        // [d_out x ng]
  int* zeros;
  float* ErrT;          // [128 x d_out]
  int d_out, d, b0, bw, G, ng;
  int sym;
  float maxq;
};

// 16 rows per workgroup, 16 lanes per row (lane q holds the block's columns
// 16t+q, t = 0..7).  Every column step is instantiated separately (template
// fold over the 128 columns), so the row slice stays in registers with
// compile-time indices.  GT > 0: groups of GT columns inside the block (group
// starts known at compile time); GT == 0: groups of G >= 128 columns, which
// can only start at the block's first column.
template <int GT>
__global__ __launch_bounds__(256) void panel_kernel(PanelArgs a) {
  __shared__ float4 sU4[kQB][kQS / 4][kQL];   // sU4[j][t/4][q] = U[b0+j][b0+16t+q], t..t+3
  __shared__ double sInv[kQB];
  __shared__ int sPerm[kQB];

  const int tid = threadIdx.x;
  float* sU = reinterpret_cast<float*>(&sU4[0][0][0]);
  // U's diagonal block, strict upper part (zero on and below the diagonal):
  // 16 float4 loads in flight per thread
  {
    // 16-byte loads when every U row starts 16-byte aligned
    const bool vec = (a.d % 4 == 0) && (reinterpret_cast<uintptr_t>(a.U) % 16 == 0);
    float4 v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = u * 256 + tid;              // float4 index: row j, columns 4m .. 4m+3
      const int j = e >> 5, c = 4 * (e & 31);
      v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (j < a.bw && c + 3 > j) {
        const float* src = a.U + (size_t)(a.b0 + j) * a.d + a.b0 + c;
        if (vec && c + 3 < a.bw) {
          v[u] = *reinterpret_cast<const float4*>(src);
        } else {
          if (c + 3 < a.bw) v[u].w = src[3];
          if (c + 0 < a.bw) v[u].x = src[0];
          if (c + 1 < a.bw) v[u].y = src[1];
          if (c + 2 < a.bw) v[u].z = src[2];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = u * 256 + tid;
      const int j = e >> 5, c = 4 * (e & 31);
      const float vv[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int cc = c + k;
        const int t = cc >> 4;
        sU[((j * (kQS / 4) + (t >> 2)) * kQL + (cc & 15)) * 4 + (t & 3)] = (cc > j) ? vv[k] : 0.0f;
      }
    }
  }
  for (int j = tid; j < kQB; j += 256) {
    sInv[j] = (j < a.bw) ? 1.0 / (double)a.U[(size_t)(a.b0 + j) * a.d + a.b0 + j] : 0.0;
    sPerm[j] = (j < a.bw) ? a.perm[a.b0 + j] : 0;
  }
  __syncthreads();

  const int q = tid & 15;
  const int row = blockIdx.x * kQRows + (tid >> 4);
  const bool rv = row < a.d_out;
  const int rowc = rv ? row : 0;     // clamped row for loads; stores are masked
  const float* wrow = a.Wp + (size_t)rowc * a.d + a.b0;
  const int bw = a.bw;

  // The block's running weights are kept in fp64: its 127 in-block updates
  // are where fp32 rounding would move near-ties to the other side.
  double w[kQS];
#pragma unroll
  for (int t = 0; t < kQS; ++t) w[t] = (kQL * t + q < bw) ? (double)wrow[kQL * t + q] : 0.0;

  float scale = 1.0f, zero = 0.0f, rscale = 1.0f;
  if (GT == 0 && a.b0 % a.G != 0) {
    // a group wider than the block started in an earlier block: continue with
    // the parameters that launch stored
    scale = a.scales[(size_t)rowc * a.ng + a.b0 / a.G];
    zero = (float)a.zeros[(size_t)rowc * a.ng + a.b0 / a.G];
    rscale = 1.0f / scale;
  }
  // results of the lane's own columns, stored once at the end
  float eown[kQS], qown[kQS];
  uint32_t cown[kQS / 4];
#pragma unroll
  for (int t = 0; t < kQS / 4; ++t) cown[t] = 0u;

  auto group_start = [&]<int J>() {
    constexpr int I = J / kQL;
    float mn = INFINITY, mx = -INFINITY;
    if constexpr (GT >= kQL) {
      // slots I .. I + GT/16 - 1 hold the group's columns J .. J + GT - 1
#pragma unroll
      for (int t = I; t < I + GT / kQL; ++t) {
        if (kQL * t + q < bw) {
          mn = fminf(mn, (float)w[t]);
          mx = fmaxf(mx, (float)w[t]);
        }
      }
    } else if constexpr (GT > 0) {
      // a group inside one slot: lanes J%16 .. J%16 + GT - 1
      constexpr int L0 = J % kQL;
      if (q >= L0 && q < L0 + GT && J + (q - L0) < bw) {
        mn = (float)w[I];
        mx = (float)w[I];
      }
    } else {
      // J == 0: the whole block (columns < bw), then the rest of the group
      // from the work copy, which holds every earlier block's lazy update
#pragma unroll
      for (int t = 0; t < kQS; ++t) {
        if (kQL * t + q < bw) {
          mn = fminf(mn, (float)w[t]);
          mx = fmaxf(mx, (float)w[t]);
        }
      }
      const int gend = min(a.b0 + a.G, a.d);
      const float* wr = a.Wp + (size_t)rowc * a.d;
      for (int cg = a.b0 + bw + q; cg < gend; cg += kQL) {
        const float v = wr[cg];
        mn = fminf(mn, v);
        mx = fmaxf(mx, v);
      }
    }
    mn = row_min16(mn);
    mx = row_max16(mx);
    if (a.sym) {
      // symmetric: [-m, m], the middle code is zero
      const float m = fmaxf(fabsf(mn), fabsf(mx));
      scale = (m == 0.0f) ? 1.0f : (m + m) / a.maxq;
      zero = 0.5f * (a.maxq + 1.0f);
    } else {
      grid_params(mn, mx, a.maxq, scale, zero);
    }
    rscale = 1.0f / scale;
    const int gi = (GT > 0) ? (a.b0 + J) / GT : a.b0 / a.G;
    if (rv && q == 0) {
      a.scales[(size_t)row * a.ng + gi] = scale;
      a.zeros[(size_t)row * a.ng + gi] = (int)zero;
    }
  };

  auto step = [&]<int J>() {
    constexpr int I = J / kQL, P = J % kQL;
    if (J >= bw) return;
    if constexpr (GT > 0) {
      if constexpr (J % GT == 0) group_start.template operator()<J>();
    } else {
      if constexpr (J == 0) {
        if (a.b0 % a.G == 0) group_start.template operator()<0>();
      }
    }
    const double wj = row_bcast16d<P>(w[I]);
    // the code is decided in fp32: correctly rounded fp32(wj)/scale from the
    // reciprocal (one residual correction)
    const float wf = (float)wj;
    const float t0 = wf * rscale;
    const float res = fmaf(-t0, scale, wf);
    const float tq = fmaf(res, rscale, t0);
    const float c = fminf(fmaxf(rintf(tq) + zero, 0.0f), a.maxq);
    const double qv = (double)scale * (double)(c - zero);    // exact
    const double e = (wj - qv) * sInv[J];
    if (q == P) {
      eown[I] = (float)e;
      qown[I] = (float)qv;
      cown[I >> 2] |= (uint32_t)c << (8 * (I & 3));
    }
    // w[t] -= e * U[J][16t+q] for the later columns of the block (slots t >= I;
    // entries at columns <= J are retired, and U is zero there)
#pragma unroll
    for (int t = (I & ~3); t < kQS; t += 4) {
      const float4 u4 = sU4[J][t >> 2][q];
      if (t + 0 >= I) w[t + 0] = fma(-e, (double)u4.x, w[t + 0]);
      if (t + 1 >= I) w[t + 1] = fma(-e, (double)u4.y, w[t + 1]);
      if (t + 2 >= I) w[t + 2] = fma(-e, (double)u4.z, w[t + 2]);
      if (t + 3 >= I) w[t + 3] = fma(-e, (double)u4.w, w[t + 3]);
    }
  };
  [&]<int... Js>(std::integer_sequence<int, Js...>) {
    (step.template operator()<Js>(), ...);
  }(std::make_integer_sequence<int, kQB>{});

  if (!rv) return;
  uint8_t* crow = a.codes + (size_t)row * a.d;
  float* qrow = a.Q ? a.Q + (size_t)row * a.d : nullptr;
#pragma unroll
  for (int t = 0; t < kQS; ++t) {
    const int j = kQL * t + q;
    if (j < bw) {
      const int oc = sPerm[j];
      crow[oc] = (uint8_t)(cown[t >> 2] >> (8 * (t & 3)));
      if (qrow) qrow[oc] = qown[t];
      a.ErrT[(size_t)j * a.d_out + row] = eown[t];
    }
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
