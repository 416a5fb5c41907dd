// Column loop of one 128-column block (GPTQ practice page m.lqnn.cn/news/117696,
// section 2.1: quantize one weight, move the not-yet-quantized ones along the
// inverse-Hessian column; section 3.3: group_size consecutive columns share a
// scale and zero point; tutorial page "大模型压缩量化技术：GPTQ 与 AWQ 原理详解 +
// Python 实战教程", section 二: min-max uniform grid), shared by the per-block
// panel kernel and the fused block-step kernel.
#pragma once
#include "common.h"

#include <utility>

namespace gptq {

constexpr int kQB = 128;          // block width (lazy batch)
constexpr int kQL = 16;           // lanes per row
constexpr int kQS = kQB / kQL;    // columns (slots) per lane
constexpr int kQRows = 16;        // rows per workgroup (4 waves x 4 rows)

// ---------------------------------------------------------------- helpers
// DPP on 16-lane rows.  dpp control: quad_perm 0x00-0xFF, row_ror:r = 0x120+r;
// bank k = lanes 4k..4k+3 of a row; lanes of banks left out of bank_mask keep
// `old`.
template <int CTRL, int BANKS>
GPTQ_DEV int dpp_upd(int old, int src) {
  return __builtin_amdgcn_update_dpp(old, src, CTRL, 0xF, BANKS, false);
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
// the same DPP pattern applied to both halves of a double
template <int CTRL>
GPTQ_DEV double dpp_d(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)b, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
// min / max over the 16 lanes of a row (butterfly: swap pairs, swap halves of
// quads, then rotate the row by 4 and by 8)
GPTQ_DEV double row_min16d(double v) {
  v = fmin(v, dpp_d<0xB1>(v));
  v = fmin(v, dpp_d<0x4E>(v));
  v = fmin(v, dpp_d<0x124>(v));
  v = fmin(v, dpp_d<0x128>(v));
  return v;
}
GPTQ_DEV double row_max16d(double v) {
  v = fmax(v, dpp_d<0xB1>(v));
  v = fmax(v, dpp_d<0x4E>(v));
  v = fmax(v, dpp_d<0x124>(v));
  v = fmax(v, dpp_d<0x128>(v));
  return v;
}

// min-max grid of one group, in fp64 with IEEE division: scale =
// (max - min)/maxq, zero = rint(-min/scale); a constant group a uses the range
// [min(a,0), max(a,0)]; all-zero -> (1, 0).
GPTQ_DEV void grid_params(double xmin, double xmax, double maxq, double& scale, double& zero) {
  if (xmax == xmin) {
    xmin = fmin(xmin, 0.0);
    xmax = fmax(xmax, 0.0);
  }
  if (xmax == xmin) {
    scale = 1.0;
    zero = 0.0;
    return;
  }
  scale = (xmax - xmin) / maxq;
  zero = rint(-xmin / scale);
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
  double* gscale;       // [d_out] fp64 scale of the group in progress (groups wider than the block)
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
// U's diagonal block in LDS, strict upper part, as float4 slot groups: lane q
// of row j reads U[b0+j][b0+16t+q] for slots t = 4g .. 4g+3 of group g.  Row j
// only needs the slots t >= j/16, so group 0 (columns < 64) is kept for rows
// j < 64 alone: group 1 of every row at [j][q], then group 0 of rows < 64 at
// kQB*kQL + [j][q] (48 KB instead of 64).
constexpr int kUPacked = (kQB + kQB / 2) * kQL;   // float4s
static_assert(kQS == 8, "two float4 slot groups per lane and row");
GPTQ_DEV int upk(int j, int g, int q) { return (g ? 0 : kQB * kQL) + j * kQL + q; }

// The column loop of the 16 rows of row block rb.  LDS: sU (kUPacked float4),
// sInv (kQB doubles), sPerm (kQB ints).  PRE: the caller has put into
// sPre[r][c] (pitch kQB + 4) the product the block's columns still owe the
// previous block's update, (Err_prev * U[prev, block])[row r][column c],
// computed like the trailing GEMM computes it, followed by a barrier; the
// running weights then start from the work copy minus it, rounded to fp32 as
// the GEMM would store it.  sPre may share LDS with sU: it is read before sU
// is written.
template <int GT, bool PRE>
GPTQ_DEV void panel_rows(const PanelArgs& a, int rb, float4* sU4, double* sInv, int* sPerm,
                         const float* sPre) {
  const int tid = threadIdx.x;
  float* sU = reinterpret_cast<float*>(sU4);
  // U's diagonal block, strict upper part (zero on and below the diagonal):
  // 16 float4 loads in flight per thread, written to LDS once the running
  // weights are set up
  // 16-byte loads when every U row starts 16-byte aligned
  const bool vec = (a.d % 4 == 0) && (reinterpret_cast<uintptr_t>(a.U) % 16 == 0);
  float4 v[16];
  {
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
  }
  for (int j = tid; j < kQB; j += 256) {
    sInv[j] = (j < a.bw) ? 1.0 / (double)a.U[(size_t)(a.b0 + j) * a.d + a.b0 + j] : 0.0;
    sPerm[j] = (j < a.bw) ? a.perm[a.b0 + j] : 0;
  }

  const int q = tid & 15;
  const int row = rb * kQRows + (tid >> 4);
  const bool rv = row < a.d_out;
  const int rowc = rv ? row : 0;     // clamped row for loads; stores are masked
  const float* wrow = a.Wp + (size_t)rowc * a.d + a.b0;
  const int bw = a.bw;

  // The block's running weights are kept in fp64: its 127 in-block updates
  // are where fp32 rounding would move near-ties to the other side.
  double w[kQS];
#pragma unroll
  for (int t = 0; t < kQS; ++t) {
    float x = (kQL * t + q < bw) ? wrow[kQL * t + q] : 0.0f;
    if constexpr (PRE) x = x - sPre[(tid >> 4) * (kQB + 4) + kQL * t + q];
    w[t] = (double)x;
  }
  if constexpr (PRE) __syncthreads();        // sPre is read: sU may overwrite it
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int e = u * 256 + tid;
    const int j = e >> 5, c = 4 * (e & 31);
    const float vv[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int cc = c + k;
      const int t = cc >> 4;
      if ((t >> 2) == 1 || j < kQB / 2) sU[upk(j, t >> 2, cc & 15) * 4 + (t & 3)] = (cc > j) ? vv[k] : 0.0f;
    }
  }
  __syncthreads();

  // the grid and every integer decision are taken in fp64, like the rest of
  // the column loop
  double scale = 1.0, zero = 0.0, rscale = 1.0;
  if (GT == 0 && a.b0 % a.G != 0) {
    // a group wider than the block started in an earlier block: continue with
    // the parameters that launch kept (the fp64 scale, the integer zero point)
    scale = a.gscale[rowc];
    zero = (double)a.zeros[(size_t)rowc * a.ng + a.b0 / a.G];
    rscale = 1.0 / scale;
  }
  // results of the lane's own columns, stored once at the end
  float eown[kQS], qown[kQS];
  uint32_t cown[kQS / 4];
#pragma unroll
  for (int t = 0; t < kQS / 4; ++t) cown[t] = 0u;

  auto group_start = [&]<int J>() {
    constexpr int I = J / kQL;
    double mn = INFINITY, mx = -INFINITY;
    if constexpr (GT >= kQL) {
      // slots I .. I + GT/16 - 1 hold the group's columns J .. J + GT - 1
#pragma unroll
      for (int t = I; t < I + GT / kQL; ++t) {
        if (kQL * t + q < bw) {
          mn = fmin(mn, w[t]);
          mx = fmax(mx, w[t]);
        }
      }
    } else if constexpr (GT > 0) {
      // a group inside one slot: lanes J%16 .. J%16 + GT - 1
      constexpr int L0 = J % kQL;
      if (q >= L0 && q < L0 + GT && J + (q - L0) < bw) {
        mn = w[I];
        mx = w[I];
      }
    } else {
      // J == 0: the whole block (columns < bw), then the rest of the group
      // from the work copy, which holds every earlier block's lazy update
#pragma unroll
      for (int t = 0; t < kQS; ++t) {
        if (kQL * t + q < bw) {
          mn = fmin(mn, w[t]);
          mx = fmax(mx, w[t]);
        }
      }
      const int gend = min(a.b0 + a.G, a.d);
      const float* wr = a.Wp + (size_t)rowc * a.d;
      for (int cg = a.b0 + bw + q; cg < gend; cg += kQL) {
        const double v = (double)wr[cg];
        mn = fmin(mn, v);
        mx = fmax(mx, v);
      }
    }
    mn = row_min16d(mn);
    mx = row_max16d(mx);
    if (a.sym) {
      // symmetric: [-m, m], the middle code is zero
      const double m = fmax(fabs(mn), fabs(mx));
      scale = (m == 0.0) ? 1.0 : (m + m) / (double)a.maxq;
      zero = 0.5 * ((double)a.maxq + 1.0);
    } else {
      grid_params(mn, mx, (double)a.maxq, scale, zero);
    }
    rscale = 1.0 / scale;
    const int gi = (GT > 0) ? (a.b0 + J) / (GT > 0 ? GT : 1) : a.b0 / a.G;
    if (rv && q == 0) {
      a.scales[(size_t)row * a.ng + gi] = (float)scale;
      a.zeros[(size_t)row * a.ng + gi] = (int)zero;
      if constexpr (GT == 0) a.gscale[row] = scale;
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
    // code = clamp(rint(wj/scale) + zero, 0, maxq) with the quotient formed from
    // the reciprocal plus one residual correction (the correctly rounded
    // quotient for every divisor whose significand is not all ones)
    const double t0 = wj * rscale;
    const double res = fma(-t0, scale, wj);
    const double tq = fma(res, rscale, t0);
    const double c = fmin(fmax(rint(tq) + zero, 0.0), (double)a.maxq);
    const double qv = scale * (c - zero);
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
      const float4 u4 = sU4[upk(J, t >> 2, q)];        // group 0 only while J < 64
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

template <int GT>
__global__ __launch_bounds__(256) void panel_kernel(PanelArgs a) {
  __shared__ float4 sU4[kUPacked];            // U's diagonal block (see upk)
  __shared__ double sInv[kQB];
  __shared__ int sPerm[kQB];
  panel_rows<GT, false>(a, (int)blockIdx.x, sU4, sInv, sPerm, nullptr);
}

// ---------------------------------------------------------------- fused block step
// One launch per block b >= 0 (b + 1 < blocks): the column loop of block b + 1,
// whose workgroups first apply the update block b + 1 still owes (block b's,
// or at a super-block's end the whole super-block's) to their own 16 rows of
// its columns (the products kept in LDS, never stored), beside the trailing
// update of later columns by the same Err rows.  The two parts share no data,
// so they run side by side without waiting on each other.
struct StepArgs {
  PanelArgs pa;          // column loop of block b + 1 (pa.b0, pa.bw, pa.ErrT: its Err buffer)
  const float* Eprev;    // Err rows owed, [kprev x d_out]
  const float* Uprev;    // the matching U rows from block b + 1's first column (row pitch d)
  float* Wrest;          // work copy from the first column of the trailing update (row pitch d)
  const float* Urest;    // the same U rows from that column (row pitch d)
  int rest;              // columns of the trailing update
  int kprev;             // the contraction length (a multiple of kQB)
};

// Whether the fused steps apply: groups of gt columns inside the block (gt > 0),
// more than one block, and every operand row 16-byte aligned for the kernel's
// vector loads (U 16-byte aligned, d and d_out multiples of 4; the workspace
// buffers are 256-byte aligned).
inline bool quant_step_applies(int d_out, int d, const float* U, int gt) {
  return gt > 0 && d > kQB && d % 4 == 0 && d_out % 4 == 0 && (reinterpret_cast<uintptr_t>(U) & 15) == 0;
}

// Launches one step (the caller has checked quant_step_applies).
void launch_quant_step(const StepArgs& f, int gt, hipStream_t s);

}  // namespace gptq
