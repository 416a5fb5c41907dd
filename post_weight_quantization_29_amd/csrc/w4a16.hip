// y = x W^T on the packed 4-bit layer (GPTQ practice page m.lqnn.cn/news/117696,
// section 4.3: at inference the 4-bit weights are dequantized to a 16-bit type
// and then multiplied; what the 4 bits save is the bytes moved, so at small
// batch this product is bound by HBM).
//
// RPW output rows per wave (1 for one or two activation rows, else 4; long
// rows with one or two activation rows take w4a16_shared_x_kernel below, which
// loads each activation chunk once per workgroup): each lane streams 16-byte groups
// of the rows' packed codes (8 codes per word, the gptq_pack_int4 layout), forms each weight
// as the fp32 product scale * (code - zero) (the codes made exact floats with
// one byte conversion each), rounds pairs of them to the
// activation's 16-bit type with one packed conversion, and multiplies them
// with up to 8 activation rows at a time with the 2-term dot instruction
// (fp32 accumulation); a wave reduction finishes each dot product.  Each
// activation chunk is loaded once per wave and serves all RPW rows.
#include "common.h"

namespace gptq {

constexpr int kWRows = 8;   // activation rows per pass over the weights

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Per activation type: a pair of dequantized fp32 weights rounded (ties to
// even) into the type's packed pair, and the 2-term dot product with fp32
// accumulation.
template <typename T> struct Act;
typedef float f32x2_t __attribute__((ext_vector_type(2)));

template <> struct Act<__bf16> {
  typedef bf16x2_t v2;
  static GPTQ_DEV v2 pack(float a, float b) {
    // one v_cvt_pk_bf16_f32 (round to nearest even) for the pair
    const f32x2_t f = {a, b};
    return __builtin_convertvector(f, v2);
  }
  static GPTQ_DEV float dot2(uint32_t x, v2 w, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2, x), w, acc, false);
  }
};
template <> struct Act<_Float16> {
  typedef f16x2_t v2;
  static GPTQ_DEV v2 pack(float a, float b) {
    v2 r;
    r[0] = (_Float16)a;
    r[1] = (_Float16)b;
    return r;
  }
  static GPTQ_DEV float dot2(uint32_t x, v2 w, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(v2, x), w, acc, false);
  }
};

template <typename TY> GPTQ_DEV TY out_cast(float v);
template <> GPTQ_DEV float out_cast<float>(float v) { return v; }
template <> GPTQ_DEV __bf16 out_cast<__bf16>(float v) { return (__bf16)v; }
template <> GPTQ_DEV _Float16 out_cast<_Float16>(float v) { return (_Float16)v; }

// The eight codes of word p as exact floats: the even codes sit in the bytes
// of p & 0x0F0F0F0F and the odd ones in those of (p >> 4) & 0x0F0F0F0F, and
// each byte converts with one v_cvt_f32_ubyteN (the masked words are kept
// opaque so that the compiler does not fold the masks back into per-code
// bit-field extracts).
GPTQ_DEV void word_codes(uint32_t p, float (&c)[8]) {
  uint32_t lo = p & 0x0F0F0F0Fu, hi = (p >> 4) & 0x0F0F0F0Fu;
  asm volatile("" : "+v"(lo), "+v"(hi));
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    c[2 * b] = (float)((lo >> (8 * b)) & 0xFFu);
    c[2 * b + 1] = (float)((hi >> (8 * b)) & 0xFFu);
  }
}

// The eight weights of word p, in packed pairs: RN(scale * (code - zero)) in
// fp32 (code - zero is exact), then rounded to the 16-bit type.  NATURAL: one
// group for the word (scale s, zero zf as a float); otherwise a group per code
// from g_idx.
template <typename T, bool NATURAL>
GPTQ_DEV void dequant_word(uint32_t p, int c0, float s, float zf, const float* srow, const int32_t* zrow,
                           const int32_t* g_idx, int ng, typename Act<T>::v2 (&w)[4]) {
  float c[8], v[8];
  word_codes(p, c);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (NATURAL) {
      v[k] = s * (c[k] - zf);
    } else {
      const int g = min(max(g_idx[c0 + k], 0), ng - 1);
      v[k] = srow[g] * (c[k] - (float)zrow[g]);
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = Act<T>::pack(v[2 * j], v[2 * j + 1]);
}

// NATURAL: column c is in group c / G (G a multiple of 8, so a word's eight
// codes share a group); otherwise group g_idx[c], clamped to [0, ng).
// WPL words (8 codes each) per lane per step: 4 when the rows allow 16-byte
// loads, else 1.  Wave w of block b takes output rows RPW(4b + w) .. +RPW-1;
// the step's weights of all RPW rows are dequantized into registers first,
// then each activation row's chunk is loaded once and dotted with all of them.
template <typename T, typename TY, bool NATURAL, int WPL, int RPW>
__global__ __launch_bounds__(256) void w4a16_kernel(const uint16_t* __restrict__ X, int64_t m, int d_in,
                                                    const uint32_t* __restrict__ packed,
                                                    const float* __restrict__ scales,
                                                    const int32_t* __restrict__ zeros,
                                                    const int32_t* __restrict__ g_idx, int G, int ng,
                                                    int d_out, TY* __restrict__ Y) {
  typedef typename Act<T>::v2 v2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r0 = (blockIdx.x * 4 + wave) * RPW;
  if (r0 >= d_out) return;
  const int nw = d_in >> 3;
  const float invG = 1.0f / (float)G;
  const bool gshared = (G % (8 * WPL)) == 0;
  for (int64_t m0 = 0; m0 < m; m0 += kWRows) {
    const int mc = (int)min<int64_t>(kWRows, m - m0);
    const uint16_t* xb = X + m0 * d_in;
    float acc[RPW][kWRows];
#pragma unroll
    for (int j = 0; j < RPW; ++j)
#pragma unroll
      for (int i = 0; i < kWRows; ++i) acc[j][i] = 0.0f;
    for (int q = lane * WPL; q < nw; q += 64 * WPL) {
      v2 w[RPW][WPL][4];
#pragma unroll
      for (int j = 0; j < RPW; ++j) {
        const int r = min(r0 + j, d_out - 1);       // rows past the end: computed, not stored
        const uint32_t* prow = packed + (size_t)r * nw;
        uint32_t pw[WPL];
        if (WPL == 4) {
          const uint4 p4 = *reinterpret_cast<const uint4*>(prow + q);
          pw[0] = p4.x; pw[WPL > 1 ? 1 : 0] = p4.y; pw[WPL > 2 ? 2 : 0] = p4.z; pw[WPL > 3 ? 3 : 0] = p4.w;
        } else {
          pw[0] = prow[q];
        }
        const float* srow = scales + (size_t)r * ng;
        const int32_t* zrow = zeros + (size_t)r * ng;
        float sc = 0.0f, zf = 0.0f;
#pragma unroll
        for (int u = 0; u < WPL; ++u) {
          const int c0 = (q + u) * 8;
          // the WPL words of a step are 8*WPL consecutive columns from a
          // multiple of 8*WPL, so they share a group when G is a multiple of it
          if (NATURAL && (u == 0 || !gshared)) {
            int g = (int)((float)c0 * invG);      // exact quotient after one correction
            if (g * G > c0) --g;
            if ((g + 1) * G <= c0) ++g;
            sc = srow[g];
            zf = (float)zrow[g];
          }
          dequant_word<T, NATURAL>(pw[u], c0, sc, zf, srow, zrow, g_idx, ng, w[j][u]);
        }
      }
#pragma unroll
      for (int i = 0; i < kWRows; ++i) {
        if (i < mc) {
#pragma unroll
          for (int u = 0; u < WPL; ++u) {
            const uint4 xv = *reinterpret_cast<const uint4*>(xb + (size_t)i * d_in + (q + u) * 8);
#pragma unroll
            for (int j = 0; j < RPW; ++j) {
              float a = acc[j][i];
              a = Act<T>::dot2(xv.x, w[j][u][0], a);
              a = Act<T>::dot2(xv.y, w[j][u][1], a);
              a = Act<T>::dot2(xv.z, w[j][u][2], a);
              a = Act<T>::dot2(xv.w, w[j][u][3], a);
              acc[j][i] = a;
            }
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < RPW; ++j)
#pragma unroll
      for (int i = 0; i < kWRows; ++i) {
        float v = acc[j][i];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
        if (lane == 0 && i < mc && r0 + j < d_out) Y[(size_t)(m0 + i) * d_out + r0 + j] = out_cast<TY>(v);
      }
  }
}

// One or two activation rows over long rows: the four waves of a workgroup
// (four output rows) walk the same columns, so each step's activation chunk
// (256 words = 2048 columns per activation row) is loaded once per workgroup
// into LDS (double buffered, one barrier per step) instead of once per wave;
// the weights are formed and dotted exactly as above.  With a group per
// column (g_idx, the act-order layout, NATURAL false) each wave first copies
// its row's (scale, zero) pairs into LDS (dynamic, ng pairs per wave), so a
// code's group costs one LDS read instead of two scattered global ones, and
// g_idx is read 16 bytes at a time (four columns).
template <typename T, typename TY, bool NATURAL>
__global__ __launch_bounds__(256) void w4a16_shared_x_kernel(const uint16_t* __restrict__ X, int m, int d_in,
                                                             const uint32_t* __restrict__ packed,
                                                             const float* __restrict__ scales,
                                                             const int32_t* __restrict__ zeros,
                                                             const int32_t* __restrict__ g_idx, int G,
                                                             int ng, int d_out, TY* __restrict__ Y) {
  typedef typename Act<T>::v2 v2;
  __shared__ uint4 sX[2][2][256];
  extern __shared__ float2 sGrp[];             // [4][ng] (scale, zero) when !NATURAL
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r0 = blockIdx.x * 4 + wave;
  const int r = min(r0, d_out - 1);            // rows past the end: computed, not stored
  const int nw = d_in >> 3;
  const float invG = 1.0f / (float)G;
  const bool gshared = (G % 32) == 0;
  const uint32_t* prow = packed + (size_t)r * nw;
  const float* srow = scales + (size_t)r * ng;
  const int32_t* zrow = zeros + (size_t)r * ng;
  // the wave's (scale, zero) table; its writes are ordered before every read
  // by the first step's barrier
  float2* sg = sGrp + (NATURAL ? 0 : wave * ng);
  if constexpr (!NATURAL) {
    for (int g = lane; g < ng; g += 64) sg[g] = make_float2(srow[g], (float)zrow[g]);
  }
  float acc[2] = {0.0f, 0.0f};
  int buf = 0;
  for (int q0 = 0; q0 < nw; q0 += 256) {
    const int q = q0 + 4 * lane;
    uint4 p4 = make_uint4(0u, 0u, 0u, 0u);
    if (q < nw) p4 = *reinterpret_cast<const uint4*>(prow + q);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (i < m) {
        const int qx = q0 + tid;
        sX[buf][i][tid] = (qx < nw) ? *reinterpret_cast<const uint4*>(X + (size_t)i * d_in + (size_t)qx * 8)
                                    : make_uint4(0u, 0u, 0u, 0u);
      }
    }
    // also orders this buffer's writes after the reads two steps back
    __syncthreads();
    if (q < nw) {
      const uint32_t pw[4] = {p4.x, p4.y, p4.z, p4.w};
      v2 w[4][4];
      if constexpr (NATURAL) {
        float sc = 0.0f, zf = 0.0f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int c0 = (q + u) * 8;
          if (u == 0 || !gshared) {
            int g = (int)((float)c0 * invG);    // exact quotient after one correction
            if (g * G > c0) --g;
            if ((g + 1) * G <= c0) ++g;
            sc = srow[g];
            zf = (float)zrow[g];
          }
          dequant_word<T, true>(pw[u], c0, sc, zf, srow, zrow, nullptr, ng, w[u]);
        }
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          // the same weights as dequant_word's per-code form, the group's
          // (scale, zero) from the wave's table
          const int c0 = (q + u) * 8;
          const int4 ga = *reinterpret_cast<const int4*>(g_idx + c0);
          const int4 gb = *reinterpret_cast<const int4*>(g_idx + c0 + 4);
          const int gk[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
          float c[8], v[8];
          word_codes(pw[u], c);
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const float2 sz = sg[min(max(gk[k], 0), ng - 1)];
            v[k] = sz.x * (c[k] - sz.y);
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) w[u][j] = Act<T>::pack(v[2 * j], v[2 * j + 1]);
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (i < m) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const uint4 xv = sX[buf][i][4 * lane + u];
            float a = acc[i];
            a = Act<T>::dot2(xv.x, w[u][0], a);
            a = Act<T>::dot2(xv.y, w[u][1], a);
            a = Act<T>::dot2(xv.z, w[u][2], a);
            a = Act<T>::dot2(xv.w, w[u][3], a);
            acc[i] = a;
          }
        }
      }
    }
    buf ^= 1;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    float v = acc[i];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0 && i < m && r0 < d_out) Y[(size_t)i * d_out + r0] = out_cast<TY>(v);
  }
}

// ---------------------------------------------------------------- many activation rows
// The same product as a tiled MFMA GEMM, for batches of activation rows where
// the weights are worth dequantizing once per 128 rows of X: a workgroup
// takes 128 rows of X by 128 rows of W; per 128-wide k chunk it copies the X
// tile to LDS, dequantizes the W tile (the same exact 16-bit weights as above)
// into LDS, and four waves (64 x 64 each) run v_mfma_f32_32x32x16 on them
// (A lane l = X[l%32][8(l/32) .. +7], B lane l = W[l%32][8(l/32) .. +7] along
// k; both tiles k-contiguous, rows padded to 136 elements).  fp32 accumulation.
constexpr int kGM = 128, kGN = 128, kGKc = 128, kGPitch = kGKc + 8;
constexpr int kGXv = kGM * kGKc / 8 / 256;     // 16-byte X loads per thread per chunk
constexpr int kGWw = kGKc / 16;                // code words per thread per chunk (2 threads per W row)

template <typename T> struct Mfma16;
template <> struct Mfma16<__bf16> {
  typedef __bf16 v8 __attribute__((ext_vector_type(8)));
  static GPTQ_DEV f32x16_t run(v8 a, v8 b, f32x16_t c) { return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0); }
};
template <> struct Mfma16<_Float16> {
  typedef _Float16 v8 __attribute__((ext_vector_type(8)));
  static GPTQ_DEV f32x16_t run(v8 a, v8 b, f32x16_t c) { return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0); }
};

template <typename T, typename TY, bool NATURAL, bool VEC>
__global__ __launch_bounds__(256) void w4a16_mfma_kernel(const uint16_t* __restrict__ X, int64_t m, int d_in,
                                                         const uint32_t* __restrict__ packed,
                                                         const float* __restrict__ scales,
                                                         const int32_t* __restrict__ zeros,
                                                         const int32_t* __restrict__ g_idx, int G, int ng,
                                                         int d_out, TY* __restrict__ Y) {
  typedef typename Act<T>::v2 v2;
  typedef typename Mfma16<T>::v8 v8;
  __shared__ __attribute__((aligned(16))) uint16_t sX[kGM * kGPitch];
  __shared__ __attribute__((aligned(16))) uint16_t sW[kGN * kGPitch];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * kGN;
  const int64_t m0 = (int64_t)blockIdx.y * kGM;
  const int nw = d_in >> 3;
  const float invG = 1.0f / (float)G;
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // this thread's W tile part: row wr, words kGWw wh .. + kGWw - 1 of the chunk
  const int wr = tid >> 1, wh = tid & 1;
  const int wrow = min(n0 + wr, d_out - 1);            // rows past the end: computed, not stored
  const uint32_t* prow = packed + (size_t)wrow * nw;
  const float* srow = scales + (size_t)wrow * ng;
  const int32_t* zrow = zeros + (size_t)wrow * ng;

  // chunk k0's global data in registers: X (rows tid/8 + 32i, 8 elements at
  // k0 + 8(tid%8)) and this thread's 4 code words; loaded one chunk ahead so
  // that their latency overlaps the MFMAs of the current chunk
  // X element columns per row of the chunk covered by one thread's loads
  constexpr int kXT = kGKc / 8;                // threads per X row (16 bytes each)
  uint4 xr[kGXv];
  uint32_t pw[kGWw];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < kGXv; ++i) {
      const int r = tid / kXT + (256 / kXT) * i, kk = k0 + 8 * (tid % kXT);
      xr[i] = (m0 + r < m && kk < d_in) ? *reinterpret_cast<const uint4*>(X + (m0 + r) * (int64_t)d_in + kk)
                                        : make_uint4(0u, 0u, 0u, 0u);
    }
    const int q0 = (k0 >> 3) + kGWw * wh;
#pragma unroll
    for (int u4 = 0; u4 < kGWw; u4 += 4) {
      if (VEC && q0 + u4 + 3 < nw) {
        const uint4 p4 = *reinterpret_cast<const uint4*>(prow + q0 + u4);
        pw[u4] = p4.x; pw[u4 + 1] = p4.y; pw[u4 + 2] = p4.z; pw[u4 + 3] = p4.w;
      } else {
#pragma unroll
        for (int u = u4; u < u4 + 4; ++u) pw[u] = (q0 + u < nw) ? prow[q0 + u] : 0u;
      }
    }
  };
  gload(0);
  for (int k0 = 0; k0 < d_in; k0 += kGKc) {
#pragma unroll
    for (int i = 0; i < kGXv; ++i)
      *reinterpret_cast<uint4*>(sX + (tid / kXT + (256 / kXT) * i) * kGPitch + 8 * (tid % kXT)) = xr[i];
    // W tile: dequantize this thread's words of row wr
    {
      const int q0 = (k0 >> 3) + kGWw * wh;
#pragma unroll
      for (int u = 0; u < kGWw; ++u) {
        v2 w[4];
        const int c0 = (q0 + u) * 8;
        if (q0 + u < nw) {
          float sc = 0.0f, zf = 0.0f;
          if (NATURAL) {
            int g = (int)((float)c0 * invG);
            if (g * G > c0) --g;
            if ((g + 1) * G <= c0) ++g;
            sc = srow[g];
            zf = (float)zrow[g];
          }
          dequant_word<T, NATURAL>(pw[u], c0, sc, zf, srow, zrow, g_idx, ng, w);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = Act<T>::pack(0.0f, 0.0f);
        }
        uint4 o;
        o.x = __builtin_bit_cast(uint32_t, w[0]);
        o.y = __builtin_bit_cast(uint32_t, w[1]);
        o.z = __builtin_bit_cast(uint32_t, w[2]);
        o.w = __builtin_bit_cast(uint32_t, w[3]);
        *reinterpret_cast<uint4*>(sW + wr * kGPitch + 8 * kGWw * wh + 8 * u) = o;
      }
    }
    __syncthreads();
    if (k0 + kGKc < d_in) gload(k0 + kGKc);
#pragma unroll
    for (int ks = 0; ks < kGKc / 16; ++ks) {
      const int kc = 16 * ks + 8 * (lane >> 5);
      v8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = __builtin_bit_cast(v8, *reinterpret_cast<const uint4*>(sX + (wm * 64 + 32 * i + (lane & 31)) * kGPitch + kc));
        b[i] = __builtin_bit_cast(v8, *reinterpret_cast<const uint4*>(sW + (wn * 64 + 32 * i + (lane & 31)) * kGPitch + kc));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = Mfma16<T>::run(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t mm = m0 + wm * 64 + 32 * i + mfma32_row(r, lane);
        const int nn = n0 + wn * 64 + 32 * j + mfma32_col(lane);
        if (mm < m && nn < d_out) Y[mm * d_out + nn] = out_cast<TY>(acc[i][j][r]);
      }
}

// activation rows from which the tiled MFMA product is used
constexpr int64_t kMfmaMinRows = 64;
// columns from which one or two activation rows are shared through LDS
constexpr int kSharedXMinCols = 8192;
// groups per row up to which a group per column (g_idx) takes the LDS
// (scale, zero) tables of w4a16_shared_x_kernel (4 x 1536 pairs = 48 KB)
constexpr int kSharedGroupsMax = 1536;

template <typename T, typename TY, int RPW>
static void launch_w4a16_rpw(const uint16_t* x, int64_t m, int d_in, const uint32_t* packed, const float* scales,
                             const int32_t* zeros, const int32_t* g_idx, int G, int ng, int d_out, TY* y,
                             hipStream_t s) {
  const unsigned grid = (unsigned)((d_out + 4 * RPW - 1) / (4 * RPW));
  // 16-byte packed loads when every row starts 16-byte aligned
  const bool vec = ((d_in / 8) % 4 == 0) && (reinterpret_cast<uintptr_t>(packed) & 15) == 0;
  if (g_idx) {
    if (vec) w4a16_kernel<T, TY, false, 4, RPW><<<grid, 256, 0, s>>>(x, m, d_in, packed, scales, zeros, g_idx, G, ng, d_out, y);
    else w4a16_kernel<T, TY, false, 1, RPW><<<grid, 256, 0, s>>>(x, m, d_in, packed, scales, zeros, g_idx, G, ng, d_out, y);
  } else {
    if (vec) w4a16_kernel<T, TY, true, 4, RPW><<<grid, 256, 0, s>>>(x, m, d_in, packed, scales, zeros, nullptr, G, ng, d_out, y);
    else w4a16_kernel<T, TY, true, 1, RPW><<<grid, 256, 0, s>>>(x, m, d_in, packed, scales, zeros, nullptr, G, ng, d_out, y);
  }
}

template <typename T, typename TY>
static void launch_w4a16(const void* X, int64_t m, int d_in, const uint32_t* packed, const float* scales,
                         const int32_t* zeros, const int32_t* g_idx, int G, int ng, int d_out, void* Y,
                         hipStream_t s) {
  const uint16_t* x = static_cast<const uint16_t*>(X);
  TY* y = static_cast<TY*>(Y);
  if (m >= kMfmaMinRows) {
    const dim3 grid((unsigned)((d_out + kGN - 1) / kGN), (unsigned)((m + kGM - 1) / kGM));
    const bool vec = ((d_in / 8) % 4 == 0) && (reinterpret_cast<uintptr_t>(packed) & 15) == 0;
    if (g_idx) {
      if (vec) w4a16_mfma_kernel<T, TY, false, true><<<grid, 256, 0, s>>>(x, m, d_in, packed, scales, zeros, g_idx, G, ng, d_out, y);
      else w4a16_mfma_kernel<T, TY, false, false><<<grid, 256, 0, s>>>(x, m, d_in, packed, scales, zeros, g_idx, G, ng, d_out, y);
    } else {
      if (vec) w4a16_mfma_kernel<T, TY, true, true><<<grid, 256, 0, s>>>(x, m, d_in, packed, scales, zeros, nullptr, G, ng, d_out, y);
      else w4a16_mfma_kernel<T, TY, true, false><<<grid, 256, 0, s>>>(x, m, d_in, packed, scales, zeros, nullptr, G, ng, d_out, y);
    }
  } else if (m <= 2) {
    // long rows with natural groups: one activation load per workgroup
    // (measured at 8192 x 28672: one row 46.8 -> 44.4 us, two rows 76 -> 58 us;
    // at 4096 columns the extra barrier does not pay)
    // (act order at 8192 x 28672: one row 410 -> 129 us with the LDS tables)
    const bool long_rows = d_in >= kSharedXMinCols && (d_in % 32) == 0 &&
                           ((reinterpret_cast<uintptr_t>(packed) | reinterpret_cast<uintptr_t>(x)) & 15) == 0;
    const unsigned grid = (unsigned)((d_out + 3) / 4);
    if (long_rows && !g_idx) {
      w4a16_shared_x_kernel<T, TY, true><<<grid, 256, 0, s>>>(x, (int)m, d_in, packed, scales, zeros, nullptr, G,
                                                              ng, d_out, y);
      return;
    }
    if (long_rows && (reinterpret_cast<uintptr_t>(g_idx) & 15) == 0 && ng <= kSharedGroupsMax) {
      w4a16_shared_x_kernel<T, TY, false><<<grid, 256, (size_t)4 * ng * sizeof(float2), s>>>(
          x, (int)m, d_in, packed, scales, zeros, g_idx, G, ng, d_out, y);
      return;
    }
    launch_w4a16_rpw<T, TY, 1>(x, m, d_in, packed, scales, zeros, g_idx, G, ng, d_out, y, s);
  } else {
    launch_w4a16_rpw<T, TY, 4>(x, m, d_in, packed, scales, zeros, g_idx, G, ng, d_out, y, s);
  }
}

}  // namespace gptq

using namespace gptq;

extern "C" int gptq_w4a16_gemm(const void* X, gptq_dtype x_dtype, int64_t m, int32_t d_in,
                               const uint32_t* packed, const float* scales, const int32_t* zeros,
                               const int32_t* g_idx, int32_t group_size, int32_t n_groups,
                               int32_t d_out, void* Y, gptq_dtype y_dtype, hipStream_t s) {
  if (!X || !packed || !scales || !zeros || !Y) return GPTQ_ERR_INVALID_ARG;
  if (m < 0 || d_in <= 0 || d_out <= 0 || (d_in % 8) != 0 || n_groups <= 0) return GPTQ_ERR_INVALID_ARG;
  if (x_dtype != GPTQ_F16 && x_dtype != GPTQ_BF16) return GPTQ_ERR_INVALID_ARG;
  if (y_dtype != GPTQ_F32 && y_dtype != GPTQ_F16 && y_dtype != GPTQ_BF16) return GPTQ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(X) & 15) != 0) return GPTQ_ERR_INVALID_ARG;
  int G = group_size;
  if (!g_idx) {
    if (G == -1) G = d_in;
    if (G <= 0 || (G % 8) != 0) return GPTQ_ERR_INVALID_ARG;
    if (n_groups != (d_in + G - 1) / G) return GPTQ_ERR_INVALID_ARG;
  } else {
    G = 1;
  }
  if (m == 0) return GPTQ_OK;
  const uint32_t* pk = packed;
  if (x_dtype == GPTQ_BF16) {
    if (y_dtype == GPTQ_F32) launch_w4a16<__bf16, float>(X, m, d_in, pk, scales, zeros, g_idx, G, n_groups, d_out, Y, s);
    else if (y_dtype == GPTQ_BF16) launch_w4a16<__bf16, __bf16>(X, m, d_in, pk, scales, zeros, g_idx, G, n_groups, d_out, Y, s);
    else launch_w4a16<__bf16, _Float16>(X, m, d_in, pk, scales, zeros, g_idx, G, n_groups, d_out, Y, s);
  } else {
    if (y_dtype == GPTQ_F32) launch_w4a16<_Float16, float>(X, m, d_in, pk, scales, zeros, g_idx, G, n_groups, d_out, Y, s);
    else if (y_dtype == GPTQ_BF16) launch_w4a16<_Float16, __bf16>(X, m, d_in, pk, scales, zeros, g_idx, G, n_groups, d_out, Y, s);
    else launch_w4a16<_Float16, _Float16>(X, m, d_in, pk, scales, zeros, g_idx, G, n_groups, d_out, Y, s);
  }
  GPTQ_LAUNCH_CHECK();
  return GPTQ_OK;
}
