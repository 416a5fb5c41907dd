// The forward pieces of one Llama decoder block that layer-sequential GPTQ
// needs between sub-layers ("GPTQ/AWQ量化导出：让大模型在消费级显卡上跑起来": a
// calibration forward pass collects each layer's inputs and the layers are
// quantized one after another; "大模型压缩量化技术：GPTQ 与 AWQ 原理详解 +
// Python 实战教程": one layer at a time, its curvature from running the
// calibration data through it).  All in fp32:
//
//   gptq_rmsnorm          y = x / sqrt(mean(x^2) + eps) * gamma
//   gptq_linear           y = x W^T (+ r), the fp32 MFMA GEMM
//   gptq_block_attention  q, k, v projections, rotary embedding (rotate-half
//                         pairs, theta_i = base^(-2i/hd)), causal softmax
//                         attention per sequence and head
//   gptq_swiglu           m = silu(g) * u
#include "common.h"
#include "gemm_f32.h"

#include <climits>

namespace gptq {

// One 256-thread block per token: the sum of squares in a fixed order (each
// thread a strided subset, then an LDS tree), then the scaled row.
template <int DT>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const void* __restrict__ X, int d,
                                                      const float* __restrict__ gamma, float eps,
                                                      float* __restrict__ Y) {
  __shared__ float red[256];
  const size_t base = (size_t)blockIdx.x * d;
  float s = 0.0f;
  for (int j = threadIdx.x; j < d; j += 256) {
    const float x = load_as_float(X, (gptq_dtype)DT, base + j);
    s += x * x;
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  const float r = 1.0f / sqrtf(red[0] / (float)d + eps);
  for (int j = threadIdx.x; j < d; j += 256) {
    const float x = load_as_float(X, (gptq_dtype)DT, base + j);
    Y[base + j] = gamma ? x * r * gamma[j] : x * r;
  }
}

// cos/sin of p * base^(-2i/hd) for p < seq_len, i < hd/2, formed in fp64.
__global__ __launch_bounds__(256) void rope_table_kernel(int seq_len, int half, int hd, double base,
                                                         float2* __restrict__ tab) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= seq_len * half) return;
  const int p = idx / half, i = idx % half;
  const double ang = (double)p * pow(base, -2.0 * (double)i / (double)hd);
  tab[idx] = make_float2((float)cos(ang), (float)sin(ang));
}

// In place on x [T x d]: in each head, pair (i, i + hd/2) of token t rotated
// by the angle of position t % seq_len.
__global__ __launch_bounds__(256) void rope_kernel(float* __restrict__ x, int64_t T, int d, int hd,
                                                   int seq_len, const float2* __restrict__ tab) {
  const int half = hd / 2;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t pairs = (int64_t)d / 2;
  if (idx >= T * pairs) return;
  const int64_t t = idx / pairs;
  const int r = (int)(idx % pairs);
  const int h = r / half, i = r % half;
  const float2 cs = tab[(t % seq_len) * half + i];
  float* row = x + t * d + (size_t)h * hd;
  const float a = row[i], b = row[i + half];
  row[i] = a * cs.x - b * cs.y;
  row[i + half] = b * cs.x + a * cs.y;
}

// out [C x R] = in [R x C]^T through 32 x 33 LDS tiles.
__global__ __launch_bounds__(256) void transpose_kernel(const float* __restrict__ in, int64_t R, int64_t C,
                                                        float* __restrict__ out) {
  __shared__ float t[32][33];
  const int64_t r0 = (int64_t)blockIdx.y * 32, c0 = (int64_t)blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int i = ty; i < 32; i += 8) {
    const int64_t r = r0 + i, c = c0 + tx;
    t[i][tx] = (r < R && c < C) ? in[r * C + c] : 0.0f;
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    const int64_t c = c0 + i, r = r0 + tx;
    if (c < C && r < R) out[c * R + r] = t[tx][i];
  }
}

// Row i of each head's scores [S x S] (already scaled): softmax over j <= i,
// zeros for j > i.  One 256-thread block per row.
__global__ __launch_bounds__(256) void causal_softmax_kernel(float* __restrict__ sc, int S) {
  __shared__ float red[256];
  const int i = blockIdx.x;
  float* row = sc + ((size_t)blockIdx.y * S + i) * S;
  float m = -INFINITY;
  for (int j = threadIdx.x; j <= i; j += 256) m = fmaxf(m, row[j]);
  red[threadIdx.x] = m;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  m = red[0];
  __syncthreads();
  float s = 0.0f;
  for (int j = threadIdx.x; j <= i; j += 256) s += expf(row[j] - m);
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  const float inv = 1.0f / red[0];
  for (int j = threadIdx.x; j < S; j += 256) row[j] = (j <= i) ? expf(row[j] - m) * inv : 0.0f;
}

__global__ __launch_bounds__(256) void swiglu_kernel(const float* __restrict__ g, const float* __restrict__ u,
                                                     int64_t n, float* __restrict__ m) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float x = g[i];
  m[i] = x / (1.0f + expf(-x)) * u[i];
}

__global__ __launch_bounds__(256) void copy_kernel(const float* __restrict__ a, int64_t n, float* __restrict__ b) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) b[i] = a[i];
}

static unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }

static void launch_transpose(const float* in, int64_t R, int64_t C, float* out, hipStream_t s) {
  transpose_kernel<<<dim3((unsigned)((C + 31) / 32), (unsigned)((R + 31) / 32)), 256, 0, s>>>(in, R, C, out);
}

// y = x W^T (+ y), x [T x d_in], W [d_out x d_in], WT scratch [d_in x d_out]
static void linear_into(const float* x, int64_t T, int d_in, const float* W, int d_out, float* WT, float* y,
                        float beta, hipStream_t s) {
  launch_transpose(W, d_out, d_in, WT, s);
  gemm_f32<false>(x, d_in, WT, d_out, y, d_out, (int)T, d_out, d_in, 1.0f, beta, 0, 0, 0, s);
}

struct AttnLayout {
  size_t off_wt, off_q, off_k, off_v, off_kt, off_sc, off_tab, total;
};

static AttnLayout attn_layout(int64_t T, int d, int n_heads, int S) {
  AttnLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L.off_wt = take((size_t)d * d * 4);
  L.off_q = take((size_t)T * d * 4);
  L.off_k = take((size_t)T * d * 4);
  L.off_v = take((size_t)T * d * 4);
  L.off_kt = take((size_t)T * d * 4);
  L.off_sc = take((size_t)n_heads * S * S * 4);
  L.off_tab = take((size_t)S * (d / n_heads / 2) * sizeof(float2));
  L.total = off;
  return L;
}

}  // namespace gptq

using namespace gptq;

extern "C" int gptq_rmsnorm(const void* X, gptq_dtype x_dtype, int64_t n_tokens, int32_t d,
                            const float* gamma, float eps, float* Y, hipStream_t s) {
  if (!X || !Y || n_tokens < 0 || d <= 0 || !(eps >= 0.0f)) return GPTQ_ERR_INVALID_ARG;
  if (x_dtype != GPTQ_F32 && x_dtype != GPTQ_F16 && x_dtype != GPTQ_BF16) return GPTQ_ERR_INVALID_ARG;
  if (n_tokens == 0) return GPTQ_OK;
  if (n_tokens > INT_MAX) return GPTQ_ERR_INVALID_ARG;
  const unsigned g = (unsigned)n_tokens;
  if (x_dtype == GPTQ_F32) rmsnorm_kernel<GPTQ_F32><<<g, 256, 0, s>>>(X, d, gamma, eps, Y);
  else if (x_dtype == GPTQ_F16) rmsnorm_kernel<GPTQ_F16><<<g, 256, 0, s>>>(X, d, gamma, eps, Y);
  else rmsnorm_kernel<GPTQ_BF16><<<g, 256, 0, s>>>(X, d, gamma, eps, Y);
  GPTQ_LAUNCH_CHECK();
  return GPTQ_OK;
}

extern "C" size_t gptq_linear_workspace_size(int32_t d_out, int32_t d_in) {
  if (d_out <= 0 || d_in <= 0) return 0;
  return align_up((size_t)d_out * d_in * 4);
}

extern "C" int gptq_linear(const float* X, int64_t n_tokens, int32_t d_in, const float* W, int32_t d_out,
                           const float* R, float* Y, void* ws, size_t ws_bytes, hipStream_t s) {
  if (!X || !W || !Y || n_tokens < 0 || d_in <= 0 || d_out <= 0) return GPTQ_ERR_INVALID_ARG;
  if (n_tokens > INT_MAX) return GPTQ_ERR_INVALID_ARG;
  if (!ws || ws_bytes < gptq_linear_workspace_size(d_out, d_in)) return GPTQ_ERR_WORKSPACE;
  if (n_tokens == 0) return GPTQ_OK;
  if (R && R != Y) {
    const int64_t n = n_tokens * d_out;
    copy_kernel<<<blocks_for(n), 256, 0, s>>>(R, n, Y);
    GPTQ_LAUNCH_CHECK();
  }
  linear_into(X, n_tokens, d_in, W, d_out, static_cast<float*>(ws), Y, R ? 1.0f : 0.0f, s);
  GPTQ_LAUNCH_CHECK();
  return GPTQ_OK;
}

extern "C" int gptq_swiglu(const float* G, const float* U, int64_t n, float* M, hipStream_t s) {
  if (!G || !U || !M || n < 0) return GPTQ_ERR_INVALID_ARG;
  if (n == 0) return GPTQ_OK;
  swiglu_kernel<<<blocks_for(n), 256, 0, s>>>(G, U, n, M);
  GPTQ_LAUNCH_CHECK();
  return GPTQ_OK;
}

static bool attn_shape_ok(int64_t T, int d, int n_heads, int S) {
  if (T <= 0 || d <= 0 || n_heads <= 0 || S <= 0) return false;
  if (d % n_heads != 0 || ((d / n_heads) % 2) != 0 || T % S != 0) return false;
  // the transpose of k [T x d] puts T / 32 in the grid's second dimension
  return T <= (int64_t)65535 * 32 && (int64_t)S * S <= INT_MAX;
}

extern "C" size_t gptq_block_attention_workspace_size(int64_t n_tokens, int32_t d, int32_t n_heads,
                                                      int32_t seq_len) {
  if (!attn_shape_ok(n_tokens, d, n_heads, seq_len)) return 0;
  return attn_layout(n_tokens, d, n_heads, seq_len).total;
}

extern "C" int gptq_block_attention(const float* x1, int64_t n_tokens, int32_t d, int32_t n_heads,
                                    int32_t seq_len, const float* Wq, const float* Wk, const float* Wv,
                                    float rope_base, float* out, void* ws, size_t ws_bytes, hipStream_t s) {
  if (!x1 || !Wq || !Wk || !Wv || !out) return GPTQ_ERR_INVALID_ARG;
  if (!attn_shape_ok(n_tokens, d, n_heads, seq_len) || !(rope_base > 0.0f)) return GPTQ_ERR_INVALID_ARG;
  const AttnLayout L = attn_layout(n_tokens, d, n_heads, seq_len);
  if (!ws || ws_bytes < L.total) return GPTQ_ERR_WORKSPACE;
  char* b = static_cast<char*>(ws);
  float* WT = reinterpret_cast<float*>(b + L.off_wt);
  float* q = reinterpret_cast<float*>(b + L.off_q);
  float* k = reinterpret_cast<float*>(b + L.off_k);
  float* v = reinterpret_cast<float*>(b + L.off_v);
  float* kt = reinterpret_cast<float*>(b + L.off_kt);
  float* sc = reinterpret_cast<float*>(b + L.off_sc);
  float2* tab = reinterpret_cast<float2*>(b + L.off_tab);
  const int64_t T = n_tokens;
  const int S = seq_len, hd = d / n_heads, half = hd / 2;

  linear_into(x1, T, d, Wq, d, WT, q, 0.0f, s);
  linear_into(x1, T, d, Wk, d, WT, k, 0.0f, s);
  linear_into(x1, T, d, Wv, d, WT, v, 0.0f, s);
  GPTQ_LAUNCH_CHECK();
  rope_table_kernel<<<blocks_for((int64_t)S * half), 256, 0, s>>>(S, half, hd, (double)rope_base, tab);
  rope_kernel<<<blocks_for(T * (d / 2)), 256, 0, s>>>(q, T, d, hd, S, tab);
  rope_kernel<<<blocks_for(T * (d / 2)), 256, 0, s>>>(k, T, d, hd, S, tab);
  launch_transpose(k, T, d, kt, s);
  GPTQ_LAUNCH_CHECK();
  const float scale = 1.0f / sqrtf((float)hd);
  for (int64_t s0 = 0; s0 < T; s0 += S) {
    for (int h0 = 0; h0 < n_heads; h0 += kGemmMaxGroup) {
      const int cnt = std::min(kGemmMaxGroup, n_heads - h0);
      GemmGroup g1, g2;
      g1.count = g2.count = cnt;
      for (int i = 0; i < cnt; ++i) {
        const int h = h0 + i;
        float* sch = sc + (size_t)h * S * S;
        // scores = q_h k_h^T / sqrt(hd)
        g1.p[i] = GemmProblem{q + s0 * d + (size_t)h * hd, kt + (size_t)h * hd * T + s0, sch, nullptr,
                              d, (int)T, S, S, S, hd};
        // out_h = P v_h
        g2.p[i] = GemmProblem{sch, v + s0 * d + (size_t)h * hd, out + s0 * d + (size_t)h * hd, nullptr,
                              S, d, d, S, hd, S};
      }
      launch_gemm_group<false, kStore>(g1, scale, 0.0f, 0, 0, 0, nullptr, s);
      GPTQ_LAUNCH_CHECK();
      causal_softmax_kernel<<<dim3((unsigned)S, (unsigned)cnt), 256, 0, s>>>(sc + (size_t)h0 * S * S, S);
      GPTQ_LAUNCH_CHECK();
      launch_gemm_group<false, kStore>(g2, 1.0f, 0.0f, 0, 0, 0, nullptr, s);
      GPTQ_LAUNCH_CHECK();
    }
  }
  return GPTQ_OK;
}
