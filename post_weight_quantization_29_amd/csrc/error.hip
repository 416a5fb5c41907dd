// Layer reconstruction error ||(W - Q) X^T||_F^2 = 1/2 tr(D H D^T), D = W - Q,
// H = 2 X^T X undamped (GPTQ practice page m.lqnn.cn/news/117696, section 5.5:
// quantify the loss).  D is formed once in fp32, T = D * H runs on the fp32
// MFMA GEMM whose epilogue dots each tile with D in fp64, and one workgroup
// adds the tile sums in a fixed order.
#include "gemm_f32.h"

namespace gptq {

__global__ __launch_bounds__(256) void diff_kernel(const void* __restrict__ W, gptq_dtype wt,
                                                   const float* __restrict__ Q, int64_t n,
                                                   float* __restrict__ D) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride)
    D[i] = load_as_float(W, wt, (size_t)i) - Q[i];
}

__global__ __launch_bounds__(256) void sum_tiles_kernel(const double* __restrict__ part, int n,
                                                        double* __restrict__ out) {
  __shared__ double red[256];
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += 256) s += part[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = 0.5 * red[0];
}

struct ErrLayout {
  size_t off_d, off_part, off_out, total;
  int tiles;
};

static ErrLayout err_layout(int d_out, int d) {
  ErrLayout L;
  L.tiles = gemm_tiles(d_out, d);
  size_t off = 0;
  L.off_d = off;
  off = align_up(off + (size_t)d_out * d * sizeof(float));
  L.off_part = off;
  off = align_up(off + (size_t)L.tiles * sizeof(double));
  L.off_out = off;
  off = align_up(off + sizeof(double));
  L.total = off;
  return L;
}

}  // namespace gptq

using namespace gptq;

extern "C" size_t gptq_layer_error_workspace_size(int32_t d_out, int32_t d_in) {
  if (d_out <= 0 || d_in <= 0) return 0;
  return err_layout(d_out, d_in).total;
}

extern "C" int gptq_layer_error(const float* H, const void* W, gptq_dtype w_dtype, const float* Q,
                                int32_t d_out, int32_t d_in, double* out_host, void* ws,
                                size_t ws_bytes, hipStream_t s) {
  if (!H || !W || !Q || !out_host || d_out <= 0 || d_in <= 0) return GPTQ_ERR_INVALID_ARG;
  if (w_dtype != GPTQ_F32 && w_dtype != GPTQ_F16 && w_dtype != GPTQ_BF16) return GPTQ_ERR_INVALID_ARG;
  const ErrLayout L = err_layout(d_out, d_in);
  if (!ws || ws_bytes < L.total) return GPTQ_ERR_WORKSPACE;
  char* base = static_cast<char*>(ws);
  float* D = reinterpret_cast<float*>(base + L.off_d);
  double* part = reinterpret_cast<double*>(base + L.off_part);
  double* out = reinterpret_cast<double*>(base + L.off_out);
  const int64_t n = (int64_t)d_out * d_in;
  diff_kernel<<<(unsigned)std::min<int64_t>((n + 255) / 256, 16384), 256, 0, s>>>(W, w_dtype, Q, n, D);
  GPTQ_LAUNCH_CHECK();
  GemmGroup g;
  g.count = 1;
  // T = D * H: Aop(m, k) = D[m][k] (m-major), Bop(k, n) = H[k][n]; dotted with D
  g.p[0] = GemmProblem{D, H, nullptr, D, d_in, d_in, d_in, d_out, d_in, d_in};
  launch_gemm_group<false, kDot>(g, 1.0f, 0.0f, 0, 0, 0, part, s);
  GPTQ_LAUNCH_CHECK();
  sum_tiles_kernel<<<1, 256, 0, s>>>(part, L.tiles, out);
  GPTQ_LAUNCH_CHECK();
  GPTQ_HIP_TRY(hipMemcpyAsync(out_host, out, sizeof(double), hipMemcpyDeviceToHost, s));
  GPTQ_HIP_TRY(hipStreamSynchronize(s));
  return GPTQ_OK;
}

extern "C" const char* gptq_status_string(int status) {
  switch (status) {
    case GPTQ_OK: return "ok";
    case GPTQ_ERR_INVALID_ARG: return "invalid argument";
    case GPTQ_ERR_NOT_PD: return "damped Hessian is not positive definite (raise damp_percent)";
    case GPTQ_ERR_HIP: return "HIP runtime error";
    case GPTQ_ERR_WORKSPACE: return "workspace missing or too small";
    case GPTQ_ERR_UNSUPPORTED: return "option not supported by this library";
    default: return "unknown status";
  }
}

extern "C" int gptq_abi_version(void) { return 2; }
