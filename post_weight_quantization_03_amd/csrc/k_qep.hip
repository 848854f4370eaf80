// Error-propagation correction before GPTQ (the QEP idea of the OneComp
// pages: the error that quantizing the earlier layers leaves in a layer's
// inputs is carried into that layer's correction).  Read as the ridge fit of
// the full-precision outputs from the quantized-model inputs X^:
//
//   W' = W + alpha W G H_d^-1,  G = 2 (X - X^)^T X^ = C - H^,
//   C = 2 X^T X^ (cross term), H^ = 2 X^T X^ (the GPTQ Hessian of X^),
//   H_d = H^ + lambda I with GPTQ's damping and dead-column rule.
//
// The cross term is the Hessian's SYRK kernel in its cross mode (every tile
// of the square grid, the B operand from X^; k_hessian.hip).  The correction
// factors H^ in place with the quantizer's own factor (H_d^-1 = U^T U, H then
// holds U exactly as the quantizer leaves it, so the layer is quantized next
// with the factor reused), and applies H_d^-1 as two triangular products with
// the library's fp32 MFMA GEMM: W' = W + alpha ((W G) U^T) U (the U^T product
// skips the zero half of its K range).
#include "common.h"

namespace gptq {
namespace {

// C -= H, n x n
__global__ void k_sub(float* C, const float* H, int64_t count) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += (int64_t)gridDim.x * blockDim.x)
    C[i] -= H[i];
}

// T = the upper triangle of H (with the diagonal), zeros below
__global__ void k_triu(const float* H, float* T, int64_t n) {
  for (int64_t i = blockIdx.y; i < n; i += gridDim.y)
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += (int64_t)gridDim.x * blockDim.x)
      T[i * n + j] = j >= i ? H[i * n + j] : 0.0f;
}

// out = W as fp32 (bf16 widens exactly)
__global__ void k_to_f32(const void* W, bool bf16, float* out, int64_t count) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += (int64_t)gridDim.x * blockDim.x)
    out[i] = bf16 ? __uint_as_float((uint32_t) static_cast<const uint16_t*>(W)[i] << 16)
                  : static_cast<const float*>(W)[i];
}

unsigned blocks_for(int64_t count) {
  const int64_t b = (count + 255) / 256;
  return (unsigned)(b < 8192 ? (b > 0 ? b : 1) : 8192);
}

}  // namespace

// W_out = W + alpha ((W G) U^T) U, G = C - H (C is overwritten by G), H factored
// in place (U in the upper triangle, dead flags below) with the scratch in f.
// P1, P2: [rows, n] scratch.  T: [n, n] scratch (may be f.A, free after the factor).
hipError_t qep_correct_run(const void* W, bool w_bf16, int64_t rows, int64_t n, float* C, float* H, float damp,
                           float alpha, float* W_out, const FactorWs& f, float* P1, float* P2, float* T,
                           hipStream_t stream) {
  hipLaunchKernelGGL(k_sub, dim3(blocks_for(n * n)), dim3(256), 0, stream, C, (const float*)H, n * n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = factor_run(H, n, damp, f, stream)) != hipSuccess) return e;
  const unsigned gy = (unsigned)(n < 65535 ? n : 65535);
  hipLaunchKernelGGL(k_triu, dim3((unsigned)((n + 255) / 256), gy), dim3(256), 0, stream, (const float*)H, T, n);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_to_f32, dim3(blocks_for(rows * n)), dim3(256), 0, stream, W, w_bf16, W_out, rows * n);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  GemmF32 g{};
  g.M = (int)rows;
  g.N = (int)n;
  g.K = (int)n;
  g.lda = n;
  g.ldb = n;
  g.ldc = n;
  g.batch = 1;
  // P1 = W G: B(k, j) = G[k][j], k-major
  g.A = W_out;
  g.B = C;
  g.b_kmajor = 1;
  g.C = P1;
  g.alpha = 1.0f;
  g.beta = 0;
  if ((e = gemm_f32(g, stream)) != hipSuccess) return e;
  // P2 = P1 U^T: B(k, j) = U[j][k] = T[j][k], n-major; U[j][k] = 0 for k < j, so a
  // tile of columns from n0 on needs only k >= n0
  g.A = P1;
  g.B = T;
  g.b_kmajor = 0;
  g.C = P2;
  g.klo_n = 1;
  if ((e = gemm_f32(g, stream)) != hipSuccess) return e;
  g.klo_n = 0;
  // W_out += alpha P2 U: B(k, j) = U[k][j] = T[k][j], k-major
  g.A = P2;
  g.B = T;
  g.b_kmajor = 1;
  g.C = W_out;
  g.alpha = alpha;
  g.beta = 1;
  return gemm_f32(g, stream);
}

}  // namespace gptq
