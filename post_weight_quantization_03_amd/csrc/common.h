// Internal declarations shared by the kernel files of libgptq.so (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gptq.h"

namespace gptq {

// ---------------------------------------------------------------------------
// MFMA operand and accumulator types.
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// 32x32 MFMA accumulator layout (v_mfma_f32_32x32x*): lane l, register r holds
// element (row, col) of the 32x32 block with col = l % 32 and
// row = 8 * (r / 4) + 4 * (l / 32) + r % 4.
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }
__device__ __forceinline__ int acc_col(int lane) { return lane & 31; }

// Device status codes are gptq_status values; kernels raise them with atomicMax.
__device__ __forceinline__ void raise_status(int* st, int code) { atomicMax(st, code); }

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------------------
// Phase timestamps, a build option (libgptq_trace.so, built with -DGPTQ_TRACE).
// The column loop's workgroups, the factor chain's kernels and the batch
// product's workgroups read the 100 MHz
// s_memrealtime clock at their phase boundaries and thread 0 of each workgroup
// appends one record to a device buffer set by gptq_trace_set:
//   buf[0] = capacity in records, buf[1] = records appended (atomic),
//   record i at buf[32 (i + 1)]: kind, workgroup, tag, stamp count, stamps.
// Device variables are per kernel file (no relocatable device code), so each
// instrumented file holds its own buffer pointer and setter.  Without the
// option the macros are empty and nothing of this is compiled.
enum TraceKind { TR_LOOP = 1, TR_POTRF = 2, TR_TRSM = 3, TR_DIAG = 4, TR_TILE = 5, TR_MMA = 6 };
constexpr int TRACE_REC = 32;           // words per record
constexpr int TRACE_STAMPS = TRACE_REC - 4;
#ifdef GPTQ_TRACE
namespace {
__device__ unsigned long long* trace_buf;
__device__ __forceinline__ void trace_write(int kind, int64_t tag, const unsigned long long* t, int n) {
  unsigned long long* b = trace_buf;
  if (b == nullptr || threadIdx.x != 0) return;
  const unsigned long long i = atomicAdd(b + 1, 1ull);
  if (i >= b[0]) return;
  unsigned long long* r = b + TRACE_REC * (i + 1);
  r[0] = (unsigned long long)kind;
  r[1] = blockIdx.x;
  r[2] = (unsigned long long)tag;
  r[3] = (unsigned long long)n;
  for (int j = 0; j < n && j < TRACE_STAMPS; ++j) r[4 + j] = t[j];
}
}  // namespace
#define GPTQ_TRACE_DECL unsigned long long trace_t_[TRACE_STAMPS]; int trace_n_ = 0
#define GPTQ_TRACE_STAMP() (trace_t_[trace_n_++] = __builtin_amdgcn_s_memrealtime())
#define GPTQ_TRACE_WRITE(kind, tag) trace_write(kind, tag, trace_t_, trace_n_)
#define GPTQ_TRACE_ONLY(...) __VA_ARGS__
#define GPTQ_TRACE_SETTER(name) \
  hipError_t name(unsigned long long* p) { return hipMemcpyToSymbol(HIP_SYMBOL(trace_buf), &p, sizeof(p)); }
#else
#define GPTQ_TRACE_ONLY(...)
#define GPTQ_TRACE_DECL
#define GPTQ_TRACE_STAMP()
#define GPTQ_TRACE_WRITE(kind, tag)
#endif
hipError_t trace_set_factor(unsigned long long* p);  // trace build only
hipError_t trace_set_quant(unsigned long long* p);
hipError_t trace_set_mma(unsigned long long* p);

// ---------------------------------------------------------------------------
// fp32 MFMA GEMM:  C(m, n) = alpha * sum_k A(m, k) B(k, n) + (beta ? C(m, n) : 0)
//   A(m, k) = A[m * lda + k]
//   B(k, n) = B[k * ldb + n]        (b_kmajor)   or   B[n * ldb + k]   (!b_kmajor)
//   C(m, n) = C[m * ldc + n]
// 128x128 tiles.  tri: grid.x enumerates only the lower tiles (tile_m >= tile_n)
// of a square tile grid.  klo_n: B is lower triangular, so k < n0 is skipped.
// khi_m: A is lower triangular, so k >= m0 + 128 is skipped.  Batches run over
// blockIdx.z with element strides sA, sB, sC.
struct GemmF32 {
  const float* A;
  const float* B;
  float* C;
  int64_t lda, ldb, ldc;
  int64_t sA, sB, sC;
  int M, N, K;
  float alpha;
  int beta;
  int b_kmajor;
  int tri;
  int klo_n;
  int khi_m;
  int kfl_lo, kfl_hi;  // tile rows m0 in [kfl_lo, kfl_hi) start their K range at m0 - kfl_lo
  int batch;
  int order;  // set by gemm_f32: 1 = tiles by ascending column, 2 = by descending row (longest K first)
};
hipError_t gemm_f32(const GemmF32& g, hipStream_t stream);

// ---------------------------------------------------------------------------
// Hessian accumulation (k_hessian.hip).
size_t hessian_workspace(int64_t n, int64_t tokens, gptq_dtype dt);
int hessian_launch(float* H, int64_t n, const void* X, gptq_dtype dt, int64_t tokens, int64_t ldx,
                   void* ws, size_t ws_bytes, hipStream_t stream);

// ---------------------------------------------------------------------------
// Damping and factor (k_factor.hip).
struct FactorWs {
  int* status;      // device int32
  float* lam;       // device: lambda (float)
  uint8_t* dead;    // device [n]
  float* A;         // [n, n] reversed damped Hessian -> L below the diagonal blocks, L^-T above
  float* Lt;        // [ceil(n / 128), 128, 128] L_kk^T of each diagonal block
};
size_t factor_scratch_floats(int64_t n);  // floats of FactorWs::Lt
// H (fp32 [n, n]) -> damped, factored; U written back to H's upper triangle, dead flags to the
// strictly lower slots.  Status (ENOTPD) is raised on the device.
hipError_t factor_run(float* H, int64_t n, float damp, const FactorWs& ws, hipStream_t stream);
// The same factor computed in fp64 (k_factor64.hip); U is rounded to fp32 when written to H.
struct Factor64Ws {
  int* status;
  double* lam;      // device: lambda (double)
  uint8_t* dead;    // device [n]
  double* A;        // [n, n] fp64 work matrix
  double* Lt;       // [ceil(n / 128), 128, 128] fp64 L_kk^T of each diagonal block
};
size_t factor64_scratch_doubles(int64_t n);  // doubles of Factor64Ws::Lt
hipError_t factor64_run(float* H, int64_t n, float damp, const Factor64Ws& ws, hipStream_t stream);
// H holds a factor from an earlier call: read the dead flags back from it.
hipError_t dead_from_factor(const float* H, int64_t n, uint8_t* dead, hipStream_t stream);

// ---------------------------------------------------------------------------
// Quantize loop (k_quant.hip).
struct QuantArgs {
  const void* W;
  gptq_dtype w_dtype;
  int64_t rows, cols;
  const float* U;  // [cols, cols], upper triangle used
  const uint8_t* dead;
  int bits, groupsize;  // groupsize already resolved (-1 -> cols)
  uint8_t* codes;
  float* scales;
  uint8_t* zeros;
  float* w_hat;
  float* row_loss;
  float* Wf;  // [rows, cols] working copy
  float* E;   // [rows, 128 ceil(cols / 128)] scaled errors of every block, kept for the layer
  uint16_t* Usplit;  // [3][cols, cols] bf16 planes of U for the split trailing GEMM, or null
  int64_t G;
};
// Bytes of the U planes quant_run needs (0 when no trailing update runs split).
size_t quant_split_bytes(int64_t cols, int64_t groupsize);
hipError_t quant_run(const QuantArgs& a, hipStream_t stream);

// ---------------------------------------------------------------------------
// Packing (k_pack.hip).
hipError_t pack_launch(const uint8_t* codes, int64_t rows, int64_t cols, int bits, uint32_t* packed,
                       hipStream_t stream);

// Dequantizing GEMV y = W^ x over packed codes (k_gemv.hip).
bool dequant_gemv_supported(int64_t cols, int32_t bits, int32_t groupsize);
hipError_t dequant_gemv(const uint32_t* packed, const float* scales, const uint8_t* zeros, int64_t rows,
                        int64_t cols, int32_t bits, int32_t groupsize, const void* x, bool x_bf16, float* y,
                        hipStream_t stream);
hipError_t dequant_gemm(const uint32_t* packed, const float* scales, const uint8_t* zeros, int64_t rows,
                        int64_t cols, int32_t bits, int32_t groupsize, const void* X, bool x_bf16, int64_t ldx,
                        int64_t batch, float* Y, int64_t ldy, hipStream_t stream);
// The batch product on the matrix cores (k_dequant_mma.hip): batches of two or
// more, groups a multiple of 128 columns or the whole row.
bool dequant_mma_supported(int64_t cols, int32_t groupsize, int64_t batch);
size_t dequant_mma_workspace(int64_t rows, int64_t cols, int64_t batch);
hipError_t dequant_mma(const uint32_t* packed, const float* scales, const uint8_t* zeros, int64_t rows,
                       int64_t cols, int32_t bits, int32_t groupsize, const void* X, bool x_bf16, int64_t ldx,
                       int64_t batch, float* Y, int64_t ldy, void* workspace, hipStream_t stream);

// Fixed randomised Hadamard rotation (k_hadamard.hip).
int64_t hadamard_chunks(int64_t n);
hipError_t hadamard_rows(const void* in, bool in_bf16, int64_t ld_in, float* out, int64_t ld_out, int64_t rows,
                         int64_t n, const float* signs, int block, hipStream_t stream);
hipError_t hadamard_hessian(float* H, int64_t n, const float* signs, int block, hipStream_t stream);

// Error-propagation correction (k_qep.hip).
// Cross term C += 2 X^T Xq: the Hessian kernels in their cross mode (k_hessian.hip).
size_t cross_workspace(int64_t n, int64_t tokens, gptq_dtype dt);
int cross_launch(float* C, int64_t n, const void* X, const void* Xq, gptq_dtype dt, int64_t tokens, int64_t ldx,
                 void* ws, size_t ws_bytes, hipStream_t stream);
hipError_t qep_correct_run(const void* W, bool w_bf16, int64_t rows, int64_t n, float* C, float* H, float damp,
                           float alpha, float* W_out, const FactorWs& f, float* P1, float* P2, float* T,
                           hipStream_t stream);

// Small utility kernels (k_factor.hip).
hipError_t fill_i32(int* p, int64_t n, int v, hipStream_t stream);
hipError_t copy_status(const int* src, int32_t* dst, hipStream_t stream);

}  // namespace gptq
