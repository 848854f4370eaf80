// The factor U (upper, positive diagonal, U^T U = inv(H_d)) computed in fp64:
// the GPTQ_FACTOR_F64 option.  The damped Hessian and every step of the
// factor are fp64; U is rounded to fp32 once, when it is written into H.
//
// Same route and data placement as the fp32 factor: with P the index
// reversal, P H_d P = L L^T, U = P L^-1 P.  A work matrix holds P H_d P in
// its lower triangle; per 128-column block k (columns [k0, c1)):
//   k_potrf64   Cholesky of the diagonal block in one workgroup (column by
//               column in LDS), L_kk^T to a buffer of its own;
//   k_trsm64    every row of block column k solved against L_kk: the panel
//               below (L_ik = A_ik L_kk^-T), the rows of the block (row r of
//               L_kk^-T), the rows above (the block column of Y = L^-T from
//               the sums accumulated there);
//   k_gemm64    A[r][j] -= A[r][k0:c1] L[j][k0:c1]^T for the columns j >= c1:
//               below c1 the Cholesky trailing update (lower tiles), above it
//               the inverse's block forward substitution (every tile), on
//               v_mfma_f64_16x16x4f64.
// k_write_factor64 writes U[i][j] = Y[n-1-j][n-1-i] into H as fp32, with the
// dead flags in H's strictly lower triangle.
#include <utility>

#include "common.h"

namespace gptq {
namespace {

constexpr int NB = 128;

typedef double f64x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(1024) void k_damp_stats64(const float* H, int64_t n, float damp, uint8_t* dead,
                                                       double* lam) {
  __shared__ double part[1024];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
    const float d = H[i * n + i];
    const bool z = (d == 0.0f);
    dead[i] = z ? 1 : 0;
    s += z ? 1.0 : (double)d;
  }
  part[threadIdx.x] = s;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *lam = (double)damp * part[0] / (double)n;
}

// A[i][j] = H_d[n-1-i][n-1-j] for j <= i, 0 above the diagonal.
__global__ void k_reverse_damped64(const float* H, int64_t n, const uint8_t* dead, const double* lam, double* A) {
  const double l = *lam;
  for (int64_t i = blockIdx.y; i < n; i += gridDim.y) {
    const int64_t si = n - 1 - i;
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += (int64_t)gridDim.x * blockDim.x) {
      const int64_t sj = n - 1 - j;
      double v = 0.0;
      if (j == i)
        v = (dead[si] ? 1.0 : (double)H[si * n + si]) + l;
      else if (j < i)
        v = (double)H[si * n + sj];  // sj > si: the upper triangle of H
      A[i * n + j] = v;
    }
  }
}

// ------------------------------------------------------------------ diagonal block

// Cholesky of A[k0:k0+kb, k0:k0+kb] (lower triangle; the identity past kb),
// column by column: pivot, column scale, rank-one update of the trailing lower
// triangle, two barriers a column.  L^T (zeros below the diagonal) goes to Lt.
// A pivot that is not positive and finite raises GPTQ_ENOTPD (its square root
// is NaN or the check below fails).
constexpr int LP = NB + 1;  // LDS pitch in doubles

__global__ __launch_bounds__(256) void k_potrf64(const double* A, int64_t n, int64_t k0, double* Lt, int* status) {
  __shared__ double As[NB][LP];
  const int kb = (int)((n - k0) < NB ? (n - k0) : NB);
  const int tid = threadIdx.x;
  for (int idx = tid; idx < NB * NB; idx += 256) {
    const int r = idx >> 7, q = idx & (NB - 1);
    double v = (r == q) ? 1.0 : 0.0;
    if (r < kb && q <= r) v = A[(k0 + r) * n + k0 + q];
    As[r][q] = v;
  }
  __syncthreads();
  const int ty = tid >> 4, tx = tid & 15;
  for (int j = 0; j < NB; ++j) {
    if (tid == 0) As[j][j] = sqrt(As[j][j]);
    __syncthreads();
    const double p = As[j][j];
    for (int i = j + 1 + tid; i < NB; i += 256) As[i][j] = As[i][j] / p;
    __syncthreads();
    // A_im -= L_ij L_mj for j < m <= i
    for (int i = j + 1 + ty; i < NB; i += 16) {
      const double li = As[i][j];
      for (int m = j + 1 + tx; m <= i; m += 16) As[i][m] = fma(-li, As[m][j], As[i][m]);
    }
    __syncthreads();
  }
  if (tid < kb) {
    const double d = As[tid][tid];
    if (!(d > 0.0 && d < INFINITY)) raise_status(status, GPTQ_ENOTPD);
  }
  for (int idx = tid; idx < NB * NB; idx += 256) {
    const int r = idx >> 7, q = idx & (NB - 1);
    Lt[r * NB + q] = q >= r ? As[q][r] : 0.0;
  }
}

// ------------------------------------------------------------------ block column solve

// Rows y = b L^-T (L y^T = b^T, forward substitution, right-looking: y_j =
// b_j / L_jj, then b_m -= y_j L_mj for m > j).  A wave holds 4 rows, 16 lanes
// a row, 8 consecutive columns per lane; y_j reaches the row's lanes by a DPP
// row broadcast of its two halves.  L^T sits in LDS with zeros on and below
// its diagonal, so step j changes only the columns after j and column j is
// final once step j starts.
//   rows below the block: the panel L_ik = A_ik L_kk^-T, in place;
//   rows above it: the block column of Y from the sums accumulated there;
//   rows of the block: b = e_r, giving row r of L_kk^-T (zeros left of it).
template <int O>
__device__ __forceinline__ double row_bcast64(double v) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), 0x150 + O, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), 0x150 + O, 0xf, 0xf, false);
  return __hiloint2double(hi, lo);
}

template <int J>
__device__ __forceinline__ void trsm64_step(double (&b)[8], const double (&rd)[8], const double (*Lt)[NB], int t) {
  constexpr int O = J >> 3, SL = J & 7;
  const double y = row_bcast64<O>(b[SL] * rd[SL]);
#pragma unroll
  for (int i = 0; i < 8; ++i) b[i] = fma(-y, Lt[J][8 * t + i], b[i]);
}

template <int... Js>
__device__ __forceinline__ void trsm64_steps(double (&b)[8], const double (&rd)[8], const double (*Lt)[NB], int t,
                                             std::integer_sequence<int, Js...>) {
  (trsm64_step<Js>(b, rd, Lt, t), ...);
}

constexpr int TRSM_THREADS = 512;
constexpr int TRSM_ROWS = TRSM_THREADS / 16;

__global__ __launch_bounds__(TRSM_THREADS) void k_trsm64(double* A, const double* Ltk, int64_t n, int64_t k0, int kb) {
  __shared__ double Lt[NB][NB];
  __shared__ double rL[NB];
  const int tid = threadIdx.x;
  for (int idx = tid; idx < NB * NB; idx += TRSM_THREADS) {
    const int j = idx >> 7, m = idx & (NB - 1);
    Lt[j][m] = m > j ? Ltk[idx] : 0.0;
  }
  if (tid < NB) rL[tid] = tid < kb ? 1.0 / Ltk[tid * (NB + 1)] : 0.0;
  __syncthreads();
  const int lane = tid & 63, t = lane & 15;
  const int64_t grow = (int64_t)blockIdx.x * TRSM_ROWS + (tid >> 4);
  const bool ok = grow < n;
  const bool ident = grow >= k0 && grow < k0 + kb;
  const int rr = (int)(grow - k0);
  double b[8], rd[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = 8 * t + i;
    if (ident)
      b[i] = c == rr ? 1.0 : 0.0;
    else
      b[i] = (ok && c < kb) ? A[grow * n + k0 + c] : 0.0;
    rd[i] = rL[c];
  }
  trsm64_steps(b, rd, Lt, t, std::make_integer_sequence<int, NB>{});
  if (!ok) return;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = 8 * t + i;
    if (c < kb) A[grow * n + k0 + c] = (ident && c < rr) ? 0.0 : b[i] * rd[i];
  }
}

// ------------------------------------------------------------------ step GEMM

// C[r][j] -= sum_k A[r][k] L[j][k] over k < kb, for 64 x 64 tiles: the
// lower tiles of the trailing matrix (rows and columns >= c1, tile row >=
// tile column) and every tile of the rectangle rows [0, c1) x columns
// [c1, n).  The workgroup stages its 64 rows of both operands (kb doubles
// each) in LDS, then four waves each take a 32 x 32 quarter as 2 x 2 blocks of
// v_mfma_f64_16x16x4f64: lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16]
// of a 16 x 16 x 4 step and holds D[4 r + l / 16][l % 16] in register r.
constexpr int GT = 64;
constexpr int GP = NB + 1;  // LDS pitch in doubles: a 16-row column read falls on 32 distinct banks

__global__ __launch_bounds__(256) void k_gemm64(double* A, int64_t n, int64_t k0, int64_t c1, int kb, int ntri,
                                                int nt) {
  __shared__ double Sa[GT][GP];
  __shared__ double Sb[GT][GP];
  const int u = blockIdx.x;
  int64_t r0, j0;
  if (u < ntri) {
    int ti = (int)((sqrtf(8.f * (float)u + 1.f) - 1.f) * 0.5f);
    while ((ti + 1) * (ti + 2) / 2 <= u) ++ti;
    while (ti * (ti + 1) / 2 > u) --ti;
    r0 = c1 + (int64_t)GT * ti;
    j0 = c1 + (int64_t)GT * (u - ti * (ti + 1) / 2);
  } else {
    const int v = u - ntri;
    r0 = (int64_t)GT * (v / nt);
    j0 = c1 + (int64_t)GT * (v % nt);
  }
  const int tid = threadIdx.x;
  // stage rows r0.. (A operand) and j0.. (B operand), columns k0 .. k0 + kb, zeros beyond
  for (int idx = tid; idx < GT * NB; idx += 256) {
    const int r = idx >> 7, k = idx & (NB - 1);
    const bool kin = k < kb;
    Sa[r][k] = (kin && r0 + r < n) ? A[(r0 + r) * n + k0 + k] : 0.0;
    Sb[r][k] = (kin && j0 + r < n) ? A[(j0 + r) * n + k0 + k] : 0.0;
  }
  __syncthreads();
  const int lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;
  const int li = lane & 15, lk = lane >> 4;
  f64x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c) acc[a][c] = f64x4{0.0, 0.0, 0.0, 0.0};
  const int ksteps = (kb + 3) / 4;
  for (int s = 0; s < ksteps; ++s) {
    const int k = 4 * s + lk;
    double av[2], bv[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) av[a] = Sa[32 * wm + 16 * a + li][k];
#pragma unroll
    for (int c = 0; c < 2; ++c) bv[c] = Sb[32 * wn + 16 * c + li][k];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int c = 0; c < 2; ++c) acc[a][c] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a], bv[c], acc[a][c], 0, 0, 0);
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t r = r0 + 32 * wm + 16 * a + 4 * q + lk;
        const int64_t j = j0 + 32 * wn + 16 * c + li;
        if (r < n && j < n) A[r * n + j] -= acc[a][c][q];
      }
}

// U[i][j] = (float) Y[n-1-j][n-1-i] for j >= i into H (Y = L^-T, the upper
// triangle of A), by 64 x 64 tiles transposed through LDS; tiles on the
// diagonal also write the dead flags (H[i][i-1], and H[n-1][0] for column 0).
__global__ __launch_bounds__(256) void k_write_factor64(const double* Y, int64_t n, const uint8_t* dead, float* H) {
  __shared__ float T[64][65];
  const int64_t I0 = (int64_t)blockIdx.y * 64, J0 = (int64_t)blockIdx.x * 64;
  if (J0 + 63 < I0) return;
  const int64_t yr0 = n - J0 - 64, yc0 = n - I0 - 64;  // negative at a ragged edge
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int k = ty; k < 64; k += 4) {
    const int64_t yr = yr0 + k, yc = yc0 + tx;
    T[k][tx] = (yr >= 0 && yc >= 0) ? (float)Y[yr * n + yc] : 0.0f;
  }
  __syncthreads();
  for (int a = ty; a < 64; a += 4) {
    const int64_t i = I0 + a, j = J0 + tx;
    if (i < n && j < n && j >= i) H[i * n + j] = T[63 - tx][63 - a];
  }
  if (I0 == J0 && ty == 0) {
    const int64_t i = I0 + tx;
    if (i >= 1 && i < n) H[i * n + i - 1] = dead[i] ? 1.0f : 0.0f;
    if (i == n - 1 && n >= 3) H[i * n + 0] = dead[0] ? 1.0f : 0.0f;
  }
}

}  // namespace

size_t factor64_scratch_doubles(int64_t n) { return (size_t)((n + NB - 1) / NB) * NB * NB; }

#define F64CHECK(x)                        \
  do {                                     \
    hipError_t e_ = (x);                   \
    if (e_ != hipSuccess) return e_;       \
  } while (0)

hipError_t factor64_run(float* H, int64_t n, float damp, const Factor64Ws& ws, hipStream_t stream) {
  hipLaunchKernelGGL(k_damp_stats64, dim3(1), dim3(1024), 0, stream, (const float*)H, n, damp, ws.dead, ws.lam);
  F64CHECK(hipGetLastError());
  {
    const unsigned gx = (unsigned)((n + 255) / 256 < 16 ? (n + 255) / 256 : 16);
    const unsigned gy = (unsigned)(n < 65535 ? n : 65535);
    hipLaunchKernelGGL(k_reverse_damped64, dim3(gx, gy), dim3(256), 0, stream, (const float*)H, n,
                       (const uint8_t*)ws.dead, (const double*)ws.lam, ws.A);
    F64CHECK(hipGetLastError());
  }
  const int64_t nk = (n + NB - 1) / NB;
  const unsigned trows = (unsigned)((n + TRSM_ROWS - 1) / TRSM_ROWS);
  for (int64_t k = 0; k < nk; ++k) {
    const int64_t k0 = k * NB;
    const int kb = (int)((n - k0) < NB ? (n - k0) : NB);
    const int64_t c1 = k0 + kb, rest = n - c1;
    double* Ltk = ws.Lt + k * NB * NB;
    hipLaunchKernelGGL(k_potrf64, dim3(1), dim3(256), 0, stream, (const double*)ws.A, n, k0, Ltk, ws.status);
    F64CHECK(hipGetLastError());
    hipLaunchKernelGGL(k_trsm64, dim3(trows), dim3(TRSM_THREADS), 0, stream, ws.A, (const double*)Ltk, n, k0, kb);
    F64CHECK(hipGetLastError());
    if (rest <= 0) break;
    const int64_t nt = (rest + GT - 1) / GT, ntri = nt * (nt + 1) / 2, rrows = (c1 + GT - 1) / GT;
    const int64_t tiles = ntri + rrows * nt;
    if (tiles > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_gemm64, dim3((unsigned)tiles), dim3(256), 0, stream, ws.A, n, k0, c1, kb, (int)ntri,
                       (int)nt);
    F64CHECK(hipGetLastError());
  }
  {
    const unsigned nt = (unsigned)((n + 63) / 64);
    hipLaunchKernelGGL(k_write_factor64, dim3(nt, nt), dim3(256), 0, stream, (const double*)ws.A, n,
                       (const uint8_t*)ws.dead, H);
    F64CHECK(hipGetLastError());
  }
  return hipSuccess;
}

}  // namespace gptq
