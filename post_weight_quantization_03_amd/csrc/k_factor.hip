// Damping and the factor U (upper, positive diagonal, U^T U = inv(H_d)), on
// the device in fp32.
//
// Route: with P the index reversal, P H_d P = L L^T (ordinary lower
// Cholesky), so H_d = R R^T with R = P L P upper, and
// inv(H_d) = R^-T R^-1 = (R^-1)^T (R^-1).  R^-1 = P L^-1 P is upper with a
// positive diagonal, hence U = P L^-1 P: one Cholesky and one triangular
// inverse (2n^3/3 flops), and inv(H_d) is never formed.
//
//  1. k_damp_stats     one workgroup: dead columns (H_ii == 0 -> 1), lambda =
//                      damp * mean(diag) (fp64 sum in a fixed order).
//  2. k_reverse_damped A = P H_d P, lower triangle, fp32.
//  3. blocked right-looking Cholesky, nb = 128: k_chol_diag factors the
//     diagonal block in registers and LDS and writes its inverse into Minv;
//     the panel below becomes L_ik = A_ik Linv_kk^T (GEMM) and the trailing
//     lower tiles take A_ij -= L_ik L_jk^T (GEMM).
//  4. triangular inverse by doubling: with the 128-blocks of Minv inverted,
//     each level joins pairs of inverted diagonal blocks,
//     [P 0; C Q]^-1 = [P^-1 0; -Q^-1 C P^-1 Q^-1], as two batched GEMMs.
//  5. k_write_factor   U[i][j] = Minv[n-1-i][n-1-j] for i <= j into H, plus the
//     dead flags in H's strictly lower triangle.
#include "common.h"

namespace gptq {
namespace {

constexpr int NB = 128;

__global__ __launch_bounds__(1024) void k_damp_stats(const float* H, int64_t n, float damp, uint8_t* dead,
                                                     float* lam) {
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
  if (threadIdx.x == 0) *lam = (float)((double)damp * part[0] / (double)n);
}

// A[i][j] = H_d[n-1-i][n-1-j] for j <= i; rows in blockIdx.y, columns in grid-stride x.
__global__ void k_reverse_damped(const float* H, int64_t n, const uint8_t* dead, const float* lam, float* A) {
  const float l = *lam;
  for (int64_t i = blockIdx.y; i < n; i += gridDim.y) {
  const int64_t si = n - 1 - i;
  for (int64_t j = blockIdx.x * blockDim.x + threadIdx.x; j <= i; j += (int64_t)gridDim.x * blockDim.x) {
    const int64_t sj = n - 1 - j;
    float v;
    if (j == i) {
      const float d = H[si * n + si];
      v = (dead[si] ? 1.0f : d) + l;
    } else {
      v = H[si * n + sj];  // sj > si: the upper triangle of H
    }
    A[i * n + j] = v;
  }
  }
}

// Factor the diagonal block A[k0:k0+kb, k0:k0+kb] (lower) and write its inverse
// (lower, zeros above the diagonal) into Minv at the same place.
//
// 256 threads, tr = tid / 16, tc = tid % 16, each holding 8x8 elements in
// registers, one barrier per column, no data-dependent branches.
//
// Cholesky: thread owns rows tr + 16a and columns 8tc + b, so column c sits in
// register slot c % 8 of the threads with tc == c / 8 (a compile-time slot in
// a loop unrolled by 8).  The column is kept unscaled: at step c its owners
// publish it to LDS, then every thread applies
//   S[r][q] -= S[r][c] S[q][c] / S[c][c]   for c < q (and r > c)
// with masked operands; L[r][c] = S[r][c] / sqrt(S[c][c]) at the end.
// Inverse X = L^-1 by forward elimination of the identity: thread owns rows
// 8tr + a and columns tc + 16b, so row c is slot c % 8 of the threads with
// tr == c / 8; at step c the owners scale row c by 1/L[c][c] and publish it,
// then B[r][q] -= L[r][c] X[c][q] for r > c.
__global__ __launch_bounds__(256) void k_chol_diag(float* A, float* Minv, int64_t n, int64_t k0, int* status) {
  __shared__ float col[2][NB];
  __shared__ float dg[NB];
  __shared__ float Ls[NB][NB + 1];
  const int kb = (int)((n - k0) < NB ? (n - k0) : NB);
  const int tid = threadIdx.x;
  const int tr = tid >> 4, tc = tid & 15;
  float S[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int r = tr + 16 * a, q = 8 * tc + b;
      S[a][b] = (r < kb && q <= r) ? A[(k0 + r) * n + k0 + q] : ((r == q) ? 1.0f : 0.0f);
    }
  bool bad = false;
  for (int cb = 0; cb < NB / 8; ++cb) {
    if (8 * cb >= kb) break;
#pragma unroll
    for (int ci = 0; ci < 8; ++ci) {
      const int c = 8 * cb + ci;
      const int buf = ci & 1;
      if (tc == cb) {
#pragma unroll
        for (int a = 0; a < 8; ++a) col[buf][tr + 16 * a] = S[a][ci];
      }
      __syncthreads();
      float piv = col[buf][c];
      const bool ok = (piv > 0.0f) && (piv < INFINITY) && (c < kb);
      bad |= (c < kb) && !ok;
      piv = ok ? piv : 1.0f;
      const float rp = 1.0f / piv;
      float cq[8];
      const float4 c0 = *reinterpret_cast<const float4*>(&col[buf][8 * tc]);
      const float4 c1 = *reinterpret_cast<const float4*>(&col[buf][8 * tc + 4]);
      cq[0] = c0.x; cq[1] = c0.y; cq[2] = c0.z; cq[3] = c0.w;
      cq[4] = c1.x; cq[5] = c1.y; cq[6] = c1.z; cq[7] = c1.w;
#pragma unroll
      for (int b = 0; b < 8; ++b) cq[b] = (8 * tc + b > c) ? cq[b] * rp : 0.0f;
#pragma unroll
      for (int a = 0; a < 8; ++a) {
        if (16 * a + 15 <= c) continue;  // uniform: every row of slot a is done
        const int r = tr + 16 * a;
        const float lr = (r > c) ? col[buf][r] : 0.0f;
#pragma unroll
        for (int b = 0; b < 8; ++b) S[a][b] = fmaf(-lr, cq[b], S[a][b]);
      }
    }
  }
  if (bad && tid == 0) raise_status(status, GPTQ_ENOTPD);
  __syncthreads();  // the last step may still be reading col[]
  // diagonal of L
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int r = tr + 16 * a, q = 8 * tc + b;
      if (r == q && r < kb) {
        const float d = S[a][b];
        dg[r] = sqrtf((d > 0.0f && d < INFINITY) ? d : 1.0f);
      }
    }
  __syncthreads();
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int r = tr + 16 * a, q = 8 * tc + b;
      // beyond kb the block is padded with the identity, so the unrolled steps
      // past the last column divide by 1 and eliminate nothing
      float v = (r == q) ? 1.0f : 0.0f;
      if (r < kb && q < kb) v = (q < r) ? S[a][b] / dg[q] : ((q == r) ? dg[r] : 0.0f);
      Ls[r][q] = v;
    }
  __syncthreads();
  // inverse: rows 8tr + a, columns tc + 16b; B starts as the identity
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) S[a][b] = ((8 * tr + a) == (tc + 16 * b)) ? 1.0f : 0.0f;
  for (int cb = 0; cb < NB / 8; ++cb) {
    if (8 * cb >= kb) break;
#pragma unroll
    for (int ci = 0; ci < 8; ++ci) {
      const int c = 8 * cb + ci;
      const int buf = ci & 1;
      if (tr == cb) {
        const float rl = 1.0f / Ls[c][c];
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          S[ci][b] *= rl;
          col[buf][tc + 16 * b] = S[ci][b];
        }
      }
      __syncthreads();
      if (32 * (tid >> 6) + 31 > c) {  // uniform per wave: its rows are 32w .. 32w+31
        float rq[8];
#pragma unroll
        for (int b = 0; b < 8; ++b) rq[b] = col[buf][tc + 16 * b];
#pragma unroll
        for (int a = 0; a < 8; ++a) {
          const int r = 8 * tr + a;
          const float lm = (r > c && r < kb) ? Ls[r][c] : 0.0f;
#pragma unroll
          for (int b = 0; b < 8; ++b) S[a][b] = fmaf(-lm, rq[b], S[a][b]);
        }
      }
    }
  }
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int r = 8 * tr + a, q = tc + 16 * b;
      if (r < kb && q < kb) Minv[(k0 + r) * n + k0 + q] = (q <= r) ? S[a][b] : 0.0f;
    }
}

// U[i][j] = Minv[n-1-i][n-1-j] for j >= i, written into H; dead flags into the
// strictly lower slots H[i][i-1] (column i >= 1) and H[n-1][0] (column 0).
__global__ void k_write_factor(const float* Minv, int64_t n, const uint8_t* dead, float* H) {
  for (int64_t i = blockIdx.y; i < n; i += gridDim.y) {
    for (int64_t j = i + blockIdx.x * blockDim.x + threadIdx.x; j < n; j += (int64_t)gridDim.x * blockDim.x)
      H[i * n + j] = Minv[(n - 1 - i) * n + (n - 1 - j)];
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      if (i >= 1) H[i * n + i - 1] = dead[i] ? 1.0f : 0.0f;
      if (i == n - 1 && n >= 3) H[i * n + 0] = dead[0] ? 1.0f : 0.0f;
    }
  }
}

__global__ void k_dead_from_factor(const float* H, int64_t n, uint8_t* dead) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float f = (i >= 1) ? H[i * n + i - 1] : H[(n - 1) * n + 0];
  dead[i] = (f != 0.0f) ? 1 : 0;
}

__global__ void k_fill_i32(int* p, int64_t n, int v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void k_copy_status(const int* src, int32_t* dst) {
  if (threadIdx.x == 0) *dst = *src;
}

}  // namespace

// Scratch for the doubling levels: level s holds one s x s product per pair.
static int64_t doubling_scratch(int64_t n) {
  int64_t best = 0;
  for (int64_t s = NB; s < n; s *= 2) {
    const int64_t pairs = n / (2 * s) + ((n - (n / (2 * s)) * 2 * s - s) > 0 ? 1 : 0);
    if (pairs * s * s > best) best = pairs * s * s;
  }
  return best;
}

size_t factor_scratch_floats(int64_t n, int64_t* tmax) {
  const int64_t t = doubling_scratch(n);
  if (tmax) *tmax = t;
  return (size_t)(2 * n * n + t);
}

hipError_t fill_i32(int* p, int64_t n, int v, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_i32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, n, v);
  return hipGetLastError();
}

hipError_t copy_status(const int* src, int32_t* dst, hipStream_t stream) {
  hipLaunchKernelGGL(k_copy_status, dim3(1), dim3(64), 0, stream, src, dst);
  return hipGetLastError();
}

hipError_t dead_from_factor(const float* H, int64_t n, uint8_t* dead, hipStream_t stream) {
  hipLaunchKernelGGL(k_dead_from_factor, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, H, n, dead);
  return hipGetLastError();
}

#define FCHECK(x)                          \
  do {                                     \
    hipError_t e_ = (x);                   \
    if (e_ != hipSuccess) return e_;       \
  } while (0)

hipError_t factor_run(float* H, int64_t n, float damp, const FactorWs& ws, hipStream_t stream) {
  hipLaunchKernelGGL(k_damp_stats, dim3(1), dim3(1024), 0, stream, (const float*)H, n, damp, ws.dead, ws.lam);
  FCHECK(hipGetLastError());
  {
    const unsigned gx = (unsigned)((n + 255) / 256 < 16 ? (n + 255) / 256 : 16);
    hipLaunchKernelGGL(k_reverse_damped, dim3(gx, (unsigned)(n < 65535 ? n : 65535)), dim3(256), 0, stream, (const float*)H, n,
                       (const uint8_t*)ws.dead, (const float*)ws.lam, ws.A);
    FCHECK(hipGetLastError());
  }
  const int64_t nk = (n + NB - 1) / NB;
  for (int64_t k = 0; k < nk; ++k) {
    const int64_t k0 = k * NB;
    const int64_t kb = (n - k0) < NB ? (n - k0) : NB;
    hipLaunchKernelGGL(k_chol_diag, dim3(1), dim3(256), 0, stream, ws.A, ws.Minv, n, k0, ws.status);
    FCHECK(hipGetLastError());
    const int64_t rest = n - k0 - kb;
    if (rest <= 0) break;
    // panel: A[k0+kb:, k0:k0+kb] <- A[..] * Linv_kk^T   (in place, one tile column)
    GemmF32 p{};
    p.A = ws.A + (k0 + kb) * n + k0;
    p.lda = n;
    p.B = ws.Minv + k0 * n + k0;
    p.ldb = n;
    p.b_kmajor = 0;  // B(k, c) = Linv[c][k]
    p.C = ws.A + (k0 + kb) * n + k0;
    p.ldc = n;
    p.M = (int)rest;
    p.N = (int)kb;
    p.K = (int)kb;
    p.alpha = 1.0f;
    p.beta = 0;
    p.batch = 1;
    FCHECK(gemm_f32(p, stream));
    // trailing lower tiles: A22 -= L21 L21^T
    GemmF32 t{};
    t.A = ws.A + (k0 + kb) * n + k0;
    t.lda = n;
    t.B = ws.A + (k0 + kb) * n + k0;
    t.ldb = n;
    t.b_kmajor = 0;  // B(k, c) = L21[c][k]
    t.C = ws.A + (k0 + kb) * n + (k0 + kb);
    t.ldc = n;
    t.M = (int)rest;
    t.N = (int)rest;
    t.K = (int)kb;
    t.alpha = -1.0f;
    t.beta = 1;
    t.tri = 1;
    t.batch = 1;
    FCHECK(gemm_f32(t, stream));
  }
  // triangular inverse by doubling over the 128-blocks already inverted in Minv
  for (int64_t s = NB; s < n; s *= 2) {
    const int64_t pairs_full = n / (2 * s);
    const int64_t a_last = pairs_full * 2 * s;  // start of a ragged pair, if any
    const int64_t s2_last = n - a_last - s;      // bottom size of that pair (<= 0: none)
    for (int pass = 0; pass < 2; ++pass) {
      const int64_t cnt = pass == 0 ? pairs_full : (s2_last > 0 ? 1 : 0);
      if (cnt == 0) continue;
      const int64_t a = pass == 0 ? 0 : a_last;
      const int64_t s2 = pass == 0 ? s : s2_last;
      // T = L21 * P      (s2 x s) = (s2 x s)(s x s), P lower
      GemmF32 g1{};
      g1.A = ws.A + (a + s) * n + a;
      g1.lda = n;
      g1.sA = 2 * s * n + 2 * s;
      g1.B = ws.Minv + a * n + a;
      g1.ldb = n;
      g1.sB = 2 * s * n + 2 * s;
      g1.b_kmajor = 1;
      g1.C = ws.T;
      g1.ldc = s;
      g1.sC = 0;
      g1.M = (int)s2;
      g1.N = (int)s;
      g1.K = (int)s;
      g1.alpha = 1.0f;
      g1.beta = 0;
      g1.klo_n = 1;
      g1.batch = 1;
      // M21 = -Q * T     (s2 x s) = (s2 x s2)(s2 x s), Q lower
      GemmF32 g2{};
      g2.A = ws.Minv + (a + s) * n + (a + s);
      g2.lda = n;
      g2.sA = 2 * s * n + 2 * s;
      g2.B = ws.T;
      g2.ldb = s;
      g2.sB = 0;
      g2.b_kmajor = 1;
      g2.C = ws.Minv + (a + s) * n + a;
      g2.ldc = n;
      g2.sC = 2 * s * n + 2 * s;
      g2.M = (int)s2;
      g2.N = (int)s;
      g2.K = (int)s2;
      g2.alpha = -1.0f;
      g2.beta = 0;
      g2.khi_m = 1;
      g2.batch = 1;
      // each pair m has its own s x s slice of T
      g1.C = ws.T + (pass == 0 ? 0 : pairs_full * s * s);
      g1.sC = s * s;
      g2.B = g1.C;
      g2.sB = s * s;
      g1.batch = (int)cnt;
      g2.batch = (int)cnt;
      FCHECK(gemm_f32(g1, stream));
      FCHECK(gemm_f32(g2, stream));
    }
  }
  {
    const unsigned gx = (unsigned)((n + 255) / 256 < 16 ? (n + 255) / 256 : 16);
    hipLaunchKernelGGL(k_write_factor, dim3(gx, (unsigned)(n < 65535 ? n : 65535)), dim3(256), 0, stream, (const float*)ws.Minv, n,
                       (const uint8_t*)ws.dead, H);
    FCHECK(hipGetLastError());
  }
  return hipSuccess;
}

}  // namespace gptq
