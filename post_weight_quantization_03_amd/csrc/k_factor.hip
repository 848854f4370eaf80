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

// Factor the diagonal block A[k0:k0+kb, k0:k0+kb] (lower) and write the
// inverse of its Cholesky factor (lower, zeros above the diagonal) into Minv
// at the same place.
//
// 256 threads, tr = tid / 16, tc = tid % 16; each thread holds the elements
// (tr + 16a, tc + 16b), a, b = 0..7, of two 128x128 register arrays: S, the
// block under elimination, and B, the inverse being formed.  Column c of the
// block lives in register slot c / 16 of the lanes with tc == c % 16; the
// slot is a template parameter, so finished rows and columns are skipped at
// compile time.
//
// Step c (one barrier) does two things:
//  * Cholesky, right-looking with the column left unscaled: the owners of
//    column c publish it, then S[r][q] -= S[r][c] S[q][c] / S[c][c] for
//    r, q > c.  L[r][c] = S[r][c] / sqrt(S[c][c]).
//  * inverse by forward elimination of the identity, one row behind: the
//    owners of row c-1 scale it by 1 / L[c-1][c-1] and publish it, then
//    B[r][q] -= L[r][c-1] X[c-1][q] for r > c-1, q <= c-1.
// L itself is never stored.  Columns are triple-buffered in LDS (step c reads
// columns c and c-1 while step c+1 publishes column c+1), rows double-buffered.
// Beyond kb the block is padded with the identity.  Pivot reciprocals use the
// hardware reciprocal and reciprocal square root (1 ulp).
namespace chol {

struct Ctx {
  float S[8][8];
  float B[8][8];
  int tr, tc, kb;
  bool bad;
};

__device__ __forceinline__ float sane(float piv) { return (piv > 0.0f && piv < INFINITY) ? piv : 1.0f; }

// K: slot of column c = 16K + L.  KP: slot of c - 1.
template <int K, int KP>
__device__ __forceinline__ void step(Ctx& x, float (*col)[NB], float (*row)[NB], int c) {
  const int L = c & 15, P = c - 1, LP = P & 15;
  float* colC = col[c % 3];
  const float* colP = col[(c + 2) % 3];
  float* rowP = row[P & 1];
  // publish column c (Cholesky) and row c - 1 of the inverse
  if (K < 8 && x.tc == L) {
#pragma unroll
    for (int a = (K < 8 ? K : 7); a < 8; ++a) colC[x.tr + 16 * a] = x.S[a][K < 8 ? K : 7];
  }
  if (KP >= 0 && c >= 1 && x.tr == LP) {
    const float rl = __builtin_amdgcn_rsqf(sane(colP[P]));
#pragma unroll
    for (int b = 0; b <= (KP >= 0 ? KP : 0); ++b) {
      x.B[KP >= 0 ? KP : 0][b] *= rl;
      rowP[x.tc + 16 * b] = x.B[KP >= 0 ? KP : 0][b];
    }
  }
  __syncthreads();
  if (K < 8) {
    constexpr int KK = K < 8 ? K : 7;
    const float piv0 = colC[c];
    x.bad |= (c < x.kb) && !(piv0 > 0.0f && piv0 < INFINITY);
    const float rp = __builtin_amdgcn_rcpf(sane(piv0));
    float cq[8];
#pragma unroll
    for (int b = KK; b < 8; ++b) {
      const float v = colC[x.tc + 16 * b] * rp;
      cq[b] = (b == KK && x.tc <= L) ? 0.0f : v;
    }
#pragma unroll
    for (int a = KK; a < 8; ++a) {
      float lr = colC[x.tr + 16 * a];
      if (a == KK && x.tr <= L) lr = 0.0f;
#pragma unroll
      for (int b = KK; b < 8; ++b) x.S[a][b] = fmaf(-lr, cq[b], x.S[a][b]);
    }
  }
  if (KP >= 0 && c >= 1) {
    constexpr int KQ = KP >= 0 ? KP : 0;
    const float rl = __builtin_amdgcn_rsqf(sane(colP[P]));
    float rq[8];
#pragma unroll
    for (int b = 0; b <= KQ; ++b) rq[b] = rowP[x.tc + 16 * b];
#pragma unroll
    for (int a = KQ; a < 8; ++a) {
      float lm = colP[x.tr + 16 * a] * rl;
      if (a == KQ && x.tr <= LP) lm = 0.0f;
#pragma unroll
      for (int b = 0; b <= KQ; ++b) x.B[a][b] = fmaf(-lm, rq[b], x.B[a][b]);
    }
  }
}

template <int K>
__device__ __forceinline__ void slot(Ctx& x, float (*col)[NB], float (*row)[NB]) {
  const int c0 = 16 * K;
  if (c0 > x.kb) return;
  step<K, K - 1>(x, col, row, c0);  // row c0 - 1 belongs to the previous slot
  if (K < 8) {
    for (int l = 1; l < 16; ++l) {
      if (c0 + l > x.kb) return;
      step<K, K>(x, col, row, c0 + l);
    }
  }
}

}  // namespace chol

__global__ __launch_bounds__(256) void k_chol_diag(float* A, float* Minv, int64_t n, int64_t k0, int* status) {
  __shared__ float col[3][NB];
  __shared__ float row[2][NB];
  chol::Ctx x;
  x.kb = (int)((n - k0) < NB ? (n - k0) : NB);
  x.tr = threadIdx.x >> 4;
  x.tc = threadIdx.x & 15;
  x.bad = false;
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int r = x.tr + 16 * a, q = x.tc + 16 * b;
      x.S[a][b] = (r < x.kb && q <= r) ? A[(k0 + r) * n + k0 + q] : ((r == q) ? 1.0f : 0.0f);
      x.B[a][b] = (r == q) ? 1.0f : 0.0f;
    }
  chol::slot<0>(x, col, row);
  chol::slot<1>(x, col, row);
  chol::slot<2>(x, col, row);
  chol::slot<3>(x, col, row);
  chol::slot<4>(x, col, row);
  chol::slot<5>(x, col, row);
  chol::slot<6>(x, col, row);
  chol::slot<7>(x, col, row);
  chol::slot<8>(x, col, row);  // the inverse's last row
  if (x.bad) raise_status(status, GPTQ_ENOTPD);
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int r = x.tr + 16 * a, q = x.tc + 16 * b;
      if (r < x.kb && q < x.kb) Minv[(k0 + r) * n + k0 + q] = (q <= r) ? x.B[a][b] : 0.0f;
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
