// fp32 MFMA GEMM used by the trailing update of the column loop and by the
// blocked factor (panel product, trailing symmetric update, triangular inverse).
//
// Tile 128x128 per workgroup of 256 threads (4 waves in a 2x2 grid, 64x64 per
// wave as 2x2 blocks of v_mfma_f32_32x32x2_f32).  K is consumed in chunks of
// 16, staged k-major in LDS (As[k][m], Bs[k][n]) so that every MFMA operand
// read is 32 consecutive floats; chunks are double-buffered with the next
// chunk's global loads in flight during the current chunk's MFMAs.
#include "common.h"

namespace gptq {
namespace {

constexpr int BM = 128, BN = 128, BK = 16, PAD = 4;
constexpr int LDA_S = BM + PAD, LDB_S = BN + PAD;

struct Frag {
  float a[2][4];  // two float4 of A
  float b[2][4];  // two float4 of B
};

// Loads one BK-chunk of A (rows m0.., k0..) and B into registers.
// A: element idx = tid + 256 i (i = 0, 1): m = idx / 4, kq = idx % 4 -> A(m, 4kq .. 4kq+3).
// B k-major: idx -> k = idx / 32, nq = idx % 32 -> B(k, 4nq .. 4nq+3).
// B n-major: idx -> n = idx / 4, kq = idx % 4 -> B(4kq .. 4kq+3, n).
template <bool BK_MAJOR>
__device__ __forceinline__ void load_chunk(const GemmF32& g, const float* A, const float* B, int m0,
                                           int n0, int k0, int kend, bool vecA, bool vecB, Frag& f) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = tid + 256 * i;
    {
      const int m = idx >> 2, k = 4 * (idx & 3);
      const int gm = m0 + m, gk = k0 + k;
      const float* p = A + (int64_t)gm * g.lda + gk;
      if (gm < g.M && vecA && gk + 3 < kend) {
        float4 v = *reinterpret_cast<const float4*>(p);
        f.a[i][0] = v.x; f.a[i][1] = v.y; f.a[i][2] = v.z; f.a[i][3] = v.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) f.a[i][e] = (gm < g.M && gk + e < kend) ? p[e] : 0.f;
      }
    }
    if (BK_MAJOR) {
      const int k = idx >> 5, n = 4 * (idx & 31);
      const int gk = k0 + k, gn = n0 + n;
      const float* p = B + (int64_t)gk * g.ldb + gn;
      if (gk < kend && vecB && gn + 3 < g.N) {
        float4 v = *reinterpret_cast<const float4*>(p);
        f.b[i][0] = v.x; f.b[i][1] = v.y; f.b[i][2] = v.z; f.b[i][3] = v.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) f.b[i][e] = (gk < kend && gn + e < g.N) ? p[e] : 0.f;
      }
    } else {
      const int n = idx >> 2, k = 4 * (idx & 3);
      const int gn = n0 + n, gk = k0 + k;
      const float* p = B + (int64_t)gn * g.ldb + gk;
      if (gn < g.N && vecB && gk + 3 < kend) {
        float4 v = *reinterpret_cast<const float4*>(p);
        f.b[i][0] = v.x; f.b[i][1] = v.y; f.b[i][2] = v.z; f.b[i][3] = v.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) f.b[i][e] = (gn < g.N && gk + e < kend) ? p[e] : 0.f;
      }
    }
  }
}

template <bool BK_MAJOR>
__device__ __forceinline__ void store_chunk(float (*As)[LDA_S], float (*Bs)[LDB_S], const Frag& f) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = tid + 256 * i;
    {
      const int m = idx >> 2, k = 4 * (idx & 3);
#pragma unroll
      for (int e = 0; e < 4; ++e) As[k + e][m] = f.a[i][e];
    }
    if (BK_MAJOR) {
      const int k = idx >> 5, n = 4 * (idx & 31);
      *reinterpret_cast<float4*>(&Bs[k][n]) = make_float4(f.b[i][0], f.b[i][1], f.b[i][2], f.b[i][3]);
    } else {
      const int n = idx >> 2, k = 4 * (idx & 3);
#pragma unroll
      for (int e = 0; e < 4; ++e) Bs[k + e][n] = f.b[i][e];
    }
  }
}

template <bool BK_MAJOR>
__global__ __launch_bounds__(256) void k_gemm_f32(GemmF32 g) {
  __shared__ __attribute__((aligned(16))) float As[2][BK][LDA_S];
  __shared__ __attribute__((aligned(16))) float Bs[2][BK][LDB_S];

  int tm, tn;
  if (g.tri) {
    // lower-triangular tile enumeration: t -> (tm, tn), tn <= tm
    const int t = blockIdx.x;
    int r = (int)((sqrtf(8.f * (float)t + 1.f) - 1.f) * 0.5f);
    while ((r + 1) * (r + 2) / 2 <= t) ++r;
    while (r * (r + 1) / 2 > t) --r;
    tm = r;
    tn = t - r * (r + 1) / 2;
  } else {
    tn = blockIdx.x;
    tm = blockIdx.y;
  }
  const int z = blockIdx.z;
  const float* A = g.A + (int64_t)z * g.sA;
  const float* B = g.B + (int64_t)z * g.sB;
  float* C = g.C + (int64_t)z * g.sC;
  const int m0 = tm * BM, n0 = tn * BN;
  if (m0 >= g.M || n0 >= g.N) return;

  int kbeg = 0, kend = g.K;
  if (g.klo_n) kbeg = n0 < g.K ? n0 : g.K;
  if (g.khi_m) kend = (m0 + BM) < g.K ? (m0 + BM) : g.K;

  const bool vecA = ((g.lda & 3) == 0) && ((reinterpret_cast<uintptr_t>(A) & 15) == 0);
  const bool vecB = ((g.ldb & 3) == 0) && ((reinterpret_cast<uintptr_t>(B) & 15) == 0);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  if (kbeg < kend) {
    Frag f;
    load_chunk<BK_MAJOR>(g, A, B, m0, n0, kbeg, kend, vecA, vecB, f);
    store_chunk<BK_MAJOR>(As[0], Bs[0], f);
    __syncthreads();
    int buf = 0;
    for (int k0 = kbeg; k0 < kend; k0 += BK) {
      const bool more = k0 + BK < kend;
      if (more) load_chunk<BK_MAJOR>(g, A, B, m0, n0, k0 + BK, kend, vecA, vecB, f);
#pragma unroll
      for (int kk = 0; kk < BK / 2; ++kk) {
        const int kr = 2 * kk + (lane >> 5);
        float a0 = As[buf][kr][wm * 64 + (lane & 31)];
        float a1 = As[buf][kr][wm * 64 + 32 + (lane & 31)];
        float b0 = Bs[buf][kr][wn * 64 + (lane & 31)];
        float b1 = Bs[buf][kr][wn * 64 + 32 + (lane & 31)];
        acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
        acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
        acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
        acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
      }
      if (more) {
        store_chunk<BK_MAJOR>(As[buf ^ 1], Bs[buf ^ 1], f);
        __syncthreads();
        buf ^= 1;
      }
    }
  }

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + 32 * i + acc_row(r, lane);
        const int n = n0 + wn * 64 + 32 * j + acc_col(lane);
        if (m < g.M && n < g.N) {
          float* p = C + (int64_t)m * g.ldc + n;
          float v = g.alpha * acc[i][j][r];
          *p = g.beta ? (*p + v) : v;
        }
      }
}

}  // namespace

hipError_t gemm_f32(const GemmF32& g, hipStream_t stream) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return hipSuccess;
  const int tm = (g.M + BM - 1) / BM, tn = (g.N + BN - 1) / BN;
  dim3 grid;
  if (g.tri) {
    grid = dim3((unsigned)(tm * (tm + 1) / 2), 1, (unsigned)g.batch);
  } else {
    grid = dim3((unsigned)tn, (unsigned)tm, (unsigned)g.batch);
  }
  if (g.b_kmajor)
    hipLaunchKernelGGL(k_gemm_f32<true>, grid, dim3(256), 0, stream, g);
  else
    hipLaunchKernelGGL(k_gemm_f32<false>, grid, dim3(256), 0, stream, g);
  return hipGetLastError();
}

}  // namespace gptq
