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
//  2. k_reverse_damped A = P H_d P in the lower triangle, zeros above, fp32.
//  3. blocked right-looking Cholesky, nb = 128, with the triangular inverse
//     folded in.  Per block k: k_trsm_block solves every row of block column
//     k against L_kk (the panel below, L_ik = A_ik L_kk^-T; the rows of the
//     block, L_kk^-T itself; the rows above, the block column k of L^-T, which
//     accumulates in A's upper triangle); then one GEMM takes all rows of the
//     columns right of block k, A[r][j] -= A[r][k0:c1] L[j][k0:c1]^T: below c1
//     the Cholesky trailing update, above it the next term of the inverse's
//     right-looking block forward substitution, X_ij -= L_ik X_kj in the
//     transposed layout.  That GEMM runs in the same launch as the factor of
//     block k+1 (k_factor_step, look-ahead; k_potrf_diag factors a diagonal
//     block and hands L^T to the solves in a buffer of its own).  The
//     inverse's work thus fills the CUs that the Cholesky's late, narrow
//     steps leave idle, and nothing of it is left after the loop.
//     On large steps the GEMM is lazy in two levels: block column k+1 (the
//     next to be solved) takes every panel at once, the columns past it only
//     every FACTOR_LAZY panels, with K = 128 FACTOR_LAZY, so the trailing
//     matrix is read and written once per FACTOR_LAZY panels instead of once
//     per panel.
//     A row of a pending panel's own block is an inverse row only for the
//     panels from its own block on (before it, its entries right of the
//     diagonal were above the trailing matrix's lower triangle, which the
//     Cholesky update leaves alone), so such rows start their K range at
//     their own block (GemmF32::kfl_lo / kfl_hi).
//  4. k_write_factor   U[i][j] = Y[n-1-j][n-1-i] for i <= j into H (Y = L^-T,
//     A's upper triangle), plus the dead flags in H's strictly lower triangle.
#include <utility>

#include "gemm_tile.h"

namespace gptq {
namespace {

constexpr int NB = 128;
constexpr int64_t FACTOR_LAZY = 2;  // panels per update of the columns past the next block
// Deferral pays only on steps whose GEMM is large: more tiles than four rounds
// of the chip's 256 CUs.  On smaller steps the doubled K of the update that
// follows costs more than the saved pass over the trailing matrix (measured at
// n = 4096, where every step is below this).
constexpr int64_t FACTOR_LAZY_TILES = 4 * 256;

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

// A[i][j] = H_d[n-1-i][n-1-j] for j <= i and 0 above the diagonal (where the
// factor accumulates the transposed inverse), four columns a thread: the
// source is the float4 of row n-1-i ending at column n-1-j, read backwards.
// Needs n % 4 == 0 and 16-byte aligned H and A.
__global__ void k_reverse_damped4(const float* H, int64_t n, const uint8_t* dead, const float* lam, float* A) {
  const float l = *lam;
  for (int64_t i = blockIdx.y; i < n; i += gridDim.y) {
    const int64_t si = n - 1 - i;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; 4 * q < n; q += (int64_t)gridDim.x * blockDim.x) {
      float o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (4 * q <= i) {
        const float4 v = *reinterpret_cast<const float4*>(H + si * n + (n - 4 - 4 * q));
        o[0] = v.w; o[1] = v.z; o[2] = v.y; o[3] = v.x;
        const int64_t e = i - 4 * q;  // the diagonal, if in this chunk
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          if (f == e) o[f] = (dead[si] ? 1.0f : o[f]) + l;
          if (f > e) o[f] = 0.0f;
        }
      }
      *reinterpret_cast<float4*>(A + i * n + 4 * q) = make_float4(o[0], o[1], o[2], o[3]);
    }
  }
}

__global__ void k_reverse_damped(const float* H, int64_t n, const uint8_t* dead, const float* lam, float* A) {
  const float l = *lam;
  for (int64_t i = blockIdx.y; i < n; i += gridDim.y) {
  const int64_t si = n - 1 - i;
  for (int64_t j = blockIdx.x * blockDim.x + threadIdx.x; j < n; j += (int64_t)gridDim.x * blockDim.x) {
    const int64_t sj = n - 1 - j;
    float v = 0.0f;
    if (j == i) {
      const float d = H[si * n + si];
      v = (dead[si] ? 1.0f : d) + l;
    } else if (j < i) {
      v = H[si * n + sj];  // sj > si: the upper triangle of H
    }
    A[i * n + j] = v;
  }
  }
}

// ------------------------------------------------------------------ diagonal block

// Cholesky of the diagonal block A[k0:k0+kb, k0:k0+kb] (lower triangle in,
// kb <= 128, padded with the identity beyond kb).  L^T goes to a 128 x 128
// buffer of its own (row-major, zeros below the diagonal, the identity past
// kb), from which the triangular solves of the block read it; A is not
// written.
//
// 16-column panels, right-looking.  A panel is factored wave-synchronously in
// registers: each wave it needs carries the panel's 16 diagonal rows in lanes
// 0..15 (the same in every such wave) and 48 rows below them in lanes 16..63,
// a row per lane, the row's 16 panel values in 16 VGPRs.  The panel is
// eliminated unscaled: step c reads the pivot d_c = a_cc from lane c and the
// entries a_jc of the later diagonal rows from lanes j with readlane, and
// every lane subtracts (a_ic / d_c) a_jc from its column j.  A step's
// dependent chain is readlane, reciprocal, multiply, FMA; the scaling of
// column c by 1/sqrt(d_c) into L waits for the end of the panel.  No barrier
// and no LDS traffic inside a panel.  The diagonal rows' lanes collect
// garbage in their entries above the diagonal, which no step reads.
//
// The panel's L then goes to LDS twice: in place (for the trailing update)
// and transposed into the block's upper triangle (a lane's row becomes a
// column there, so consecutive lanes write consecutive addresses).  The
// trailing lower 16x16 tiles take A_ij -= L_i L_j^T on
// v_mfma_f32_16x16x4f32, each wave loading all of its tiles' operands before
// its first MFMA.  Two barriers per panel.
//
// A pivot that is not positive and finite makes its diagonal entry
// d * rsq(d) NaN (0 * inf, inf * 0, or rsq of a negative), so one check of
// L's diagonal at the end finds it.
constexpr int PB = 16;      // panel width
constexpr int LP = NB + 1;  // LDS pitch: a column read by 16 lanes hits 16 banks

__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// waves holding rows of panel P: 48 rows below the diagonal rows per wave
template <int P>
constexpr int panel_waves() {
  return (NB - PB * (P + 1) + 47) / 48 > 1 ? (NB - PB * (P + 1) + 47) / 48 : 1;
}

template <int P>
__device__ __forceinline__ void potrf_panel(float (*As)[LP], int wave, int lane) {
  if (wave >= panel_waves<P>()) return;
  const int row = lane < PB ? PB * P + lane : PB * P + PB + 48 * wave + (lane - PB);
  const bool act = row < NB;
  float a[PB];
#pragma unroll
  for (int c = 0; c < PB; ++c) a[c] = act ? As[row][PB * P + c] : 0.0f;
  float piv[PB];
#pragma unroll
  for (int c = 0; c < PB; ++c) {
    const float d = readlane_f(a[c], c);
    piv[c] = d;
    float s[PB];
#pragma unroll
    for (int j = c + 1; j < PB; ++j) s[j] = readlane_f(a[c], j);
    const float t = a[c] * __builtin_amdgcn_rcpf(d);
#pragma unroll
    for (int j = c + 1; j < PB; ++j) a[j] = fmaf(-t, s[j], a[j]);
  }
#pragma unroll
  for (int c = 0; c < PB; ++c) a[c] *= __builtin_amdgcn_rsqf(piv[c]);
  // rows below the diagonal rows from every wave; the diagonal rows (their
  // lower part) once, from wave 0
  if (act && (lane >= PB || wave == 0)) {
#pragma unroll
    for (int c = 0; c < PB; ++c) {
      if (lane >= PB || c <= lane) {
        As[row][PB * P + c] = a[c];
        As[PB * P + c][row] = a[c];
      }
    }
  }
}

template <int P>
__device__ __forceinline__ void potrf_update(float (*As)[LP], int wave, int lane) {
  constexpr int T0 = P + 1, NT = NB / PB - T0, NTILES = NT * (NT + 1) / 2, U = (NTILES + 3) / 4;
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const int i16 = lane & 15, g = lane >> 4;
  // v_mfma_f32_16x16x4f32: lane supplies A[i16][g] and B[g][i16] and holds
  // D[4g + r][i16].  Tile t of the lower triangle (row-major over tile rows
  // T0..7) goes to wave t % 4; a wave with fewer tiles repeats its last one
  // and does not store it.
  int ti[U], tj[U];
  f32x4 acc[U];
  float av[U][PB / 4], bv[U][PB / 4];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int t = wave + 4 * u < NTILES ? wave + 4 * u : NTILES - 1;
    int r = 0;
    while ((r + 1) * (r + 2) / 2 <= t) ++r;
    ti[u] = r + T0;
    tj[u] = t - r * (r + 1) / 2 + T0;
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[u][q] = As[PB * ti[u] + 4 * g + q][PB * tj[u] + i16];
#pragma unroll
    for (int kk = 0; kk < PB / 4; ++kk) {
      av[u][kk] = As[PB * ti[u] + i16][PB * P + 4 * kk + g];
      bv[u][kk] = As[PB * tj[u] + i16][PB * P + 4 * kk + g];
    }
  }
#pragma unroll
  for (int kk = 0; kk < PB / 4; ++kk)
#pragma unroll
    for (int u = 0; u < U; ++u)
      acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(-av[u][kk], bv[u][kk], acc[u], 0, 0, 0);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (wave + 4 * u < NTILES) {
#pragma unroll
      for (int q = 0; q < 4; ++q) As[PB * ti[u] + 4 * g + q][PB * tj[u] + i16] = acc[u][q];
    }
  }
}

template <int P>
__device__ __forceinline__ void potrf_step(float (*As)[LP], int wave, int lane, unsigned long long* tr) {
  potrf_panel<P>(As, wave, lane);
  __syncthreads();
  GPTQ_TRACE_ONLY(tr[2 + 2 * P] = __builtin_amdgcn_s_memrealtime();)  // panel P
  if constexpr (P + 1 < NB / PB) {
    potrf_update<P>(As, wave, lane);
    __syncthreads();
    GPTQ_TRACE_ONLY(tr[3 + 2 * P] = __builtin_amdgcn_s_memrealtime();)  // its update
    potrf_step<P + 1>(As, wave, lane, tr);
  }
}

// Whole blocks with 16-byte rows move as float4, all loads of a thread in
// flight at once; a ragged last block goes element by element.
__device__ __forceinline__ bool block_vec(const float* A, int64_t n, int kb) {
  return kb == NB && (n & 3) == 0 && (reinterpret_cast<uintptr_t>(A) & 15) == 0;
}

constexpr int POTRF_LDS = NB * LP * 4;

__device__ __forceinline__ void potrf_diag(const float* A, int64_t n, int64_t k0, float* Lt, int* status, char* lds) {
  // stamps: start, loaded, then panel / update pairs, written
  unsigned long long tr[2 + 2 * (NB / PB) - 1 + 1];
  GPTQ_TRACE_ONLY(tr[0] = __builtin_amdgcn_s_memrealtime();)
  float(*As)[LP] = reinterpret_cast<float(*)[LP]>(lds);
  const int kb = (int)((n - k0) < NB ? (n - k0) : NB);
  const int tid = threadIdx.x;
  if (block_vec(A, n, kb)) {
    constexpr int PER = NB * NB / 4 / 256;
    float4 v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + 256 * i, r = idx >> 5, q = 4 * (idx & 31);
      v[i] = *reinterpret_cast<const float4*>(A + (k0 + r) * n + k0 + q);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + 256 * i, r = idx >> 5, q = 4 * (idx & 31);
      // the block's upper triangle holds no data yet: zeros there
      As[r][q + 0] = q + 0 <= r ? v[i].x : 0.0f;
      As[r][q + 1] = q + 1 <= r ? v[i].y : 0.0f;
      As[r][q + 2] = q + 2 <= r ? v[i].z : 0.0f;
      As[r][q + 3] = q + 3 <= r ? v[i].w : 0.0f;
    }
  } else {
    for (int idx = tid; idx < NB * NB; idx += 256) {
      const int r = idx >> 7, q = idx & (NB - 1);
      float v = (r == q) ? 1.0f : 0.0f;
      if (r < kb && q <= r) v = A[(k0 + r) * n + k0 + q];
      As[r][q] = v;
    }
  }
  __syncthreads();
  GPTQ_TRACE_ONLY(tr[1] = __builtin_amdgcn_s_memrealtime();)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  potrf_step<0>(As, wave, lane, tr);
  if (tid < kb) {
    const float d = As[tid][tid];
    if (!(d > 0.0f && d < INFINITY)) raise_status(status, GPTQ_ENOTPD);
  }
  // L^T, whole rows
#pragma unroll 4
  for (int i = 0; i < NB * NB / 4 / 256; ++i) {
    const int idx = tid + 256 * i, r = idx >> 5, q = 4 * (idx & 31);
    float4 v;
    v.x = q + 0 >= r ? As[r][q + 0] : 0.0f;
    v.y = q + 1 >= r ? As[r][q + 1] : 0.0f;
    v.z = q + 2 >= r ? As[r][q + 2] : 0.0f;
    v.w = q + 3 >= r ? As[r][q + 3] : 0.0f;
    *reinterpret_cast<float4*>(Lt + r * NB + q) = v;
  }
  GPTQ_TRACE_ONLY(tr[2 * (NB / PB) + 1] = __builtin_amdgcn_s_memrealtime();
                  trace_write(TR_POTRF, k0 / NB, tr, 2 * (NB / PB) + 2);)
}

__global__ __launch_bounds__(256) void k_potrf_diag(const float* A, int64_t n, int64_t k0, float* Lt, int* status) {
  __shared__ __attribute__((aligned(16))) char lds[POTRF_LDS];
  potrf_diag(A, n, k0, Lt, status, lds);
}

// One step of the blocked factor with look-ahead, block k (columns
// [k0, c1)): one GEMM over all rows and the columns right of the block,
//   A[r][j] -= A[r][k0:c1] L[j][k0:c1]^T   (r in [0, n), j in [c1, n)),
// beside the factor of block k+1.  Rows r >= c1 are the Cholesky trailing
// update A22 -= L21 L21^T, lower tiles only.  Rows r < c1 accumulate the
// inverse: there A[r][k0:c1] holds finished entries of L^-T (transposed
// inverse, upper triangle), and A[r][j] the running sums that the solve of
// block column j finishes.  Block k+1's diagonal block has been updated by a
// small launch before this one; workgroup 0 factors it while the other
// workgroups take the 128-tiles: the lower tiles of the trailing matrix but
// its first (that diagonal block), then the rectangle above c1 (`rrows` tile
// rows of `nt` tiles), row-major.  The tiles run on bf16 matrix cores with
// both operands split three ways in registers (gemm_tile.h, fp32 accuracy).
// (64-tiles, which fill the CUs more evenly when the tiles are few, measured
// slower here: with K = 128 a tile is mostly its fixed costs.)
constexpr int cmax(int a, int b) { return a > b ? a : b; }

// More than half of the CU's LDS per workgroup: one workgroup per CU, so the
// diagonal factor never shares its CU with a tile (sharing one made the factor
// up to 1.9x slower; the tiles lose less than that gains).
__global__ __launch_bounds__(256) void k_factor_step(GemmF32 g, int ntri, int rrows, int nt, int near_only,
                                                     const float* A, int64_t n, int64_t k0n, float* Lt,
                                                     int* status) {
  __shared__ __attribute__((aligned(16))) char lds[cmax(96 * 1024, cmax(POTRF_LDS, gemm_tile_lds<128>()))];
  if (blockIdx.x == 0) {
    potrf_diag(A, n, k0n, Lt, status, lds);
    return;
  }
  GPTQ_TRACE_DECL;
  GPTQ_TRACE_STAMP();
  const int u = (int)blockIdx.x - 1;
  if (near_only) {
    // tile column 0 only (block column k+1): the lower tiles below its
    // diagonal block, then the rectangle above
    if (u < nt - 1)
      gemm_tile<128, false, true>(g, rrows + u + 1, 0, 0, lds);
    else
      gemm_tile<128, false, true>(g, u - (nt - 1), 0, 0, lds);
    GPTQ_TRACE_STAMP();
    GPTQ_TRACE_WRITE(TR_TILE, k0n / NB);
    return;
  }
  if (u < ntri - 1) {
    const int t = u + 1;
    int r = (int)((sqrtf(8.f * (float)t + 1.f) - 1.f) * 0.5f);
    while ((r + 1) * (r + 2) / 2 <= t) ++r;
    while (r * (r + 1) / 2 > t) --r;
    gemm_tile<128, false, true>(g, rrows + r, t - r * (r + 1) / 2, 0, lds);
  } else {
    const int v = u - (ntri - 1);
    gemm_tile<128, false, true>(g, v / nt, v % nt, 0, lds);
  }
  GPTQ_TRACE_STAMP();
  GPTQ_TRACE_WRITE(TR_TILE, k0n / NB);
}

// Look-ahead update of block k+1's diagonal block, D -= P P^T, with P =
// A[c1:c1+kb1, k0:k0+128] (that block's rows of the panel just solved) and D =
// A[c1:c1+kb1, c1:c1+kb1]: lower 32 x 32 tiles, the diagonal tiles whole.  One
// workgroup per tile; its four waves split K = 128 in quarters of 16
// v_mfma_f32_32x32x2_f32 steps, lane half h of step s taking k = 32w + 16h + s
// (the order of k is free), so a lane's operands are four contiguous float4
// of each row, all in flight at once with the workgroup's elements of D.  The
// quarters are summed through LDS in a fixed order.  On the factor's critical
// path, so it is built for latency.
template <int PASSES>
__global__ __launch_bounds__(256) void k_diag_update(float* A, int64_t n, int64_t k0, int64_t c1, int kb1) {
  __shared__ float part[4][32 * 32];
  GPTQ_TRACE_DECL;
  GPTQ_TRACE_STAMP();
  const int t = blockIdx.x;
  int ti = 0;
  while ((ti + 1) * (ti + 2) / 2 <= t) ++ti;
  const int tj = t - ti * (ti + 1) / 2;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, j = lane & 31;
  const int ra = 32 * ti + j, rb = 32 * tj + j;
  const int kq = 32 * w + 16 * h;
  const bool vec = (n & 3) == 0 && (k0 & 3) == 0 && (reinterpret_cast<uintptr_t>(A) & 15) == 0;
  // pass p covers k0 + 128 p .. k0 + 128 p + 127 (PASSES pending panels)
  float a[PASSES][16], b[PASSES][16];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int64_t kp = k0 + 128 * p + kq;
    if (vec) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 va = ra < kb1 ? *reinterpret_cast<const float4*>(A + (c1 + ra) * n + kp + 4 * q)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
        const float4 vb = rb < kb1 ? *reinterpret_cast<const float4*>(A + (c1 + rb) * n + kp + 4 * q)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
        a[p][4 * q + 0] = va.x; a[p][4 * q + 1] = va.y; a[p][4 * q + 2] = va.z; a[p][4 * q + 3] = va.w;
        b[p][4 * q + 0] = vb.x; b[p][4 * q + 1] = vb.y; b[p][4 * q + 2] = vb.z; b[p][4 * q + 3] = vb.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        a[p][e] = ra < kb1 ? A[(c1 + ra) * n + kp + e] : 0.0f;
        b[p][e] = rb < kb1 ? A[(c1 + rb) * n + kp + e] : 0.0f;
      }
    }
  }
  // this thread's four elements of D, read now so that their latency hides too
  float dv[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid + 256 * q, gi = 32 * ti + (e >> 5), gj = 32 * tj + (e & 31);
    dv[q] = (gi < kb1 && gj < kb1) ? A[(c1 + gi) * n + c1 + gj] : 0.0f;
  }
  // two accumulators (even and odd steps), added at the end
  f32x16 acc0, acc1;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc0[r] = acc1[r] = 0.0f;
#pragma unroll
  for (int p = 0; p < PASSES; ++p)
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a[p][e], b[p][e], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a[p][e + 1], b[p][e + 1], acc1, 0, 0, 0);
    }
#pragma unroll
  for (int r = 0; r < 16; ++r) part[w][acc_row(r, lane) * 32 + j] = acc0[r] + acc1[r];
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid + 256 * q, gi = 32 * ti + (e >> 5), gj = 32 * tj + (e & 31);
    const float sum = ((part[0][e] + part[1][e]) + part[2][e]) + part[3][e];
    if (gi < kb1 && gj < kb1) A[(c1 + gi) * n + c1 + gj] = dv[q] - sum;
  }
  GPTQ_TRACE_STAMP();
  GPTQ_TRACE_WRITE(TR_DIAG, c1 / NB);
}

// ------------------------------------------------------------------ triangular solves

// Rows y = b L^-T for block k's L, i.e. L y^T = b^T by forward substitution,
// right-looking: y_j = b_j / L_jj, then b_m -= y_j L_mj for m > j.  L^T comes
// from the factor's buffer.  The same layout as the column loop: a 64-lane wave
// holds 4 rows, 16 lanes a row, 8 consecutive columns per lane; y_j reaches
// the row's lanes by a DPP row broadcast; L^T sits in LDS without its
// diagonal, and the row of step j+1 is read during step j.  Column j is final
// after step j, so y is formed after the loop as b * (1 / L_jj).
//
// One launch takes every row of block column k (columns [k0, k0 + kb)):
//   rows below the block: the panel, L_ik = A_ik L_kk^-T, in place;
//   rows above it: the block column of the transposed inverse, finished in
//     place from the sums the earlier steps accumulated there;
//   rows of the block: b = e_r, y = row r of L_kk^-T, written over the
//     block's row r (zeros left of the diagonal).
template <int O>
__device__ __forceinline__ float row_bcast(float v) {
  return __builtin_amdgcn_update_dpp(0.0f, v, 0x150 + O, 0xf, 0xf, false);
}

struct TrsmLane {
  float b[8], ru[8];
  float4 un[2];
  int t;
};

template <int J>
__device__ __forceinline__ void trsm_step(TrsmLane& L, const float (*Lt)[NB]) {
  constexpr int O = J >> 3, SL = J & 7, NX = (J + 1) & 7;
  const float4 u0 = L.un[0], u1 = L.un[1];
  if constexpr (J + 1 < NB) {
    L.un[0] = *reinterpret_cast<const float4*>(&Lt[J + 1][8 * L.t]);
    L.un[1] = *reinterpret_cast<const float4*>(&Lt[J + 1][8 * L.t + 4]);
  }
  const float yb = row_bcast<O>(L.b[SL] * L.ru[SL]);
  const float uu[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
  L.b[NX] = fmaf(-yb, uu[NX], L.b[NX]);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (i != NX) L.b[i] = fmaf(-yb, uu[i], L.b[i]);
}

template <int... Js>
__device__ __forceinline__ void trsm_steps(TrsmLane& L, const float (*Lt)[NB], std::integer_sequence<int, Js...>) {
  (trsm_step<Js>(L, Lt), ...);
}

// 16 rows a workgroup (4 waves): one wave a SIMD keeps each row's 128-step
// chain at full issue rate (32-row workgroups, two waves a SIMD, measured
// slower per launch at n = 4096 and 11008).
constexpr int TRSM_THREADS = 256;
constexpr int TRSM_ROWS = TRSM_THREADS / 16;

__global__ __launch_bounds__(TRSM_THREADS) void k_trsm_block(float* A, const float* Ltk, int64_t n, int64_t k0,
                                                             int kb) {
  __shared__ __attribute__((aligned(16))) float Lt[NB][NB];
  __shared__ float rL[NB];
  GPTQ_TRACE_DECL;
  GPTQ_TRACE_STAMP();  // start
  const int tid = threadIdx.x;
  TrsmLane L;
  const int lane = tid & 63;
  L.t = lane & 15;
  const int64_t grow = (int64_t)blockIdx.x * TRSM_ROWS + (tid >> 6) * 4 + (lane >> 4);
  const bool ok = grow < n;
  const bool ident = grow >= k0 && grow < k0 + kb;
  const int rr = (int)(grow - k0);
  const bool vec = kb == NB && (n & 3) == 0 && (reinterpret_cast<uintptr_t>(A) & 15) == 0;
  // the row's right-hand side first, so that its load is in flight with L^T's
  if (ok && !ident && vec) {
    const float4 b0 = *reinterpret_cast<const float4*>(A + grow * n + k0 + 8 * L.t);
    const float4 b1 = *reinterpret_cast<const float4*>(A + grow * n + k0 + 8 * L.t + 4);
    L.b[0] = b0.x; L.b[1] = b0.y; L.b[2] = b0.z; L.b[3] = b0.w;
    L.b[4] = b1.x; L.b[5] = b1.y; L.b[6] = b1.z; L.b[7] = b1.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = 8 * L.t + i;
      if (ident)
        L.b[i] = c == rr ? 1.0f : 0.0f;
      else
        L.b[i] = (ok && c < kb) ? A[grow * n + k0 + c] : 0.0f;
    }
  }
  // Lt[j][m] = L[m][j] for m > j, else 0 (the buffer holds zeros below its diagonal)
  {
    constexpr int PER = NB * NB / 4 / TRSM_THREADS;
    float4 v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + TRSM_THREADS * i, j = idx >> 5, m = 4 * (idx & 31);
      v[i] = *reinterpret_cast<const float4*>(Ltk + j * NB + m);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + TRSM_THREADS * i, j = idx >> 5, m = 4 * (idx & 31);
      float4 w = v[i];
      w.x = m + 0 > j ? w.x : 0.0f;
      w.y = m + 1 > j ? w.y : 0.0f;
      w.z = m + 2 > j ? w.z : 0.0f;
      w.w = m + 3 > j ? w.w : 0.0f;
      *reinterpret_cast<float4*>(&Lt[j][m]) = w;
    }
  }
  if (tid < NB) rL[tid] = tid < kb ? 1.0f / Ltk[tid * (NB + 1)] : 0.0f;
  __syncthreads();
  GPTQ_TRACE_STAMP();  // rows loaded, L^T in LDS

#pragma unroll
  for (int i = 0; i < 8; ++i) L.ru[i] = rL[8 * L.t + i];
  L.un[0] = *reinterpret_cast<const float4*>(&Lt[0][8 * L.t]);
  L.un[1] = *reinterpret_cast<const float4*>(&Lt[0][8 * L.t + 4]);
  trsm_steps(L, Lt, std::make_integer_sequence<int, NB>{});
  GPTQ_TRACE_STAMP();  // 128 steps
  GPTQ_TRACE_WRITE(TR_TRSM, k0 / NB);
  if (!ok) return;
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = (ident && 8 * L.t + i < rr) ? 0.0f : L.b[i] * L.ru[i];
  if (vec) {
    *reinterpret_cast<float4*>(A + grow * n + k0 + 8 * L.t) = make_float4(y[0], y[1], y[2], y[3]);
    *reinterpret_cast<float4*>(A + grow * n + k0 + 8 * L.t + 4) = make_float4(y[4], y[5], y[6], y[7]);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (8 * L.t + i < kb) A[grow * n + k0 + 8 * L.t + i] = y[i];
  }
}

// U[i][j] = Y[n-1-j][n-1-i] for j >= i into H, with Y = L^-T the upper
// triangle of A (U = P L^-1 P), by 64 x 64 tiles transposed through LDS: both
// the reads of Y and the writes of H run along rows.  Tiles on the diagonal
// also write the dead flags of their rows into H[i][i-1], and H[n-1][0] for
// column 0.
__global__ __launch_bounds__(256) void k_write_factor(const float* Y, int64_t n, const uint8_t* dead, float* H) {
  __shared__ float T[64][65];
  const int64_t I0 = (int64_t)blockIdx.y * 64, J0 = (int64_t)blockIdx.x * 64;
  if (J0 + 63 < I0) return;
  const int64_t yr0 = n - J0 - 64, yc0 = n - I0 - 64;  // negative at a ragged edge
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int k = ty; k < 64; k += 4) {
    const int64_t yr = yr0 + k, yc = yc0 + tx;
    T[k][tx] = (yr >= 0 && yc >= 0) ? Y[yr * n + yc] : 0.0f;
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

#ifdef GPTQ_TRACE
GPTQ_TRACE_SETTER(trace_set_factor)
#endif

size_t factor_scratch_floats(int64_t n) { return (size_t)((n + NB - 1) / NB) * NB * NB; }

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
  const bool vec4 = (n % 4) == 0 && (reinterpret_cast<uintptr_t>(H) & 15) == 0 &&
                    (reinterpret_cast<uintptr_t>(ws.A) & 15) == 0;
  const unsigned gy = (unsigned)(n < 65535 ? n : 65535);
  if (vec4) {
    const unsigned gx = (unsigned)((n / 4 + 255) / 256);
    hipLaunchKernelGGL(k_reverse_damped4, dim3(gx, gy), dim3(256), 0, stream, (const float*)H, n,
                       (const uint8_t*)ws.dead, (const float*)ws.lam, ws.A);
  } else {
    const unsigned gx = (unsigned)((n + 255) / 256 < 16 ? (n + 255) / 256 : 16);
    hipLaunchKernelGGL(k_reverse_damped, dim3(gx, gy), dim3(256), 0, stream, (const float*)H, n,
                       (const uint8_t*)ws.dead, (const float*)ws.lam, ws.A);
  }
  FCHECK(hipGetLastError());
  const int64_t nk = (n + NB - 1) / NB;
  hipLaunchKernelGGL(k_potrf_diag, dim3(1), dim3(256), 0, stream, (const float*)ws.A, n, (int64_t)0, ws.Lt,
                     ws.status);
  FCHECK(hipGetLastError());
  const unsigned grows = (unsigned)((n + TRSM_ROWS - 1) / TRSM_ROWS);
  int64_t kp = 0;  // first column of the panels whose update of the columns past the next block is pending
  for (int64_t k = 0; k < nk; ++k) {
    const int64_t k0 = k * NB;
    const int64_t kb = (n - k0) < NB ? (n - k0) : NB;
    const int64_t c1 = k0 + kb, rest = n - c1;
    // block column k: the panel below, the inverse above, L_kk^-T on its rows
    hipLaunchKernelGGL(k_trsm_block, dim3(grows), dim3(TRSM_THREADS), 0, stream, ws.A,
                       (const float*)(ws.Lt + k * NB * NB), n, k0, (int)kb);
    FCHECK(hipGetLastError());
    if (rest <= 0) break;
    const int kb1 = (int)(rest < NB ? rest : NB);
    // the pending panels kp .. c1 reach block column k+1 now, the columns past
    // it once FACTOR_LAZY panels are pending (or none are past it)
    const int64_t kn = c1 - kp;
    const int64_t nt = (rest + 127) / 128, ntri = nt * (nt + 1) / 2, rrows = c1 / 128;
    const bool flush = kn >= FACTOR_LAZY * NB || rest <= kb1 || rrows * nt + ntri - 1 <= FACTOR_LAZY_TILES;
    // A[r][j] -= A[r][kp:c1] L[j][kp:c1]^T for every row r and the columns j >= c1
    GemmF32 t{};
    t.A = ws.A + kp;
    t.lda = n;
    t.B = ws.A + c1 * n + kp;
    t.ldb = n;
    t.b_kmajor = 0;  // B(k, j) = L[c1 + j][kp + k]
    t.C = ws.A + c1;
    t.ldc = n;
    t.M = (int)n;
    t.N = (int)rest;
    t.K = (int)kn;
    t.kfl_lo = (int)kp;  // rows of a pending panel's block: only the panels from their own block on
    t.kfl_hi = (int)c1;
    t.alpha = -1.0f;
    t.beta = 1;
    t.batch = 1;
    {
      // look-ahead: the diagonal block of block k+1 alone, every pending panel
      const int t32 = (kb1 + 31) / 32;
      if (kn > NB)
        hipLaunchKernelGGL(k_diag_update<2>, dim3((unsigned)(t32 * (t32 + 1) / 2)), dim3(256), 0, stream, ws.A, n, kp,
                           c1, kb1);
      else
        hipLaunchKernelGGL(k_diag_update<1>, dim3((unsigned)(t32 * (t32 + 1) / 2)), dim3(256), 0, stream, ws.A, n, kp,
                           c1, kb1);
      FCHECK(hipGetLastError());
    }
    // the rest beside block k+1's factor
    const int64_t tiles = flush ? rrows * nt + ntri - 1 : rrows + nt - 1;
    hipLaunchKernelGGL(k_factor_step, dim3((unsigned)(1 + tiles)), dim3(256), 0, stream, t, (int)ntri, (int)rrows,
                       (int)nt, flush ? 0 : 1, (const float*)ws.A, n, c1, ws.Lt + (k + 1) * NB * NB, ws.status);
    FCHECK(hipGetLastError());
    if (flush) kp = c1;
  }
  {
    const unsigned nt = (unsigned)((n + 63) / 64);
    hipLaunchKernelGGL(k_write_factor, dim3(nt, nt), dim3(256), 0, stream, (const float*)ws.A, n,
                       (const uint8_t*)ws.dead, H);
    FCHECK(hipGetLastError());
  }
  return hipSuccess;
}

}  // namespace gptq
