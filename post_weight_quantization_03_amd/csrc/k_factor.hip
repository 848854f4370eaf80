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
//  3. blocked right-looking Cholesky, nb = 128: k_potrf_diag factors the
//     diagonal block; the panel below becomes L_ik = A_ik L_kk^-T by
//     row-parallel forward substitution (k_trsm_rows) and the trailing lower
//     tiles take A_ij -= L_ik L_jk^T (GEMM), in the same launch as the factor
//     of the next diagonal block (k_factor_step, look-ahead).  The inverses of the diagonal
//     blocks are formed after the loop, all at once and off the loop's
//     critical path (k_trsm_rows on identity rows).
//  4. triangular inverse by doubling: with the 128-blocks of Minv inverted,
//     each level joins pairs of inverted diagonal blocks,
//     [P 0; C Q]^-1 = [P^-1 0; -Q^-1 C P^-1 Q^-1], as two batched GEMMs.
//  5. k_write_factor   U[i][j] = Minv[n-1-i][n-1-j] for i <= j into H, plus the
//     dead flags in H's strictly lower triangle.
#include <utility>

#include "gemm_tile.h"

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

// A[i][j] = H_d[n-1-i][n-1-j] for j <= i, four columns a thread: the source
// is the float4 of row n-1-i ending at column n-1-j, read backwards.  Chunks
// reaching past the diagonal also write A's upper triangle, which nothing reads.
// Needs n % 4 == 0 and 16-byte aligned H and A.
__global__ void k_reverse_damped4(const float* H, int64_t n, const uint8_t* dead, const float* lam, float* A) {
  const float l = *lam;
  for (int64_t i = blockIdx.y; i < n; i += gridDim.y) {
    const int64_t si = n - 1 - i;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; 4 * q <= i; q += (int64_t)gridDim.x * blockDim.x) {
      const float4 v = *reinterpret_cast<const float4*>(H + si * n + (n - 4 - 4 * q));
      float o[4] = {v.w, v.z, v.y, v.x};
      const int64_t e = i - 4 * q;  // the diagonal, if in this chunk
      if (e < 4) o[e] = (dead[si] ? 1.0f : o[e]) + l;
      *reinterpret_cast<float4*>(A + i * n + 4 * q) = make_float4(o[0], o[1], o[2], o[3]);
    }
  }
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

// ------------------------------------------------------------------ diagonal block

// Cholesky of the diagonal block A[k0:k0+kb, k0:k0+kb] (lower triangle in,
// kb <= 128, padded with the identity beyond kb).  The block goes back as L^T
// in its upper triangle, diagonal included: the triangular solves and inverses
// read rows of L^T only, and the block's strict lower triangle is unspecified
// afterwards.
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
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int kk = 0; kk < PB / 4; ++kk)
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
__device__ __forceinline__ void potrf_step(float (*As)[LP], int wave, int lane) {
  potrf_panel<P>(As, wave, lane);
  __syncthreads();
  if constexpr (P + 1 < NB / PB) {
    potrf_update<P>(As, wave, lane);
    __syncthreads();
    potrf_step<P + 1>(As, wave, lane);
  }
}

// Whole blocks with 16-byte rows move as float4, all loads of a thread in
// flight at once; a ragged last block goes element by element.
__device__ __forceinline__ bool block_vec(const float* A, int64_t n, int kb) {
  return kb == NB && (n & 3) == 0 && (reinterpret_cast<uintptr_t>(A) & 15) == 0;
}

constexpr int POTRF_LDS = NB * LP * 4;

__device__ __forceinline__ void potrf_diag(float* A, int64_t n, int64_t k0, int* status, char* lds) {
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
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  potrf_step<0>(As, wave, lane);
  if (tid < kb) {
    const float d = As[tid][tid];
    if (!(d > 0.0f && d < INFINITY)) raise_status(status, GPTQ_ENOTPD);
  }
  // L^T: chunks that reach the diagonal or lie above it
  if (block_vec(A, n, kb)) {
#pragma unroll 4
    for (int i = 0; i < NB * NB / 4 / 256; ++i) {
      const int idx = tid + 256 * i, r = idx >> 5, q = 4 * (idx & 31);
      if (q + 3 >= r)
        *reinterpret_cast<float4*>(A + (k0 + r) * n + k0 + q) =
            make_float4(As[r][q + 0], As[r][q + 1], As[r][q + 2], As[r][q + 3]);
    }
  } else {
    for (int idx = tid; idx < NB * NB; idx += 256) {
      const int r = idx >> 7, q = idx & (NB - 1);
      if (q >= r && q < kb) A[(k0 + r) * n + k0 + q] = As[r][q];
    }
  }
}

__global__ __launch_bounds__(256) void k_potrf_diag(float* A, int64_t n, int64_t k0, int* status) {
  __shared__ __attribute__((aligned(16))) char lds[POTRF_LDS];
  potrf_diag(A, n, k0, status, lds);
}

// One step of the blocked factor with look-ahead: the trailing update of
// block k, A22 -= L21 L21^T on lower tiles, beside the factor of block k+1.
// Block k+1's diagonal block (A22's first 128 x 128 tile) has been updated by
// a small launch before this one; workgroup 0 factors it while the other
// workgroups update the remaining lower tiles (the first `skip` tiles of size
// TM cover that block and are left out).
constexpr int cmax(int a, int b) { return a > b ? a : b; }

// More than half of the CU's LDS per workgroup: one workgroup per CU, so the
// diagonal factor never shares its CU with a tile (sharing one made the factor
// up to 1.9x slower; the tiles lose less than that gains).
template <int TM>
__global__ __launch_bounds__(256) void k_factor_step(GemmF32 trail, int skip, float* A, int64_t n, int64_t k0n,
                                                     int* status) {
  __shared__ __attribute__((aligned(16))) char
      lds[cmax(96 * 1024, cmax(POTRF_LDS, cmax(gemm_tile_lds<128>(), gemm_tile_lds<TM>())))];
  if (blockIdx.x == 0) {
    potrf_diag(A, n, k0n, status, lds);
    return;
  }
  const int t = (int)blockIdx.x - 1 + skip;
  int r = (int)((sqrtf(8.f * (float)t + 1.f) - 1.f) * 0.5f);
  while ((r + 1) * (r + 2) / 2 <= t) ++r;
  while (r * (r + 1) / 2 > t) --r;
  gemm_tile<TM, false>(trail, r, t - r * (r + 1) / 2, 0, lds);
}

// ------------------------------------------------------------------ triangular solves

// Rows y = b L^-T for the diagonal block's L (read as L^T from the block's
// upper triangle, diagonal from the block), i.e. L y^T = b^T by forward
// substitution, right-looking: y_j = b_j / L_jj, then b_m -= y_j L_mj for m > j.
// The same layout as the column loop: a 64-lane wave holds 4 rows, 16 lanes a
// row, 8 consecutive columns per lane; y_j reaches the row's lanes by a DPP
// row broadcast; L^T sits in LDS without its diagonal, and the row of step
// j+1 is read during step j.  Column j is final after step j, so y is formed
// after the loop as b * (1 / L_jj).
//
// IDENT = false: the panel below the block, rows [r0, r0 + rows) of A at
//   columns [k0, k0 + 128), solved in place (L_ik = A_ik L_kk^-T).
// IDENT = true: b = e_r for r = 0 .. 127 of diagonal block blockIdx.y: y is
//   row r of L^-T, i.e. column r of L^-1, stored into the same block of Minv
//   (lower, zeros above the diagonal).
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

template <bool IDENT>
__global__ __launch_bounds__(256) void k_trsm_rows(float* A, float* Minv, int64_t n, int64_t k0_, int64_t r0,
                                                   int64_t rows) {
  __shared__ __attribute__((aligned(16))) float Lt[NB][NB];
  __shared__ float rL[NB];
  const int64_t k0 = IDENT ? (int64_t)blockIdx.y * NB : k0_;
  const int kb = (int)((n - k0) < NB ? (n - k0) : NB);
  const int tid = threadIdx.x;
  // Lt[j][m] = L[m][j] for m > j (the block's upper triangle), else 0
  if (block_vec(A, n, kb)) {
    constexpr int PER = NB * NB / 4 / 256;
    float4 v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + 256 * i, j = idx >> 5, m = 4 * (idx & 31);
      v[i] = *reinterpret_cast<const float4*>(A + (k0 + j) * n + k0 + m);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + 256 * i, j = idx >> 5, m = 4 * (idx & 31);
      float4 w = v[i];
      w.x = m + 0 > j ? w.x : 0.0f;
      w.y = m + 1 > j ? w.y : 0.0f;
      w.z = m + 2 > j ? w.z : 0.0f;
      w.w = m + 3 > j ? w.w : 0.0f;
      *reinterpret_cast<float4*>(&Lt[j][m]) = w;
    }
  } else {
    for (int idx = tid; idx < NB * NB / 4; idx += 256) {
      const int j = idx >> 5, m = 4 * (idx & 31);
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (j < kb) {
        const float* src = A + (k0 + j) * n + k0 + m;
        v.x = (m + 0 > j && m + 0 < kb) ? src[0] : 0.0f;
        v.y = (m + 1 > j && m + 1 < kb) ? src[1] : 0.0f;
        v.z = (m + 2 > j && m + 2 < kb) ? src[2] : 0.0f;
        v.w = (m + 3 > j && m + 3 < kb) ? src[3] : 0.0f;
      }
      *reinterpret_cast<float4*>(&Lt[j][m]) = v;
    }
  }
  if (tid < NB) rL[tid] = tid < kb ? 1.0f / A[(k0 + tid) * (n + 1)] : 0.0f;
  __syncthreads();

  TrsmLane L;
  const int lane = tid & 63;
  L.t = lane & 15;
  const int64_t rr = (int64_t)blockIdx.x * 16 + (tid >> 6) * 4 + (lane >> 4);
  const bool ok = IDENT ? rr < kb : rr < rows;
  const int64_t grow = r0 + rr;
  if (!IDENT && ok && block_vec(A, n, kb)) {
    const float4 b0 = *reinterpret_cast<const float4*>(A + grow * n + k0 + 8 * L.t);
    const float4 b1 = *reinterpret_cast<const float4*>(A + grow * n + k0 + 8 * L.t + 4);
    L.b[0] = b0.x; L.b[1] = b0.y; L.b[2] = b0.z; L.b[3] = b0.w;
    L.b[4] = b1.x; L.b[5] = b1.y; L.b[6] = b1.z; L.b[7] = b1.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = 8 * L.t + i;
      if constexpr (IDENT)
        L.b[i] = (ok && c == rr) ? 1.0f : 0.0f;
      else
        L.b[i] = ok ? A[grow * n + k0 + c] : 0.0f;
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) L.ru[i] = rL[8 * L.t + i];
  L.un[0] = *reinterpret_cast<const float4*>(&Lt[0][8 * L.t]);
  L.un[1] = *reinterpret_cast<const float4*>(&Lt[0][8 * L.t + 4]);
  trsm_steps(L, Lt, std::make_integer_sequence<int, NB>{});
  if (!ok) return;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = 8 * L.t + i;
    const float y = L.b[i] * L.ru[i];
    if constexpr (IDENT) {
      if (c < kb) Minv[(k0 + c) * n + k0 + rr] = (c >= rr) ? y : 0.0f;
    } else {
      A[grow * n + k0 + c] = y;
    }
  }
}

// U[i][j] = Minv[n-1-i][n-1-j] for j >= i into H, four columns a thread (the
// chunk holding the diagonal element by element, so H[i][j < i] keeps its
// dead flags); dead flags into H[i][i-1] and H[n-1][0].  Needs n % 4 == 0 and
// 16-byte aligned Minv and H.
__global__ void k_write_factor4(const float* Minv, int64_t n, const uint8_t* dead, float* H) {
  for (int64_t i = blockIdx.y; i < n; i += gridDim.y) {
    const int64_t si = n - 1 - i;
    for (int64_t q = i / 4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; 4 * q < n;
         q += (int64_t)gridDim.x * blockDim.x) {
      const float4 v = *reinterpret_cast<const float4*>(Minv + si * n + (n - 4 - 4 * q));
      const float o[4] = {v.w, v.z, v.y, v.x};
      if (4 * q >= i) {
        *reinterpret_cast<float4*>(H + i * n + 4 * q) = make_float4(o[0], o[1], o[2], o[3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * q + e >= i) H[i * n + 4 * q + e] = o[e];
      }
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      if (i >= 1) H[i * n + i - 1] = dead[i] ? 1.0f : 0.0f;
      if (i == n - 1 && n >= 3) H[i * n + 0] = dead[0] ? 1.0f : 0.0f;
    }
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
  const bool vec4 = (n % 4) == 0 && (reinterpret_cast<uintptr_t>(H) & 15) == 0 &&
                    (reinterpret_cast<uintptr_t>(ws.A) & 15) == 0 && (reinterpret_cast<uintptr_t>(ws.Minv) & 15) == 0;
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
  hipLaunchKernelGGL(k_potrf_diag, dim3(1), dim3(256), 0, stream, ws.A, n, (int64_t)0, ws.status);
  FCHECK(hipGetLastError());
  for (int64_t k = 0; k < nk; ++k) {
    const int64_t k0 = k * NB;
    const int64_t kb = (n - k0) < NB ? (n - k0) : NB;
    const int64_t rest = n - k0 - kb;
    if (rest <= 0) break;
    // panel: A[k0+kb:, k0:k0+kb] <- A[..] L_kk^-T   (in place, a row per 16 lanes)
    hipLaunchKernelGGL(k_trsm_rows<false>, dim3((unsigned)((rest + 15) / 16)), dim3(256), 0, stream, ws.A,
                       ws.Minv, n, k0, k0 + kb, rest);
    FCHECK(hipGetLastError());
    // trailing lower tiles A22 -= L21 L21^T: first the 128 x 128 diagonal
    // block of block k+1 alone, then the rest beside that block's factor
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
    {
      GemmF32 d = t;
      d.M = d.N = (int)(rest < NB ? rest : NB);
      FCHECK(gemm_f32(d, stream));
    }
    const int64_t t128 = (rest + 127) / 128;
    if (t128 * (t128 + 1) / 2 >= 256) {
      const int64_t tiles = t128 * (t128 + 1) / 2;
      hipLaunchKernelGGL(k_factor_step<128>, dim3((unsigned)(1 + tiles - 1)), dim3(256), 0, stream, t, 1, ws.A, n,
                         k0 + kb, ws.status);
    } else {
      const int64_t t64 = (rest + 63) / 64;
      const int64_t tiles = t64 * (t64 + 1) / 2;
      const int64_t skip = tiles < 3 ? tiles : 3;
      hipLaunchKernelGGL(k_factor_step<64>, dim3((unsigned)(1 + tiles - skip)), dim3(256), 0, stream, t, (int)skip,
                         ws.A, n, k0 + kb, ws.status);
    }
    FCHECK(hipGetLastError());
  }
  // inverses of all diagonal blocks at once, into Minv's diagonal blocks
  hipLaunchKernelGGL(k_trsm_rows<true>, dim3(NB / 16, (unsigned)nk), dim3(256), 0, stream, ws.A, ws.Minv, n,
                     (int64_t)0, (int64_t)0, (int64_t)0);
  FCHECK(hipGetLastError());
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
  if (vec4) {
    const unsigned gx = (unsigned)((n / 4 + 255) / 256);
    hipLaunchKernelGGL(k_write_factor4, dim3(gx, gy), dim3(256), 0, stream, (const float*)ws.Minv, n,
                       (const uint8_t*)ws.dead, H);
  } else {
    const unsigned gx = (unsigned)((n + 255) / 256 < 16 ? (n + 255) / 256 : 16);
    hipLaunchKernelGGL(k_write_factor, dim3(gx, gy), dim3(256), 0, stream, (const float*)ws.Minv, n,
                       (const uint8_t*)ws.dead, H);
  }
  FCHECK(hipGetLastError());
  return hipSuccess;
}

}  // namespace gptq
