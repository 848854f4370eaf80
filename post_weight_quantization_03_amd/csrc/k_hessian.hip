// Hessian accumulation H += 2 X^T X as a symmetric rank-k update on MFMA.
//
// X is [tokens, n] row-major: both MFMA operands of an output tile H[I, J] are
// column slabs of the same token rows, and the contraction runs over tokens.
// Only upper tiles (I <= J) are computed; each writes its block and the
// mirrored block, so both triangles of H hold bit-identical values.
//
// bf16 path (v_mfma_f32_32x32x16_bf16): a lane supplies 8 consecutive k
// (tokens) of one row/column, so token-major X is transposed on its way into
// LDS.  Each thread loads a 4-token x 4-column block as four 8-byte reads,
// transposes it in registers and stores four 8-byte column pieces; LDS holds
// Xs[column][token] with an 80-byte row pitch, which keeps both the stores
// and the 16-byte MFMA operand reads free of bank conflicts.
// fp32 path (v_mfma_f32_32x32x2_f32): a lane supplies one k, so X stays
// token-major in LDS and operand reads are 32 consecutive floats.
//
// Work items are (tile, token split).  With one split an item adds 2*acc to H
// directly.  With S splits each item stores its partial tile; the last of the
// S items of a tile to finish (per-tile arrival counter) sums the S partials
// in split order and writes H, so the result does not depend on scheduling.
#include "common.h"

namespace gptq {
namespace {

constexpr int TILE = 128;
constexpr int KT_BF16 = 32;   // tokens per LDS stage, bf16 path
constexpr int KT_F32 = 16;    // tokens per LDS stage, fp32 path
constexpr int ROWB = 40;      // LDS pitch of a column row in bf16 elements (80 bytes)
constexpr int PARTIAL = TILE * TILE;  // floats per partial tile

struct SyrkArgs {
  const void* X;
  float* H;
  float* part;     // [T * S][PARTIAL] (S > 1)
  int* counters;   // [T] (S > 1)
  int64_t ldx;
  int n, tokens;
  int nbt;         // tiles per dimension
  int T;           // upper tiles
  int S;           // token splits
  int tps;         // tokens per split
};

__device__ __forceinline__ void decode_upper(int t, int nbt, int& I, int& J) {
  // row-major enumeration of upper tiles: row I holds nbt - I tiles
  int i = 0, base = 0;
  while (base + (nbt - i) <= t) {
    base += nbt - i;
    ++i;
  }
  I = i;
  J = i + (t - base);
}

// Epilogue shared by both paths: add 2*v to H at (gr, gc) and mirror, upper tiles only.
__device__ __forceinline__ void write_tile(const SyrkArgs& a, int I, int J, f32x16 (&acc)[2][2], int lane,
                                           int wm, int wn) {
  const int n = a.n;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int gr = I * TILE + wm * 64 + 32 * i + acc_row(r, lane);
        const int gc = J * TILE + wn * 64 + 32 * j + acc_col(lane);
        if (gr < n && gc < n && gr <= gc) {
          float* p = a.H + (int64_t)gr * n + gc;
          const float v = *p + 2.0f * acc[i][j][r];
          *p = v;
          if (gr != gc) a.H[(int64_t)gc * n + gr] = v;
        }
      }
}

// Split-K bookkeeping: store this item's partial; the last arrival reduces.
// Returns true when this workgroup must write H with acc = sum of partials.
__device__ __forceinline__ bool splitk_reduce(const SyrkArgs& a, int tile, int s, f32x16 (&acc)[2][2],
                                              int lane, int wave) {
  __shared__ int last;
  float* mine = a.part + ((int64_t)tile * a.S + s) * PARTIAL;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) mine[(((wave * 4 + i * 2 + j) * 16 + r) << 6) + lane] = acc[i][j][r];
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = atomicAdd(a.counters + tile, 1);
    last = (prev == a.S - 1);
  }
  __syncthreads();
  if (!last) return false;
  __threadfence();
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  for (int q = 0; q < a.S; ++q) {
    const float* pq = a.part + ((int64_t)tile * a.S + q) * PARTIAL;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          acc[i][j][r] += pq[(((wave * 4 + i * 2 + j) * 16 + r) << 6) + lane];
  }
  if (threadIdx.x == 0) a.counters[tile] = 0;  // ready for the next call
  return true;
}

// ------------------------------------------------------------------ bf16 path

struct Blk4x4 {
  uint2 v[4];  // v[i] = 4 bf16 of token i (columns c..c+3)
};

template <bool VEC>
__device__ __forceinline__ void load_bf16(const SyrkArgs& a, const uint16_t* X, int col0, int t, int t1,
                                          int q, int cg, Blk4x4& b) {
  const int c = col0 + 4 * cg;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tok = t + 4 * q + i;
    const uint16_t* p = X + (int64_t)tok * a.ldx + c;
    if (VEC && tok < t1 && c + 3 < a.n) {
      b.v[i] = *reinterpret_cast<const uint2*>(p);
    } else {
      uint16_t e[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) e[k] = (tok < t1 && c + k < a.n) ? p[k] : (uint16_t)0;
      b.v[i].x = (uint32_t)e[0] | ((uint32_t)e[1] << 16);
      b.v[i].y = (uint32_t)e[2] | ((uint32_t)e[3] << 16);
    }
  }
}

// Transposes the 4x4 block and stores four 8-byte column pieces: Xs[col][4q .. 4q+3].
__device__ __forceinline__ void store_bf16(uint16_t (*Xs)[ROWB], int q, int cg, const Blk4x4& b) {
  // column k of the block, tokens 0..3: low/high halves of v[i].x (k = 0, 1) or v[i].y (k = 2, 3)
  const uint32_t x0 = b.v[0].x, x1 = b.v[1].x, x2 = b.v[2].x, x3 = b.v[3].x;
  const uint32_t y0 = b.v[0].y, y1 = b.v[1].y, y2 = b.v[2].y, y3 = b.v[3].y;
  uint2 c0, c1, c2, c3;
  c0.x = (x0 & 0xffffu) | (x1 << 16);          // tok0.col0 | tok1.col0
  c0.y = (x2 & 0xffffu) | (x3 << 16);          // tok2.col0 | tok3.col0
  c1.x = (x0 >> 16) | (x1 & 0xffff0000u);      // tok0.col1 | tok1.col1
  c1.y = (x2 >> 16) | (x3 & 0xffff0000u);
  c2.x = (y0 & 0xffffu) | (y1 << 16);
  c2.y = (y2 & 0xffffu) | (y3 << 16);
  c3.x = (y0 >> 16) | (y1 & 0xffff0000u);
  c3.y = (y2 >> 16) | (y3 & 0xffff0000u);
  const int col = 4 * cg;
  *reinterpret_cast<uint2*>(&Xs[col + 0][4 * q]) = c0;
  *reinterpret_cast<uint2*>(&Xs[col + 1][4 * q]) = c1;
  *reinterpret_cast<uint2*>(&Xs[col + 2][4 * q]) = c2;
  *reinterpret_cast<uint2*>(&Xs[col + 3][4 * q]) = c3;
}

__device__ __forceinline__ bf16x8 frag_bf16(const uint16_t (*Xs)[ROWB], int row, int chunk) {
  const uint4 v = *reinterpret_cast<const uint4*>(&Xs[row][8 * chunk]);
  return __builtin_bit_cast(bf16x8, v);
}

template <bool VEC>
__global__ __launch_bounds__(256) void k_syrk_bf16(SyrkArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][TILE][ROWB];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][TILE][ROWB];

  const int item = blockIdx.x;
  const int tile = item / a.S, s = item % a.S;
  int I, J;
  decode_upper(tile, a.nbt, I, J);
  const bool diag = (I == J);
  const int t0 = s * a.tps;
  const int t1 = min(a.tokens, t0 + a.tps);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int q = lane & 7, cg = (lane >> 3) + 8 * wave;
  const uint16_t* X = static_cast<const uint16_t*>(a.X);

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  if (t0 < t1) {
    Blk4x4 ba, bb;
    load_bf16<VEC>(a, X, I * TILE, t0, t1, q, cg, ba);
    if (!diag) load_bf16<VEC>(a, X, J * TILE, t0, t1, q, cg, bb);
    store_bf16(As[0], q, cg, ba);
    if (!diag) store_bf16(Bs[0], q, cg, bb);
    __syncthreads();
    int buf = 0;
    for (int t = t0; t < t1; t += KT_BF16) {
      const bool more = t + KT_BF16 < t1;
      if (more) {
        load_bf16<VEC>(a, X, I * TILE, t + KT_BF16, t1, q, cg, ba);
        if (!diag) load_bf16<VEC>(a, X, J * TILE, t + KT_BF16, t1, q, cg, bb);
      }
      const uint16_t(*Bsrc)[ROWB] = diag ? As[buf] : Bs[buf];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int chunk = 2 * kk + (lane >> 5);
        const bf16x8 a0 = frag_bf16(As[buf], wm * 64 + (lane & 31), chunk);
        const bf16x8 a1 = frag_bf16(As[buf], wm * 64 + 32 + (lane & 31), chunk);
        const bf16x8 b0 = frag_bf16(Bsrc, wn * 64 + (lane & 31), chunk);
        const bf16x8 b1 = frag_bf16(Bsrc, wn * 64 + 32 + (lane & 31), chunk);
        acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc[0][0], 0, 0, 0);
        acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, acc[0][1], 0, 0, 0);
        acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, acc[1][0], 0, 0, 0);
        acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc[1][1], 0, 0, 0);
      }
      if (more) {
        store_bf16(As[buf ^ 1], q, cg, ba);
        if (!diag) store_bf16(Bs[buf ^ 1], q, cg, bb);
        __syncthreads();
        buf ^= 1;
      }
    }
  }

  if (a.S > 1) {
    if (!splitk_reduce(a, tile, s, acc, lane, wave)) return;
  }
  write_tile(a, I, J, acc, lane, wm, wn);
}

// ------------------------------------------------------------------ fp32 path

constexpr int F32_PITCH = TILE + 4;

template <bool VEC>
__device__ __forceinline__ void load_f32(const SyrkArgs& a, const float* X, int col0, int t, int t1,
                                         float4 (&v)[2]) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = threadIdx.x + 256 * i;
    const int tok = t + (idx >> 5), c = col0 + 4 * (idx & 31);
    const float* p = X + (int64_t)tok * a.ldx + c;
    if (VEC && tok < t1 && c + 3 < a.n) {
      v[i] = *reinterpret_cast<const float4*>(p);
    } else {
      v[i].x = (tok < t1 && c + 0 < a.n) ? p[0] : 0.f;
      v[i].y = (tok < t1 && c + 1 < a.n) ? p[1] : 0.f;
      v[i].z = (tok < t1 && c + 2 < a.n) ? p[2] : 0.f;
      v[i].w = (tok < t1 && c + 3 < a.n) ? p[3] : 0.f;
    }
  }
}

__device__ __forceinline__ void store_f32(float (*Xs)[F32_PITCH], const float4 (&v)[2]) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = threadIdx.x + 256 * i;
    *reinterpret_cast<float4*>(&Xs[idx >> 5][4 * (idx & 31)]) = v[i];
  }
}

template <bool VEC>
__global__ __launch_bounds__(256) void k_syrk_f32(SyrkArgs a) {
  __shared__ __attribute__((aligned(16))) float As[2][KT_F32][F32_PITCH];
  __shared__ __attribute__((aligned(16))) float Bs[2][KT_F32][F32_PITCH];

  const int item = blockIdx.x;
  const int tile = item / a.S, s = item % a.S;
  int I, J;
  decode_upper(tile, a.nbt, I, J);
  const bool diag = (I == J);
  const int t0 = s * a.tps;
  const int t1 = min(a.tokens, t0 + a.tps);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const float* X = static_cast<const float*>(a.X);

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  if (t0 < t1) {
    float4 va[2], vb[2];
    load_f32<VEC>(a, X, I * TILE, t0, t1, va);
    if (!diag) load_f32<VEC>(a, X, J * TILE, t0, t1, vb);
    store_f32(As[0], va);
    if (!diag) store_f32(Bs[0], vb);
    __syncthreads();
    int buf = 0;
    for (int t = t0; t < t1; t += KT_F32) {
      const bool more = t + KT_F32 < t1;
      if (more) {
        load_f32<VEC>(a, X, I * TILE, t + KT_F32, t1, va);
        if (!diag) load_f32<VEC>(a, X, J * TILE, t + KT_F32, t1, vb);
      }
      float(*Bsrc)[F32_PITCH] = diag ? As[buf] : Bs[buf];
#pragma unroll
      for (int kk = 0; kk < KT_F32 / 2; ++kk) {
        const int kr = 2 * kk + (lane >> 5);
        const float a0 = As[buf][kr][wm * 64 + (lane & 31)];
        const float a1 = As[buf][kr][wm * 64 + 32 + (lane & 31)];
        const float b0 = Bsrc[kr][wn * 64 + (lane & 31)];
        const float b1 = Bsrc[kr][wn * 64 + 32 + (lane & 31)];
        acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
        acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
        acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
        acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
      }
      if (more) {
        store_f32(As[buf ^ 1], va);
        if (!diag) store_f32(Bs[buf ^ 1], vb);
        __syncthreads();
        buf ^= 1;
      }
    }
  }

  if (a.S > 1) {
    if (!splitk_reduce(a, tile, s, acc, lane, wave)) return;
  }
  write_tile(a, I, J, acc, lane, wm, wn);
}

__global__ void k_zero_i32(int* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// Work decomposition: enough (tile, split) items to keep every CU busy, with
// at least 512 tokens per split.
void plan(int64_t n, int64_t tokens, gptq_dtype dt, int& nbt, int& T, int& S, int& tps) {
  nbt = (int)((n + TILE - 1) / TILE);
  T = nbt * (nbt + 1) / 2;
  const int kt = dt == GPTQ_BF16 ? KT_BF16 : KT_F32;
  const int64_t target = 1024;
  int64_t s = (target + T - 1) / T;
  const int64_t max_s = (tokens + 511) / 512;
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  int64_t per = (tokens + s - 1) / s;
  per = (per + kt - 1) / kt * kt;
  s = (tokens + per - 1) / per;
  if (s < 1) s = 1;
  S = (int)s;
  tps = (int)per;
}

}  // namespace

size_t hessian_workspace(int64_t n, int64_t tokens, gptq_dtype dt) {
  if (n <= 0 || tokens <= 0) return 0;
  int nbt, T, S, tps;
  plan(n, tokens, dt, nbt, T, S, tps);
  if (S == 1) return 0;
  return align_up((size_t)T * S * PARTIAL * sizeof(float), 256) + align_up((size_t)T * sizeof(int), 256);
}

int hessian_launch(float* H, int64_t n, const void* X, gptq_dtype dt, int64_t tokens, int64_t ldx, void* ws,
                   size_t ws_bytes, hipStream_t stream) {
  int nbt, T, S, tps;
  plan(n, tokens, dt, nbt, T, S, tps);
  SyrkArgs a{};
  a.X = X;
  a.H = H;
  a.ldx = ldx;
  a.n = (int)n;
  a.tokens = (int)tokens;
  a.nbt = nbt;
  a.T = T;
  a.S = S;
  a.tps = tps;
  if (S > 1) {
    if (ws_bytes < hessian_workspace(n, tokens, dt) || ws == nullptr) return GPTQ_EWORKSPACE;
    a.part = static_cast<float*>(ws);
    a.counters = reinterpret_cast<int*>(static_cast<char*>(ws) +
                                        align_up((size_t)T * S * PARTIAL * sizeof(float), 256));
    hipLaunchKernelGGL(k_zero_i32, dim3((T + 255) / 256), dim3(256), 0, stream, a.counters, T);
    if (hipGetLastError() != hipSuccess) return GPTQ_EHIP;
  }
  const dim3 grid((unsigned)(T * S));
  if (dt == GPTQ_BF16) {
    const bool vec = (ldx % 4 == 0) && ((reinterpret_cast<uintptr_t>(X) & 7) == 0);
    if (vec)
      hipLaunchKernelGGL(k_syrk_bf16<true>, grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(k_syrk_bf16<false>, grid, dim3(256), 0, stream, a);
  } else {
    const bool vec = (ldx % 4 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0);
    if (vec)
      hipLaunchKernelGGL(k_syrk_f32<true>, grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(k_syrk_f32<false>, grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError() == hipSuccess ? GPTQ_OK : GPTQ_EHIP;
}

}  // namespace gptq
