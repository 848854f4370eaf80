// The GPTQ column loop in lazy batches of 128 columns.
//
// k_stage_w      W (bf16 or fp32) -> fp32 working copy Wf, dead columns zeroed.
// k_quant_block  one 128-column block: per-row grid at group starts from the
//                current weights, then 128 serial steps
//                  q = clamp(rint(w_j / s) + z, 0, maxq), w^ = s (q - z),
//                  e_j = (w_j - w^) / U_jj, w_k -= e_j U_jk (k in the block)
//                writing codes, grid, w^, row loss and E (the block's e_j).
// Then the trailing update W[:, c1:] -= E U[c0:c1, c1:]: in fp32 accuracy on
// bf16 MFMA with three-way split operands (sgemm_tile.h) when it runs beside
// the next block, else as an fp32 MFMA GEMM.
//
// Layout of k_quant_block: a 64-lane wave holds 4 rows, 16 lanes per row; lane
// t of a row owns columns 8t .. 8t+7 of the block in registers.  At step j the
// owner lane (j / 8) rounds its column, and e_j reaches the row's 16 lanes by
// a DPP row broadcast (row_newbcast, one instruction, rows of 16 lanes are
// exactly the wave's DPP rows).  The U block sits in LDS; each lane reads the
// 8 entries of row j+1 it needs as two 16-byte reads during step j.  Group
// ranges are reduced over the lanes that hold the group with xor shuffles.
// The serial chain of a step is the quotient (div_rn, 5 instructions), the
// rounding and clamp, e_j, the broadcast and one fma.
#include <utility>

#include "gemm_tile.h"
#include "quant_schedule.h"
#include "sgemm_tile.h"

namespace gptq {
namespace {

constexpr int B = 128;

enum GroupMode { GM_BIG = 0, GM_32 = 1, GM_64 = 2 };

// Eight columns a thread; needs cols % 8 == 0, W 16-byte aligned (bf16) or
// 32-byte (fp32), Wf 32-byte aligned.
__global__ void k_stage_w8(const void* W, int is_bf16, int64_t rows, int64_t cols, const uint8_t* dead,
                           float* Wf) {
  const int64_t chunks = rows * cols / 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < chunks; q += stride) {
    const int64_t i = 8 * q, c = i % cols;
    float v[8];
    if (is_bf16) {
      const uint4 b = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(W) + i);
      const uint32_t w[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] = __uint_as_float(w[e] << 16);
        v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
      }
    } else {
      const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(W) + i);
      const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(W) + i + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    const uint2 d = *reinterpret_cast<const uint2*>(dead + c);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if ((((e < 4 ? d.x : d.y) >> (8 * (e & 3))) & 0xff) != 0) v[e] = 0.0f;
    *reinterpret_cast<float4*>(Wf + i) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(Wf + i + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
}

__global__ void k_stage_w(const void* W, int is_bf16, int64_t rows, int64_t cols, const uint8_t* dead,
                          float* Wf) {
  const int64_t total = rows * cols;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t c = i % cols;
    float v;
    if (is_bf16) {
      const uint16_t b = static_cast<const uint16_t*>(W)[i];
      v = __uint_as_float((uint32_t)b << 16);
    } else {
      v = static_cast<const float*>(W)[i];
    }
    Wf[i] = dead[c] ? 0.0f : v;
  }
}

struct BlockArgs {
  float* Wf;
  const float* U;
  int64_t rows, cols;
  int64_t c0;
  int bw;  // columns in this block (<= 128)
  float maxq;
  int64_t g;  // resolved group size
  int64_t G;
  uint8_t* codes;
  float* scales;
  uint8_t* zeros;
  float* w_hat;
  float* row_loss;
  float* E;            // this block's scaled errors: E[r * ldE + j], j < 128
  const float* Eprev;  // the previous block's, when its update of this block is applied here (else null)
  int64_t ldE;
};

// U's upper triangle -> three bf16 planes (the split GEMM's B operand), eight
// columns a thread; the chunk holding the diagonal also fills the planes'
// lower triangle, which nothing reads.  Needs n % 8 == 0 and 16-byte aligned U.
__global__ void k_split_u8(const float* U, int64_t n, uint16_t* P) {
  const int64_t plane = n * n;
  for (int64_t i = blockIdx.y; i < n; i += gridDim.y) {
    for (int64_t q = i / 8 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; 8 * q < n;
         q += (int64_t)gridDim.x * blockDim.x) {
      const float4 a = *reinterpret_cast<const float4*>(U + i * n + 8 * q);
      const float4 b = *reinterpret_cast<const float4*>(U + i * n + 8 * q + 4);
      const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      uint32_t w[3][4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        __bf16 h[2][3];
        split3(x[2 * e], h[0][0], h[0][1], h[0][2]);
        split3(x[2 * e + 1], h[1][0], h[1][1], h[1][2]);
#pragma unroll
        for (int p = 0; p < 3; ++p)
          w[p][e] = (uint32_t)__builtin_bit_cast(uint16_t, h[0][p]) | ((uint32_t)__builtin_bit_cast(uint16_t, h[1][p]) << 16);
      }
#pragma unroll
      for (int p = 0; p < 3; ++p)
        *reinterpret_cast<uint4*>(P + p * plane + i * n + 8 * q) = make_uint4(w[p][0], w[p][1], w[p][2], w[p][3]);
    }
  }
}

// U's upper triangle -> three bf16 planes (the split GEMM's B operand).
__global__ void k_split_u(const float* U, int64_t n, uint16_t* P) {
  const int64_t plane = n * n;
  for (int64_t i = blockIdx.y; i < n; i += gridDim.y) {
    for (int64_t j = i + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += (int64_t)gridDim.x * blockDim.x) {
      __bf16 h1, h2, h3;
      split3(U[i * n + j], h1, h2, h3);
      P[i * n + j] = __builtin_bit_cast(uint16_t, h1);
      P[plane + i * n + j] = __builtin_bit_cast(uint16_t, h2);
      P[2 * plane + i * n + j] = __builtin_bit_cast(uint16_t, h3);
    }
  }
}

template <int O>
__device__ __forceinline__ float row_bcast(float v) {
  // DPP row_newbcast: every lane of a 16-lane row reads lane O of that row.
  return __builtin_amdgcn_update_dpp(0.0f, v, 0x150 + O, 0xf, 0xf, false);
}

// The value of lane i ^ m for m = 1, 2 (DPP quad permutations), and of a
// lane in the other half of its group of 8 or 16 for m = 4, 8 (half-row and
// row mirrors).  Used after the steps for the smaller m, when every lane of a
// group of m lanes holds the same value, the mirror's partner holds what lane
// i ^ m holds, so these reductions equal the xor butterfly bit for bit.
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
  constexpr int CTRL = M == 1 ? 0xB1 : M == 2 ? 0x4E : M == 4 ? 0x141 : 0x140;
  return __builtin_amdgcn_update_dpp(0.0f, v, CTRL, 0xf, 0xf, false);
}

template <int WIDTH>
__device__ __forceinline__ void reduce_minmax(float& mn, float& mx) {
  static_assert(WIDTH == 4 || WIDTH == 8 || WIDTH == 16, "lane groups of 4, 8 or 16");
  mn = fminf(mn, lane_xor<1>(mn));
  mx = fmaxf(mx, lane_xor<1>(mx));
  mn = fminf(mn, lane_xor<2>(mn));
  mx = fmaxf(mx, lane_xor<2>(mx));
  if constexpr (WIDTH >= 8) {
    mn = fminf(mn, lane_xor<4>(mn));
    mx = fmaxf(mx, lane_xor<4>(mx));
  }
  if constexpr (WIDTH >= 16) {
    mn = fminf(mn, lane_xor<8>(mn));
    mx = fmaxf(mx, lane_xor<8>(mx));
  }
}

// Asymmetric min/max grid with zero forced into the range; an all-zero group
// uses [-1, 1].  rs is 1/s rounded to nearest, for div_rn.
__device__ __forceinline__ void grid_from_range(float mn, float mx, float maxq, float& s, float& z, float& rs) {
  float xmin = fminf(mn, 0.0f), xmax = fmaxf(mx, 0.0f);
  if (xmin == 0.0f && xmax == 0.0f) {
    xmin = -1.0f;
    xmax = 1.0f;
  }
  s = (xmax - xmin) / maxq;
  z = rintf(-xmin / s);
  rs = 1.0f / s;
}

// x / s rounded to nearest, given rs = 1/s rounded to nearest (s a positive
// normal number, x / s far from overflow and underflow).  Markstein's
// correction (P. Markstein, IBM J. Res. Dev. 34(1), 1990; also the
// Handbook of Floating-Point Arithmetic, division by iteration): when q is a
// faithful quotient, the residual x - q s is exact in one fma and
// q + residual * rs rounded to nearest is the correctly rounded quotient.
// x * rs is within 1.5 ulp, so a first correction makes it faithful and a
// second rounds it correctly; this keeps the loop's decision w / s identical
// to an IEEE division at 5 dependent instructions instead of the full
// division sequence.
__device__ __forceinline__ float div_rn(float x, float s, float rs) {
  float q = x * rs;
  float r = fmaf(-q, s, x);
  q = fmaf(r, rs, q);
  r = fmaf(-q, s, x);
  return fmaf(r, rs, q);
}

struct Lane {
  float w[8];    // the lane's 8 columns of the row
  float ru[8];   // 1 / U_jj of those columns (0 past the block's width)
  float4 un[2];  // U row of the next step at the lane's columns, read one step ahead
  float s, z, rs;
  int t;
};

// Step J of the block.  Columns past the block's width (a ragged last block)
// hold w = 0, U = 0 and 1/U_jj = 0, so their steps change nothing and every
// block runs all 128 steps without a branch between them.  Only the serial
// chain is done here: the owner lane of column J rounds it and forms e_J, the
// row's 16 lanes receive e_J and update their columns.  U is upper
// triangular, so no later step changes column J again: the final registers
// still hold every column's value at its decision, and codes, w^, e and the
// loss are formed after the loop from them with the same operations.
template <int MODE, int J>
__device__ __forceinline__ void step(Lane& L, const BlockArgs& a, const float (*Us)[B], int64_t row, bool row_ok) {
  constexpr int O = J >> 3, SL = J & 7;
  if constexpr (MODE != GM_BIG) {
    constexpr int GW = (MODE == GM_32) ? 32 : 64;
    if constexpr (J % GW == 0) {
      // every lane reduces its own aligned lane group; only the group starting at
      // column J is used from here on, the others are recomputed at their start
      constexpr int LANES = GW / 8;
      float mn = L.w[0], mx = L.w[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) {
        mn = fminf(mn, L.w[i]);
        mx = fmaxf(mx, L.w[i]);
      }
      reduce_minmax<LANES>(mn, mx);
      float s, z, rs;
      grid_from_range(mn, mx, a.maxq, s, z, rs);
      if ((L.t / LANES) == (O / LANES)) {
        L.s = s;
        L.z = z;
        L.rs = rs;
      }
      if (L.t == O && row_ok && J < a.bw) {
        const int64_t gi = (a.c0 + J) / a.g;
        a.scales[row * a.G + gi] = s;
        a.zeros[row * a.G + gi] = (uint8_t)z;
      }
    }
  }
  const float4 u0 = L.un[0], u1 = L.un[1];
  if constexpr (J + 1 < B) {
    L.un[0] = *reinterpret_cast<const float4*>(&Us[J + 1][8 * L.t]);
    L.un[1] = *reinterpret_cast<const float4*>(&Us[J + 1][8 * L.t + 4]);
  }
  const float x = L.w[SL];
  const float qv = fminf(fmaxf(rintf(div_rn(x, L.s, L.rs)) + L.z, 0.0f), a.maxq);
  const float ev = fmaf(-L.s, qv - L.z, x) * L.ru[SL];  // meaningful in the owner lane
  const float eb = row_bcast<O>(ev);
  // the column the next step rounds first, then the rest
  constexpr int NX = (J + 1) & 7;
  const float uu[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
  L.w[NX] = fmaf(-eb, uu[NX], L.w[NX]);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (i != NX) L.w[i] = fmaf(-eb, uu[i], L.w[i]);
}

template <int MODE, int... Js>
__device__ __forceinline__ void run_steps(Lane& L, const BlockArgs& a, const float (*Us)[B], int64_t row,
                                          bool row_ok, std::integer_sequence<int, Js...>) {
  (step<MODE, Js>(L, a, Us, row, row_ok), ...);
}

// LDS of one column-loop workgroup: the U block, 1/U_jj, and the previous
// block's update of its 16 rows.
constexpr int QUANT_LDS = B * B * 4 + B * 4 + 16 * B * 4;

// One workgroup of the block: rows 16 wg .. 16 wg + 15.  With a.Eprev the
// previous block's update of this block's columns, W[r, c0:c0+bw] -=
// Eprev[r, :] U[c0-128:c0, c0:c0+bw], is applied to the rows first (the rest
// of that update runs beside this block, see quant_run).  It runs on
// v_mfma_f32_16x16x4f32 with both operands straight from global memory
// (both are read by every workgroup of the launch, so they come from L2):
// wave v owns columns 32v .. 32v+31 as two 16-column tiles, and lane (i, g)
// (i = lane % 16, g = lane / 16) supplies k = 32g + kk at step kk, an order
// of k the sum does not care about, which makes its 32 values of E one
// contiguous run.  The product reaches the loop's layout through LDS.  The
// U block of the loop is loaded before that update, so its latency hides
// under it.
template <int MODE>
__device__ __forceinline__ void quant_block_wg(const BlockArgs& a, int64_t wg, char* lds) {
  GPTQ_TRACE_DECL;
  GPTQ_TRACE_STAMP();  // start
  float(*Us)[B] = reinterpret_cast<float(*)[B]>(lds);
  float* rUd = reinterpret_cast<float*>(lds + B * B * 4);
  float(*Es)[B] = reinterpret_cast<float(*)[B]>(lds + B * B * 4 + B * 4);
  const int tid = threadIdx.x;
  const int64_t c0 = a.c0, cols = a.cols;
  const int lane = tid & 63;
  const int64_t row = wg * 16 + (tid >> 6) * 4 + (lane >> 4);
  const bool row_ok = row < a.rows;
  const int t8 = 8 * (lane & 15);
  const int64_t base = row * cols + c0 + t8;
  const bool vec = a.bw == B && (cols & 3) == 0 && (reinterpret_cast<uintptr_t>(a.U) & 15) == 0;
  float w[8];
  if (vec && row_ok) {
    const float4 w0 = *reinterpret_cast<const float4*>(a.Wf + base);
    const float4 w1 = *reinterpret_cast<const float4*>(a.Wf + base + 4);
    w[0] = w0.x; w[1] = w0.y; w[2] = w0.z; w[3] = w0.w;
    w[4] = w1.x; w[5] = w1.y; w[6] = w1.z; w[7] = w1.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = (row_ok && t8 + i < a.bw) ? a.Wf[base + i] : 0.0f;
  }
  // loads first: E and U operands of the previous block's update, then the
  // U block of this one
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const int i16 = lane & 15, g = lane >> 4, wv = tid >> 6;
  float ea[32], ub[2][32];
  if (a.Eprev) {
    const int64_t er = wg * 16 + i16, cp = c0 - B;
    if (er < a.rows) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(a.Eprev + er * a.ldE + 32 * g + 4 * q);
        ea[4 * q + 0] = v.x; ea[4 * q + 1] = v.y; ea[4 * q + 2] = v.z; ea[4 * q + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < 32; ++kk) ea[kk] = 0.0f;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int col = 32 * wv + 16 * h + i16;
      const bool ok = col < a.bw;
      const float* src = a.U + (cp + 32 * g) * cols + c0 + (ok ? col : 0);
#pragma unroll
      for (int kk = 0; kk < 32; ++kk) ub[h][kk] = ok ? src[kk * cols] : 0.0f;
    }
  }
  // U block without its diagonal: Us[j][k] = U[c0+j][c0+k] for k > j inside
  // the block, else 0 (the feedback of step j reaches only k > j, so a column
  // keeps its decision-time value; 1/U_jj comes separately).  Whole blocks
  // with 16-byte rows load as 16 float4 per thread, all in flight at once.
  float4 uv[B * B / 4 / 256];
  if (vec) {
#pragma unroll
    for (int i = 0; i < B * B / 4 / 256; ++i) {
      const int idx = tid + 256 * i, j = idx >> 5, k = 4 * (idx & 31);
      uv[i] = *reinterpret_cast<const float4*>(a.U + (c0 + j) * cols + c0 + k);
    }
  }
  // U_jj for 1/U_jj, with the other loads
  const float udiag = tid < a.bw ? a.U[(c0 + tid) * cols + c0 + tid] : 1.0f;
  f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  if (a.Eprev) {
#pragma unroll
    for (int kk = 0; kk < 32; ++kk)
#pragma unroll
      for (int h = 0; h < 2; ++h) acc[h] = __builtin_amdgcn_mfma_f32_16x16x4f32(ea[kk], ub[h][kk], acc[h], 0, 0, 0);
  }
  GPTQ_TRACE_STAMP();  // operands loaded, near update issued
  if (vec) {
#pragma unroll
    for (int i = 0; i < B * B / 4 / 256; ++i) {
      const int idx = tid + 256 * i, j = idx >> 5, k = 4 * (idx & 31);
      float4 u = uv[i];
      u.x = k + 0 > j ? u.x : 0.0f;
      u.y = k + 1 > j ? u.y : 0.0f;
      u.z = k + 2 > j ? u.z : 0.0f;
      u.w = k + 3 > j ? u.w : 0.0f;
      *reinterpret_cast<float4*>(&Us[j][k]) = u;
    }
  } else {
    for (int idx = tid; idx < B * B; idx += 256) {
      const int j = idx >> 7, k = idx & (B - 1);
      float v = 0.0f;
      if (j < a.bw && k < a.bw && k > j) v = a.U[(c0 + j) * cols + c0 + k];
      Us[j][k] = v;
    }
  }
  if (tid < B) rUd[tid] = tid < a.bw ? 1.0f / udiag : 0.0f;
  if (a.Eprev) {
    // tile h holds D[4g + r][i16] for columns 32 wv + 16 h + i16
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) Es[4 * g + r][32 * wv + 16 * h + i16] = acc[h][r];
  }
  GPTQ_TRACE_STAMP();  // U block and update stored
  __syncthreads();
  GPTQ_TRACE_STAMP();  // barrier
  if (a.Eprev) {
    const int rl = (tid >> 6) * 4 + (lane >> 4);
    const float4 d0 = *reinterpret_cast<const float4*>(&Es[rl][t8]);
    const float4 d1 = *reinterpret_cast<const float4*>(&Es[rl][t8 + 4]);
    w[0] -= d0.x; w[1] -= d0.y; w[2] -= d0.z; w[3] -= d0.w;
    w[4] -= d1.x; w[5] -= d1.y; w[6] -= d1.z; w[7] -= d1.w;
  }

  Lane L;
  L.t = lane & 15;
#pragma unroll
  for (int i = 0; i < 8; ++i) L.w[i] = w[i];
#pragma unroll
  for (int i = 0; i < 8; ++i) L.ru[i] = rUd[8 * L.t + i];
  L.un[0] = *reinterpret_cast<const float4*>(&Us[0][8 * L.t]);
  L.un[1] = *reinterpret_cast<const float4*>(&Us[0][8 * L.t + 4]);
  L.s = 1.0f;
  L.z = 0.0f;
  L.rs = 1.0f;

  if constexpr (MODE == GM_BIG) {
    const int64_t gi = c0 / a.g;
    if (c0 % a.g == 0) {
      // group starts here: range over its columns in the current weights
      float mn = L.w[0], mx = L.w[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) {
        mn = fminf(mn, L.w[i]);
        mx = fmaxf(mx, L.w[i]);
      }
      const int64_t gend = (c0 + a.g) < cols ? (c0 + a.g) : cols;
      if (row_ok) {
        for (int64_t cb = c0 + B; cb < gend; cb += B) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int64_t c = cb + 8 * L.t + i;
            if (c < gend) {
              const float v = a.Wf[row * cols + c];
              mn = fminf(mn, v);
              mx = fmaxf(mx, v);
            }
          }
        }
      }
      reduce_minmax<16>(mn, mx);
      grid_from_range(mn, mx, a.maxq, L.s, L.z, L.rs);
      if (L.t == 0 && row_ok) {
        a.scales[row * a.G + gi] = L.s;
        a.zeros[row * a.G + gi] = (uint8_t)L.z;
      }
    } else if (row_ok) {
      L.s = a.scales[row * a.G + gi];
      L.z = (float)a.zeros[row * a.G + gi];
      L.rs = 1.0f / L.s;
    }
  }

  GPTQ_TRACE_STAMP();  // update applied, group range taken
  run_steps<MODE>(L, a, Us, row, row_ok, std::make_integer_sequence<int, B>{});
  GPTQ_TRACE_STAMP();  // 128 steps

  // every column's decision again, from its value at decision time (the step's
  // operations exactly); e and the loss vanish past the block's width
  float q[8], wh[8], e[8], ls = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float x = L.w[i];
    q[i] = fminf(fmaxf(rintf(div_rn(x, L.s, L.rs)) + L.z, 0.0f), a.maxq);
    wh[i] = L.s * (q[i] - L.z);
    e[i] = fmaf(-L.s, q[i] - L.z, x) * L.ru[i];
    ls += 0.5f * e[i] * e[i];
  }
  // loss over the row's 16 lanes
  ls += lane_xor<1>(ls);
  ls += lane_xor<2>(ls);
  ls += lane_xor<4>(ls);
  ls += lane_xor<8>(ls);
  if (!row_ok) return;
  if (L.t == 0) a.row_loss[row] = (c0 == 0 ? 0.0f : a.row_loss[row]) + ls;
  const bool full = (8 * L.t + 8 <= a.bw);
  uint8_t* cp = a.codes + base;
  if (full && ((cols & 7) == 0)) {
    uint2 pk;
    pk.x = (uint32_t)q[0] | ((uint32_t)q[1] << 8) | ((uint32_t)q[2] << 16) | ((uint32_t)q[3] << 24);
    pk.y = (uint32_t)q[4] | ((uint32_t)q[5] << 8) | ((uint32_t)q[6] << 16) | ((uint32_t)q[7] << 24);
    *reinterpret_cast<uint2*>(cp) = pk;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (8 * L.t + i < a.bw) cp[i] = (uint8_t)q[i];
  }
  if (a.w_hat) {
    float* hp = a.w_hat + base;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (8 * L.t + i < a.bw) hp[i] = wh[i];
  }
  float* ep = a.E + row * a.ldE + 8 * L.t;
  *reinterpret_cast<float4*>(ep) = make_float4(e[0], e[1], e[2], e[3]);
  *reinterpret_cast<float4*>(ep + 4) = make_float4(e[4], e[5], e[6], e[7]);
  GPTQ_TRACE_STAMP();  // outputs written
  GPTQ_TRACE_WRITE(TR_LOOP, a.c0 / B);
}

// One launch per 128-column block b: the column loop of block b (workgroups
// 0 .. nq-1, each applying the previous block's update of its own columns
// first) and, beside it, up to two jobs of the trailing update as split-bf16
// GEMM tiles (sgemm_tile.h, workgroups nq ..).  All of them touch columns past
// block b and read errors of blocks before b, so nothing in one launch
// depends on another part of it; a loop workgroup (latency bound) and a GEMM
// tile fit on one CU together, so the GEMM fills the loop's idle issue slots.
struct FarJobs {
  SplitGemm g[2];
  int tn[2];      // tile columns of each job
  int start[3];   // first tile of each job; start[2] = all tiles
};

template <int MODE>
__global__ __launch_bounds__(256, 2) void k_quant_fused(BlockArgs a, FarJobs far, int64_t nq) {
  constexpr int LDS = QUANT_LDS > SGEMM_LDS ? QUANT_LDS : SGEMM_LDS;
  __shared__ __attribute__((aligned(16))) char lds[LDS];
  if ((int64_t)blockIdx.x < nq) {
    quant_block_wg<MODE>(a, blockIdx.x, lds);
  } else {
    const int t = (int)(blockIdx.x - nq);
    const int j = t < far.start[1] ? 0 : 1;
    const int u = t - far.start[j];
    sgemm_tile(far.g[j], u / far.tn[j], u % far.tn[j], lds);
  }
}

template <int MODE>
hipError_t launch_block(const BlockArgs& a, FarJobs far, int64_t nq, hipStream_t stream) {
  int64_t tiles = 0;
  for (int j = 0; j < 2; ++j) {
    far.start[j] = (int)tiles;
    far.tn[j] = 1;
    if (far.g[j].M > 0 && far.g[j].N > 0 && far.g[j].K > 0) {
      far.tn[j] = (far.g[j].N + STM - 1) / STM;
      tiles += (int64_t)((far.g[j].M + STM - 1) / STM) * far.tn[j];
    }
  }
  far.start[2] = (int)tiles;
  hipLaunchKernelGGL((k_quant_fused<MODE>), dim3((unsigned)(nq + tiles)), dim3(256), 0, stream, a, far, nq);
  return hipGetLastError();
}

}  // namespace

#ifdef GPTQ_TRACE
GPTQ_TRACE_SETTER(trace_set_quant)
#endif

size_t quant_split_bytes(int64_t cols, int64_t groupsize) {
  const bool overlap = groupsize <= B || groupsize >= cols;
  if (!overlap || cols <= 2 * B) return 0;
  return (size_t)3 * cols * cols * sizeof(uint16_t);
}

hipError_t quant_run(const QuantArgs& q, hipStream_t stream) {
  const int64_t rows = q.rows, cols = q.cols;
  {
    const int64_t total = rows * cols;
    const int is_bf16 = q.w_dtype == GPTQ_BF16 ? 1 : 0;
    const uintptr_t wa = reinterpret_cast<uintptr_t>(q.W);
    if (cols % 8 == 0 && (wa & (is_bf16 ? 15 : 31)) == 0 && (reinterpret_cast<uintptr_t>(q.Wf) & 31) == 0) {
      int64_t blocks = (total / 8 + 255) / 256;
      if (blocks > 16384) blocks = 16384;
      hipLaunchKernelGGL(k_stage_w8, dim3((unsigned)blocks), dim3(256), 0, stream, q.W, is_bf16, rows, cols, q.dead,
                         q.Wf);
    } else {
      int64_t blocks = (total + 255) / 256;
      if (blocks > 65536) blocks = 65536;
      hipLaunchKernelGGL(k_stage_w, dim3((unsigned)blocks), dim3(256), 0, stream, q.W, is_bf16, rows, cols, q.dead,
                         q.Wf);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  BlockArgs a{};
  a.Wf = q.Wf;
  a.U = q.U;
  a.rows = rows;
  a.cols = cols;
  a.maxq = (float)((1 << q.bits) - 1);
  a.g = q.groupsize;
  a.G = q.G;
  a.codes = q.codes;
  a.scales = q.scales;
  a.zeros = q.zeros;
  a.w_hat = q.w_hat;
  a.row_loss = q.row_loss;
  const int mode = (q.groupsize == 32) ? GM_32 : (q.groupsize == 64) ? GM_64 : GM_BIG;
  // The previous block's update of later columns can run beside a block only
  // when no group range reaches past the block being quantized: groups inside
  // a block, or one group per row (its range is taken before any update).
  const bool overlap = q.groupsize <= B || q.groupsize >= cols;
  // errors of every block, kept for the whole layer: E_b = E[:, 128 b : 128 b + 128]
  const int64_t nb = (cols + B - 1) / B, ldE = nb * B;
  a.ldE = ldE;
  if (overlap && cols > 2 * B) {
    if (!q.Usplit) return hipErrorInvalidValue;
    const unsigned gy = (unsigned)(cols < 65535 ? cols : 65535);
    if (cols % 8 == 0 && (reinterpret_cast<uintptr_t>(q.U) & 15) == 0) {
      const unsigned gx = (unsigned)((cols / 8 + 255) / 256);
      hipLaunchKernelGGL(k_split_u8, dim3(gx, gy), dim3(256), 0, stream, q.U, cols, q.Usplit);
    } else {
      const unsigned gx = (unsigned)((cols + 255) / 256 < 16 ? (cols + 255) / 256 : 16);
      hipLaunchKernelGGL(k_split_u, dim3(gx, gy), dim3(256), 0, stream, q.U, cols, q.Usplit);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t nq = (rows + 15) / 16;
  int64_t b = 0;
  for (int64_t c0 = 0; c0 < cols; c0 += B, ++b) {
    a.c0 = c0;
    a.bw = (int)((cols - c0) < B ? (cols - c0) : B);
    a.E = q.E + b * B;
    a.Eprev = (overlap && b > 0) ? q.E + (b - 1) * B : nullptr;
    // The trailing update in two levels (quant_schedule.h): the errors of
    // block e reach the column blocks of its own group beyond e + 1 in launch
    // e + 1 (block e + 1 itself from the loop workgroups of that launch), and
    // the column blocks past the group receive the whole group at once in the
    // launch after the group's last block.
    FarJobs far{};
    if (overlap && b > 0) {
      auto job = [&](SplitGemm& g, int64_t e0, int64_t ne, int64_t j0, int64_t j1) {  // blocks [e0, e0+ne) -> [j0, j1]
        g.A = q.E + e0 * B;
        for (int p = 0; p < 3; ++p) g.B[p] = q.Usplit + (int64_t)p * cols * cols + (e0 * B) * cols + j0 * B;
        g.C = q.Wf + j0 * B;
        g.lda = ldE;
        g.ldb = cols;
        g.ldc = cols;
        g.M = (int)rows;
        g.N = (int)((j1 + 1) * B < cols ? (j1 + 1 - j0) * B : cols - j0 * B);
        g.K = (int)(ne * B);
      };
      UpdateJob jobs[2];
      update_jobs(b, nb, jobs);
      for (int k = 0; k < 2; ++k)
        if (jobs[k].ne > 0) job(far.g[k], jobs[k].e0, jobs[k].ne, jobs[k].j0, jobs[k].j1);
    }
    hipError_t e;
    if (mode == GM_32)
      e = launch_block<GM_32>(a, far, nq, stream);
    else if (mode == GM_64)
      e = launch_block<GM_64>(a, far, nq, stream);
    else
      e = launch_block<GM_BIG>(a, far, nq, stream);
    if (e != hipSuccess) return e;
    const int64_t c1 = c0 + B;
    if (!overlap && c1 < cols) {
      GemmF32 g{};
      g.A = a.E;
      g.lda = ldE;
      g.B = q.U + c0 * cols + c1;
      g.ldb = cols;
      g.b_kmajor = 1;
      g.C = q.Wf + c1;
      g.ldc = cols;
      g.M = (int)rows;
      g.N = (int)(cols - c1);
      g.K = B;
      g.alpha = -1.0f;
      g.beta = 1;
      g.batch = 1;
      e = gemm_f32(g, stream);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace gptq
