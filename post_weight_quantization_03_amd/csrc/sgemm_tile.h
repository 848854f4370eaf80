// fp32 GEMM update C -= A B on bf16 MFMA, by splitting each fp32 operand into
// three bf16 terms, x = x1 + x2 + x3 (x1 = bf16(x), x2 = bf16(x - x1),
// x3 = bf16(x - x1 - x2); both differences are exact in fp32).  With
// |x2| <= 2^-8 |x| and |x3| <= 2^-16 |x| (round to nearest on 8 significant
// bits), the six products
//
//   a1 b1 + a1 b2 + a2 b1 + a1 b3 + a2 b2 + a3 b1
//
// leave out terms of relative size 2^-24 and below (a2 b3, a3 b2, a3 b3, and
// the 2^-24 residue of each split), the unit roundoff of fp32 itself.  Each
// bf16 x bf16 product is exact in fp32 and the MFMA accumulates in fp32, so
// the update is as accurate as an fp32 GEMM, at six bf16 MFMAs per product
// where an fp32 MFMA of the same shape takes sixteen times as long.
//
// A is fp32, m-major (row m holds its K values), and is split in registers
// after its LDS read.  B comes pre-split as three k-major bf16 planes (row k
// holds its N values).
//
// Tile 128 x 128 per workgroup of 256 threads: four waves in a 2x2 grid, each
// owning 64 x 64 as 2x2 blocks of v_mfma_f32_32x32x16_bf16.  A stage is 16 k:
//   A part: 128 rows x 64 bytes of fp32, the fp32 GEMM's m-major layout; a
//     lane's 8 k of one row are two 16-byte reads;
//   B part: three planes of 16 k rows x 256 bytes, chunk XORed with
//     4 (row & 3); a lane's 8 k of one column come from two ds_read_b64_tr_b16
//     (rows +0 and +4 of its 8-row group), as in the Hessian kernel.
// 20 KB a stage; stages reach LDS by direct loads, four buffers rotate with
// the fp32 GEMM's counted-wait pipeline.  Tiles not whole or not aligned take
// a guarded register path into the same layouts.
#pragma once
#include "gemm_tile.h"

namespace gptq {
namespace {

struct SplitGemm {
  const float* A;        // m-major [M][lda] fp32
  const uint16_t* B[3];  // k-major planes [K][ldb] (bf16 bits)
  float* C;              // C[m * ldc + n] -= sum_k A(m, k) B(k, n)
  int64_t lda, ldb, ldc;
  int M, N, K;           // K a multiple of 16
};

constexpr int SKS = 16;                          // k per stage
constexpr int STM = 128;                         // tile
constexpr int S_AB = STM * SKS * 4;              // 8 KB: A part (fp32)
constexpr int S_BROW = STM * 2;                  // bytes of one k row of a B plane
constexpr int S_BP = SKS * S_BROW;               // 4 KB: one B plane
constexpr int S_STAGE = S_AB + 3 * S_BP;         // 20 KB
constexpr int SGEMM_LDS = 4 * S_STAGE;           // 80 KB
constexpr int S_LPW = 5;                         // direct loads per wave and stage (2 A + 3 B)

__device__ __forceinline__ int sb_off(int row, int col) {
  const int phys = (col >> 3) ^ ((row & 3) << 2);
  return row * S_BROW + (phys << 4) + ((col & 7) << 1);
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) f32x4_t lds_f32x4_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;

// B operand of the 32-column block at c0 (see the Hessian kernel's frag_off:
// the same pattern on 256-byte rows).
__device__ __forceinline__ int sb_frag_off(int c0, int lane) {
  const int g = lane >> 4, s = lane & 15;
  return sb_off(8 * (g >> 1) + (s >> 2), c0 + 16 * (g & 1) + 4 * (s & 3));
}

__device__ __forceinline__ bf16x8 sb_frag(const char* p) {
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(lds_char*)p);
  const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(lds_char*)(p + 4 * S_BROW));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// fp32 -> three bf16 terms (round to nearest even each time).

// Direct loads of one stage (5 a wave).  A: 1 KB = 16 rows of 64 bytes
// (the fp32 GEMM's dma_mmajor offsets); B: 1 KB = 4 k rows of one plane.
struct SDma {
  uint32_t a_off[2], b_off[3];
  int b_plane[3], b_dst[3];
};

__device__ __forceinline__ SDma sdma_offsets(const SplitGemm& g, int wave, int lane) {
  SDma d;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int inst = wave * 2 + i;
    const int r = 16 * inst + (lane >> 2);
    const int lc = (lane & 3) ^ ((r >> 2) & 3);
    d.a_off[i] = (uint32_t)(((int64_t)r * g.lda + 4 * lc) * 4);
  }
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int inst = wave * 3 + i;  // 0 .. 11: plane inst / 4, rows 4 (inst % 4) ..
    const int plane = inst >> 2, kr = 4 * (inst & 3) + (lane >> 4);
    const int c = (lane & 15) ^ ((kr & 3) << 2);
    d.b_off[i] = (uint32_t)(((int64_t)kr * g.ldb + 8 * c) * 2);
    d.b_plane[i] = plane;
    d.b_dst[i] = S_AB + plane * S_BP + (inst & 3) * 1024;
  }
  return d;
}

__device__ __forceinline__ const char* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  return reinterpret_cast<const char*>((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v) |
                                       ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32))
                                        << 32));
}

// Queue stage st into buf.  Issued from asm: every wait on these loads is an
// explicit counted s_waitcnt, so the compiler's wait insertion must not see
// them.
__device__ __forceinline__ void sdma_issue(const SplitGemm& g, const SDma& d, int st, int m0, int n0, char* buf,
                                           int wave) {
  const int k0 = st * SKS;
  const char* ab = uniform_ptr(g.A + (int64_t)m0 * g.lda + k0);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t la = (uint32_t)(uintptr_t)(lds_char*)(buf + (wave * 2 + i) * 1024);
    asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(d.a_off[i]), "s"(ab), "{m0}"(la));
  }
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int plane = __builtin_amdgcn_readfirstlane(d.b_plane[i]);
    const char* bb = uniform_ptr(g.B[plane] + (int64_t)k0 * g.ldb + n0);
    const uint32_t lb = (uint32_t)(uintptr_t)(lds_char*)(buf + __builtin_amdgcn_readfirstlane(d.b_dst[i]));
    asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(d.b_off[i]), "s"(bb), "{m0}"(lb));
  }
}

// Guarded stage: zero outside [0, M) x [0, N).
__device__ __forceinline__ void sstage_guarded(const SplitGemm& g, int st, int m0, int n0, char* buf) {
  const int k0 = st * SKS;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = threadIdx.x + 256 * i;  // 512 float4 chunks of A
    const int r = q >> 2, c = q & 3;
    const int64_t gm = m0 + r;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = gm < g.M ? g.A[gm * g.lda + k0 + 4 * c + e] : 0.f;
    const f32x4_t vv = {v[0], v[1], v[2], v[3]};
    *(lds_f32x4_t*)(lds_char*)(buf + mm_off(r, c)) = vv;
  }
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int q = threadIdx.x + 256 * i;  // 768 chunks of 8 bf16: plane q / 256
    const int plane = q >> 8, kr = (q >> 4) & 15, c = q & 15;
    const uint16_t* Bp = g.B[plane];
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t gn0 = n0 + 8 * c + 2 * e;
      const uint32_t lo = gn0 < g.N ? Bp[(int64_t)(k0 + kr) * g.ldb + gn0] : 0u;
      const uint32_t hi = gn0 + 1 < g.N ? Bp[(int64_t)(k0 + kr) * g.ldb + gn0 + 1] : 0u;
      w[e] = lo | (hi << 16);
    }
    const u32x4_t wv = {w[0], w[1], w[2], w[3]};
    *(lds_u32x4_t*)(lds_char*)(buf + S_AB + plane * S_BP + sb_off(kr, 8 * c)) = wv;
  }
}

__device__ __forceinline__ void sstage_mfma(const char* buf, int wm, int wn, int lane, f32x16 (&acc)[2][2]) {
  const int j = lane & 31, h = lane >> 5;
  // A: this lane's 8 k (8h .. 8h+7) of rows wm*64 + 32 bi + j, split three ways
  bf16x8 a[2][3];
#pragma unroll
  for (int bi = 0; bi < 2; ++bi) {
    const int row = wm * 64 + 32 * bi + j;
    const f32x4_t lo = *(const lds_f32x4_t*)(lds_char*)(buf + mm_off(row, 2 * h));
    const f32x4_t hi = *(const lds_f32x4_t*)(lds_char*)(buf + mm_off(row, 2 * h + 1));
    const float x[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      __bf16 h1, h2, h3;
      split3(x[e], h1, h2, h3);
      a[bi][0][e] = h1;
      a[bi][1][e] = h2;
      a[bi][2][e] = h3;
    }
  }
  bf16x8 b[2][3];
#pragma unroll
  for (int bj = 0; bj < 2; ++bj)
#pragma unroll
    for (int p = 0; p < 3; ++p) b[bj][p] = sb_frag(buf + S_AB + p * S_BP + sb_frag_off(wn * 64 + 32 * bj, lane));
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) {
      f32x16 c = acc[bi][bj];
      c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[bi][2], b[bj][0], c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[bi][1], b[bj][1], c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[bi][0], b[bj][2], c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[bi][1], b[bj][0], c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[bi][0], b[bj][1], c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[bi][0], b[bj][0], c, 0, 0, 0);
      acc[bi][bj] = c;
    }
}

template <int N>
__device__ __forceinline__ void swait_barrier() {
  if constexpr (N == 0)
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 5)
    asm volatile("s_waitcnt vmcnt(5)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 10)
    asm volatile("s_waitcnt vmcnt(10)\n\ts_barrier" ::: "memory");
  else
    static_assert(N == 0, "unsupported count");
}

// One 128 x 128 tile (tm, tn) of C -= A B; lds holds SGEMM_LDS bytes.
__device__ __forceinline__ void sgemm_tile(const SplitGemm& g, int tm, int tn, char* lds) {
  const int m0 = tm * STM, n0 = tn * STM;
  if (m0 >= g.M || n0 >= g.N) return;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  const int nst = g.K / SKS;
  bool aligned = (g.lda % 4) == 0 && (g.ldb % 8) == 0 && (reinterpret_cast<uintptr_t>(g.A) & 15) == 0;
#pragma unroll
  for (int p = 0; p < 3; ++p) aligned = aligned && (reinterpret_cast<uintptr_t>(g.B[p]) & 15) == 0;
  const bool whole = aligned && m0 + STM <= g.M && n0 + STM <= g.N;
  auto ccol = [&](int bj) { return n0 + wn * 64 + 32 * bj + (lane & 31); };
  auto crow = [&](int bi, int r) { return m0 + wm * 64 + 32 * bi + acc_row(r, lane); };

  if (whole && nst > 0) {
    // C is read ahead of the K loop (older than every direct load, so the
    // counted waits retire it first)
    float cpre[2][16][2];
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
      for (int r = 0; r < 16; ++r)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj) cpre[bi][r][bj] = g.C[(int64_t)crow(bi, r) * g.ldc + ccol(bj)];
    const SDma d = sdma_offsets(g, wave, lane);
    char* bufs[4] = {lds, lds + S_STAGE, lds + 2 * S_STAGE, lds + 3 * S_STAGE};
    // stages 0..2 queued; stage 0 and stage 1 retired a barrier apart
    sdma_issue(g, d, 0, m0, n0, bufs[0], wave);
    if (nst > 1) sdma_issue(g, d, 1, m0, n0, bufs[1], wave);
    if (nst > 2) sdma_issue(g, d, 2, m0, n0, bufs[2], wave);
    if (nst > 2)
      swait_barrier<2 * S_LPW>();
    else if (nst > 1)
      swait_barrier<S_LPW>();
    else
      swait_barrier<0>();
    if (nst > 2)
      swait_barrier<S_LPW>();
    else
      swait_barrier<0>();
    // stage s: queue s+3 into the buffer stage s-1 used, MFMAs on s, retire
    // s+2 (read one full stage later)
    for (int s = 0; s < nst; ++s) {
      const bool more = s + 3 < nst;
      if (more) sdma_issue(g, d, s + 3, m0, n0, bufs[(s + 3) & 3], wave);
      sstage_mfma(bufs[s & 3], wm, wn, lane, acc);
      if (more)
        swait_barrier<S_LPW>();
      else
        swait_barrier<0>();
    }
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
      for (int r = 0; r < 16; ++r)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
          g.C[(int64_t)crow(bi, r) * g.ldc + ccol(bj)] = cpre[bi][r][bj] - acc[bi][bj][r];
    return;
  }
  for (int s = 0; s < nst; ++s) {
    __syncthreads();
    sstage_guarded(g, s, m0, n0, lds);
    __syncthreads();
    sstage_mfma(lds, wm, wn, lane, acc);
  }
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = crow(bi, r);
      if (m >= g.M) continue;
#pragma unroll
      for (int bj = 0; bj < 2; ++bj) {
        const int n = ccol(bj);
        if (n < g.N) {
          float* p = g.C + (int64_t)m * g.ldc + n;
          *p = *p - acc[bi][bj][r];
        }
      }
    }
}

}  // namespace
}  // namespace gptq
