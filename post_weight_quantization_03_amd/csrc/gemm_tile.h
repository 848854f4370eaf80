// fp32 MFMA GEMM tile, shared by the GEMM kernel and the fused column-loop
// kernel.  See k_gemm.hip for the design.
#pragma once
#include <type_traits>

#include "common.h"

namespace gptq {
namespace {


constexpr int KS = 16;  // k per stage

typedef __attribute__((address_space(3))) char lds_char;

template <int TM>
struct Geo {
  static constexpr int NB = TM / 64;            // 32x32 blocks per wave and dimension
  static constexpr int HALF = TM / 2;           // wave quarter edge
  static constexpr int OPB = TM * KS * 4;       // bytes of one operand stage
  static constexpr int LPW = OPB / 1024 / 4;    // direct loads per wave and operand stage
  static constexpr int KROW = TM * 4;           // bytes of one k row of a k-major stage
};

__device__ __forceinline__ int mm_off(int row, int chunk) { return row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4); }

// Direct loads of one operand: a wave-uniform base (advanced one stage per
// call; the empty asm keeps loop strength reduction from turning it into one
// VGPR address per load) plus per-lane byte offsets fixed for the whole K loop.
template <int TM>
struct DmaOp {
  const char* base;
  int64_t step;  // bytes per stage
  uint32_t off[Geo<TM>::LPW];
};

// m-major operand rows r0 .. r0+TM-1 of P (leading dimension ld), k from k0.
template <int TM>
__device__ __forceinline__ DmaOp<TM> dma_mmajor(const float* P, int64_t ld, int64_t r0, int64_t k0, int wave,
                                                int lane) {
  DmaOp<TM> d;
  d.base = reinterpret_cast<const char*>(P + r0 * ld + k0);
  d.step = KS * 4;
#pragma unroll
  for (int i = 0; i < Geo<TM>::LPW; ++i) {
    const int inst = wave * Geo<TM>::LPW + i;  // 1 KB = 16 rows of 64 bytes
    const int r = 16 * inst + (lane >> 2);
    const int lc = (lane & 3) ^ ((r >> 2) & 3);
    d.off[i] = (uint32_t)(((int64_t)r * ld + 4 * lc) * 4);
  }
  return d;
}

// k-major B: rows k0 .. k0+15 of Bm (leading dimension ld), columns n0 ..
template <int TM>
__device__ __forceinline__ DmaOp<TM> dma_kmajor(const float* Bm, int64_t ld, int64_t k0, int64_t n0, int wave,
                                                int lane) {
  DmaOp<TM> d;
  d.base = reinterpret_cast<const char*>(Bm + k0 * ld + n0);
  d.step = (int64_t)KS * ld * 4;
  constexpr int CPR = TM / 4;  // 16-byte chunks per k row
#pragma unroll
  for (int i = 0; i < Geo<TM>::LPW; ++i) {
    const int inst = wave * Geo<TM>::LPW + i;
    const int q = inst * 64 + lane;  // chunk index in the stage
    const int r = q / CPR, c = q % CPR;
    d.off[i] = (uint32_t)(((int64_t)r * ld + 4 * c) * 4);
  }
  return d;
}

template <int TM>
__device__ __forceinline__ void dma_issue(DmaOp<TM>& d, char* dst, int wave) {
  // issued from asm: only the whole-tile pipeline uses these loads and every
  // wait on them there is an explicit counted s_waitcnt, so the compiler's
  // wait insertion (which would drain them all at the loop's back edge) must
  // not see them
#pragma unroll
  for (int i = 0; i < Geo<TM>::LPW; ++i) {
    const uint32_t lds = (uint32_t)(uintptr_t)(lds_char*)(dst + (wave * Geo<TM>::LPW + i) * 1024);
    asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(d.off[i]), "s"(d.base), "{m0}"(lds));
  }
  uint64_t b = reinterpret_cast<uint64_t>(d.base) + (uint64_t)d.step;
  asm volatile("" : "+s"(b));
  d.base = reinterpret_cast<const char*>(b);
}

// Guarded stage load: element (row, k) of an m-major operand or (k, col) of a
// k-major one, zero outside [0, rows) x [kbeg, kend).
template <int TM>
__device__ __forceinline__ void guarded_mmajor(const float* P, int64_t ld, int64_t r0, int64_t rows, int64_t k0,
                                               int64_t kend, char* dst) {
  constexpr int PER = TM * 4 / 256;  // float4 chunks per thread
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int q = threadIdx.x + 256 * i;
    const int r = q >> 2, c = q & 3;
    const int64_t gr = r0 + r, gk = k0 + 4 * c;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (gr < rows && gk + e < kend) ? P[gr * ld + gk + e] : 0.f;
    *reinterpret_cast<float4*>(dst + mm_off(r, c)) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

template <int TM>
__device__ __forceinline__ void guarded_kmajor(const float* Bm, int64_t ld, int64_t k0, int64_t kend, int64_t n0,
                                               int64_t cols, char* dst) {
  constexpr int PER = TM * 4 / 256;
  constexpr int CPR = TM / 4;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int q = threadIdx.x + 256 * i;
    const int r = q / CPR, c = q % CPR;
    const int64_t gk = k0 + r, gn = n0 + 4 * c;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (gk < kend && gn + e < cols) ? Bm[gk * ld + gn + e] : 0.f;
    *reinterpret_cast<float4*>(dst + r * Geo<TM>::KROW + 16 * c) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

// MFMAs of one stage held in `buf` (A part at 0, B part at OPB).
template <int TM, bool BKM>
__device__ __forceinline__ void stage_mfma(const char* buf, int wm, int wn, int lane,
                                           f32x16 (&acc)[Geo<TM>::NB][Geo<TM>::NB]) {
  constexpr int NB = Geo<TM>::NB, HALF = Geo<TM>::HALF;
  const char* As = buf;
  const char* Bs = buf + Geo<TM>::OPB;
  const int j = lane & 31, h = lane >> 5;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    float4 a[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
      a[b] = *reinterpret_cast<const float4*>(As + mm_off(wm * HALF + 32 * b + j, 2 * h + q));
    if constexpr (!BKM) {
      float4 bv[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b)
        bv[b] = *reinterpret_cast<const float4*>(Bs + mm_off(wn * HALF + 32 * b + j, 2 * h + q));
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int bi = 0; bi < NB; ++bi)
#pragma unroll
          for (int bj = 0; bj < NB; ++bj)
            acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[bi][e], bv[bj][e], acc[bi][bj], 0, 0, 0);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k = 8 * h + 4 * q + e;
        float bv[NB];
        const char* p = Bs + k * Geo<TM>::KROW + (wn * HALF + NB * j) * 4;
        if constexpr (NB == 2) {
          const float2 v = *reinterpret_cast<const float2*>(p);
          bv[0] = v.x;
          bv[1] = v.y;
        } else {
          bv[0] = *reinterpret_cast<const float*>(p);
        }
#pragma unroll
        for (int bi = 0; bi < NB; ++bi)
#pragma unroll
          for (int bj = 0; bj < NB; ++bj)
            acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[bi][e], bv[bj], acc[bi][bj], 0, 0, 0);
      }
    }
  }
}

// x = h1 + h2 + h3 in bf16 terms (both differences exact in fp32); see
// sgemm_tile.h for why six products of the terms keep fp32 accuracy.
__device__ __forceinline__ void split3(float x, __bf16& h1, __bf16& h2, __bf16& h3) {
  h1 = (__bf16)x;
  const float r1 = x - (float)h1;
  h2 = (__bf16)r1;
  const float r2 = r1 - (float)h2;
  h3 = (__bf16)r2;
}

// The stage's MFMAs on bf16 matrix cores with both fp32 operands split three
// ways in registers (A m-major, B n-major, the same LDS layout): lane half h
// supplies k = 8h .. 8h+7 of its row and column to v_mfma_f32_32x32x16_bf16,
// exactly the 8 values of its two 16-byte reads; six products per block
// pair, the small ones first.
template <int TM>
__device__ __forceinline__ void stage_mfma_split(const char* buf, int wm, int wn, int lane,
                                                 f32x16 (&acc)[Geo<TM>::NB][Geo<TM>::NB]) {
  constexpr int NB = Geo<TM>::NB, HALF = Geo<TM>::HALF;
  const int j = lane & 31, h = lane >> 5;
  bf16x8 a[NB][3], b[NB][3];
#pragma unroll
  for (int o = 0; o < 2; ++o) {
    const char* S = o == 0 ? buf : buf + Geo<TM>::OPB;
    const int w0 = o == 0 ? wm : wn;
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const int row = w0 * HALF + 32 * q + j;
      const float4 lo = *reinterpret_cast<const float4*>(S + mm_off(row, 2 * h));
      const float4 hi = *reinterpret_cast<const float4*>(S + mm_off(row, 2 * h + 1));
      const float x[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        __bf16 h1, h2, h3;
        split3(x[e], h1, h2, h3);
        if (o == 0) {
          a[q][0][e] = h1; a[q][1][e] = h2; a[q][2][e] = h3;
        } else {
          b[q][0][e] = h1; b[q][1][e] = h2; b[q][2][e] = h3;
        }
      }
    }
  }
#pragma unroll
  for (int bi = 0; bi < NB; ++bi)
#pragma unroll
    for (int bj = 0; bj < NB; ++bj) {
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
__device__ __forceinline__ void wait_barrier() {
  if constexpr (N == 0)
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 2)
    asm volatile("s_waitcnt vmcnt(2)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 4)
    asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 8)
    asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 16)
    asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
  else
    static_assert(N == 0, "unsupported count");
}

template <int TM>
__device__ __forceinline__ void issue_stage(DmaOp<TM>& da, DmaOp<TM>& db, char* dst, int wave) {
  dma_issue<TM>(da, dst, wave);
  dma_issue<TM>(db, dst + Geo<TM>::OPB, wave);
}

// stage s: queue s+3 into the buffer stage s-1 used, MFMAs on stage s,
// retire stage s+2
template <int TM, bool BKM, bool SPLIT>
__device__ __forceinline__ void pipe_body(int s, int nst, const char* cur, char* nxt3, DmaOp<TM>& da,
                                          DmaOp<TM>& db, int wave, int wm, int wn, int lane,
                                          f32x16 (&acc)[Geo<TM>::NB][Geo<TM>::NB]) {
  const bool more = s + 3 < nst;
  if (more) issue_stage<TM>(da, db, nxt3, wave);
  if constexpr (SPLIT)
    stage_mfma_split<TM>(cur, wm, wn, lane, acc);
  else
    stage_mfma<TM, BKM>(cur, wm, wn, lane, acc);
  if (more)
    wait_barrier<2 * Geo<TM>::LPW>();
  else
    wait_barrier<0>();
}

// The whole-tile K loop.  The four buffers arrive as distinct restrict
// pointers so that every direct load and LDS read inside carries alias-scope
// information: the compiler's wait insertion then only waits for loads into
// the buffer being read (retired long before by the counted barriers) instead
// of draining every direct load before each read.
template <int TM, bool BKM, bool SPLIT>
__device__ __forceinline__ void pipeline(char* __restrict__ S0, char* __restrict__ S1, char* __restrict__ S2,
                                         char* __restrict__ S3, DmaOp<TM>& da, DmaOp<TM>& db, int nst, int wave,
                                         int wm, int wn, int lane, f32x16 (&acc)[Geo<TM>::NB][Geo<TM>::NB]) {
  constexpr int LW = 2 * Geo<TM>::LPW;  // direct loads per wave and stage (both operands)
  issue_stage<TM>(da, db, S0, wave);
  if (nst > 1) issue_stage<TM>(da, db, S1, wave);
  if (nst > 2) issue_stage<TM>(da, db, S2, wave);
  // retire stage 0, then stage 1, a barrier apart
  if (nst > 2)
    wait_barrier<2 * LW>();
  else if (nst > 1)
    wait_barrier<LW>();
  else
    wait_barrier<0>();
  if (nst > 2)
    wait_barrier<LW>();
  else
    wait_barrier<0>();
  for (int s = 0; s < nst; s += 4) {
    pipe_body<TM, BKM, SPLIT>(s, nst, S0, S3, da, db, wave, wm, wn, lane, acc);
    if (s + 1 >= nst) break;
    pipe_body<TM, BKM, SPLIT>(s + 1, nst, S1, S0, da, db, wave, wm, wn, lane, acc);
    if (s + 2 >= nst) break;
    pipe_body<TM, BKM, SPLIT>(s + 2, nst, S2, S1, da, db, wave, wm, wn, lane, acc);
    if (s + 3 >= nst) break;
    pipe_body<TM, BKM, SPLIT>(s + 3, nst, S3, S2, da, db, wave, wm, wn, lane, acc);
  }
}

// Bytes of LDS one tile needs: four stage buffers of both operands.
template <int TM>
constexpr int gemm_tile_lds() {
  return 4 * 2 * Geo<TM>::OPB;
}

// Row and column of C held by accumulator element (bi, r, bj) of this lane:
// k-major B interleaves the wave's column blocks.
template <int TM, bool BKM>
__device__ __forceinline__ int gemm_ccol(int n0, int wn, int lane, int bj) {
  return n0 + wn * Geo<TM>::HALF + (BKM ? Geo<TM>::NB * (lane & 31) + bj : 32 * bj + (lane & 31));
}
template <int TM>
__device__ __forceinline__ int gemm_crow(int m0, int wm, int lane, int bi, int r) {
  return m0 + wm * Geo<TM>::HALF + 32 * bi + acc_row(r, lane);
}

// One TM x TM tile (tm, tn) of batch entry z; lds holds gemm_tile_lds<TM>()
// bytes (16-byte aligned).  All 256 threads of the workgroup take part.
// SPLIT (m-major A and n-major B only): the MFMAs run on bf16 matrix cores
// with both operands split three ways (fp32 accuracy, stage_mfma_split).
template <int TM, bool BKM, bool SPLIT = false>
__device__ __forceinline__ void gemm_tile(const GemmF32& g, int tm, int tn, int z, char* lds) {
  static_assert(!SPLIT || !BKM, "split operands need an n-major B");
  using G = Geo<TM>;
  constexpr int NB = G::NB, HALF = G::HALF;
  char* S0 = lds;
  char* S1 = lds + 2 * G::OPB;
  char* S2 = lds + 4 * G::OPB;
  char* S3 = lds + 6 * G::OPB;
  const float* A = g.A + (int64_t)z * g.sA;
  const float* B = g.B + (int64_t)z * g.sB;
  float* C = g.C + (int64_t)z * g.sC;
  const int m0 = tm * TM, n0 = tn * TM;
  if (m0 >= g.M || n0 >= g.N) return;

  int kbeg = 0, kend = g.K;
  if (g.klo_n) kbeg = n0 < g.K ? n0 : g.K;
  if (g.khi_m) kend = (m0 + TM) < g.K ? (m0 + TM) : g.K;
  if (m0 >= g.kfl_lo && m0 < g.kfl_hi) {
    const int f = m0 - g.kfl_lo;
    kbeg = f > kbeg ? (f < kend ? f : kend) : kbeg;
  }

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  f32x16 acc[NB][NB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nst = kend > kbeg ? (kend - kbeg + KS - 1) / KS : 0;
  const bool aligned = ((g.lda & 3) == 0) && ((g.ldb & 3) == 0) &&
                       ((reinterpret_cast<uintptr_t>(A) & 15) == 0) && ((reinterpret_cast<uintptr_t>(B) & 15) == 0);
  const bool whole = aligned && m0 + TM <= g.M && n0 + TM <= g.N && ((kend - kbeg) % KS) == 0;

#define ccol(bj) gemm_ccol<TM, BKM>(n0, wn, lane, bj)
#define crow(bi, r) gemm_crow<TM>(m0, wm, lane, bi, r)

  if (nst > 0 && whole) {
    // C of a whole tile is read ahead of the K loop (older than every direct
    // load, so the counted waits below retire it first)
    float cpre[NB][16][NB];
    if (g.beta) {
#pragma unroll
      for (int bi = 0; bi < NB; ++bi)
#pragma unroll
        for (int r = 0; r < 16; ++r)
#pragma unroll
          for (int bj = 0; bj < NB; ++bj) cpre[bi][r][bj] = C[(int64_t)crow(bi, r) * g.ldc + ccol(bj)];
    }
    DmaOp<TM> da = dma_mmajor<TM>(A, g.lda, m0, kbeg, wave, lane);
    DmaOp<TM> db = BKM ? dma_kmajor<TM>(B, g.ldb, kbeg, n0, wave, lane) : dma_mmajor<TM>(B, g.ldb, n0, kbeg, wave, lane);
    pipeline<TM, BKM, SPLIT>(S0, S1, S2, S3, da, db, nst, wave, wm, wn, lane, acc);
#pragma unroll
    for (int bi = 0; bi < NB; ++bi)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float* p = C + (int64_t)crow(bi, r) * g.ldc + ccol(0);
        float v[NB];
#pragma unroll
        for (int bj = 0; bj < NB; ++bj) v[bj] = g.alpha * acc[bi][bj][r] + (g.beta ? cpre[bi][r][bj] : 0.f);
        if constexpr (BKM && NB == 2) {
          if ((g.ldc & 1) == 0 && (reinterpret_cast<uintptr_t>(C) & 7) == 0) {
            *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
            continue;
          }
        }
#pragma unroll
        for (int bj = 0; bj < NB; ++bj) C[(int64_t)crow(bi, r) * g.ldc + ccol(bj)] = v[bj];
      }
    return;
  }

  if (nst > 0) {
    for (int s = 0; s < nst; ++s) {
      const int k0 = kbeg + s * KS;
      __syncthreads();
      guarded_mmajor<TM>(A, g.lda, m0, g.M, k0, kend, S0);
      if constexpr (BKM)
        guarded_kmajor<TM>(B, g.ldb, k0, kend, n0, g.N, S0 + G::OPB);
      else
        guarded_mmajor<TM>(B, g.ldb, n0, g.N, k0, kend, S0 + G::OPB);
      __syncthreads();
      if constexpr (SPLIT)
        stage_mfma_split<TM>(S0, wm, wn, lane, acc);
      else
        stage_mfma<TM, BKM>(S0, wm, wn, lane, acc);
    }
  }

#pragma unroll
  for (int bi = 0; bi < NB; ++bi)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = crow(bi, r);
      if (m >= g.M) continue;
#pragma unroll
      for (int bj = 0; bj < NB; ++bj) {
        const int n = ccol(bj);
        if (n < g.N) {
          float* p = C + (int64_t)m * g.ldc + n;
          const float v = g.alpha * acc[bi][bj][r];
          *p = g.beta ? (*p + v) : v;
        }
      }
    }
#undef ccol
#undef crow
}

}  // namespace
}  // namespace gptq
