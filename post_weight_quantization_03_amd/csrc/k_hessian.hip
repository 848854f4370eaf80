// Hessian accumulation H += 2 X^T X as a symmetric rank-k update on MFMA.
//
// X is [tokens, n] row-major: both MFMA operands of an output tile H[I, J] are
// column slabs of the same token rows, and the contraction runs over tokens.
// Only upper tiles (I <= J) are computed; each writes its block and the
// mirrored block, so both triangles of H hold bit-identical values.
//
// bf16 path (v_mfma_f32_32x32x16_bf16), 256x256 tiles: four waves in a 2x2
// grid, each owning a 128x128 quarter as 4x4 MFMA blocks whose accumulators
// live in AGPRs.  A stage is 32 tokens of both column slabs.  Global memory is
// copied into LDS by direct loads (global_load_lds, 16 bytes a lane, no
// registers), token-major: a 256-column slab of one token is a 512-byte LDS
// row.  An MFMA operand needs 8 consecutive tokens of one column per lane;
// ds_read_b64_tr_b16 returns exactly that from token-major rows, so the
// transpose happens on the read.  The 16-byte chunks of each row are XOR
// swizzled by the row's low bits so the transposing reads of a 16-lane group
// hit distinct banks.
//
// Four LDS buffers per operand rotate: loads run four stages ahead of the
// MFMAs, and each buffer is read at least one full stage after the barrier
// that retired its loads (reading it in the very stage whose barrier waited on
// the loads was seen to return stale data).  The barrier waits with a counted
// vmcnt so later stages' loads stay in flight.  On diagonal tiles one operand
// is loaded and the wave whose quarter lies below the diagonal skips its
// MFMAs.
//
// fp32 path (v_mfma_f32_32x32x2_f32), 128x128 tiles for fp32 activations: a
// lane supplies one k, so X stays token-major in LDS.
//
// Work items are (tile, token range).  Blocks are dispatched to the 8 XCDs
// round robin, so with S = 8 token splits and split = block % 8 every XCD
// works on its own eighth of the tokens and streams only that part of X
// through its L2.  With one split an item adds 2*acc to H directly.  With S
// splits each item stores its partial tile, and a second kernel sums every
// tile's partials in a fixed order and adds twice the sum to H, so the result
// does not depend on scheduling.  Tiles that would make up a last, mostly
// empty round of an XCD run as shorter token pieces instead, so that round
// keeps every CU busy.
//
// Cross term (CROSS = true): the same kernels compute C += 2 X^T Xq for two
// activation matrices of one shape, the B operand streamed from Xq.  C is not
// symmetric, so every tile of the square grid is computed and written once,
// with no mirror and no diagonal specialisation.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "syrk_plan.h"

namespace gptq {
namespace {

struct SyrkArgs {
  const void* X;
  const void* X2;  // source of the B operand: X for the Hessian, Xq for the cross term
  float* H;
  float* part;     // partial tiles, [slots][tile * tile] (S > 1)
  int64_t ldx;
  int n, tokens;
  int nbt;         // tiles per dimension
  int T;           // upper tiles (Hessian) or all tiles (cross term)
  int S;           // token splits
  int tps;         // tokens per split
  int full;        // tiles computed whole per split; tiles full .. T-1 run in pieces
  int P;           // pieces per split of those tiles
  int tpp;         // tokens per piece
  int h_vec;       // H rows are 16-byte aligned (n % 4 == 0, aligned base)
  int h_vec_x;     // X rows are 16-byte aligned (ldx % 8 == 0, aligned base): direct loads allowed
};

// acc[i][j] is the 32x32 block (i, j) of this wave's (32 WB) x (32 WB) quarter.
// H += 2 acc on the upper triangle, mirrored into the lower one.  The 16 H
// values a lane adds to in one block are loaded together, one block ahead of
// the block being stored: loaded one at a time, each load would wait out a
// full memory round trip before its store (the compiler cannot move a load
// above a store that might alias it), which under the streaming load of the
// other workgroups costs hundreds of microseconds per tile.
template <int TILE, int WB, bool CROSS>
__device__ __forceinline__ void load_block(const SyrkArgs& a, int I, int J, int b, int lane, int wm, int wn,
                                           float (&h)[16]) {
  const int n = a.n;
  const int i = b / WB, j = b % WB;
  const int gc = J * TILE + wn * 32 * WB + 32 * j + acc_col(lane);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int gr = I * TILE + wm * 32 * WB + 32 * i + acc_row(r, lane);
    h[r] = (gr < n && gc < n && (CROSS || gr <= gc)) ? a.H[(int64_t)gr * n + gc] : 0.f;
  }
}

template <int TILE, int WB, bool CROSS>
__device__ __forceinline__ void write_tile(const SyrkArgs& a, int I, int J, f32x16 (&acc)[WB][WB], int lane,
                                           int wm, int wn) {
  const int n = a.n;
  const bool vec_mirror = a.h_vec != 0;
  float hc[16], hn[16];
  load_block<TILE, WB, CROSS>(a, I, J, 0, lane, wm, wn, hc);
#pragma unroll
  for (int b = 0; b < WB * WB; ++b) {
    const int i = b / WB, j = b % WB;
    if (b + 1 < WB * WB) load_block<TILE, WB, CROSS>(a, I, J, b + 1, lane, wm, wn, hn);
    const int gc = J * TILE + wn * 32 * WB + 32 * j + acc_col(lane);
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int gr0 = I * TILE + wm * 32 * WB + 32 * i + acc_row(4 * r4, lane);
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int gr = gr0 + e;
        v[e] = hc[4 * r4 + e] + 2.0f * acc[i][j][4 * r4 + e];
        if (gr < n && gc < n && (CROSS || gr <= gc)) a.H[(int64_t)gr * n + gc] = v[e];
      }
      // mirror: rows gr0..gr0+3 of column gc become four consecutive floats of row gc
      if (!CROSS && gc < n) {
        float* m = a.H + (int64_t)gc * n + gr0;
        if (vec_mirror && gr0 + 3 < gc && gr0 + 3 < n) {
          *reinterpret_cast<float4*>(m) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (gr0 + e < gc && gr0 + e < n) m[e] = v[e];
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) hc[r] = hn[r];
  }
}

// Split tokens: each item stores its partial tile, thread-major (float4 k of
// thread tid at [(k * 256 + tid) * 4]), and k_syrk_reduce sums the partials.
template <int TILE, int WB>
__device__ __forceinline__ void store_partial(const SyrkArgs& a, int slot, f32x16 (&acc)[WB][WB]) {
  constexpr int NV = WB * WB * 4;  // float4s per thread
  float4* mine = reinterpret_cast<float4*>(a.part + (int64_t)slot * TILE * TILE);
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int i = k / (4 * WB), j = (k / 4) % WB, r4 = k % 4;
    mine[k * 256 + threadIdx.x] = make_float4(acc[i][j][4 * r4], acc[i][j][4 * r4 + 1], acc[i][j][4 * r4 + 2],
                                              acc[i][j][4 * r4 + 3]);
  }
}

// H += 2 * (sum of a tile's partials, in slot order), mirrored.  Workgroup
// (tile, k) takes float4 k of every thread of the producing workgroup, so
// thread tid recovers that thread's (wave, lane) and with it the H
// coordinates of the four values, as write_tile does.  Each thread has eight
// partial loads in flight at a time; the whole chip runs the reduction, so it
// is bound by HBM bandwidth rather than by one workgroup's memory latency.
template <int TILE, int WB, bool CROSS>
__global__ __launch_bounds__(256) void k_syrk_reduce(SyrkArgs a) {
  constexpr int PARTIAL4 = TILE * TILE / 4;
  const int tile = blockIdx.x, k = blockIdx.y, tid = threadIdx.x;
  int I, J;
  if constexpr (CROSS) {
    I = tile / a.nbt;
    J = tile % a.nbt;
  } else if constexpr (TILE == 256) {
    decode_offdiag_first(tile, a.nbt, I, J);
  } else {
    decode_upper(tile, a.nbt, I, J);
  }
  const int lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  if (!CROSS && I == J && wm > wn) return;  // quarter below the diagonal: not computed
  const int i = k / (4 * WB), j = (k / 4) % WB, r4 = k % 4;
  int first, count;
  tile_slots(a, tile, first, count);
  const float4* p = reinterpret_cast<const float4*>(a.part) + (int64_t)first * PARTIAL4 + k * 256 + tid;
  float sum[4] = {0.f, 0.f, 0.f, 0.f};
  for (int q0 = 0; q0 < count; q0 += 8) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[(int64_t)min(q0 + u, count - 1) * PARTIAL4];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool ok = q0 + u < count;
      sum[0] += ok ? v[u].x : 0.f;
      sum[1] += ok ? v[u].y : 0.f;
      sum[2] += ok ? v[u].z : 0.f;
      sum[3] += ok ? v[u].w : 0.f;
    }
  }
  const int n = a.n;
  const int gr0 = I * TILE + wm * 32 * WB + 32 * i + acc_row(4 * r4, lane);
  const int gc = J * TILE + wn * 32 * WB + 32 * j + acc_col(lane);
  float h[4], v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int gr = gr0 + e;
    h[e] = (gr < n && gc < n && (CROSS || gr <= gc)) ? a.H[(int64_t)gr * n + gc] : 0.f;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int gr = gr0 + e;
    v[e] = h[e] + 2.0f * sum[e];
    if (gr < n && gc < n && (CROSS || gr <= gc)) a.H[(int64_t)gr * n + gc] = v[e];
  }
  if (!CROSS && gc < n) {
    float* m = a.H + (int64_t)gc * n + gr0;
    if (a.h_vec && gr0 + 3 < gc && gr0 + 3 < n) {
      *reinterpret_cast<float4*>(m) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (gr0 + e < gc && gr0 + e < n) m[e] = v[e];
    }
  }
}

// ------------------------------------------------------------------ bf16 path

constexpr int ROWB = TB * 2;        // bytes per token row of one operand stage (no padding)
constexpr int STAGEB = KB * ROWB;   // 16 KB per operand stage

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Byte offset of element (row = token, col) in a stage buffer.  The 16-byte
// chunk index is XORed with 4 * (row & 3), so the transposing operand reads
// (4 consecutive rows x 4 chunks per 32 lanes) hit 16 distinct bank groups.
__device__ __forceinline__ int sw_off(int row, int col) {
  const int phys = (col >> 3) ^ ((row & 3) << 2);
  return row * ROWB + (phys << 4) + ((col & 7) << 1);
}

// Fast path: the whole stage lies inside X.  Each wave copies 8 token rows
// with 4 direct global->LDS loads of 16 bytes per lane (2 rows per load; lane
// p lands at chunk position p & 31 and fetches the chunk that the swizzle
// places there).  The address is a wave-uniform base (first token of the
// stage, first column of the slab; kept in SGPRs and advanced one stage per
// call) plus a per-lane 32-bit byte offset that is the same for every stage.
struct DirectSrc {
  const char* base;
  uint32_t off[4];
};

__device__ __forceinline__ DirectSrc direct_src(const SyrkArgs& a, const uint16_t* X, int col0, int t, int wave,
                                                int lane) {
  DirectSrc d;
  d.base = reinterpret_cast<const char*>(X + (int64_t)t * a.ldx + col0);
  const int pos = lane & 31;
#pragma unroll
  for (int i = 0; i < KB / 8; ++i) {
    const int row = (KB / 4) * wave + 2 * i + (lane >> 5);
    const int gchunk = pos ^ ((row & 3) << 2);
    d.off[i] = (uint32_t)(((int64_t)row * a.ldx + 8 * gchunk) * 2);
  }
  return d;
}

// ASM: the load is issued from inline asm, invisible to the compiler's wait
// insertion.  Only the whole-tile kernel does so: there every wait on these
// loads is an explicit counted s_waitcnt, and without alias information the
// compiler would otherwise drain all of them (vmcnt(0)) at the loop's back
// edge before the first LDS read.
typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ void dma_piece(const DirectSrc& d, char* buf, int wave, int i) {
  const int r0 = (KB / 4) * wave + 2 * i;
  const uint32_t lds = (uint32_t)(uintptr_t)(lds_char*)(buf + r0 * ROWB);
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(d.off[i]), "s"(d.base), "{m0}"(lds));
}
__device__ __forceinline__ void dma_advance(DirectSrc& d, int64_t stage_step) {
  uint64_t b = reinterpret_cast<uint64_t>(d.base) + (uint64_t)(stage_step * 2);
  asm volatile("" : "+s"(b));
  d.base = reinterpret_cast<const char*>(b);
}

template <bool ASM>
__device__ __forceinline__ void stage_direct(DirectSrc& d, char* buf, int wave, int64_t stage_step) {
#pragma unroll
  for (int i = 0; i < KB / 8; ++i) {
    const int r0 = (KB / 4) * wave + 2 * i;
    if constexpr (ASM) {
      const uint32_t lds = (uint32_t)(uintptr_t)(lds_char*)(buf + r0 * ROWB);
      asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(d.off[i]), "s"(d.base), "{m0}"(lds));
    } else {
      __builtin_amdgcn_global_load_lds(d.base + d.off[i], (lds_void*)(buf + r0 * ROWB), 16, 0, 0);
    }
  }
  // The empty asm hides the stage-to-stage relation of the base from loop
  // strength reduction, which would otherwise keep one 64-bit VGPR address
  // per load and unrolled stage (and spill them).
  uint64_t b = reinterpret_cast<uint64_t>(d.base) + (uint64_t)(stage_step * 2);
  asm volatile("" : "+s"(b));
  d.base = reinterpret_cast<const char*>(b);
}

// Guarded path for ragged stages or tiles: zero-filled register loads and
// 16-byte LDS stores into the same swizzled layout.
__device__ __forceinline__ void stage_guarded(const SyrkArgs& a, const uint16_t* X, int col0, int t, int t1,
                                              char* buf) {
#pragma unroll
  for (int i = 0; i < KB / 8; ++i) {
    const int idx = threadIdx.x + 256 * i;
    const int row = idx >> 5, c = idx & 31;
    const int tok = t + row, col = col0 + 8 * c;
    const uint16_t* p = X + (int64_t)tok * a.ldx + col;
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t lo = (tok < t1 && col + 2 * k < a.n) ? p[2 * k] : 0u;
      const uint32_t hi = (tok < t1 && col + 2 * k + 1 < a.n) ? p[2 * k + 1] : 0u;
      w[k] = lo | (hi << 16);
    }
    *reinterpret_cast<uint4*>(buf + sw_off(row, 8 * c)) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// MFMA operand of the 32-column block at m0 for tokens 16kk .. 16kk+15.  In a
// 16-lane group, source lane s points at 4 columns (m0 + 16(g&1) + 4(s&3)) of
// token row 16kk + 8(g>>1) + s/4; the transposing read hands lane l of the
// group 4 consecutive tokens of column m0 + 16(g&1) + l.  Two reads (rows +0
// and +4) give the 8 tokens a lane supplies to v_mfma_f32_32x32x16_bf16.
// Rows +4 and +16kk keep row & 3, hence the swizzle: both are fixed byte
// offsets from the kk = 0 address, which is computed once per block.
__device__ __forceinline__ int frag_off(int m0, int lane) {
  const int g = lane >> 4, s = lane & 15;
  return sw_off(8 * (g >> 1) + (s >> 2), m0 + 16 * (g & 1) + 4 * (s & 3));
}

__device__ __forceinline__ bf16x8 frag_at(const char* p) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * ROWB));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

struct StageFrags {
  bf16x8 a[KB / 16][4], b[KB / 16][4];
};

__device__ __forceinline__ void read_frags(const char* Ab, const char* Bb, const int (&offA)[4],
                                           const int (&offB)[4], StageFrags& f) {
#pragma unroll
  for (int kk = 0; kk < KB / 16; ++kk) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f.a[kk][i] = frag_at(Ab + offA[i] + kk * 16 * ROWB);
#pragma unroll
    for (int j = 0; j < 4; ++j) f.b[kk][j] = frag_at(Bb + offB[j] + kk * 16 * ROWB);
  }
}

__device__ __forceinline__ void mfma_frags(const StageFrags& f, f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int kk = 0; kk < KB / 16; ++kk)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[kk][i], f.b[kk][j], acc[i][j], 0, 0, 0);
}

// FULL: every tile is inside X and every stage holds 32 tokens (n % 256 == 0,
// tokens % 32 == 0, 16-byte aligned rows), so only direct loads are compiled.
//
// Pipeline (stage s lives in buffer s % 4; fragments alternate between two
// register sets):
//   wait + barrier   -- FULL: a counted vmcnt retires this wave's loads of stage
//                       s+2 and leaves those of stage s+3 in flight; otherwise
//                       a plain __syncthreads()
//   read stage s+1 fragments into the other register set (in flight during
//                       this stage's MFMAs)
//   queue stage s+4 loads into the buffer stage s used
//   32 MFMAs on stage s
// Loads are queued four stages ahead and retired two stages later (two
// stages of latency slack), and a buffer is read one full stage after the
// barrier that retired its loads (reading a buffer straight after that
// barrier returned stale data on this hardware).  The buffers are distinct
// LDS objects, so fragment reads never wait for loads into another buffer.
template <bool FULL, bool CROSS>
__global__ __launch_bounds__(256, 1) void k_syrk_bf16(SyrkArgs a) {
  __shared__ __attribute__((aligned(16))) char B0[2 * STAGEB];
  __shared__ __attribute__((aligned(16))) char B1[2 * STAGEB];
  __shared__ __attribute__((aligned(16))) char B2[2 * STAGEB];
  __shared__ __attribute__((aligned(16))) char B3[2 * STAGEB];

  const SyrkItem it = decode_item(a, blockIdx.x);
  int I, J;
  if constexpr (CROSS) {
    if (a.S == 1) {
      decode_square_supertiles(blockIdx.x, a.nbt, a.T, I, J);
    } else {
      I = it.tile / a.nbt;
      J = it.tile % a.nbt;
    }
  } else {
    if (a.S == 1)
      decode_supertiles(blockIdx.x, a.nbt, a.T, I, J);
    else
      decode_offdiag_first(it.tile, a.nbt, I, J);
  }
  const bool diag = !CROSS && (I == J);
  const int t0 = it.t0, t1 = it.t1;
  const int nst = t1 > t0 ? (t1 - t0 + KB - 1) / KB : 0;

  // wave index through readfirstlane: provably uniform, so per-wave branches
  // and the values they define stay scalar
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const bool idle = diag && wm > wn;  // quarter strictly below the diagonal
  const uint16_t* X = static_cast<const uint16_t*>(a.X);
  const uint16_t* X2 = static_cast<const uint16_t*>(a.X2);
  const int colA = I * TB, colB = J * TB;
  const bool fullA = a.h_vec_x && colA + TB <= a.n;
  const bool fullB = a.h_vec_x && colB + TB <= a.n;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  int offA[4], offB[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    offA[i] = frag_off(wm * 128 + 32 * i, lane);
    offB[i] = frag_off(wn * 128 + 32 * i, lane);
  }
  const int64_t stage_step = (int64_t)KB * a.ldx;
  DirectSrc dA = direct_src(a, X, colA, t0, wave, lane);
  DirectSrc dB = direct_src(a, X2, colB, t0, wave, lane);

  // stages are issued in order, so the direct sources simply advance
  auto issue = [&](int st, char* buf) {
    const int t = t0 + st * KB;
    if constexpr (FULL) {
      stage_direct<true>(dA, buf, wave, stage_step);
      if (!diag) stage_direct<true>(dB, buf + STAGEB, wave, stage_step);
      return;
    }
    const bool full_t = t + KB <= t1;
    if (full_t && fullA)
      stage_direct<false>(dA, buf, wave, stage_step);
    else
      stage_guarded(a, X, colA, t, t1, buf);
    if (!diag) {
      if (full_t && fullB)
        stage_direct<false>(dB, buf + STAGEB, wave, stage_step);
      else
        stage_guarded(a, X2, colB, t, t1, buf + STAGEB);
    }
  };
  auto rd = [&](const char* buf, StageFrags& f) {
    if (!idle) read_frags(buf, diag ? buf : buf + STAGEB, offA, offB, f);
  };
  // Barrier at the start of stage st.  FULL: each wave queued 4 (diagonal
  // tile) or 8 direct loads per stage; leaving the newest stage's loads
  // (st+3) outstanding retires stage st+2's.  The asm carries a memory clobber
  // so no LDS access moves across it.
  auto barrier = [&](int st) {
    if constexpr (FULL) {
      if (st + 3 >= nst)
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      else if (diag)
        asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    } else {
      __syncthreads();
    }
  };
  // stage st: fragments fc (stage st) are in registers; read stage st+1 from
  // `nxt` into fn; queue stage st+4 into `dma` (stage st's buffer).
  auto stage = [&](int st, const char* nxt, char* dma, StageFrags& fc, StageFrags& fn) {
    barrier(st);
    if (st + 1 < nst) rd(nxt, fn);
    if (st + 4 < nst) issue(st + 4, dma);
    if (!idle) mfma_frags(fc, acc);
  };
  // Steady state of the FULL kernel: every stage reads its successor and
  // queues stage +4, so the body has no branch and the scheduler may
  // interleave the 32 transposing reads and the direct loads with the 32
  // MFMAs (left in separate blocks, the reads stall the wave on the LDS
  // queue before its MFMAs start).  TWO: off-diagonal tile (both operands);
  // COMP: this wave reads fragments and runs MFMAs.
  auto steady = [&](auto two_c, auto comp_c, StageFrags& f0, StageFrags& f1) {
    constexpr bool TWO = decltype(two_c)::value, COMP = decltype(comp_c)::value;
    auto body = [&](const char* nxt, char* dma, StageFrags& fc, StageFrags& fn) {
      if constexpr (TWO)
        asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if constexpr (COMP) {
        // direct loads spread over the stage: one before every two fragments
        const char* Ab = nxt;
        const char* Bb = TWO ? nxt + STAGEB : nxt;
#pragma unroll
        for (int kk = 0; kk < KB / 16; ++kk)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int g = 4 * kk + i;  // 0..7
            if constexpr (TWO) {
              if (g < 4) dma_piece(dA, dma, wave, g); else dma_piece(dB, dma + STAGEB, wave, g - 4);
            } else {
              if ((g & 1) == 0) dma_piece(dA, dma, wave, g >> 1);
            }
            fn.a[kk][i] = frag_at(Ab + offA[i] + kk * 16 * ROWB);
            fn.b[kk][i] = frag_at(Bb + offB[i] + kk * 16 * ROWB);
          }
        dma_advance(dA, stage_step);
        if constexpr (TWO) dma_advance(dB, stage_step);
        mfma_frags(fc, acc);
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        }
      } else {
        stage_direct<true>(dA, dma, wave, stage_step);
        if constexpr (TWO) stage_direct<true>(dB, dma + STAGEB, wave, stage_step);
      }
    };
    int st = 0;
    for (; st + 8 <= nst; st += 4) {
      body(B1, B0, f0, f1);
      body(B2, B1, f1, f0);
      body(B3, B2, f0, f1);
      body(B0, B3, f1, f0);
    }
    return st;
  };

  if (nst > 0) {
    StageFrags f0, f1;
    // stages 0 and 1 retire first; retiring stage 2 (counted, if stage 3 was
    // queued) gives them a full load latency before stage 0 is read
    issue(0, B0);
    if (nst > 1) issue(1, B1);
    __syncthreads();
    if (nst > 2) issue(2, B2);
    if (nst > 3) issue(3, B3);
    barrier(-1);
    rd(B0, f0);
    int st0 = 0;
    if constexpr (FULL) {
      using yes = std::true_type;
      using no = std::false_type;
      if (!diag)
        st0 = steady(yes{}, yes{}, f0, f1);
      else if (!idle)
        st0 = steady(no{}, yes{}, f0, f1);
      else
        st0 = steady(no{}, no{}, f0, f1);
    }
    // the last stages (and every stage of a guarded tile), fragments of
    // stage st0 in f0
    for (int st = st0; st < nst; st += 4) {
      stage(st + 0, B1, B0, f0, f1);
      if (st + 1 >= nst) break;
      stage(st + 1, B2, B1, f1, f0);
      if (st + 2 >= nst) break;
      stage(st + 2, B3, B2, f0, f1);
      if (st + 3 >= nst) break;
      stage(st + 3, B0, B3, f1, f0);
    }
  }

  if (a.S > 1)
    store_partial<TB, 4>(a, it.slot, acc);
  else if (!idle)
    write_tile<TB, 4, CROSS>(a, I, J, acc, lane, wm, wn);
}

// ------------------------------------------------------------------ fp32 path

constexpr int F32_PITCH = TF + 4;

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

template <bool VEC, bool CROSS>
__global__ __launch_bounds__(256) void k_syrk_f32(SyrkArgs a) {
  __shared__ __attribute__((aligned(16))) float As[2][KT_F32][F32_PITCH];
  __shared__ __attribute__((aligned(16))) float Bs[2][KT_F32][F32_PITCH];

  const SyrkItem it = decode_item(a, blockIdx.x);
  int I, J;
  if constexpr (CROSS) {
    I = it.tile / a.nbt;
    J = it.tile % a.nbt;
  } else {
    decode_upper(it.tile, a.nbt, I, J);
  }
  const bool diag = !CROSS && (I == J);
  const int t0 = it.t0, t1 = it.t1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const float* X = static_cast<const float*>(a.X);
  const float* X2 = static_cast<const float*>(a.X2);

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  if (t0 < t1) {
    float4 va[2], vb[2];
    load_f32<VEC>(a, X, I * TF, t0, t1, va);
    if (!diag) load_f32<VEC>(a, X2, J * TF, t0, t1, vb);
    store_f32(As[0], va);
    if (!diag) store_f32(Bs[0], vb);
    __syncthreads();
    int buf = 0;
    for (int t = t0; t < t1; t += KT_F32) {
      const bool more = t + KT_F32 < t1;
      if (more) {
        load_f32<VEC>(a, X, I * TF, t + KT_F32, t1, va);
        if (!diag) load_f32<VEC>(a, X2, J * TF, t + KT_F32, t1, vb);
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

  if (a.S > 1)
    store_partial<TF, 2>(a, it.slot, acc);
  else
    write_tile<TF, 2, CROSS>(a, I, J, acc, lane, wm, wn);
}

int cu_count() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                               hipSuccess || cus <= 0)
    return 256;
  return cus;
}

SyrkPlan plan(int64_t n, int64_t tokens, gptq_dtype dt, bool cross = false) {
  return syrk_plan(n, tokens, dt == GPTQ_BF16, cross, cu_count());
}

}  // namespace

namespace {

size_t syrk_workspace(int64_t n, int64_t tokens, gptq_dtype dt, bool cross) {
  if (n <= 0 || tokens <= 0) return 0;
  const SyrkPlan p = plan(n, tokens, dt, cross);
  if (p.S == 1) return 0;
  return align_up((size_t)p.slots * p.tile * p.tile * sizeof(float), 256);
}

template <bool CROSS>
int syrk_launch(float* H, int64_t n, const void* X, const void* X2, gptq_dtype dt, int64_t tokens, int64_t ldx,
                void* ws, size_t ws_bytes, hipStream_t stream) {
  const SyrkPlan p = plan(n, tokens, dt, CROSS);
  SyrkArgs a{};
  a.X = X;
  a.X2 = X2;
  a.H = H;
  a.ldx = ldx;
  a.n = (int)n;
  a.tokens = (int)tokens;
  a.nbt = p.nbt;
  a.T = p.T;
  a.S = p.S;
  a.tps = p.tps;
  a.full = p.full;
  a.P = p.P;
  a.tpp = p.tpp;
  a.h_vec = (n % 4 == 0) && ((reinterpret_cast<uintptr_t>(H) & 15) == 0);
  if (p.S > 1) {
    if (ws_bytes < syrk_workspace(n, tokens, dt, CROSS) || ws == nullptr) return GPTQ_EWORKSPACE;
    a.part = static_cast<float*>(ws);
  }
  const int64_t items = ((int64_t)p.full + (int64_t)(p.T - p.full) * p.P) * p.S;
  if (items > INT32_MAX) return GPTQ_EUNSUPPORTED;
  const dim3 grid((unsigned)items);
  const auto aligned16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
  if (dt == GPTQ_BF16) {
    a.h_vec_x = (ldx % 8 == 0) && aligned16(X) && aligned16(X2);
    if (a.h_vec_x && n % TB == 0 && tokens % KB == 0)
      hipLaunchKernelGGL((k_syrk_bf16<true, CROSS>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((k_syrk_bf16<false, CROSS>), grid, dim3(256), 0, stream, a);
    if (p.S > 1) hipLaunchKernelGGL((k_syrk_reduce<TB, 4, CROSS>), dim3(p.T, 64), dim3(256), 0, stream, a);
  } else {
    const bool vec = (ldx % 4 == 0) && aligned16(X) && aligned16(X2);
    if (vec)
      hipLaunchKernelGGL((k_syrk_f32<true, CROSS>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((k_syrk_f32<false, CROSS>), grid, dim3(256), 0, stream, a);
    if (p.S > 1) hipLaunchKernelGGL((k_syrk_reduce<TF, 2, CROSS>), dim3(p.T, 16), dim3(256), 0, stream, a);
  }
  return hipGetLastError() == hipSuccess ? GPTQ_OK : GPTQ_EHIP;
}

}  // namespace

size_t hessian_workspace(int64_t n, int64_t tokens, gptq_dtype dt) { return syrk_workspace(n, tokens, dt, false); }

int hessian_launch(float* H, int64_t n, const void* X, gptq_dtype dt, int64_t tokens, int64_t ldx, void* ws,
                   size_t ws_bytes, hipStream_t stream) {
  return syrk_launch<false>(H, n, X, X, dt, tokens, ldx, ws, ws_bytes, stream);
}

size_t cross_workspace(int64_t n, int64_t tokens, gptq_dtype dt) { return syrk_workspace(n, tokens, dt, true); }

int cross_launch(float* C, int64_t n, const void* X, const void* Xq, gptq_dtype dt, int64_t tokens, int64_t ldx,
                 void* ws, size_t ws_bytes, hipStream_t stream) {
  return syrk_launch<true>(C, n, X, Xq, dt, tokens, ldx, ws, ws_bytes, stream);
}

}  // namespace gptq
