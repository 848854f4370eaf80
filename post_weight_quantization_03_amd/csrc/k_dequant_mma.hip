// Y[t, :] = W^ X[t, :] for a batch of activation vectors on the bf16 matrix
// cores, straight from the quantizer's outputs (packed b-bit codes, fp32 group
// scales, integer group zeros; w^ = s_g (q - z_g)).
//
// The product is Y^T = X W^T with v_mfma_f32_16x16x32_bf16: the A operand is
// the activations (16 rows: vectors, or the bf16 parts of fp32 vectors), the B
// operand 16 weight rows, and the output lane (a, j) = (l / 16, l % 16) holds
// x-rows 4a .. 4a+3 of weight row j.  Both operands are exact in bf16:
//   - a code q < 2^8 is an exact bf16 integer (2- and 4-bit codes are read as
//     fp8 e4m3 bytes, exactly q 2^-9, and converted with the scale 2^9);
//   - a bf16 x is itself; an fp32 x is the exact sum of three bf16 parts
//     hi + mid + lo (each the round-to-nearest bf16 of what the parts before it
//     leave), so the matrix core forms exact products q x_part and only the
//     fp32 accumulation rounds.
// Zero point and scale are applied per 128-column chunk, which lies in one
// group when the group size is a multiple of 128 (or the row is one group):
//   y += s_g (sum_chunk q x - z_g sum_chunk x).
//
// Work split: a work item is 128 weight rows (4 waves of two 16-row tiles) by
// a slice of 2, 4 or 8 chunks; the slice count is chosen to fill the chip, and
// items go to the XCDs in contiguous ranges.  A workgroup loads its whole slice
// at once (x from the last-level cache, the rows' scales and zeros, every code
// run), splits the x into parts laid out as MFMA operand fragments in LDS while
// the codes are in flight (so each fragment is one conflict-free 16-byte read
// per lane), and applies the chunks as their loads retire.  A lane's B operand
// for chunk c is run l / 16 (32 codes) of its weight row; MFMA m of the chunk
// takes codes 8m .. 8m+7 of every lane's run, so the four k-slots of one MFMA
// are four runs of one chunk.  Slices write fixed-order partial sums to the
// workspace and a second kernel adds them in slice order; with one slice the
// kernel writes Y.
// Everything is fp32 in a fixed order, so results are reproducible.
#include <type_traits>

#include "common.h"

namespace gptq {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4a __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2a __attribute__((ext_vector_type(2), aligned(4)));
typedef float f32x4a __attribute__((ext_vector_type(4), aligned(4)));
typedef uint16_t u16x4a __attribute__((ext_vector_type(4), aligned(4)));

constexpr int MM_NW = 4;                     // waves per workgroup
constexpr int MM_RT = 2;                     // 16-row tiles per wave
constexpr int MM_ROWS = 16 * MM_RT * MM_NW;  // weight rows per workgroup
constexpr int MM_MAXT = 16;                  // vectors per launch
constexpr int MM_TARGET_WG = 512;            // workgroups the slice count aims for

// Code position of each of the 8 operand slots of an MFMA k-slot, by code width
// (the order the conversions below produce).
__device__ __forceinline__ int slot_code(int bits, int e) {
  if (bits == 4) return (e & 3) * 2 + (e >> 2);  // 0 2 4 6 1 3 5 7
  if (bits == 2) return (e >> 1) + 4 * (e & 1);  // 0 4 1 5 2 6 3 7
  return e;
}

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Codes 8m .. 8m+7 of a run (BITS words) as exact bf16 values, in slot order.
template <int BITS, int M>
__device__ __forceinline__ bf16x8 run_frag(const uint32_t (&w)[BITS]) {
  uint32_t o[4];
  if constexpr (BITS == 4) {
    const uint32_t lo = w[M] & 0x0f0f0f0fu, hi = (w[M] >> 4) & 0x0f0f0f0fu;
    o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 512.0f, false));
    o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 512.0f, true));
    o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 512.0f, false));
    o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 512.0f, true));
  } else if constexpr (BITS == 2) {
    // byte b of mask t holds code 4b + t of the word; the low half of the word
    // (codes 0..7) is bytes 0, 1, the high half bytes 2, 3
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t c = (w[M >> 1] >> (2 * t)) & 0x03030303u;
      o[t] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, 512.0f, (M & 1) != 0));
    }
  } else if constexpr (BITS == 8) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t v = w[2 * M + h];
      o[2 * h] = pack2((float)(v & 0xffu), (float)((v >> 8) & 0xffu));
      o[2 * h + 1] = pack2((float)((v >> 16) & 0xffu), (float)(v >> 24));
    }
  } else {
    // 3 bits: codes 8m .. 8m+7 are stream bits [24m, 24m + 24) of the run
    uint32_t f;
    if constexpr (M == 0) f = w[0];
    else if constexpr (M == 1) f = __builtin_amdgcn_alignbit(w[1], w[0], 24);
    else if constexpr (M == 2) f = __builtin_amdgcn_alignbit(w[2], w[1], 16);
    else f = w[2] >> 8;
#pragma unroll
    for (int h = 0; h < 4; ++h)
      o[h] = pack2((float)((f >> (6 * h)) & 7u), (float)((f >> (6 * h + 3)) & 7u));
  }
  const u32x4a v = {o[0], o[1], o[2], o[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// x = hi + mid + lo exactly (normal range): each part the nearest bf16 to
// what the parts before it leave.
__device__ __forceinline__ void split3(float x, float& hi, float& mid, float& lo) {
  hi = (float)(__bf16)x;
  const float r1 = x - hi;
  mid = (float)(__bf16)r1;
  lo = r1 - mid;  // exactly a bf16 value
}

// Barrier for LDS traffic only: this wave's LDS operations are done, then every
// wave meets; the code loads in flight stay in flight.  (The memory clobber keeps
// the compiler from moving LDS accesses across it.)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Slot of the 16-byte fragment piece of k-slot s and A row i within its 1 KB
// block (MFMA step m): the piece index 16 s + i with its low three bits XOR
// (m + 4 (s & 1)).  A wave's reads (lane l = 16 s + i) stay a permutation of
// each 8-lane group; the staging stores, whose 8 consecutive lanes hold the 8
// (s, m) pairs of one A row, land on 8 different banks instead of one.
__device__ __forceinline__ int frag_slot(int s, int i, int m) { return (16 * s + i) ^ ((m + 4 * (s & 1)) & 7); }

// Template: BITS code width, NM operand planes (x rows per MFMA chain), WHOLE
// (cols % 32 == 0: every run has whole words), XT float or uint16_t (bf16),
// CPS chunks per column slice, GPT staging groups per thread (T CPS 16 / 256
// rounded up).  Runtime layout of the A rows: vector t's part p is plane p / rp,
// row t + rs (p % rp); parts are 3 for fp32 x, 1 for bf16.  Vector t's
// zero-point sum goes to row t.
//
// A workgroup's slice is loaded in one go: first the slice's x (from the
// last-level cache), then every code run, scale and zero of the slice (512
// contiguous bytes a row at 4 bits and 8 chunks), so the x can be split and
// stored while the codes are in flight (loads retire in issue order: waiting
// for x waits for nothing queued after it).  One barrier, then the chunks are
// applied in order as their loads retire.
template <int BITS, int NM, bool WHOLE, typename XT, int CPS, int GPT>
__global__ __launch_bounds__(64 * MM_NW) void k_dequant_mma(
    const uint32_t* __restrict__ packed, const float* __restrict__ scales, const uint8_t* __restrict__ zeros,
    int64_t rows, int64_t cols, int64_t G, int64_t gchunks, const XT* __restrict__ X, int64_t ldx, int T, int rs,
    int rp, int64_t ks, float* __restrict__ out, int64_t ldo, int64_t slice_stride) {
  constexpr int NP = std::is_same<XT, float>::value ? 3 : 1;  // parts per x value
  constexpr int FRAG_BYTES = CPS * 4 * NM * 1024;                // [chunk][m][plane] x 64 lanes x 16 B
  constexpr int SX_BYTES = CPS * 16 * 4;                         // then the chunks' x sums per A row
  constexpr int SZ_BYTES = 2 * MM_ROWS * CPS * 4;                // then the rows' scales and zeros
  constexpr int LDS_BYTES = FRAG_BYTES + SX_BYTES + SZ_BYTES;
  static_assert(FRAG_BYTES >= MM_NW * MM_RT * 16 * 16 * 4, "the row combine reuses the fragments' LDS");
  static_assert(GPT * 64 * MM_NW >= CPS * 16, "");
  __shared__ __align__(16) char lds[LDS_BYTES];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int a = lane >> 4, j = lane & 15;
  const int64_t wpr = cols * BITS / 32;  // words per row
  const int64_t nrun = (cols + 31) / 32;
  const int64_t nch = (cols + 127) / 128;
  // Work item = (row block, slice), slices fastest.  Workgroups go to the 8 XCDs
  // in turn, so each XCD takes a contiguous range of items: the slices of a row
  // block share their scale and zero lines in one L2, and the items running
  // together read whole contiguous blocks of rows.
  const int64_t nwg = gridDim.x, per = nwg / 8, rem = nwg % 8;
  const int64_t xcd = blockIdx.x % 8, k = blockIdx.x / 8;
  const int64_t item = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + k;
  const int64_t slice = item % ks, rblock = item / ks;
  const int64_t c_begin = slice * CPS;
  const int64_t r0 = rblock * MM_ROWS + (int64_t)wave * 16 * MM_RT;
  float* sx = reinterpret_cast<float*>(lds + FRAG_BYTES);
  float* sgl = reinterpret_cast<float*>(lds + FRAG_BYTES + SX_BYTES);  // [row][group] scales
  float* zgl = sgl + MM_ROWS * CPS;                                     // [row][group] zero points
  GPTQ_TRACE_DECL;
  GPTQ_TRACE_STAMP();

  // 1. The slice's x: 8-column groups g = (t, chunk, h), h = 4 s + m: columns
  // 32 s + 8 m .. +7 of the chunk, k-slot s of MFMA m.
  const int ngroups = T * CPS * 16;
  using XR = typename std::conditional<std::is_same<XT, float>::value, f32x4a, u16x4a>::type;
  XR xr[GPT][2];
#pragma unroll
  for (int it = 0; it < GPT; ++it) {
    const int g = threadIdx.x + 64 * MM_NW * it;
    const int t = g / (CPS * 16), cc = (g / 16) % CPS, h = g & 15;
    const int64_t col = (c_begin + cc) * 128 + 8 * h;
    const XT* xp = X + (int64_t)(t < T ? t : 0) * ldx;
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      // cols is a multiple of 4: each 4-vector is all in or all out; out reloads the
      // last one and is zeroed when stored
      const int64_t c = col + 4 * v;
      xr[it][v] = *reinterpret_cast<const XR*>(xp + (c + 4 <= cols ? c : cols - 4));
    }
  }

  GPTQ_TRACE_STAMP();
  // 2. The scales and zero points of the workgroup's rows for the CPS groups
  // from the slice's first (clamped to the row's last group): the groups of its
  // chunks lie among them.  Coalesced (a row's groups are contiguous), staged
  // through LDS below.
  const int64_t gk0 = (int64_t)((uint32_t)c_begin / (uint32_t)gchunks);
  const int64_t rb0 = rblock * MM_ROWS;
  constexpr int SZT = (MM_ROWS * CPS + 64 * MM_NW - 1) / (64 * MM_NW);  // per thread
  float sreg[SZT];
  uint32_t zreg[SZT];
#pragma unroll
  for (int q = 0; q < SZT; ++q) {
    const int e = threadIdx.x + 64 * MM_NW * q;
    const int64_t row = rb0 + e / CPS, gk = gk0 + e % CPS;
    const int64_t rc = row < rows ? row : rows - 1;
    const int64_t off = rc * G + (gk < G ? gk : G - 1);
    sreg[q] = scales[off];
    zreg[q] = zeros[off];
  }

  // 3. Every code run of the slice, chunk by chunk.  No branch: a chunk past the
  // row's end reloads its last run (x is 0 there), so the compiler's waits count
  // these loads exactly.
  const uint32_t* prow[MM_RT];
#pragma unroll
  for (int r = 0; r < MM_RT; ++r) {
    const int64_t row = r0 + 16 * r + j < rows ? r0 + 16 * r + j : rows - 1;  // past the end: unwritten
    prow[r] = packed + row * wpr;
  }
  uint32_t w[CPS][MM_RT][BITS];
#pragma unroll
  for (int cc = 0; cc < CPS; ++cc) {
    const int64_t ch = c_begin + cc < nch ? c_begin + cc : nch - 1;
    const int64_t run = ch * 4 + a;
#pragma unroll
    for (int r = 0; r < MM_RT; ++r) {
      if constexpr (WHOLE) {
        const int64_t rc = run < nrun ? run : nrun - 1;
        const uint32_t* p = prow[r] + rc * BITS;
        if constexpr (BITS == 2) {
          const u32x2a v = *reinterpret_cast<const u32x2a*>(p);
          w[cc][r][0] = v.x; w[cc][r][1] = v.y;
        } else if constexpr (BITS == 3) {
          w[cc][r][0] = p[0]; w[cc][r][1] = p[1]; w[cc][r][2] = p[2];
        } else {
#pragma unroll
          for (int q = 0; q < BITS; q += 4) {
            const u32x4a v = *reinterpret_cast<const u32x4a*>(p + q);
            w[cc][r][q] = v.x; w[cc][r][q + 1] = v.y; w[cc][r][q + 2] = v.z; w[cc][r][q + 3] = v.w;
          }
        }
      } else {
        // the partial last run has (cols - 32 run) b / 32 whole words; words past the
        // row read as 0 (x is 0 there), loaded from the row's last word
#pragma unroll
        for (int q = 0; q < BITS; ++q) {
          const int64_t wi = run * BITS + q;
          const uint32_t v = prow[r][wi < wpr ? wi : wpr - 1];
          w[cc][r][q] = wi < wpr ? v : 0u;
        }
      }
    }
  }

  GPTQ_TRACE_STAMP();
  // 4. Zero the fragments (rows no part occupies stay zero), then store the
  // slice's x split into parts, in operand order, with each chunk's sums, and
  // the scales and zero points.
  for (int i = threadIdx.x; i < LDS_BYTES / 16; i += 64 * MM_NW)
    reinterpret_cast<f32x4*>(lds)[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  lds_barrier();
  GPTQ_TRACE_STAMP();
#pragma unroll
  for (int q = 0; q < SZT; ++q) {
    const int e = threadIdx.x + 64 * MM_NW * q;
    if (e < MM_ROWS * CPS) {
      sgl[e] = sreg[q];
      zgl[e] = (float)zreg[q];
    }
  }
#pragma unroll
  for (int it = 0; it < GPT; ++it) {
    const int g = threadIdx.x + 64 * MM_NW * it;
    const int t = g / (CPS * 16), cc = (g / 16) % CPS, h = g & 15;
    const int s = h >> 2, m = h & 3;
    const int64_t col = (c_begin + cc) * 128 + 8 * h;
    float x[8];
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      f32x4 f;
      if constexpr (std::is_same<XT, float>::value)
        f = f32x4{xr[it][v].x, xr[it][v].y, xr[it][v].z, xr[it][v].w};
      else
        f = f32x4{__uint_as_float((uint32_t)xr[it][v].x << 16), __uint_as_float((uint32_t)xr[it][v].y << 16),
                  __uint_as_float((uint32_t)xr[it][v].z << 16), __uint_as_float((uint32_t)xr[it][v].w << 16)};
      const bool in = g < ngroups && col + 4 * v < cols;
      x[4 * v] = in ? f.x : 0.0f;
      x[4 * v + 1] = in ? f.y : 0.0f;
      x[4 * v + 2] = in ? f.z : 0.0f;
      x[4 * v + 3] = in ? f.w : 0.0f;
    }
    // the chunk's sum of x for vector t, over its 16 groups in 16 consecutive lanes
    float sm = ((x[0] + x[1]) + (x[2] + x[3])) + ((x[4] + x[5]) + (x[6] + x[7]));
    sm += __shfl_xor(sm, 1, 64);
    sm += __shfl_xor(sm, 2, 64);
    sm += __shfl_xor(sm, 4, 64);
    sm += __shfl_xor(sm, 8, 64);
    if (g < ngroups) {
      if (h == 0) sx[cc * 16 + t] = sm;
      float part[NP][8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = x[slot_code(BITS, e)];
        if constexpr (NP == 3)
          split3(v, part[0][e], part[1][e], part[2][e]);
        else
          part[0][e] = v;
      }
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int plane = p / rp, arow = t + rs * (p % rp);
        const u32x4a v = {pack2(part[p][0], part[p][1]), pack2(part[p][2], part[p][3]),
                          pack2(part[p][4], part[p][5]), pack2(part[p][6], part[p][7])};
        *reinterpret_cast<u32x4a*>(lds + ((cc * 4 + m) * NM + plane) * 1024 + frag_slot(s, arow, m) * 16) = v;
      }
    }
  }
  lds_barrier();
  GPTQ_TRACE_STAMP();

  // 5. The chunks in order: 4 MFMA steps per plane and tile (one accumulator
  // each), then the planes' sum and the chunk's zero point and scale.
  f32x4 yacc[MM_RT];
#pragma unroll
  for (int r = 0; r < MM_RT; ++r) yacc[r] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const int64_t nvalid = nch - c_begin < CPS ? nch - c_begin : CPS;
#pragma unroll
  for (int cc = 0; cc < CPS; ++cc) {
    if (cc < nvalid) {
      f32x4 acc[MM_RT][NM];
#pragma unroll
      for (int r = 0; r < MM_RT; ++r)
#pragma unroll
        for (int p = 0; p < NM; ++p) acc[r][p] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      auto step = [&](auto mc) {
        constexpr int M = decltype(mc)::value;
        bf16x8 af[NM];
#pragma unroll
        for (int p = 0; p < NM; ++p)
          af[p] = *reinterpret_cast<const bf16x8*>(lds + ((cc * 4 + M) * NM + p) * 1024 + frag_slot(a, j, M) * 16);
#pragma unroll
        for (int r = 0; r < MM_RT; ++r) {
          const bf16x8 bf = run_frag<BITS, M>(w[cc][r]);
#pragma unroll
          for (int p = 0; p < NM; ++p)
            acc[r][p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[p], bf, acc[r][p], 0, 0, 0);
        }
      };
      step(std::integral_constant<int, 0>{});
      step(std::integral_constant<int, 1>{});
      step(std::integral_constant<int, 2>{});
      step(std::integral_constant<int, 3>{});
      const f32x4 sv = *reinterpret_cast<const f32x4*>(sx + cc * 16 + 4 * a);
      const int gi = (int)((uint32_t)(c_begin + cc) / (uint32_t)gchunks - gk0);
#pragma unroll
      for (int r = 0; r < MM_RT; ++r) {
        const int lr = wave * 16 * MM_RT + 16 * r + j;  // the lane's row within the workgroup
        const float sc = sgl[lr * CPS + gi], z = zgl[lr * CPS + gi];
        f32x4 t = acc[r][0];
#pragma unroll
        for (int p = 1; p < NM; ++p) t += acc[r][p];
#pragma unroll
        for (int v = 0; v < 4; ++v) yacc[r][v] = fmaf(sc, fmaf(-z, sv[v], t[v]), yacc[r][v]);
      }
    }
  }

  GPTQ_TRACE_STAMP();
  // 6. Vector t's rows t + rs k (k < rp) hold its parts: add them in that order,
  // through the fragments' LDS once every wave is done with it.
  lds_barrier();
  float* yb = reinterpret_cast<float*>(lds) + wave * (MM_RT * 256);
#pragma unroll
  for (int r = 0; r < MM_RT; ++r)
#pragma unroll
    for (int v = 0; v < 4; ++v) yb[r * 256 + (4 * a + v) * 16 + j] = yacc[r][v];
  // (a wave's LDS operations complete in order: its reads below see these stores)
  float* o = out + slice * slice_stride;
#pragma unroll
  for (int r = 0; r < MM_RT; ++r)
#pragma unroll
    for (int q = 0; q < MM_MAXT / 4; ++q) {
      const int t = a + 4 * q;
      const int64_t row = r0 + 16 * r + j;
      if (t < T && row < rows) {
        float v = yb[r * 256 + t * 16 + j];
        for (int k = 1; k < rp; ++k) v += yb[r * 256 + (t + rs * k) * 16 + j];
        o[(int64_t)t * ldo + row] = v;
      }
    }
  GPTQ_TRACE_STAMP();
  GPTQ_TRACE_WRITE(TR_MMA, item);
}

// Y[t, r] = sum over slices s (in order) of P[s][t][r]; the loads of up to 64
// slices are queued before they are added (one memory round trip a call for
// every slice count the plans make).
template <int NS>
__global__ void k_mma_reduce(const float* __restrict__ P, int64_t nslices, int64_t T, int64_t rows,
                             float* __restrict__ Y, int64_t ldy) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * rows) return;
  const int64_t t = i / rows, r = i % rows, n = T * rows;
  float v = 0.0f;
  for (int64_t s0 = 0; s0 < nslices; s0 += NS) {
    float p[NS];
#pragma unroll
    for (int k = 0; k < NS; ++k) p[k] = P[(s0 + k < nslices ? s0 + k : nslices - 1) * n + i];
#pragma unroll
    for (int k = 0; k < NS; ++k)
      if (s0 + k < nslices) v = (s0 + k == 0) ? p[k] : v + p[k];
  }
  Y[t * ldy + r] = v;
}

struct MmaPlan {
  int64_t nch, nrb, cps, ks;
};

// Chunks per slice: the most (8, then 4, 2) that still gives enough workgroups
// to fill the chip, so each row is read in long runs.
MmaPlan mma_plan(int64_t rows, int64_t cols) {
  MmaPlan p;
  p.nch = (cols + 127) / 128;
  p.nrb = (rows + MM_ROWS - 1) / MM_ROWS;
  p.cps = 2;
  for (int64_t c : {8, 4}) {
    if (p.nrb * ((p.nch + c - 1) / c) >= MM_TARGET_WG) {
      p.cps = c;
      break;
    }
  }
  p.ks = (p.nch + p.cps - 1) / p.cps;
  return p;
}

// A-row layout for T vectors: parts 3 (fp32) or 1 (bf16); rp parts per plane.
void mma_layout(int T, bool bf16, int& nm, int& rs, int& rp) {
  if (bf16) {
    nm = 1; rs = 16; rp = 1;
  } else if (T <= 5) {
    nm = 1; rs = T; rp = 3;
  } else if (T <= 8) {
    nm = 2; rs = 8; rp = 2;
  } else {
    nm = 3; rs = 16; rp = 1;
  }
}

template <int BITS, int NM, typename XT, int CPS>
hipError_t launch_mma_cps(const uint32_t* packed, const float* scales, const uint8_t* zeros, int64_t rows,
                          int64_t cols, int64_t G, int64_t gchunks, const XT* X, int64_t ldx, int T, int rs, int rp,
                          const MmaPlan& pl, float* out, int64_t ldo, int64_t slice_stride, hipStream_t stream) {
  const dim3 grid((unsigned)(pl.ks * pl.nrb));
  // staging groups per thread: T CPS 16 over 256 threads, at most 16 vectors
  // (fp32 in one or two planes is at most 8)
  constexpr bool F32 = std::is_same<XT, float>::value;
  constexpr int GMAX = (F32 && NM < 3 ? 8 : 16) * CPS * 16 / (64 * MM_NW);
  constexpr int GPT = GMAX < 1 ? 1 : GMAX;
  if (cols % 32 == 0)
    hipLaunchKernelGGL((k_dequant_mma<BITS, NM, true, XT, CPS, GPT>), grid, dim3(64 * MM_NW), 0, stream, packed,
                       scales, zeros, rows, cols, G, gchunks, X, ldx, T, rs, rp, pl.ks, out, ldo, slice_stride);
  else
    hipLaunchKernelGGL((k_dequant_mma<BITS, NM, false, XT, CPS, GPT>), grid, dim3(64 * MM_NW), 0, stream, packed,
                       scales, zeros, rows, cols, G, gchunks, X, ldx, T, rs, rp, pl.ks, out, ldo, slice_stride);
  return hipGetLastError();
}

template <int BITS, int NM, typename XT>
hipError_t launch_mma_nm(const uint32_t* packed, const float* scales, const uint8_t* zeros, int64_t rows,
                         int64_t cols, int64_t G, int64_t gchunks, const XT* X, int64_t ldx, int T, int rs, int rp,
                         const MmaPlan& pl, float* out, int64_t ldo, int64_t slice_stride, hipStream_t stream) {
  if (pl.cps == 8)
    return launch_mma_cps<BITS, NM, XT, 8>(packed, scales, zeros, rows, cols, G, gchunks, X, ldx, T, rs, rp, pl, out,
                                           ldo, slice_stride, stream);
  if (pl.cps == 4)
    return launch_mma_cps<BITS, NM, XT, 4>(packed, scales, zeros, rows, cols, G, gchunks, X, ldx, T, rs, rp, pl, out,
                                           ldo, slice_stride, stream);
  return launch_mma_cps<BITS, NM, XT, 2>(packed, scales, zeros, rows, cols, G, gchunks, X, ldx, T, rs, rp, pl, out,
                                         ldo, slice_stride, stream);
}

template <int BITS, typename XT>
hipError_t launch_mma(const uint32_t* packed, const float* scales, const uint8_t* zeros, int64_t rows, int64_t cols,
                      int64_t G, int64_t gchunks, const XT* X, int64_t ldx, int T, const MmaPlan& pl, float* out,
                      int64_t ldo, int64_t slice_stride, hipStream_t stream) {
  int nm, rs, rp;
  mma_layout(T, std::is_same<XT, uint16_t>::value, nm, rs, rp);
  if (nm == 1)
    return launch_mma_nm<BITS, 1>(packed, scales, zeros, rows, cols, G, gchunks, X, ldx, T, rs, rp, pl, out, ldo,
                                  slice_stride, stream);
  if constexpr (std::is_same<XT, float>::value) {
    if (nm == 2)
      return launch_mma_nm<BITS, 2>(packed, scales, zeros, rows, cols, G, gchunks, X, ldx, T, rs, rp, pl, out, ldo,
                                    slice_stride, stream);
    return launch_mma_nm<BITS, 3>(packed, scales, zeros, rows, cols, G, gchunks, X, ldx, T, rs, rp, pl, out, ldo,
                                  slice_stride, stream);
  }
  return hipErrorInvalidValue;
}

template <typename XT>
hipError_t dequant_mma_x(const uint32_t* packed, const float* scales, const uint8_t* zeros, int64_t rows,
                         int64_t cols, int32_t bits, int32_t groupsize, const XT* X, int64_t ldx, int64_t batch,
                         float* Y, int64_t ldy, void* workspace, hipStream_t stream) {
  const MmaPlan pl = mma_plan(rows, cols);
  const int64_t G = groupsize == -1 ? 1 : (cols + groupsize - 1) / groupsize;
  // chunks per group (a group of the whole row: more chunks than the row has)
  const int64_t gchunks = groupsize == -1 ? pl.nch + 1 : groupsize / 128;
  for (int64_t b0 = 0; b0 < batch; b0 += MM_MAXT) {
    const int T = (int)(batch - b0 < MM_MAXT ? batch - b0 : MM_MAXT);
    const XT* xb = X + b0 * ldx;
    float* yb = Y + b0 * ldy;
    float* out = pl.ks > 1 ? static_cast<float*>(workspace) : yb;
    const int64_t ldo = pl.ks > 1 ? rows : ldy;
    const int64_t sstride = pl.ks > 1 ? (int64_t)T * rows : 0;
    hipError_t e;
    switch (bits) {
      case 2: e = launch_mma<2>(packed, scales, zeros, rows, cols, G, gchunks, xb, ldx, T, pl, out, ldo, sstride, stream); break;
      case 3: e = launch_mma<3>(packed, scales, zeros, rows, cols, G, gchunks, xb, ldx, T, pl, out, ldo, sstride, stream); break;
      case 4: e = launch_mma<4>(packed, scales, zeros, rows, cols, G, gchunks, xb, ldx, T, pl, out, ldo, sstride, stream); break;
      default: e = launch_mma<8>(packed, scales, zeros, rows, cols, G, gchunks, xb, ldx, T, pl, out, ldo, sstride, stream); break;
    }
    if (e != hipSuccess) return e;
    if (pl.ks > 1) {
      const int64_t n = (int64_t)T * rows;
      const dim3 rg((unsigned)((n + 255) / 256));
      const float* P = static_cast<const float*>(workspace);
      if (pl.ks <= 16)
        hipLaunchKernelGGL(k_mma_reduce<16>, rg, dim3(256), 0, stream, P, pl.ks, (int64_t)T, rows, yb, ldy);
      else if (pl.ks <= 32)
        hipLaunchKernelGGL(k_mma_reduce<32>, rg, dim3(256), 0, stream, P, pl.ks, (int64_t)T, rows, yb, ldy);
      else
        hipLaunchKernelGGL(k_mma_reduce<64>, rg, dim3(256), 0, stream, P, pl.ks, (int64_t)T, rows, yb, ldy);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace

#ifdef GPTQ_TRACE
GPTQ_TRACE_SETTER(trace_set_mma)
#endif

bool dequant_mma_supported(int64_t cols, int32_t groupsize, int64_t batch) {
  return batch >= 2 && cols >= 4 && (groupsize == -1 || (groupsize > 0 && groupsize % 128 == 0));
}

size_t dequant_mma_workspace(int64_t rows, int64_t cols, int64_t batch) {
  if (rows <= 0 || cols <= 0 || batch <= 0) return 0;
  const MmaPlan pl = mma_plan(rows, cols);
  if (pl.ks <= 1) return 0;
  const int64_t T = batch < MM_MAXT ? batch : MM_MAXT;
  return align_up((size_t)(pl.ks * T * rows) * sizeof(float), 256);
}

hipError_t dequant_mma(const uint32_t* packed, const float* scales, const uint8_t* zeros, int64_t rows,
                       int64_t cols, int32_t bits, int32_t groupsize, const void* X, bool x_bf16, int64_t ldx,
                       int64_t batch, float* Y, int64_t ldy, void* workspace, hipStream_t stream) {
  if (x_bf16)
    return dequant_mma_x(packed, scales, zeros, rows, cols, bits, groupsize, static_cast<const uint16_t*>(X), ldx,
                         batch, Y, ldy, workspace, stream);
  return dequant_mma_x(packed, scales, zeros, rows, cols, bits, groupsize, static_cast<const float*>(X), ldx, batch,
                       Y, ldy, workspace, stream);
}

}  // namespace gptq
