// y = W^ x straight from the quantizer's outputs: the packed codes (per row a
// little-endian bitstream of b-bit codes, code i at stream bits [i b, (i+1) b)),
// the fp32 group scales and the integer group zeros, w^ = s_g (q - z_g).
//
// HBM-bound: a row costs cols b / 8 bytes of codes plus its G scales and zeros,
// and x is shared by every row.  The unit of work is a run of 32 codes, which
// is b whole words and lies in one group (groups are multiples of 32 columns).
// A workgroup stages x through LDS, a chunk at a time, read once from memory in
// whole coalesced vectors.  A wave owns R rows and one of S column slices; its
// lane l takes the runs l, l + 64, ... of the slice (so a wave's loads from a
// row are contiguous), reads the run's 32 x values from LDS once and applies
// them to its R rows:
//   y_r += s_g (sum_i q_i x_i - z_g sum_i x_i).
// Lanes meet in a butterfly over the wave, slices in LDS.  Accumulation is
// fp32 in a fixed order, so results are reproducible.  A small-batch variant
// (k_dequant_gemm, below) converts each run's codes to floats once and applies
// them to up to 8 vectors staged together.
#include <type_traits>

#include "common.h"

namespace gptq {
namespace {

// dword-aligned vector loads (global loads of several dwords need only dword
// alignment, so rows whose word count is not a multiple of 4 still load whole)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2), aligned(4)));
typedef float f32x4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4), aligned(4)));

// Four consecutive x values as fp32 (bf16 widens exactly).
__device__ __forceinline__ f32x4 load_x4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 load_x4(const uint16_t* p) {
  const u16x4 v = *reinterpret_cast<const u16x4*>(p);
  return f32x4{__uint_as_float((uint32_t)v.x << 16), __uint_as_float((uint32_t)v.y << 16),
               __uint_as_float((uint32_t)v.z << 16), __uint_as_float((uint32_t)v.w << 16)};
}

template <int BITS>
__device__ __forceinline__ void load_run(const uint32_t* p, uint32_t (&w)[BITS]) {
  if constexpr (BITS == 2) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(p);
    w[0] = v.x; w[1] = v.y;
  } else if constexpr (BITS == 3) {
    w[0] = p[0]; w[1] = p[1]; w[2] = p[2];
  } else {
#pragma unroll
    for (int j = 0; j < BITS; j += 4) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(p + j);
      w[j] = v.x; w[j + 1] = v.y; w[j + 2] = v.z; w[j + 3] = v.w;
    }
  }
}

__device__ __forceinline__ float byte_f(uint32_t v, int b) { return (float)((v >> (8 * b)) & 0xffu); }

// Codes narrower than 5 bits convert two at a time: a byte holding q < 16 read
// as an fp8 e4m3 value is a subnormal or the smallest binade, exactly q times a
// power of two (q m / 8 2^(1 - bias) either way), so one pair conversion gives
// two codes up to that factor.  code_unit() is the factor's inverse, exact.
__device__ __forceinline__ float code_unit() { return 1.0f / __builtin_amdgcn_cvt_f32_fp8(1, 0); }

// sum_i q_i x_i over one run: for 2 and 4 bits scaled by 1 / code_unit(), else
// exact codes.  One mask isolates four codes in the four bytes of a word.
template <int BITS>
__device__ __forceinline__ float run_dot(const uint32_t (&w)[BITS], const float (&x)[32]) {
  float acc = 0.0f;
  if constexpr (BITS == 8) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc = fmaf(byte_f(w[j], b), x[4 * j + b], acc);
  } else if constexpr (BITS == 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = w[j] & 0x0f0f0f0fu, hi = (w[j] >> 4) & 0x0f0f0f0fu;
      // byte b of lo holds code 8j + 2b, of hi code 8j + 2b + 1
      const auto l01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);
      const auto h01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
      const auto l23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
      const auto h23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
      acc = fmaf(l01[0], x[8 * j + 0], acc);
      acc = fmaf(h01[0], x[8 * j + 1], acc);
      acc = fmaf(l01[1], x[8 * j + 2], acc);
      acc = fmaf(h01[1], x[8 * j + 3], acc);
      acc = fmaf(l23[0], x[8 * j + 4], acc);
      acc = fmaf(h23[0], x[8 * j + 5], acc);
      acc = fmaf(l23[1], x[8 * j + 6], acc);
      acc = fmaf(h23[1], x[8 * j + 7], acc);
    }
  } else if constexpr (BITS == 2) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        // byte b of c holds code 16j + 4b + s
        const uint32_t c = (w[j] >> (2 * s)) & 0x03030303u;
        const auto c01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c, false);
        const auto c23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c, true);
        acc = fmaf(c01[0], x[16 * j + s], acc);
        acc = fmaf(c01[1], x[16 * j + 4 + s], acc);
        acc = fmaf(c23[0], x[16 * j + 8 + s], acc);
        acc = fmaf(c23[1], x[16 * j + 12 + s], acc);
      }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int bit = 3 * i, wi = bit >> 5, sh = bit & 31;
      const uint32_t v = sh + 3 > 32 ? __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) : w[wi] >> sh;
      acc = fmaf((float)(v & 7u), x[i], acc);
    }
  }
  return acc;
}

// A run's 32 codes as floats, in code order, scaled as run_dot scales them
// (1 / code_unit() for 2 and 4 bits, exact otherwise).
template <int BITS>
__device__ __forceinline__ void run_codes(const uint32_t (&w)[BITS], float (&q)[32]) {
  if constexpr (BITS == 8) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int b = 0; b < 4; ++b) q[4 * j + b] = byte_f(w[j], b);
  } else if constexpr (BITS == 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = w[j] & 0x0f0f0f0fu, hi = (w[j] >> 4) & 0x0f0f0f0fu;
      const auto l01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);
      const auto h01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
      const auto l23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
      const auto h23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
      q[8 * j + 0] = l01[0]; q[8 * j + 1] = h01[0]; q[8 * j + 2] = l01[1]; q[8 * j + 3] = h01[1];
      q[8 * j + 4] = l23[0]; q[8 * j + 5] = h23[0]; q[8 * j + 6] = l23[1]; q[8 * j + 7] = h23[1];
    }
  } else if constexpr (BITS == 2) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t c = (w[j] >> (2 * s)) & 0x03030303u;
        const auto c01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c, false);
        const auto c23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c, true);
        q[16 * j + s] = c01[0]; q[16 * j + 4 + s] = c01[1]; q[16 * j + 8 + s] = c23[0]; q[16 * j + 12 + s] = c23[1];
      }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int bit = 3 * i, wi = bit >> 5, sh = bit & 31;
      const uint32_t v = sh + 3 > 32 ? __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) : w[wi] >> sh;
      q[i] = (float)(v & 7u);
    }
  }
}

// x goes through LDS in chunks of XCH runs, each run's 32 values in a row of XP
// floats: the padding puts the rows of eight consecutive runs on different
// banks, so the lanes' 16-byte reads of their runs do not collide.  Two chunk
// buffers alternate: the next chunk's x is loaded into registers before the
// lane's weight prefetches are issued and written to the other buffer after
// the current chunk is applied.  Loads retire in issue order, so waiting for x
// never waits for the weights queued after it, and the barrier between chunks
// waits only for LDS: the weight loads of the next two runs stay in flight
// across it.
constexpr int XCH = 128;
constexpr int XP = 36;

// Barrier for LDS traffic only: this wave's LDS operations are done, then every
// wave of the workgroup meets.  (__syncthreads also waits for every outstanding
// global load, which would drain the weight prefetches at each chunk.)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Template: NW waves per workgroup, R rows per wave, S waves share a row group
// (column slices).  gr = runs per group (any value above the last run when the
// row is one group).
template <int BITS, int R, int S, int NW, bool WHOLE, typename XT>
__global__ __launch_bounds__(64 * NW) void k_dequant_gemv(const uint32_t* __restrict__ packed,
                                                      const float* __restrict__ scales,
                                                      const uint8_t* __restrict__ zeros, int64_t rows, int64_t cols,
                                                      int64_t G, uint32_t gr, const XT* __restrict__ x,
                                                      float* __restrict__ y) {
  constexpr int RG = NW / S;             // row groups per workgroup
  constexpr int IT = XCH / (64 * S);     // runs per lane per chunk
  constexpr int XV = XCH * 32 / (256 * NW);  // 4-float x vectors per thread and chunk
  static_assert(IT >= 1 && IT * 64 * S == XCH, "chunk must be whole lane sweeps");
  __shared__ __align__(16) float xs[2][XCH * XP];
  __shared__ float sxs[2][XCH];  // sum of each run's 32 x values
  __shared__ float part[RG][R][S];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rg = wave / S, cs = wave % S;
  const int64_t r0 = ((int64_t)blockIdx.x * RG + rg) * R;
  const int64_t wpr = cols * BITS / 32;  // words per row
  const int64_t nfull = cols / 32, nrun = (cols + 31) / 32;
  const float unit = (BITS == 2 || BITS == 4) ? code_unit() : 1.0f;
  const uint32_t* prow[R];
  const float* srow[R];
  const uint8_t* zrow[R];
#pragma unroll
  for (int q = 0; q < R; ++q) {
    const int64_t r = r0 + q < rows ? r0 + q : rows - 1;  // rows past the end repeat the last, unwritten
    prow[q] = packed + r * wpr;
    srow[q] = scales + r * G;
    zrow[q] = zeros + r * G;
  }
  // Operands of one run for the R rows: codes, scale, zero point.
  struct Ops {
    uint32_t w[R][BITS];
    float s[R], z[R];
  };
  // WHOLE (cols % 32 == 0): every run is whole, and a lane past the last run
  // reloads the last one (ignored), so the loads carry no branch and the
  // compiler's waits count them exactly.
  auto fetch = [&](int64_t k, Ops& o) {
    if constexpr (WHOLE) {
      const int64_t kc = k < nrun ? k : nrun - 1;
#pragma unroll
      for (int q = 0; q < R; ++q) load_run<BITS>(prow[q] + BITS * kc, o.w[q]);
      const uint32_t gk = (uint32_t)kc / gr;
#pragma unroll
      for (int q = 0; q < R; ++q) {
        o.s[q] = srow[q][gk];
        o.z[q] = (float)zrow[q][gk];
      }
      return;
    }
    if (k >= nrun) return;
    if (k < nfull) {
#pragma unroll
      for (int q = 0; q < R; ++q) load_run<BITS>(prow[q] + BITS * k, o.w[q]);
    } else {
      // the last, partial run: m codes in m b / 32 whole words (x past cols is 0 in xs)
      const int nw = (int)(cols - 32 * k) * BITS / 32;
#pragma unroll
      for (int q = 0; q < R; ++q)
#pragma unroll
        for (int j = 0; j < BITS; ++j) o.w[q][j] = j < nw ? prow[q][BITS * k + j] : 0u;
    }
    const uint32_t gk = (uint32_t)k / gr;
#pragma unroll
    for (int q = 0; q < R; ++q) {
      o.s[q] = srow[q][gk];
      o.z[q] = (float)zrow[q][gk];
    }
  };
  // raw x vectors (bf16 stays packed until stored, so nothing waits for its load before then)
  using XR = typename std::conditional<std::is_same<XT, float>::value, f32x4, u16x4>::type;
  XR xr[XV];
  auto load_x = [&](int64_t c0) {
#pragma unroll
    for (int j = 0; j < XV; ++j) {
      const int e = 4 * (threadIdx.x + 64 * NW * j);  // float index within the chunk
      const int64_t col = 32 * c0 + e;
      // cols is a multiple of 4 (cols b is whole words), so a vector is all in or all
      // out; one past the end reloads the last vector (no branch) and is zeroed when
      // stored, not here, so that nothing waits for the load before then
      xr[j] = *reinterpret_cast<const XR*>(x + (col < cols ? col : cols - 4));
    }
  };
  // a run's 8 vectors lie in 8 consecutive threads of one wave, whose butterfly gives
  // every one of them the same sum
  auto store_x = [&](float* buf, float* sbuf, int64_t c0) {
#pragma unroll
    for (int j = 0; j < XV; ++j) {
      const int e = 4 * (threadIdx.x + 64 * NW * j);
      const bool in = 32 * c0 + e < cols;
      f32x4 v;
      if constexpr (std::is_same<XT, float>::value)
        v = xr[j];
      else
        v = f32x4{__uint_as_float((uint32_t)xr[j].x << 16), __uint_as_float((uint32_t)xr[j].y << 16),
                  __uint_as_float((uint32_t)xr[j].z << 16), __uint_as_float((uint32_t)xr[j].w << 16)};
      if (!in) v = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      *reinterpret_cast<float4*>(buf + (e >> 5) * XP + (e & 31)) = make_float4(v.x, v.y, v.z, v.w);
      float t = (v.x + v.y) + (v.z + v.w);
      t += __shfl_xor(t, 1, 64);
      t += __shfl_xor(t, 2, 64);
      t += __shfl_xor(t, 4, 64);
      if ((threadIdx.x & 7) == 0) sbuf[e >> 5] = t;
    }
  };
  float yacc[R] = {};
  const int64_t step = 64 * S;  // the lane's next run
  const int64_t k0 = (int64_t)cs * 64 + lane;
  load_x(0);
  Ops cur, nx1;
  fetch(k0, cur);
  fetch(k0 + step, nx1);
  store_x(xs[0], sxs[0], 0);
  lds_barrier();
  int buf = 0;
  for (int64_t c0 = 0; c0 < nrun; c0 += XCH) {
    const bool more = c0 + XCH < nrun;
    if (more) load_x(c0 + XCH);
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int kk = cs * 64 + lane + it * 64 * S;
      const int64_t k = c0 + kk;
      // two runs of the lane ahead are in flight while this one is applied
      Ops nx2;
      fetch(k + 2 * step, nx2);
      if (k < nrun) {
        float xv[32];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float4 v = *reinterpret_cast<const float4*>(xs[buf] + kk * XP + 4 * i);
          xv[4 * i] = v.x; xv[4 * i + 1] = v.y; xv[4 * i + 2] = v.z; xv[4 * i + 3] = v.w;
        }
        const float sx = sxs[buf][kk];
#pragma unroll
        for (int q = 0; q < R; ++q)
          yacc[q] = fmaf(cur.s[q], fmaf(run_dot<BITS>(cur.w[q], xv), unit, -cur.z[q] * sx), yacc[q]);
      }
      cur = nx1;
      nx1 = nx2;
    }
    // the other buffer was last read in the previous chunk, before the last barrier
    if (more) store_x(xs[buf ^ 1], sxs[buf ^ 1], c0 + XCH);
    lds_barrier();
    buf ^= 1;
  }
#pragma unroll
  for (int q = 0; q < R; ++q) {
    float v = yacc[q];
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) v += __shfl_xor(v, m, 64);
    yacc[q] = v;
  }
  if constexpr (S == 1) {
    if (lane < R) {
      float v = yacc[0];
#pragma unroll
      for (int q = 1; q < R; ++q)
        if (lane == q) v = yacc[q];
      if (r0 + lane < rows) y[r0 + lane] = v;
    }
  } else {
    if (lane == 0)
#pragma unroll
      for (int q = 0; q < R; ++q) part[rg][q][cs] = yacc[q];
    __syncthreads();
    if (threadIdx.x < RG * R) {
      const int trg = threadIdx.x / R, tq = threadIdx.x % R;
      float v = 0.0f;
#pragma unroll
      for (int c = 0; c < S; ++c) v += part[trg][tq][c];
      const int64_t r = ((int64_t)blockIdx.x * RG + trg) * R + tq;
      if (r < rows) y[r] = v;
    }
  }
}

template <int BITS, int R, int S, int NW, typename XT>
hipError_t launch(const uint32_t* packed, const float* scales, const uint8_t* zeros, int64_t rows, int64_t cols,
                  int64_t G, uint32_t gr, const XT* x, float* y, hipStream_t stream) {
  constexpr int64_t rows_per_wg = (NW / S) * R;
  const unsigned grid = (unsigned)((rows + rows_per_wg - 1) / rows_per_wg);
  if (cols % 32 == 0 && cols >= 32)
    hipLaunchKernelGGL((k_dequant_gemv<BITS, R, S, NW, true, XT>), dim3(grid), dim3(64 * NW), 0, stream, packed,
                       scales, zeros, rows, cols, G, gr, x, y);
  else
    hipLaunchKernelGGL((k_dequant_gemv<BITS, R, S, NW, false, XT>), dim3(grid), dim3(64 * NW), 0, stream, packed,
                       scales, zeros, rows, cols, G, gr, x, y);
  return hipGetLastError();
}

template <int BITS, typename XT>
hipError_t launch_bits(const uint32_t* packed, const float* scales, const uint8_t* zeros, int64_t rows, int64_t cols,
                       int64_t G, uint32_t gr, const XT* x, float* y, hipStream_t stream) {
  // Few rows: two rows a wave and the columns split over two waves, for enough
  // waves to fill the chip, eight waves a workgroup so one staging of x serves
  // eight rows; many rows: four rows a wave, x reused more.
  if (rows < 8192) return launch<BITS, 2, 2, 8>(packed, scales, zeros, rows, cols, G, gr, x, y, stream);
  return launch<BITS, 4, 1, 4>(packed, scales, zeros, rows, cols, G, gr, x, y, stream);
}

// Y[t, :] = W^ X[t, :] for a small batch of T activation vectors.  Same
// layout as the single-vector kernel with R = 2, S = 1 and chunks of 64 runs:
// a lane converts its run's codes to floats once and applies them to all T
// vectors, staged together in LDS.
constexpr int BCH = 64;
constexpr int GEMM_NW = 8;  // waves per workgroup (one staging of x serves 16 rows)

template <int BITS, int T, int NW, bool WHOLE, typename XT>
__global__ __launch_bounds__(64 * NW) void k_dequant_gemm(const uint32_t* __restrict__ packed,
                                                      const float* __restrict__ scales,
                                                      const uint8_t* __restrict__ zeros, int64_t rows, int64_t cols,
                                                      int64_t G, uint32_t gr, const XT* __restrict__ X, int64_t ldx,
                                                      float* __restrict__ Y, int64_t ldy) {
  constexpr int R = 2;
  static_assert(BCH * 32 == 256 * NW, "one 4-float x vector per thread and activation vector");
  __shared__ __align__(16) float xs[T][BCH * XP];
  __shared__ float sxs[T][BCH];  // sum of each run's 32 x values
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r0 = ((int64_t)blockIdx.x * NW + wave) * R;
  const int64_t wpr = cols * BITS / 32;
  const int64_t nfull = cols / 32, nrun = (cols + 31) / 32;
  const float unit = (BITS == 2 || BITS == 4) ? code_unit() : 1.0f;
  const uint32_t* prow[R];
  const float* srow[R];
  const uint8_t* zrow[R];
#pragma unroll
  for (int q = 0; q < R; ++q) {
    const int64_t r = r0 + q < rows ? r0 + q : rows - 1;  // rows past the end repeat the last, unwritten
    prow[q] = packed + r * wpr;
    srow[q] = scales + r * G;
    zrow[q] = zeros + r * G;
  }
  struct Ops {
    uint32_t w[R][BITS];
    float s[R], z[R];
  };
  // as in k_dequant_gemv: WHOLE runs load without a branch (a lane past the last
  // run reloads it, ignored)
  auto fetch = [&](int64_t k, Ops& o) {
    if constexpr (WHOLE) {
      const int64_t kc = k < nrun ? k : nrun - 1;
#pragma unroll
      for (int q = 0; q < R; ++q) load_run<BITS>(prow[q] + BITS * kc, o.w[q]);
      const uint32_t gk = (uint32_t)kc / gr;
#pragma unroll
      for (int q = 0; q < R; ++q) {
        o.s[q] = srow[q][gk];
        o.z[q] = (float)zrow[q][gk];
      }
      return;
    }
    if (k >= nrun) return;
    if (k < nfull) {
#pragma unroll
      for (int q = 0; q < R; ++q) load_run<BITS>(prow[q] + BITS * k, o.w[q]);
    } else {
      const int nw = (int)(cols - 32 * k) * BITS / 32;  // the partial last run's whole words
#pragma unroll
      for (int q = 0; q < R; ++q)
#pragma unroll
        for (int j = 0; j < BITS; ++j) o.w[q][j] = j < nw ? prow[q][BITS * k + j] : 0u;
    }
    const uint32_t gk = (uint32_t)k / gr;
#pragma unroll
    for (int q = 0; q < R; ++q) {
      o.s[q] = srow[q][gk];
      o.z[q] = (float)zrow[q][gk];
    }
  };
  // The next chunk's x is loaded into registers before the next run's weights
  // are queued, and written to LDS after this chunk is applied, between two
  // LDS-only barriers, so the weight loads stay in flight across them.
  using XR = typename std::conditional<std::is_same<XT, float>::value, f32x4, u16x4>::type;
  XR xr[T];
  const int e = 4 * threadIdx.x;  // this thread's float index within a chunk
  auto load_x = [&](int64_t c0) {
    const int64_t col = 32 * c0 + e;
    const int64_t cc = col < cols ? col : cols - 4;  // cols >= 4 (a multiple of 4)
#pragma unroll
    for (int t = 0; t < T; ++t) xr[t] = *reinterpret_cast<const XR*>(X + t * ldx + cc);
  };
  auto store_x = [&](int64_t c0) {
    const bool in = 32 * c0 + e < cols;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      f32x4 v;
      if constexpr (std::is_same<XT, float>::value)
        v = xr[t];
      else
        v = f32x4{__uint_as_float((uint32_t)xr[t].x << 16), __uint_as_float((uint32_t)xr[t].y << 16),
                  __uint_as_float((uint32_t)xr[t].z << 16), __uint_as_float((uint32_t)xr[t].w << 16)};
      if (!in) v = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      *reinterpret_cast<float4*>(&xs[t][(e >> 5) * XP + (e & 31)]) = make_float4(v.x, v.y, v.z, v.w);
      float sm = (v.x + v.y) + (v.z + v.w);
      sm += __shfl_xor(sm, 1, 64);
      sm += __shfl_xor(sm, 2, 64);
      sm += __shfl_xor(sm, 4, 64);
      if ((threadIdx.x & 7) == 0) sxs[t][e >> 5] = sm;
    }
  };
  float yacc[T][R] = {};
  Ops cur;
  load_x(0);
  fetch(lane, cur);
  store_x(0);
  lds_barrier();
  for (int64_t c0 = 0; c0 < nrun; c0 += BCH) {
    const bool more = c0 + BCH < nrun;
    if (more) load_x(c0 + BCH);
    Ops nxt;
    fetch(c0 + BCH + lane, nxt);
    const int64_t k = c0 + lane;
    if (k < nrun) {
      float qv[R][32];
#pragma unroll
      for (int q = 0; q < R; ++q) run_codes<BITS>(cur.w[q], qv[q]);
#pragma unroll
      for (int t = 0; t < T; ++t) {
        float xv[32];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float4 v = *reinterpret_cast<const float4*>(&xs[t][lane * XP + 4 * i]);
          xv[4 * i] = v.x; xv[4 * i + 1] = v.y; xv[4 * i + 2] = v.z; xv[4 * i + 3] = v.w;
        }
        const float sx = sxs[t][lane];
#pragma unroll
        for (int q = 0; q < R; ++q) {
          float dot = 0.0f;
#pragma unroll
          for (int i = 0; i < 32; ++i) dot = fmaf(qv[q][i], xv[i], dot);
          yacc[t][q] = fmaf(cur.s[q], fmaf(dot, unit, -cur.z[q] * sx), yacc[t][q]);
        }
      }
    }
    if (more) {
      lds_barrier();  // every wave is done with this chunk's x
      store_x(c0 + BCH);
      lds_barrier();
    }
    cur = nxt;
  }
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int q = 0; q < R; ++q) {
      float v = yacc[t][q];
#pragma unroll
      for (int m = 32; m > 0; m >>= 1) v += __shfl_xor(v, m, 64);
      if (lane == 0 && r0 + q < rows) Y[t * ldy + r0 + q] = v;
    }
}

template <int BITS, int T, typename XT>
hipError_t launch_gemm(const uint32_t* packed, const float* scales, const uint8_t* zeros, int64_t rows, int64_t cols,
                       int64_t G, uint32_t gr, const XT* X, int64_t ldx, float* Y, int64_t ldy, hipStream_t stream) {
  constexpr int NW = GEMM_NW;
  const unsigned grid = (unsigned)((rows + 2 * NW - 1) / (2 * NW));
  if (cols % 32 == 0 && cols >= 32)
    hipLaunchKernelGGL((k_dequant_gemm<BITS, T, NW, true, XT>), dim3(grid), dim3(64 * NW), 0, stream, packed, scales,
                       zeros, rows, cols, G, gr, X, ldx, Y, ldy);
  else
    hipLaunchKernelGGL((k_dequant_gemm<BITS, T, NW, false, XT>), dim3(grid), dim3(64 * NW), 0, stream, packed, scales,
                       zeros, rows, cols, G, gr, X, ldx, Y, ldy);
  return hipGetLastError();
}

template <int BITS, typename XT>
hipError_t gemm_bits(const uint32_t* packed, const float* scales, const uint8_t* zeros, int64_t rows, int64_t cols,
                     int64_t G, uint32_t gr, const XT* X, int64_t ldx, int t, float* Y, int64_t ldy,
                     hipStream_t stream) {
  if (t >= 8) return launch_gemm<BITS, 8>(packed, scales, zeros, rows, cols, G, gr, X, ldx, Y, ldy, stream);
  if (t >= 4) return launch_gemm<BITS, 4>(packed, scales, zeros, rows, cols, G, gr, X, ldx, Y, ldy, stream);
  return launch_gemm<BITS, 2>(packed, scales, zeros, rows, cols, G, gr, X, ldx, Y, ldy, stream);
}

}  // namespace

bool dequant_gemv_supported(int64_t cols, int32_t bits, int32_t groupsize) {
  if (!(bits == 2 || bits == 3 || bits == 4 || bits == 8)) return false;
  if ((cols * bits) % 32 != 0) return false;
  return groupsize == -1 || (groupsize > 0 && groupsize % 32 == 0);
}

template <typename XT>
hipError_t dequant_gemv_x(const uint32_t* packed, const float* scales, const uint8_t* zeros, int64_t rows,
                          int64_t cols, int32_t bits, int32_t groupsize, const XT* x, float* y, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  // no columns: every y is 0, written by a fill kernel (the product kernel's
  // branch-free loads assume at least one whole run)
  if (cols <= 0) return fill_i32(reinterpret_cast<int*>(y), rows, 0, stream);
  const int64_t nrun = (cols + 31) / 32;
  const int64_t G = groupsize == -1 ? 1 : (cols + groupsize - 1) / groupsize;
  const uint32_t gr = groupsize == -1 ? (uint32_t)(nrun > 0 ? nrun : 1) : (uint32_t)(groupsize / 32);
  switch (bits) {
    case 2: return launch_bits<2>(packed, scales, zeros, rows, cols, G, gr, x, y, stream);
    case 3: return launch_bits<3>(packed, scales, zeros, rows, cols, G, gr, x, y, stream);
    case 4: return launch_bits<4>(packed, scales, zeros, rows, cols, G, gr, x, y, stream);
    default: return launch_bits<8>(packed, scales, zeros, rows, cols, G, gr, x, y, stream);
  }
}

hipError_t dequant_gemv(const uint32_t* packed, const float* scales, const uint8_t* zeros, int64_t rows,
                        int64_t cols, int32_t bits, int32_t groupsize, const void* x, bool x_bf16, float* y,
                        hipStream_t stream) {
  if (x_bf16)
    return dequant_gemv_x(packed, scales, zeros, rows, cols, bits, groupsize, static_cast<const uint16_t*>(x), y,
                          stream);
  return dequant_gemv_x(packed, scales, zeros, rows, cols, bits, groupsize, static_cast<const float*>(x), y, stream);
}

template <typename XT>
hipError_t dequant_gemm_x(const uint32_t* packed, const float* scales, const uint8_t* zeros, int64_t rows,
                          int64_t cols, int32_t bits, int32_t groupsize, const XT* X, int64_t ldx, int64_t batch,
                          float* Y, int64_t ldy, hipStream_t stream) {
  if (cols <= 0) {
    // no columns: every output is 0 (the product kernels' loads assume a column)
    for (int64_t t = 0; t < batch; ++t) {
      const hipError_t e = fill_i32(reinterpret_cast<int*>(Y + t * ldy), rows, 0, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  const int64_t nrun = (cols + 31) / 32;
  const int64_t G = groupsize == -1 ? 1 : (cols + groupsize - 1) / groupsize;
  const uint32_t gr = groupsize == -1 ? (uint32_t)(nrun > 0 ? nrun : 1) : (uint32_t)(groupsize / 32);
  for (int64_t b0 = 0; b0 < batch;) {
    const int64_t left = batch - b0;
    const XT* xb = X + b0 * ldx;
    float* yb = Y + b0 * ldy;
    hipError_t e;
    int took;
    if (left == 1) {
      e = dequant_gemv_x(packed, scales, zeros, rows, cols, bits, groupsize, xb, yb, stream);
      took = 1;
    } else {
      took = left >= 8 ? 8 : (left >= 4 ? 4 : 2);
      switch (bits) {
        case 2: e = gemm_bits<2>(packed, scales, zeros, rows, cols, G, gr, xb, ldx, took, yb, ldy, stream); break;
        case 3: e = gemm_bits<3>(packed, scales, zeros, rows, cols, G, gr, xb, ldx, took, yb, ldy, stream); break;
        case 4: e = gemm_bits<4>(packed, scales, zeros, rows, cols, G, gr, xb, ldx, took, yb, ldy, stream); break;
        default: e = gemm_bits<8>(packed, scales, zeros, rows, cols, G, gr, xb, ldx, took, yb, ldy, stream); break;
      }
    }
    if (e != hipSuccess) return e;
    b0 += took;
  }
  return hipSuccess;
}

hipError_t dequant_gemm(const uint32_t* packed, const float* scales, const uint8_t* zeros, int64_t rows,
                        int64_t cols, int32_t bits, int32_t groupsize, const void* X, bool x_bf16, int64_t ldx,
                        int64_t batch, float* Y, int64_t ldy, hipStream_t stream) {
  if (rows <= 0 || batch <= 0) return hipSuccess;
  if (x_bf16)
    return dequant_gemm_x(packed, scales, zeros, rows, cols, bits, groupsize, static_cast<const uint16_t*>(X), ldx,
                          batch, Y, ldy, stream);
  return dequant_gemm_x(packed, scales, zeros, rows, cols, bits, groupsize, static_cast<const float*>(X), ldx, batch,
                        Y, ldy, stream);
}

}  // namespace gptq
