// fp32 MFMA GEMM for the blocked factor (panel product, trailing symmetric
// update, triangular inverse) and for the trailing update of the column loop:
//
//   C[m][n] = alpha * sum_k A(m, k) B(k, n)  (+ C[m][n] when beta != 0)
//
// A is m-major (row m of A holds its k values).  B is k-major (row k holds n)
// or n-major (row n holds k).
//
// Tiles are TM x TM (TM = 128, or 64 when 128-tiles would leave CUs idle) per
// workgroup of 256 threads: 4 waves in a 2x2 grid, each wave owning a
// (TM/2)^2 quarter as 32x32 blocks of v_mfma_f32_32x32x2_f32.  K runs in
// stages of 16.  An MFMA lane supplies one k of one row, and the order in
// which k is summed is free, so lane half h of MFMA step kk takes
// k = 8h + kk: a lane's 8 values of a stage are contiguous in an m-major row
// and arrive with two 16-byte LDS reads.  Stages reach LDS by direct
// global->LDS loads in the operand's own orientation, no transpose:
//   m-major operand: [TM rows][16 k], 64-byte rows whose four 16-byte chunks
//     are XORed with (row >> 2) & 3 (16 rows read by 16 lanes hit all 64
//     banks once);
//   k-major B: [16 k][TM n]; with two column blocks per wave a lane reads 2
//     adjacent columns (8 bytes) and feeds one to each block, so block b of a
//     wave holds columns 2j + b, which the store of C undoes.
// Four stage buffers rotate (64 KB at TM = 128, so two workgroups share a
// CU and one's loads and C traffic overlap the other's MFMAs): loads run
// three stages ahead of the MFMAs and a buffer is read one full stage after
// the barrier that retired its loads (reading right after that barrier was
// seen to return stale LDS data).  With beta set, the tile's C is loaded into
// registers before the K loop so its latency hides under the MFMAs.
// Tiles that are not whole (edges, ragged K, unaligned rows) take a guarded
// path: zero-filled register loads stored into the same layouts.
#include "gemm_tile.h"

namespace gptq {
namespace {

template <int TM, bool BKM>
__global__ __launch_bounds__(256, 2) void k_gemm_f32(GemmF32 g) {
  __shared__ __attribute__((aligned(16))) char lds[gemm_tile_lds<TM>()];
  int tm, tn;
  if (g.tri) {
    // lower-triangular tile enumeration: t -> (tm, tn), tn <= tm
    const int t = blockIdx.x;
    int r = (int)((sqrtf(8.f * (float)t + 1.f) - 1.f) * 0.5f);
    while ((r + 1) * (r + 2) / 2 <= t) ++r;
    while (r * (r + 1) / 2 > t) --r;
    tm = r;
    tn = t - r * (r + 1) / 2;
  } else if (g.order) {
    // K limited by the tile's column (klo_n) or row (khi_m): tiles with the
    // longest K go first, so the last ones to start are the short ones
    const int mt = (g.M + TM - 1) / TM;
    const int t = blockIdx.x;
    tn = t / mt;
    tm = t % mt;
    if (g.order == 2) {
      const int nt = (g.N + TM - 1) / TM;
      tm = mt - 1 - t / nt;
      tn = t % nt;
    }
  } else {
    tn = blockIdx.x;
    tm = blockIdx.y;
  }
  gemm_tile<TM, BKM>(g, tm, tn, blockIdx.z, lds);
}

template <int TM>
hipError_t launch(const GemmF32& g, hipStream_t stream) {
  const int tm = (g.M + TM - 1) / TM, tn = (g.N + TM - 1) / TM;
  dim3 grid;
  if (g.tri)
    grid = dim3((unsigned)(tm * (tm + 1) / 2), 1, (unsigned)g.batch);
  else if (g.order)
    grid = dim3((unsigned)(tm * tn), 1, (unsigned)g.batch);
  else
    grid = dim3((unsigned)tn, (unsigned)tm, (unsigned)g.batch);
  if (g.b_kmajor)
    hipLaunchKernelGGL((k_gemm_f32<TM, true>), grid, dim3(256), 0, stream, g);
  else
    hipLaunchKernelGGL((k_gemm_f32<TM, false>), grid, dim3(256), 0, stream, g);
  return hipGetLastError();
}

}  // namespace

hipError_t gemm_f32(const GemmF32& g_in, hipStream_t stream) {
  GemmF32 g = g_in;
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return hipSuccess;
  // triangular K ranges: small tiles, longest K first, to balance the round
  if (!g.tri && g.C != g.A && (g.klo_n || g.khi_m)) {
    g.order = g.klo_n ? 1 : 2;
    return launch<64>(g, stream);
  }
  const int64_t tm = (g.M + 127) / 128, tn = (g.N + 127) / 128;
  const int64_t tiles = (g.tri ? tm * (tm + 1) / 2 : tm * tn) * g.batch;
  // In place (C is A, as in the factor's panel product): a tile reads whole
  // rows of A before it writes, so one tile must span all of N.
  if (g.C == g.A) return g.N <= 128 ? launch<128>(g, stream) : hipErrorInvalidValue;
  // fewer 128-tiles than compute units: quarter the tile
  if (tiles < 256) return launch<64>(g, stream);
  return launch<128>(g, stream);
}

}  // namespace gptq
