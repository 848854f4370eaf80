// Code packing: per row one little-endian bitstream of b-bit codes cut into
// 32-bit words (code i in stream bits [i*b, (i+1)*b)).  One thread turns a run
// of 32 codes (32 bytes) into b words, so every run starts on a word boundary;
// consecutive threads write consecutive words of a row.
#include "common.h"

namespace gptq {
namespace {

template <int BITS>
__global__ void k_pack(const uint8_t* codes, int64_t rows, int64_t cols, uint32_t* packed) {
  const int64_t runs = (cols + 31) / 32;
  const int64_t words_per_row = cols * BITS / 32;
  const int64_t total = rows * runs;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total; u += stride) {
    const int64_t r = u / runs, run = u % runs;
    const int64_t c0 = run * 32;
    const int nc = (int)((cols - c0) < 32 ? (cols - c0) : 32);
    const uint8_t* src = codes + r * cols + c0;
    uint32_t c[32];
    if (nc == 32 && (cols & 15) == 0) {
      const uint4 a = reinterpret_cast<const uint4*>(src)[0];
      const uint4 b = reinterpret_cast<const uint4*>(src)[1];
      const uint32_t v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 32; ++i) c[i] = (v[i >> 2] >> (8 * (i & 3))) & 0xffu;
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) c[i] = i < nc ? src[i] : 0u;
    }
    uint32_t w[BITS];
#pragma unroll
    for (int k = 0; k < BITS; ++k) w[k] = 0u;
    constexpr uint32_t mask = (1u << BITS) - 1u;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t v = c[i] & mask;
      const int bit = i * BITS;
      w[bit >> 5] |= v << (bit & 31);
      if ((bit & 31) + BITS > 32) w[(bit >> 5) + 1] |= v >> (32 - (bit & 31));
    }
    uint32_t* dst = packed + r * words_per_row + run * BITS;
    const int nw = (nc * BITS + 31) / 32;
#pragma unroll
    for (int k = 0; k < BITS; ++k)
      if (k < nw) dst[k] = w[k];
  }
}

}  // namespace

hipError_t pack_launch(const uint8_t* codes, int64_t rows, int64_t cols, int bits, uint32_t* packed,
                       hipStream_t stream) {
  const int64_t total = rows * ((cols + 31) / 32);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  const dim3 grid((unsigned)blocks), block(256);
  switch (bits) {
    case 2: hipLaunchKernelGGL(k_pack<2>, grid, block, 0, stream, codes, rows, cols, packed); break;
    case 3: hipLaunchKernelGGL(k_pack<3>, grid, block, 0, stream, codes, rows, cols, packed); break;
    case 4: hipLaunchKernelGGL(k_pack<4>, grid, block, 0, stream, codes, rows, cols, packed); break;
    case 8: hipLaunchKernelGGL(k_pack<8>, grid, block, 0, stream, codes, rows, cols, packed); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gptq
