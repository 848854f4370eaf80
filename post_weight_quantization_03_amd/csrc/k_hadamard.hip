// Fixed randomised Hadamard rotation Q = D blockdiag(H_b, ..., H_b) / sqrt(b)
// (D = diag(signs), H_b the Sylvester Hadamard matrix, b a power of two that
// divides n): rows A -> A Q for weights and activations, and H -> Q^T H Q for
// the Hessian (OneComp hub article, rotation preprocessing and the Hadamard
// transform of its pre-processing package; the pages leave the rotation itself
// open, this is the fixed, untrained one).
//
// Row transform.  A workgroup takes a chunk of 4096 consecutive elements of a
// row (chunks start at multiples of 4096, so every b-block lies in one chunk).
// The Walsh-Hadamard transform of order b is a butterfly on each of the low
// log2 b bits of the element index, and those butterflies commute, so the chunk
// goes through three register passes of four bits each: a thread holds 16
// elements whose indices differ exactly in bits 8-11, then 4-7, then 0-3, and
// the elements move between passes through LDS (one pad word per 16 keeps the
// strided reads on distinct banks).  Loads and stores are coalesced; the sign
// is applied on load and 1/sqrt(b) on store.  HBM-bound.
//
// Hessian.  H Q row-wise, an in-place transpose (tile pairs), Q^T H Q row-wise
// again (H^T = H), then the upper triangle mirrored into the lower so the
// result is exactly symmetric.
#include "common.h"

namespace gptq {
namespace {

constexpr int HCH = 4096;  // elements per chunk

__device__ __forceinline__ int lidx(int e) { return e + (e >> 4); }

__device__ __forceinline__ float to_f32(const float* p, int i) { return p[i]; }
__device__ __forceinline__ float to_f32(const uint16_t* p, int i) { return __uint_as_float((uint32_t)p[i] << 16); }

// Butterflies on register-index bits 0-3, which stand for element-index bits
// base..base+3; only the element bits below kb (= log2 b) take part.
__device__ __forceinline__ void stages16(float (&v)[16], int base, int kb) {
#pragma unroll
  for (int bit = 0; bit < 4; ++bit) {
    if (base + bit < kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (!(i & (1 << bit))) {
          const float a = v[i], c = v[i | (1 << bit)];
          v[i] = a + c;
          v[i | (1 << bit)] = a - c;
        }
      }
    }
  }
}

template <typename InT>
__global__ __launch_bounds__(256) void k_hadamard_rows(const InT* in, int64_t ld_in, float* out, int64_t ld_out,
                                                       int64_t n, int64_t nchunk, const float* __restrict__ signs,
                                                       int kb, float scale) {
  __shared__ float buf[HCH + HCH / 16];
  const int t = threadIdx.x;
  const int64_t row = blockIdx.x / nchunk;
  const int64_t c0 = ((int64_t)blockIdx.x - row * nchunk) * HCH;
  const InT* src = in + row * ld_in + c0;
  float* dst = out + row * ld_out + c0;
  const int m = (int)(n - c0 < HCH ? n - c0 : HCH);  // valid elements; a multiple of b
  float v[16];
  // element t + 256 i: register index = element bits 8-11
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = t + 256 * i;
    v[i] = e < m ? to_f32(src, e) * signs[c0 + e] : 0.0f;
  }
  stages16(v, 8, kb);
#pragma unroll
  for (int i = 0; i < 16; ++i) buf[lidx(t + 256 * i)] = v[i];
  __syncthreads();
  // element (t & 15) + 16 i + 256 (t >> 4): register index = element bits 4-7.
  // Each slot is read and rewritten by the one thread that owns it here.
  const int eb = (t & 15) + 256 * (t >> 4);
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = buf[lidx(eb + 16 * i)];
  stages16(v, 4, kb);
#pragma unroll
  for (int i = 0; i < 16; ++i) buf[lidx(eb + 16 * i)] = v[i];
  __syncthreads();
  // element 16 t + i: register index = element bits 0-3
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = buf[lidx(16 * t + i)];
  stages16(v, 0, kb);
#pragma unroll
  for (int i = 0; i < 16; ++i) buf[lidx(16 * t + i)] = v[i];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = t + 256 * i;
    if (e < m) dst[e] = buf[lidx(e)] * scale;
  }
}

// Tile pairs of a square matrix, one workgroup per unordered pair of 64 x 64
// tiles {(bi, bj), (bj, bi)}, bi <= bj.  mode 0: H := H^T in place.  mode 1:
// the strictly lower triangle := the upper one, mirrored.
__global__ __launch_bounds__(256) void k_tile_pairs(float* H, int64_t n, int mode) {
  const int bi = blockIdx.y, bj = blockIdx.x;
  if (bi > bj) return;
  __shared__ float ta[64][65], tb[64][65];
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int64_t r0 = (int64_t)bi * 64, c0 = (int64_t)bj * 64;
  for (int r = ty; r < 64; r += 4) {  // upper tile: ta[r][c] = H[r0 + r][c0 + c]
    const int64_t gr = r0 + r, gc = c0 + tx;
    ta[r][tx] = (gr < n && gc < n) ? H[gr * n + gc] : 0.0f;
  }
  if (mode == 0 && bi != bj) {
    for (int r = ty; r < 64; r += 4) {  // lower tile: tb[r][c] = H[c0 + r][r0 + c]
      const int64_t gr = c0 + r, gc = r0 + tx;
      tb[r][tx] = (gr < n && gc < n) ? H[gr * n + gc] : 0.0f;
    }
  }
  __syncthreads();
  for (int r = ty; r < 64; r += 4) {
    if (mode == 0) {
      if (bi == bj) {
        const int64_t gr = r0 + r, gc = r0 + tx;
        if (gr < n && gc < n) H[gr * n + gc] = ta[tx][r];
      } else {
        int64_t gr = r0 + r, gc = c0 + tx;
        if (gr < n && gc < n) H[gr * n + gc] = tb[tx][r];
        gr = c0 + r;
        gc = r0 + tx;
        if (gr < n && gc < n) H[gr * n + gc] = ta[tx][r];
      }
    } else {
      const int64_t gr = c0 + r, gc = r0 + tx;  // lower-tile element = upper element (gc, gr)
      if (gr < n && gc < n && (bi != bj || gr > gc)) H[gr * n + gc] = ta[tx][r];
    }
  }
}

int log2_exact(int b) {
  int k = 0;
  while ((1 << k) < b) ++k;
  return k;
}

}  // namespace

int64_t hadamard_chunks(int64_t n) { return (n + HCH - 1) / HCH; }

hipError_t hadamard_rows(const void* in, bool in_bf16, int64_t ld_in, float* out, int64_t ld_out, int64_t rows,
                         int64_t n, const float* signs, int block, hipStream_t stream) {
  if (rows <= 0 || n <= 0) return hipSuccess;
  const int64_t nchunk = hadamard_chunks(n);
  const unsigned grid = (unsigned)(rows * nchunk);
  const int kb = log2_exact(block);
  const float scale = (float)(1.0 / std::sqrt((double)block));
  if (in_bf16)
    hipLaunchKernelGGL(k_hadamard_rows<uint16_t>, dim3(grid), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(in), ld_in, out, ld_out, n, nchunk, signs, kb, scale);
  else
    hipLaunchKernelGGL(k_hadamard_rows<float>, dim3(grid), dim3(256), 0, stream, static_cast<const float*>(in),
                       ld_in, out, ld_out, n, nchunk, signs, kb, scale);
  return hipGetLastError();
}

hipError_t hadamard_hessian(float* H, int64_t n, const float* signs, int block, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const unsigned nb = (unsigned)((n + 63) / 64);
  hipError_t e = hadamard_rows(H, false, n, H, n, n, n, signs, block, stream);  // H Q
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_tile_pairs, dim3(nb, nb), dim3(256), 0, stream, H, n, 0);  // Q^T H
  if ((e = hipGetLastError()) != hipSuccess) return e;
  e = hadamard_rows(H, false, n, H, n, n, n, signs, block, stream);  // Q^T H Q
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_tile_pairs, dim3(nb, nb), dim3(256), 0, stream, H, n, 1);  // exact symmetry
  return hipGetLastError();
}

}  // namespace gptq
