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
// goes through three register passes of four bits each (a thread holds 16
// elements whose indices differ in four of the bits), and the elements move
// between passes through padded LDS.  Aligned rows enter and leave in 16-byte
// (fp32) or 8-byte (bf16) vectors per lane, others element by element; both are
// coalesced.  The sign is applied on load and 1/sqrt(b) on store.  HBM-bound.
//
// Hessian.  H Q row-wise, an in-place transpose (tile pairs), Q^T H Q row-wise
// again (H^T = H), then the upper triangle mirrored into the lower so the
// result is exactly symmetric.
#include "common.h"

namespace gptq {
namespace {

constexpr int HCH = 4096;  // elements per chunk

__device__ __forceinline__ float to_f32(const float* p, int i) { return p[i]; }
__device__ __forceinline__ float to_f32(const uint16_t* p, int i) { return __uint_as_float((uint32_t)p[i] << 16); }

// Butterflies on the four register-index bits; register bit r stands for
// element-index bit eb[r], and only element bits below kb (= log2 b) take part.
__device__ __forceinline__ void stages16(float (&v)[16], int eb0, int eb1, int eb2, int eb3, int kb) {
  const int eb[4] = {eb0, eb1, eb2, eb3};
#pragma unroll
  for (int bit = 0; bit < 4; ++bit) {
    if (eb[bit] < kb) {
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

// Scalar form: any alignment.  A thread's 16 elements differ in element bits
// 8-11, then 4-7, then 0-3; LDS index e + e / 16.
template <typename InT>
__device__ __forceinline__ void chunk_scalar(const InT* src, float* dst, const float* sg, int m, int kb, float scale,
                                             float* buf) {
  const int t = threadIdx.x;
  auto li = [](int e) { return e + (e >> 4); };
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = t + 256 * i;
    v[i] = e < m ? to_f32(src, e) * sg[e] : 0.0f;
  }
  stages16(v, 8, 9, 10, 11, kb);
#pragma unroll
  for (int i = 0; i < 16; ++i) buf[li(t + 256 * i)] = v[i];
  __syncthreads();
  // each slot below is read and rewritten by the one thread that owns it
  const int eb = (t & 15) + 256 * (t >> 4);
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = buf[li(eb + 16 * i)];
  stages16(v, 4, 5, 6, 7, kb);
#pragma unroll
  for (int i = 0; i < 16; ++i) buf[li(eb + 16 * i)] = v[i];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = buf[li(16 * t + i)];
  stages16(v, 0, 1, 2, 3, kb);
#pragma unroll
  for (int i = 0; i < 16; ++i) buf[li(16 * t + i)] = v[i];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = t + 256 * i;
    if (e < m) dst[e] = buf[li(e)] * scale;
  }
}

typedef float f32x4a __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4a __attribute__((ext_vector_type(4)));

// Vector form: rows 16-byte (fp32) or 8-byte (bf16) aligned, m a multiple of 4.
// A thread's 16 elements are 4 consecutive ones in each of 4 segments 1024
// apart (element bits 0-1 and 10-11), then differ in bits 2-5, then 6-9; the
// chunk enters and leaves in whole vectors.  LDS index e + 4 (e / 64) keeps
// each group of 4 contiguous and 16-byte aligned.
template <typename InT>
__device__ __forceinline__ void chunk_vector(const InT* src, float* dst, const float* sg, int m, int kb, float scale,
                                             float* buf) {
  const int t = threadIdx.x;
  auto li = [](int e) { return e + 4 * (e >> 6); };
  float v[16];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * t + 1024 * j;
    if (e < m) {
      float a[4];
      if constexpr (sizeof(InT) == 4) {
        const f32x4a x = *reinterpret_cast<const f32x4a*>(src + e);
        a[0] = x.x; a[1] = x.y; a[2] = x.z; a[3] = x.w;
      } else {
        const u16x4a x = *reinterpret_cast<const u16x4a*>(src + e);
        a[0] = __uint_as_float((uint32_t)x.x << 16); a[1] = __uint_as_float((uint32_t)x.y << 16);
        a[2] = __uint_as_float((uint32_t)x.z << 16); a[3] = __uint_as_float((uint32_t)x.w << 16);
      }
      const f32x4a d = *reinterpret_cast<const f32x4a*>(sg + e);
      v[4 * j] = a[0] * d.x; v[4 * j + 1] = a[1] * d.y; v[4 * j + 2] = a[2] * d.z; v[4 * j + 3] = a[3] * d.w;
    } else {
      v[4 * j] = v[4 * j + 1] = v[4 * j + 2] = v[4 * j + 3] = 0.0f;
    }
  }
  stages16(v, 0, 1, 10, 11, kb);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    *reinterpret_cast<float4*>(buf + li(4 * t + 1024 * j)) = make_float4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
  __syncthreads();
  // register bits = element bits 2-5; thread = bits 0-1 and 6-11
  const int e2 = (t & 3) + 64 * (t >> 2);
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = buf[li(e2 + 4 * i)];
  stages16(v, 2, 3, 4, 5, kb);
#pragma unroll
  for (int i = 0; i < 16; ++i) buf[li(e2 + 4 * i)] = v[i];
  __syncthreads();
  // register bits = element bits 6-9; thread = bits 0-5 and 10-11
  const int e3 = (t & 63) + 1024 * (t >> 6);
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = buf[li(e3 + 64 * i)];
  stages16(v, 6, 7, 8, 9, kb);
#pragma unroll
  for (int i = 0; i < 16; ++i) buf[li(e3 + 64 * i)] = v[i];
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * t + 1024 * j;
    if (e < m) {
      const float4 r = *reinterpret_cast<const float4*>(buf + li(e));
      *reinterpret_cast<float4*>(dst + e) = make_float4(r.x * scale, r.y * scale, r.z * scale, r.w * scale);
    }
  }
}

template <typename InT, bool VEC>
__global__ __launch_bounds__(256) void k_hadamard_rows(const InT* in, int64_t ld_in, float* out, int64_t ld_out,
                                                       int64_t n, int64_t nchunk, const float* __restrict__ signs,
                                                       int kb, float scale) {
  __shared__ __align__(16) float buf[HCH + HCH / 16];
  const int64_t row = blockIdx.x / nchunk;
  const int64_t c0 = ((int64_t)blockIdx.x - row * nchunk) * HCH;
  const int m = (int)(n - c0 < HCH ? n - c0 : HCH);  // valid elements; a multiple of b
  if constexpr (VEC)
    chunk_vector(in + row * ld_in + c0, out + row * ld_out + c0, signs + c0, m, kb, scale, buf);
  else
    chunk_scalar(in + row * ld_in + c0, out + row * ld_out + c0, signs + c0, m, kb, scale, buf);
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

// The same, with whole 16-byte vectors in global memory (n % 4 == 0, H 16-byte
// aligned): a tile row is 16 float4, each staged into or out of LDS element by
// element, so the transposed LDS reads stay on the padded column layout.
__global__ __launch_bounds__(256) void k_tile_pairs4(float* H, int64_t n, int mode) {
  const int bi = blockIdx.y, bj = blockIdx.x;
  if (bi > bj) return;
  __shared__ float ta[64][65], tb[64][65];
  const int64_t r0 = (int64_t)bi * 64, c0 = (int64_t)bj * 64;
  const bool two = mode == 0 && bi != bj;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int idx = threadIdx.x + 256 * it, r = idx >> 4, c4 = 4 * (idx & 15);
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r0 + r < n && c0 + c4 < n) v = *reinterpret_cast<const float4*>(H + (r0 + r) * n + c0 + c4);
    ta[r][c4] = v.x; ta[r][c4 + 1] = v.y; ta[r][c4 + 2] = v.z; ta[r][c4 + 3] = v.w;
    if (two) {
      float4 w = make_float4(0.f, 0.f, 0.f, 0.f);
      if (c0 + r < n && r0 + c4 < n) w = *reinterpret_cast<const float4*>(H + (c0 + r) * n + r0 + c4);
      tb[r][c4] = w.x; tb[r][c4 + 1] = w.y; tb[r][c4 + 2] = w.z; tb[r][c4 + 3] = w.w;
    }
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int idx = threadIdx.x + 256 * it, rr = idx >> 4, c4 = 4 * (idx & 15);
    if (mode == 0) {
      if (bi == bj) {
        if (r0 + rr < n && r0 + c4 < n)
          *reinterpret_cast<float4*>(H + (r0 + rr) * n + r0 + c4) =
              make_float4(ta[c4][rr], ta[c4 + 1][rr], ta[c4 + 2][rr], ta[c4 + 3][rr]);
      } else {
        if (r0 + rr < n && c0 + c4 < n)
          *reinterpret_cast<float4*>(H + (r0 + rr) * n + c0 + c4) =
              make_float4(tb[c4][rr], tb[c4 + 1][rr], tb[c4 + 2][rr], tb[c4 + 3][rr]);
        if (c0 + rr < n && r0 + c4 < n)
          *reinterpret_cast<float4*>(H + (c0 + rr) * n + r0 + c4) =
              make_float4(ta[c4][rr], ta[c4 + 1][rr], ta[c4 + 2][rr], ta[c4 + 3][rr]);
      }
    } else {
      // lower-tile element (c0 + rr, r0 + c4 + e) = upper element (r0 + c4 + e, c0 + rr)
      const int64_t gr = c0 + rr, gc = r0 + c4;
      if (gr >= n || gc >= n) continue;
      if (bi != bj) {
        *reinterpret_cast<float4*>(H + gr * n + gc) =
            make_float4(ta[c4][rr], ta[c4 + 1][rr], ta[c4 + 2][rr], ta[c4 + 3][rr]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (gr > gc + e) H[gr * n + gc + e] = ta[c4 + e][rr];
      }
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
  const int64_t esz = in_bf16 ? 2 : 4;
  auto al = [](const void* p, int64_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; };
  // whole vectors: every row start aligned, and a chunk's valid length a multiple of 4
  const bool vec = n % 4 == 0 && al(in, 4 * esz) && (ld_in * esz) % (4 * esz) == 0 && al(out, 16) &&
                   (ld_out * 4) % 16 == 0 && al(signs, 16);
  if (in_bf16) {
    const uint16_t* p = static_cast<const uint16_t*>(in);
    if (vec)
      hipLaunchKernelGGL((k_hadamard_rows<uint16_t, true>), dim3(grid), dim3(256), 0, stream, p, ld_in, out, ld_out,
                         n, nchunk, signs, kb, scale);
    else
      hipLaunchKernelGGL((k_hadamard_rows<uint16_t, false>), dim3(grid), dim3(256), 0, stream, p, ld_in, out,
                         ld_out, n, nchunk, signs, kb, scale);
  } else {
    const float* p = static_cast<const float*>(in);
    if (vec)
      hipLaunchKernelGGL((k_hadamard_rows<float, true>), dim3(grid), dim3(256), 0, stream, p, ld_in, out, ld_out, n,
                         nchunk, signs, kb, scale);
    else
      hipLaunchKernelGGL((k_hadamard_rows<float, false>), dim3(grid), dim3(256), 0, stream, p, ld_in, out, ld_out,
                         n, nchunk, signs, kb, scale);
  }
  return hipGetLastError();
}

hipError_t hadamard_hessian(float* H, int64_t n, const float* signs, int block, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const unsigned nb = (unsigned)((n + 63) / 64);
  hipError_t e = hadamard_rows(H, false, n, H, n, n, n, signs, block, stream);  // H Q
  if (e != hipSuccess) return e;
  const bool vec = n % 4 == 0 && (reinterpret_cast<uintptr_t>(H) & 15) == 0;
  auto pairs = [&](int mode) {
    if (vec)
      hipLaunchKernelGGL(k_tile_pairs4, dim3(nb, nb), dim3(256), 0, stream, H, n, mode);
    else
      hipLaunchKernelGGL(k_tile_pairs, dim3(nb, nb), dim3(256), 0, stream, H, n, mode);
    return hipGetLastError();
  };
  if ((e = pairs(0)) != hipSuccess) return e;  // Q^T H
  e = hadamard_rows(H, false, n, H, n, n, n, signs, block, stream);  // Q^T H Q
  if (e != hipSuccess) return e;
  if ((e = pairs(1)) != hipSuccess) return e;  // exact symmetry
  return hipGetLastError();
}

}  // namespace gptq
