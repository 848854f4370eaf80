// C ABI of libgptq.so: argument checks on the host, workspace carving and the
// launch sequence of each entry point.  Every declaration is documented in
// include/gptq.h.
#include <mutex>

#include "common.h"

namespace {

using namespace gptq;

constexpr int VERSION = 100;  // 0.1.0
constexpr int64_t MAX_DIM = (int64_t)1 << 30;

struct QuantLayout {
  size_t status, lam, dead, loss, Wf, E, Us, A, Lt, total;
};

bool params_ok(const gptq_params* p, int64_t cols, int* why) {
  if (!p) return (*why = GPTQ_EINVAL), false;
  if (!(p->bits == 2 || p->bits == 3 || p->bits == 4 || p->bits == 8)) return (*why = GPTQ_EINVAL), false;
  if (!(p->damp >= 0.0f) || !(p->damp < INFINITY)) return (*why = GPTQ_EINVAL), false;
  if (p->flags & ~(GPTQ_H_IS_FACTOR | GPTQ_FACTOR_F64)) return (*why = GPTQ_EINVAL), false;
  if (p->groupsize == 0 || p->groupsize < -1) return (*why = GPTQ_EINVAL), false;
  if (p->blocksize != 128) return (*why = GPTQ_EUNSUPPORTED), false;
  const int64_t g = p->groupsize;
  if (!(g == -1 || g == 32 || g == 64 || g % 128 == 0)) return (*why = GPTQ_EUNSUPPORTED), false;
  if ((p->flags & GPTQ_H_IS_FACTOR) && cols < 3) return (*why = GPTQ_EINVAL), false;
  return true;
}

QuantLayout layout(int64_t rows, int64_t cols, const gptq_params* p) {
  QuantLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, 256);
    return at;
  };
  L.status = take(4 * sizeof(int));
  L.lam = take(sizeof(double));
  L.dead = take((size_t)cols);
  L.loss = take((size_t)rows * sizeof(float));
  L.Wf = take((size_t)rows * cols * sizeof(float));
  L.E = take((size_t)rows * ((cols + 127) / 128) * 128 * sizeof(float));  // every block's errors
  {
    const size_t ub = quant_split_bytes(cols, p->groupsize == -1 ? cols : p->groupsize);
    L.Us = ub ? take(ub) : 0;
  }
  if (!(p->flags & GPTQ_H_IS_FACTOR)) {
    if (p->flags & GPTQ_FACTOR_F64) {
      L.A = take((size_t)cols * cols * sizeof(double));
      L.Lt = take(factor64_scratch_doubles(cols) * sizeof(double));
    } else {
      L.A = take((size_t)cols * cols * sizeof(float));
      L.Lt = take(factor_scratch_floats(cols) * sizeof(float));
    }
  }
  L.total = off;
  return L;
}

}  // namespace

extern "C" {

const char* gptq_status_string(int status) {
  switch (status) {
    case GPTQ_OK: return "ok";
    case GPTQ_EINVAL: return "invalid argument";
    case GPTQ_ENOTPD: return "damped Hessian is not positive definite";
    case GPTQ_EWORKSPACE: return "workspace too small";
    case GPTQ_EUNSUPPORTED: return "unsupported parameter combination";
    case GPTQ_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int gptq_version(void) { return VERSION; }

int gptq_trace_set(void* buf) {
#ifdef GPTQ_TRACE
  auto* p = static_cast<unsigned long long*>(buf);
  if (gptq::trace_set_factor(p) != hipSuccess || gptq::trace_set_quant(p) != hipSuccess ||
      gptq::trace_set_mma(p) != hipSuccess)
    return GPTQ_EHIP;
  return GPTQ_OK;
#else
  (void)buf;
  return GPTQ_EUNSUPPORTED;
#endif
}

size_t gptq_hessian_workspace_bytes(int64_t n, int64_t tokens, gptq_dtype x_dtype) {
  if (n <= 0 || tokens <= 0 || n > MAX_DIM || tokens > MAX_DIM) return 0;
  return hessian_workspace(n, tokens, x_dtype);
}

int gptq_accumulate_hessian(float* H, int64_t n, const void* X, gptq_dtype x_dtype, int64_t tokens, int64_t ldx,
                            void* workspace, size_t workspace_bytes, gptq_stream_t stream) {
  if (n < 0 || tokens < 0 || n > MAX_DIM || tokens > MAX_DIM) return GPTQ_EINVAL;
  if (!(x_dtype == GPTQ_BF16 || x_dtype == GPTQ_F32)) return GPTQ_EINVAL;
  if (n == 0 || tokens == 0) return GPTQ_OK;
  if (!H || !X || ldx < n) return GPTQ_EINVAL;
  if (n * n > ((int64_t)1 << 31) * 2) return GPTQ_EUNSUPPORTED;
  const size_t need = hessian_workspace(n, tokens, x_dtype);
  if (workspace_bytes < need || (need > 0 && !workspace)) return GPTQ_EWORKSPACE;
  return hessian_launch(H, n, X, x_dtype, tokens, ldx, workspace, workspace_bytes, (hipStream_t)stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Hessian accumulation without allocation: the split-K partial tiles go to this
// fixed array instead of a caller workspace.  The name is a host-side stand-in
// for the device symbol: host code uses only the per-device address that
// hipGetSymbolAddress returns.
static __device__ __align__(256) unsigned char scratch[GPTQ_HESSIAN_STATIC_BYTES];

namespace {

constexpr int MAX_DEVICES = 256;
std::mutex scratch_mu;
void* scratch_addr[MAX_DEVICES] = {};

// The current device's address of `scratch`, taken once per device with that
// device current.
int scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return GPTQ_EHIP;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return GPTQ_EHIP;
    scratch_addr[dev] = p;
  }
  *out = scratch_addr[dev];
  return GPTQ_OK;
}

}  // namespace

extern "C" {

int gptq_accumulate_hessian_static(float* H, int64_t n, const void* X, gptq_dtype x_dtype, int64_t tokens,
                                   int64_t ldx, gptq_stream_t stream) {
  if (n < 0 || tokens < 0 || n > MAX_DIM || tokens > MAX_DIM) return GPTQ_EINVAL;
  if (!(x_dtype == GPTQ_BF16 || x_dtype == GPTQ_F32)) return GPTQ_EINVAL;
  if (n == 0 || tokens == 0) return GPTQ_OK;
  if (!H || !X || ldx < n) return GPTQ_EINVAL;
  if (n * n > ((int64_t)1 << 31) * 2) return GPTQ_EUNSUPPORTED;
  const size_t need = hessian_workspace(n, tokens, x_dtype);
  if (need > GPTQ_HESSIAN_STATIC_BYTES) return GPTQ_EWORKSPACE;
  if (stream) {
    int cur = -1, sdev = -1;
    if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess)
      return GPTQ_EHIP;
    if (cur != sdev) return GPTQ_EINVAL;
  }
  void* ws = nullptr;
  const int st = scratch_ptr(&ws);
  if (st != GPTQ_OK) return st;
  return hessian_launch(H, n, X, x_dtype, tokens, ldx, ws, GPTQ_HESSIAN_STATIC_BYTES, (hipStream_t)stream);
}

size_t gptq_quantize_workspace_bytes(int64_t rows, int64_t cols, const gptq_params* p) {
  int why = 0;
  if (rows <= 0 || cols <= 0 || rows > MAX_DIM || cols > MAX_DIM || !params_ok(p, cols, &why)) return 0;
  return layout(rows, cols, p).total;
}

int gptq_quantize_layer(const void* W, gptq_dtype w_dtype, int64_t rows, int64_t cols, float* H,
                        const gptq_params* p, uint8_t* codes, float* scales, uint8_t* zeros, float* w_hat,
                        float* row_loss, void* workspace, size_t workspace_bytes, int32_t* d_status,
                        gptq_stream_t stream_) {
  hipStream_t stream = (hipStream_t)stream_;
  if (rows < 0 || cols < 0 || rows > MAX_DIM || cols > MAX_DIM) return GPTQ_EINVAL;
  if (!(w_dtype == GPTQ_BF16 || w_dtype == GPTQ_F32)) return GPTQ_EINVAL;
  int why = GPTQ_EINVAL;
  if (!params_ok(p, cols, &why)) return why;
  if (rows == 0 || cols == 0) return GPTQ_OK;
  if (!W || !H || !codes || !scales || !zeros || !workspace) return GPTQ_EINVAL;
  if (cols > 65535 * 4 || rows * cols > ((int64_t)1 << 40)) return GPTQ_EUNSUPPORTED;
  const QuantLayout L = layout(rows, cols, p);
  if (workspace_bytes < L.total) return GPTQ_EWORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return GPTQ_EINVAL;

  char* ws = static_cast<char*>(workspace);
  int* status = reinterpret_cast<int*>(ws + L.status);
  uint8_t* dead = reinterpret_cast<uint8_t*>(ws + L.dead);
  const int64_t g = p->groupsize == -1 ? cols : p->groupsize;
  const int64_t G = (cols + g - 1) / g;

  // the row loss is always accumulated; without a caller buffer it lands in the workspace
  float* loss = row_loss ? row_loss : reinterpret_cast<float*>(ws + L.loss);

  hipError_t e = fill_i32(status, 1, GPTQ_OK, stream);
  if (e != hipSuccess) return GPTQ_EHIP;
  if (p->flags & GPTQ_H_IS_FACTOR) {
    e = dead_from_factor(H, cols, dead, stream);
  } else if (p->flags & GPTQ_FACTOR_F64) {
    Factor64Ws f{};
    f.status = status;
    f.lam = reinterpret_cast<double*>(ws + L.lam);
    f.dead = dead;
    f.A = reinterpret_cast<double*>(ws + L.A);
    f.Lt = reinterpret_cast<double*>(ws + L.Lt);
    e = factor64_run(H, cols, p->damp, f, stream);
  } else {
    FactorWs f{};
    f.status = status;
    f.lam = reinterpret_cast<float*>(ws + L.lam);
    f.dead = dead;
    f.A = reinterpret_cast<float*>(ws + L.A);
    f.Lt = reinterpret_cast<float*>(ws + L.Lt);
    e = factor_run(H, cols, p->damp, f, stream);
  }
  if (e != hipSuccess) return GPTQ_EHIP;

  QuantArgs q{};
  q.W = W;
  q.w_dtype = w_dtype;
  q.rows = rows;
  q.cols = cols;
  q.U = H;
  q.dead = dead;
  q.bits = p->bits;
  q.groupsize = (int)g;
  q.codes = codes;
  q.scales = scales;
  q.zeros = zeros;
  q.w_hat = w_hat;
  q.row_loss = loss;
  q.Wf = reinterpret_cast<float*>(ws + L.Wf);
  q.E = reinterpret_cast<float*>(ws + L.E);
  q.Usplit = quant_split_bytes(cols, g) ? reinterpret_cast<uint16_t*>(ws + L.Us) : nullptr;
  q.G = G;
  e = quant_run(q, stream);
  if (e != hipSuccess) return GPTQ_EHIP;

  if (d_status) {
    e = copy_status(status, d_status, stream);
    return e == hipSuccess ? GPTQ_OK : GPTQ_EHIP;
  }
  int host = 0;
  if (hipMemcpyAsync(&host, status, sizeof(int), hipMemcpyDeviceToHost, stream) != hipSuccess) return GPTQ_EHIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return GPTQ_EHIP;
  return host;
}

int gptq_pack(const uint8_t* codes, int64_t rows, int64_t cols, int32_t bits, uint32_t* packed,
              gptq_stream_t stream) {
  if (rows < 0 || cols < 0 || rows > MAX_DIM || cols > MAX_DIM) return GPTQ_EINVAL;
  if (!(bits == 2 || bits == 3 || bits == 4 || bits == 8)) return GPTQ_EINVAL;
  if ((cols * bits) % 32 != 0) return GPTQ_EINVAL;
  if (rows == 0 || cols == 0) return GPTQ_OK;
  if (!codes || !packed) return GPTQ_EINVAL;
  return pack_launch(codes, rows, cols, bits, packed, (hipStream_t)stream) == hipSuccess ? GPTQ_OK : GPTQ_EHIP;
}

int gptq_dequant_gemv(const uint32_t* packed, const float* scales, const uint8_t* zeros, int64_t rows,
                      int64_t cols, int32_t bits, int32_t groupsize, const void* x, gptq_dtype x_dtype, float* y,
                      gptq_stream_t stream) {
  if (rows < 0 || cols < 0 || rows > MAX_DIM || cols > MAX_DIM) return GPTQ_EINVAL;
  if (!(bits == 2 || bits == 3 || bits == 4 || bits == 8)) return GPTQ_EINVAL;
  if (groupsize == 0 || groupsize < -1) return GPTQ_EINVAL;
  if (x_dtype != GPTQ_BF16 && x_dtype != GPTQ_F32) return GPTQ_EINVAL;
  if ((cols * bits) % 32 != 0) return GPTQ_EINVAL;
  if (!dequant_gemv_supported(cols, bits, groupsize)) return GPTQ_EUNSUPPORTED;
  if (rows == 0) return GPTQ_OK;
  if (!y || (cols > 0 && (!packed || !scales || !zeros || !x))) return GPTQ_EINVAL;
  auto misaligned = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3) != 0; };
  if (misaligned(packed) || misaligned(scales) || misaligned(x) || misaligned(y)) return GPTQ_EINVAL;
  return dequant_gemv(packed, scales, zeros, rows, cols, bits, groupsize, x, x_dtype == GPTQ_BF16, y,
                      (hipStream_t)stream) == hipSuccess
             ? GPTQ_OK
             : GPTQ_EHIP;
}

size_t gptq_dequant_gemm_workspace_bytes(int64_t rows, int64_t cols, int32_t bits, int32_t groupsize,
                                        int64_t batch) {
  if (rows <= 0 || cols <= 0 || batch <= 0 || rows > MAX_DIM || cols > MAX_DIM || batch > MAX_DIM) return 0;
  if (!dequant_gemv_supported(cols, bits, groupsize) || !dequant_mma_supported(cols, groupsize, batch)) return 0;
  return dequant_mma_workspace(rows, cols, batch);
}

int gptq_dequant_gemm(const uint32_t* packed, const float* scales, const uint8_t* zeros, int64_t rows,
                      int64_t cols, int32_t bits, int32_t groupsize, const void* X, gptq_dtype x_dtype, int64_t ldx,
                      int64_t batch, float* Y, int64_t ldy, void* workspace, size_t workspace_bytes,
                      gptq_stream_t stream) {
  if (rows < 0 || cols < 0 || batch < 0 || rows > MAX_DIM || cols > MAX_DIM || batch > MAX_DIM) return GPTQ_EINVAL;
  if (!(bits == 2 || bits == 3 || bits == 4 || bits == 8)) return GPTQ_EINVAL;
  if (groupsize == 0 || groupsize < -1) return GPTQ_EINVAL;
  if (x_dtype != GPTQ_BF16 && x_dtype != GPTQ_F32) return GPTQ_EINVAL;
  if ((cols * bits) % 32 != 0) return GPTQ_EINVAL;
  if (!dequant_gemv_supported(cols, bits, groupsize)) return GPTQ_EUNSUPPORTED;
  if (rows == 0 || batch == 0) return GPTQ_OK;
  if (ldx < cols || ldy < rows) return GPTQ_EINVAL;
  if (!Y || (cols > 0 && (!packed || !scales || !zeros || !X))) return GPTQ_EINVAL;
  auto misaligned = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3) != 0; };
  if (misaligned(packed) || misaligned(scales) || misaligned(X) || misaligned(Y)) return GPTQ_EINVAL;
  if (x_dtype == GPTQ_BF16 && (ldx & 1)) return GPTQ_EINVAL;  // every row of X dword aligned
  if (cols > 0 && dequant_mma_supported(cols, groupsize, batch)) {
    const size_t need = dequant_mma_workspace(rows, cols, batch);
    if (workspace_bytes < need || (need > 0 && !workspace)) return GPTQ_EWORKSPACE;
    if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 3)) return GPTQ_EINVAL;
    return dequant_mma(packed, scales, zeros, rows, cols, bits, groupsize, X, x_dtype == GPTQ_BF16, ldx, batch, Y,
                       ldy, workspace, (hipStream_t)stream) == hipSuccess
               ? GPTQ_OK
               : GPTQ_EHIP;
  }
  return dequant_gemm(packed, scales, zeros, rows, cols, bits, groupsize, X, x_dtype == GPTQ_BF16, ldx, batch, Y,
                      ldy, (hipStream_t)stream) == hipSuccess
             ? GPTQ_OK
             : GPTQ_EHIP;
}

static bool hadamard_block_ok(int64_t n, int32_t block) {
  return block >= 1 && block <= 4096 && (block & (block - 1)) == 0 && n % block == 0;
}

int gptq_hadamard_rows(const void* in, gptq_dtype in_dtype, int64_t ld_in, float* out, int64_t ld_out,
                       int64_t rows, int64_t n, const float* signs, int32_t block, gptq_stream_t stream) {
  if (rows < 0 || n < 0 || rows > MAX_DIM || n > MAX_DIM) return GPTQ_EINVAL;
  if (in_dtype != GPTQ_BF16 && in_dtype != GPTQ_F32) return GPTQ_EINVAL;
  if (!hadamard_block_ok(n, block)) return GPTQ_EINVAL;
  if (rows == 0 || n == 0) return GPTQ_OK;
  if (!in || !out || !signs || ld_in < n || ld_out < n) return GPTQ_EINVAL;
  if (static_cast<const void*>(out) == in && (in_dtype != GPTQ_F32 || ld_in != ld_out)) return GPTQ_EINVAL;
  if (rows * hadamard_chunks(n) > INT32_MAX) return GPTQ_EUNSUPPORTED;
  return hadamard_rows(in, in_dtype == GPTQ_BF16, ld_in, out, ld_out, rows, n, signs, block,
                       (hipStream_t)stream) == hipSuccess
             ? GPTQ_OK
             : GPTQ_EHIP;
}

int gptq_hadamard_hessian(float* H, int64_t n, const float* signs, int32_t block, gptq_stream_t stream) {
  if (n < 0 || n > MAX_DIM) return GPTQ_EINVAL;
  if (!hadamard_block_ok(n, block)) return GPTQ_EINVAL;
  if (n == 0) return GPTQ_OK;
  if (!H || !signs) return GPTQ_EINVAL;
  if (n * hadamard_chunks(n) > INT32_MAX || (n + 63) / 64 > 65535) return GPTQ_EUNSUPPORTED;
  return hadamard_hessian(H, n, signs, block, (hipStream_t)stream) == hipSuccess ? GPTQ_OK : GPTQ_EHIP;
}

size_t gptq_cross_workspace_bytes(int64_t n, int64_t tokens, gptq_dtype x_dtype) {
  if (n <= 0 || tokens <= 0 || n > MAX_DIM || tokens > MAX_DIM) return 0;
  if (!(x_dtype == GPTQ_BF16 || x_dtype == GPTQ_F32)) return 0;
  return cross_workspace(n, tokens, x_dtype);
}

int gptq_accumulate_cross(float* C, int64_t n, const void* X, const void* Xq, gptq_dtype x_dtype, int64_t tokens,
                          int64_t ldx, void* workspace, size_t workspace_bytes, gptq_stream_t stream) {
  if (n < 0 || tokens < 0 || n > MAX_DIM || tokens > MAX_DIM) return GPTQ_EINVAL;
  if (!(x_dtype == GPTQ_BF16 || x_dtype == GPTQ_F32)) return GPTQ_EINVAL;
  if (n == 0 || tokens == 0) return GPTQ_OK;
  if (!C || !X || !Xq || ldx < n) return GPTQ_EINVAL;
  if (n * n > ((int64_t)1 << 31) * 2) return GPTQ_EUNSUPPORTED;
  const size_t need = cross_workspace(n, tokens, x_dtype);
  if (workspace_bytes < need || (need > 0 && !workspace)) return GPTQ_EWORKSPACE;
  return cross_launch(C, n, X, Xq, x_dtype, tokens, ldx, workspace, workspace_bytes, (hipStream_t)stream);
}

namespace {
struct QepLayout {
  size_t status, lam, dead, A, Lt, P1, P2, total;
};
QepLayout qep_layout(int64_t rows, int64_t cols) {
  QepLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, 256);
    return at;
  };
  L.status = take(4 * sizeof(int));
  L.lam = take(sizeof(float));
  L.dead = take((size_t)cols);
  L.A = take((size_t)cols * cols * sizeof(float));
  L.Lt = take(factor_scratch_floats(cols) * sizeof(float));
  L.P1 = take((size_t)rows * cols * sizeof(float));
  L.P2 = take((size_t)rows * cols * sizeof(float));
  L.total = off;
  return L;
}
}  // namespace

size_t gptq_qep_workspace_bytes(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0 || rows > MAX_DIM || cols > MAX_DIM) return 0;
  return qep_layout(rows, cols).total;
}

int gptq_qep_correct(const void* W, gptq_dtype w_dtype, int64_t rows, int64_t cols, float* C, float* H, float damp,
                     float alpha, float* W_out, void* workspace, size_t workspace_bytes, int32_t* d_status,
                     gptq_stream_t stream_) {
  hipStream_t stream = (hipStream_t)stream_;
  if (rows < 0 || cols < 0 || rows > MAX_DIM || cols > MAX_DIM) return GPTQ_EINVAL;
  if (!(w_dtype == GPTQ_BF16 || w_dtype == GPTQ_F32)) return GPTQ_EINVAL;
  if (!(damp >= 0.0f) || !(damp < INFINITY) || !(alpha >= 0.0f) || !(alpha <= 1.0f)) return GPTQ_EINVAL;
  if (rows == 0 || cols == 0) return GPTQ_OK;
  if (!W || !C || !H || !W_out || !workspace) return GPTQ_EINVAL;
  if (cols > 65535 * 4 || rows > INT32_MAX || rows * cols > ((int64_t)1 << 40)) return GPTQ_EUNSUPPORTED;
  const QepLayout L = qep_layout(rows, cols);
  if (workspace_bytes < L.total) return GPTQ_EWORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return GPTQ_EINVAL;
  char* ws = static_cast<char*>(workspace);
  int* status = reinterpret_cast<int*>(ws + L.status);
  FactorWs f{};
  f.status = status;
  f.lam = reinterpret_cast<float*>(ws + L.lam);
  f.dead = reinterpret_cast<uint8_t*>(ws + L.dead);
  f.A = reinterpret_cast<float*>(ws + L.A);
  f.Lt = reinterpret_cast<float*>(ws + L.Lt);
  if (fill_i32(status, 1, GPTQ_OK, stream) != hipSuccess) return GPTQ_EHIP;
  if (qep_correct_run(W, w_dtype == GPTQ_BF16, rows, cols, C, H, damp, alpha, W_out, f,
                      reinterpret_cast<float*>(ws + L.P1), reinterpret_cast<float*>(ws + L.P2), f.A,
                      stream) != hipSuccess)
    return GPTQ_EHIP;
  if (d_status) return copy_status(status, d_status, stream) == hipSuccess ? GPTQ_OK : GPTQ_EHIP;
  int host = 0;
  if (hipMemcpyAsync(&host, status, sizeof(int), hipMemcpyDeviceToHost, stream) != hipSuccess) return GPTQ_EHIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return GPTQ_EHIP;
  return host;
}

}  // extern "C"
