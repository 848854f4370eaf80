/*
 * gptq.h -- C ABI of libgptq.so, a GPTQ layer quantizer for AMD Instinct
 * MI355X (gfx950).
 *
 * The pages describe GPTQ as the Hessian-guided 2-4 bit weight quantizer at
 * the base of OneComp's pipeline (OneComp hub article, "core features", item 2,
 * quantizer table; item 3, the LPCD example GPTQ(wbits=3, groupsize=128)),
 * run layer by layer (same article, "limitations", point 3), with a Quantizer
 * interface exposing quantize() and save() (same article, "code
 * architecture").  The first three entry points below are that layer pass:
 * calibration statistics (gptq_accumulate_hessian), quantize()
 * (gptq_quantize_layer) and the packed artefact behind save() (gptq_pack).
 * After them: the dequantizing product that serves the packed layer
 * (gptq_dequant_gemv, gptq_dequant_gemm), a fixed Hadamard rotation applied
 * before quantizing (gptq_hadamard_rows, gptq_hadamard_hessian), and an
 * error-propagation correction of W before quantizing (gptq_accumulate_cross,
 * gptq_qep_correct).
 *
 * Conventions for every call
 *   - Tensor pointers are DEVICE pointers owned by the caller.  Row-major.
 *   - Work is queued on `stream` in order; calls return before the GPU is done
 *     unless stated otherwise.  The library allocates and frees no memory:
 *     scratch memory is the caller's workspace argument (or, for
 *     gptq_accumulate_hessian_static, a fixed device array of the library).
 *   - Return 0 (GPTQ_OK) on success, a positive gptq_status otherwise.
 *     Argument errors are detected on the host and return before any launch.
 *   - Calls that share a workspace or an output buffer on one device must not
 *     overlap in time (same stream, or ordered by the caller).
 */
#ifndef GPTQ_H
#define GPTQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* gptq_stream_t; /* a hipStream_t; NULL = default stream */

typedef enum {
  GPTQ_OK = 0,
  GPTQ_EINVAL = 1,       /* bad shape, pointer, dtype or parameter */
  GPTQ_ENOTPD = 2,       /* damped Hessian not positive definite (pivot <= 0 or not finite) */
  GPTQ_EWORKSPACE = 3,   /* workspace smaller than the matching *_workspace_bytes() */
  GPTQ_EUNSUPPORTED = 4, /* valid request this build does not implement */
  GPTQ_EHIP = 5          /* a HIP runtime call or kernel launch failed */
} gptq_status;

typedef enum { GPTQ_BF16 = 0, GPTQ_F32 = 1 } gptq_dtype;

/* gptq_params.flags */
enum {
  /* H already holds the factor U written by an earlier gptq_quantize_layer
     call with the same cols (shared Hessian: q/k/v, gate/up).  Damping and the
     factor are skipped; the dead-column mask is read back from H's strictly
     lower triangle (see gptq_quantize_layer).  Needs cols >= 3. */
  GPTQ_H_IS_FACTOR = 1,
  /* Damping and the factor in fp64 (the factor's precision option): lambda,
     H_d and every step of the factor are fp64, and U is rounded to fp32 once,
     when it is written into H.  The workspace holds an fp64 work matrix
     (gptq_quantize_workspace_bytes grows by 4 * cols^2 bytes).  Ignored with
     GPTQ_H_IS_FACTOR. */
  GPTQ_FACTOR_F64 = 2
};

/* Quantizer knobs: wbits and groupsize as in GPTQ(wbits, groupsize) on the
   OneComp hub article (LPCD example). */
typedef struct {
  int32_t bits;      /* 2, 3, 4 or 8; maxq = 2^bits - 1 */
  int32_t groupsize; /* -1 (one group per row), 32, 64, or a multiple of 128 */
  int32_t blocksize; /* lazy-batch width; 128 is the one supported value */
  float damp;        /* lambda = damp * mean(diag H); typically 0.01; >= 0 and finite */
  int32_t flags;     /* GPTQ_H_IS_FACTOR, GPTQ_FACTOR_F64, both, or 0 */
} gptq_params;

/* ---------------------------------------------------------------------------
 * Hessian accumulation.  H[n, n] += 2 * X^T X over one chunk of calibration
 * tokens X[tokens, n] (row stride ldx elements, dtype x_dtype).
 *
 * H is fp32, full symmetric (both triangles written, bit-identical).  The
 * caller zero-fills H before the first chunk and calls once per chunk; each
 * call reads H and adds to it.  Accumulation is in fp32 (bf16 products are
 * exact in fp32); the summation order is fixed, so repeated calls give
 * bit-identical H.  Alignment: X may have any alignment; 8-byte-aligned X
 * with ldx % 4 == 0 takes the vector path.
 * workspace: at least gptq_hessian_workspace_bytes(n, tokens, x_dtype) bytes
 * of device memory (may be 0 bytes, then NULL is accepted), 256-byte aligned.
 * tokens == 0 or n == 0: no work, GPTQ_OK.
 * ------------------------------------------------------------------------- */
size_t gptq_hessian_workspace_bytes(int64_t n, int64_t tokens, gptq_dtype x_dtype);

int gptq_accumulate_hessian(float* H, int64_t n, const void* X, gptq_dtype x_dtype,
                            int64_t tokens, int64_t ldx, void* workspace,
                            size_t workspace_bytes, gptq_stream_t stream);

/* gptq_accumulate_hessian for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving or calibration loops, harnesses that
 * forbid hipMalloc.  No workspace argument: the split-K partial tiles go to a
 * fixed device array inside the library, GPTQ_HESSIAN_STATIC_BYTES per device,
 * which a device holds from the library's first use on it until the process
 * ends.  The call allocates and frees nothing.
 *
 * Same arguments (less the workspace), work split, kernels and result (bit for
 * bit) as gptq_accumulate_hessian.  A call whose
 * gptq_hessian_workspace_bytes(n, tokens, x_dtype) exceeds
 * GPTQ_HESSIAN_STATIC_BYTES returns GPTQ_EWORKSPACE before any work.  For bf16
 * X that admits every n <= 1792 at any token count, every n >= 9729 (those
 * need no partials) and, in between, calls of fewer than 1024 tokens; a
 * 4096-wide layer must therefore be fed in chunks of at most 1023 tokens.
 * `stream` must belong to the current device (GPTQ_EINVAL otherwise); the
 * array used is that device's.
 *
 * Every call on a device shares that device's array, and a call leaves its
 * partials there.  Nothing needs clearing between calls (every partial slot a
 * call reads is written by that call first), but calls that overlap in time on
 * one device -- on different streams, or from different host threads without
 * ordering -- race on the array and leave H undefined. */
#define GPTQ_HESSIAN_STATIC_BYTES ((size_t)64 << 20)

int gptq_accumulate_hessian_static(float* H, int64_t n, const void* X, gptq_dtype x_dtype,
                                   int64_t tokens, int64_t ldx, gptq_stream_t stream);

/* ---------------------------------------------------------------------------
 * Quantize one linear layer W[rows, cols] (dtype w_dtype, row stride cols)
 * against its Hessian H[cols, cols] (fp32, full symmetric as written by
 * gptq_accumulate_hessian).
 *
 * Steps (all on the device, in order): dead columns (H_ii == 0: H_ii := 1,
 * W[:, i] := 0); damping H_d = H + lambda I, lambda = damp * mean(diag H);
 * the upper factor U with positive diagonal and U^T U = inv(H_d); then the
 * column loop in lazy batches of 128 columns: per-row asymmetric min/max grid
 * at each group start from the current, error-updated weights;
 * q = clamp(rint(w/s) + z, 0, maxq); w^ = s (q - z); e = (w - w^) / U_jj fed
 * back into the later columns of the block; after each block the trailing
 * update W[:, c1:] -= E U[c0:c1, c1:].
 *
 * H is overwritten IN PLACE (unless GPTQ_H_IS_FACTOR): its upper triangle
 * (with the diagonal) holds U in fp32; H[i][i-1] = 1.0f if column i is dead
 * else 0.0f (i >= 1) and H[cols-1][0] carries the same flag for column 0
 * (cols >= 3); the rest of the lower triangle is unspecified.
 *
 * Outputs (device, caller-owned):
 *   codes    uint8 [rows, cols]     integer codes in [0, maxq]
 *   scales   float [rows, G]        G = ceil(cols / groupsize) (1 if groupsize == -1)
 *   zeros    uint8 [rows, G]        integer zero points in [0, maxq]
 *   w_hat    float [rows, cols]     s (q - z); may be NULL
 *   row_loss float [rows]           sum_j (w_j - w^_j)^2 / (2 U_jj^2); may be NULL
 * workspace: gptq_quantize_workspace_bytes(rows, cols, p) bytes, 256-byte aligned.
 * d_status: if non-NULL, a device int32 that receives the final status
 *   (GPTQ_OK or GPTQ_ENOTPD) and the call is fully asynchronous; if NULL the
 *   call synchronizes `stream` once at the end and returns that status.
 *   With GPTQ_ENOTPD the outputs and H hold unspecified values (they may
 *   be non-finite).  Argument errors (GPTQ_EINVAL, GPTQ_EWORKSPACE,
 *   GPTQ_EUNSUPPORTED) are returned before any work and leave them untouched.
 * W, X and the outputs must not alias each other, H or the workspace.
 * rows == 0 or cols == 0: no work, GPTQ_OK.
 * ------------------------------------------------------------------------- */
size_t gptq_quantize_workspace_bytes(int64_t rows, int64_t cols, const gptq_params* p);

int gptq_quantize_layer(const void* W, gptq_dtype w_dtype, int64_t rows, int64_t cols,
                        float* H, const gptq_params* p, uint8_t* codes, float* scales,
                        uint8_t* zeros, float* w_hat, float* row_loss, void* workspace,
                        size_t workspace_bytes, int32_t* d_status, gptq_stream_t stream);

/* ---------------------------------------------------------------------------
 * Pack codes[rows, cols] (uint8, each < 2^bits) into packed[rows, cols*bits/32]
 * uint32 words: per row one little-endian bitstream, code i in bits
 * [i*bits, (i+1)*bits), word w holding stream bits [32w, 32w+32).  For bits = 3
 * a run of 32 codes fills three words.  bits in {2, 3, 4, 8};
 * (cols * bits) % 32 == 0.  Codes >= 2^bits are masked to their low bits.
 * ------------------------------------------------------------------------- */
int gptq_pack(const uint8_t* codes, int64_t rows, int64_t cols, int32_t bits, uint32_t* packed,
              gptq_stream_t stream);

/* ---------------------------------------------------------------------------
 * Dequantizing matrix-vector product y = W^ x over the quantizer's outputs, with
 * w^[r, j] = scales[r, j / g] * (code[r, j] - zeros[r, j / g]) (g = cols when
 * groupsize == -1): the packed codes as written by gptq_pack, and the scales
 * and zeros as written by gptq_quantize_layer.  This is the inference side of
 * the grid the OneComp hub article's quantizer table describes, as the
 * OneComp release post's vLLM plugins consume it.
 *   packed  uint32 [rows, cols*bits/32]   gptq_pack layout, dword aligned
 *   scales  float  [rows, G]              G = ceil(cols / g)
 *   zeros   uint8  [rows, G]
 *   x       [cols], x_dtype bf16 or fp32 (bf16 widens exactly to fp32)
 *   y       float  [rows]                 written, not accumulated into
 * Accumulation is fp32 in a fixed order (bit-reproducible run to run).
 * bits in {2, 3, 4, 8}; (cols * bits) % 32 == 0; groupsize -1 or a positive
 * multiple of 32 (else GPTQ_EUNSUPPORTED).  Pointers must be 4-byte aligned.
 * rows == 0: no work.  cols == 0: y := 0 (the input pointers may then be
 * NULL).  Argument errors return before any
 * launch.  y must not alias the inputs.
 * ------------------------------------------------------------------------- */
int gptq_dequant_gemv(const uint32_t* packed, const float* scales, const uint8_t* zeros, int64_t rows,
                      int64_t cols, int32_t bits, int32_t groupsize, const void* x, gptq_dtype x_dtype, float* y,
                      gptq_stream_t stream);

/* The same product for a batch: Y[t, :] = W^ X[t, :] for t < batch, with
 * X [batch, cols] (row stride ldx >= cols, bf16 or fp32; for bf16 ldx even)
 * and Y [batch, rows] fp32 (row stride ldy >= rows).  X finite.
 *   - batch of one: exactly gptq_dequant_gemv's result.
 *   - batch >= 2 with groupsize -1 or a multiple of 128: the matrix-core path.
 *     The codes are read once per group of up to 16 vectors and converted
 *     exactly to bf16; a bf16 x is exact in bf16 and an fp32 x is split
 *     exactly into three bf16 parts, so the products are exact and only the
 *     fp32 accumulation rounds (inside the matrix core, then per 128-column
 *     chunk, slice and part, in a fixed order).  Column slices go to the
 *     workspace as partial sums, which a second kernel adds in slice order.
 *   - other batches: VALU kernels, groups of up to 8 vectors, accumulation as
 *     in gptq_dequant_gemv; no workspace.
 * Results are bit-reproducible run to run.  workspace: at least
 * gptq_dequant_gemm_workspace_bytes(rows, cols, bits, groupsize, batch) bytes,
 * 4-byte aligned (NULL when that is 0; GPTQ_EWORKSPACE when short).  batch == 0
 * or rows == 0: no work.  Y must not alias the inputs or the workspace. */
size_t gptq_dequant_gemm_workspace_bytes(int64_t rows, int64_t cols, int32_t bits, int32_t groupsize,
                                        int64_t batch);
int gptq_dequant_gemm(const uint32_t* packed, const float* scales, const uint8_t* zeros, int64_t rows,
                      int64_t cols, int32_t bits, int32_t groupsize, const void* X, gptq_dtype x_dtype, int64_t ldx,
                      int64_t batch, float* Y, int64_t ldy, void* workspace, size_t workspace_bytes,
                      gptq_stream_t stream);

/* ---------------------------------------------------------------------------
 * Fixed randomised Hadamard rotation, the untrained form of the rotation
 * preprocessing on the OneComp hub article (rotations absorbed into the
 * weights, Hadamard transforms applied online to activations):
 *   Q = diag(signs) * blockdiag(H_b, ..., H_b) / sqrt(b),
 * H_b the Sylvester Hadamard matrix of order b = block (H_1 = [1],
 * H_2m = [[H_m, H_m], [H_m, -H_m]]), orthogonal when every sign is +-1.
 * A layer y = W x becomes W' = W Q with inputs x' = Q^T x (W' x' = W x), and
 * its Hessian H' = Q^T H Q; quantize W' against H'.
 * block: a power of two, 1 <= block <= 4096, dividing n (else GPTQ_EINVAL).
 * signs: device float [n].  Accumulation is fp32; log2(block) butterfly
 * stages, the sign on input, 1/sqrt(block) on output.
 * ------------------------------------------------------------------------- */

/* out[r, :] = in[r, :] Q for r < rows (row strides ld_in, ld_out elements,
 * >= n).  in is bf16 or fp32; out is fp32.  In place is allowed for fp32 input
 * with out == in and ld_out == ld_in; otherwise the two must not overlap.
 * Used for the weights (W -> W Q) and for activations or inputs (x^T -> x^T Q,
 * which is (Q^T x)^T).  rows == 0 or n == 0: no work. */
int gptq_hadamard_rows(const void* in, gptq_dtype in_dtype, int64_t ld_in, float* out, int64_t ld_out,
                       int64_t rows, int64_t n, const float* signs, int32_t block, gptq_stream_t stream);

/* H[n, n] := Q^T H Q in place, for a symmetric fp32 H (as written by
 * gptq_accumulate_hessian).  The result is written in full and exactly
 * symmetric (the lower triangle mirrors the upper).  No workspace. */
int gptq_hadamard_hessian(float* H, int64_t n, const float* signs, int32_t block, gptq_stream_t stream);

/* ---------------------------------------------------------------------------
 * Error-propagation correction before GPTQ: the QEP idea on the OneComp pages
 * (the error that quantizing earlier layers leaves in a layer's inputs is
 * carried into that layer's correction), read as the ridge fit of the
 * full-precision outputs from the quantized-model inputs.  With X [tokens, n]
 * the layer's inputs in the full-precision model and Xq those in the partly
 * quantized one:
 *   H = 2 Xq^T Xq (gptq_accumulate_hessian on Xq),
 *   C = 2 X^T Xq  (gptq_accumulate_cross),
 *   W' = W + alpha W G H_d^-1, G = C - H = 2 (X - Xq)^T Xq, H_d = H damped as
 *        in gptq_quantize_layer (same lambda, same dead-column rule)
 *        (gptq_qep_correct),
 * then gptq_quantize_layer(W', H, flags = GPTQ_H_IS_FACTOR): the correction
 * leaves H holding the factor.  alpha = 1 minimises
 *   ||X W^T - Xq W'^T||^2 + (lambda / 2) ||W' - W||^2;  alpha = 0 is plain GPTQ.
 * ------------------------------------------------------------------------- */

/* Workspace bytes for gptq_accumulate_cross over `tokens` tokens: the split-K
 * partial tiles, as for the Hessian (0 when the tokens are not split). */
size_t gptq_cross_workspace_bytes(int64_t n, int64_t tokens, gptq_dtype x_dtype);

/* C[n, n] += 2 X^T Xq over one chunk of tokens.  X and Xq: [tokens, n], the same
 * dtype (bf16 or fp32) and row stride ldx >= n.  C is fp32, not symmetric
 * (C[i][j] pairs column i of X with column j of Xq); the caller zero-fills it
 * before the first chunk.  The Hessian's MFMA kernels in their cross mode:
 * every tile of the square grid, bf16 products exact in fp32, fp32
 * accumulation in a fixed order (bit-reproducible run to run).  workspace:
 * gptq_cross_workspace_bytes(n, tokens, x_dtype) bytes, 256-byte aligned (may be
 * 0 bytes, then NULL is accepted).  tokens == 0 or n == 0: no work. */
int gptq_accumulate_cross(float* C, int64_t n, const void* X, const void* Xq, gptq_dtype x_dtype, int64_t tokens,
                          int64_t ldx, void* workspace, size_t workspace_bytes, gptq_stream_t stream);

size_t gptq_qep_workspace_bytes(int64_t rows, int64_t cols);

/* W_out[rows, cols] (fp32) = W + alpha W (C - H) H_d^-1 for W (bf16 or fp32,
 * row stride cols), C and H as accumulated above (both [cols, cols] fp32).
 * On return C holds G = C - H and H holds the factor U and the dead flags,
 * exactly as gptq_quantize_layer leaves them, for a following
 * gptq_quantize_layer with GPTQ_H_IS_FACTOR.  alpha in [0, 1], damp >= 0.
 * d_status as in gptq_quantize_layer (GPTQ_ENOTPD when H_d is not positive
 * definite; W_out then unspecified).  Workspace: gptq_qep_workspace_bytes,
 * 256-byte aligned.  W_out must not alias W, C, H or the workspace. */
int gptq_qep_correct(const void* W, gptq_dtype w_dtype, int64_t rows, int64_t cols, float* C, float* H, float damp,
                     float alpha, float* W_out, void* workspace, size_t workspace_bytes, int32_t* d_status,
                     gptq_stream_t stream);

/* Static description of a status code (never NULL). */
const char* gptq_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int gptq_version(void);

/* ---------------------------------------------------------------------------
 * Phase timestamps, a measurement aid (not an operation of the method).  The
 * library built with the GPTQ_TRACE option (libgptq_trace.so) records, for
 * each workgroup of the column loop, of the factor's chain (diagonal-block
 * factor, block-column solve, diagonal-block update, step tiles) and of the
 * matrix-core batch product, the 100 MHz
 * s_memrealtime clock at its phase boundaries into buf, a device buffer of
 * uint64 words:
 *   buf[0] = capacity in records (set by the caller), buf[1] = records
 *   appended (set to 0 by the caller; the kernels add to it atomically),
 *   record i at buf[32 * (i + 1)]: kind (1 loop, 2 diagonal factor, 3 solve,
 *   4 diagonal update, 5 step tile, 6 batch product), workgroup index (for
 *   6 the column slice), tag (the 128-column block; for 6 the 128-row
 *   block), stamp count, then the stamps.
 * Records past the capacity are dropped (buf[1] still counts them).  buf ==
 * NULL stops recording.  The pointer is per device (the current one) and
 * process-wide, so concurrent calls append to the same buffer.  The library
 * built without the option returns GPTQ_EUNSUPPORTED and records nothing. */
int gptq_trace_set(void* buf);

#ifdef __cplusplus
}
#endif

#endif /* GPTQ_H */
