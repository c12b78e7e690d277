/*
 * dsfp8 -- block-scaled FP8 linear layer for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libdsfp8.so.  Every entry point takes plain device pointers and
 * sizes, enqueues its kernels on the caller's HIP stream and returns without
 * synchronising.  The library allocates no memory; all buffers are owned by
 * the caller.  Its only global state is (1) a per-device cache of the
 * compute-unit count (read once with hipDeviceGetAttribute, used to size
 * grids) and (2) the static device scratch of dsfp8_grouped_gemm_noalloc
 * (one copy per GPU, with its address cached per device).
 *
 * Sources of the operations (the DeepSeek-V3 inference code as described by):
 *   [AG]  "DeepSeek-V3 Administrator & Developer Guide" (doccompiler.ai)
 *   [UG]  "DeepSeek-V3 User Guide" (doccompiler.ai)
 *   [DF]  "CodeVetter Repo Unpack: deepseek-v3 / Data flow"
 *   [DS]  DocSearch (Algolia) index of the deepseek-ai/DeepSeek-V3 README
 *
 * Number formats
 *   e4m3  OCP FP8 E4M3 "fn" (bias 7, max +-448, no infinity, NaN = S.1111.111),
 *         i.e. torch.float8_e4m3fn ([DS] item 10).  Stored as one byte.
 *   bf16  bfloat16, stored as two bytes.
 *   Scales are IEEE fp32.
 *
 * Layout conventions (all entry points)
 *   Matrices are row-major with the innermost dimension contiguous; "ld" is the
 *   row stride in ELEMENTS and must be >= the row length.  Block size is fixed
 *   at 128 ([DS] item 10: weight_block_size [128, 128]).  KB(K) = ceil(K/128).
 *   Activation scales: fp32, logically [M, KB(K)]; element (m, b) is stored
 *     at s[m * s_row_stride + b * s_kb_stride].  Row-major storage has
 *     s_kb_stride = 1, s_row_stride >= KB(K); K-block-major ("column-major")
 *     storage has s_row_stride = 1, s_kb_stride >= M.  The products read a
 *     K-block's scales for consecutive rows with one coalesced access when
 *     they are K-block-major, which is the layout to prefer.
 *   Weight scales:     fp32 [KB(N), KB(K)], row stride in elements.
 *   A last block narrower than 128 (K or N not a multiple of 128) is treated
 *   as zero-padded to 128 ([DS] item 3); only its real elements are read or
 *   written.
 *
 * Error behaviour
 *   Arguments are checked on the host before anything is enqueued.  A call
 *   that returns a negative status has launched nothing and written nothing.
 *   Sizes of zero are valid and launch nothing, except where an output must
 *   still be written (a product with K == 0 writes zeros).  Device-resident
 *   data (values, expert offsets) is not validated.  DSFP8_ERR_LAUNCH reports
 *   a failure returned by the HIP runtime at launch.  No C++ exception
 *   crosses this interface.
 *
 * Rounding
 *   Scales and quotients are correctly rounded fp32 divisions; fp32 -> e4m3
 *   is round-to-nearest-even with saturation to +-448, keeping the sign of
 *   zero and producing subnormals; fp32 -> bf16 is round-to-nearest-even.
 */
#ifndef DSFP8_H
#define DSFP8_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSFP8_ABI_VERSION 6
#define DSFP8_BLOCK 128

typedef int dsfp8_status;

enum {
  DSFP8_OK = 0,
  DSFP8_ERR_NULL = -1,       /* a required pointer is NULL                        */
  DSFP8_ERR_SHAPE = -2,      /* a size is negative or exceeds the supported range */
  DSFP8_ERR_LD = -3,         /* a leading dimension is smaller than its row       */
  DSFP8_ERR_ALIGN = -4,      /* a pointer is not aligned to its element size      */
  DSFP8_ERR_SCALE_FMT = -5,  /* unknown scale format                              */
  DSFP8_ERR_WORKSPACE = -6,  /* workspace smaller than the size query returned    */
  DSFP8_ERR_LAUNCH = -7,     /* the HIP runtime reported a launch failure         */
  DSFP8_ERR_DTYPE = -8,      /* unknown input element type                        */
  DSFP8_ERR_UNSUPPORTED = -9, /* a fused form does not support this operand layout */
  DSFP8_ERR_SCRATCH = -10     /* the problem exceeds the static scratch of a
                                 *_noalloc entry point                            */
};

/* Scale formats.  UE8M0 rounds each scale value up to a power of two
 * ([UG] FAQ "What is scale_fmt: ue8m0?"; [AG] 8.5.1); the scale is still
 * stored as fp32. */
enum { DSFP8_SCALE_FP32 = 0, DSFP8_SCALE_UE8M0 = 1 };

/* Element types accepted by dsfp8_weight_quant. */
enum { DSFP8_DTYPE_F32 = 0, DSFP8_DTYPE_BF16 = 1 };

/* Library ABI version (DSFP8_ABI_VERSION of the build). */
int dsfp8_abi_version(void);

/* Static description of a status code; never NULL. */
const char* dsfp8_status_string(dsfp8_status status);

/*
 * Activation quantisation, [AG] 8.5.1 act_quant_kernel; [DF] (FP8 bullet)
 * states that the per-block scales are kept as an fp32 tensor.
 *
 * For every row m and 128-column block b of x:
 *   amax   = max |x[m, k]| over the block's real columns (fp32)
 *   s      = max(amax, 1e-4f) / 448             (fp32 division)
 *   s      = 2^ceil(log2 s)                     if scale_fmt == UE8M0 (exact)
 *   y[m,k] = e4m3(x[m,k] / s)                   (fp32 division, RNE, saturating)
 *   s_out[m, b] = s
 *
 *   x      bf16 [M, K], row stride ldx >= K            (device, read)
 *   y      e4m3 [M, K], row stride ldy >= K            (device, written)
 *   s      fp32 [M, KB(K)], strides s_row_stride, s_kb_stride (see above)
 *                                                      (device, written)
 * K need not be a multiple of 128 (the pages' assertion that it is is relaxed;
 * the partial block follows the zero-padding rule).
 * Errors: NULL (x/y/s NULL with M*K > 0), SHAPE (M or K < 0), LD, ALIGN (x not
 * 2-byte or s not 4-byte aligned), SCALE_FMT, LAUNCH.
 */
dsfp8_status dsfp8_act_quant(const void* x, int64_t M, int64_t K, int64_t ldx,
                             void* y, int64_t ldy,
                             float* s, int64_t s_row_stride, int64_t s_kb_stride,
                             int scale_fmt, hipStream_t stream);

/*
 * Fused SiLU-gate and activation quantisation for the feed-forward step
 * between the up- and down-projections, [AG] 1.2 (MLP / Expert: w2(SiLU(w1 x)
 * * w3 x)) followed by [AG] 8.5.1.
 *
 *   h[m,i] = bf16( SiLU(g[m,i]) * u[m,i] )       SiLU(v) = v / (1 + e^-v), fp32
 *   (y, s) = act_quant(h)                        exactly as dsfp8_act_quant
 *
 *   g, u   bf16 [M, I], row strides ldg, ldu >= I  (device, read; g and u may be
 *          the two halves of one [M, 2I] product, e.g. u = g + I, ldg = ldu = 2I)
 *   y      e4m3 [M, I], row stride ldy             (device, written)
 *   s      fp32 [M, KB(I)], strides as act_quant   (device, written)
 *   h      bf16 [M, I], row stride ldh, or NULL    (device, written if not NULL)
 * The exponential is the hardware's, so h is reproducible only to within one
 * bf16 unit in the last place of a correctly rounded evaluation; (y, s) are
 * always act_quant of the h that this call computes.
 * Errors: as dsfp8_act_quant.
 */
dsfp8_status dsfp8_silu_mul_act_quant(const void* g, int64_t ldg,
                                      const void* u, int64_t ldu,
                                      int64_t M, int64_t I,
                                      void* y, int64_t ldy,
                                      float* s, int64_t s_row_stride, int64_t s_kb_stride,
                                      void* h, int64_t ldh,
                                      int scale_fmt, hipStream_t stream);

/*
 * Weight block quantisation: produces the stored weight format of [DS] item 3
 * (weight_scale_inv holds one fp32 multiplier per 128x128 block, a block is
 * dequantised by multiplying it by that value, and a block that is not
 * 128-aligned is zero-padded when its scale is computed) from real-valued
 * weights.  The scale of a block mirrors act_quant:
 *   S[i, j] = max(max |w| over the block, 1e-4f) / 448   (optionally UE8M0)
 *   q[n, k] = e4m3(w[n, k] / S[n/128, k/128])
 *
 *   w      fp32 or bf16 (dtype) [N, K], row stride ldw  (device, read)
 *   q      e4m3 [N, K], row stride ldq                  (device, written)
 *   S      fp32 [KB(N), KB(K)], row stride ldS          (device, written)
 * Errors: NULL, SHAPE, LD, ALIGN, SCALE_FMT, DTYPE, LAUNCH.
 */
dsfp8_status dsfp8_weight_quant(const void* w, int dtype, int64_t N, int64_t K, int64_t ldw,
                                void* q, int64_t ldq, float* S, int64_t ldS,
                                int scale_fmt, hipStream_t stream);

/*
 * Weight dequantisation, [AG] 8.5.2 weight_dequant_kernel and [DS] item 3:
 *   out[n, k] = bf16( fp32( dec(w[n, k]) * S[n/128, k/128] ) )
 * (the product is rounded to fp32, then to bf16, as the pages load as fp32,
 * multiply, and store in the default dtype).
 *
 *   w      e4m3 [N, K], row stride ldw                 (device, read)
 *   S      fp32 [KB(N), KB(K)], row stride ldS         (device, read)
 *   out    bf16 [N, K], row stride ldo                 (device, written)
 * Errors: NULL, SHAPE, LD, ALIGN, LAUNCH.
 */
dsfp8_status dsfp8_weight_dequant(const void* w, int64_t N, int64_t K, int64_t ldw,
                                  const float* S, int64_t ldS,
                                  void* out, int64_t ldo, hipStream_t stream);

/*
 * Block-scaled FP8 product, [AG] 8.5.3 fp8_gemm_kernel and 6.3 (linear():
 * y = x W^T with W [out, in]):
 *   C[m, n] = bf16( sum_b  a_s[m, b] * b_s[n/128, b] * sum_{k in block b} dec(A[m,k]) dec(B[n,k]) )
 * accumulated in fp32; the order of accumulation is unspecified.
 *
 *   A      e4m3 [M, K], row stride lda                  (device, read)
 *   a_s    fp32 [M, KB(K)], strides as_row_stride, as_kb_stride (see
 *          above; K-block-major is fastest)             (device, read)
 *   B      e4m3 [N, K], row stride ldb (the weight)     (device, read)
 *   b_s    fp32 [KB(N), KB(K)], row stride ldbs         (device, read)
 *   C      bf16 [M, N], row stride ldc                  (device, written)
 *   scale_fmt  DSFP8_SCALE_FP32: any positive finite scales.
 *          DSFP8_SCALE_UE8M0: the caller guarantees that every a_s and b_s
 *          value is a positive normal power of two (what act_quant and the
 *          weight quantiser produce with that format, [UG] FAQ on
 *          scale_fmt); only the exponent bits are read and the scaling is
 *          done inside the matrix instruction (CDNA4's block-scaled MFMA).
 *          The result definition is the same.
 *   workspace / workspace_bytes: scratch of at least
 *          dsfp8_gemm_workspace_bytes(M, N, K) bytes (may be NULL when that
 *          is 0), 16-byte aligned.  It must hold zeros before the first call
 *          that uses it (allocate it zero-filled, or clear it once); every
 *          call leaves it so again (the products that split K keep per-tile
 *          arrival counters at its start and clear them when they finish), so
 *          one workspace serves any later calls, of any shape, without being
 *          cleared again.  Calls that may run at the same time must not share
 *          a workspace.
 * Errors: NULL, SHAPE, LD, ALIGN, SCALE_FMT, WORKSPACE, LAUNCH.
 */
dsfp8_status dsfp8_gemm(const void* A, int64_t lda,
                        const float* a_s, int64_t as_row_stride, int64_t as_kb_stride,
                        const void* B, int64_t ldb, const float* b_s, int64_t ldbs,
                        void* C, int64_t ldc, int64_t M, int64_t N, int64_t K, int scale_fmt,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

size_t dsfp8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * Grouped block-scaled FP8 product over per-expert row ranges: the batched form
 * of the routed-expert loop of [AG] 6.4 / 8.4 (each expert's tokens pass
 * through that expert's FP8 linear layer).  Rows of A are sorted by expert;
 * expert e owns rows [offsets[e], offsets[e+1]) and has its own weight
 * B[e] [N, K] and scale grid b_s[e] [KB(N), KB(K)]:
 *   C[o_e:o_{e+1}] = dsfp8_gemm(A[o_e:o_{e+1}], a_s[o_e:o_{e+1}], B[e], b_s[e])
 *
 *   A        e4m3 [M_total, K], row stride lda              (device, read)
 *   a_s      fp32 [M_total, KB(K)], strides as_row_stride, as_kb_stride
 *                                                           (device, read)
 *   B        e4m3 [E, N, K]: row stride ldb, expert stride N*ldb       (device)
 *   b_s      fp32 [E, KB(N), KB(K)]: row stride ldbs, expert stride
 *            KB(N)*ldbs                                     (device, read)
 *   offsets  int32 [E+1] in DEVICE memory, offsets[0] = 0, non-decreasing,
 *            offsets[E] = M_total.  Not validated (that would need a host
 *            synchronisation); the kernels clamp every range to [0, M_total],
 *            so malformed offsets give unspecified output but no access
 *            outside A, a_s or C.  Experts with no rows cost nothing.
 *   C        bf16 [M_total, N], row stride ldc              (device, written)
 *   scale_fmt  as for dsfp8_gemm.
 *   workspace  at least dsfp8_grouped_gemm_workspace_bytes(E, M_total, N, K)
 *            bytes of device memory, 4-byte aligned (scratch: the per-expert
 *            tile schedule, then, if 16-byte aligned, a table of every
 *            workgroup's tile that saves each tile a chain of dependent
 *            loads; its size grows with E, M_total and N / 256).  Its
 *            contents need no initialisation and are rewritten by every call.
 * The combine step (scatter-add of each row times its routing weight) is not
 * part of this call.
 * Errors: NULL, SHAPE (E < 1, or E > 65536), LD, ALIGN, SCALE_FMT, WORKSPACE,
 * LAUNCH.
 */
dsfp8_status dsfp8_grouped_gemm(const void* A, int64_t lda,
                                const float* a_s, int64_t as_row_stride, int64_t as_kb_stride,
                                const void* B, int64_t ldb, const float* b_s, int64_t ldbs,
                                const int32_t* offsets, int64_t E, int64_t M_total,
                                int64_t N, int64_t K, void* C, int64_t ldc, int scale_fmt,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

size_t dsfp8_grouped_gemm_workspace_bytes(int64_t E, int64_t M_total, int64_t N, int64_t K);

/*
 * dsfp8_grouped_gemm without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * forbid allocation).  It computes exactly what dsfp8_grouped_gemm computes,
 * with the same kernels, so the two give bit-identical results.  The only
 * scratch, the per-expert tile schedule, lives in a static device array of
 * 3 * (DSFP8_NOALLOC_MAX_EXPERTS + 1) int32 (about 48 KB) that every GPU the
 * library runs on holds until the process ends; no call allocates anything.
 * Each call rewrites every schedule entry it reads before reading it, so no
 * state carries over from earlier calls.  All calls on one GPU share that
 * GPU's array: calls that may overlap in time on the same GPU (different
 * streams without ordering between them) race and must not be issued.
 * Arguments as for dsfp8_grouped_gemm.
 * Errors: as dsfp8_grouped_gemm without WORKSPACE; SCRATCH when
 * E > DSFP8_NOALLOC_MAX_EXPERTS (nothing launched); LAUNCH also when the
 * scratch's device address cannot be obtained.
 */
#define DSFP8_NOALLOC_MAX_EXPERTS 4096
dsfp8_status dsfp8_grouped_gemm_noalloc(const void* A, int64_t lda,
                                        const float* a_s, int64_t as_row_stride, int64_t as_kb_stride,
                                        const void* B, int64_t ldb, const float* b_s, int64_t ldbs,
                                        const int32_t* offsets, int64_t E, int64_t M_total,
                                        int64_t N, int64_t K, void* C, int64_t ldc, int scale_fmt,
                                        hipStream_t stream);

/*
 * Gated up-projection: the block-scaled FP8 product with the SiLU gate and
 * the next activation quantisation in its epilogue, i.e. the feed-forward
 * step w2(SiLU(w1 x) * w3 x) of [AG] 1.2 (MLP and Expert rows) up to the input
 * of w2, with linear() of [AG] 6.3 / 8.5.3 for w1 and w3 and act_quant of
 * [AG] 8.5.1 for the w2 input:
 *   h1 = dsfp8_gemm(A, a_s, W13[0:F], w_s[0:F/128])         bf16 [M, F]
 *   h3 = dsfp8_gemm(A, a_s, W13[F:2F], w_s[F/128:2F/128])   bf16 [M, F]
 *   h  = bf16(SiLU(h1) * h3)          as dsfp8_silu_mul_act_quant
 *   (y, s) = act_quant(h)             as dsfp8_act_quant
 * without writing h1 or h3 to memory.  The result equals
 * dsfp8_gemm(A, a_s, W13, w_s) followed by dsfp8_silu_mul_act_quant on its two
 * halves (same arithmetic, same order).
 *
 *   A      e4m3 [M, K], row stride lda                    (device, read)
 *   a_s    fp32 [M, KB(K)], strides as for dsfp8_gemm     (device, read)
 *   W13    e4m3 [2F, K], row stride ldw: w1 in rows 0..F-1, w3 in rows
 *          F..2F-1 (the two weights stacked)               (device, read)
 *   w_s    fp32 [2F/128, KB(K)], row stride ldws (the two scale grids
 *          stacked likewise)                               (device, read)
 *   y      e4m3 [M, F], row stride ldy                    (device, written)
 *   s      fp32 [M, F/128], strides s_row_stride, s_kb_stride (device, written)
 *   h      bf16 [M, F], row stride ldh, or NULL           (device, written if not NULL)
 *   scale_fmt  applies to both the product's operand scales (as for
 *          dsfp8_gemm) and the scales written to s (as for dsfp8_act_quant).
 * Supported layouts (else DSFP8_ERR_UNSUPPORTED; use the unfused calls):
 * F a positive multiple of 128; K, lda, ldw multiples of 16; A and W13
 * 16-byte aligned; (F + 128) * ldw + K < 2^31; y 8-byte aligned with ldy a
 * multiple of 8; h (if given) 16-byte aligned with ldh a multiple of 8.
 * Errors: NULL, SHAPE, LD, ALIGN, SCALE_FMT, UNSUPPORTED, LAUNCH.
 */
dsfp8_status dsfp8_gemm_silu_mul_act_quant(const void* A, int64_t lda,
                                           const float* a_s, int64_t as_row_stride, int64_t as_kb_stride,
                                           const void* W13, int64_t ldw, const float* w_s, int64_t ldws,
                                           int64_t M, int64_t F, int64_t K,
                                           void* y, int64_t ldy,
                                           float* s, int64_t s_row_stride, int64_t s_kb_stride,
                                           void* h, int64_t ldh, int scale_fmt, hipStream_t stream);

/*
 * Grouped form of dsfp8_gemm_silu_mul_act_quant over per-expert row ranges
 * ([AG] 6.4 / 8.4): rows offsets[e]..offsets[e+1]-1 of A use expert e's
 * stacked weight W13[e] [2F, K] (expert stride 2F*ldw) and scales w_s[e]
 * [2F/128, KB(K)] (expert stride (2F/128)*ldws).  offsets as for
 * dsfp8_grouped_gemm (device memory, not validated, clamped).  workspace:
 * at least dsfp8_grouped_gemm_workspace_bytes(E, M_total, 2F, K) bytes.
 * Supported layouts as above.
 * Errors: NULL, SHAPE, LD, ALIGN, SCALE_FMT, WORKSPACE, UNSUPPORTED, LAUNCH.
 */
dsfp8_status dsfp8_grouped_gemm_silu_mul_act_quant(const void* A, int64_t lda,
                                                   const float* a_s, int64_t as_row_stride, int64_t as_kb_stride,
                                                   const void* W13, int64_t ldw, const float* w_s, int64_t ldws,
                                                   const int32_t* offsets, int64_t E, int64_t M_total,
                                                   int64_t F, int64_t K,
                                                   void* y, int64_t ldy,
                                                   float* s, int64_t s_row_stride, int64_t s_kb_stride,
                                                   void* h, int64_t ldh, int scale_fmt,
                                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * dsfp8_grouped_gemm_silu_mul_act_quant with the activation rows read through
 * an index, so the per-token quantised input feeds the experts without a
 * gathered copy ([AG] 6.4 / 8.4: expert e's input is x[idx]; the per-row,
 * per-128-column quantisation of 8.5.1 commutes with that row selection):
 * row r of the product is row rows[r] of A, with its scales.
 *
 *   A      e4m3 [a_rows, K], row stride lda                 (device, read)
 *   a_s    fp32 [a_rows, KB(K)], strides as for dsfp8_gemm  (device, read)
 *   rows   int32 [M_total]; each entry is clamped to [0, a_rows) (device, read)
 * All other arguments as for dsfp8_grouped_gemm_silu_mul_act_quant (y, s, h
 * have M_total rows, in product-row order).  Also required: a_rows >= 1
 * when M_total > 0, and a_rows * lda + K < 2^31 (else UNSUPPORTED).
 * Errors: NULL, SHAPE, LD, ALIGN, SCALE_FMT, WORKSPACE, UNSUPPORTED, LAUNCH.
 */
dsfp8_status dsfp8_grouped_gemm_silu_mul_act_quant_gather(const void* A, int64_t a_rows, int64_t lda,
                                                          const float* a_s, int64_t as_row_stride,
                                                          int64_t as_kb_stride, const int32_t* rows,
                                                          const void* W13, int64_t ldw, const float* w_s,
                                                          int64_t ldws, const int32_t* offsets, int64_t E,
                                                          int64_t M_total, int64_t F, int64_t K,
                                                          void* y, int64_t ldy,
                                                          float* s, int64_t s_row_stride, int64_t s_kb_stride,
                                                          void* h, int64_t ldh, int scale_fmt,
                                                          void* workspace, size_t workspace_bytes,
                                                          hipStream_t stream);

/*
 * act_quant of gathered rows: the expert inputs x[idx] of [AG] 6.4 / 8.4
 * quantised without writing the gathered bf16 copy:
 *   y[m], s[m] = act_quant(x[rows[m]])   for 0 <= m < M.
 *
 *   x      bf16 [x_rows, K], row stride ldx                  (device, read)
 *   rows   int32 [M]; each entry is clamped to [0, x_rows)  (device, read)
 *   y, s   e4m3 [M, K] and fp32 scales, as for dsfp8_act_quant (device, written)
 * Errors: NULL, SHAPE, LD, ALIGN, SCALE_FMT, LAUNCH.
 */
dsfp8_status dsfp8_act_quant_rows(const void* x, int64_t x_rows, int64_t ldx, const int32_t* rows,
                                  int64_t M, int64_t K, void* y, int64_t ldy,
                                  float* s, int64_t s_row_stride, int64_t s_kb_stride,
                                  int scale_fmt, hipStream_t stream);

/*
 * Routing for the grouped product ([AG] 6.4 / 8.4: for each expert i in
 * increasing order, the (idx, top) pairs with indices == i, in the order
 * torch.where lists them).  The T*k (token, slot) pairs are sorted stably by
 * expert: rows offsets[e] .. offsets[e+1]-1 are expert e's pairs in increasing
 * t*k + j.  Deterministic (no atomics on global memory).
 *
 *   indices     int32 [T, k], row stride ldi: expert of each (token, slot)
 *                                                           (device, read)
 *   offsets     int32 [E+1]; offsets[E] = number of routed pairs
 *                                                           (device, written)
 *   row_token   int32 [T*k]: token of each row; entries at or past
 *               offsets[E] are left untouched               (device, written)
 *   token_rows  int32 [T, k] contiguous: row of each pair; -1 for a pair whose
 *               index is outside [0, E) (it gets no row)    (device, written)
 *   workspace   at least dsfp8_moe_route_workspace_bytes(T, k, E) bytes,
 *               4-byte aligned                              (device, scratch)
 * Limits: 1 <= k <= 16, 1 <= E <= 4096, T*k < 2^31.
 * Errors: NULL, SHAPE, LD, ALIGN, WORKSPACE, LAUNCH.
 */
dsfp8_status dsfp8_moe_route(const int32_t* indices, int64_t T, int64_t k, int64_t ldi, int64_t E,
                             int32_t* offsets, int32_t* row_token, int32_t* token_rows,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

size_t dsfp8_moe_route_workspace_bytes(int64_t T, int64_t k, int64_t E);

/*
 * Weighted combine of the expert outputs ([AG] 6.4 / 8.4:
 * y[idx] += expert(x[idx]) * weights[idx, top] for each expert in increasing
 * order, y starting at zero, in bf16):
 *   out[t] = the sum over the token's pairs, taken in increasing expert index,
 *            of bf16(yr[token_rows[t, j]] * weights[t, j]), each addition
 *            rounded to bf16 (round-to-nearest-even).
 *
 *   yr          bf16 [R, D], row stride ldy: expert outputs by row (device, read)
 *   indices     int32 [T, k], row stride ldi                       (device, read)
 *   weights     bf16 [T, k], row stride ldw                        (device, read)
 *   token_rows  int32 [T, k] contiguous, from dsfp8_moe_route; entries
 *               outside [0, R) are skipped                         (device, read)
 *   out         bf16 [T, D], row stride ldo                        (device, written)
 * Limits: 1 <= k <= 16.  Errors: NULL, SHAPE, LD, ALIGN, LAUNCH.
 */
dsfp8_status dsfp8_moe_combine(const void* yr, int64_t R, int64_t ldy,
                               const int32_t* indices, int64_t ldi, const void* weights, int64_t ldw,
                               const int32_t* token_rows, int64_t T, int64_t k, int64_t D,
                               void* out, int64_t ldo, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DSFP8_H */
