// C ABI of libdsfp8: argument validation (plain host code, no HIP call before
// every check has passed) and dispatch to the kernel launchers.
#include <atomic>

#include "../../include/dsfp8.h"
#include "launch.h"

namespace dsfp8 {

int device_cu_count() {
  // Read-only cache of a device attribute; a race only repeats the query.
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

}  // namespace dsfp8

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;  // rows, columns and K below 2^31
constexpr int64_t kMaxExperts = 65536;

inline int64_t nblk(int64_t n) { return (n + DSFP8_BLOCK - 1) / DSFP8_BLOCK; }
inline bool al(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }
inline bool dim_ok(int64_t v) { return v >= 0 && v < kMaxDim; }

// A matrix argument: rows x cols elements with row stride ld.
inline dsfp8_status check_mat(const void* p, int64_t rows, int64_t cols, int64_t ld, size_t elt) {
  if (ld < cols || ld < 0 || ld >= ((int64_t)1 << 40)) return DSFP8_ERR_LD;
  if (rows > 0 && cols > 0 && p == nullptr) return DSFP8_ERR_NULL;
  if (p != nullptr && !al(p, elt)) return DSFP8_ERR_ALIGN;
  return DSFP8_OK;
}

#define DSFP8_TRY(expr)              \
  do {                               \
    const dsfp8_status st_ = (expr); \
    if (st_ != DSFP8_OK) return st_; \
  } while (0)

inline dsfp8_status launched(hipError_t e) { return e == hipSuccess ? DSFP8_OK : DSFP8_ERR_LAUNCH; }

// An activation-scale matrix: rows x kbs fp32 values, element (m, b) at
// p[m * rs + b * ks].  Accepted layouts are row-major (ks == 1, rs >= kbs) and
// K-block-major (rs == 1, ks >= rows); with a single row or K-block only the
// other stride matters.
dsfp8_status check_scales(const void* p, int64_t rows, int64_t kbs, int64_t rs, int64_t ks) {
  const int64_t kBig = (int64_t)1 << 40;
  if (rs < 0 || ks < 0 || rs >= kBig || ks >= kBig) return DSFP8_ERR_LD;
  if (rows > 1 && kbs > 1) {
    const bool row_major = ks == 1 && rs >= kbs;
    const bool kb_major = rs == 1 && ks >= rows;
    if (!row_major && !kb_major) return DSFP8_ERR_LD;
  } else if (rows > 1) {
    if (rs < 1) return DSFP8_ERR_LD;
  } else if (kbs > 1) {
    if (ks < 1) return DSFP8_ERR_LD;
  }
  if (rows > 0 && kbs > 0 && p == nullptr) return DSFP8_ERR_NULL;
  if (p != nullptr && !al(p, 4)) return DSFP8_ERR_ALIGN;
  return DSFP8_OK;
}

dsfp8_status check_quant_out(int64_t M, int64_t K, void* y, int64_t ldy, float* s, int64_t srs, int64_t sks) {
  DSFP8_TRY(check_mat(y, M, K, ldy, 1));
  DSFP8_TRY(check_scales(s, M, nblk(K), srs, sks));
  return DSFP8_OK;
}

}  // namespace

extern "C" {

int dsfp8_abi_version(void) { return DSFP8_ABI_VERSION; }

const char* dsfp8_status_string(dsfp8_status st) {
  switch (st) {
    case DSFP8_OK: return "ok";
    case DSFP8_ERR_NULL: return "a required pointer is NULL";
    case DSFP8_ERR_SHAPE: return "a size is negative or outside the supported range";
    case DSFP8_ERR_LD: return "a leading dimension is smaller than its row length";
    case DSFP8_ERR_ALIGN: return "a pointer is not aligned to its element size";
    case DSFP8_ERR_SCALE_FMT: return "unknown scale format";
    case DSFP8_ERR_WORKSPACE: return "workspace is smaller than required";
    case DSFP8_ERR_LAUNCH: return "the HIP runtime reported a launch failure";
    case DSFP8_ERR_DTYPE: return "unknown element type";
    case DSFP8_ERR_UNSUPPORTED: return "the fused form does not support this operand layout";
    case DSFP8_ERR_SCRATCH: return "the problem needs more scratch than the library's static buffer holds";
    default: return "unknown status";
  }
}

dsfp8_status dsfp8_act_quant(const void* x, int64_t M, int64_t K, int64_t ldx, void* y, int64_t ldy, float* s,
                             int64_t s_row_stride, int64_t s_kb_stride, int scale_fmt, hipStream_t stream) {
  if (!dim_ok(M) || !dim_ok(K)) return DSFP8_ERR_SHAPE;
  if (scale_fmt != DSFP8_SCALE_FP32 && scale_fmt != DSFP8_SCALE_UE8M0) return DSFP8_ERR_SCALE_FMT;
  DSFP8_TRY(check_mat(x, M, K, ldx, 2));
  DSFP8_TRY(check_quant_out(M, K, y, ldy, s, s_row_stride, s_kb_stride));
  dsfp8::ActQuantArgs a{};
  a.g = static_cast<const uint16_t*>(x);
  a.ldg = ldx;
  a.u = nullptr;
  a.ldu = 0;
  a.M = M;
  a.K = K;
  a.y = static_cast<uint8_t*>(y);
  a.ldy = ldy;
  a.s = s;
  a.s_rs = s_row_stride;
  a.s_ks = s_kb_stride;
  a.h = nullptr;
  a.ldh = 0;
  a.ue8m0 = scale_fmt == DSFP8_SCALE_UE8M0;
  return launched(dsfp8::launch_act_quant(a, stream));
}

dsfp8_status dsfp8_silu_mul_act_quant(const void* g, int64_t ldg, const void* u, int64_t ldu, int64_t M, int64_t I,
                                      void* y, int64_t ldy, float* s, int64_t s_row_stride, int64_t s_kb_stride,
                                      void* h, int64_t ldh, int scale_fmt, hipStream_t stream) {
  if (!dim_ok(M) || !dim_ok(I)) return DSFP8_ERR_SHAPE;
  if (scale_fmt != DSFP8_SCALE_FP32 && scale_fmt != DSFP8_SCALE_UE8M0) return DSFP8_ERR_SCALE_FMT;
  DSFP8_TRY(check_mat(g, M, I, ldg, 2));
  DSFP8_TRY(check_mat(u, M, I, ldu, 2));
  DSFP8_TRY(check_quant_out(M, I, y, ldy, s, s_row_stride, s_kb_stride));
  if (h != nullptr) DSFP8_TRY(check_mat(h, M, I, ldh, 2));
  dsfp8::ActQuantArgs a{};
  a.g = static_cast<const uint16_t*>(g);
  a.ldg = ldg;
  a.u = static_cast<const uint16_t*>(u);
  a.ldu = ldu;
  a.M = M;
  a.K = I;
  a.y = static_cast<uint8_t*>(y);
  a.ldy = ldy;
  a.s = s;
  a.s_rs = s_row_stride;
  a.s_ks = s_kb_stride;
  a.h = static_cast<uint16_t*>(h);
  a.ldh = h ? ldh : 0;
  a.ue8m0 = scale_fmt == DSFP8_SCALE_UE8M0;
  // The fused path needs a non-null u to select SiLU gating; an empty problem
  // launches nothing anyway.
  if (M == 0 || I == 0) return DSFP8_OK;
  return launched(dsfp8::launch_act_quant(a, stream));
}

dsfp8_status dsfp8_weight_quant(const void* w, int dtype, int64_t N, int64_t K, int64_t ldw, void* q, int64_t ldq,
                                float* S, int64_t ldS, int scale_fmt, hipStream_t stream) {
  if (!dim_ok(N) || !dim_ok(K)) return DSFP8_ERR_SHAPE;
  if (dtype != DSFP8_DTYPE_F32 && dtype != DSFP8_DTYPE_BF16) return DSFP8_ERR_DTYPE;
  if (scale_fmt != DSFP8_SCALE_FP32 && scale_fmt != DSFP8_SCALE_UE8M0) return DSFP8_ERR_SCALE_FMT;
  DSFP8_TRY(check_mat(w, N, K, ldw, dtype == DSFP8_DTYPE_F32 ? 4 : 2));
  DSFP8_TRY(check_mat(q, N, K, ldq, 1));
  DSFP8_TRY(check_mat(S, nblk(N), nblk(K), ldS, 4));
  dsfp8::WeightQuantArgs a{};
  a.w = w;
  a.bf16_in = dtype == DSFP8_DTYPE_BF16;
  a.N = N;
  a.K = K;
  a.ldw = ldw;
  a.q = static_cast<uint8_t*>(q);
  a.ldq = ldq;
  a.S = S;
  a.ldS = ldS;
  a.ue8m0 = scale_fmt == DSFP8_SCALE_UE8M0;
  return launched(dsfp8::launch_weight_quant(a, stream));
}

dsfp8_status dsfp8_weight_dequant(const void* w, int64_t N, int64_t K, int64_t ldw, const float* S, int64_t ldS,
                                  void* out, int64_t ldo, hipStream_t stream) {
  if (!dim_ok(N) || !dim_ok(K)) return DSFP8_ERR_SHAPE;
  DSFP8_TRY(check_mat(w, N, K, ldw, 1));
  DSFP8_TRY(check_mat(S, nblk(N), nblk(K), ldS, 4));
  DSFP8_TRY(check_mat(out, N, K, ldo, 2));
  dsfp8::DequantArgs a{};
  a.w = static_cast<const uint8_t*>(w);
  a.N = N;
  a.K = K;
  a.ldw = ldw;
  a.S = S;
  a.ldS = ldS;
  a.out = static_cast<uint16_t*>(out);
  a.ldo = ldo;
  return launched(dsfp8::launch_weight_dequant(a, stream));
}

size_t dsfp8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (!dim_ok(M) || !dim_ok(N) || !dim_ok(K)) return 0;
  return dsfp8::gemm_workspace_bytes(M, N, K);
}

dsfp8_status dsfp8_gemm(const void* A, int64_t lda, const float* a_s, int64_t as_row_stride, int64_t as_kb_stride,
                        const void* B, int64_t ldb, const float* b_s, int64_t ldbs, void* C, int64_t ldc, int64_t M,
                        int64_t N, int64_t K, int scale_fmt, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  if (!dim_ok(M) || !dim_ok(N) || !dim_ok(K)) return DSFP8_ERR_SHAPE;
  if (scale_fmt != DSFP8_SCALE_FP32 && scale_fmt != DSFP8_SCALE_UE8M0) return DSFP8_ERR_SCALE_FMT;
  DSFP8_TRY(check_mat(A, M, K, lda, 1));
  DSFP8_TRY(check_scales(a_s, M, nblk(K), as_row_stride, as_kb_stride));
  DSFP8_TRY(check_mat(B, N, K, ldb, 1));
  DSFP8_TRY(check_mat(b_s, nblk(N), nblk(K), ldbs, 4));
  DSFP8_TRY(check_mat(C, M, N, ldc, 2));
  const size_t need = dsfp8_gemm_workspace_bytes(M, N, K);
  if (workspace_bytes < need) return DSFP8_ERR_WORKSPACE;
  if (need > 0 && workspace == nullptr) return DSFP8_ERR_NULL;
  if (!al(workspace, 16)) return DSFP8_ERR_ALIGN;
  dsfp8::GemmArgs a{};
  a.A = static_cast<const uint8_t*>(A);
  a.lda = lda;
  a.a_s = a_s;
  a.as_rs = as_row_stride;
  a.as_ks = as_kb_stride;
  a.B = static_cast<const uint8_t*>(B);
  a.ldb = ldb;
  a.b_s = b_s;
  a.ldbs = ldbs;
  a.C = static_cast<uint16_t*>(C);
  a.ldc = ldc;
  a.M = M;
  a.N = N;
  a.K = K;
  a.partial = static_cast<float*>(workspace);
  a.pow2 = scale_fmt == DSFP8_SCALE_UE8M0;
  return launched(dsfp8::launch_gemm(a, stream));
}

size_t dsfp8_grouped_gemm_workspace_bytes(int64_t E, int64_t M_total, int64_t N, int64_t K) {
  (void)K;
  if (E < 1 || E > kMaxExperts || !dim_ok(M_total) || !dim_ok(N)) return 0;
  return dsfp8::grouped_workspace_bytes(E, M_total, N);
}

namespace {

// The workspace of a grouped launch: the tile schedule, then (when the
// workspace is 16-byte aligned for its int4 entries) the tile plan.
void grouped_workspace(dsfp8::GemmArgs& a, void* workspace) {
  a.tile_start = static_cast<int32_t*>(workspace);
  a.tile_plan = al(workspace, 16) ? reinterpret_cast<int32_t*>(static_cast<uint8_t*>(workspace) +
                                                               dsfp8::grouped_schedule_bytes(a.E))
                                  : nullptr;
}

// Arguments of the grouped product (everything but the workspace).
dsfp8_status grouped_args(const void* A, int64_t lda, const float* a_s, int64_t as_row_stride,
                          int64_t as_kb_stride, const void* B, int64_t ldb, const float* b_s, int64_t ldbs,
                          const int32_t* offsets, int64_t E, int64_t M_total, int64_t N, int64_t K, void* C,
                          int64_t ldc, int scale_fmt, dsfp8::GemmArgs& a) {
  if (!dim_ok(M_total) || !dim_ok(N) || !dim_ok(K)) return DSFP8_ERR_SHAPE;
  if (scale_fmt != DSFP8_SCALE_FP32 && scale_fmt != DSFP8_SCALE_UE8M0) return DSFP8_ERR_SCALE_FMT;
  if (E < 1 || E > kMaxExperts) return DSFP8_ERR_SHAPE;
  if (offsets == nullptr) return DSFP8_ERR_NULL;
  if (!al(offsets, 4)) return DSFP8_ERR_ALIGN;
  DSFP8_TRY(check_mat(A, M_total, K, lda, 1));
  DSFP8_TRY(check_scales(a_s, M_total, nblk(K), as_row_stride, as_kb_stride));
  // Every expert's weight must exist even when no row is routed to it.
  DSFP8_TRY(check_mat(B, E * N, K, ldb, 1));
  DSFP8_TRY(check_mat(b_s, E * nblk(N), nblk(K), ldbs, 4));
  DSFP8_TRY(check_mat(C, M_total, N, ldc, 2));
  a = dsfp8::GemmArgs{};
  a.A = static_cast<const uint8_t*>(A);
  a.lda = lda;
  a.a_s = a_s;
  a.as_rs = as_row_stride;
  a.as_ks = as_kb_stride;
  a.B = static_cast<const uint8_t*>(B);
  a.ldb = ldb;
  a.b_s = b_s;
  a.ldbs = ldbs;
  a.C = static_cast<uint16_t*>(C);
  a.ldc = ldc;
  a.M = M_total;
  a.N = N;
  a.K = K;
  a.offsets = offsets;
  a.E = E;
  a.pow2 = scale_fmt == DSFP8_SCALE_UE8M0;
  return DSFP8_OK;
}

}  // namespace

dsfp8_status dsfp8_grouped_gemm(const void* A, int64_t lda, const float* a_s, int64_t as_row_stride,
                                int64_t as_kb_stride, const void* B, int64_t ldb, const float* b_s, int64_t ldbs,
                                const int32_t* offsets, int64_t E, int64_t M_total, int64_t N, int64_t K, void* C,
                                int64_t ldc, int scale_fmt, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  dsfp8::GemmArgs a;
  DSFP8_TRY(grouped_args(A, lda, a_s, as_row_stride, as_kb_stride, B, ldb, b_s, ldbs, offsets, E, M_total, N, K, C,
                         ldc, scale_fmt, a));
  const size_t need = dsfp8_grouped_gemm_workspace_bytes(E, M_total, N, K);
  if (workspace_bytes < need) return DSFP8_ERR_WORKSPACE;
  if (need > 0 && workspace == nullptr) return DSFP8_ERR_NULL;
  if (!al(workspace, 4)) return DSFP8_ERR_ALIGN;
  grouped_workspace(a, workspace);
  return launched(dsfp8::launch_grouped_gemm(a, stream));
}

dsfp8_status dsfp8_grouped_gemm_noalloc(const void* A, int64_t lda, const float* a_s, int64_t as_row_stride,
                                        int64_t as_kb_stride, const void* B, int64_t ldb, const float* b_s,
                                        int64_t ldbs, const int32_t* offsets, int64_t E, int64_t M_total, int64_t N,
                                        int64_t K, void* C, int64_t ldc, int scale_fmt, hipStream_t stream) {
  dsfp8::GemmArgs a;
  DSFP8_TRY(grouped_args(A, lda, a_s, as_row_stride, as_kb_stride, B, ldb, b_s, ldbs, offsets, E, M_total, N, K, C,
                         ldc, scale_fmt, a));
  if (E > DSFP8_NOALLOC_MAX_EXPERTS) return DSFP8_ERR_SCRATCH;
  static_assert(DSFP8_NOALLOC_MAX_EXPERTS == dsfp8::kNoAllocMaxExperts, "header and library agree");
  return launched(dsfp8::launch_grouped_gemm_noalloc(a, stream));
}

namespace {

// Arguments of the gated product, checked as the product and the quantiser
// check theirs; E experts of 2F weight rows each (E = 1: the dense form).
dsfp8_status glu_args(const void* A, int64_t a_rows, int64_t lda, const float* a_s, int64_t as_rs, int64_t as_ks,
                      const void* W13, int64_t ldw, const float* w_s, int64_t ldws, int64_t E, int64_t M, int64_t F,
                      int64_t K, void* y, int64_t ldy, float* s, int64_t s_rs, int64_t s_ks, void* h, int64_t ldh,
                      int scale_fmt, dsfp8::GemmArgs& a) {
  if (!dim_ok(M) || !dim_ok(F) || !dim_ok(K) || !dim_ok(2 * F) || !dim_ok(a_rows)) return DSFP8_ERR_SHAPE;
  if (scale_fmt != DSFP8_SCALE_FP32 && scale_fmt != DSFP8_SCALE_UE8M0) return DSFP8_ERR_SCALE_FMT;
  DSFP8_TRY(check_mat(A, a_rows, K, lda, 1));
  DSFP8_TRY(check_scales(a_s, a_rows, nblk(K), as_rs, as_ks));
  DSFP8_TRY(check_mat(W13, E * 2 * F, K, ldw, 1));
  DSFP8_TRY(check_mat(w_s, E * nblk(2 * F), nblk(K), ldws, 4));
  DSFP8_TRY(check_quant_out(M, F, y, ldy, s, s_rs, s_ks));
  if (h != nullptr) DSFP8_TRY(check_mat(h, M, F, ldh, 2));
  a = dsfp8::GemmArgs{};
  a.A = static_cast<const uint8_t*>(A);
  a.lda = lda;
  a.a_s = a_s;
  a.as_rs = as_rs;
  a.as_ks = as_ks;
  a.B = static_cast<const uint8_t*>(W13);
  a.ldb = ldw;
  a.b_s = w_s;
  a.ldbs = ldws;
  a.M = M;
  a.N = 2 * F;
  a.K = K;
  a.pow2 = scale_fmt == DSFP8_SCALE_UE8M0;
  a.glu_f = F;
  a.qy = static_cast<uint8_t*>(y);
  a.ldqy = ldy;
  a.qs = s;
  a.qs_rs = s_rs;
  a.qs_ks = s_ks;
  a.qh = static_cast<uint16_t*>(h);
  a.ldqh = h ? ldh : 0;
  a.q_ue8m0 = scale_fmt == DSFP8_SCALE_UE8M0;
  if (M > 0 && F > 0 && !dsfp8::gemm_glu_supported(a)) return DSFP8_ERR_UNSUPPORTED;
  return DSFP8_OK;
}

}  // namespace

namespace {

// The grouped gated product, with A's rows read directly (rows == NULL,
// a_rows == M_total) or through the index rows.
dsfp8_status grouped_glu(const void* A, int64_t a_rows, int64_t lda, const float* a_s, int64_t as_rs, int64_t as_ks,
                         const int32_t* rows, const void* W13, int64_t ldw, const float* w_s, int64_t ldws,
                         const int32_t* offsets, int64_t E, int64_t M_total, int64_t F, int64_t K, void* y,
                         int64_t ldy, float* s, int64_t s_rs, int64_t s_ks, void* h, int64_t ldh, int scale_fmt,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (E < 1 || E > kMaxExperts) return DSFP8_ERR_SHAPE;
  if (offsets == nullptr) return DSFP8_ERR_NULL;
  if (!al(offsets, 4)) return DSFP8_ERR_ALIGN;
  dsfp8::GemmArgs a;
  DSFP8_TRY(glu_args(A, a_rows, lda, a_s, as_rs, as_ks, W13, ldw, w_s, ldws, E, M_total, F, K, y, ldy, s, s_rs, s_ks,
                     h, ldh, scale_fmt, a));
  const size_t need = dsfp8_grouped_gemm_workspace_bytes(E, M_total, 2 * F, K);
  if (workspace_bytes < need) return DSFP8_ERR_WORKSPACE;
  if (need > 0 && workspace == nullptr) return DSFP8_ERR_NULL;
  if (!al(workspace, 4)) return DSFP8_ERR_ALIGN;
  if (rows != nullptr) {
    // one buffer descriptor spans every row of A (32-bit offsets); lda is
    // tested first so that the product cannot overflow
    if (lda >= ((int64_t)1 << 31) || a_rows * lda + K >= ((int64_t)1 << 31)) return DSFP8_ERR_UNSUPPORTED;
    a.a_rows = rows;
    a.a_rows_n = a_rows;
  }
  if (M_total == 0 || F == 0) return DSFP8_OK;
  a.offsets = offsets;
  a.E = E;
  grouped_workspace(a, workspace);
  return launched(dsfp8::launch_grouped_gemm_glu(a, stream));
}

}  // namespace

dsfp8_status dsfp8_gemm_silu_mul_act_quant(const void* A, int64_t lda, const float* a_s, int64_t as_row_stride,
                                           int64_t as_kb_stride, const void* W13, int64_t ldw, const float* w_s,
                                           int64_t ldws, int64_t M, int64_t F, int64_t K, void* y, int64_t ldy,
                                           float* s, int64_t s_row_stride, int64_t s_kb_stride, void* h,
                                           int64_t ldh, int scale_fmt, hipStream_t stream) {
  dsfp8::GemmArgs a;
  DSFP8_TRY(glu_args(A, M, lda, a_s, as_row_stride, as_kb_stride, W13, ldw, w_s, ldws, 1, M, F, K, y, ldy, s,
                     s_row_stride, s_kb_stride, h, ldh, scale_fmt, a));
  if (M == 0 || F == 0) return DSFP8_OK;
  return launched(dsfp8::launch_gemm_glu(a, stream));
}

dsfp8_status dsfp8_grouped_gemm_silu_mul_act_quant(const void* A, int64_t lda, const float* a_s,
                                                   int64_t as_row_stride, int64_t as_kb_stride, const void* W13,
                                                   int64_t ldw, const float* w_s, int64_t ldws,
                                                   const int32_t* offsets, int64_t E, int64_t M_total, int64_t F,
                                                   int64_t K, void* y, int64_t ldy, float* s, int64_t s_row_stride,
                                                   int64_t s_kb_stride, void* h, int64_t ldh, int scale_fmt,
                                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return grouped_glu(A, M_total, lda, a_s, as_row_stride, as_kb_stride, nullptr, W13, ldw, w_s, ldws, offsets, E,
                     M_total, F, K, y, ldy, s, s_row_stride, s_kb_stride, h, ldh, scale_fmt, workspace,
                     workspace_bytes, stream);
}

dsfp8_status dsfp8_grouped_gemm_silu_mul_act_quant_gather(const void* A, int64_t a_rows, int64_t lda,
                                                          const float* a_s, int64_t as_row_stride,
                                                          int64_t as_kb_stride, const int32_t* rows,
                                                          const void* W13, int64_t ldw, const float* w_s,
                                                          int64_t ldws, const int32_t* offsets, int64_t E,
                                                          int64_t M_total, int64_t F, int64_t K, void* y,
                                                          int64_t ldy, float* s, int64_t s_row_stride,
                                                          int64_t s_kb_stride, void* h, int64_t ldh, int scale_fmt,
                                                          void* workspace, size_t workspace_bytes,
                                                          hipStream_t stream) {
  if (M_total > 0 && rows == nullptr) return DSFP8_ERR_NULL;
  if (!al(rows, 4)) return DSFP8_ERR_ALIGN;
  if (M_total > 0 && a_rows < 1) return DSFP8_ERR_SHAPE;
  return grouped_glu(A, a_rows, lda, a_s, as_row_stride, as_kb_stride, rows, W13, ldw, w_s, ldws, offsets, E,
                     M_total, F, K, y, ldy, s, s_row_stride, s_kb_stride, h, ldh, scale_fmt, workspace,
                     workspace_bytes, stream);
}

dsfp8_status dsfp8_act_quant_rows(const void* x, int64_t x_rows, int64_t ldx, const int32_t* rows, int64_t M,
                                  int64_t K, void* y, int64_t ldy, float* s, int64_t s_row_stride,
                                  int64_t s_kb_stride, int scale_fmt, hipStream_t stream) {
  if (!dim_ok(M) || !dim_ok(K) || !dim_ok(x_rows)) return DSFP8_ERR_SHAPE;
  if (M > 0 && K > 0 && x_rows == 0) return DSFP8_ERR_SHAPE;
  if (scale_fmt != DSFP8_SCALE_FP32 && scale_fmt != DSFP8_SCALE_UE8M0) return DSFP8_ERR_SCALE_FMT;
  DSFP8_TRY(check_mat(x, x_rows, K, ldx, 2));
  if (M > 0 && rows == nullptr) return DSFP8_ERR_NULL;
  if (!al(rows, 4)) return DSFP8_ERR_ALIGN;
  DSFP8_TRY(check_quant_out(M, K, y, ldy, s, s_row_stride, s_kb_stride));
  dsfp8::ActQuantArgs a{};
  a.g = static_cast<const uint16_t*>(x);
  a.ldg = ldx;
  a.M = M;
  a.K = K;
  a.y = static_cast<uint8_t*>(y);
  a.ldy = ldy;
  a.s = s;
  a.s_rs = s_row_stride;
  a.s_ks = s_kb_stride;
  a.ue8m0 = scale_fmt == DSFP8_SCALE_UE8M0;
  a.rows = rows;
  a.g_rows = x_rows;
  return launched(dsfp8::launch_act_quant(a, stream));
}

size_t dsfp8_moe_route_workspace_bytes(int64_t T, int64_t k, int64_t E) {
  if (!dim_ok(T) || k < 1 || k > 16 || E < 1 || E > dsfp8::kMaxRouteExperts) return 0;
  if (T * k >= kMaxDim) return 0;
  return dsfp8::route_workspace_bytes(T * k, E);
}

dsfp8_status dsfp8_moe_route(const int32_t* indices, int64_t T, int64_t k, int64_t ldi, int64_t E, int32_t* offsets,
                             int32_t* row_token, int32_t* token_rows, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  if (!dim_ok(T) || k < 1 || k > 16 || E < 1 || E > dsfp8::kMaxRouteExperts) return DSFP8_ERR_SHAPE;
  if (T * k >= kMaxDim) return DSFP8_ERR_SHAPE;
  DSFP8_TRY(check_mat(indices, T, k, ldi, 4));
  DSFP8_TRY(check_mat(token_rows, T, k, k, 4));
  DSFP8_TRY(check_mat(row_token, T * k, 1, 1, 4));
  DSFP8_TRY(check_mat(offsets, E + 1, 1, 1, 4));
  const size_t need = dsfp8_moe_route_workspace_bytes(T, k, E);
  if (workspace_bytes < need) return DSFP8_ERR_WORKSPACE;
  if (workspace == nullptr) return DSFP8_ERR_NULL;
  if (!al(workspace, 4)) return DSFP8_ERR_ALIGN;
  dsfp8::RouteArgs a{};
  a.indices = indices;
  a.ldi = ldi;
  a.k = k;
  a.n = T * k;
  a.E = (int)E;
  a.offsets = offsets;
  a.row_token = row_token;
  a.token_rows = token_rows;
  a.work = static_cast<int32_t*>(workspace);
  return launched(dsfp8::launch_route(a, stream));
}

dsfp8_status dsfp8_moe_combine(const void* yr, int64_t R, int64_t ldy, const int32_t* indices, int64_t ldi,
                               const void* weights, int64_t ldw, const int32_t* token_rows, int64_t T, int64_t k,
                               int64_t D, void* out, int64_t ldo, hipStream_t stream) {
  if (!dim_ok(R) || !dim_ok(T) || !dim_ok(D) || k < 1 || k > 16) return DSFP8_ERR_SHAPE;
  DSFP8_TRY(check_mat(yr, R, D, ldy, 2));
  DSFP8_TRY(check_mat(indices, T, k, ldi, 4));
  DSFP8_TRY(check_mat(weights, T, k, ldw, 2));
  DSFP8_TRY(check_mat(token_rows, T, k, k, 4));
  DSFP8_TRY(check_mat(out, T, D, ldo, 2));
  dsfp8::CombineArgs a{};
  a.yr = static_cast<const uint16_t*>(yr);
  a.ldy = ldy;
  a.R = R;
  a.indices = indices;
  a.ldi = ldi;
  a.weights = static_cast<const uint16_t*>(weights);
  a.ldw = ldw;
  a.token_rows = token_rows;
  a.T = T;
  a.k = k;
  a.D = D;
  a.out = static_cast<uint16_t*>(out);
  a.ldo = ldo;
  return launched(dsfp8::launch_combine(a, stream));
}

}  // extern "C"
