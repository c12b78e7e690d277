// Internal launch interface between the C ABI (api.cpp) and the kernels.
// Arguments reaching these functions have already been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsfp8 {

struct ActQuantArgs {
  const uint16_t* g;  // bf16 input (the SiLU gate input when u != nullptr)
  int64_t ldg;
  const uint16_t* u;  // bf16 up-projection input, or nullptr for plain act_quant
  int64_t ldu;
  int64_t M, K;
  uint8_t* y;
  int64_t ldy;
  float* s;
  int64_t s_rs, s_ks;  // scale (m, b) at s[m * s_rs + b * s_ks]
  uint16_t* h;        // optional bf16 output of SiLU(g)*u
  int64_t ldh;
  bool ue8m0;
  // optional row gather (plain act_quant only): output row m quantises input
  // row rows[m], clamped to [0, g_rows)
  const int32_t* rows;
  int64_t g_rows;
};

// Routing of T*k (token, slot) pairs to experts (stable counting sort).
constexpr int kRouteChunk = 512;      // least pairs per chunk
constexpr int kMaxRouteChunks = 64;   // most chunks
constexpr int kMaxRouteExperts = 4096;
struct RouteArgs {
  const int32_t* indices;  // [T, k], row stride ldi
  int64_t ldi, k, n;       // n = T * k
  int E;
  int32_t* offsets;        // [E + 1]
  int32_t* row_token;      // [n]
  int32_t* token_rows;     // [T, k] contiguous
  int32_t* work;           // [chunks, E]
  int64_t chunk, chunks;   // pairs per chunk, number of chunks
};

// Weighted combine of the expert outputs per token.
struct CombineArgs {
  const uint16_t* yr;  // bf16 [R, D], row stride ldy
  int64_t ldy, R;
  const int32_t* indices;     // [T, k], row stride ldi
  int64_t ldi;
  const uint16_t* weights;    // bf16 [T, k], row stride ldw
  int64_t ldw;
  const int32_t* token_rows;  // [T, k] contiguous
  int64_t T, k, D;
  uint16_t* out;              // bf16 [T, D], row stride ldo
  int64_t ldo;
  bool vec;
};

struct WeightQuantArgs {
  const void* w;
  bool bf16_in;
  int64_t N, K, ldw;
  uint8_t* q;
  int64_t ldq;
  float* S;
  int64_t ldS;
  bool ue8m0;
};

struct DequantArgs {
  const uint8_t* w;
  int64_t N, K, ldw;
  const float* S;
  int64_t ldS;
  uint16_t* out;
  int64_t ldo;
};

struct GemmArgs {
  const uint8_t* A;
  int64_t lda;
  const float* a_s;
  int64_t as_rs, as_ks;  // activation scale (m, b) at a_s[m * as_rs + b * as_ks]
  const uint8_t* B;
  int64_t ldb;
  const float* b_s;
  int64_t ldbs;
  uint16_t* C;
  int64_t ldc;
  int64_t M, N, K;
  // grouped form only
  const int32_t* offsets;
  int64_t E;
  int32_t* tile_start;  // workspace: E+1 ints (this launch's tile class)
  // workspace after the schedule: the merged launch's tile of every
  // workgroup, 4 ints each (NULL: each workgroup maps its id itself)
  int32_t* tile_plan;
  // tile classes of the grouped launches: this launch's class, the number of
  // classes and their row-tile heights (increasing)
  int grp_class, grp_classes;
  int grp_h[3];
  // dense form with split K: fp32 partial products [splits, M, N] (workspace)
  float* partial;
  // every scale is a power of two: the MFMA applies them (exponents only)
  bool pow2;
  // grouped gated form: product row r reads row a_rows[r] of A and a_s
  // (clamped to [0, a_rows_n)); NULL: row r itself
  const int32_t* a_rows;
  int64_t a_rows_n;
  // gated form: B stacks w1 (rows 0..F-1) over w3 (rows F..2F-1), N = 2F; the
  // epilogue computes h = bf16(SiLU(bf16(x w1^T)) * bf16(x w3^T)) and writes
  // act_quant(h) as e4m3 qy [M, F] and fp32 scales qs (element (m, b) at
  // qs[m * qs_rs + b * qs_ks]), and h itself to qh when that is not null.
  int64_t glu_f;   // F (0: plain product into C)
  int64_t glu_nt;  // output column blocks of 128 this launch computes (0: all F / 128)
  uint8_t* qy;
  int64_t ldqy;
  float* qs;
  int64_t qs_rs, qs_ks;
  uint16_t* qh;
  int64_t ldqh;
  bool q_ue8m0;
};

hipError_t launch_act_quant(const ActQuantArgs& a, hipStream_t stream);
// Gated products: false if the operands do not fit the direct-to-LDS pipeline
// the gated epilogue is built on (nothing launched).
bool gemm_glu_supported(const GemmArgs& a);
hipError_t launch_gemm_glu(const GemmArgs& a, hipStream_t stream);
hipError_t launch_grouped_gemm_glu(const GemmArgs& a, hipStream_t stream);
hipError_t launch_route(RouteArgs a, hipStream_t stream);
size_t route_workspace_bytes(int64_t n, int64_t E);
hipError_t launch_combine(CombineArgs a, hipStream_t stream);
hipError_t launch_weight_quant(const WeightQuantArgs& a, hipStream_t stream);
hipError_t launch_weight_dequant(const DequantArgs& a, hipStream_t stream);
hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream);
hipError_t launch_grouped_gemm(const GemmArgs& a, hipStream_t stream);

size_t grouped_schedule_bytes(int64_t E);
size_t grouped_workspace_bytes(int64_t E, int64_t M, int64_t N);
int64_t merged_workgroups(int64_t E, int64_t M, int64_t tn);

// The grouped product with its tile schedule in a static device array of
// 3 * (kNoAllocMaxExperts + 1) int32 per GPU instead of a caller workspace
// (for callers that cannot allocate).  Calls that overlap on one GPU share
// the array and race.
constexpr int64_t kNoAllocMaxExperts = 4096;
hipError_t launch_grouped_gemm_noalloc(GemmArgs a, hipStream_t stream);

// Number of K splits the dense product uses for this shape (1 = none), and the
// fp32 workspace that requires.  Small products (few output tiles) split their
// K-blocks over several workgroups so that the weight streams from every CU.
int gemm_k_splits(int64_t M, int64_t N, int64_t K);
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

// Number of compute units of the current device (cached per device).
int device_cu_count();

}  // namespace dsfp8
