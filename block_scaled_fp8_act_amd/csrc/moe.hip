// Routed-expert steps around the grouped product on gfx950 ("DeepSeek-V3
// Administrator & Developer Guide", sections 6.4 and 8.4: for each expert in
// increasing order, the (token, slot) pairs that chose it run through the
// expert, and each token's output accumulates weight * expert output).
//
// Routing: a stable counting sort of the T*k pairs by expert.  The rows of
// expert e are its pairs in increasing pair index t*k + j (the order in which
// torch.where lists them).  Three kernels, none with global atomics, so the
// result is deterministic:
//   count   -- one workgroup per chunk of kRouteChunk pairs, per-expert counts
//              in LDS;
//   scan    -- one workgroup: exclusive prefix over (expert, chunk) in
//              expert-major order, giving every chunk's first row per expert
//              and the expert offsets;
//   scatter -- one wavefront per chunk, 64 pairs at a time: a lane's row is
//              the chunk's running count of its expert plus the number of
//              lower lanes with the same expert.
//
// Combine: one token per workgroup row, 8 columns per lane; the token's
// contributions are taken in increasing expert order, each weighted product
// rounded to bf16 and each addition rounded to bf16, as the pages' bf16 loop
// computes them.  A product of two bf16 values and the sum of two bf16 values
// are exact in fp32, so one fp32 operation followed by bf16 rounding gives
// the correctly rounded bf16 result.
#include "device.h"
#include "launch.h"

namespace dsfp8 {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---- routing -----------------------------------------------------------------------

__global__ __launch_bounds__(64) void route_count_kernel(RouteArgs a) {
  extern __shared__ int32_t cnt[];
  const int lane = threadIdx.x;
  for (int e = lane; e < a.E; e += 64) cnt[e] = 0;
  __syncthreads();
  const int64_t p0 = (int64_t)blockIdx.x * kRouteChunk;
  for (int i = lane; i < kRouteChunk; i += 64) {
    const int64_t p = p0 + i;
    if (p >= a.n) break;
    const int32_t e = a.indices[(p / a.k) * a.ldi + p % a.k];
    if (e >= 0 && e < a.E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  for (int e = lane; e < a.E; e += 64) a.work[(int64_t)blockIdx.x * a.E + e] = cnt[e];
}

// Exclusive prefix over q = e * chunks + c (expert-major) of work[c * E + e],
// written back in place; offsets[e] = first row of expert e, offsets[E] = the
// number of routed pairs.  Each thread scans a contiguous range of q.
constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void route_scan_kernel(RouteArgs a) {
  __shared__ int64_t part[kScanThreads];
  const int t = threadIdx.x;
  if (a.chunks == 0) {  // no pairs: every expert is empty
    for (int e = t; e <= a.E; e += kScanThreads) a.offsets[e] = 0;
    return;
  }
  const int64_t Q = a.chunks * a.E;
  const int64_t per = (Q + kScanThreads - 1) / kScanThreads;
  const int64_t q0 = t * per, q1 = q0 + per < Q ? q0 + per : Q;
  auto at = [&](int64_t q) -> int32_t& {
    const int64_t e = q / a.chunks, c = q % a.chunks;
    return a.work[c * a.E + e];
  };
  int64_t sum = 0;
  for (int64_t q = q0; q < q1; ++q) sum += at(q);
  part[t] = sum;
  __syncthreads();
  // Inclusive scan of the per-thread sums (Hillis-Steele over LDS).
  for (int d = 1; d < kScanThreads; d <<= 1) {
    const int64_t v = t >= d ? part[t - d] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int64_t run = t > 0 ? part[t - 1] : 0;
  for (int64_t q = q0; q < q1; ++q) {
    int32_t& w = at(q);
    const int32_t c = w;
    if (q % a.chunks == 0) a.offsets[q / a.chunks] = (int32_t)run;
    w = (int32_t)run;
    run += c;
  }
  if (t == kScanThreads - 1) a.offsets[a.E] = (int32_t)part[kScanThreads - 1];
}

__global__ __launch_bounds__(64) void route_scatter_kernel(RouteArgs a) {
  extern __shared__ int32_t next[];
  const int lane = threadIdx.x;
  for (int e = lane; e < a.E; e += 64) next[e] = a.work[(int64_t)blockIdx.x * a.E + e];
  __syncthreads();
  const int64_t p0 = (int64_t)blockIdx.x * kRouteChunk;
  for (int r = 0; r < kRouteChunk / 64; ++r) {
    const int64_t p = p0 + r * 64 + lane;
    const bool in = p < a.n;
    const int64_t t = in ? p / a.k : 0;
    const int32_t e = in ? a.indices[t * a.ldi + p % a.k] : -1;
    const bool valid = e >= 0 && e < a.E;
    int rank = 0, later = 0;
#pragma unroll
    for (int l = 0; l < 64; ++l) {
      const int32_t el = __builtin_amdgcn_readlane(e, l);
      rank += (el == e && l < lane) ? 1 : 0;
      later += (el == e && l > lane) ? 1 : 0;
    }
    // Every lane reads its expert's running count before the last lane of
    // each expert advances it (LDS operations of one wavefront complete in
    // order).
    const int32_t pos = valid ? next[e] + rank : -1;
    if (valid) a.row_token[pos] = (int32_t)t;
    if (in) a.token_rows[p] = pos;
    if (valid && later == 0) next[e] = pos + 1;
    __builtin_amdgcn_wave_barrier();
  }
}

// ---- combine --------------------------------------------------------------------------

constexpr int kCombineThreads = 256;

__device__ __forceinline__ float bf16_round(float v) { return bf16_lo(pack_bf16x2(v, 0.0f)); }

template <int KMAX>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(CombineArgs a) {
  const int64_t t = blockIdx.x;
  const int64_t col = ((int64_t)blockIdx.y * kCombineThreads + threadIdx.x) * 8;
  if (col >= a.D) return;
  // The token's pairs, sorted by expert (insertion sort, stable).
  int32_t ex[KMAX], row[KMAX];
  float w[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const bool use = j < a.k;
    ex[j] = use ? a.indices[t * a.ldi + j] : INT32_MAX;
    row[j] = use ? a.token_rows[t * a.k + j] : -1;
    w[j] = use ? bf16_lo(a.weights[t * a.ldw + j]) : 0.0f;
  }
#pragma unroll
  for (int i = 1; i < KMAX; ++i)
#pragma unroll
    for (int j = i; j > 0; --j) {
      const bool sw = ex[j] < ex[j - 1];
      const int32_t e0 = ex[j - 1], r0 = row[j - 1];
      const float w0 = w[j - 1];
      ex[j - 1] = sw ? ex[j] : e0;   row[j - 1] = sw ? row[j] : r0;   w[j - 1] = sw ? w[j] : w0;
      ex[j] = sw ? e0 : ex[j];       row[j] = sw ? r0 : row[j];       w[j] = sw ? w0 : w[j];
    }
  // All rows' loads in flight before the accumulation.
  u32x4 v[KMAX];
  const bool vec = a.vec && col + 8 <= a.D;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    v[j] = u32x4{0u, 0u, 0u, 0u};
    if (row[j] < 0 || row[j] >= a.R) continue;
    const uint16_t* src = a.yr + (int64_t)row[j] * a.ldy + col;
    if (vec) {
      v[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
    } else {
      uint32_t e[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) e[c] = col + c < a.D ? (uint32_t)src[c] : 0u;
      v[j] = u32x4{e[0] | e[1] << 16, e[2] | e[3] << 16, e[4] | e[5] << 16, e[6] | e[7] << 16};
    }
  }
  float acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (row[j] < 0 || row[j] >= a.R) continue;
    const uint32_t words[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float y = (c & 1) ? bf16_hi(words[c >> 1]) : bf16_lo(words[c >> 1]);
      acc[c] = bf16_round(acc[c] + bf16_round(y * w[j]));
    }
  }
  uint16_t* dst = a.out + t * a.ldo + col;
  if (vec) {
    *reinterpret_cast<u32x4*>(dst) = u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                           pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
  } else {
#pragma unroll
    for (int c = 0; c < 8; ++c)
      if (col + c < a.D) dst[c] = (uint16_t)(pack_bf16x2(acc[c], 0.0f) & 0xffff);
  }
}

inline bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

}  // namespace

size_t route_workspace_bytes(int64_t n, int64_t E) {
  const int64_t chunks = (n + kRouteChunk - 1) / kRouteChunk;
  return (size_t)(chunks > 0 ? chunks : 1) * (size_t)E * sizeof(int32_t);
}

hipError_t launch_route(RouteArgs a, hipStream_t stream) {
  a.chunks = (a.n + kRouteChunk - 1) / kRouteChunk;
  const size_t lds = (size_t)a.E * sizeof(int32_t);
  if (a.chunks > 0) {
    hipLaunchKernelGGL(route_count_kernel, dim3((unsigned)a.chunks), dim3(64), lds, stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.chunks == 0) return err;
  hipLaunchKernelGGL(route_scatter_kernel, dim3((unsigned)a.chunks), dim3(64), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_combine(CombineArgs a, hipStream_t stream) {
  if (a.T == 0 || a.D == 0) return hipSuccess;
  a.vec = aligned(a.yr, 16) && a.ldy % 8 == 0 && aligned(a.out, 16) && a.ldo % 8 == 0;
  dim3 g((unsigned)a.T, (unsigned)((a.D + kCombineThreads * 8 - 1) / (kCombineThreads * 8)));
  dim3 blk(kCombineThreads);
  if (a.k <= 2) hipLaunchKernelGGL(combine_kernel<2>, g, blk, 0, stream, a);
  else if (a.k <= 4) hipLaunchKernelGGL(combine_kernel<4>, g, blk, 0, stream, a);
  else if (a.k <= 8) hipLaunchKernelGGL(combine_kernel<8>, g, blk, 0, stream, a);
  else hipLaunchKernelGGL(combine_kernel<16>, g, blk, 0, stream, a);
  return hipGetLastError();
}

}  // namespace dsfp8
