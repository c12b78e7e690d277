// Routed-expert steps around the grouped product on gfx950 ("DeepSeek-V3
// Administrator & Developer Guide", sections 6.4 and 8.4: for each expert in
// increasing order, the (token, slot) pairs that chose it run through the
// expert, and each token's output accumulates weight * expert output).
//
// Routing: a stable counting sort of the T*k pairs by expert (T*k < 2^31, so
// pair indices are divided by k in 32 bits).  The rows of
// expert e are its pairs in increasing pair index t*k + j (the order in which
// torch.where lists them).  Two kernels, no atomics on global memory, so the
// result is deterministic:
//   count   -- one workgroup per chunk of pairs, per-expert counts in LDS,
//              stored chunk-major (counts[c][e], so that a wave's reads of
//              one chunk's counts for consecutive experts are contiguous);
//   scatter -- one workgroup per chunk.  All its threads first reduce the
//              (small) count table: expert totals, an exclusive scan of them
//              for the expert offsets, and the counts of earlier chunks, so
//              the chunk's first row for each expert is known.  Then one
//              wavefront walks the chunk 64 pairs at a time: a lane's row is
//              the running count of its expert plus the number of lower lanes
//              with the same expert (found with ballots over the bits of the
//              expert index).
// The chunk size grows with the number of pairs so that there are at most
// kMaxRouteChunks chunks and the table stays small.
//
// Combine: one token per workgroup row, 8 columns per lane; the token's
// contributions are taken in increasing expert order, each weighted product
// rounded to bf16 and each addition rounded to bf16, as the pages' bf16 loop
// computes them.  Each step is one fp32 operation followed by rounding to
// bf16, and that equals the correctly rounded bf16 result: a product of two
// bf16 values (8-bit significands) is exact in fp32; a sum of two bf16 values
// is not always exact in fp32 (exponents more than 16 apart), but rounding it
// first to fp32 and then to bf16 gives the same bf16 value as rounding the
// exact sum once, because fp32's 24-bit significand is at least 2 * 8 + 2
// bits (double rounding to nearest is then innocuous; S. A. Figueroa, "When
// is double rounding innocuous?", 1995).
#include "device.h"
#include "launch.h"

namespace dsfp8 {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---- routing -----------------------------------------------------------------------

constexpr int kRouteExpertBits = 12;  // experts below 2^12
static_assert(kMaxRouteExperts <= (1 << kRouteExpertBits), "expert bits");
constexpr int kRouteThreads = 256;

__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ __launch_bounds__(kRouteThreads) void route_count_kernel(RouteArgs a) {
  extern __shared__ int32_t cnt[];
  const int t = threadIdx.x;
  for (int e = t; e < a.E; e += kRouteThreads) cnt[e] = 0;
  __syncthreads();
  const int64_t p0 = (int64_t)blockIdx.x * a.chunk;
  const int64_t p1 = p0 + a.chunk < a.n ? p0 + a.chunk : a.n;
  for (int64_t p = p0 + t; p < p1; p += kRouteThreads) {
    const int32_t e = a.indices[(int64_t)((uint32_t)p / (uint32_t)a.k) * a.ldi + (uint32_t)p % (uint32_t)a.k];
    if (e >= 0 && e < a.E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  for (int e = t; e < a.E; e += kRouteThreads) a.work[(int64_t)blockIdx.x * a.E + e] = cnt[e];
}

__global__ __launch_bounds__(kRouteThreads) void route_scatter_kernel(RouteArgs a) {
  extern __shared__ int32_t lds[];
  int32_t* next = lds;                       // [E]: next row of each expert
  int32_t* total = lds + a.E;                // [E]: pairs of each expert
  __shared__ int32_t wsum[kRouteThreads];
  const int t = threadIdx.x;
  const int c = blockIdx.x;
  // Per expert: the total over all chunks and the part in chunks before this
  // one.  An expert's counts in every chunk (at most kMaxRouteChunks) are
  // loaded at once; consecutive threads take consecutive experts, so each
  // load instruction reads one contiguous stretch of a chunk's row.  A
  // thread's experts are contiguous, so the exclusive scan of the totals is
  // a per-thread sum plus a block scan.
  const int per = (a.E + kRouteThreads - 1) / kRouteThreads;
  const int e0 = t * per < a.E ? t * per : a.E;
  const int e1 = e0 + per < a.E ? e0 + per : a.E;
  int32_t tsum = 0;
  for (int e = e0; e < e1; ++e) {
    int32_t v[kMaxRouteChunks];
#pragma unroll
    for (int j = 0; j < kMaxRouteChunks; ++j) v[j] = j < a.chunks ? a.work[(int64_t)j * a.E + e] : 0;
    int32_t tot = 0, before = 0;
#pragma unroll
    for (int j = 0; j < kMaxRouteChunks; ++j) {
      tot += v[j];
      before += j < c ? v[j] : 0;
    }
    next[e] = before;
    total[e] = tot;
    tsum += tot;
  }
  wsum[t] = tsum;
  __syncthreads();
  for (int d = 1; d < kRouteThreads; d <<= 1) {
    const int32_t v = t >= d ? wsum[t - d] : 0;
    __syncthreads();
    wsum[t] += v;
    __syncthreads();
  }
  // Expert e's first row is the scanned total of the experts before it.
  int32_t run = t > 0 ? wsum[t - 1] : 0;
  for (int e = e0; e < e1; ++e) {
    if (c == 0) a.offsets[e] = run;
    next[e] += run;
    run += total[e];
  }
  if (c == 0 && t == kRouteThreads - 1) a.offsets[a.E] = wsum[kRouteThreads - 1];
  __syncthreads();
  if (t >= 64) return;

  // One wavefront assigns the chunk's rows, 64 pairs per round; the indices
  // of kBatch rounds are loaded together.
  const int lane = t;
  const int64_t p0 = (int64_t)c * a.chunk;
  const int64_t p1 = p0 + a.chunk < a.n ? p0 + a.chunk : a.n;
  constexpr int kBatch = 8;
  for (int64_t pbb = p0; pbb < p1; pbb += 64 * kBatch) {
    int32_t ev[kBatch];
#pragma unroll
    for (int r = 0; r < kBatch; ++r) {
      const int64_t p = pbb + r * 64 + lane;
      ev[r] = p < p1 ? a.indices[(int64_t)((uint32_t)p / (uint32_t)a.k) * a.ldi + (uint32_t)p % (uint32_t)a.k] : -1;
    }
#pragma unroll
    for (int r = 0; r < kBatch; ++r) {
      const int64_t p = pbb + r * 64 + lane;
      const bool in = p < p1;
      const int32_t e = ev[r];
      const bool valid = e >= 0 && e < a.E;
      // Lanes with the same expert: intersect, over the expert's bits and a
      // validity bit, the ballot of lanes agreeing with this lane on that bit.
      uint64_t same = ~0ull;
      {
        const uint64_t vb = __ballot(valid);
        same &= valid ? vb : ~vb;
      }
#pragma unroll
      for (int b = 0; b < kRouteExpertBits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t bb = __ballot(bit);
        same &= bit ? bb : ~bb;
      }
      const int rank =
          (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(same >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)same, 0u));
      const int later = __popcll(same) - rank - 1;
      // Every lane reads its expert's running count before the last lane of
      // each expert advances it (LDS operations of one wavefront complete in
      // order).
      const int32_t pos = valid ? next[e] + rank : -1;
      if (valid) a.row_token[pos] = (int32_t)((uint32_t)p / (uint32_t)a.k);
      if (in) a.token_rows[p] = pos;
      if (valid && later == 0) next[e] = pos + 1;
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// ---- combine --------------------------------------------------------------------------

constexpr int kCombineThreads = 256;

__device__ __forceinline__ float bf16_round(float v) { return bf16_lo(pack_bf16x2(v, 0.0f)); }

// One token per workgroup row; each lane takes CPT chunks of 8 columns,
// kCombineThreads * 8 apart, and issues the loads of all of the token's rows
// for all of its chunks before the first addition (two chunks: 109 -> 97 us
// for 4096 x top-8 rows of [*, 7168] inside the routed-expert step, 57 -> 43
// us where only the pairs of 32 of the 256 experts have rows; four: 104 and
// 44 us).
template <int KMAX, int CPT>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(CombineArgs a) {
  const int64_t t = blockIdx.x;
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
  auto column = [&](int c) { return (((int64_t)blockIdx.y * CPT + c) * kCombineThreads + threadIdx.x) * 8; };
  // All rows' loads of every chunk in flight before the accumulation.
  u32x4 v[CPT][KMAX];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int64_t col = column(c);
    const bool vec = a.vec && col + 8 <= a.D;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      v[c][j] = u32x4{0u, 0u, 0u, 0u};
      if (col >= a.D || row[j] < 0 || row[j] >= a.R) continue;
      const uint16_t* src = a.yr + (int64_t)row[j] * a.ldy + col;
      if (vec) {
        v[c][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
      } else {
        uint32_t e[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) e[q] = col + q < a.D ? (uint32_t)src[q] : 0u;
        v[c][j] = u32x4{e[0] | e[1] << 16, e[2] | e[3] << 16, e[4] | e[5] << 16, e[6] | e[7] << 16};
      }
    }
  }
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int64_t col = column(c);
    if (col >= a.D) continue;
    const bool vec = a.vec && col + 8 <= a.D;
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (row[j] < 0 || row[j] >= a.R) continue;
      const uint32_t words[4] = {v[c][j].x, v[c][j].y, v[c][j].z, v[c][j].w};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float y = (q & 1) ? bf16_hi(words[q >> 1]) : bf16_lo(words[q >> 1]);
        acc[q] = bf16_round(acc[q] + bf16_round(y * w[j]));
      }
    }
    uint16_t* dst = a.out + t * a.ldo + col;
    if (vec) {
      *reinterpret_cast<u32x4*>(dst) = u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                             pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (col + q < a.D) dst[q] = (uint16_t)(pack_bf16x2(acc[q], 0.0f) & 0xffff);
    }
  }
}

inline bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

}  // namespace

// Chunk size: at least kRouteChunk pairs, at most kMaxRouteChunks chunks.
static int64_t route_chunk(int64_t n) {
  int64_t c = (n + kMaxRouteChunks - 1) / kMaxRouteChunks;
  c = (c + 63) / 64 * 64;
  return c > kRouteChunk ? c : kRouteChunk;
}

size_t route_workspace_bytes(int64_t n, int64_t E) {
  const int64_t chunk = route_chunk(n);
  const int64_t chunks = (n + chunk - 1) / chunk;
  return (size_t)(chunks > 0 ? chunks : 1) * (size_t)E * sizeof(int32_t);
}

hipError_t launch_route(RouteArgs a, hipStream_t stream) {
  a.chunk = route_chunk(a.n);
  a.chunks = (a.n + a.chunk - 1) / a.chunk;
  const size_t lds = (size_t)a.E * sizeof(int32_t);  // count; the scatter uses twice this
  if (a.chunks == 0) {  // no pairs: every expert is empty
    hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((a.E + 1 + 255) / 256)), dim3(256), 0, stream, a.offsets,
                       (int64_t)a.E + 1, 0);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(route_count_kernel, dim3((unsigned)a.chunks), dim3(kRouteThreads), lds, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(route_scatter_kernel, dim3((unsigned)a.chunks), dim3(kRouteThreads), 2 * lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_combine(CombineArgs a, hipStream_t stream) {
  if (a.T == 0 || a.D == 0) return hipSuccess;
  a.vec = aligned(a.yr, 16) && a.ldy % 8 == 0 && aligned(a.out, 16) && a.ldo % 8 == 0;
  // two column chunks per lane up to k = 8; one for k up to 16, whose
  // sixteen rows already keep as many loads in flight
  auto grid = [&](int cpt) {
    return dim3((unsigned)a.T, (unsigned)((a.D + kCombineThreads * 8 * cpt - 1) / (kCombineThreads * 8 * cpt)));
  };
  const dim3 blk(kCombineThreads);
  if (a.k <= 2) hipLaunchKernelGGL((combine_kernel<2, 2>), grid(2), blk, 0, stream, a);
  else if (a.k <= 4) hipLaunchKernelGGL((combine_kernel<4, 2>), grid(2), blk, 0, stream, a);
  else if (a.k <= 8) hipLaunchKernelGGL((combine_kernel<8, 2>), grid(2), blk, 0, stream, a);
  else hipLaunchKernelGGL((combine_kernel<16, 1>), grid(1), blk, 0, stream, a);
  return hipGetLastError();
}

}  // namespace dsfp8
