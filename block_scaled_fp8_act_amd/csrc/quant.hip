// Bandwidth-bound kernels of the FP8 linear layer on gfx950:
//   act_quant (optionally fused with SiLU(g)*u), weight block quantisation,
//   weight dequantisation.
//
// act_quant ("DeepSeek-V3 Administrator & Developer Guide", 8.5.1): one
// 128-element block of a row is handled by one DPP row of 16 lanes, 8 elements
// (16 bytes of bf16) per lane, so a wavefront covers four blocks with one
// 16-byte load per lane and the block maximum is a four-step DPP reduction
// that never leaves the row.  Each lane computes the block scale and its
// correctly rounded reciprocal once, and every quotient x/s costs one multiply
// and two fma.  Work is distributed as (row, block) units in a grid-stride
// loop sized to the machine; each lane keeps kUnroll independent 16-byte loads
// in flight.
#include <type_traits>

#include "device.h"
#include "launch.h"

namespace dsfp8 {
namespace {

constexpr int kThreads = 256;
// Units in flight per lane.  Two (rather than four or eight) keeps the
// register count low enough for more resident waves, which measured faster
// for both the plain and the fused kernel.
constexpr int kUnroll = 2;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x4 mk4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 v;
  v.x = a; v.y = b; v.z = c; v.w = d;
  return v;
}

// Activation quantisation of one (row, block) unit held by 16 lanes.
// `v` holds this lane's 8 values (already SiLU-gated if fused); `valid` says
// which of them are real columns.  Writes y, s (and nothing for padding).
// NT: store y with the nontemporal hint (faster for the fused kernel, slower
// for the plain one on large tensors, both measured).
template <bool VEC, bool NT>
__device__ __forceinline__ void quantise_unit(const float (&v)[8], int nvalid, const ActQuantArgs& a,
                                              int64_t m, int64_t b, int lane16, bool live) {
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, j < nvalid ? fabsf(v[j]) : 0.0f);
  amax = max_row16(amax);
  const float s = block_scale_bf16(amax, a.ue8m0);
  const float r = recip_rn(s);
  float q[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) q[j] = div_by_scale(v[j], s, r);
  if (!live) return;
  const int64_t col = b * kBlock + lane16 * 8;
  uint8_t* yrow = a.y + m * a.ldy;
  if (VEC) {
    if (nvalid == 8) {
      u32x2 o;
      o.x = pack_e4m3x4(q[0], q[1], q[2], q[3]);
      o.y = pack_e4m3x4(q[4], q[5], q[6], q[7]);
      if (NT) __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(yrow + col));
      else *reinterpret_cast<u32x2*>(yrow + col) = o;
    }
  } else {
    uint32_t lo = pack_e4m3x4(q[0], q[1], q[2], q[3]);
    uint32_t hi = pack_e4m3x4(q[4], q[5], q[6], q[7]);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < nvalid) yrow[col + j] = (uint8_t)(((j < 4 ? lo : hi) >> (8 * (j & 3))) & 0xff);
  }
  if (lane16 == 0) a.s[m * a.s_rs + b * a.s_ks] = s;
}

// Load this lane's 8 bf16 values of one unit.  VEC: one 16-byte load (the
// host guarantees alignment and K % 8 == 0, so a lane's 8 columns are either
// all real or all padding).
template <bool VEC>
__device__ __forceinline__ u32x4 load8(const uint16_t* base, int64_t ld, int64_t m, int64_t col, int64_t K,
                                       bool live) {
  u32x4 w = mk4(0, 0, 0, 0);
  if (!live) return w;
  const uint16_t* p = base + m * ld + col;
  if (VEC) {
    if (col < K) w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  } else {
    uint32_t e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = (col + j < K) ? (uint32_t)p[j] : 0u;
    w.x = e[0] | (e[1] << 16);
    w.y = e[2] | (e[3] << 16);
    w.z = e[4] | (e[5] << 16);
    w.w = e[6] | (e[7] << 16);
  }
  return w;
}

__device__ __forceinline__ void unpack8(u32x4 w, float (&v)[8]) {
  v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
  v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
  v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
  v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
}

// A wave-unit is (row group g, K-block b): DPP row r of the wave (lanes
// 16r..16r+15) quantises row 4g + r of block b.  Wave-units are numbered
// block-major (w = b * G + g), so consecutive waves read consecutive row
// groups of the same column block and their scale stores (four consecutive
// rows, one K-block) are contiguous when the scales are stored K-block-major.
template <bool VEC, bool FUSED>
__global__ __launch_bounds__(kThreads) void act_quant_kernel(ActQuantArgs a, int64_t nb, FastDiv G, bool fast) {
  const int lane = threadIdx.x & 63;
  const int lane16 = lane & 15;
  const int drow = lane >> 4;
  const int64_t waves = (int64_t)gridDim.x * (kThreads / 64);
  const int64_t wave0 = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t total = (int64_t)G.d * nb;
  for (int64_t base = wave0; base < total; base += waves * kUnroll) {
    u32x4 wg[kUnroll], wu[kUnroll];
    int64_t ms[kUnroll], bs[kUnroll];
    bool live[kUnroll];
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
      const int64_t w = base + i * waves;
      const int64_t b = fast ? (int64_t)fastdiv((uint32_t)w, G) : w / (int64_t)G.d;
      const int64_t m = (w - b * (int64_t)G.d) * 4 + drow;
      live[i] = w < total && m < a.M;
      ms[i] = m;
      bs[i] = b;
      const int64_t col = b * kBlock + lane16 * 8;
      int64_t msrc = m;
      if (!FUSED && a.rows != nullptr && live[i]) {
        msrc = a.rows[m];
        msrc = msrc < 0 ? 0 : (msrc >= a.g_rows ? a.g_rows - 1 : msrc);
      }
      wg[i] = load8<VEC>(a.g, a.ldg, msrc, col, a.K, live[i]);
      if (FUSED) wu[i] = load8<VEC>(a.u, a.ldu, m, col, a.K, live[i]);
    }
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
      const int64_t col = bs[i] * kBlock + lane16 * 8;
      const int64_t rem = a.K - col;
      const int nvalid = rem >= 8 ? 8 : (rem > 0 ? (int)rem : 0);
      float v[8];
      unpack8(wg[i], v);
      if (FUSED) {
        float uv[8];
        unpack8(wu[i], uv);
        __bf16 hb[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = silu_mul_bf16(v[j], uv[j], &hb[j]);
        if (a.h != nullptr && live[i]) {
          uint16_t* hrow = a.h + ms[i] * a.ldh + col;
          if (VEC) {
            if (nvalid == 8) {
              u32x4 o;
              o.x = pack_bf16x2(v[0], v[1]);
              o.y = pack_bf16x2(v[2], v[3]);
              o.z = pack_bf16x2(v[4], v[5]);
              o.w = pack_bf16x2(v[6], v[7]);
              *reinterpret_cast<u32x4*>(hrow) = o;
            }
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
              if (j < nvalid) hrow[j] = __builtin_bit_cast(uint16_t, hb[j]);
          }
        }
      }
      quantise_unit<VEC, FUSED>(v, nvalid, a, ms[i], bs[i], lane16, live[i]);
    }
  }
}

// The same kernel for aligned operands whose extents fit 32-bit byte
// offsets: every access goes through a buffer resource, and a lane with
// nothing to load or store passes an offset past the resource's end (loads
// then return zero and stores are dropped), so there is no per-lane branch
// and all address arithmetic is 32-bit.  The result is bit-identical to
// act_quant_kernel; it runs 18% faster on [4096, 7168] (measured): the general
// kernel spends most of its issue slots on 64-bit address arithmetic and the
// branches around each access.  Columns past K read as zero, so they never
// raise a block's maximum.
constexpr uint32_t kOffNone = 0x80000000u;  // above every resource's size

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}

struct LeanExtents {
  uint32_t nb, total;                    // K-blocks, wave-units
  uint32_t x, u, y, s, h, rows;          // resource sizes in bytes
};

template <bool FUSED, bool ROWS, int THREADS, int U>
__global__ __launch_bounds__(THREADS) void act_quant_lean_kernel(ActQuantArgs a, FastDiv G, LeanExtents e) {
  constexpr int kNt = 2;  // cache-policy bit of a nontemporal access
  const int lane = threadIdx.x & 63;
  const uint32_t lane16 = lane & 15;
  const uint32_t drow = lane >> 4;
  const uint32_t waves = gridDim.x * (THREADS / 64);
  const uint32_t wave0 = blockIdx.x * (THREADS / 64) + (threadIdx.x >> 6);
  const auto rx = buffer_of(a.g, e.x);
  const auto ru = buffer_of(FUSED ? static_cast<const void*>(a.u) : static_cast<const void*>(a.g), e.u);
  const auto ry = buffer_of(a.y, e.y);
  const auto rs = buffer_of(a.s, e.s);
  const auto rh = buffer_of(a.h != nullptr ? static_cast<const void*>(a.h) : static_cast<const void*>(a.y), e.h);
  const auto rr = buffer_of(ROWS ? static_cast<const void*>(a.rows) : static_cast<const void*>(a.g), e.rows);
  const uint32_t M = (uint32_t)a.M, K = (uint32_t)a.K, grows = (uint32_t)a.g_rows;
  const uint32_t ldg = (uint32_t)a.ldg, ldu = (uint32_t)a.ldu, ldy = (uint32_t)a.ldy, ldh = (uint32_t)a.ldh;
  const uint32_t srs = (uint32_t)a.s_rs, sks = (uint32_t)a.s_ks;
  const bool want_h = FUSED && a.h != nullptr;
  for (uint32_t base = wave0; base < e.total; base += waves * U) {
    u32x4 wg[U], wu[U];
    uint32_t ms[U], cs[U], bs[U];
    bool lv[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const uint32_t w = base + i * waves;
      // Unit w: 4 rows of one K-block.  Units go row group by row group (G
      // divides by the K-block count), so a workgroup's 4 waves read 1 KB of
      // each of 4 rows; the gathered form goes block by block (G divides by
      // the row-group count), where neighbouring waves often read the same
      // source rows.
      uint32_t b, m;
      if constexpr (ROWS) {
        b = fastdiv(w, G);
        m = (w - b * G.d) * 4 + drow;
      } else {
        const uint32_t g = fastdiv(w, G);
        b = w - g * G.d;
        m = g * 4 + drow;
      }
      const uint32_t col = b * kBlock + lane16 * 8;
      const bool live = w < e.total && m < M;
      const bool in = live && col < K;
      uint32_t msrc = m;
      if (ROWS) {
        const int32_t r = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(rr, live ? m * 4 : kOffNone, 0, 0);
        msrc = r < 0 ? 0u : ((uint32_t)r >= grows ? grows - 1 : (uint32_t)r);
      }
      ms[i] = m;
      cs[i] = col;
      bs[i] = b;
      lv[i] = live;
      wg[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, in ? (msrc * ldg + col) * 2 : kOffNone, 0, kNt);
      if (FUSED) wu[i] = __builtin_amdgcn_raw_buffer_load_b128(ru, in ? (m * ldu + col) * 2 : kOffNone, 0, kNt);
    }
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const bool in = lv[i] && cs[i] < K;
      float v[8];
      unpack8(wg[i], v);
      if (FUSED) {
        float uv[8];
        unpack8(wu[i], uv);
        __bf16 hb[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = silu_mul_bf16(v[j], uv[j], &hb[j]);
        if (want_h)
          __builtin_amdgcn_raw_buffer_store_b128(mk4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                     pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])),
                                                 rh, in ? (ms[i] * ldh + cs[i]) * 2 : kOffNone, 0, 0);
      }
      float amax = fmaxf(fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))),
                         fmaxf(fmaxf(fabsf(v[4]), fabsf(v[5])), fmaxf(fabsf(v[6]), fabsf(v[7]))));
      amax = max_row16(amax);
      const float s = block_scale_bf16(amax, a.ue8m0);
      const float r = recip_rn(s);
      u32x2 o;
      o.x = pack_e4m3x4(div_by_scale(v[0], s, r), div_by_scale(v[1], s, r), div_by_scale(v[2], s, r),
                        div_by_scale(v[3], s, r));
      o.y = pack_e4m3x4(div_by_scale(v[4], s, r), div_by_scale(v[5], s, r), div_by_scale(v[6], s, r),
                        div_by_scale(v[7], s, r));
      // the fused kernel's codes are stored nontemporal (measured faster there,
      // slower for the plain kernel)
      __builtin_amdgcn_raw_buffer_store_b64(o, ry, in ? ms[i] * ldy + cs[i] : kOffNone, 0, FUSED ? kNt : 0);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s), rs,
                                            (lv[i] && lane16 == 0) ? (ms[i] * srs + bs[i] * sks) * 4 : kOffNone, 0, 0);
    }
  }
}

// ---- weight block quantisation ---------------------------------------------------
//
// One workgroup per 128x128 block: 16 lanes cover a 128-column row segment
// (8 columns each), 16 row segments per pass, 8 passes.  The block's values
// stay in registers between the maximum and the quantisation, so the weight
// is read from memory once.

template <typename T>
__device__ __forceinline__ float load_w(const T* p);
template <>
__device__ __forceinline__ float load_w<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_w<uint16_t>(const uint16_t* p) { return __uint_as_float((uint32_t)*p << 16); }

template <typename T>
__global__ __launch_bounds__(kThreads) void weight_quant_kernel(WeightQuantArgs a) {
  __shared__ float wave_max[kThreads / 64];
  const int t = threadIdx.x;
  const int lane16 = t & 15;
  const int seg = t >> 4;                 // 0..15
  const int64_t bj = blockIdx.x, bi = blockIdx.y;
  const int64_t c0 = bj * kBlock + lane16 * 8;
  const T* w = reinterpret_cast<const T*>(a.w);
  float v[8][8];
  float amax = 0.0f;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int64_t n = bi * kBlock + p * 16 + seg;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool ok = n < a.N && c0 + j < a.K;
      v[p][j] = ok ? load_w<T>(w + n * a.ldw + c0 + j) : 0.0f;
      amax = fmaxf(amax, fabsf(v[p][j]));
    }
  }
  amax = max_wave(amax);
  if ((t & 63) == 0) wave_max[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
  const float s = block_scale(amax, a.ue8m0);
  if (t == 0) a.S[bi * a.ldS + bj] = s;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int64_t n = bi * kBlock + p * 16 + seg;
    if (n >= a.N) continue;
    // The correctly rounded IEEE division (the library is built with
    // correctly rounded fp32 division): fp32 weights lie outside the domain
    // on which the reciprocal-and-correction quotient of act_quant is proven,
    // and this kernel is not on the timed path.
    float q[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = v[p][j] / s;
    const uint32_t lo = pack_e4m3x4(q[0], q[1], q[2], q[3]);
    const uint32_t hi = pack_e4m3x4(q[4], q[5], q[6], q[7]);
    uint8_t* out = a.q + n * a.ldq + c0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (c0 + j < a.K) out[j] = (uint8_t)(((j < 4 ? lo : hi) >> (8 * (j & 3))) & 0xff);
  }
}

// ---- weight dequantisation -----------------------------------------------------
//
// ("DeepSeek-V3 Administrator & Developer Guide", 8.5.2.)  Each lane converts
// 8 consecutive e4m3 bytes of a row with four v_cvt_pk_f32_fp8, multiplies
// each value by the block's scale in fp32 and rounds pairs to bf16 with
// v_cvt_pk_bf16_f32.  A lane handles two such column chunks 2048 apart in
// each of kDqRows rows, so a wave's loads read 512 contiguous bytes and its
// 16-byte stores write 1 KB contiguous (two 16-byte stores per lane 32 bytes
// apart wrote each line half at a time and ran 22% slower).  A workgroup
// covers 4096 columns of kDqRows rows (4 rows: 2% faster than 8, 16 slower).

constexpr int kDqRows = 4;

template <bool VEC>
__global__ __launch_bounds__(kThreads) void weight_dequant_kernel(DequantArgs a) {
  const int64_t cbase = (int64_t)blockIdx.x * (kThreads * 16) + threadIdx.x * 8;
  const int64_t row0 = (int64_t)blockIdx.y * kDqRows;
  u32x2 w[2][kDqRows];
  float sc[2][kDqRows];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t col = cbase + h * (kThreads * 8);
    const int64_t cc = col < a.K ? col : 0;
    const int64_t kb = cc / kBlock;
#pragma unroll
    for (int r = 0; r < kDqRows; ++r) {
      const int64_t n = row0 + r;
      const int64_t nn = n < a.N ? n : row0;
      sc[h][r] = a.S[(nn / kBlock) * a.ldS + kb];
      const uint8_t* src = a.w + nn * a.ldw + cc;
      if (VEC) {
        w[h][r] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(src));
      } else {
        uint32_t bytes[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) bytes[j] = (col + j < a.K) ? src[j] : 0u;
        w[h][r].x = bytes[0] | bytes[1] << 8 | bytes[2] << 16 | bytes[3] << 24;
        w[h][r].y = bytes[4] | bytes[5] << 8 | bytes[6] << 16 | bytes[7] << 24;
      }
    }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t col = cbase + h * (kThreads * 8);
    if (col >= a.K) continue;
#pragma unroll
    for (int r = 0; r < kDqRows; ++r) {
      const int64_t n = row0 + r;
      if (n >= a.N) break;
      typedef float f2 __attribute__((ext_vector_type(2)));
      const float s = sc[h][r];
      const uint32_t words[2] = {w[h][r].x, w[h][r].y};
      uint32_t out[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        f2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)words[i], false);
        f2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)words[i], true);
        out[2 * i] = pack_bf16x2(lo[0] * s, lo[1] * s);
        out[2 * i + 1] = pack_bf16x2(hi[0] * s, hi[1] * s);
      }
      uint16_t* dst = a.out + n * a.ldo + col;
      if (VEC) {
        __builtin_nontemporal_store(mk4(out[0], out[1], out[2], out[3]), reinterpret_cast<u32x4*>(dst));
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (col + j < a.K) dst[j] = (uint16_t)((out[j >> 1] >> (16 * (j & 1))) & 0xffff);
      }
    }
  }
}

// The same kernel for aligned operands whose extents fit 32-bit byte
// offsets, through buffer resources (no per-lane branches, 32-bit address
// arithmetic; a lane past N or K passes an offset past the resource's end),
// with kDqLeanRows rows per workgroup: 69.5 us against 71.3 us for the
// general kernel on [18432, 7168] (2 rows measured faster than 4, 8 slower;
// plain instead of nontemporal stores 5% slower).  Bit-identical results.
// The workgroup size is chosen per K (dequant_threads): the fewest
// workgroups of at most 256 threads that cover a row, each thread taking 16
// columns, so no lane idles where K allows it; against a fixed 256 threads:
// [18432, 7168] 69.2 -> 63.3 us (224 threads), [36864, 7168] 139.9 -> 126.9,
// [4096, 2048] 6.3 -> 6.0; [7168, 18432] unchanged.
constexpr int kDqLeanRows = 2;
constexpr int kDqMaxThreads = 256;

inline int64_t dequant_threads(int64_t K) {
  const int64_t chunks = (K + 15) / 16;
  const int64_t blocks = (chunks + kDqMaxThreads - 1) / kDqMaxThreads;
  return ((chunks + blocks - 1) / blocks + 15) / 16 * 16;
}

__global__ __launch_bounds__(kDqMaxThreads) void weight_dequant_lean_kernel(DequantArgs a, uint32_t wbytes, uint32_t sbytes,
                                                                       uint32_t obytes) {
  constexpr int kNt = 2;
  const uint32_t T = blockDim.x;  // dequant_threads(K)
  const auto rw = buffer_of(a.w, wbytes);
  const auto rs = buffer_of(a.S, sbytes);
  const auto ro = buffer_of(a.out, obytes);
  const uint32_t K = (uint32_t)a.K, N = (uint32_t)a.N;
  const uint32_t ldw = (uint32_t)a.ldw, ldS = (uint32_t)a.ldS, ldo = (uint32_t)a.ldo;
  const uint32_t cbase = blockIdx.x * (T * 16) + threadIdx.x * 8;
  const uint32_t row0 = blockIdx.y * kDqLeanRows;
  u32x2 w[2][kDqLeanRows];
  float sc[2][kDqLeanRows];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t col = cbase + h * (T * 8);
#pragma unroll
    for (int r = 0; r < kDqLeanRows; ++r) {
      const uint32_t n = row0 + r;
      const bool in = n < N && col < K;
      sc[h][r] = __uint_as_float(
          __builtin_amdgcn_raw_buffer_load_b32(rs, in ? ((n / kBlock) * ldS + col / kBlock) * 4 : kOffNone, 0, 0));
      w[h][r] = __builtin_amdgcn_raw_buffer_load_b64(rw, in ? n * ldw + col : kOffNone, 0, kNt);
    }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t col = cbase + h * (T * 8);
#pragma unroll
    for (int r = 0; r < kDqLeanRows; ++r) {
      const uint32_t n = row0 + r;
      const bool in = n < N && col < K;
      typedef float f2 __attribute__((ext_vector_type(2)));
      const float s = sc[h][r];
      const uint32_t words[2] = {w[h][r].x, w[h][r].y};
      uint32_t out[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        f2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)words[i], false);
        f2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)words[i], true);
        out[2 * i] = pack_bf16x2(lo[0] * s, lo[1] * s);
        out[2 * i + 1] = pack_bf16x2(hi[0] * s, hi[1] * s);
      }
      __builtin_amdgcn_raw_buffer_store_b128(mk4(out[0], out[1], out[2], out[3]), ro,
                                             in ? (n * ldo + col) * 2 : kOffNone, 0, kNt);
    }
  }
}

inline bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

}  // namespace

hipError_t launch_act_quant(const ActQuantArgs& a, hipStream_t stream) {
  if (a.M == 0 || a.K == 0) return hipSuccess;
  const int64_t nb = (a.K + kBlock - 1) / kBlock;
  const int64_t G = (a.M + 3) / 4;  // groups of four rows
  const int64_t units = G * nb;
  const FastDiv gdiv = make_fastdiv((uint32_t)G);
  const bool fused = a.u != nullptr;
  // 16-byte loads of x (and u), 8-byte stores of y, 16-byte stores of h.
  bool vec = (a.K % 8 == 0) && aligned(a.g, 16) && (a.ldg % 8 == 0) && aligned(a.y, 8) && (a.ldy % 8 == 0);
  if (fused) vec = vec && aligned(a.u, 16) && (a.ldu % 8 == 0);
  if (a.h) vec = vec && aligned(a.h, 16) && (a.ldh % 8 == 0);
  const int64_t waves_per_wg = kThreads / 64;
  const int64_t want = (units + waves_per_wg * kUnroll - 1) / (waves_per_wg * kUnroll);
  // Workgroups per CU (measured): 32 for the plain kernel (1.5-3% faster than
  // 16 on the dense-input, routed-row and gathered shapes), 8 for the fused one.
  const int64_t cap = (int64_t)device_cu_count() * (fused ? 8 : 32);
  const int64_t grid = want < cap ? want : cap;
  // The multiply-shift division needs every wave-unit index the loop forms
  // (up to kUnroll grid-widths past the end) below 2^31.
  const bool fast = units + (int64_t)kUnroll * grid * waves_per_wg < ((int64_t)1 << 31);
  dim3 g((unsigned)grid), blk(kThreads);
  // The buffer-resource kernel when every extent fits 32-bit byte offsets
  // (below 2^31, so that kOffNone lies past every resource).
  auto extent = [](int64_t rows, int64_t ld, int64_t cols, int64_t elt) {
    return rows > 0 ? ((rows - 1) * ld + cols) * elt : (int64_t)0;
  };
  const int64_t src_rows = a.rows != nullptr ? a.g_rows : a.M;
  const int64_t ex = extent(src_rows, a.ldg, a.K, 2), eu = fused ? extent(a.M, a.ldu, a.K, 2) : 0;
  const int64_t ey = extent(a.M, a.ldy, a.K, 1), eh = a.h != nullptr ? extent(a.M, a.ldh, a.K, 2) : 0;
  const int64_t es = ((a.M - 1) * a.s_rs + (nb - 1) * a.s_ks + 1) * 4, er = a.rows != nullptr ? a.M * 4 : 0;
  const int64_t lim = (int64_t)1 << 31;
  if (vec && fast && ex < lim && eu < lim && ey < lim && eh < lim && es < lim && er < lim && units < lim) {
    LeanExtents e{(uint32_t)nb, (uint32_t)units, (uint32_t)ex, (uint32_t)eu, (uint32_t)ey,
                  (uint32_t)es, (uint32_t)eh, (uint32_t)er};
    // Row-group order against block order (measured, graph of launches):
    // [4096, 7168] 16.9 against 17.3 us, [4096, 18432] 39.5 against 44.4 us,
    // [32768, 7168] 117.9 against 120.2 us, the fused gate on [4096, 18432]
    // 71.1 against 77.3 us; the gathered rows 106.2 against 97.5 us, so they
    // keep the block order.  (One row and four K-blocks per wave, in either
    // order, was slower than both: 18.6 us on [4096, 7168].)
    const FastDiv nbdiv = make_fastdiv((uint32_t)nb);
    // Waves per workgroup (W), units in flight per wave (U) and the most
    // waves in the grid, per form (measured, graph of launches, against the
    // first form's 4 waves, 2 units and 128 waves per CU):
    //  * plain, when 1-wave workgroups of 2 units cover every unit in one
    //    pass: W 1, U 2 ([4096, 7168] 17.0 -> 16.3 us);
    //  * plain, several passes: W 2, U 1, up to 256 waves per CU
    //    ([32768, 7168] 118.2 -> 112.1 us, [4096, 18432] 40.1 -> 38.3);
    //  * fused: W 2, U 1, up to 32 waves per CU (one unit: 70.9 -> 67.4 us on
    //    the gate of [4096, 18432]);
    //  * gathered rows: W 2, U 2, up to 128 waves per CU (one unit in
    //    flight: 97 -> 133 us).
    // Workgroups of 8 or 16 waves were slower on every shape.
    auto lean = [&](auto w_c, auto u_c, int64_t waves_per_cu) {
      constexpr int W = decltype(w_c)::value, U = decltype(u_c)::value;
      const int64_t want_w = (units + W * U - 1) / (W * U);
      const int64_t cap_w = (int64_t)device_cu_count() * waves_per_cu / W;
      const dim3 gw((unsigned)(want_w < cap_w ? want_w : cap_w)), bw(64 * W);
      if (fused) hipLaunchKernelGGL((act_quant_lean_kernel<true, false, 64 * W, U>), gw, bw, 0, stream, a, nbdiv, e);
      else if (a.rows != nullptr)
        hipLaunchKernelGGL((act_quant_lean_kernel<false, true, 64 * W, U>), gw, bw, 0, stream, a, gdiv, e);
      else hipLaunchKernelGGL((act_quant_lean_kernel<false, false, 64 * W, U>), gw, bw, 0, stream, a, nbdiv, e);
      return hipGetLastError();
    };
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    if (fused) return lean(I2(), I1(), 32);
    if (a.rows != nullptr) return lean(I2(), I2(), 128);
    if ((units + 1) / 2 <= (int64_t)device_cu_count() * 128) return lean(I1(), I2(), 128);
    return lean(I2(), I1(), 256);
  }
  if (fused) {
    if (vec) hipLaunchKernelGGL((act_quant_kernel<true, true>), g, blk, 0, stream, a, nb, gdiv, fast);
    else hipLaunchKernelGGL((act_quant_kernel<false, true>), g, blk, 0, stream, a, nb, gdiv, fast);
  } else {
    if (vec) hipLaunchKernelGGL((act_quant_kernel<true, false>), g, blk, 0, stream, a, nb, gdiv, fast);
    else hipLaunchKernelGGL((act_quant_kernel<false, false>), g, blk, 0, stream, a, nb, gdiv, fast);
  }
  return hipGetLastError();
}

hipError_t launch_weight_quant(const WeightQuantArgs& a, hipStream_t stream) {
  if (a.N == 0 || a.K == 0) return hipSuccess;
  dim3 g((unsigned)((a.K + kBlock - 1) / kBlock), (unsigned)((a.N + kBlock - 1) / kBlock)), blk(kThreads);
  if (a.bf16_in) hipLaunchKernelGGL((weight_quant_kernel<uint16_t>), g, blk, 0, stream, a);
  else hipLaunchKernelGGL((weight_quant_kernel<float>), g, blk, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_weight_dequant(const DequantArgs& a, hipStream_t stream) {
  if (a.N == 0 || a.K == 0) return hipSuccess;
  const bool vec = (a.K % 16 == 0) && aligned(a.w, 16) && (a.ldw % 16 == 0) && aligned(a.out, 16) &&
                   (a.ldo % 8 == 0);
  const int64_t wb = (a.N - 1) * a.ldw + a.K, ob = ((a.N - 1) * a.ldo + a.K) * 2;
  const int64_t sb = (((a.N - 1) / kBlock) * a.ldS + (a.K - 1) / kBlock + 1) * 4;
  const int64_t lim = (int64_t)1 << 31;
  if (vec && wb < lim && ob < lim && sb < lim) {
    const int64_t T = dequant_threads(a.K);
    dim3 g2((unsigned)((a.K + T * 16 - 1) / (T * 16)), (unsigned)((a.N + kDqLeanRows - 1) / kDqLeanRows));
    hipLaunchKernelGGL(weight_dequant_lean_kernel, g2, dim3((unsigned)T), 0, stream, a, (uint32_t)wb, (uint32_t)sb,
                       (uint32_t)ob);
    return hipGetLastError();
  }
  dim3 g((unsigned)((a.K + kThreads * 16 - 1) / (kThreads * 16)), (unsigned)((a.N + kDqRows - 1) / kDqRows));
  dim3 blk(kThreads);
  if (vec) hipLaunchKernelGGL((weight_dequant_kernel<true>), g, blk, 0, stream, a);
  else hipLaunchKernelGGL((weight_dequant_kernel<false>), g, blk, 0, stream, a);
  return hipGetLastError();
}

}  // namespace dsfp8
