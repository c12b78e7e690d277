// Block-scaled FP8 products on gfx950 MFMA: dense and grouped over per-expert
// row ranges.
//
// The product ("DeepSeek-V3 Administrator & Developer Guide", 8.5.3) adds,
// for every 128-wide K-block b, the block's partial dot product multiplied by
// the activation scale a_s[m, b] and the weight scale b_s[n/128, b].  On CDNA4
// one v_mfma_f32_16x16x128_f8f6f4 consumes exactly one K-block of a 16x16
// output tile, so each K-block's partial product comes out of a single MFMA
// (started from zero) and is folded into the fp32 accumulator with one VALU
// fma per output element, using the per-row product a_s * b_s.  A workgroup
// stages BM x 128 bytes of A and BN x 128 bytes of B per K-block in LDS
// (double-buffered, 16-byte chunks XOR-swizzled by row so that the fragment
// reads of eight consecutive rows hit distinct banks), together with the BM
// activation scales of that K-block.  Global loads for K-block b+1 are issued
// before the MFMAs of block b, so their latency overlaps the math.
//
// Workgroups are mapped to tiles so that each XCD (workgroup i runs on XCD
// i % 8) owns a contiguous range of tiles, ordered in groups of GROUP_M tile
// rows, which keeps the A and B panels in use on one XCD inside its L2.
//
// Kernels: gemm_persistent_kernel (one workgroup per CU walking its XCD's
// 256x256 tiles) for large dense products, plain or with the SiLU gate and
// act_quant in the epilogue; gemm_kernel (one workgroup per tile) otherwise;
// for products with few output tiles gemm_rd_kernel and gemm_rdr_kernel (one
// launch: K split over the waves of a workgroup and, through arrival
// counters in the workspace, over workgroups), or gemm_kernel with split K
// and splitk_reduce_kernel for operands those do not take;
// skinny_gemm_kernel for decode rows; grouped_merged_kernel for the
// per-expert products (three tile heights in one launch, scheduled by
// tile_schedule_kernel from the device-side offsets).
#include <atomic>

#include "device.h"
#include "launch.h"

namespace dsfp8 {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BK = 128;
constexpr int kXcds = 8;
constexpr int kGroupM = 8;

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int kThreads = 64 * WAVES_M * WAVES_N;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int TM = WM / 16, TN = WN / 16;
  static constexpr int kRowsPerPass = kThreads / 8;  // 8 threads load one 128-byte row
  static constexpr int A_CHUNKS = BM / kRowsPerPass;
  static constexpr int B_CHUNKS = BN / kRowsPerPass;
  static constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK;
  static constexpr int CPAD = 8;                     // bf16 elements of padding per staged C row
  static constexpr int C_BYTES = WAVES_M * WAVES_N * WM * (WN + CPAD) * 2;
  static constexpr int MAIN_BYTES = 2 * (A_BYTES + B_BYTES) + 2 * BM * 4;
  static constexpr int LDS_BYTES = MAIN_BYTES > C_BYTES ? MAIN_BYTES : C_BYTES;
  static_assert(BM % kRowsPerPass == 0 && BN % kRowsPerPass == 0, "tile rows");
  static_assert(WN <= 128 && 128 % WN == 0, "a wave's columns must lie in one 128-block");
  static_assert(BM <= kThreads, "one thread per activation scale");
};

using Cfg128 = Cfg<128, 128, 2, 2>;

// 16 bytes of one row starting at column k (a multiple of 16); bytes at
// columns >= K, or of a row outside the matrix, read as zero.  VEC is the
// widest access the host proved aligned; it divides K, so each VEC-wide piece
// is entirely inside or entirely outside the row.
template <int VEC>
__device__ __forceinline__ u32x4 load_chunk(const uint8_t* row, int64_t k, int64_t K, bool row_ok) {
  u32x4 v = {0u, 0u, 0u, 0u};
  if (!row_ok) return v;
  if constexpr (VEC == 16) {
    if (k < K) v = *reinterpret_cast<const u32x4*>(row + k);
  } else if constexpr (VEC == 8) {
    if (k < K) { u32x2 t = *reinterpret_cast<const u32x2*>(row + k); v.x = t.x; v.y = t.y; }
    if (k + 8 < K) { u32x2 t = *reinterpret_cast<const u32x2*>(row + k + 8); v.z = t.x; v.w = t.y; }
  } else if constexpr (VEC == 4) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(row + k);
    if (k < K) v.x = p[0];
    if (k + 4 < K) v.y = p[1];
    if (k + 8 < K) v.z = p[2];
    if (k + 12 < K) v.w = p[3];
  } else {
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (k + i < K) w[i >> 2] |= (uint32_t)row[k + i] << (8 * (i & 3));
    v.x = w[0]; v.y = w[1]; v.z = w[2]; v.w = w[3];
  }
  return v;
}

// Byte offset of 16-byte chunk c of tile row r in LDS.  The chunk index is
// XOR-ed with (r & 7) ^ ((r >> 3) & 1), which gives distinct chunks to the 8
// rows of each aligned group of 8 and distinct (row parity, chunk) pairs to
// the 16 rows of each aligned group of 16.  An MFMA fragment read (16
// consecutive rows, one logical chunk) is then free of bank conflicts whether
// the LDS serves it as 8 lanes over 128 bytes of banks or as 16 lanes over
// 256 bytes (measured: no SQ_LDS_BANK_CONFLICT cycles, against 42% of the
// LDS's active cycles with (r >> 1) & 7 or r & 7).  The key repeats every 16
// rows, so all fragment reads of a wave share their lane offsets.
__device__ __forceinline__ int swz_key(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz(int r, int c) { return r * BK + ((c ^ swz_key(r)) << 4); }

// MFMA operand of one 16-row slice: lane (r, g) = (lane % 16, lane / 16) holds
// K bytes [32g, 32g + 32) of row r.  A and B use the same K assignment, so the
// dot product over the K-block does not depend on the order in which the
// matrix core consumes the bytes.
__device__ __forceinline__ v8i read_frag(const uint8_t* tile, int r, int g) {
  const u32x4 lo = *reinterpret_cast<const u32x4*>(tile + swz(r, 2 * g));
  const u32x4 hi = *reinterpret_cast<const u32x4*>(tile + swz(r, 2 * g + 1));
  v8i f;
  f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
  f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
  return f;
}

struct TileRef {
  const uint8_t* A;      // matrix base (absolute rows)
  const float* a_s;
  const uint8_t* B;      // this tile's weight [N, K]
  const float* b_s;      // this tile's weight scales
  int64_t row0, row_end; // rows [row0, min(row0 + BM, row_end)) are computed
  int64_t n0;
  int kb0, kb1;          // K-blocks [kb0, kb1) are accumulated
  float* partial;        // non-null: store the fp32 partial [M, N] here instead of C
};

// Accumulator layouts of a 16 x 16 output subtile (i, j) of a wave, lane =
// (fr, fg) = (lane % 16, lane / 16):
//   row layout (activations as the MFMA's first operand): acc[i][j][v] is
//     C[16i + 4fg + v][16j + fr];
//   column layout (weights as the first operand): acc[i][j][v] is
//     C[16i + fr][16j + 4fg + v], four consecutive columns of one row.

// Round the accumulators to bf16 and stage each wave's WM x WN tile in LDS
// (which the caller has finished reading): wave w's tile starts at element
// w * WM * CS, rows CS = WN + CPAD elements apart.
template <class CF, bool COLS>
__device__ __forceinline__ void stage_c(const v4f (&acc)[CF::TM][CF::TN], uint8_t* smem, int wave, int lane) {
  const int fr = lane & 15, fg = lane >> 4;
  constexpr int CS = CF::WN + CF::CPAD;
  uint16_t* cst = reinterpret_cast<uint16_t*>(smem) + wave * CF::WM * CS;
#pragma unroll
  for (int i = 0; i < CF::TM; ++i)
#pragma unroll
    for (int j = 0; j < CF::TN; ++j) {
      if constexpr (COLS) {
        uint2 w;
        w.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
        w.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
        *reinterpret_cast<uint2*>(cst + (i * 16 + fr) * CS + j * 16 + 4 * fg) = w;
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const __bf16 h = (__bf16)acc[i][j][v];
          cst[(i * 16 + 4 * fg + v) * CS + j * 16 + fr] = __builtin_bit_cast(uint16_t, h);
        }
      }
    }
}

// Epilogue: stage the tile in LDS, read each lane's rows of it into
// registers, call hook() (which may wait for those reads and reuse the LDS),
// then write rows of C with 16-byte stores.
template <class CF, bool COLS, class Hook>
__device__ __forceinline__ void store_tile(const GemmArgs& p, const TileRef& t, const v4f (&acc)[CF::TM][CF::TN],
                                           uint8_t* smem, int wave, int wm, int wn, int lane, Hook&& hook) {
  asm volatile("" : "+v"(lane));
  const int64_t N = p.N;
  constexpr int CS = CF::WN + CF::CPAD;
  const uint16_t* cst = reinterpret_cast<const uint16_t*>(smem) + wave * CF::WM * CS;
  stage_c<CF, COLS>(acc, smem, wave, lane);
  __syncthreads();
  const int64_t crow0 = t.row0 + wm * CF::WM;
  const int64_t ccol0 = t.n0 + wn * CF::WN;
  const int64_t row_lim = t.row_end;
  const bool cvec = ((reinterpret_cast<uintptr_t>(p.C) & 15) == 0) && (p.ldc % 8 == 0);
  constexpr int CPR = CF::WN / 8;  // 16-byte chunks per staged row
  constexpr int IT = CF::WM * CPR / 64;
  u32x4 v[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int c = lane + 64 * it;
    v[it] = *reinterpret_cast<const u32x4*>(cst + (c / CPR) * CS + (c % CPR) * 8);
  }
  hook();
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int c = lane + 64 * it;
    const int r = c / CPR, cc = c % CPR;
    const int64_t row = crow0 + r;
    const int64_t col = ccol0 + cc * 8;
    if (row >= row_lim || col >= N) continue;
    uint16_t* dst = p.C + row * p.ldc + col;
    if (cvec && col + 8 <= N) {
      *reinterpret_cast<u32x4*>(dst) = v[it];
    } else {
      const uint32_t w[4] = {v[it].x, v[it].y, v[it].z, v[it].w};
      for (int e = 0; e < 8 && col + e < N; ++e) dst[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
    }
  }
}

// Split K: the fp32 partial of this tile goes straight from registers to the
// workspace [M, N] of its split (row layout: 16 lanes write 64 contiguous
// bytes; column layout: each lane writes 16 contiguous bytes).
template <class CF, bool COLS>
__device__ __forceinline__ void store_partial(const GemmArgs& p, const TileRef& t,
                                              const v4f (&acc)[CF::TM][CF::TN], int wm, int wn, int lane) {
  const int fr = lane & 15, fg = lane >> 4;
#pragma unroll
  for (int i = 0; i < CF::TM; ++i)
#pragma unroll
    for (int j = 0; j < CF::TN; ++j) {
      if constexpr (COLS) {
        const int64_t row = t.row0 + wm * CF::WM + i * 16 + fr;
        const int64_t col = t.n0 + wn * CF::WN + j * 16 + 4 * fg;
        if (row >= t.row_end) continue;
        float* dst = t.partial + row * p.N + col;
        if (col + 4 <= p.N && (p.N & 3) == 0) {
          *reinterpret_cast<v4f*>(dst) = acc[i][j];
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (col + v < p.N) dst[v] = acc[i][j][v];
        }
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int64_t row = t.row0 + wm * CF::WM + i * 16 + 4 * fg + v;
          const int64_t col = t.n0 + wn * CF::WN + j * 16 + fr;
          if (row < t.row_end && col < p.N) t.partial[row * p.N + col] = acc[i][j][v];
        }
      }
    }
}

template <class CF, int VEC>
__device__ __forceinline__ void gemm_tile(const GemmArgs& p, const TileRef& t, uint8_t* smem) {
  constexpr int BM = CF::BM;
  uint8_t* As = smem;
  uint8_t* Bs = smem + 2 * CF::A_BYTES;
  float* Ss = reinterpret_cast<float*>(smem + 2 * (CF::A_BYTES + CF::B_BYTES));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / CF::WAVES_N, wn = wave % CF::WAVES_N;
  const int64_t K = p.K, N = p.N;
  const int nkb = (int)((K + BK - 1) / BK);
  const int64_t kbn = (N + BK - 1) / BK;

  const int ck = tid & 7;
  const int rbase = tid >> 3;

  u32x4 ra[CF::A_CHUNKS], rb[CF::B_CHUNKS];
  float rs = 0.0f;

  auto gload = [&](int kb) {
    const int64_t k = (int64_t)kb * BK + ck * 16;
#pragma unroll
    for (int i = 0; i < CF::A_CHUNKS; ++i) {
      const int64_t row = t.row0 + rbase + i * CF::kRowsPerPass;
      const bool ok = row < t.row_end;
      ra[i] = load_chunk<VEC>(t.A + (ok ? row : 0) * p.lda, k, K, ok);
    }
#pragma unroll
    for (int i = 0; i < CF::B_CHUNKS; ++i) {
      const int64_t n = t.n0 + rbase + i * CF::kRowsPerPass;
      const bool ok = n < N;
      rb[i] = load_chunk<VEC>(t.B + (ok ? n : 0) * p.ldb, k, K, ok);
    }
    if (tid < BM) {
      const int64_t row = t.row0 + tid;
      rs = row < t.row_end ? t.a_s[row * p.as_rs + (int64_t)kb * p.as_ks] : 0.0f;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CF::A_CHUNKS; ++i)
      *reinterpret_cast<u32x4*>(As + buf * CF::A_BYTES + swz(rbase + i * CF::kRowsPerPass, ck)) = ra[i];
#pragma unroll
    for (int i = 0; i < CF::B_CHUNKS; ++i)
      *reinterpret_cast<u32x4*>(Bs + buf * CF::B_BYTES + swz(rbase + i * CF::kRowsPerPass, ck)) = rb[i];
    if (tid < BM) Ss[buf * BM + tid] = rs;
  };

  v4f acc[CF::TM][CF::TN];
#pragma unroll
  for (int i = 0; i < CF::TM; ++i)
#pragma unroll
    for (int j = 0; j < CF::TN; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  // The weight scale row of this wave's 128-column block (clamped for waves
  // past the last column, whose results are never stored).
  int64_t nbi = (t.n0 + wn * CF::WN) / BK;
  if (nbi > kbn - 1) nbi = kbn - 1;
  const float* bsrow = t.b_s + nbi * p.ldbs;

  const int kb0 = t.kb0, kb1 = t.kb1;
  (void)nkb;
  if (kb0 < kb1) {
    gload(kb0);
    lstore(0);
  }
  __syncthreads();

  const int fr = lane & 15, fg = lane >> 4;
  for (int kb = kb0; kb < kb1; ++kb) {
    const int buf = (kb - kb0) & 1;
    if (kb + 1 < kb1) gload(kb + 1);
    const float bsv = bsrow[kb];
    const uint8_t* at = As + buf * CF::A_BYTES;
    const uint8_t* bt = Bs + buf * CF::B_BYTES;
    v8i bfr[CF::TN];
#pragma unroll
    for (int j = 0; j < CF::TN; ++j) bfr[j] = read_frag(bt, wn * CF::WN + j * 16 + fr, fg);
#pragma unroll
    for (int i = 0; i < CF::TM; ++i) {
      const v8i afr = read_frag(at, wm * CF::WM + i * 16 + fr, fg);
      const v4f sa = *reinterpret_cast<const v4f*>(Ss + buf * BM + wm * CF::WM + i * 16 + 4 * fg);
      const v4f sc = sa * bsv;
#pragma unroll
      for (int j = 0; j < CF::TN; ++j) {
        const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            afr, bfr[j], v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[i][j][v] = __builtin_fmaf(part[v], sc[v], acc[i][j][v]);
      }
    }
    if (kb + 1 < kb1) lstore(buf ^ 1);
    __syncthreads();
  }

  __syncthreads();
  if (t.partial != nullptr) {
    store_partial<CF, false>(p, t, acc, wm, wn, lane);
    return;
  }
  store_tile<CF, false>(p, t, acc, smem, wave, wm, wn, lane, [] {});
}

// Gated epilogue ("DeepSeek-V3 Administrator & Developer Guide" 1.2, the
// feed-forward w2(SiLU(w1 x) * w3 x), with the act_quant of 8.5.1 that feeds
// the w2 product).  The tile's columns 0..127 hold x w1^T and columns
// 128..255 hold x w3^T for the same 128 outputs (the weight rows were loaded
// that way).  After the bf16 results are staged in LDS, each DPP row of 16
// lanes takes one tile row, 8 outputs per lane: h = bf16(SiLU(h1) * h3), the
// block maximum over the 16 lanes, then the block's scale and e4m3 codes,
// computed exactly as the standalone gate-and-quantise kernel does.
template <class CF, class Hook>
__device__ __forceinline__ void store_glu_quant(const GemmArgs& p, const TileRef& t,
                                                const v4f (&acc)[CF::TM][CF::TN], uint8_t* smem, int wave,
                                                int lane, Hook&& hook) {
  asm volatile("" : "+v"(lane));
  static_assert(CF::BN == 2 * kBlock && kBlock % CF::WN == 0, "one 128-column block of each half per tile");
  static_assert(CF::BM % (4 * CF::NW) == 0, "whole groups of four rows per wave");
  stage_c<CF, true>(acc, smem, wave, lane);
  __syncthreads();
  constexpr int CS = CF::WN + CF::CPAD;
  const uint16_t* cst = reinterpret_cast<const uint16_t*>(smem);
  const int l16 = lane & 15, quad = lane >> 4;
  const int c = l16 * 8;
  // Staged column c of the w1 half lies in wave column c / WN, the matching
  // w3 column in wave column (128 + c) / WN; both at column c % WN there.
  const int wc1 = c / CF::WN, wc3 = (kBlock + c) / CF::WN, cc = c % CF::WN;
  const int64_t blk = t.n0 / kBlock;
  // All of this lane's staged values are read first, so hook() may reuse the LDS.
  constexpr int IT = CF::BM / (4 * CF::NW);
  u32x4 gs[IT], us[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int r = (it * CF::NW + wave) * 4 + quad;
    const int rw = r / CF::WM, rr = r % CF::WM;
    gs[it] = *reinterpret_cast<const u32x4*>(cst + ((rw * CF::WAVES_N + wc1) * CF::WM + rr) * CS + cc);
    us[it] = *reinterpret_cast<const u32x4*>(cst + ((rw * CF::WAVES_N + wc3) * CF::WM + rr) * CS + cc);
  }
  hook();
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int r = (it * CF::NW + wave) * 4 + quad;
    const u32x4 g = gs[it], u = us[it];
    const float gv[8] = {bf16_lo(g.x), bf16_hi(g.x), bf16_lo(g.y), bf16_hi(g.y),
                         bf16_lo(g.z), bf16_hi(g.z), bf16_lo(g.w), bf16_hi(g.w)};
    const float uv[8] = {bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y),
                         bf16_lo(u.z), bf16_hi(u.z), bf16_lo(u.w), bf16_hi(u.w)};
    float v[8];
    __bf16 hb[8];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[j] = silu_mul_bf16(gv[j], uv[j], &hb[j]);
      amax = fmaxf(amax, fabsf(v[j]));
    }
    amax = max_row16(amax);
    const float sc = block_scale_bf16(amax, p.q_ue8m0);
    const float rc = recip_rn(sc);
    const int64_t row = t.row0 + r;
    if (row < t.row_end) {
      u32x2 o;
      o.x = pack_e4m3x4(div_by_scale(v[0], sc, rc), div_by_scale(v[1], sc, rc), div_by_scale(v[2], sc, rc),
                        div_by_scale(v[3], sc, rc));
      o.y = pack_e4m3x4(div_by_scale(v[4], sc, rc), div_by_scale(v[5], sc, rc), div_by_scale(v[6], sc, rc),
                        div_by_scale(v[7], sc, rc));
      *reinterpret_cast<u32x2*>(p.qy + row * p.ldqy + t.n0 + c) = o;
      if (p.qh != nullptr) {
        u32x4 h;
        h.x = pack_bf16x2(v[0], v[1]);
        h.y = pack_bf16x2(v[2], v[3]);
        h.z = pack_bf16x2(v[4], v[5]);
        h.w = pack_bf16x2(v[6], v[7]);
        *reinterpret_cast<u32x4*>(p.qh + row * p.ldqh + t.n0 + c) = h;
      }
      if (l16 == 0) p.qs[row * p.qs_rs + blk * p.qs_ks] = sc;
    }
  }
}

// ---- direct-to-LDS pipeline (16-byte aligned operands) --------------------------------
//
// Each stage of a STAGES-deep LDS ring holds one K-block: BM rows of A, BN rows
// of B (128 bytes each, in the same swizzled layout as above) and the BM
// activation scales.  Stages are filled with buffer_load_dwordx4 ... lds, which
// writes a wavefront's 64 x 16 bytes straight into LDS without passing through
// VGPRs; the swizzle is applied on the global side (the lane that lands on LDS
// chunk p fetches the logical chunk stored there).  The buffer descriptors
// start at the tile's first row and end after its last valid row, so rows past
// the matrix edge read as zero without a branch; a chunk past K is sent to an
// out-of-range offset for the same effect.  One barrier per K-block: after it,
// stage kb is complete for every wave and stage kb-1 is no longer read, so the
// loads of K-block kb+STAGES-1 are issued into it before the MFMAs of kb.

typedef int i32x4 __attribute__((ext_vector_type(4)));

// The loads are issued from inline assembly so that the compiler, which
// cannot tell the stages of the ring apart, does not add a vmcnt(0) wait in
// front of every LDS read; the kernel waits for each stage itself.  M0 holds
// the wave's LDS destination and is set in the same statement (and declared
// clobbered, so the compiler keeps nothing of its own in M0 across it); the
// s_nop provides the wait state required between an SALU write of M0 and an
// LDS DMA that reads it.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

// M0 is a reserved register, so clang warns that a clobber of it is not
// saved and restored around the statement; that is intended (nothing needs
// the old value), and the clobber still records the write of M0 in the
// statement's dependencies, so no instruction of the compiler's that reads
// M0 is moved across it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"

// Byte address of lane l: rsrc base + voff + soff (the scalar part carries the
// K-block offset, so the per-lane offsets stay fixed over the K loop).
__device__ __forceinline__ void dma_b128(i32x4 rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 1\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}

// Four bytes per lane (for rows that are only 4-byte aligned).
__device__ __forceinline__ void dma_b32(i32x4 rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 1\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}

// The same with the nontemporal hint: for weight panels that one tile
// streams once (the short, wide tiles of the grouped and gated products).
__device__ __forceinline__ void dma_b128_nt(i32x4 rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 1\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
               :
               : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}

// Per-lane 64-bit addresses: each active lane fetches one dword from anywhere.
__device__ __forceinline__ void dma_gather_b32(uint32_t lds, const float* addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 1\n\tglobal_load_lds_dword %1, off"
               :
               : "s"(lds), "v"(addr)
               : "memory", "m0");
}

#pragma clang diagnostic pop

// The lane index behind an empty statement: values derived from it are
// computed where they are used instead of being hoisted out of a persistent
// kernel's tile loop, where they would stay live across the K loop.
__device__ __forceinline__ int lane_id() {
  int l = (int)(threadIdx.x & 63);
  asm volatile("" : "+v"(l));
  return l;
}

constexpr uint32_t kOob = 0x80000000u;  // above every descriptor's size

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int STAGES_>
struct DmaCfg {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, STAGES = STAGES_;
  static constexpr int NW = WAVES_M * WAVES_N;
  static constexpr int kThreads = 64 * NW;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int TM = WM / 16, TN = WN / 16;
  // Scale area of a stage: one slot of SA_ROWS + 4 floats per wave holding the
  // activation scales of the rows that wave fetches, then (at index SA_ROWS)
  // the weight scale of the wave's own 128-column block.
  // (At least 16: with fewer tile rows than 16 per wave, the first BM / 16
  // waves fetch all of them and the rest only their weight scale.)
  static constexpr int SA_ROWS = BM / NW < 16 ? 16 : BM / NW;
  static constexpr int SAW = SA_ROWS + 4;
  static constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK;
  static constexpr int S_OFF = A_BYTES + B_BYTES;
  static constexpr int STAGE_BYTES = S_OFF + NW * SAW * 4;
  static constexpr int A_INSTR = A_BYTES / 1024 / NW;   // 1 KB (8 rows) per wave instruction
  static constexpr int B_INSTR = B_BYTES / 1024 / NW;
  static constexpr int LOADS = A_INSTR + B_INSTR + 1;    // vector-memory instructions per stage and wave
  static constexpr int CPAD = 8;
  static constexpr int C_BYTES = NW * WM * (WN + CPAD) * 2;
  static constexpr int MAIN_BYTES = STAGES * STAGE_BYTES;
  static constexpr int LDS_BYTES = MAIN_BYTES > C_BYTES ? MAIN_BYTES : C_BYTES;
  static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0, "whole 1 KB segments per wave");
  static_assert(SA_ROWS >= 16 && SA_ROWS % 16 == 0 && SA_ROWS < 64 && BM % NW == 0, "scale rows per wave");
  static_assert(WN <= 128 && 128 % WN == 0, "a wave's columns must lie in one 128-block");
  static_assert(WM % SA_ROWS == 0, "a wave's rows start on a scale slot");
  static_assert(STAGES >= 2 && LOADS * (STAGES - 2) < 64, "vmcnt range");
  // Weight loads with the nontemporal hint for the 64- and 128-row tiles of
  // 256 columns: with at most 128 rows per weight panel the panel is streamed
  // once (routed-expert up-projection −5%, down −1%; on the 256-row tiles,
  // whose panels neighbouring tiles share, the hint cost the down-projection 7%).
  static constexpr bool NT_B = BN == 256 && BM <= 128;
};

// Large products: 256x256 tiles, 8 waves of 128x64 (one workgroup per CU);
// products with too few of those tiles and split-K products: 128x128 tiles,
// 4 waves of 64x64 (two workgroups per CU).
// Large dense products run as one persistent workgroup per CU.
using CfgDmaBig = DmaCfg<256, 256, 2, 4, 2>;
using CfgDma = DmaCfg<128, 128, 2, 2, 2>;
// Dense products of 17 to 64 rows (and their split-K form): 64-row tiles,
// 4 waves of 64x32.
using CfgGrp = DmaCfg<64, 128, 1, 4, 2>;
// Gated form, and the grouped classes of at most 64 and 65-128 rows of both
// forms: 256-column tiles (for the gated form 128 columns of each half),
// 8 waves of 32x64 or 64x64; the large dense tile otherwise.  The small tiles
// take 83 KB and 100 KB of LDS per stage pair, so one workgroup fits per CU;
// a third stage (125 KB, 149 KB) keeps more weight bytes in flight, which
// measured 8% faster on the routed-expert up-projection, whose small experts
// stream their weights once.  With all three classes at 8 waves, a grouped
// product runs them in one launch (grouped_merged_kernel).
using CfgGlu64 = DmaCfg<64, 256, 2, 4, 3>;
using CfgGlu128 = DmaCfg<128, 256, 2, 4, 3>;

__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));  // stride 0: raw buffer
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

// Wait until at most n vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <class CF>
__device__ __forceinline__ void wait_stage(int later) {
  // `later` = number of stages issued after the one waited for (0..STAGES-2).
  if constexpr (CF::STAGES >= 4) {
    if (later >= 2) { wait_vmcnt<CF::LOADS * 2>(); return; }
  }
  if constexpr (CF::STAGES >= 3) {
    if (later >= 1) { wait_vmcnt<CF::LOADS>(); return; }
  }
  wait_vmcnt<0>();
}

// KFULL: K is a multiple of 128, so no K-block has chunks past K.
// POW2: every scale is a power of two.  The block-scaled form of the MFMA
// then applies them: with the operand layout used here, lane l supplies the
// E8M0 scale (the fp32 exponent field, value 2^(e-127)) of operand row l % 16
// for the 32-byte K slice l / 16, and a 128-K-block's four slices share
// their scale, so each lane passes its own row's exponent and the MFMA
// accumulates straight into the accumulator.  (Without POW2 the scale
// operands are the literal 0, for which the compiler emits the unscaled
// instruction; a zero scale supplied at run time would mean 2^-127.)
// GLU: the gated form (BN = 256): the tile's weight rows are w1 rows
// n0..n0+127 followed by w3 rows F+n0..F+n0+127, and the epilogue is the
// gate and quantisation instead of the bf16 store.
// Per-wave state of the direct-to-LDS loads of one tile: the buffer
// descriptors of the tile's A rows and B rows, the per-lane source offsets of
// the wave's segments and the address of its scale gather.  Re-initialised
// for every tile.
template <class CF, bool KFULL, bool GLU>
struct DmaLoader {
  i32x4 rsA, rsB;
  uint32_t offA[CF::A_INSTR], offB[CF::B_INSTR];
  // Logical 16-byte chunk (0..7) of segment n's lane at bits 3n..3n+2
  // (A segments, then B segments); only read for a K-block with chunks past K.
  uint32_t kc;
  const float* sbase;
  uint32_t sstep;
  bool s_act;
  int64_t K;
  uint32_t lds0;
  int wave;

  __device__ __forceinline__ void init(const GemmArgs& p, const TileRef& t, uint8_t* smem) {
    constexpr int NW = CF::NW;
    const int lane = lane_id();
    wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int wn = wave % CF::WAVES_N;
    K = p.K;
    const int64_t N = p.N;
    const int64_t kbn = (N + BK - 1) / BK;
    const int64_t rowsA = t.row_end - t.row0 < CF::BM ? t.row_end - t.row0 : CF::BM;
    // Gathered rows: one descriptor over all of A, each lane's source row
    // from the index (clamped); rows past the tile's end read as zero.
    const bool gather = p.a_rows != nullptr;
    auto src_row = [&](int r) __attribute__((always_inline)) {
      int64_t v = p.a_rows[t.row0 + r];
      return v < 0 ? (int64_t)0 : (v >= p.a_rows_n ? p.a_rows_n - 1 : v);
    };
    rsA = gather ? make_rsrc(t.A, (uint32_t)(p.a_rows_n * p.lda))
                 : make_rsrc(t.A + t.row0 * p.lda, (uint32_t)(rowsA * p.lda));
    // The weight-scale row of this wave's 128-column block (clamped for waves
    // past the last column, whose results are never stored).
    int64_t nbi;
    if constexpr (GLU) {
      static_assert(CF::BN == 2 * BK, "gated tiles hold one 128-row block of w1 and of w3");
      // One descriptor from w1 row n0 to the end of w3 row F + n0 + 127.
      rsB = make_rsrc(t.B + t.n0 * p.ldb, (uint32_t)((p.glu_f + BK) * p.ldb));
      nbi = (wn * CF::WN < BK ? 0 : p.glu_f / BK) + t.n0 / BK;
    } else {
      const int64_t rowsB = N - t.n0 < CF::BN ? N - t.n0 : CF::BN;
      rsB = make_rsrc(t.B + t.n0 * p.ldb, (uint32_t)(rowsB * p.ldb));
      nbi = (t.n0 + wn * CF::WN) / BK;
      if (nbi > kbn - 1) nbi = kbn - 1;
    }
    // Scale gather: lane l < SA_ROWS fetches a_s of tile row wave*SA_ROWS + l,
    // lane SA_ROWS fetches b_s[nbi, kb]; K-block kb adds kb * sstep bytes.
    const int srow = wave * CF::SA_ROWS + lane;
    s_act = lane < CF::SA_ROWS ? srow < rowsA : lane == CF::SA_ROWS;
    const int64_t arow = !s_act || lane >= CF::SA_ROWS ? 0 : (gather ? src_row(srow) : t.row0 + srow);
    sbase = lane < CF::SA_ROWS ? t.a_s + arow * p.as_rs : t.b_s + nbi * p.ldbs;
    sstep = lane < CF::SA_ROWS ? (uint32_t)(p.as_ks * 4) : 4u;
    // Per-lane source offsets (K-block independent): lane -> LDS chunk (row
    // r, physical chunk lane % 8) <- logical chunk c of row r.
    static_assert(CF::A_INSTR + CF::B_INSTR <= 10, "chunk indices packed in 32 bits");
    kc = 0;
#pragma unroll
    for (int i = 0; i < CF::A_INSTR; ++i) {
      const int r = (wave + NW * i) * 8 + (lane >> 3);
      const int c = (lane & 7) ^ swz_key(r);
      offA[i] = !gather ? (uint32_t)(r * p.lda + c * 16)
                        : (r < rowsA ? (uint32_t)(src_row(r) * p.lda + c * 16) : kOob);
      kc |= (uint32_t)c << (3 * i);
    }
#pragma unroll
    for (int i = 0; i < CF::B_INSTR; ++i) {
      const int r = (wave + NW * i) * 8 + (lane >> 3);
      const int c = (lane & 7) ^ swz_key(r);
      const int64_t rb = (GLU && r >= BK) ? p.glu_f + (r - BK) : (int64_t)r;  // row past the descriptor base
      offB[i] = (uint32_t)(rb * p.ldb + c * 16);
      kc |= (uint32_t)c << (3 * (CF::A_INSTR + i));
    }
    lds0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr(smem));
  }

  // Load n (0 .. LOADS-1) of K-block kb into `stage`: n < A_INSTR are A
  // segments, then B segments, then the scale gather.  Chunks past K (only
  // in a last, partial K-block) go to an offset beyond the descriptor and
  // read as zero.
  __device__ __forceinline__ void issue(int n, int kb, int stage) const {
    constexpr int NW = CF::NW;
    const uint32_t st = lds0 + (uint32_t)(stage * CF::STAGE_BYTES);
    const uint32_t kbyte = (uint32_t)kb * BK;
    const int64_t kchunk = (int64_t)kbyte + (int64_t)(((kc >> (3 * n)) & 7u) * 16u);
    if (n < CF::A_INSTR) {
      const uint32_t off = (KFULL || kchunk < K) ? offA[n] : kOob;
      dma_b128(rsA, st + (uint32_t)((wave + NW * n) * 1024), off, kbyte);
    } else if (n < CF::A_INSTR + CF::B_INSTR) {
      const int m = n - CF::A_INSTR;
      const uint32_t off = (KFULL || kchunk < K) ? offB[m] : kOob;
      if constexpr (CF::NT_B)
        dma_b128_nt(rsB, st + (uint32_t)(CF::A_BYTES + (wave + NW * m) * 1024), off, kbyte);
      else
        dma_b128(rsB, st + (uint32_t)(CF::A_BYTES + (wave + NW * m) * 1024), off, kbyte);
    } else if (s_act) {
      const float* src = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(sbase) +
                                                        (uint64_t)(uint32_t)kb * sstep);
      dma_gather_b32(st + (uint32_t)(CF::S_OFF + wave * CF::SAW * 4), src);
    }
  }

  // K-blocks kb0 .. kb0 + n - 1 (at most kb1 - 1) into stages 0 .. n - 1.
  __device__ __forceinline__ void preload(int kb0, int kb1, int n) const {
    for (int s = 0; s < n; ++s)
      if (kb0 + s < kb1)
#pragma unroll
        for (int i = 0; i < CF::LOADS; ++i) issue(i, kb0 + s, s);
  }
};

// The K loop of one tile over K-blocks [kb0, kb1) into acc.  K-blocks kb0 ..
// kb0 + pre - 1 were issued into stages 0 .. pre - 1 before the call (pre is
// STAGES - 1, or STAGES when the previous tile's epilogue issued them);
// K-block kb + STAGES - 1 is issued during K-block kb unless it already was.
// first_all: the first wait covers every outstanding vector-memory operation
// (required when pre = STAGES, and when the previous tile's stores may still
// be in flight: loads and stores need not complete in order).
//
// KFULL: K is a multiple of 128, so no K-block has chunks past K.
// POW2: every scale is a power of two.  The block-scaled form of the MFMA
// then applies them: with the operand layout used here, lane l supplies the
// E8M0 scale (the fp32 exponent field, value 2^(e-127)) of operand row l % 16
// for the 32-byte K slice l / 16, and a 128-K-block's four slices share
// their scale, so each lane passes its own row's exponent and the MFMA
// accumulates straight into the accumulator.  (Without POW2 the scale
// operands are the literal 0, for which the compiler emits the unscaled
// instruction; a zero scale supplied at run time would mean 2^-127.)
template <class CF, bool KFULL, bool POW2, bool GLU>
__device__ __forceinline__ void k_loop(const DmaLoader<CF, KFULL, GLU>& ld, int kb0, int kb1, int pre, bool first_all,
                                       uint8_t* smem, v4f (&acc)[CF::TM][CF::TN]) {
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wm = wave / CF::WAVES_N, wn = wave % CF::WAVES_N;
#pragma unroll
  for (int i = 0; i < CF::TM; ++i)
#pragma unroll
    for (int j = 0; j < CF::TN; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  // Fragment addressing.  Row R + fr of an operand tile (R a multiple of 16)
  // keeps its logical chunk c at fr*128 + ((c ^ key(fr)) << 4) past row R, so
  // a lane's two chunk offsets are fixed and each 16-row slice is a constant
  // offset from the wave's base: the reads take immediate offsets.
  const int fr = lane & 15, fg = lane >> 4;
  const uint32_t fkey = (uint32_t)((fr & 7) ^ (fr >> 3));
  const uint32_t lf0 = (uint32_t)(fr * BK) + ((((uint32_t)(2 * fg)) ^ fkey) << 4);
  const uint32_t lf1 = (uint32_t)(fr * BK) + ((((uint32_t)(2 * fg + 1)) ^ fkey) << 4);
  auto frag = [&](const uint8_t* base) __attribute__((always_inline)) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(base + lf0);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(base + lf1);
    v8i f;
    f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
    f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
    return f;
  };
  // The activation scale of row wm*WM + 16i + fr sits in slot row / SA_ROWS at
  // index row % SA_ROWS; WM and 16i are whole multiples of 16, so the lane
  // part is fr and the rest is a constant per subtile.
  constexpr int SCALE_WAVE = CF::WM / CF::SA_ROWS * CF::SAW;

  // The loads of K-block kb + STAGES - 1 are spread over the row-subtile
  // steps of kb (PER per step) instead of being issued together after the
  // barrier: a burst of 8 waves x LOADS vector-memory instructions stalls
  // instruction issue until the load unit has accepted them.
  constexpr int PER = (CF::LOADS + CF::TM - 1) / CF::TM;
  for (int kb = kb0; kb < kb1; ++kb) {
    if (first_all && kb == kb0) {
      wait_vmcnt<0>();
    } else {
      const int later = (kb1 - 1 - kb) < (CF::STAGES - 2) ? (kb1 - 1 - kb) : (CF::STAGES - 2);
      wait_stage<CF>(later);
    }
    __syncthreads();
    // K-block kn is issued now unless it was issued before the loop or lies
    // past the end (a uniform branch: the last STAGES - 1 K-blocks issue
    // nothing).
    const int kn = kb + CF::STAGES - 1;
    const bool more = kn < kb1 && kn >= kb0 + pre;
    const int slot = (kb - kb0 + CF::STAGES - 1) % CF::STAGES;
    const uint8_t* st = smem + ((kb - kb0) % CF::STAGES) * CF::STAGE_BYTES;
    const float* sarea = reinterpret_cast<const float*>(st + CF::S_OFF);
    const float bsv = sarea[wave * CF::SAW + CF::SA_ROWS];
    const uint8_t* at = st + wm * CF::WM * BK;
    const uint8_t* bt = st + CF::A_BYTES + wn * CF::WN * BK;
    const float* sl = sarea + wm * SCALE_WAVE + fr;
    v8i bfr[CF::TN];
#pragma unroll
    for (int j = 0; j < CF::TN; ++j) bfr[j] = frag(bt + j * 16 * BK);
    // The weight fragment is the MFMA's first operand, so a lane's four
    // results of a subtile are four columns of one row (the column layout)
    // and share one activation scale.  Row-subtile i's MFMAs are issued
    // before the rescale of row-subtile i-1, so the fma of a partial product
    // never waits for the MFMA that has just produced it.
    // Row-subtile i+1's activation fragment and scale are read before
    // subtile i's MFMAs (in program order ahead of the inline-asm load
    // issues, which the compiler does not move memory reads across), so the
    // LDS latency is covered by a subtile's MFMAs instead of stalling the
    // first MFMA of every subtile.
    auto ascale = [&](int i) __attribute__((always_inline)) {
      return sl[(i * 16 / CF::SA_ROWS) * CF::SAW + (i * 16) % CF::SA_ROWS];
    };
    v8i afr = frag(at);
    float asv = ascale(0);
    if constexpr (POW2) {
      const int eb = (int)(__float_as_uint(bsv) >> 23);
#pragma unroll
      for (int i = 0; i < CF::TM; ++i) {
        v8i afr_next = afr;
        float asv_next = asv;
        if (i + 1 < CF::TM) {
          afr_next = frag(at + (i + 1) * 16 * BK);
          asv_next = ascale(i + 1);
        }
        const int ea = (int)(__float_as_uint(asv) >> 23);
#pragma unroll
        for (int j = 0; j < CF::TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bfr[j], afr, acc[i][j], 0, 0, 0, eb, 0, ea);
        if (more) {
#pragma unroll
          for (int n = i * PER; n < (i + 1) * PER && n < CF::LOADS; ++n) ld.issue(n, kn, slot);
        }
        afr = afr_next;
        asv = asv_next;
      }
      continue;
    }
    v4f part[2][CF::TN];
    float scv[2];
#pragma unroll
    for (int i = 0; i <= CF::TM; ++i) {
      if (i < CF::TM) {
        v8i afr_next = afr;
        float asv_next = asv;
        if (i + 1 < CF::TM) {
          afr_next = frag(at + (i + 1) * 16 * BK);
          asv_next = ascale(i + 1);
        }
        scv[i & 1] = asv * bsv;
#pragma unroll
        for (int j = 0; j < CF::TN; ++j)
          part[i & 1][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              bfr[j], afr, v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0, 0, 0, 0);
        afr = afr_next;
        asv = asv_next;
        if (more) {
#pragma unroll
          for (int n = i * PER; n < (i + 1) * PER && n < CF::LOADS; ++n) ld.issue(n, kn, slot);
        }
      }
      if (i > 0) {
        const int r = i - 1;
#pragma unroll
        for (int j = 0; j < CF::TN; ++j) {
#pragma unroll
          for (int v = 0; v < 4; ++v)
            acc[r][j][v] = __builtin_fmaf(part[r & 1][j][v], scv[r & 1], acc[r][j][v]);
          // An empty statement that takes the new accumulators: the fmas stay
          // here instead of being sunk to the end of the K-block, where all of
          // the block's partial products would have to be live at once.
          asm volatile("" ::"v"(acc[r][j][0]), "v"(acc[r][j][1]), "v"(acc[r][j][2]), "v"(acc[r][j][3]));
        }
      }
    }
  }
}

// One tile by itself: preload STAGES - 1 K-blocks, the K loop, the epilogue.
// GLU: the gated form (BN = 256): the tile's weight rows are w1 rows
// n0..n0+127 followed by w3 rows F+n0..F+n0+127, and the epilogue is the
// gate and quantisation instead of the bf16 store.
template <class CF, bool KFULL, bool POW2, bool GLU>
__device__ __forceinline__ void gemm_tile_dma(const GemmArgs& p, const TileRef& t, uint8_t* smem) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wm = wave / CF::WAVES_N, wn = wave % CF::WAVES_N;
  DmaLoader<CF, KFULL, GLU> ld;
  ld.init(p, t, smem);
  ld.preload(t.kb0, t.kb1, CF::STAGES - 1);
  v4f acc[CF::TM][CF::TN];
  k_loop<CF, KFULL, POW2, GLU>(ld, t.kb0, t.kb1, CF::STAGES - 1, false, smem, acc);
  // Every load has landed and every wave is done with the ring before the
  // epilogue reuses the LDS.
  wait_vmcnt<0>();
  __syncthreads();
  auto none = [] {};
  if constexpr (GLU) {
    store_glu_quant<CF>(p, t, acc, smem, wave, lane, none);
    return;
  }
  if (t.partial != nullptr) {
    store_partial<CF, true>(p, t, acc, wm, wn, lane);
    return;
  }
  store_tile<CF, true>(p, t, acc, smem, wave, wm, wn, lane, none);
}

// Workgroup i runs on XCD i % 8.  Renumber ids 0..total-1 so that each XCD
// owns one contiguous range (and so shares its L2 among neighbouring tiles).
__device__ __forceinline__ int64_t xcd_contiguous(int64_t pid, int64_t total) {
  const int64_t q = total / kXcds, r = total % kXcds;
  const int64_t xcd = pid % kXcds, idx = pid / kXcds;
  return (xcd < r) ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

// x / d for x >= 0, d > 0 (tile-index arithmetic at the start of a tile):
// the 32-bit division whenever both fit, since a 64-bit integer division is
// a long instruction sequence that delays the tile's first loads.
__device__ __forceinline__ int64_t div_u(int64_t x, int64_t d) {
  if ((uint64_t)(x | d) <= 0xffffffffull) return (int64_t)((uint32_t)x / (uint32_t)d);
  return x / d;
}

// Map a linear workgroup id to (tile_m, tile_n): XCD-contiguous ranges, then
// GROUP_M-row groups inside a range.
__device__ __forceinline__ void tile_of(int64_t pid, int64_t tiles_m, int64_t tiles_n, int64_t& tm, int64_t& tn) {
  const int64_t total = tiles_m * tiles_n;
  pid = xcd_contiguous(pid, total);
  const int64_t per_group = (int64_t)kGroupM * tiles_n;
  const int64_t gid = div_u(pid, per_group);
  const int64_t first_m = gid * kGroupM;
  const int64_t gsize = (tiles_m - first_m) < kGroupM ? (tiles_m - first_m) : kGroupM;
  const int64_t in = pid - gid * per_group;
  tn = div_u(in, gsize);
  tm = first_m + (in - tn * gsize);
}

// VEC > 0: the register-staged pipeline with VEC-byte loads (any alignment;
// power-of-two scales take the general fp32 path there);
// VEC <= 0: the direct-to-LDS pipeline (16-byte aligned operands,
// K % 16 == 0): 0 / -1 for K % 128 == 0 / otherwise, -2 / -3 the same with
// power-of-two scales.
// GLU (direct-to-LDS only): the gated form, whose column tiles are the F/128
// output blocks.
template <class CF, int VEC, bool GLU>
__device__ __forceinline__ void run_tile(const GemmArgs& p, const TileRef& t, uint8_t* smem) {
  if constexpr (VEC <= 0) {
    gemm_tile_dma<CF, VEC == 0 || VEC == -2, VEC <= -2, GLU>(p, t, smem);
  } else {
    static_assert(!GLU, "the gated form runs on the direct-to-LDS pipeline only");
    gemm_tile<CF, VEC>(p, t, smem);
  }
}

// Column tiles of a launch and the output column where tile tn starts.
template <class CF, bool GLU>
__device__ __forceinline__ int64_t col_tiles(const GemmArgs& p) {
  return GLU ? (p.glu_nt > 0 ? p.glu_nt : p.glu_f / BK) : (p.N + CF::BN - 1) / CF::BN;
}
template <class CF, bool GLU>
constexpr int kColStep = GLU ? BK : CF::BN;

template <class CF, int VEC, bool GLU = false>
__global__ __launch_bounds__(CF::kThreads) void gemm_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[CF::LDS_BYTES];
  const int64_t tiles_m = (p.M + CF::BM - 1) / CF::BM;
  const int64_t tiles_n = col_tiles<CF, GLU>(p);
  int64_t tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  TileRef t;
  t.A = p.A;
  t.a_s = p.a_s;
  t.B = p.B;
  t.b_s = p.b_s;
  t.row0 = tm * CF::BM;
  t.row_end = p.M;
  t.n0 = tn * kColStep<CF, GLU>;
  t.kb0 = 0;
  t.kb1 = (int)((p.K + BK - 1) / BK);
  t.partial = nullptr;
  if (gridDim.y > 1) {
    // split K: blockIdx.y selects a contiguous range of K-blocks
    const int per = (t.kb1 + (int)gridDim.y - 1) / (int)gridDim.y;
    t.kb0 = (int)blockIdx.y * per;
    t.kb1 = t.kb0 + per < t.kb1 ? t.kb0 + per : t.kb1;
    t.partial = p.partial + (int64_t)blockIdx.y * p.M * p.N;
  }
  run_tile<CF, VEC, GLU>(p, t, smem);
}

// Large dense products as a persistent kernel: one workgroup per CU walks
// the tiles pid = blockIdx.x, + gridDim.x, ...  gridDim.x is a multiple of the
// 8 XCDs, so all of a workgroup's tiles lie in its own XCD's range and the
// tiles in flight together are the ones a launch of one workgroup per tile
// would run together.  The next tile's first STAGES K-blocks are issued from
// the epilogue as soon as the staged results have been read back from LDS,
// so their latency is covered by the epilogue's arithmetic and stores.
template <class CF, int VEC, bool GLU = false>
__global__ __launch_bounds__(CF::kThreads) void gemm_persistent_kernel(GemmArgs p) {
  static_assert(VEC <= 0, "direct-to-LDS pipeline only");
  constexpr bool KFULL = VEC == 0 || VEC == -2, POW2 = VEC <= -2;
  __shared__ __attribute__((aligned(16))) uint8_t smem[CF::LDS_BYTES];
  const int64_t tiles_m = (p.M + CF::BM - 1) / CF::BM;
  const int64_t tiles_n = col_tiles<CF, GLU>(p);
  const int64_t total = tiles_m * tiles_n;
  const int kb1 = (int)((p.K + BK - 1) / BK);
  const int pre = kb1 < CF::STAGES ? kb1 : CF::STAGES;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wm = wave / CF::WAVES_N, wn = wave % CF::WAVES_N;
  auto tile = [&](int64_t pid) __attribute__((always_inline)) {
    int64_t tm, tn;
    tile_of(pid, tiles_m, tiles_n, tm, tn);
    TileRef r;
    r.A = p.A;
    r.a_s = p.a_s;
    r.B = p.B;
    r.b_s = p.b_s;
    r.row0 = tm * CF::BM;
    r.row_end = p.M;
    r.n0 = tn * kColStep<CF, GLU>;
    r.kb0 = 0;
    r.kb1 = kb1;
    r.partial = nullptr;
    return r;
  };
  int64_t pid = blockIdx.x;
  TileRef t = tile(pid);
  DmaLoader<CF, KFULL, GLU> ld;
  ld.init(p, t, smem);
  ld.preload(0, kb1, pre);
  v4f acc[CF::TM][CF::TN];
  for (;;) {
    k_loop<CF, KFULL, POW2, GLU>(ld, 0, kb1, pre, true, smem, acc);
    wait_vmcnt<0>();
    __syncthreads();
    const int64_t next = pid + gridDim.x;
    auto prefetch = [&]() __attribute__((always_inline)) {
      __syncthreads();  // every wave has read its staged results
      if (next < total) {
        ld.init(p, tile(next), smem);
        ld.preload(0, kb1, pre);
      }
    };
    if constexpr (GLU)
      store_glu_quant<CF>(p, t, acc, smem, wave, lane, prefetch);
    else
      store_tile<CF, true>(p, t, acc, smem, wave, wm, wn, lane, prefetch);
    if (next >= total) break;
    pid = next;
    t = tile(pid);
  }
}

// Sum the split-K partials in split order (deterministic) and round to bf16.
// The kernel is bound by the latency of its loads, so each thread keeps
// IN_FLIGHT splits' loads in flight before adding them in order: VEC = 4
// (four consecutive outputs per thread, 16-byte loads, 8 splits at a time)
// for few splits over many outputs, VEC = 1 (one output per thread, 32 splits
// at a time) for many splits over few outputs.
template <int VEC, int IN_FLIGHT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs p, int splits) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * VEC;
  const int64_t MN = p.M * p.N;
  if (i >= MN) return;
  const bool full = i + VEC <= MN && (MN % VEC) == 0;
  float s[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) s[e] = 0.0f;
  for (int k0 = 0; k0 < splits; k0 += IN_FLIGHT) {
    float v[IN_FLIGHT][VEC];
#pragma unroll
    for (int u = 0; u < IN_FLIGHT; ++u) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) v[u][e] = 0.0f;
      if (k0 + u < splits) {
        const float* src = p.partial + (int64_t)(k0 + u) * MN + i;
        if (VEC == 4 && full) {
          const float4 f = *reinterpret_cast<const float4*>(src);
          v[u][0] = f.x;
          v[u][VEC > 1 ? 1 : 0] = VEC > 1 ? f.y : v[u][0];
          v[u][VEC > 2 ? 2 : 0] = VEC > 2 ? f.z : v[u][0];
          v[u][VEC > 3 ? 3 : 0] = VEC > 3 ? f.w : v[u][0];
        } else {
#pragma unroll
          for (int e = 0; e < VEC; ++e)
            if (i + e < MN) v[u][e] = src[e];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < IN_FLIGHT; ++u)
      if (k0 + u < splits)
#pragma unroll
        for (int e = 0; e < VEC; ++e) s[e] += v[u][e];
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    const int64_t idx = i + e;
    if (idx >= MN) break;
    const int64_t row = idx / p.N, col = idx - row * p.N;
    p.C[row * p.ldc + col] = __builtin_bit_cast(uint16_t, (__bf16)s[e]);
  }
}

// Products with at most 16 rows (decode at small batch): the weight is
// streamed once and every output needs all of K, so one workgroup of
// kSkinnyWaves waves owns 16 output columns over the whole of K.  Its waves
// take the K-blocks in turn (wave w: w, w + W, ...), skinny_depth K-blocks in
// flight: the weight's 16 rows of each K-block go straight to the wave's own
// LDS slot as two 8-row, full-line segments (the large kernels' swizzled
// layout), the activation fragments straight into registers; the wave then
// multiplies the 16-column weight fragment by the 16-row activation fragment
// per K-block.  The per-wave sums are added in wave order through LDS (the
// staging slots again) and rounded to bf16.  No split of K across
// workgroups, so no fp32 partials and no second kernel.  Against loading the
// weight fragment into registers (16 rows of 64 bytes per instruction, half
// of each line), at three K-blocks per wave: 1x7168x18432 26.5 against 28.9
// us, 4x36864x7168 54.2 against 57.9, 8x1536x7168 7.0 against 8.3.  Fewer
// K-blocks per wave then let two workgroups share a CU (64 KB of LDS or less
// and at most 92 registers, against 123 at three): one K-block per wave
// 1x18432x7168 29.5 -> 24.1 us, 4x36864x7168 54.1 -> 43.9, 32x7168x2048
// 10.0 -> 8.0, 8x1536x7168 7.0 -> 6.5; with ue8m0 scales and one activation
// fragment two K-blocks per wave are faster still (1x18432x7168 25.6 against
// 27.9 us at one, 33.0 at three; 4x36864x7168 46.6 against 49.3).  8 or 12
// waves per workgroup were no better; nontemporal loads of the weight
// measured 8% slower.
constexpr int kSkinnyWaves = 16;
constexpr int skinny_depth(bool pow2, int frags) { return pow2 && frags == 1 ? 2 : 1; }
constexpr int kSkinnyRows = 16;
// 17 to 32 rows take the two-fragment form where it measured faster than the
// one-launch small-product kernel and the tiled kernels:
// * 2048 < N <= 8192 (32x7168x2048 8.0 against 9.6 us, 32x4096x7168 12.9
//   against 13.7, 17x2100x1040 with ue8m0 scales 3.5 against 7.1);
// * N and K at most 2048: every wave takes one K-block, one pass, no split
//   (17x1000x1040 3.3 against 6.9 us, 32x2048x2048 5.6 against 8.0,
//   32x256x2048 4.9 against 6.9);
// * 16384 <= N < 32768 with K > 2048, where the tiled kernel has fewer
//   64x128 tiles than CUs (32x18432x7168 46.3 against 54.9 us, 24x16384x4096
//   20.9 against 32.3; with K = 2048 the tiled kernel stays faster,
//   32x30000x2048 19.0 against 23.4).
// Not below N = 2048 with longer K (32x1536x7168 12.3 against 9.0 us: too few
// workgroups to stream the weight) nor from N = 32768 (32x36864x7168 83
// against 63 us: every 16-column workgroup re-reads all activation rows).
inline bool skinny_two_fragment(int64_t N, int64_t K) {
  return (N > 2048 && N <= 8192) || (N <= 2048 && K <= 2048) || (N >= 16384 && N < 32768 && K > 2048);
}

// 32 bytes of one operand row for a lane: two 16-byte chunks; a chunk at or
// past K (K is a multiple of 16 here) or of a row outside the matrix reads as
// zero.
__device__ __forceinline__ v8i skinny_frag(const uint8_t* row, bool valid, int64_t k, int64_t K) {
  u32x4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
  if (valid && k < K) lo = *reinterpret_cast<const u32x4*>(row + k);
  if (valid && k + 16 < K) hi = *reinterpret_cast<const u32x4*>(row + k + 16);
  v8i f;
  f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
  f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
  return f;
}

// FRAGS 16-row activation fragments (up to 16 * FRAGS rows): each wave
// multiplies its weight fragment by every activation fragment of a K-block.
constexpr int kSkinnySlot = 16 * BK;  // one K-block of the 16 weight rows

template <bool POW2, int FRAGS>
__global__ __launch_bounds__(64 * kSkinnyWaves) void skinny_gemm_kernel(GemmArgs p) {
  constexpr int kSkinnyDepth = skinny_depth(POW2, FRAGS);
  constexpr int kSkinnyLds = kSkinnyWaves * kSkinnyDepth * kSkinnySlot;
  static_assert(kSkinnyLds >= kSkinnyWaves * FRAGS * 64 * 16, "reduction area within the staging slots");
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSkinnyLds];
  float (*red)[FRAGS][64][4] = reinterpret_cast<float (*)[FRAGS][64][4]>(smem);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int fr = lane & 15, fg = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t K = p.K;
  const int64_t nk = (K + BK - 1) / BK;
  // Column layout (weight fragment first): lane (fr, fg) of fragment f ends
  // with outputs C[16f + fr][n0 + 4fg + v]; it reads weight row n0 + fr from
  // LDS and loads activation rows 16f + fr, bytes 32fg .. 32fg + 31 of each
  // K-block.
  const float* bsr = p.b_s + (n0 / BK) * p.ldbs;
  // The workgroup's weight rows under one descriptor (rows past N read as
  // zero); lane -> LDS chunk lane % 8 of row 8h + lane / 8, which holds
  // logical chunk dc[h] of that row.
  const int64_t nrows = p.N - n0 < 16 ? p.N - n0 : 16;
  const i32x4 rsb = make_rsrc(p.B + n0 * p.ldb, (uint32_t)((nrows - 1) * p.ldb + K));
  const uint32_t lds0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr(smem));
  const int dr = lane >> 3;
  const uint32_t dc[2] = {(uint32_t)((lane & 7) ^ swz_key(dr)), (uint32_t)((lane & 7) ^ swz_key(dr + 8))};
  bool av[FRAGS];
  const uint8_t* arow[FRAGS];
  const float* asr[FRAGS];
#pragma unroll
  for (int f = 0; f < FRAGS; ++f) {
    const int r = 16 * f + fr;
    av[f] = r < p.M;
    arow[f] = p.A + (av[f] ? r : 0) * p.lda;
    asr[f] = p.a_s + (av[f] ? r : 0) * p.as_rs;
  }
  v4f acc[FRAGS];
#pragma unroll
  for (int f = 0; f < FRAGS; ++f) acc[f] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  for (int64_t kb0 = wave; kb0 < nk; kb0 += (int64_t)kSkinnyWaves * kSkinnyDepth) {
    v8i bf[kSkinnyDepth], af[kSkinnyDepth][FRAGS];
    float sa[kSkinnyDepth][FRAGS], sb[kSkinnyDepth];
    // The previous pass's fragment reads from these slots have completed:
    // their MFMAs have consumed them.
#pragma unroll
    for (int d = 0; d < kSkinnyDepth; ++d) {
      const int64_t kb = kb0 + (int64_t)d * kSkinnyWaves;
      if (kb >= nk) break;
      const uint32_t slot = lds0 + (uint32_t)((wave * kSkinnyDepth + d) * kSkinnySlot);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t kk = (uint32_t)kb * BK + 16 * dc[h];
        const bool ok = 8 * h + dr < nrows && kk < (uint32_t)K;
        dma_b128(rsb, slot + (uint32_t)(h * 1024), ok ? (uint32_t)(8 * h + dr) * (uint32_t)p.ldb + kk : kOob, 0);
      }
    }
#pragma unroll
    for (int d = 0; d < kSkinnyDepth; ++d) {
      const int64_t kb = kb0 + (int64_t)d * kSkinnyWaves;
      const bool live = kb < nk;
      const int64_t k = kb * BK + 32 * fg;
#pragma unroll
      for (int f = 0; f < FRAGS; ++f) {
        af[d][f] = skinny_frag(arow[f], av[f] && live, k, K);
        sa[d][f] = live && av[f] ? asr[f][kb * p.as_ks] : 0.0f;
      }
      sb[d] = live ? bsr[kb] : 0.0f;
    }
    // this wave's own slots: its own loads complete (vmcnt 0) is enough
    wait_vmcnt<0>();
#pragma unroll
    for (int d = 0; d < kSkinnyDepth; ++d)
      if (kb0 + (int64_t)d * kSkinnyWaves < nk) bf[d] = read_frag(smem + (wave * kSkinnyDepth + d) * kSkinnySlot, fr, fg);
#pragma unroll
    for (int d = 0; d < kSkinnyDepth; ++d) {
      if (kb0 + (int64_t)d * kSkinnyWaves >= nk) break;
#pragma unroll
      for (int f = 0; f < FRAGS; ++f) {
        if constexpr (POW2) {
          // a row past M carries scale 0 here, which the MFMA reads as 2^-127
          // times a zero fragment: still zero
          acc[f] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[d], af[d][f], acc[f], 0, 0, 0,
                                                                    (int)(__float_as_uint(sb[d]) >> 23), 0,
                                                                    (int)(__float_as_uint(sa[d][f]) >> 23));
        } else {
          const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
          const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[d], af[d][f], z, 0, 0, 0, 0, 0, 0);
          const float sc = sa[d][f] * sb[d];
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[f][v] = __builtin_fmaf(part[v], sc, acc[f][v]);
        }
      }
    }
  }
  __syncthreads();  // every wave is done with its staging slots
#pragma unroll
  for (int f = 0; f < FRAGS; ++f)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave][f][lane][v] = acc[f][v];
  __syncthreads();
  // Thread t < 256 * FRAGS finishes output (row t / 16, column t % 16).
  const int t = threadIdx.x;
  if (t >= kSkinnyRows * FRAGS * 16) return;
  const int r = t >> 4, c = t & 15;
  const int f = r >> 4, l = (c >> 2) * 16 + (r & 15), v = c & 3;
  float sum = 0.0f;
#pragma unroll
  for (int w = 0; w < kSkinnyWaves; ++w) sum += red[w][f][l][v];
  if (r < p.M && n0 + c < p.N) p.C[(int64_t)r * p.ldc + n0 + c] = __builtin_bit_cast(uint16_t, (__bf16)sum);
}

// ---- small products in one launch ------------------------------------------------
//
// Products with few output tiles (decode rows, the ragged shape) are bound by
// latency, not by bandwidth or the matrix cores.  gemm_rd_kernel gives each
// workgroup of W waves (kRdWaves in every launch) one 16FM x 16FN output tile
// and a range of K-blocks; wave w takes the range's K-blocks w, w + W, ... (at
// most DEPTH of them) and issues all of their operand loads at once, so a
// workgroup needs one memory round trip.  The loads go straight to LDS, each
// wave into its own slots (one per K-block: the tile's A rows, then its B
// rows, 128 bytes each in the swizzled layout of the large kernels), as full
// 128-byte rows: 8 rows per 16-byte-per-lane instruction, or 2 rows per
// 4-byte-per-lane instruction when the rows are only 8-byte aligned.  Loading
// the MFMA operands straight into registers instead (16 rows of 64 bytes per
// instruction, half of every 128-byte line) took 13-16% longer on the decode
// shapes.  Each K-block's partial product is rescaled into fp32 accumulators
// as in the large kernels (the weight fragment is the MFMA's first operand,
// so a lane's four results are four columns of one row and share one
// activation scale); the waves' sums are then added in wave order through
// LDS (reusing the staging area).  When a tile's K-blocks are split over
// several workgroups, each writes its fp32 sum to the workspace and
// increments the tile's arrival counter; the workgroup that arrives last adds
// all the sums in split order (the result does not depend on which one that
// is) and stores bf16, then clears the counter for the next call.  One
// launch, deterministic.  All accesses go through buffer resources: a lane
// with nothing to load (a row past the matrix, bytes past K) passes an offset
// past the resource's end and reads zero.

constexpr int kRdWaves = 8;

struct RdPlan {
  int32_t tiles_m, tiles_n, splits, per;  // per: K-blocks per split
  int32_t nkb;
  uint32_t a_bytes, b_bytes, as_bytes;    // extents of A, B and the activation scales
  int32_t* counters;                      // [tiles], zero between calls (splits > 1)
  float* partials;                        // [splits][tiles][16FM * 16FN] (splits > 1)
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rd_buffer(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}

// LDS bytes of the one-launch kernel: the staging slots, or the reduction
// area that reuses them, whichever is larger.
constexpr int rd_lds_bytes(int fm, int fn, int depth, int waves) {
  const int stage = waves * depth * 16 * (fm + fn) * BK;
  const int red = waves * fm * fn * 64 * 16;
  return stage > red ? stage : red;
}
constexpr int kRdMaxLds = 128 * 1024;

// The split hand-off of both one-launch kernels.  Wave `wave` holds the sums
// of subtiles wave, wave + W, ... (OWN of them, those below SUB) for its
// lanes.  Every workgroup of a split product stores them to its split's block
// of the workspace and counts its arrival at the tile's counter; the last to
// arrive replaces them with the sum over all splits, in split order, and
// returns true (it stores the tile); the others return false.  The sums, the
// counter and the final reads are device-scope atomic accesses, which the
// hardware keeps coherent across the XCDs' separate L2 caches without writing
// back or invalidating them (a device-scope fence would do both, for the
// whole cache, in every workgroup).  The stores are complete (vmcnt 0)
// before the workgroup's arrival counts.  The final reads are issued
// kRdBatch splits at a time, all before the first is added.
template <int SUB, int OWN, int W>
__device__ __forceinline__ bool rd_split_sum(const RdPlan& q, int tile, int split, int wave, int lane, int64_t elems,
                                             v4f (&sum)[OWN], int& last) {
  constexpr int kRdBatch = 8;
  const int64_t split_elems = (int64_t)q.tiles_m * q.tiles_n * elems;
#pragma unroll
  for (int o = 0; o < OWN; ++o) {
    const int t = wave + o * W;
    if (t < SUB) {
      float* mine = q.partials + split * split_elems + (((int64_t)tile * SUB + t) * 64 + lane) * 4;
#pragma unroll
      for (int v = 0; v < 4; ++v) __hip_atomic_store(mine + v, sum[o][v], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  wait_vmcnt<0>();
  __syncthreads();
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(q.counters + tile, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == q.splits - 1;
  __syncthreads();
  if (!last) return false;
#pragma unroll
  for (int o = 0; o < OWN; ++o) {
    const int t = wave + o * W;
    if (t < SUB) {
      sum[o] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
      const float* src = q.partials + (((int64_t)tile * SUB + t) * 64 + lane) * 4;
      for (int sp0 = 0; sp0 < q.splits; sp0 += kRdBatch) {
        v4f part[kRdBatch];
#pragma unroll
        for (int b = 0; b < kRdBatch; ++b) {
          part[b] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
          if (sp0 + b < q.splits) {
#pragma unroll
            for (int v = 0; v < 4; ++v)
              part[b][v] = __hip_atomic_load(src + (sp0 + b) * split_elems + v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
#pragma unroll
        for (int b = 0; b < kRdBatch; ++b)
          if (sp0 + b < q.splits) sum[o] += part[b];
      }
    }
  }
  if (threadIdx.x == 0) __hip_atomic_store(q.counters + tile, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

template <int FM, int FN, int DEPTH, int W, int VEC, bool POW2>
__global__ __launch_bounds__(64 * W) void gemm_rd_kernel(GemmArgs p, RdPlan q) {
  constexpr int TM = 16 * FM, TN = 16 * FN, ELEMS = TM * TN, SUB = FM * FN;
  constexpr int ROWS = TM + TN, SLOT = ROWS * BK;
  constexpr int OWN = (SUB + W - 1) / W;  // subtiles each wave finishes
  static_assert(128 % TN == 0, "a tile's columns in one 128-column weight block");
  static_assert(SUB <= W || SUB % W == 0, "subtiles shared evenly by the waves");
  static_assert(rd_lds_bytes(FM, FN, DEPTH, W) <= kRdMaxLds, "LDS");
  __shared__ __attribute__((aligned(16))) uint8_t smem[rd_lds_bytes(FM, FN, DEPTH, W)];
  __shared__ int last;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int fr = lane & 15, fg = lane >> 4;
  const int tiles = q.tiles_m * q.tiles_n;
  const int tile = (int)(blockIdx.x % (unsigned)tiles), split = (int)(blockIdx.x / (unsigned)tiles);
  const int tm = tile % q.tiles_m, tn = tile / q.tiles_m;
  const uint32_t M = (uint32_t)p.M, N = (uint32_t)p.N, K = (uint32_t)p.K;
  const uint32_t m0 = (uint32_t)tm * TM, n0 = (uint32_t)tn * TN;
  const int kb_lo = split * q.per, kb_hi = kb_lo + q.per < q.nkb ? kb_lo + q.per : q.nkb;
  const float* bsrow = p.b_s + (int64_t)(n0 / BK) * p.ldbs;

  // the scales first (branch-free buffer loads: 0 for rows past M and
  // K-blocks past the range), then the operands
  float sa[DEPTH][FM], sb[DEPTH];
  const auto rsa = rd_buffer(p.a_s, q.as_bytes);
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    const int kb = kb_lo + wave + d * W;
    const bool live = kb < kb_hi;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const uint32_t m = m0 + 16 * i + fr;
      sa[d][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          rsa, (live && m < M) ? (m * (uint32_t)p.as_rs + (uint32_t)kb * (uint32_t)p.as_ks) * 4 : kOob, 0, 0));
    }
    sb[d] = live ? bsrow[kb] : 0.0f;
  }
  const i32x4 ra = make_rsrc(p.A, q.a_bytes), rb = make_rsrc(p.B, q.b_bytes);
  const uint32_t lds0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr(smem));
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    const int kb = kb_lo + wave + d * W;
    if (kb >= kb_hi) break;
    const uint32_t slot = lds0 + (uint32_t)((wave * DEPTH + d) * SLOT), kbyte = (uint32_t)kb * BK;
    if constexpr (VEC == 16) {
      // instruction s: tile rows 8s .. 8s + 7 (all of A or all of B, TM being
      // a multiple of 16); lane -> LDS chunk lane % 8 of row 8s + lane / 8
#pragma unroll
      for (int s = 0; s < ROWS / 8; ++s) {
        const int r = 8 * s + (lane >> 3);
        const uint32_t c = (uint32_t)((lane & 7) ^ swz_key(r)), kk = kbyte + 16 * c;
        const bool isa = 8 * s < TM;
        const uint32_t g = isa ? m0 + (uint32_t)r : n0 + (uint32_t)(r - TM);
        const bool ok = (isa ? g < M : g < N) && kk < K;
        dma_b128(isa ? ra : rb, slot + (uint32_t)(s * 1024), ok ? g * (uint32_t)(isa ? p.lda : p.ldb) + kk : kOob, 0);
      }
    } else {
      static_assert(VEC == 8, "16- or 8-byte aligned rows");
      // instruction s: tile rows 2s, 2s + 1; lane -> dword lane % 32 of row
      // 2s + lane / 32 (K a multiple of 8: a dword is wholly before or past K)
#pragma unroll
      for (int s = 0; s < ROWS / 2; ++s) {
        const int r = 2 * s + (lane >> 5), dw = lane & 31;
        const uint32_t c = (uint32_t)((dw >> 2) ^ swz_key(r)), kk = kbyte + 16 * c + 4 * (uint32_t)(dw & 3);
        const bool isa = 2 * s < TM;
        const uint32_t g = isa ? m0 + (uint32_t)r : n0 + (uint32_t)(r - TM);
        const bool ok = (isa ? g < M : g < N) && kk < K;
        dma_b32(isa ? ra : rb, slot + (uint32_t)(s * 256), ok ? g * (uint32_t)(isa ? p.lda : p.ldb) + kk : kOob, 0);
      }
    }
  }
  v4f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  wait_vmcnt<0>();
  __syncthreads();
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    if (kb_lo + wave + d * W >= kb_hi) break;
    const uint8_t* sl = smem + (wave * DEPTH + d) * SLOT;
    v8i bf[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) bf[j] = read_frag(sl, TM + 16 * j + fr, fg);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const v8i af = read_frag(sl, 16 * i + fr, fg);
      if constexpr (POW2) {
        // a row past M carries scale 0 (2^-127) times a zero fragment
        const int ea = (int)(__float_as_uint(sa[d][i]) >> 23), eb = (int)(__float_as_uint(sb[d]) >> 23);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af, acc[i][j], 0, 0, 0, eb, 0, ea);
      } else {
        const float sc = sa[d][i] * sb[d];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af, v4f{0.0f, 0.0f, 0.0f, 0.0f},
                                                                            0, 0, 0, 0, 0, 0);
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[i][j][v] = __builtin_fmaf(part[v], sc, acc[i][j][v]);
        }
      }
    }
  }
  // Reduction area [wave][subtile][lane] over the staging slots: wait until
  // every wave has read its fragments.
  __syncthreads();
  v4f* red = reinterpret_cast<v4f*>(smem);
#pragma unroll
  for (int t = 0; t < SUB; ++t) red[(wave * SUB + t) * 64 + lane] = acc[t / FN][t % FN];
  __syncthreads();
  // Wave w finishes subtiles w, w + W, ... (t = FN i + j): the waves'
  // sums of its four outputs per lane (row 16i + fr, columns 16j + 4fg .. +3)
  // added in wave order, each lane reading 16 consecutive bytes.
  v4f sum[OWN];
#pragma unroll
  for (int o = 0; o < OWN; ++o) {
    const int t = wave + o * W;
    sum[o] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    if (t < SUB) {
      sum[o] = red[t * 64 + lane];
#pragma unroll
      for (int w = 1; w < W; ++w) sum[o] += red[(w * SUB + t) * 64 + lane];
    }
  }
  if (q.splits > 1 && !rd_split_sum<SUB, OWN, W>(q, tile, split, wave, lane, ELEMS, sum, last)) return;
#pragma unroll
  for (int o = 0; o < OWN; ++o) {
    const int t = wave + o * W;
    if (t >= SUB) continue;
    const uint32_t row = m0 + 16 * (t / FN) + fr, col = n0 + 16 * (t % FN) + 4 * fg;
    if (row < M) {
      uint16_t* dst = p.C + (int64_t)row * p.ldc + col;
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (col + v < N) dst[v] = __builtin_bit_cast(uint16_t, (__bf16)sum[o][v]);
    }
  }
}

// Register-staged form of the one-launch kernel: each wave loads the MFMA
// operands of up to kRdrDepth K-blocks straight into registers (16 rows of 64
// bytes per instruction), so its LDS holds only the reduction area (64 KB at
// 64x32 tiles) and two workgroups share a CU.  Used where the LDS-staged
// form, at one workgroup per CU, would need more than one round of
// workgroups or more K splits (64x4096x7168: 20.6 against 27.1 us;
// 48x2048x7168 with ue8m0 scales: 13.2 against 16.4 us).
constexpr int kRdrDepth = 2;

// 32 bytes of one operand row for a lane (bytes k .. k + 31 of the row at
// byte offset `row`, or kOob for a row to skip); VEC-byte pieces at or past K
// read as zero (VEC divides K).
template <int VEC>
__device__ __forceinline__ v8i rd_frag(__amdgpu_buffer_rsrc_t r, uint32_t row, uint32_t k, uint32_t K) {
  v8i f;
  if constexpr (VEC == 16) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t kk = k + 16 * h;
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (row != kOob && kk < K) ? row + kk : kOob, 0, 0);
      f[4 * h] = v.x; f[4 * h + 1] = v.y; f[4 * h + 2] = v.z; f[4 * h + 3] = v.w;
    }
  } else {
    static_assert(VEC == 8, "8- or 16-byte pieces");
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const uint32_t kk = k + 8 * h;
      const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (row != kOob && kk < K) ? row + kk : kOob, 0, 0);
      f[2 * h] = v.x; f[2 * h + 1] = v.y;
    }
  }
  return f;
}

template <int FM, int FN, int VEC, bool POW2>
__global__ __launch_bounds__(64 * kRdWaves) void gemm_rdr_kernel(GemmArgs p, RdPlan q) {
  constexpr int TM = 16 * FM, TN = 16 * FN, ELEMS = TM * TN;
  static_assert(FM * FN <= kRdWaves && 128 % TN == 0, "a wave per subtile; a tile's columns in one 128-block");
  __shared__ v4f red[kRdWaves][FM * FN][64];
  __shared__ int last;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int fr = lane & 15, fg = lane >> 4;
  const int tiles = q.tiles_m * q.tiles_n;
  const int tile = (int)(blockIdx.x % (unsigned)tiles), split = (int)(blockIdx.x / (unsigned)tiles);
  const int tm = tile % q.tiles_m, tn = tile / q.tiles_m;
  const uint32_t M = (uint32_t)p.M, N = (uint32_t)p.N, K = (uint32_t)p.K;
  const uint32_t m0 = (uint32_t)tm * TM, n0 = (uint32_t)tn * TN;
  const int kb_lo = split * q.per, kb_hi = kb_lo + q.per < q.nkb ? kb_lo + q.per : q.nkb;
  const auto ra = rd_buffer(p.A, q.a_bytes);
  const auto rb = rd_buffer(p.B, q.b_bytes);
  const float* bsrow = p.b_s + (int64_t)(n0 / BK) * p.ldbs;

  v8i bf[kRdrDepth][FN], af[kRdrDepth][FM];
  float sa[kRdrDepth][FM], sb[kRdrDepth];
  // the scales first (branch-free buffer loads: 0 for rows past M and
  // K-blocks past the range), then the operands
  const auto rsa = rd_buffer(p.a_s, q.as_bytes);
#pragma unroll
  for (int d = 0; d < kRdrDepth; ++d) {
    const int kb = kb_lo + wave + d * kRdWaves;
    const bool live = kb < kb_hi;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const uint32_t m = m0 + 16 * i + fr;
      sa[d][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          rsa, (live && m < M) ? (m * (uint32_t)p.as_rs + (uint32_t)kb * (uint32_t)p.as_ks) * 4 : kOob, 0, 0));
    }
    sb[d] = live ? bsrow[kb] : 0.0f;
  }
#pragma unroll
  for (int d = 0; d < kRdrDepth; ++d) {
    const int kb = kb_lo + wave + d * kRdWaves;
    const bool live = kb < kb_hi;
    const uint32_t k = (uint32_t)kb * BK + 32 * fg;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const uint32_t n = n0 + 16 * j + fr;
      bf[d][j] = rd_frag<VEC>(rb, (live && n < N) ? n * (uint32_t)p.ldb : kOob, k, K);
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const uint32_t m = m0 + 16 * i + fr;
      af[d][i] = rd_frag<VEC>(ra, (live && m < M) ? m * (uint32_t)p.lda : kOob, k, K);
    }
  }
  v4f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int d = 0; d < kRdrDepth; ++d) {
    if (kb_lo + wave + d * kRdWaves >= kb_hi) break;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if constexpr (POW2) {
        // a row past M carries scale 0 (2^-127) times a zero fragment
        const int ea = (int)(__float_as_uint(sa[d][i]) >> 23), eb = (int)(__float_as_uint(sb[d]) >> 23);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[d][j], af[d][i], acc[i][j], 0, 0, 0, eb, 0, ea);
      } else {
        const float sc = sa[d][i] * sb[d];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[d][j], af[d][i],
                                                                            v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0, 0, 0, 0);
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[i][j][v] = __builtin_fmaf(part[v], sc, acc[i][j][v]);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) red[wave][i * FN + j][lane] = acc[i][j];
  __syncthreads();
  // Wave w < FM*FN finishes subtile w = (i, j): the waves' sums of its four
  // outputs per lane (row 16i + fr, columns 16j + 4fg .. +3) added in wave
  // order, each lane reading 16 consecutive bytes (no bank conflicts).
  const bool owner = wave < FM * FN;
  const int si = wave / FN, sj = wave % FN;
  v4f sum[1] = {v4f{0.0f, 0.0f, 0.0f, 0.0f}};
  if (owner) {
    sum[0] = red[0][wave][lane];
#pragma unroll
    for (int w = 1; w < kRdWaves; ++w) sum[0] += red[w][wave][lane];
  }
  if (q.splits > 1 && !rd_split_sum<FM * FN, 1, kRdWaves>(q, tile, split, wave, lane, ELEMS, sum, last)) return;
  if (!owner) return;
  const uint32_t row = m0 + 16 * si + fr, col = n0 + 16 * sj + 4 * fg;
  if (row < M) {
    uint16_t* dst = p.C + (int64_t)row * p.ldc + col;
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (col + v < N) dst[v] = __builtin_bit_cast(uint16_t, (__bf16)sum[0][v]);
  }
}

// Expert row range [lo, hi) with every bound clamped into [0, M_total].
__device__ __forceinline__ void expert_rows(const int32_t* offsets, int64_t e, int64_t M, int64_t& lo, int64_t& hi) {
  int64_t a = offsets[e], b = offsets[e + 1];
  a = a < 0 ? 0 : (a > M ? M : a);
  b = b < a ? a : (b > M ? M : b);
  lo = a;
  hi = b;
}

// Tile classes of the grouped product.  With one class, every expert's rows
// run in tiles of height h[0].  With three (heights h0 < h1 < h2), an expert
// with at most h0 rows is class 0's and one with at most h1 rows class 1's;
// a larger expert runs whole h2-row tiles in class 2, and a remainder of at
// most h1 rows after its last whole tile goes to the class of that height
// instead of padding one more h2-row tile (a larger remainder takes the
// padded h2 tile).  class_rows gives the rows [lo, hi), relative to the
// expert's first row, that class c computes for an expert of n rows.
constexpr int kMaxClasses = 3;
__device__ __forceinline__ void class_rows(int64_t n, int c, int classes, const int (&h)[3], int64_t& lo,
                                           int64_t& hi) {
  lo = hi = 0;
  if (classes == 1) {
    if (c == 0) hi = n;
    return;
  }
  int64_t split = 0;  // class 2 computes [0, split), class rc computes [split, n)
  int rc = -1;
  if (n <= h[0]) {
    rc = 0;
  } else if (n <= h[1]) {
    rc = 1;
  } else {
    const int64_t full = n / h[2], rem = n - full * h[2];
    if (full > 0 && rem > 0 && rem <= h[1]) {
      split = full * h[2];
      rc = rem <= h[0] ? 0 : 1;
    } else {
      split = n;
    }
  }
  if (c == 2) {
    hi = split;
  } else if (c == rc) {
    lo = split;
    hi = n;
  }
}

// tile_start[c * (E + 1) + e] = number of class-c row tiles of the experts
// before e.  One workgroup of 16 waves takes 1024 experts per step and all
// classes at once: an inclusive scan inside each wave (lane shuffles), the
// 16 wave totals through LDS, and a running carry per class across steps.
__global__ __launch_bounds__(1024) void tile_schedule_kernel(GemmArgs p) {
  constexpr int kWaves = 1024 / 64;
  const int32_t* offsets = p.offsets;
  const int64_t E = p.E, M = p.M;
  const int C = p.grp_classes;
  int32_t* tile_start = p.tile_start;
  __shared__ int32_t wsum[kMaxClasses][kWaves];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int32_t carry[kMaxClasses] = {0, 0, 0};
  if (t < C) tile_start[(int64_t)t * (E + 1)] = 0;
  for (int64_t base = 0; base < E; base += 1024) {
    const int64_t e = base + t;
    int32_t v[kMaxClasses] = {0, 0, 0};
    if (e < E) {
      int64_t lo, hi;
      expert_rows(offsets, e, M, lo, hi);
#pragma unroll
      for (int c = 0; c < kMaxClasses; ++c) {
        if (c < C) {
          int64_t a, b;
          class_rows(hi - lo, c, C, p.grp_h, a, b);
          v[c] = (int32_t)((b - a + p.grp_h[c] - 1) / p.grp_h[c]);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < kMaxClasses; ++c) {
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int32_t y = __shfl_up(v[c], d, 64);
        if (lane >= d) v[c] += y;
      }
      if (lane == 63) wsum[c][w] = v[c];
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kMaxClasses; ++c) {
      int32_t before = carry[c];
#pragma unroll
      for (int i = 0; i < kWaves; ++i) {
        const int32_t s = wsum[c][i];
        before += i < w ? s : 0;
        carry[c] += s;
      }
      if (c < C && e < E) tile_start[(int64_t)c * (E + 1) + e + 1] = before + v[c];
    }
    __syncthreads();  // wsum is rewritten by the next step
  }
}

// The last expert e in [0, E) with ts[e] <= slot, for ts non-decreasing and
// ts[0] <= slot < ts[E].  UNIFORM (slot the same in every lane of the wave):
// each round the wave's 64 lanes test 64 evenly spaced candidates at once and
// a ballot keeps the bracket between the last one at or below slot and the
// next, so up to 4096 experts take two rounds of loads where a bisection
// takes twelve dependent ones.  Otherwise each lane bisects on its own.
template <bool UNIFORM>
__device__ __forceinline__ int64_t find_expert(const int32_t* ts, int64_t E, int64_t slot) {
  int64_t lo = 0, hi = E;  // invariant: ts[lo] <= slot < ts[hi]
  if constexpr (UNIFORM) {
    const int lane = lane_id();
    while (hi - lo > 1) {
      const int64_t step = (hi - lo + 63) / 64;
      const int64_t i = lo + (int64_t)lane * step;
      const bool ok = i < hi && ts[i] <= slot;  // true on a prefix of the lanes, lane 0 included
      const uint64_t m = __ballot(ok);
      const int64_t nlo = lo + (int64_t)(63 - __builtin_clzll(m)) * step;
      hi = nlo + step < hi ? nlo + step : hi;
      lo = nlo;
    }
  } else {
    while (hi - lo > 1) {
      const int64_t mid = (lo + hi) >> 1;
      if (ts[mid] <= slot) lo = mid;
      else hi = mid;
    }
  }
  return lo;
}

// One row tile x column tile of a grouped product: expert e, rows
// [row0, row_end) of A and C (at most the class's tile height), column tile tn.
struct GroupedSlot {
  int64_t e, row0, row_end, tn;
};

// One workgroup per (row tile of an expert, column tile).  The grid is sized
// for the worst case; the real number of row tiles is ts[E].  Ids past the
// real work exit at once; the rest are renumbered XCD-contiguously over the
// real work, expert by expert, so the concurrent tiles of an XCD share the
// expert's activation rows and weight panels in its L2.  pid is the
// workgroup's index within its launch range, which starts at a multiple of 8
// (so pid % 8 is still its XCD).
//
// The tile of workgroup pid of class p.grp_class (p.tile_start is that
// class's schedule, tile height BM).  class_tiles: the class's row-tile count
// ts[E] when the caller has loaded it already (negative: load it here).
// False for ids past the class's tiles.
template <int BM, bool UNIFORM>
__device__ __forceinline__ bool grouped_slot(const GemmArgs& p, int64_t pid, int64_t tiles_n, int64_t class_tiles,
                                             GroupedSlot& out) {
  const int32_t* ts = p.tile_start;
  const int64_t total = (class_tiles >= 0 ? class_tiles : (int64_t)ts[p.E]) * tiles_n;
  if (pid >= total) return false;
  const int64_t L = xcd_contiguous(pid, total);
  const int64_t slot0 = div_u(L, tiles_n);
  const int64_t e = find_expert<UNIFORM>(ts, p.E, slot0);
  // Expert e's row tiles x column tiles are one contiguous id range; inside
  // it the ids run in groups of up to kGroupM row tiles, row tile fastest,
  // so the concurrent tiles of a large expert share each weight panel as
  // well as each activation panel in L2 (as the dense product's groups do).
  const int64_t rt = ts[e + 1] - ts[e];
  const int64_t l = L - (int64_t)ts[e] * tiles_n;
  const int64_t per_group = (int64_t)kGroupM * tiles_n;
  const int64_t g0 = div_u(l, per_group) * kGroupM;
  const int64_t gsize = rt - g0 < kGroupM ? rt - g0 : kGroupM;
  const int64_t in = l - g0 * tiles_n;
  const int64_t tn = div_u(in, gsize);
  const int64_t slot = ts[e] + g0 + (in - tn * gsize);
  int64_t r0, r1;
  expert_rows(p.offsets, e, p.M, r0, r1);
  int64_t clo, chi;
  class_rows(r1 - r0, p.grp_class, p.grp_classes, p.grp_h, clo, chi);
  out.e = e;
  out.row0 = r0 + clo + (slot - ts[e]) * BM;
  out.row_end = r0 + chi;
  out.tn = tn;
  return true;
}

template <class CF, int VEC, bool GLU>
__device__ __forceinline__ void grouped_run(const GemmArgs& p, const GroupedSlot& g, uint8_t* smem) {
  const int64_t kbn = (p.N + BK - 1) / BK;
  TileRef t;
  t.A = p.A;
  t.a_s = p.a_s;
  t.B = p.B + g.e * p.N * p.ldb;
  t.b_s = p.b_s + g.e * kbn * p.ldbs;
  t.row0 = g.row0;
  t.row_end = g.row_end;
  t.n0 = g.tn * kColStep<CF, GLU>;
  t.kb0 = 0;
  t.kb1 = (int)((p.K + BK - 1) / BK);
  t.partial = nullptr;
  run_tile<CF, VEC, GLU>(p, t, smem);
}

template <class CF, int VEC, bool GLU = false>
__global__ __launch_bounds__(CF::kThreads) void grouped_gemm_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[CF::LDS_BYTES];
  GroupedSlot g;
  if (grouped_slot<CF::BM, true>(p, blockIdx.x, col_tiles<CF, GLU>(p), -1, g)) grouped_run<CF, VEC, GLU>(p, g, smem);
}

// The three tile classes of a grouped product in one launch.  Workgroup ids
// go in chunks of 8 (one per XCD, so a class's local id keeps the XCD of the
// workgroup and grouped_slot's XCD-contiguous ranges hold).  From the tile
// counts the schedule kernel wrote, chunk q belongs to class 2 (the 256-row
// tiles, compute-bound) at evenly spread positions over the first `pct`
// percent of the chunks, and the other chunks to class 1 (128-row tiles),
// then class 0 (64-row tiles), both bound by streaming their experts'
// weights: the longer tiles go first, so the launch ends with the shortest
// (routed-expert down-projection −0.5% against interleaving the two).  The
// CUs run tall and short tiles at once, so the weight stream of the small
// experts overlaps the products of the large ones.  Chunks past the last tile
// have no class.  p.tile_start holds the class-0 schedule;
// class c's is c*(E+1) later.  Returns the class (-1: none) and the id within
// the class.
__device__ __forceinline__ int merged_class(const GemmArgs& p, int64_t bid, int64_t tiles_n, int64_t pct,
                                            const int64_t (&tc)[3], int64_t& pid) {
  auto chunks_of = [&](int64_t t) __attribute__((always_inline)) { return (t * tiles_n + kXcds - 1) / kXcds; };
  const int64_t c0 = chunks_of(tc[0]), c1 = chunks_of(tc[1]), c2 = chunks_of(tc[2]);
  const int64_t C = c0 + c1 + c2;
  const int64_t q = bid / kXcds, x = bid % kXcds;
  if (q >= C) return -1;
  int64_t span = C * pct / 100;
  if (span < c2) span = c2;
  if (span < 1) span = 1;
  int c;
  int64_t local;
  const int64_t b2 = q < span ? div_u((q + 1) * c2, span) : c2;  // class-2 chunks at positions <= q
  if (q < span && b2 > div_u(q * c2, span)) {
    c = 2;
    local = b2 - 1;
  } else {
    const int64_t r = q - b2;  // rank among the other chunks
    if (r < c1) {
      c = 1;
      local = r;
    } else {
      c = 0;
      local = r - c1;
    }
  }
  pid = local * kXcds + x;
  return c;
}

// The tile of merged-launch workgroup bid (false: none).
template <class C0, class C1, class C2, bool GLU, bool UNIFORM>
__device__ __forceinline__ bool merged_slot(const GemmArgs& p, int64_t bid, int64_t pct, int& c, GroupedSlot& g) {
  const int64_t tiles_n = col_tiles<C2, GLU>(p);
  const int64_t tc[3] = {p.tile_start[p.E], p.tile_start[(p.E + 1) + p.E], p.tile_start[2 * (p.E + 1) + p.E]};
  int64_t pid;
  c = merged_class(p, bid, tiles_n, pct, tc, pid);
  if (c < 0) return false;
  GemmArgs a = p;
  a.grp_class = c;
  a.tile_start = p.tile_start + c * (p.E + 1);
  if (c == 2) return grouped_slot<C2::BM, UNIFORM>(a, pid, tiles_n, tc[2], g);
  if (c == 1) return grouped_slot<C1::BM, UNIFORM>(a, pid, tiles_n, tc[1], g);
  return grouped_slot<C0::BM, UNIFORM>(a, pid, tiles_n, tc[0], g);
}

// The merged launch's tile of every workgroup id, computed ahead of it by one
// thread per id: int4 {expert (-1: no tile), first row, row end, column tile
// * 4 + class}.  A workgroup of the merged launch then finds its tile with one
// 16-byte load instead of the dependent loads of the class totals, the
// expert search and the expert's rows, which delay every tile's first weight
// load by about 2 us (13% of a 64-row tile of the routed-expert
// down-projection).
template <class C0, class C1, class C2, bool GLU>
__global__ __launch_bounds__(256) void tile_plan_kernel(GemmArgs p, int64_t pct, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  int c = -1;
  GroupedSlot g;
  int4 v = make_int4(-1, 0, 0, 0);
  if (merged_slot<C0, C1, C2, GLU, false>(p, i, pct, c, g))
    v = make_int4((int)g.e, (int)g.row0, (int)g.row_end, (int)(g.tn * 4 + c));
  reinterpret_cast<int4*>(p.tile_plan)[i] = v;
}

// All three classes use 8 waves, 256-column tiles and one workgroup per CU
// (their LDS rings take 125 to 149 KB), so sharing one kernel costs no
// occupancy.  With p.tile_plan each workgroup reads its tile from the plan;
// without it (a caller without room for the plan) it maps its id itself.
template <class C0, class C1, class C2, int VEC, bool GLU>
__global__ __launch_bounds__(C2::kThreads) void grouped_merged_kernel(GemmArgs p, int64_t pct) {
  static_assert(C0::kThreads == C2::kThreads && C1::kThreads == C2::kThreads, "one workgroup size");
  static_assert(C0::BN == C2::BN && C1::BN == C2::BN, "one column tiling");
  constexpr int L01 = C0::LDS_BYTES > C1::LDS_BYTES ? C0::LDS_BYTES : C1::LDS_BYTES;
  constexpr int LDS = L01 > C2::LDS_BYTES ? L01 : C2::LDS_BYTES;
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS];
  int c;
  GroupedSlot g;
  if (p.tile_plan != nullptr) {
    const int4 v = reinterpret_cast<const int4*>(p.tile_plan)[blockIdx.x];
    if (v.x < 0) return;
    g.e = v.x;
    g.row0 = v.y;
    g.row_end = v.z;
    g.tn = v.w >> 2;
    c = v.w & 3;
  } else if (!merged_slot<C0, C1, C2, GLU, true>(p, blockIdx.x, pct, c, g)) {
    return;
  }
  if (c == 2) grouped_run<C2, VEC, GLU>(p, g, smem);
  else if (c == 1) grouped_run<C1, VEC, GLU>(p, g, smem);
  else grouped_run<C0, VEC, GLU>(p, g, smem);
}

inline bool aligned(const void* q, size_t n) { return (reinterpret_cast<uintptr_t>(q) % n) == 0; }

// Load width for the operands: 0 (K % 128 == 0) or -1 selects the
// direct-to-LDS pipeline, which needs 16-byte aligned rows, K % 16 == 0,
// 32-bit tile offsets and a 32-bit K-block step of the activation scales;
// otherwise the widest aligned width for the register-staged pipeline.
template <class CF>
int pick_vec(const GemmArgs& a) {
  if (a.K % 16 == 0 && a.lda % 16 == 0 && a.ldb % 16 == 0 && aligned(a.A, 16) && aligned(a.B, 16) &&
      (int64_t)CF::BM * a.lda < ((int64_t)1 << 31) && (int64_t)CF::BN * a.ldb < ((int64_t)1 << 31) &&
      a.as_ks < ((int64_t)1 << 29))
    return a.K % BK == 0 ? 0 : -1;
  const int cands[3] = {16, 8, 4};
  for (int v : cands)
    if (a.K % v == 0 && a.lda % v == 0 && a.ldb % v == 0 && aligned(a.A, v) && aligned(a.B, v)) return v;
  return 1;
}

#define DSFP8_LAUNCH(KERN, CF, VEC, GRID) hipLaunchKernelGGL((KERN<CF, VEC>), GRID, dim3(CF::kThreads), 0, s, a)
// A direct-to-LDS launch, its variant chosen from K and the scale format.
#define DSFP8_LAUNCH_DMA(KERN, CF, GLU, GRID, STREAM, ARGS)                                          \
  do {                                                                                              \
    const bool kfull_ = (ARGS).K % BK == 0;                                                         \
    if ((ARGS).pow2) {                                                                              \
      if (kfull_) hipLaunchKernelGGL((KERN<CF, -2, GLU>), GRID, dim3(CF::kThreads), 0, STREAM, ARGS); \
      else hipLaunchKernelGGL((KERN<CF, -3, GLU>), GRID, dim3(CF::kThreads), 0, STREAM, ARGS);        \
    } else {                                                                                        \
      if (kfull_) hipLaunchKernelGGL((KERN<CF, 0, GLU>), GRID, dim3(CF::kThreads), 0, STREAM, ARGS);  \
      else hipLaunchKernelGGL((KERN<CF, -1, GLU>), GRID, dim3(CF::kThreads), 0, STREAM, ARGS);        \
    }                                                                                               \
  } while (0)

template <class CFD, class CFG, bool GROUPED>
hipError_t dispatch(const GemmArgs& a, dim3 gd, dim3 gg, hipStream_t s) {
  switch (pick_vec<CFD>(a)) {
    case 0:
    case -1:
      if constexpr (GROUPED) DSFP8_LAUNCH_DMA(grouped_gemm_kernel, CFD, false, gd, s, a);
      else DSFP8_LAUNCH_DMA(gemm_kernel, CFD, false, gd, s, a);
      break;
    case 16:
      if constexpr (GROUPED) DSFP8_LAUNCH(grouped_gemm_kernel, CFG, 16, gg);
      else DSFP8_LAUNCH(gemm_kernel, CFG, 16, gg);
      break;
    case 8:
      if constexpr (GROUPED) DSFP8_LAUNCH(grouped_gemm_kernel, CFG, 8, gg);
      else DSFP8_LAUNCH(gemm_kernel, CFG, 8, gg);
      break;
    case 4:
      if constexpr (GROUPED) DSFP8_LAUNCH(grouped_gemm_kernel, CFG, 4, gg);
      else DSFP8_LAUNCH(gemm_kernel, CFG, 4, gg);
      break;
    default:
      if constexpr (GROUPED) DSFP8_LAUNCH(grouped_gemm_kernel, CFG, 1, gg);
      else DSFP8_LAUNCH(gemm_kernel, CFG, 1, gg);
      break;
  }
  return hipGetLastError();
}

template <class CF>
dim3 dense_grid(const GemmArgs& a) {
  return dim3((unsigned)(((a.M + CF::BM - 1) / CF::BM) * ((a.N + CF::BN - 1) / CF::BN)));
}

template <class CF>
dim3 grouped_grid(const GemmArgs& a) {
  const int64_t slots = (a.M + CF::BM - 1) / CF::BM + a.E;  // bound on the row tiles
  return dim3((unsigned)(slots * ((a.N + CF::BN - 1) / CF::BN)));
}

}  // namespace

int gemm_k_splits(int64_t M, int64_t N, int64_t K) {
  const int64_t nkb = (K + BK - 1) / BK;
  const int64_t tiles = ((M + CfgDma::BM - 1) / CfgDma::BM) * ((N + CfgDma::BN - 1) / CfgDma::BN);
  constexpr int64_t kTargetWorkgroups = 512;  // two per CU on a 256-CU part
  if (M == 0 || N == 0 || nkb < 4 || tiles * 4 >= kTargetWorkgroups) return 1;
  int64_t splits = (kTargetWorkgroups + tiles - 1) / tiles;
  if (splits > nkb / 2) splits = nkb / 2;  // at least two K-blocks per split
  if (splits < 2) return 1;
  const int64_t per = (nkb + splits - 1) / splits;
  return (int)((nkb + per - 1) / per);     // no empty split
}

// Tile shape, K split and form of the one-launch small-product kernel.
// 32-row tiles for at most 32 rows, else 64.  The LDS-staged form takes the
// first of these that fits in one round of workgroups (one per CU) with at
// most 4 K splits: for 32-row tiles 64 then 32 columns, for 64-row tiles 32
// then 64 columns; each wave takes one K-block, or two where their staging
// fits in LDS and the range needs more than one workgroup (fewer splits:
// decode 32x1536x7168 9.9 against 11.2 us).  Otherwise the register-staged
// form: 64 columns for 32-row tiles unless that leaves fewer than 256
// workgroups, else 32, two K-blocks per wave when K is split.  Measured
// (graph of launches, weights rotated): decode 32x1536x7168 8.8 us
// (register-staged 10.0), ragged 333x2500x1000 with 64x64 tiles 9.0 us
// (64x32 tiles: 11.5; register-staged 10.2), 100x1024x4096 10.5 us (12.2).
struct RdShape {
  int fm, fn, depth;
  bool regs;  // register-staged form
  int64_t tiles_m, tiles_n, splits, per, nkb;
};

RdShape rd_shape(int64_t M, int64_t N, int64_t K) {
  RdShape r{};
  r.nkb = (K + BK - 1) / BK;
  r.fm = M <= 32 ? 2 : 4;
  // one round of workgroups at one per CU on a 256-CU part (a constant, so
  // that the workspace size does not depend on the device)
  constexpr int64_t kRound = 256;
  auto make = [&](int fn, bool regs) {
    r.fn = fn;
    r.regs = regs;
    r.depth = 1;
    r.tiles_m = (M + 16 * r.fm - 1) / (16 * r.fm);
    r.tiles_n = (N + 16 * fn - 1) / (16 * fn);
    r.per = kRdWaves;
    r.splits = (r.nkb + r.per - 1) / r.per;
    if (r.splits > 1 && (regs || rd_lds_bytes(r.fm, fn, 2, kRdWaves) <= kRdMaxLds)) {
      r.depth = 2;
      r.per = 2 * kRdWaves;
      r.splits = (r.nkb + r.per - 1) / r.per;
    }
    return r.tiles_m * r.tiles_n * r.splits;
  };
  const int first = r.fm == 2 ? 4 : 2, second = 6 - first;
  for (int fn : {first, second})
    if (make(fn, false) <= kRound && r.splits <= 4) return r;
  if (make(r.fm == 4 ? 2 : 4, true) < kRound && r.fm == 2) make(2, true);
  return r;
}

// Workspace of a split product: the one-launch kernel's arrival counters
// (one int per tile, 256-byte aligned area) first, then the fp32 partial
// sums of whichever split form runs.
size_t rd_counter_bytes(int64_t M, int64_t N, int64_t K) {
  const RdShape r = rd_shape(M, N, K);
  return ((size_t)(r.tiles_m * r.tiles_n) * sizeof(int32_t) + 255) & ~(size_t)255;
}

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const int s = gemm_k_splits(M, N, K);
  if (s <= 1) return 0;
  const RdShape r = rd_shape(M, N, K);
  const size_t rd = r.splits > 1 ? (size_t)(r.splits * r.tiles_m * r.tiles_n) * 256 * r.fm * r.fn * sizeof(float) : 0;
  const size_t old = (size_t)s * (size_t)M * (size_t)N * sizeof(float);
  return rd_counter_bytes(M, N, K) + (rd > old ? rd : old);
}

// The one-launch kernel needs 8-byte pieces of A and B rows (K, lda, ldb
// multiples of 8, 8-byte aligned operands) and 32-bit offsets; returns the
// piece width (16 or 8), or 0 if it does not apply.
int rd_vec(const GemmArgs& a) {
  const int64_t lim = (int64_t)1 << 31;
  if ((a.M - 1) * a.lda + a.K >= lim || (a.N - 1) * a.ldb + a.K >= lim) return 0;
  if (((a.M - 1) * a.as_rs + ((a.K + BK - 1) / BK - 1) * a.as_ks + 1) * 4 >= lim) return 0;
  if (a.K % 16 == 0 && a.lda % 16 == 0 && a.ldb % 16 == 0 && aligned(a.A, 16) && aligned(a.B, 16)) return 16;
  if (a.K % 8 == 0 && a.lda % 8 == 0 && a.ldb % 8 == 0 && aligned(a.A, 8) && aligned(a.B, 8)) return 8;
  return 0;
}

template <int FM, int FN, int DEPTH>
hipError_t launch_rd(const GemmArgs& a, const RdPlan& q, int vec, dim3 grid, hipStream_t stream) {
  constexpr int W = kRdWaves;
  const dim3 blk(64 * W);
  if (vec == 16) {
    if (a.pow2) hipLaunchKernelGGL((gemm_rd_kernel<FM, FN, DEPTH, W, 16, true>), grid, blk, 0, stream, a, q);
    else hipLaunchKernelGGL((gemm_rd_kernel<FM, FN, DEPTH, W, 16, false>), grid, blk, 0, stream, a, q);
  } else {
    if (a.pow2) hipLaunchKernelGGL((gemm_rd_kernel<FM, FN, DEPTH, W, 8, true>), grid, blk, 0, stream, a, q);
    else hipLaunchKernelGGL((gemm_rd_kernel<FM, FN, DEPTH, W, 8, false>), grid, blk, 0, stream, a, q);
  }
  return hipGetLastError();
}

template <int FM, int FN>
hipError_t launch_rdr(const GemmArgs& a, const RdPlan& q, int vec, dim3 grid, hipStream_t stream) {
  const dim3 blk(64 * kRdWaves);
  if (vec == 16) {
    if (a.pow2) hipLaunchKernelGGL((gemm_rdr_kernel<FM, FN, 16, true>), grid, blk, 0, stream, a, q);
    else hipLaunchKernelGGL((gemm_rdr_kernel<FM, FN, 16, false>), grid, blk, 0, stream, a, q);
  } else {
    if (a.pow2) hipLaunchKernelGGL((gemm_rdr_kernel<FM, FN, 8, true>), grid, blk, 0, stream, a, q);
    else hipLaunchKernelGGL((gemm_rdr_kernel<FM, FN, 8, false>), grid, blk, 0, stream, a, q);
  }
  return hipGetLastError();
}

// The skinny kernel loads 16-byte chunks of A and B rows.  Measured against
// the tiled kernels it is faster up to 16 rows (1 x 18432 x 7168: 24 vs 52 us;
// 16 x 7168 x 2048: 6.0 vs 12.1 us); from 17 to 32 rows see
// skinny_two_fragment.
bool skinny_ok(const GemmArgs& a) {
  const bool rows = a.M <= kSkinnyRows || (a.M <= 2 * kSkinnyRows && skinny_two_fragment(a.N, a.K));
  // a workgroup's 16 weight rows under one descriptor with 32-bit offsets
  const bool span = 15 * a.ldb + a.K < ((int64_t)1 << 31);
  return rows && span && a.K % 16 == 0 && a.lda % 16 == 0 && a.ldb % 16 == 0 && aligned(a.A, 16) && aligned(a.B, 16);
}

// Split K over workgroups for operands the one-launch kernel does not take:
// fp32 partials [splits, M, N] in a.partial, summed in split order by a
// second kernel.
hipError_t launch_gemm_splitk(const GemmArgs& a, int splits, hipStream_t stream) {
  static_assert(CfgDma::BM == Cfg128::BM && CfgDma::BN == Cfg128::BN, "same split grid for both pipelines");
  dim3 g = dense_grid<CfgDma>(a);
  g.y = (unsigned)splits;
  hipError_t err;
  if (a.M <= CfgGrp::BM && pick_vec<CfgGrp>(a) <= 0) {
    // at most 64 rows: the 64-row tiles (same grid, one row tile)
    static_assert(CfgGrp::BN == CfgDma::BN, "same column tiles");
    DSFP8_LAUNCH_DMA(gemm_kernel, CfgGrp, false, g, stream, a);
    err = hipGetLastError();
  } else {
    err = dispatch<CfgDma, Cfg128, false>(a, g, g, stream);
  }
  if (err != hipSuccess) return err;
  if (splits > 8) {
    const int64_t groups = (a.M * a.N + 255) / 256;
    hipLaunchKernelGGL((splitk_reduce_kernel<1, 32>), dim3((unsigned)groups), dim3(256), 0, stream, a, splits);
  } else {
    const int64_t groups = (a.M * a.N + 1023) / 1024;
    hipLaunchKernelGGL((splitk_reduce_kernel<4, 8>), dim3((unsigned)groups), dim3(256), 0, stream, a, splits);
  }
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  if (skinny_ok(a)) {
    const dim3 grid((unsigned)((a.N + 15) / 16)), blk(64 * kSkinnyWaves);
    if (a.M <= kSkinnyRows) {
      if (a.pow2) hipLaunchKernelGGL((skinny_gemm_kernel<true, 1>), grid, blk, 0, stream, a);
      else hipLaunchKernelGGL((skinny_gemm_kernel<false, 1>), grid, blk, 0, stream, a);
    } else {
      if (a.pow2) hipLaunchKernelGGL((skinny_gemm_kernel<true, 2>), grid, blk, 0, stream, a);
      else hipLaunchKernelGGL((skinny_gemm_kernel<false, 2>), grid, blk, 0, stream, a);
    }
    return hipGetLastError();
  }
  const int splits = gemm_k_splits(a.M, a.N, a.K);
  if (splits > 1 && a.partial != nullptr) {
    // the workspace starts with the one-launch kernel's counters
    uint8_t* ws = reinterpret_cast<uint8_t*>(a.partial);
    const size_t cbytes = rd_counter_bytes(a.M, a.N, a.K);
    const int vec = rd_vec(a);
    if (vec > 0) {
      const RdShape r = rd_shape(a.M, a.N, a.K);
      RdPlan q;
      q.tiles_m = (int32_t)r.tiles_m;
      q.tiles_n = (int32_t)r.tiles_n;
      q.splits = (int32_t)r.splits;
      q.per = (int32_t)r.per;
      q.nkb = (int32_t)r.nkb;
      q.a_bytes = (uint32_t)((a.M - 1) * a.lda + a.K);
      q.b_bytes = (uint32_t)((a.N - 1) * a.ldb + a.K);
      q.as_bytes = (uint32_t)(((a.M - 1) * a.as_rs + ((a.K + BK - 1) / BK - 1) * a.as_ks + 1) * 4);
      q.counters = reinterpret_cast<int32_t*>(ws);
      q.partials = reinterpret_cast<float*>(ws + cbytes);
      const dim3 grid((unsigned)(r.tiles_m * r.tiles_n * r.splits));
      if (r.regs) {
        if (r.fm == 2 && r.fn == 4) return launch_rdr<2, 4>(a, q, vec, grid, stream);
        if (r.fm == 2) return launch_rdr<2, 2>(a, q, vec, grid, stream);
        return launch_rdr<4, 2>(a, q, vec, grid, stream);
      }
      if (r.fm == 2 && r.fn == 4) return launch_rd<2, 4, 1>(a, q, vec, grid, stream);
      if (r.fm == 2) return r.depth == 2 ? launch_rd<2, 2, 2>(a, q, vec, grid, stream)
                                         : launch_rd<2, 2, 1>(a, q, vec, grid, stream);
      if (r.fn == 4) return launch_rd<4, 4, 1>(a, q, vec, grid, stream);
      return launch_rd<4, 2, 1>(a, q, vec, grid, stream);
    }
    GemmArgs b = a;
    b.partial = reinterpret_cast<float*>(ws + cbytes);
    return launch_gemm_splitk(b, splits, stream);
  }
  const int64_t big_tiles = ((a.M + CfgDmaBig::BM - 1) / CfgDmaBig::BM) * ((a.N + CfgDmaBig::BN - 1) / CfgDmaBig::BN);
  if (a.M >= CfgDmaBig::BM && big_tiles >= device_cu_count() && pick_vec<CfgDmaBig>(a) <= 0) {
    DSFP8_LAUNCH_DMA(gemm_persistent_kernel, CfgDmaBig, false, dim3((unsigned)device_cu_count()), stream, a);
    return hipGetLastError();
  }
  if (a.M <= CfgGrp::BM && pick_vec<CfgGrp>(a) <= 0) {
    DSFP8_LAUNCH_DMA(gemm_kernel, CfgGrp, false, dense_grid<CfgGrp>(a), stream, a);
    return hipGetLastError();
  }
  return dispatch<CfgDma, Cfg128, false>(a, dense_grid<CfgDma>(a), dense_grid<Cfg128>(a), stream);
}

// Tile heights of the merged grouped launch's three classes.
constexpr int kGrpH0 = 64, kGrpH1 = 128, kGrpH2 = 256;

// Workgroups of a merged grouped launch over E experts, M rows and tn column
// tiles (a bound: the tile counts are on the device).  A non-empty expert has
// at most one tile of class 0 or 1 (its only tile, or the remainder after its
// whole 256-row tiles), so classes 0 and 1 together have at most min(E, M).
// The large class's tiles hold at least 129 rows each on average: a whole
// tile 256, an expert of 129 to 256 rows one tile, and an expert whose
// remainder exceeds 128 rows spreads its rows over whole tiles plus one, at
// more than 128 rows per tile; so it has at most M/129 tiles.  Ids go in
// chunks of 8: each class rounds its tiles up to whole chunks, which classes
// 0 and 1 together take at most one chunk more than their joint bound.  The
// kernel maps chunks to the actual tiles and the rest exit.
int64_t merged_workgroups(int64_t E, int64_t M, int64_t tn) {
  const int64_t s01 = E < M ? E : M;
  const int64_t s2 = M / (kGrpH1 + 1);
  return ((s01 * tn + 7) / 8 + 1 + (s2 * tn + 7) / 8) * 8;
}

// Spread of the 256-row tiles over a grouped launch (percent of its chunks):
// measured on the routed-expert products, mixing them with the small-expert
// tiles made the down-projection (K = 2048) 3.3% faster than running them
// first and the up-projection (K = 7168, long compute-bound tall tiles that
// share weight panels when they run together) 8% slower.  Spreading them over
// the first 80% of the launch instead of all of it, so that the launch ends
// with short tiles only, took another 2.5% off the down-projection (70 to 95%
// measured within 1.5% of each other; 60% and below 2 to 5% slower again).
inline int64_t tall_span_pct(int64_t K) { return K >= 4096 ? 0 : 80; }

// Grouped launches.  With the direct-to-LDS pipeline the rows are split into
// three tile classes (class_rows), each run with its own tile height, so a
// row tile is never padded by more than its own height and a large expert
// streams its weight once per C2::BM rows instead of once per C0::BM.
template <class C0, class C1, class C2, bool GLU>
hipError_t grouped_classes(const GemmArgs& a, hipStream_t stream) {
  static_assert(C0::BM < C1::BM && C1::BM < C2::BM, "increasing tile heights");
  GemmArgs s = a;
  s.grp_classes = 3;
  s.grp_h[0] = C0::BM;
  s.grp_h[1] = C1::BM;
  s.grp_h[2] = C2::BM;
  hipLaunchKernelGGL(tile_schedule_kernel, dim3(1), dim3(1024), 0, stream, s);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  static_assert(C0::BN == C1::BN && C1::BN == C2::BN, "one column tiling");
  static_assert(C0::BM == kGrpH0 && C1::BM == kGrpH1 && C2::BM == kGrpH2, "the heights the grid bound assumes");
  GemmArgs c0 = s;
  c0.grp_class = 0;
  const int64_t n = merged_workgroups(a.E, a.M, GLU ? a.glu_f / BK : (a.N + C2::BN - 1) / C2::BN);
  if (n > INT32_MAX) return hipErrorInvalidConfiguration;  // more workgroups than one launch takes
  const dim3 grid((unsigned)n), blk(C2::kThreads);
  const bool kfull = a.K % BK == 0;
  const int64_t pct = tall_span_pct(a.K);
  if (c0.tile_plan != nullptr) {
    hipLaunchKernelGGL((tile_plan_kernel<C0, C1, C2, GLU>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, c0,
                       pct, n);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (a.pow2) {
    if (kfull) hipLaunchKernelGGL((grouped_merged_kernel<C0, C1, C2, -2, GLU>), grid, blk, 0, stream, c0, pct);
    else hipLaunchKernelGGL((grouped_merged_kernel<C0, C1, C2, -3, GLU>), grid, blk, 0, stream, c0, pct);
  } else {
    if (kfull) hipLaunchKernelGGL((grouped_merged_kernel<C0, C1, C2, 0, GLU>), grid, blk, 0, stream, c0, pct);
    else hipLaunchKernelGGL((grouped_merged_kernel<C0, C1, C2, -1, GLU>), grid, blk, 0, stream, c0, pct);
  }
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(const GemmArgs& a, hipStream_t stream) {
  if (a.N == 0 || a.M == 0) return hipSuccess;
  if (pick_vec<CfgGlu64>(a) <= 0 && pick_vec<CfgGlu128>(a) <= 0 && pick_vec<CfgDmaBig>(a) <= 0)
    return grouped_classes<CfgGlu64, CfgGlu128, CfgDmaBig, false>(a, stream);
  static_assert(CfgDma::BM == Cfg128::BM, "one tile height for both pipelines");
  GemmArgs s = a;
  s.grp_class = 0;
  s.grp_classes = 1;
  s.grp_h[0] = Cfg128::BM;
  hipLaunchKernelGGL(tile_schedule_kernel, dim3(1), dim3(1024), 0, stream, s);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return dispatch<CfgDma, Cfg128, true>(s, grouped_grid<CfgDma>(s), grouped_grid<Cfg128>(s), stream);
}

// ---- gated form ----------------------------------------------------------------

bool gemm_glu_supported(const GemmArgs& a) {
  const int64_t F = a.glu_f;
  if (F <= 0 || F % BK != 0 || a.N != 2 * F) return false;
  if (pick_vec<CfgGlu64>(a) > 0 || pick_vec<CfgGlu128>(a) > 0 || pick_vec<CfgDmaBig>(a) > 0) return false;
  // one descriptor spans w1 row n0 .. w3 row F + n0 + 127 with 32-bit offsets
  if ((F + BK) * a.ldb + a.K >= ((int64_t)1 << 31)) return false;
  if (!aligned(a.qy, 8) || a.ldqy % 8 != 0) return false;
  if (a.qh != nullptr && (!aligned(a.qh, 16) || a.ldqh % 8 != 0)) return false;
  return true;
}

// Column split of a gated product whose 256-row tiles fill the CUs R >= 1
// times with a partial round left over: the persistent kernel takes the
// first n1 output column blocks (exactly R rounds of tiles), and the last
// nt - n1 blocks follow as 64-row tiles (128-row tiles when the 64-row ones
// would not fit in one round of workgroups).  A partial round of 256-row
// tiles takes as long as a full one; the shorter tiles spread the remaining
// weight panels over more CUs.  Every output element goes through the same
// arithmetic in either tile, so the results are bit-identical.  Measured
// (M = 4096, K = 7168, graph of launches): F = 2304 (288 tiles on 256 CUs)
// 177.9 -> 149.8 us, F = 4608 276.9 -> 248.0 us, F = 9216 464.8 -> 455.4 us.
// Returns the tail's tile height, or 0 when the product is not split.
static int glu_tail_height(int64_t M, int64_t nt, int64_t cus, int64_t& n1) {
  n1 = 0;
  const int64_t tm = (M + CfgDmaBig::BM - 1) / CfgDmaBig::BM;
  const int64_t rounds = tm * nt / cus;
  if (M < CfgDmaBig::BM || rounds < 1 || (rounds * cus) % tm != 0) return 0;
  n1 = rounds * cus / tm;
  if (n1 >= nt) return 0;
  const int64_t n2 = nt - n1;
  if (((M + CfgGlu64::BM - 1) / CfgGlu64::BM) * n2 <= cus) return CfgGlu64::BM;
  if (((M + CfgGlu128::BM - 1) / CfgGlu128::BM) * n2 <= cus) return CfgGlu128::BM;
  return 0;
}

hipError_t launch_gemm_glu(const GemmArgs& a, hipStream_t stream) {
  if (a.M == 0) return hipSuccess;
  const int64_t nt = a.glu_f / BK;
  const int64_t cus = device_cu_count();
  auto grid = [&](int bm) { return dim3((unsigned)(((a.M + bm - 1) / bm) * nt)); };
  const int64_t big_tiles = ((a.M + CfgDmaBig::BM - 1) / CfgDmaBig::BM) * nt;
  int64_t n1 = 0;
  const int tail = glu_tail_height(a.M, nt, cus, n1);
  if (tail != 0) {
    GemmArgs head = a;
    head.glu_nt = n1;
    DSFP8_LAUNCH_DMA(gemm_persistent_kernel, CfgDmaBig, true, dim3((unsigned)cus), stream, head);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // the last nt - n1 column blocks: w1 rows from n1 * 128 (w3 rows F
    // further, as before), their scale rows, and the matching output columns
    GemmArgs rest = a;
    const int64_t f1 = n1 * BK;
    rest.B = a.B + f1 * a.ldb;
    rest.b_s = a.b_s + n1 * a.ldbs;
    rest.qy = a.qy + f1;
    rest.qs = a.qs + n1 * a.qs_ks;
    rest.qh = a.qh != nullptr ? a.qh + f1 : nullptr;
    rest.glu_nt = nt - n1;
    const dim3 g((unsigned)(((a.M + tail - 1) / tail) * (nt - n1)));
    if (tail == CfgGlu64::BM) DSFP8_LAUNCH_DMA(gemm_kernel, CfgGlu64, true, g, stream, rest);
    else DSFP8_LAUNCH_DMA(gemm_kernel, CfgGlu128, true, g, stream, rest);
    return hipGetLastError();
  }
  if (a.M >= CfgDmaBig::BM && big_tiles >= cus)
    DSFP8_LAUNCH_DMA(gemm_persistent_kernel, CfgDmaBig, true, dim3((unsigned)cus), stream, a);
  else if (a.M > CfgGlu64::BM)
    DSFP8_LAUNCH_DMA(gemm_kernel, CfgGlu128, true, grid(CfgGlu128::BM), stream, a);
  else
    DSFP8_LAUNCH_DMA(gemm_kernel, CfgGlu64, true, grid(CfgGlu64::BM), stream, a);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm_glu(const GemmArgs& a, hipStream_t stream) {
  if (a.M == 0) return hipSuccess;
  return grouped_classes<CfgGlu64, CfgGlu128, CfgDmaBig, true>(a, stream);
}

size_t grouped_schedule_bytes(int64_t E) {
  const size_t n = (size_t)kMaxClasses * (size_t)(E + 1) * sizeof(int32_t);
  return (n + 255) & ~(size_t)255;
}

size_t grouped_workspace_bytes(int64_t E, int64_t M, int64_t N) {
  // the schedule, then the tile plan: one int4 per workgroup of the merged
  // launch (N / 256 column tiles; the gated form passes N = 2F)
  return grouped_schedule_bytes(E) + (size_t)merged_workgroups(E, M, (N + 255) / 256) * sizeof(int4);
}
}  // namespace dsfp8

// ---- allocation-free grouped product ------------------------------------------
//
// The grouped product's only scratch is the tile schedule (kMaxClasses
// int32 rows of E + 1 entries).  For callers that cannot allocate, it lives
// in this static device array instead of a caller workspace; every GPU the
// library runs on holds its own copy (zero-initialised at load, kept until
// the process ends).  Host code never passes the array's name to a kernel:
// the name is a host-side stand-in, so the device address is looked up once
// per device with hipGetSymbolAddress and that pointer is used instead.
static __device__ __align__(256) int32_t scratch[dsfp8::kMaxClasses * (dsfp8::kNoAllocMaxExperts + 1)];

namespace dsfp8 {

hipError_t noalloc_scratch(int32_t** out) {
  constexpr int kDevices = 64;
  static std::atomic<int32_t*> cache[kDevices];
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kDevices) return hipErrorInvalidDevice;
  int32_t* p = cache[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // Called with device `dev` current; two threads racing here both store
    // the same address.
    void* q = nullptr;
    err = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (q == nullptr) return hipErrorInvalidSymbol;
    p = static_cast<int32_t*>(q);
    cache[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

hipError_t launch_grouped_gemm_noalloc(GemmArgs a, hipStream_t stream) {
  if (a.E > kNoAllocMaxExperts) return hipErrorInvalidValue;  // checked by the caller first
  int32_t* p = nullptr;
  const hipError_t err = noalloc_scratch(&p);
  if (err != hipSuccess) return err;
  a.tile_start = p;
  return launch_grouped_gemm(a, stream);
}

}  // namespace dsfp8
