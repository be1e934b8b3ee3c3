// Projection step of the largest workload: per-tensor e4m3 quantization and an
// FP8 GEMM on the gfx950 matrix cores.
//
// The pages name a fused FP8 matmul in the serving step (page "Runway explains
// how it serves a 57B video model in real time", fourth paragraph) without a
// formula; the reading implemented here is one scale per tensor,
//   s = RN(amax / 448),  code = e4m3(RN(x / s))  (the cache's row rule with the
//   whole tensor as the row),
//   C = bf16( (s_a * s_b) * sum_k dec(A[m,k]) * dec(B[k,n]) ), f32 accumulation.
//
// GEMM decomposition: one workgroup = a 256 x 256 tile of C, 16 waves in a
// 4 (M) x 4 (N) grid, each wave 64 x 64 = 2 x 2 blocks of
// v_mfma_f32_32x32x64_f8f6f4 (four waves per SIMD, so that one wave's
// operand reads and barrier waits overlap the others' products).  The Bt
// block is the MFMA A operand and the A block the B operand, so a lane of
// the result holds four consecutive output columns of one row; the plain
// GEMM passes the tile through LDS as bf16 and writes it in whole rows, 16
// bytes per lane.  K advances 128 bytes per stage
// through two LDS stages (rows padded to 144 B, conflict-free 16-byte reads);
// the global loads of stage t+1 are in flight while stage t is computed.
// Tiles are numbered XCD-aware (each XCD walks a contiguous range) and grouped
// four M-rows at a time so the workgroups resident on one XCD share operands
// in its L2.  With one workgroup per compute unit the tiles run in whole
// rounds; a last round that would fill at most half the device runs as
// 256 x 128 half tiles in a second launch (twice the workgroups, half the
// time).
//
// Fused QKV epilogue (gemm_fp8_kernel<D>, D = head_dim): the output columns
// are [Q heads | K heads | V heads] of one chunk's tokens.  Q columns are
// written as bf16 like the plain GEMM (tiles of Q columns only take the plain
// GEMM's epilogue); K and V heads never reach HBM in bf16:
// from the f32 result (times s_a s_b) the epilogue applies RoPE to K at the
// chunk's positions and quantizes each (token, head) row to e4m3 with the
// cache's row rule, straight into the ring slots of the current chunk (the
// fused FP8 matmul of page "Runway explains how it serves a 57B video model in
// real time", fourth paragraph, with the write-time RoPE and FP8 of the same
// paragraph).  The accumulator tile goes through LDS (f32, 128 tokens at a
// time); then each wave takes 16 RoPE pairs of one head in one 64-token ring
// tile, one lane per token, so a row's RoPE pairs stay in one lane and its
// amax takes one exchange through LDS between the waves of the head; K rows
// are written as 16-byte runs and the transposed V tile as 64-byte rows.
#include "device_common.hpp"
#include "kernels.hpp"

#include <algorithm>
#include <mutex>

namespace rtv {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kBM = 256, kBN = 256, kBK = 128;
constexpr int kGemmWaves = 16;
constexpr int kGemmThreads = kGemmWaves * kWave;
constexpr int kRow = kBK + 16;                       // padded LDS row (bytes)
constexpr int kGroupM = 4;
// A launch of BN-wide tiles (BN = kBN, or kBN / 2 for the tiles of a last,
// partial round): LDS bytes of one stage and 16-byte chunks per thread
template <int BN> constexpr int stage_bytes() { return (kBM + BN) * kRow; }   // 73728 / 55296
template <int BN> constexpr int chunks_per_thread() { return (kBM + BN) * (kBK / 16) / kGemmThreads; }

constexpr int kQuantThreads = 256;

__device__ __forceinline__ v16f mfma_fp8(const v8i& a, const v8i& b, const v16f& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// ---- per-tensor quantization ------------------------------------------------

// largest |x| over bf16 values, as bits: for non-NaN bf16 the order of
// (bits & 0x7FFF) is the order of |x|
__device__ __forceinline__ uint32_t mag_max8(uint4 w) {
  uint32_t m = 0;
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m = max(m, ws[i] & 0x7FFFu);
    m = max(m, (ws[i] >> 16) & 0x7FFFu);
  }
  return m;
}

__device__ __forceinline__ uint32_t block_max(uint32_t m, uint32_t* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) red[w] = m;
  __syncthreads();
  m = 0;
#pragma unroll
  for (int i = 0; i < kQuantThreads / kWave; ++i) m = max(m, red[i]);
  return m;
}

__global__ void __launch_bounds__(kQuantThreads)
quant_amax_kernel(const uint16_t* __restrict__ x, int64_t n, uint32_t* __restrict__ partial) {
  __shared__ uint32_t red[kQuantThreads / kWave];
  const int64_t n8 = n >> 3;
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  uint32_t m = 0;
  const int64_t stride = (int64_t)gridDim.x * kQuantThreads;
  for (int64_t i = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x; i < n8; i += stride)
    m = max(m, mag_max8(xv[i]));
  if (blockIdx.x == 0)
    for (int64_t i = (n8 << 3) + threadIdx.x; i < n; i += kQuantThreads) m = max(m, x[i] & 0x7FFFu);
  m = block_max(m, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

__device__ __forceinline__ uint32_t quant_one(float x, const RowQuant& q) {
  const uint32_t sign = (__float_as_uint(x) >> 31) << 7;
  if (q.s == 0.0f) return sign;
  return (cvt_fp8x2<false>(quant_mag(x, q), 0.0f, 0u) & 0xFFu) | sign;
}

__global__ void __launch_bounds__(kQuantThreads)
quant_apply_kernel(const uint16_t* __restrict__ x, int64_t n, const uint32_t* __restrict__ partial,
                   int n_partial, uint8_t* __restrict__ codes, float* __restrict__ scale) {
  __shared__ uint32_t red[kQuantThreads / kWave];
  uint32_t m = 0;
  for (int i = threadIdx.x; i < n_partial; i += kQuantThreads) m = max(m, partial[i]);
  m = block_max(m, red);
  const float amax = __uint_as_float(m << 16);
  const RowQuant q = row_quant(amax);
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale = q.s;
  const int64_t n8 = n >> 3;
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  uint2* cv = reinterpret_cast<uint2*>(codes);
  const int64_t stride = (int64_t)gridDim.x * kQuantThreads;
  if (fast_amax(amax)) {
    // the short form of the quantization (same codes; the scale q.s equals
    // scale448(amax) in this range)
    const float fs = scale448(amax);
    const float fr = 1.0f / fs;
    for (int64_t i = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x; i < n8; i += stride) {
      const uint4 w = xv[i];
      uint2 o;
      o.x = quant4_fast(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y), fs, fr);
      o.y = quant4_fast(bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w), fs, fr);
      cv[i] = o;
    }
  } else {
    for (int64_t i = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x; i < n8; i += stride) {
      const uint4 w = xv[i];
      uint2 o;
      o.x = quant4(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y), q);
      o.y = quant4(bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w), q);
      cv[i] = o;
    }
  }
  if (blockIdx.x == 0)
    for (int64_t i = (n8 << 3) + threadIdx.x; i < n; i += kQuantThreads)
      codes[i] = (uint8_t)quant_one(__uint_as_float((uint32_t)x[i] << 16), q);
}

// ---- GEMM -------------------------------------------------------------------

struct GemmArgs {
  const uint8_t* a;    // [M][K]
  const uint8_t* bt;   // [N][K]
  const float* sa;
  const float* sb;
  uint16_t* c;         // [M][ldc] bf16
  int64_t ldc;
  int32_t M, N, K;
  int32_t n_mt, n_nt, n_tiles;
  int32_t tile_base;   // first logical tile of the launch
  int32_t n_launch;    // work items of the launch (tiles, or half tiles)
  int32_t vec_store;   // 16-byte stores allowed (c 16-aligned, ldc % 8 == 0)
  // fused QKV epilogue: columns [0, q_cols) are Q (bf16 into c), then
  // n_kv_heads K heads and n_kv_heads V heads of D columns into the ring
  int32_t q_cols;
  int32_t n_kv_heads;
  const float* rope;   // (cos, sin) pairs of the chunk's first position: [M][D/2][2]
  uint8_t* kc;         // layer ring, as for the append
  uint8_t* vc;
  float* ks;
  float* vs;
  int64_t slots_padded;
  int64_t write_slot;  // first slot of the chunk, a multiple of 64
};

// global -> register loads of one stage: chunk c of 16 bytes, rows [0, 256)
// of A then of Bt, 8 chunks per row; rows past M / N repeat the last row and
// k past K reads zeros
template <int BN>
struct StageRegs {
  uint4 r[chunks_per_thread<BN>()];
};

template <int BN>
__device__ __forceinline__ void load_stage(StageRegs<BN>& s, const GemmArgs& g, int m0, int n0, int k0) {
#pragma unroll
  for (int j = 0; j < chunks_per_thread<BN>(); ++j) {
    const int c = threadIdx.x + j * kGemmThreads;
    const int row = c >> 3;                 // 0..511
    const int col = (c & 7) * 16;
    const bool is_a = row < kBM;
    const int r = is_a ? min(m0 + row, g.M - 1) : min(n0 + row - kBM, g.N - 1);
    const uint8_t* base = is_a ? g.a : g.bt;
    if (k0 + col < g.K)
      s.r[j] = *reinterpret_cast<const uint4*>(base + (int64_t)r * g.K + k0 + col);
    else
      s.r[j] = make_uint4(0, 0, 0, 0);
  }
}

template <int BN>
__device__ __forceinline__ void store_stage(const StageRegs<BN>& s, uint8_t* st) {
#pragma unroll
  for (int j = 0; j < chunks_per_thread<BN>(); ++j) {
    const int c = threadIdx.x + j * kGemmThreads;
    *reinterpret_cast<uint4*>(st + (c >> 3) * kRow + (c & 7) * 16) = s.r[j];
  }
}

// 32-row operand fragment at k-substep ks: lane (i, hh) reads row i, bytes
// [64 ks + 32 hh, +32) (A and B use the same byte-to-k assignment)
__device__ __forceinline__ v8i frag(const uint8_t* st, int row0, int ks, int lane) {
  const uint8_t* p = st + (row0 + (lane & 31)) * kRow + ks * 64 + (lane >> 5) * 32;
  const uint4 lo = *reinterpret_cast<const uint4*>(p);
  const uint4 hi = *reinterpret_cast<const uint4*>(p + 16);
  v8i v;
  v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
  v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
  return v;
}

// bytes per token row of the f32 tile in LDS, and the per-row amax exchange after it
template <int BN> constexpr int epi_row() { return BN * 4 + 16; }
template <int BN> constexpr int epi_amax() { return 128 * epi_row<BN>(); }

// Fused epilogue of one 256 x BN tile (see the file comment).  acc[i][j]
// (i < 2) holds D[n][m] for m = m0+wm+32i + lane%32 and n = n0+wn+32j +
// 8(r/4) + 4(lane/32) + r%4; tokens m >= M are skipped.
template <int D, int BN, typename Acc>
__device__ __forceinline__ void fused_epilogue(const GemmArgs& g, const Acc& acc, float s, uint8_t* smem,
                                               int m0, int n0, int wm, int wn, int wave, int lane) {
  constexpr int HALF = D / 2;
  constexpr int PAIRS = 16;                      // RoPE pairs per lane
  constexpr int PARTS = HALF / PAIRS;            // waves per head
  constexpr int kEpiRow = epi_row<BN>();
  const int hh = lane >> 5;
  float* amax_x = reinterpret_cast<float*>(smem + epi_amax<BN>());
  const int kv_cols = g.n_kv_heads * D;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    __syncthreads();                             // LDS free: operands or the previous half consumed
    // (1) tokens 64 half + [0, 64) and 128 + 64 half + [0, 64) of the tile ->
    // rows [0, 64) and [64, 128): the waves whose 64 rows they are (wm = 64
    // half or 128 + 64 half) write their accumulators
    const int wblk = wm / 64;
    if ((wblk & 1) == half) {
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const int row = (wblk >> 1) * 64 + ii * 32 + (lane & 31);
#pragma unroll
        for (int j = 0; j < BN / 128; ++j)
#pragma unroll
          for (int grp4 = 0; grp4 < 4; ++grp4) {
            const int n = wn + 32 * j + 8 * grp4 + 4 * hh;
            const auto& a4 = acc[ii][j];
            *reinterpret_cast<float4*>(smem + row * kEpiRow + n * 4) =
                make_float4(a4[4 * grp4] * s, a4[4 * grp4 + 1] * s, a4[4 * grp4 + 2] * s, a4[4 * grp4 + 3] * s);
          }
      }
    }
    __syncthreads();
    // (2) wave -> (ring tile t, head of the tile, part of PAIRS RoPE pairs);
    // lane -> token.  (In a BN = 128 tile the waves of the heads outside it
    // only take part in the barriers.)
    const int t = wave / (kGemmWaves / 2);
    const int hp = wave % (kGemmWaves / 2);
    const int head_local = hp / PARTS;
    const int part = hp % PARTS;
    const int m = m0 + 128 * t + 64 * half + lane;
    const bool valid = m < g.M;
    const int col = n0 + head_local * D;         // first column of the head (uniform)
    const bool in_tile = head_local * D < BN;
    const float* erow =
        reinterpret_cast<const float*>(smem + (64 * t + lane) * kEpiRow) + (in_tile ? head_local : 0) * D;
    float x0[PAIRS], x1[PAIRS];
#pragma unroll
    for (int q = 0; q < PAIRS; q += 4) {
      const float4 a = *reinterpret_cast<const float4*>(erow + PAIRS * part + q);
      const float4 b = *reinterpret_cast<const float4*>(erow + HALF + PAIRS * part + q);
      x0[q] = a.x; x0[q + 1] = a.y; x0[q + 2] = a.z; x0[q + 3] = a.w;
      x1[q] = b.x; x1[q + 1] = b.y; x1[q + 2] = b.z; x1[q + 3] = b.w;
    }
    const bool is_q = col < g.q_cols;
    const bool is_k = !is_q && col < g.q_cols + kv_cols;
    const bool in_range = col < g.N && in_tile;
    if (is_k) {
      // RoPE at position (chunk start) + m, rounded as in the append
      const float* cs = g.rope + (int64_t)(valid ? m : 0) * D + 2 * PAIRS * part;
#pragma unroll
      for (int q = 0; q < PAIRS; q += 2) {
        const float4 c = *reinterpret_cast<const float4*>(cs + 2 * q);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float co = e ? c.z : c.x;
          const float si = e ? c.w : c.y;
          const float a0 = x0[q + e] * co;
          const float b0 = x1[q + e] * si;
          const float a1 = x1[q + e] * co;
          const float b1 = x0[q + e] * si;
          x0[q + e] = a0 - b0;
          x1[q + e] = a1 + b1;
        }
      }
    }
    float amax = 0.0f;
#pragma unroll
    for (int q = 0; q < PAIRS; ++q) amax = fmaxf(amax, fmaxf(fabsf(x0[q]), fabsf(x1[q])));
    // the row's amax over the PARTS waves of its head
    amax_x[wave * 64 + lane] = amax;
    __syncthreads();
#pragma unroll
    for (int p = 0; p < PARTS; ++p) amax = fmaxf(amax, amax_x[(wave - part + p) * 64 + lane]);
    // rows with a normal scale take the short form of the quantization (one
    // uniform choice per wave, taken before the lanes of other rows leave)
    const bool fast = __all(!valid || !in_range || fast_amax(amax));
    if (!valid || !in_range) continue;
    if (is_q) {
      uint16_t* dst = g.c + (int64_t)m * g.ldc + col + PAIRS * part;
#pragma unroll
      for (int q = 0; q < PAIRS; q += 8) {
        uint4 w0, w1;
        w0.x = pack_bf16x2(x0[q], x0[q + 1]); w0.y = pack_bf16x2(x0[q + 2], x0[q + 3]);
        w0.z = pack_bf16x2(x0[q + 4], x0[q + 5]); w0.w = pack_bf16x2(x0[q + 6], x0[q + 7]);
        w1.x = pack_bf16x2(x1[q], x1[q + 1]); w1.y = pack_bf16x2(x1[q + 2], x1[q + 3]);
        w1.z = pack_bf16x2(x1[q + 4], x1[q + 5]); w1.w = pack_bf16x2(x1[q + 6], x1[q + 7]);
        *reinterpret_cast<uint4*>(dst + q) = w0;
        *reinterpret_cast<uint4*>(dst + HALF + q) = w1;
      }
      continue;
    }
    uint32_t c0[PAIRS / 4], c1[PAIRS / 4];
    const float row_s = quant_row<PAIRS>(x0, x1, c0, c1, amax, fast);
    const int64_t slot = g.write_slot + m;
    if (is_k) {
      const int h = (col - g.q_cols) / D;
      uint8_t* dst = g.kc + ((int64_t)h * g.slots_padded + slot) * D + PAIRS * part;
      *reinterpret_cast<uint4*>(dst) = make_uint4(c0[0], c0[1], c0[2], c0[3]);
      *reinterpret_cast<uint4*>(dst + HALF) = make_uint4(c1[0], c1[1], c1[2], c1[3]);
      if (part == 0) g.ks[(int64_t)h * g.slots_padded + slot] = row_s;
    } else {
      // transposed V tile: byte vt_pos(slot % 64) of row d; the wave's 64
      // lanes fill one 64-byte row per d
      const int h = (col - g.q_cols - kv_cols) / D;
      uint8_t* vt = g.vc + (((int64_t)h * (g.slots_padded / kTileKeys) + slot / kTileKeys) * D) * kTileKeys +
                    vt_pos_of_key((int)(slot % kTileKeys));
#pragma unroll
      for (int q = 0; q < PAIRS; ++q) {
        vt[(int64_t)(PAIRS * part + q) * kTileKeys] = (uint8_t)(c0[q >> 2] >> (8 * (q & 3)));
        vt[(int64_t)(HALF + PAIRS * part + q) * kTileKeys] = (uint8_t)(c1[q >> 2] >> (8 * (q & 3)));
      }
      if (part == 0) g.vs[(int64_t)h * g.slots_padded + slot] = row_s;
    }
  }
}

// BN = kBN: work item = logical tile tile_base + item.  BN = kBN / 2: the
// tiles of a last, partial round as two halves each (item = 2 x tile +
// half), so that twice as many workgroups share that round's work.
template <int FUSED_D, int BN>
__global__ void __launch_bounds__(kGemmThreads, 1) gemm_fp8_kernel(GemmArgs g) {
  static_assert(BN == kBN || 2 * BN == kBN, "full or half tiles");
  constexpr int NJ = BN / 128;              // 32-column blocks per wave
  constexpr int kStageBytes = stage_bytes<BN>();
  extern __shared__ __align__(16) uint8_t smem[];
  const int item = xcd_remap(blockIdx.x, g.n_launch);
  if (item < 0) return;
  const int logical = g.tile_base + (BN == kBN ? item : item >> 1);
  // group kGroupM tile rows: consecutive logical tiles walk down a column of
  // the group first
  const int group_size = kGroupM * g.n_nt;
  const int grp = logical / group_size;
  const int first_m = grp * kGroupM;
  const int gm = min(g.n_mt - first_m, kGroupM);
  const int in_grp = logical - grp * group_size;
  const int mt = first_m + in_grp % gm;
  const int nt = in_grp / gm;
  const int m0 = mt * kBM, n0 = nt * kBN + (BN == kBN ? 0 : (item & 1) * BN);

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int wm = (wave & 3) * 64;       // wave's M offset in the tile
  const int wn = (wave >> 2) * (BN / 4);  // wave's N offset in the tile

  v16f acc[2][NJ];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int n_k = (g.K + kBK - 1) / kBK;
  StageRegs<BN> regs;
  load_stage<BN>(regs, g, m0, n0, 0);
  store_stage(regs, smem);
  __syncthreads();
  for (int t = 0; t < n_k; ++t) {
    const bool more = t + 1 < n_k;
    if (more) load_stage<BN>(regs, g, m0, n0, (t + 1) * kBK);
    const uint8_t* st = smem + (t & 1) * kStageBytes;
    const uint8_t* sa = st;                 // A rows
    const uint8_t* sbt = st + kBM * kRow;   // Bt rows
#pragma unroll
    for (int ks = 0; ks < kBK / 64; ++ks) {
      v8i bop[NJ], aop[2];
#pragma unroll
      for (int j = 0; j < NJ; ++j) bop[j] = frag(sbt, wn + 32 * j, ks, lane);
#pragma unroll
      for (int i = 0; i < 2; ++i) aop[i] = frag(sa, wm + 32 * i, ks, lane);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = mfma_fp8(bop[j], aop[i], acc[i][j]);
    }
    if (more) store_stage(regs, smem + ((t + 1) & 1) * kStageBytes);
    __syncthreads();
  }

  // epilogue: acc[i][j] holds D[n][m] for m = m0+wm+32i + lane%32 and
  // n = n0+wn+32j + 8(r/4) + 4(lane/32) + r%4
  const float s = (*g.sa) * (*g.sb);
  if constexpr (FUSED_D > 0) {
    // tiles with K or V columns take the fused epilogue; tiles of Q columns
    // only are plain bf16 and leave like the plain GEMM's
    if (n0 + BN > g.q_cols) {
      fused_epilogue<FUSED_D, BN>(g, acc, s, smem, m0, n0, wm, wn, wave, lane);
      return;
    }
  }
  // The tile goes through LDS as bf16 (the operand stages are free once every
  // wave has left the loop), so that it leaves in whole rows: each store
  // instruction writes two 512-byte runs (16 bytes per lane) instead of 32
  // rows of 16 bytes.
  constexpr int kOutRow = BN * 2 + 16;          // bytes per tile row in LDS (padded)
  static_assert(kBM * kOutRow <= 2 * kStageBytes, "the bf16 tile fits the operand stages");
  const int hh = lane >> 5;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = wm + 32 * i + (lane & 31);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int grp4 = 0; grp4 < 4; ++grp4) {
        const int col = wn + 32 * j + 8 * grp4 + 4 * hh;
        const auto& a4 = acc[i][j];
        *reinterpret_cast<uint2*>(smem + row * kOutRow + col * 2) =
            make_uint2(pack_bf16x2(a4[4 * grp4] * s, a4[4 * grp4 + 1] * s),
                       pack_bf16x2(a4[4 * grp4 + 2] * s, a4[4 * grp4 + 3] * s));
      }
  }
  __syncthreads();
  constexpr int kRowChunks = BN * 2 / 16;       // 16-byte chunks per tile row
#pragma unroll
  for (int c = threadIdx.x; c < kBM * kRowChunks; c += kGemmThreads) {
    const int row = c / kRowChunks;
    const int n = n0 + (c % kRowChunks) * 8;
    const int m = m0 + row;
    if (m >= g.M || n >= g.N) continue;
    const uint4 v = *reinterpret_cast<const uint4*>(smem + row * kOutRow + (c % kRowChunks) * 16);
    uint16_t* dst = g.c + (int64_t)m * g.ldc + n;
    if (g.vec_store && n + 8 <= g.N) {
      *reinterpret_cast<uint4*>(dst) = v;
    } else {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (n + e < g.N) dst[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
    }
  }
}

}  // namespace

int quant_max_partials() { return 1024; }

static int quant_blocks(int64_t n) {
  const int64_t per_block = (int64_t)kQuantThreads * 8 * 4;
  return (int)std::min<int64_t>(quant_max_partials(), std::max<int64_t>(1, (n + per_block - 1) / per_block));
}

hipError_t launch_quant_fp8(const uint16_t* x, int64_t n, uint8_t* codes, float* scale,
                            uint32_t* partial, hipStream_t stream) {
  const int blocks = quant_blocks(n);
  hipLaunchKernelGGL(quant_amax_kernel, dim3(blocks), dim3(kQuantThreads), 0, stream, x, n, partial);
  hipLaunchKernelGGL(quant_apply_kernel, dim3(blocks), dim3(kQuantThreads), 0, stream, x, n,
                     (const uint32_t*)partial, blocks, codes, scale);
  return hipGetLastError();
}

// Workspace of the per-tensor quantization held by the library itself, for
// callers that cannot allocate: one block's max |x| per word.  Every call
// writes the words it reads, so nothing needs clearing; calls that overlap on
// one GPU share the array and race.  Each GPU holds its own copy; host code
// reaches it only through the address hipGetSymbolAddress gives per device.
constexpr int kQuantScratchWords = 1024;
static __device__ __align__(256) uint32_t scratch[kQuantScratchWords];

static hipError_t quant_scratch(uint32_t** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex lock;
  static uint32_t* ptrs[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(lock);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptrs[dev] = static_cast<uint32_t*>(p);
  }
  *out = ptrs[dev];
  return hipSuccess;
}

int quant_scratch_words() { return kQuantScratchWords; }

hipError_t launch_quant_fp8_static(const uint16_t* x, int64_t n, uint8_t* codes, float* scale,
                                   hipStream_t stream) {
  if (quant_blocks(n) > kQuantScratchWords) return hipErrorInvalidValue;
  uint32_t* partial = nullptr;
  const hipError_t e = quant_scratch(&partial);
  if (e != hipSuccess) return e;
  return launch_quant_fp8(x, n, codes, scale, partial, stream);
}

static GemmArgs gemm_args(const uint8_t* a, const float* sa, const uint8_t* bt, const float* sb, uint16_t* c,
                          int M, int N, int K, int64_t ldc) {
  GemmArgs g{};
  g.a = a; g.bt = bt; g.sa = sa; g.sb = sb; g.c = c; g.ldc = ldc;
  g.M = M; g.N = N; g.K = K;
  g.n_mt = (M + kBM - 1) / kBM;
  g.n_nt = (N + kBN - 1) / kBN;
  g.n_tiles = g.n_mt * g.n_nt;
  g.vec_store = (reinterpret_cast<uintptr_t>(c) % 16 == 0) && (ldc % 8 == 0);
  return g;
}

// LDS of a launch: the two operand stages, or the fused epilogue's f32 tile
// and amax exchange if larger
template <int FUSED_D, int BN>
constexpr int gemm_lds_bytes() {
  return FUSED_D > 0 && epi_amax<BN>() + kGemmWaves * 64 * 4 > 2 * stage_bytes<BN>()
             ? epi_amax<BN>() + kGemmWaves * 64 * 4
             : 2 * stage_bytes<BN>();
}

template <int FUSED_D, int BN>
static hipError_t launch_part(const GemmArgs& g, hipStream_t stream) {
  constexpr int lds = gemm_lds_bytes<FUSED_D, BN>();
  static_assert(lds <= 160 * 1024, "one workgroup's LDS");
  const hipError_t e = hipFuncSetAttribute((const void*)gemm_fp8_kernel<FUSED_D, BN>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  const int grid = (g.n_launch + 7) / 8 * 8;
  hipLaunchKernelGGL((gemm_fp8_kernel<FUSED_D, BN>), dim3(grid), dim3(kGemmThreads), lds, stream, g);
  return hipGetLastError();
}

// compute units of the current device (one GEMM workgroup each), looked up
// once per device
static hipError_t device_cus(int* out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static int cus[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (cus[dev] == 0) {
    e = hipDeviceGetAttribute(&cus[dev], hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
  }
  *out = cus[dev];
  return hipSuccess;
}

// Whole rounds of 256 x 256 tiles (one workgroup per compute unit), then the
// tiles of a last round that would fill at most half the device as 256 x 128
// halves: that round then takes about half a tile's time instead of a whole
// one (846 tiles on 256 units: 3 rounds + 78 tiles, the projection chunk).
template <int FUSED_D>
static hipError_t launch_gemm(GemmArgs g, hipStream_t stream) {
  int cus = 0;
  hipError_t e = device_cus(&cus);
  if (e != hipSuccess) return e;
  const int full = cus > 0 ? g.n_tiles / cus * cus : g.n_tiles;
  const int rem = g.n_tiles - full;
  if (rem == 0 || 2 * rem > cus) {
    g.tile_base = 0;
    g.n_launch = g.n_tiles;
    return launch_part<FUSED_D, kBN>(g, stream);
  }
  if (full > 0) {
    g.tile_base = 0;
    g.n_launch = full;
    e = launch_part<FUSED_D, kBN>(g, stream);
    if (e != hipSuccess) return e;
  }
  g.tile_base = full;
  g.n_launch = 2 * rem;
  return launch_part<FUSED_D, kBN / 2>(g, stream);
}

hipError_t launch_gemm_fp8(const uint8_t* a, const float* sa, const uint8_t* bt, const float* sb,
                           uint16_t* c, int M, int N, int K, int64_t ldc, hipStream_t stream) {
  return launch_gemm<0>(gemm_args(a, sa, bt, sb, c, M, N, K, ldc), stream);
}

hipError_t launch_qkv_gemm_append(const QkvAppendArgs& q, hipStream_t stream) {
  const int N = q.q_cols + 2 * q.n_kv_heads * q.head_dim;
  GemmArgs g = gemm_args(q.x, q.sx, q.wt, q.sw, q.q_out, q.M, N, q.K, q.ldq);
  g.q_cols = q.q_cols;
  g.n_kv_heads = q.n_kv_heads;
  g.rope = q.rope;
  g.kc = q.kc; g.vc = q.vc; g.ks = q.ks; g.vs = q.vs;
  g.slots_padded = q.slots_padded;
  g.write_slot = q.write_slot;
  return q.head_dim == 128 ? launch_gemm<128>(g, stream) : launch_gemm<64>(g, stream);
}

}  // namespace rtv
