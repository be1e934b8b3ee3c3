// Chunk attention over the FP8 ring window (gfx950 matrix cores).
//
// The chunk's queries attend to every key of the valid window, the chunk
// itself included (240 such calls per diffusion step: page "Runway: Πώς ένα
// AI 57 δισ. παραμέτρων παράγει βίντεο στα 24 fps", section "Από οκτώ H100 σε
// τέσσερις"; the cache holds RoPE-rotated e4m3 K and e4m3 V, page "Runway
// explains how it serves a 57B video model in real time", fourth paragraph).
//
// Work decomposition: one workgroup = 256 queries of one query head, 8 waves
// of 32 queries, one workgroup per CU.  Waves w and w + 4 share a SIMD and,
// held together by the per-tile barrier, run their softmax at the same time:
// a lone wave issues VALU instructions at about half the SIMD's rate, so two
// waves in the same phase keep the VALU busy while the matrix-core phases of
// both follow back to back.  The workgroup walks 64-key tiles of the
// window's (at most two) slot segments through a 4-stage LDS ring with one
// barrier per tile; waves 0-3 stage the K rows and waves 4-7 the V rows of
// tile t+2 while tile t is computed.
//
// Per wave and tile (e4m3 operands, f32 accumulate):
//   S^T[key][query] = K . Q^T + C_key     head dim 64 (attend_kernel): with
//   v_mfma_f32_32x32x64_f8f6f4, 2 key halves x D/64 k-steps; lane (hh, i)
//   holds query i and 32 of the 64 keys: the softmax row is per lane plus one
//   v_permlane32_swap with lane i^32.  Head dim 128 (attend16_kernel): with
//   v_mfma_f32_16x16x128_f8f6f4, 4 key blocks x 2 query blocks; a lane holds
//   16 keys of 2 queries, which halves its per-key factor reads, and P' is
//   brought to the PV operand layout by v_permlane16_swap (see there);
//   O^T[d][query] += V^T . P'^T           D/32 d sub-tiles (32x32x64)
//   L[r][query]   += U . P'^T             one product: the row sum (32x32x64
//                                         for head dim 64; for head dim 128 a
//                                         16x16x128 on the same P' registers)
// Scores: each query carries its own power-of-two scale 2^e_q (its largest
// rotated element maps into [128, 256)), applied exactly by the matrix core
// through the E8M0 scale of the query operand, so the score products come out
// in the units of the rotated query and the rest of the per-score scale is a
// per-key factor kf = sk * log2(e)/sqrt(D) from the factors kernel.
// P' carries the V scale of its key: P' = p * 55 * rho_key with
// rho = sv / 2^e, 2^e the least power of two above the largest V scale of
// the key's 64-slot tile; the PV product scales P' back by 2^e through the
// E8M0 scale of its B operand (exact), so that it sums 55 p sv Vcodes.
// log2(55 rho) enters as the accumulator's initial value
// C = log2(55 rho) / kf, so t = fma(S, kf, -m) = log2 P' and P' costs one
// FMA and one conversion per score.  Long windows take the e4m3 code of P'
// straight from t: with kf and m in units of 1/8 octave the FMA gives
// u = 8 t + 56, and v_cvt_pk_u8_f32 rounds u to the nearest integer and
// saturates it to [0, 255], which is the code of the e4m3 value whose
// piecewise-linear log2 (exponent + mantissa / 8) lies nearest to t (within
// one code of the RNE e4m3 of 2^t; no exponential).  Short windows take
// 2^t with v_exp_f32 and carry it as two e4m3 terms.  The row sum is taken
// from the same e4m3 P' by the matrix cores, against U = 1/rho as two e4m3
// terms (rows 0 and 1 of U): numerator and denominator share P'.  The per-key
// factors come from a small factors kernel run before the attention.  The
// running max m is lazy: it moves only when some P' would exceed 440, and
// then leaves a factor 2^kTau of headroom.  Output O = acc / L, rounded to
// bf16.
//
// Peaked rows.  The one-code P' (and one-term Q) errors, a few per cent per
// weight, average out only when a row's weight spreads over many keys.  With
// check_peaked the one-code kernels also take G = sum_k P'_k^2 per query on
// the matrix cores (the diagonal of P' P'^T, one more product per tile whose
// operands are the P' codes already in registers), and G / L^2 = sum_k
// (p_k rho_k)^2 / (sum_k p_k)^2, a lower bound of sum p^2 over the normalised
// weights, measures how few keys carry the row.  A unit (query tile x head)
// with a row above kPeakedGram is flagged (for a key-range part, by the
// combine kernel from the merged sums), and a second launch recomputes only
// the flagged units with two-term Q and P' (relative error about 2^-8 each).
#include "device_common.hpp"
#include "kernels.hpp"
#include "ring.hpp"

namespace rtv {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

#ifndef RTV_ATTEND_WAVES
#define RTV_ATTEND_WAVES 8
#endif
#ifndef RTV_ATTEND_WG_PER_CU
#define RTV_ATTEND_WG_PER_CU 1
#endif
constexpr int kWaves = RTV_ATTEND_WAVES;
constexpr int kThreads = kWaves * kWave;
#ifndef RTV_ATTEND_QPB
#define RTV_ATTEND_QPB 256
#endif
constexpr int kQPB = RTV_ATTEND_QPB;        // queries per workgroup
constexpr int kQPW = kQPB / kWaves;         // queries per wave
constexpr int kSub = kQPW / 32;             // 32-query sub-tiles per wave (they share the K/V operands)
constexpr int kStages = 4;                  // LDS ring: tiles it - 1 .. it + 2
constexpr float kTau = 3.0f;
constexpr float kLogPmax = 8.78135971f;     // log2(440): bound on P' (below the e4m3 max 448)
// log-domain units of the scores: u = kUnit * log2 P' + kOff.  Exact path
// (two-term P' from v_exp_f32): u = t.  Linear-code path: u = 8 t + 56 is the
// e4m3 code of P' before rounding (code 8 e + m <-> 2^(e - 7) (1 + m / 8)).
template <bool EXACT> struct LogUnits {
  static constexpr float kUnit = EXACT ? 1.0f : 8.0f;
  static constexpr float kOff = EXACT ? 0.0f : 56.0f;
  static constexpr float kTop = kUnit * kLogPmax + kOff;    // u bound: P' <= 440
  static constexpr float kReset = kTop - kUnit * kTau;      // largest u after a rescale
};
constexpr float kPW = 55.0f;                // P' = p * kPW * rho, rho <= 1
constexpr float kLogPW = 5.78135971f;       // log2(kPW)
constexpr float kRhoMin = 0.0009765625f;    // 2^-10: floor of rho (U = 2^-2 / rho <= 256)
constexpr float kScaleMin = 8.6736174e-19f; // 2^-60: floor of sk, so that C stays finite
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kMaskFactor = 1e30f;        // kf of a key outside the window segment
// Peaked-row threshold on G / L^2 (sum over the window of (p rho)^2, p the
// normalised weights).  Rows of N(0,1) queries and keys stay below 2.5e-5 on
// a 47872-key window and 4e-4 on 8192 keys; simulated one-code errors stay
// inside the attention tolerance below it, while every simulated row family
// that breaks the tolerance (keys of a chunk scaled by 1.5 to 4, weight spread
// evenly over 50-400 keys) lies above it.
constexpr float kPeakedGram = 5e-4f;

__device__ __forceinline__ v16f mfma_fp8(const v8i& a, const v8i& b, const v16f& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

typedef float v4f __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4f mfma16_fp8(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ v4f mfma16_fp8_bscaled(const v8i& a, const v8i& b, const v4f& c, int e) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, e);
}
__device__ __forceinline__ v4f mfma16_fp8_scaled(const v8i& a, const v8i& b, const v4f& c, int ea, int eb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, ea, 0, eb);
}

// the same with the B operand scaled by 2^(e - 127) (E8M0 exponent e):
// adds the low-order e4m3 part of a two-term operand
__device__ __forceinline__ v16f mfma_fp8_bscaled(const v8i& a, const v8i& b, const v16f& c, int e) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, e);
}
// both operands scaled: A by 2^(ea - 127), B by 2^(eb - 127)
__device__ __forceinline__ v16f mfma_fp8_scaled(const v8i& a, const v8i& b, const v16f& c, int ea, int eb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, ea, 0, eb);
}

// two-term e4m3 of two values: hi = e4m3(x), lo = e4m3((x - hi) * 2^kLoShift)
// (|x - hi| <= 2^-4 |x|, so the scaled residual stays in range)
constexpr int kLoShift = 4;
// windows shorter than this many keys also carry P' as two terms (PLO)
constexpr int64_t kPreciseKeys = 8192;
// split-key-range parts are bounded so that the workspace has a fixed size
constexpr int kMaxParts = 512;
template <bool HIGH>
__device__ __forceinline__ void split_fp8x2(float a, float b, uint32_t& hi, uint32_t& lo) {
  constexpr float kLoMul = (float)(1 << kLoShift);
  hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)hi, HIGH);
  const auto h = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, HIGH);
  lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32((a - h[0]) * kLoMul, (b - h[1]) * kLoMul, (int)lo, HIGH);
}

// max over lane i and lane i^32 (the two halves of a softmax row)
__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// key index held by byte p of a transposed V tile row
__device__ __forceinline__ int vt_key(int p) {
  const int h = p >> 5, b = p & 31;
  return 32 * (b >> 4) + 8 * ((b >> 2) & 3) + 4 * h + (b & 3);
}

template <int D>
struct Smem {
  static constexpr int KROW = D + 16;       // padded K row (bytes): conflict-free 16 B reads
  static constexpr int VROW = 64 + 16;      // padded transposed-V row
  static constexpr int K_BYTES = 64 * KROW;
  // V^T rows, then the two U rows and a zero row (zeroed once, never staged)
  static constexpr int V_BYTES = (D + 3) * VROW;
  static constexpr int U_OFF = K_BYTES + D * VROW;
  static constexpr int KF_OFF = K_BYTES + V_BYTES;    // kf[64], C[64], the tile's V exponent
  static constexpr int STAGE = KF_OFF + 2 * 64 * 4 + 16;
};

// Staged tile: with 512 threads, threads 0..255 (waves 0-3) move the K rows
// and write kf and C, threads 256..511 (waves 4-7) move the transposed V rows
// and the U rows; with 256 threads every thread does both.  D/4 bytes of codes
// each, and every thread holds the factors of key (thread & 63).
constexpr int kStageJobs = kThreads >= 512 ? 1 : 2;
struct TileRegs {
  uint4 c[kStageJobs][2];
  // K side: the factor record (max(sk, kScaleMin), log2(55 rho) / that, the
  // tile's E8M0 V exponent, 0) of key (thread & 63); V side: 16-byte piece
  // (thread & 7) of the U rows
  uint4 x[kStageJobs];
};

struct TileRef {
  int tile;
  int lo, hi;         // the segment the tile belongs to (slot indices fit in int32)
};

// dword 3 of a raw buffer descriptor (32-bit elements, no swizzle)
constexpr int kBufferFlags = 0x00020000;

// Byte offset in a 64-slot tile of the first of the D/64 adjacent 16-byte
// pieces of codes that thread g (0..255) of a side moves.  The 16 lanes of
// each quarter wave take 16 different rows at one column, as the operand
// reads do, so that the padded LDS rows spread their writes over the banks.
// K: 64 rows of D bytes, 4 threads per row, 16 rows per wave.
template <int D>
__device__ __forceinline__ int k_code_off(int g) {
  return (16 * (g >> 6) + (g & 15)) * D + ((g >> 4) & 3) * (D / 4);
}
// transposed V: D rows of 64 bytes, 256 / D threads per row
template <int D>
__device__ __forceinline__ int v_code_off(int g) {
  constexpr int RPW = 64 / (256 / D);       // rows per wave
  return (RPW * (g >> 6) + (g % RPW)) * 64 + ((g & 63) / RPW) * (D / 4);
}

// The side (K or V) of a thread is uniform over its wave (side = -1 for
// 256-thread workgroups, where every thread does both); the addresses are a
// wave-uniform base plus a per-lane offset that does not change with the tile.
template <int D>
__device__ __forceinline__ void load_tile(TileRegs& r, const TileRef& t, const uint8_t* kc,
                                          const uint8_t* vc, const uint8_t* frec, const uint8_t* fu,
                                          int side, int k_off, int v_off, int xk_off, int xv_off) {
  constexpr int LD_BYTES = D / 4;
#pragma unroll
  for (int j = 0; j < kStageJobs; ++j) {
    const bool isv = kStageJobs == 1 ? side == 1 : j == 1;
    // buffer loads through a descriptor of exactly this tile's bytes
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((isv ? vc : kc) + (int64_t)t.tile * 64 * D), 0, 64 * D, kBufferFlags);
    const int code_off = isv ? v_off : k_off;
    r.c[j][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rc, code_off, 0, 0));
    if constexpr (LD_BYTES == 32)
      r.c[j][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rc, code_off + 16, 0, 0));
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(isv ? fu + (int64_t)t.tile * 128 : frec + (int64_t)t.tile * 1024), 0, isv ? 128 : 1024,
        kBufferFlags);
    r.x[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, isv ? xv_off : xk_off, 0, 0));
  }
}

// Byte offset in a stage of the 16-byte piece at byte b of a staged tile: K
// rows (row = key b / D), or the transposed V rows (row = d, col = slot
// position).
template <int D>
__device__ __forceinline__ int k_piece_at(int b) {
  using SM = Smem<D>;
  return (b / D) * SM::KROW + (b % D);
}
template <int D>
__device__ __forceinline__ int v_piece_at(int b) {
  using SM = Smem<D>;
  return SM::K_BYTES + (b / 64) * SM::VROW + (b % 64);
}
// Keys of a partial tile outside the segment get zero codes (they may hold
// anything, NaN codes included).
template <int D>
__device__ __forceinline__ uint4 mask_k_piece(uint4 q, int b, int base, int lo, int hi) {
  const int kslot = base + b / D;
  return (kslot >= lo && kslot < hi) ? q : make_uint4(0, 0, 0, 0);
}
__device__ __forceinline__ uint4 mask_v_piece(uint4 v, int b, int base, int lo, int hi) {
  const int col = b % 64;
  uint32_t m[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    m[w] = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int slot = base + vt_key(col + 4 * w + e);
      if (slot >= lo && slot < hi) m[w] |= 0xFFu << (8 * e);
    }
  }
  v.x &= m[0]; v.y &= m[1]; v.z &= m[2]; v.w &= m[3];
  return v;
}

// byte position of key k in a transposed V (and U) row: the inverse of vt_key
__device__ __forceinline__ int vt_pos(int k) {
  return 32 * ((k >> 2) & 1) + 16 * (k >> 5) + 4 * ((k >> 3) & 3) + (k & 3);
}

// kunit: the score units per octave (kf is staged in those units).
// The codes are stored branch-free apart from the masking of partial tiles:
// K and V pieces differ only in their address.  The first K-side wave writes
// kf and C (lane = key), lanes 0..7 of the first V-side wave the U rows.
template <int D, bool MASK>
__device__ __forceinline__ void store_tile(const TileRegs& r, const TileRef& t, uint8_t* st,
                                           float kunit, int tid) {
  using SM = Smem<D>;
  constexpr int LD_BYTES = D / 4;
  const int gt = tid & 255;
  const int base = t.tile * 64;
  const bool partial = MASK && (t.lo > base || t.hi < base + 64);
#pragma unroll
  for (int j = 0; j < kStageJobs; ++j) {
    const bool isv = kStageJobs == 1 ? tid >= 256 : j == 1;
    const int b = isv ? v_code_off<D>(gt) : k_code_off<D>(gt);
#pragma unroll
    for (int h = 0; h < LD_BYTES / 16; ++h) {
      const int bb = b + 16 * h;
      uint4 q = r.c[j][h];
      if (partial) q = isv ? mask_v_piece(q, bb, base, t.lo, t.hi) : mask_k_piece<D>(q, bb, base, t.lo, t.hi);
      *(uint4*)(st + (isv ? v_piece_at<D>(bb) : k_piece_at<D>(bb))) = q;
    }
  }
  const int wave = __builtin_amdgcn_readfirstlane(tid) >> 6;
  const bool kside = wave == 0;
  const bool vside = wave == (kStageJobs == 2 ? 0 : 4) && (tid & 63) < 8;
  const uint4 xk = r.x[0];
  const uint4 xv = r.x[kStageJobs - 1];
  if (kside) {
    // u = (S + C) * kf - m = kUnit (S * kf1 + log2(55 rho)) - m with kf1 the
    // factor in log2 units.  A key outside the segment gets kf = kMaskFactor
    // and C = 0: its raw score is the bias -448*448 added by the masking MFMA,
    // so u ~ -2e35 and P' = 0
    const int key = tid & 63;
    const bool ok = !MASK || (base + key >= t.lo && base + key < t.hi);
    const float kf = __uint_as_float(xk.x) * kunit;
    const float c = __uint_as_float(xk.y);
    float* kfp = (float*)(st + SM::KF_OFF);
    kfp[key] = ok ? kf : kMaskFactor;
    kfp[64 + key] = ok ? c : 0.0f;
    if (key == 0) ((uint32_t*)kfp)[128] = xk.z;
  }
  if (vside) {
    const int piece = tid & 7;
    *(uint4*)(st + SM::U_OFF + (piece >> 2) * SM::VROW + 16 * (piece & 3)) = xv;
  }
}

__device__ __forceinline__ TileRef tile_of(int it, int t_count0, int t_first0, int t_first1,
                                           int lo0, int hi0, int lo1, int hi1) {
  const bool second = it >= t_count0;
  TileRef r;
  r.lo = second ? lo1 : lo0;
  r.hi = second ? hi1 : hi0;
  r.tile = second ? t_first1 + (it - t_count0) : t_first0 + it;
  return r;
}

// Per-window key factors: one wave per (KV head, window tile).  The tile's V
// exponent e is the least power of two 2^e >= its largest V scale; for each
// slot rho = sv / 2^e (exact; 1 for a zero V row, at least kRhoMin), the
// record (kf = max(sk, kScaleMin) log2(e) / sqrt(D), log2(55 rho) / kf,
// 127 + e, 0) and the two e4m3 terms of 2^-2 / rho at the slot's byte
// position in the U rows.  Slots of a partial tile outside the window get
// factors too (from whatever their scales hold; the attention masks them).
// The first workgroup also clears the peaked-unit flags of the call.
// Device-state mode: the window's segments, the chunk's RoPE rows and the
// split schedule from the layer's ring state, with the same arithmetic as the
// host's in host-state mode.  False, with the state's error set, when the
// chunk would run past the RoPE table or the state is not a ring state: the
// call's kernels then write nothing.
__device__ __forceinline__ bool attend_derive(AttendArgs& a) {
  const RingShape& g = a.shape;
  const int64_t next = a.dstate->next_global_frame;
  RingWindow w;
  if (next + g.chunk_frames > g.max_global_frames ||
      ring_window(next, a.dstate->committed, g.tokens_per_frame, g.chunk_frames, g.capacity_frames,
                  g.max_window_frames, &w) != kRingOk) {
    if (blockIdx.x == 0 && threadIdx.x == 0) a.dstate->error = 1;
    return false;
  }
  a.rope = a.rope_table + next * g.tokens_per_frame * g.head_dim;
  a.n_segments = w.n_segments;
  a.seg_lo[0] = w.seg_start[0];
  a.seg_hi[0] = w.seg_start[0] + w.seg_len[0];
  a.seg_lo[1] = w.seg_start[1];
  a.seg_hi[1] = w.seg_start[1] + w.seg_len[1];
  attend_schedule(a, attend_window_tiles(a), kMaxParts);
  return true;
}

template <int D>
__global__ __launch_bounds__(256) void factors_kernel(AttendArgs a) {
  if (a.flags && blockIdx.x == 0)
    for (int i = threadIdx.x; i <= a.n_work; i += 256) a.flags[i] = 0u;
  if (a.dstate && !attend_derive(a)) return;
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lo0 = (int)a.seg_lo[0], hi0 = (int)a.seg_hi[0];
  const int lo1 = a.n_segments > 1 ? (int)a.seg_lo[1] : 0;
  const int hi1 = a.n_segments > 1 ? (int)a.seg_hi[1] : 0;
  const int t_first0 = lo0 / 64;
  const int t_count0 = hi0 > lo0 ? (hi0 - 1) / 64 - t_first0 + 1 : 0;
  const int t_first1 = lo1 / 64;
  const int t_count1 = hi1 > lo1 ? (hi1 - 1) / 64 - t_first1 + 1 : 0;
  const int n_all = t_count0 + t_count1;
  if (w >= n_all * a.n_kv_heads) return;      // whole waves leave together
  const int h = w / n_all;
  const int i = w % n_all;
  const int tile = i < t_count0 ? t_first0 + i : t_first1 + (i - t_count0);
  const int64_t slot = (int64_t)h * a.slots_padded + (int64_t)tile * 64 + lane;
  const float sv = a.vs[slot];
  const float sk = a.ks[slot];
  // (non-finite or negative scales, which only unused slots could hold, count as 0)
  float m = sv > 0.0f && sv <= 3.40282347e38f ? sv : 0.0f;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, o));
  int e = 0;
  if (m > 0.0f) {
    (void)frexpf(m, &e);                // m = f * 2^e, f in [0.5, 1): 2^e > m
    e = e < -126 ? -126 : e;
  }
  const float rho = sv > 0.0f ? __builtin_fmaxf(ldexpf(sv, -e), kRhoMin) : 1.0f;
  const float kf = __builtin_fmaxf(sk, kScaleMin) * (kLog2e / sqrtf((float)D));
  const int64_t rt = (int64_t)h * a.ring_tiles + tile;
  ((float4*)a.fac_l)[rt * 64 + lane] =
      make_float4(kf, (kLogPW + __builtin_amdgcn_logf(rho)) / kf, __uint_as_float((uint32_t)(127 + e)), 0.0f);
  const float u = 0.25f / rho;
  const int hi = __builtin_amdgcn_cvt_pk_fp8_f32(u, 0.0f, 0, false);
  const float uh = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false)[0];
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(u - uh, 0.0f, 0, false);
  a.fac_u[rt * 128 + vt_pos(lane)] = (uint8_t)hi;
  a.fac_u[rt * 128 + 64 + vt_pos(lane)] = (uint8_t)lo;
}

// t = S_raw * kf - m for the 32 keys of this lane
__device__ __forceinline__ void scores(const v16f (&s)[2], const float* kf, int hh, float m,
                                       float (&t)[32]) {
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int key0 = 32 * kh + 8 * g + 4 * hh;
      const float4 k4 = *(const float4*)(kf + key0);
      const float kk[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) t[16 * kh + 4 * g + e] = __builtin_fmaf(s[kh][4 * g + e], kk[e], -m);
    }
}

// max of 32 values as a tree of three-input maxima: 10 of them leave 12
// values (two of the inputs pass through), 4 more leave 4, then one three-input
// and one two-input maximum (16 instructions, the fewest for 32 inputs)
__device__ __forceinline__ float max32(const float (&t)[32]) {
  float a[12];
#pragma unroll
  for (int i = 0; i < 10; ++i) a[i] = __builtin_fmaxf(__builtin_fmaxf(t[3 * i], t[3 * i + 1]), t[3 * i + 2]);
  a[10] = t[30];
  a[11] = t[31];
  float b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = __builtin_fmaxf(__builtin_fmaxf(a[3 * i], a[3 * i + 1]), a[3 * i + 2]);
  return __builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(b[0], b[1]), b[2]), b[3]);
}

// Softmax of one 32-query tile over one 64-key tile, first half (after
// u = fma(S, kf, -m), mx = the lane's max of u, all in the units of LU): the
// lazy running-max update.  Rare: only when some P' would exceed 440; it
// rescales the O and row-sum accumulators, shifts u and leaves the largest
// P' of the row at 440 / 2^kTau.  m is finite from the first tile on (set
// from tile 0 before the loop), so the raw row max is max(u) + m and no
// score is recomputed.
template <int NDT, class LU, bool STAT>
__device__ __forceinline__ void lazy_rescale(float mx, float& m, v16f (&o)[NDT], v16f& lsum, v16f& gsum,
                                             float (&t)[32]) {
  if (__builtin_expect(__any(mx > LU::kTop), 0)) {
    const float raw = xhalf_max(mx) + m;
    const float m_new = __builtin_fmaxf(m, raw - LU::kReset);
    const float shift = m - m_new;
    const float alpha = exp2f(shift * (1.0f / LU::kUnit));
#pragma unroll
    for (int d = 0; d < NDT; ++d) o[d] *= alpha;
    lsum *= alpha;
    if constexpr (STAT) gsum *= alpha * alpha;
#pragma unroll
    for (int j = 0; j < 32; ++j) t[j] += shift;
    m = m_new;
  }
}

// Second half, in quarters (keys 8c .. 8c + 7 of the lane): P' in e4m3, the
// B operand of the PV and row-sum products.  PRECISE: 2^t as two terms;
// otherwise the code is u = 8 t + 56 rounded and saturated to [0, 255] (u
// stays below 126.5 by the running max, so codes reach at most 0x7E = 448; a
// key far below the max, or masked, gives +0).
template <bool PRECISE>
__device__ __forceinline__ void probs_quarter(int c, const float (&t)[32], v8i& pop, v8i& plo) {
#pragma unroll
  for (int w = 2 * c; w < 2 * c + 2; ++w) {
    if constexpr (PRECISE) {
      float pp[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) pp[e] = __builtin_amdgcn_exp2f(t[4 * w + e]);
      uint32_t hi = 0, lo = 0;
      split_fp8x2<false>(pp[0], pp[1], hi, lo);
      split_fp8x2<true>(pp[2], pp[3], hi, lo);
      pop[w] = (int)hi;
      plo[w] = (int)lo;
    } else {
      // bytes 0..3 in turn: every byte of the register is written, so its
      // old contents (t[4 w], dead after the first conversion) do not matter
      uint32_t x = __builtin_amdgcn_cvt_pk_u8_f32(t[4 * w + 0], 0, __float_as_uint(t[4 * w + 0]));
      x = __builtin_amdgcn_cvt_pk_u8_f32(t[4 * w + 1], 1, x);
      x = __builtin_amdgcn_cvt_pk_u8_f32(t[4 * w + 2], 2, x);
      x = __builtin_amdgcn_cvt_pk_u8_f32(t[4 * w + 3], 3, x);
      pop[w] = (int)x;
    }
  }
}

// scheduling fence between the interleaved chunks of matrix-core and vector
// work: LDS reads, scalar and global-read instructions may still move across
__device__ __forceinline__ void chunk_fence() { __builtin_amdgcn_sched_barrier(0x0124); }

// Work item of a workgroup: a whole unit (query tile x head; part = -1) or
// one key-range part of a unit; false when the workgroup has none.
__device__ __forceinline__ bool work_item(const AttendArgs& a, int& unit, int& part) {
  const int xcd = blockIdx.x & 7;
  const int local = blockIdx.x >> 3;
  if (local < a.full_per_xcd) {
    unit = xcd * a.full_per_xcd + local;
    part = -1;
    return unit < a.n_full;
  }
  // (device-state grids are sized for the largest window: surplus workgroups
  // of an XCD leave instead of taking another XCD's parts)
  if (local - a.full_per_xcd >= a.parts_per_xcd) return false;
  const int j = xcd * a.parts_per_xcd + (local - a.full_per_xcd);
  if (j >= a.n_parts) return false;
  unit = a.n_full + j / a.parts_per_unit;
  part = j;
  return true;
}

// E8M0 exponent e of a query's power-of-two scale: its largest rotated |q|
// divided by 2^e lies in [128, 256) (e4m3 reaches 448).  Clamped so that both
// terms of a two-term query keep their E8M0 scales in range (an all-zero query
// takes 2^0).
__device__ __forceinline__ int query_exp(float amax) {
  int e = 0;
  if (amax > 0.0f) {
    (void)frexpf(amax, &e);             // amax = f 2^e, f in [0.5, 1)
    e -= 8;
  }
  return e < -120 ? -120 : (e > 120 ? 120 : e);
}

// Peaked-row statistic: G = sum_k P'_k^2 of each query, the diagonal of the
// 32x32 product P' P'^T of the wave's P' codes with themselves (the A and B
// operand layouts of v_mfma_f32_32x32x64 agree: lane (hh, li) holds row /
// column li and the keys of half hh).  Diagonal element (li, li) sits in lane
// 32 ((li >> 2) & 1) + li, register 4 (li >> 3) + (li & 3); both lanes of the
// query (li and li + 32) receive it.
__device__ __forceinline__ float gram_diag(const v16f& g, int li, int hh) {
  const int gi = 4 * (li >> 3) + (li & 3);
  float x = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) x = i == gi ? g[i] : x;
  return xhalf_sum(hh == ((li >> 2) & 1) ? x : 0.0f);
}

// flag a unit as peaked; the first flag of a unit counts it
__device__ __forceinline__ void flag_unit(const AttendArgs& a, int unit) {
  if (atomicOr(&a.flags[unit], 1u) == 0u) atomicAdd(&a.flags[a.n_work], 1u);
}

// Result of one lane for its query (PV layout: lane (hh, li) holds query li
// of a 32-query sub-tile, q its index in the workgroup): a whole unit writes O
// = acc / L as bf16; a key-range part writes sum p V / 55 and (m, sum p / 55,
// sum p'^2 / 55^2) with m back in log2 units (u = kUnit t + kOff, so m =
// (m_u + kOff) / kUnit).
template <int D, class LU>
__device__ __forceinline__ void write_result(const AttendArgs& a, const v16f (&o)[D / 32], float l_tot, float m_u,
                                             float g, int part, int q, int row, int head, int hh) {
  constexpr int NDT = D / 32;
  if (part >= 0) {
    float* po = a.ws_o + ((int64_t)part * kQPB + q) * D;
    const float inv_c = 1.0f / kPW;
#pragma unroll
    for (int d = 0; d < NDT; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * d + 8 * g + 4 * hh;
        *(float4*)(po + d0) = make_float4(o[d][4 * g + 0] * inv_c, o[d][4 * g + 1] * inv_c,
                                          o[d][4 * g + 2] * inv_c, o[d][4 * g + 3] * inv_c);
      }
    if (hh == 0)
      *(float4*)(a.ws_ml + ((int64_t)part * kQPB + q) * 4) =
          make_float4((m_u + LU::kOff) * (1.0f / LU::kUnit), l_tot / kPW, g * (1.0f / (kPW * kPW)), 0.0f);
    return;
  }
  const float scale = 1.0f / l_tot;
  if (row < a.n_tokens) {
    uint16_t* dst = a.out + (int64_t)row * a.ldo + (int64_t)head * D;
#pragma unroll
    for (int d = 0; d < NDT; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * d + 8 * g + 4 * hh;
        uint2 w;
        w.x = pack_bf16x2(o[d][4 * g + 0] * scale, o[d][4 * g + 1] * scale);
        w.y = pack_bf16x2(o[d][4 * g + 2] * scale, o[d][4 * g + 3] * scale);
        *(uint2*)(dst + d0) = w;
      }
  }
}

// MASK = false: every segment boundary of the window falls on a 64-slot tile
// boundary (the host checks), so no tile needs masking and the kernel carries
// no masking code.  MASK = true handles any boundary.
// QLO / PLO: Q / P' are carried as two e4m3 terms, hi + 2^-kLoShift * lo,
// each product taking a second MFMA whose B operand is scaled by
// 2^-kLoShift; the relative error of the operand drops from 2^-4 to about
// 2^-8.  The rounding error of P' averages out over the keys (it shrinks with
// the square root of the window length), so only short windows need PLO.  The
// rounding error of Q moves every score of a row coherently and is amplified
// by large K channels: short windows always carry QLO, longer ones when the
// cache was created for two query terms (keys with outlier channels).
template <int D, bool MASK, bool QLO, bool PLO, bool STAT>
__global__ __launch_bounds__(kThreads, RTV_ATTEND_WG_PER_CU) void attend_kernel(AttendArgs a) {
  static_assert(!(STAT && PLO), "the peaked-row check serves the one-code kernels");
  if (a.redo && a.flags[a.n_work] == 0u) return;      // no unit flagged
  if (a.dstate && !attend_derive(a)) return;
  using SM = Smem<D>;
  using LU = LogUnits<PLO>;
  constexpr int NSTEP = D / 64;             // MFMA k-steps for K.Q^T
  constexpr int NDT = D / 32;               // 32-row d sub-tiles of O^T
  constexpr int P = D / 4;                  // RoPE pairs per lane
  __shared__ __attribute__((aligned(16))) uint8_t smem[kStages * SM::STAGE];

  int unit, part;
  if (!work_item(a, unit, part)) return;
  if (a.redo && a.flags[unit] == 0u) return;
  const int head = unit / a.n_qtiles;
  const int qtile = unit % a.n_qtiles;
  const int kvh = head / a.group;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int hh = lane >> 5;
  const int li = lane & 31;

  const int64_t Sp = a.slots_padded;
  const uint8_t* kc = a.kc + (int64_t)kvh * Sp * D;
  const uint8_t* vc = a.vc + (int64_t)kvh * Sp * D;
  const uint8_t* frec = (const uint8_t*)a.fac_l + (int64_t)kvh * a.ring_tiles * 1024;
  const uint8_t* fu = a.fac_u + (int64_t)kvh * a.ring_tiles * 128;
  const int side = kStageJobs == 1 ? (__builtin_amdgcn_readfirstlane(tid) >= 256 ? 1 : 0) : -1;
  const int k_off = k_code_off<D>(tid & 255), v_off = v_code_off<D>(tid & 255);
  const int xk_off = (tid & 63) * 16, xv_off = (tid & 7) * 16;

  // ---- Q prologue: RoPE, the query's power-of-two scale, e4m3 codes in the
  // B-operand layout.  Operand step s, byte b <-> d: D=128: d = 64 s + 32 hh +
  // b; D=64: byte b < 16 -> d = 16 hh + b, b >= 16 -> d = 32 + 16 hh + b - 16
  // (RoPE pairs stay in-lane); lanes li and li + 32 hold one query
  int q_rows[kSub];
  int qexp[kSub];                           // E8M0 scale of the lane's query
  v8i qop[kSub][NSTEP];
  v8i qlo[kSub][NSTEP];
#pragma unroll
  for (int sub = 0; sub < kSub; ++sub) {
    const int row = qtile * kQPB + wave * kQPW + sub * 32 + li;
    q_rows[sub] = row;
    const int src_row = row < a.n_tokens ? row : a.n_tokens - 1;
    const uint16_t* q_src = a.q + (int64_t)src_row * a.ldq + (int64_t)head * D;
    const float* q_cs = a.rope + ((int64_t)src_row * (D / 2) + P * hh) * 2;
    float r0[P], r1[P];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < P; j += 8) {
      const uint4 w0 = *(const uint4*)(q_src + P * hh + j);
      const uint4 w1 = *(const uint4*)(q_src + D / 2 + P * hh + j);
      const uint32_t x0w[4] = {w0.x, w0.y, w0.z, w0.w};
      const uint32_t x1w[4] = {w1.x, w1.y, w1.z, w1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x0 = (e & 1) ? bf16_hi(x0w[e >> 1]) : bf16_lo(x0w[e >> 1]);
        const float x1 = (e & 1) ? bf16_hi(x1w[e >> 1]) : bf16_lo(x1w[e >> 1]);
        const float2 c = *(const float2*)(q_cs + 2 * (j + e));
        r0[j + e] = x0 * c.x - x1 * c.y;
        r1[j + e] = x1 * c.x + x0 * c.y;
        amax = __builtin_fmaxf(amax, __builtin_fmaxf(fabsf(r0[j + e]), fabsf(r1[j + e])));
      }
    }
    const int e = query_exp(xhalf_max(amax));
    qexp[sub] = 127 + e;
#pragma unroll
    for (int w = 0; w < NSTEP * 8; ++w) {
      float v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int b = 4 * w + k;
        const float x = (D == 128) ? ((b < 32) ? r0[b] : r1[b - 32]) : ((b < 16) ? r0[b] : r1[b - 16]);
        v[k] = __builtin_amdgcn_ldexpf(x, -e);   // exact
      }
      uint32_t c = 0, lo = 0;
      if constexpr (QLO) {
        split_fp8x2<false>(v[0], v[1], c, lo);
        split_fp8x2<true>(v[2], v[3], c, lo);
      } else {
        c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
        c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], (int)c, true);
      }
      qop[sub][w / 8][w % 8] = (int)c;
      qlo[sub][w / 8][w % 8] = (int)lo;
    }
  }

  // ---- tile schedule over the segments -------------------------------------
  const int lo0 = (int)a.seg_lo[0], hi0 = (int)a.seg_hi[0];
  const int lo1 = a.n_segments > 1 ? (int)a.seg_lo[1] : 0;
  const int hi1 = a.n_segments > 1 ? (int)a.seg_hi[1] : 0;
  const int t_first0 = (int)(lo0 / 64);
  const int t_count0 = hi0 > lo0 ? (int)((hi0 - 1) / 64) - t_first0 + 1 : 0;
  const int t_first1 = (int)(lo1 / 64);
  const int t_count1 = hi1 > lo1 ? (int)((hi1 - 1) / 64) - t_first1 + 1 : 0;
  const int n_all = t_count0 + t_count1;
  const int pidx = part < 0 ? 0 : part % a.parts_per_unit;
  const int pcount = part < 0 ? 1 : a.parts_per_unit;
  const int it_begin = (int)((int64_t)n_all * pidx / pcount);
  const int n_it = (int)((int64_t)n_all * (pidx + 1) / pcount) - it_begin;
  auto tref = [&](int it) {
    return tile_of(it_begin + it, t_count0, t_first0, t_first1, lo0, hi0, lo1, hi1);
  };
  auto clamp_it = [&](int it) { return it < n_it ? it : n_it - 1; };
  auto stage_of = [&](int it) { return smem + (it & (kStages - 1)) * SM::STAGE; };

  // S^T = K . Q^T + C of the tile in stage st: the K operands (shared by the
  // sub-tiles), the accumulator initial value C of the lane's 32 keys, and
  // product j (key half j % 2, k-step j / 2) of the 2 * NSTEP of one sub-tile
  auto load_kop = [&](const uint8_t* st, v8i (&kop)[2][NSTEP]) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const uint8_t* krow = st + (32 * kh + li) * SM::KROW;
#pragma unroll
      for (int s = 0; s < NSTEP; ++s) {
        uint4 k0, k1;
        if constexpr (D == 128) {
          k0 = *(const uint4*)(krow + 64 * s + 32 * hh);
          k1 = *(const uint4*)(krow + 64 * s + 32 * hh + 16);
        } else {
          k0 = *(const uint4*)(krow + 16 * hh);
          k1 = *(const uint4*)(krow + 32 + 16 * hh);
        }
        kop[kh][s] = v8i{(int)k0.x, (int)k0.y, (int)k0.z, (int)k0.w,
                         (int)k1.x, (int)k1.y, (int)k1.z, (int)k1.w};
      }
    }
  };
  auto load_c = [&](const uint8_t* st, v16f (&acc)[2]) {
    const float* cp = (const float*)(st + SM::KF_OFF) + 64;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 c4 = *(const float4*)(cp + 32 * kh + 8 * g + 4 * hh);
        acc[kh][4 * g + 0] = c4.x;
        acc[kh][4 * g + 1] = c4.y;
        acc[kh][4 * g + 2] = c4.z;
        acc[kh][4 * g + 3] = c4.w;
      }
  };
  auto qk_step = [&](int j, int sub, const v8i (&kop)[2][NSTEP], v16f (&acc)[2]) {
    const int kh = j & 1, s = j >> 1;
    acc[kh] = mfma_fp8_bscaled(kop[kh][s], qop[sub][s], acc[kh], qexp[sub]);
    if constexpr (QLO) acc[kh] = mfma_fp8_bscaled(kop[kh][s], qlo[sub][s], acc[kh], qexp[sub] - kLoShift);
  };
  // keys of tile it outside its segment: add -448 * 448 to their raw scores
  // with one MFMA per key half (A: -448 at one k position of a masked key row,
  // B: 448 at the same k position of every query column)
  auto mask_scores = [&](int it, v16f (&acc)[2]) {
    const TileRef tr = tref(it);
    const int base = tr.tile * 64;
    if (tr.lo > base || tr.hi < base + 64) {
      const v8i ones = v8i{hh == 0 ? 0x7E : 0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const int slot = base + 32 * kh + li;
        const bool masked = !(slot >= tr.lo && slot < tr.hi);
        const v8i bias = v8i{(hh == 0 && masked) ? 0xFE : 0, 0, 0, 0, 0, 0, 0, 0};
        acc[kh] = mfma_fp8(bias, ones, acc[kh]);
      }
    }
  };
  // O^T += V^T . P'^T with the V tile in stage st, and the row sum
  // L += U . P'^T: lanes of rows 0 and 1 read the U rows of the stage, the
  // others a zero row.  (P' of a tile carries rho relative to the tile's 2^e:
  // the V products scale it back by the E8M0 exponent ev = 127 + e.)
  v16f acc_o[kSub][NDT];
  v16f acc_l[kSub];
  v16f acc_g[kSub];                         // P' P'^T (peaked-row check)
#pragma unroll
  for (int sub = 0; sub < kSub; ++sub) {
#pragma unroll
    for (int d = 0; d < NDT; ++d) acc_o[sub][d] = v16f{};
    acc_l[sub] = v16f{};
    acc_g[sub] = v16f{};
  }
  const int u_off = SM::U_OFF + (li < 2 ? li : 2) * SM::VROW + 32 * hh;
  auto load_v = [&](const uint8_t* st, v8i (&vop)[NDT + 1]) {
#pragma unroll
    for (int d = 0; d <= NDT; ++d) {
      const uint8_t* vrow = d < NDT ? st + SM::K_BYTES + (32 * d + li) * SM::VROW + 32 * hh : st + u_off;
      const uint4 v0 = *(const uint4*)(vrow);
      const uint4 v1 = *(const uint4*)(vrow + 16);
      vop[d] = v8i{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w,
                   (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
    }
  };
  // product j of the NDT + 1 of one sub-tile: d sub-tile j, or the row sum (j = NDT)
  v8i pop[kSub], plo[kSub];
  auto pv_step = [&](int j, int sub, const v8i (&vop)[NDT + 1], int ev) {
    if (j < NDT) {
      acc_o[sub][j] = mfma_fp8_scaled(vop[j], pop[sub], acc_o[sub][j], 127, ev);
      if constexpr (PLO) acc_o[sub][j] = mfma_fp8_scaled(vop[j], plo[sub], acc_o[sub][j], 127, ev - kLoShift);
    } else {
      acc_l[sub] = mfma_fp8_scaled(vop[NDT], pop[sub], acc_l[sub], 127 + 2, 127);
      if constexpr (PLO) acc_l[sub] = mfma_fp8_scaled(vop[NDT], plo[sub], acc_l[sub], 127 + 2, 127 - kLoShift);
      if constexpr (STAT) acc_g[sub] = mfma_fp8(pop[sub], pop[sub], acc_g[sub]);
    }
  };

  // ---- prologue: tiles 0 and 1 staged, tile 2 in registers, the V and U
  // rows of the stage of tile -1 zeroed (the first iteration's products of the
  // previous tile then add nothing), the zero rows of the other stages; scores
  // of tile 0
  TileRegs regs;
  if (n_it > 0) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      load_tile<D>(regs, tref(clamp_it(p)), kc, vc, frec, fu, side, k_off, v_off, xk_off, xv_off);
      store_tile<D, MASK>(regs, tref(clamp_it(p)), stage_of(p), LU::kUnit, tid);
    }
    load_tile<D>(regs, tref(clamp_it(2)), kc, vc, frec, fu, side, k_off, v_off, xk_off, xv_off);
  }
  for (int i = tid; i < SM::V_BYTES / 16; i += kThreads)
    ((uint4*)(stage_of(-1) + SM::K_BYTES))[i] = make_uint4(0, 0, 0, 0);
  if (tid == 0) ((int*)(stage_of(-1) + SM::KF_OFF))[128] = 127;
  if (tid < (kStages - 1) * (SM::VROW / 16))
    ((uint4*)(smem + (tid / (SM::VROW / 16)) * SM::STAGE + SM::U_OFF + 2 * SM::VROW))[tid % (SM::VROW / 16)] =
        make_uint4(0, 0, 0, 0);
  __syncthreads();

  v16f acc_s[kSub][2];
  float m_run[kSub];
  {
    v8i kop[2][NSTEP];
    load_kop(stage_of(0), kop);
#pragma unroll
    for (int sub = 0; sub < kSub; ++sub) {
      load_c(stage_of(0), acc_s[sub]);
#pragma unroll
      for (int j = 0; j < 2 * NSTEP; ++j) qk_step(j, sub, kop, acc_s[sub]);
      if constexpr (MASK) mask_scores(0, acc_s[sub]);
      // running max: from the raw row max of tile 0, so that the first tile
      // leaves the same headroom as every rescale
      float t0[32];
      scores(acc_s[sub], (const float*)(stage_of(0) + SM::KF_OFF), hh, 0.0f, t0);
      m_run[sub] = xhalf_max(max32(t0)) - LU::kReset;
      pop[sub] = v8i{};
      plo[sub] = v8i{};
    }
  }

  // ---- main loop: iteration it computes the softmax of tile it while the
  // matrix cores take the PV product of tile it - 1 and the scores of tile
  // it + 1; the ring holds tiles it - 1 .. it + 2.  r = it mod 4 (a constant
  // after the unrolling below), so that every LDS address is a lane base plus
  // an immediate offset.
  auto tile_step = [&](const int it, const int r) __attribute__((always_inline)) {
    // (0) staging of tile it + 2 into the stage that tile it - 2 held (last
    // read before the previous barrier; first read of tile it + 2 after the
    // next one) and the loads of tile it + 3; at the top of the iteration so
    // that its latency overlaps the products.  Unconditional with the tile
    // index clamped: past the end the copy lands in a stage nobody reads again
    store_tile<D, MASK>(regs, tref(clamp_it(it + 2)), stage_of(r + 2), LU::kUnit, tid);
    load_tile<D>(regs, tref(clamp_it(it + 3)), kc, vc, frec, fu, side, k_off, v_off, xk_off, xv_off);

    // (1) the PV and row-sum products of tile it - 1, interleaved with the
    // scores of tile it: t = fma(S, kf, -m), a quarter (8 keys) per product
    const float* kf = (const float*)(stage_of(r) + SM::KF_OFF);
    float4 kf4[8];
#pragma unroll
    for (int w = 0; w < 8; ++w) kf4[w] = *(const float4*)(kf + 32 * (w >> 2) + 8 * (w & 3) + 4 * hh);
    v8i vop[NDT + 1];
    load_v(stage_of(r + 3), vop);
    const int ev = __builtin_amdgcn_readfirstlane(((const int*)(stage_of(r + 3) + SM::KF_OFF))[128]);
    float t[kSub][32];
#pragma unroll
    for (int c = 0; c < 4 || c <= NDT; ++c) {
#pragma unroll
      for (int sub = 0; sub < kSub; ++sub) {
        // vector work first: the operand reads of the product land meanwhile
        if (c < 4) {
#pragma unroll
          for (int w = 2 * c; w < 2 * c + 2; ++w) {
            const float kk[4] = {kf4[w].x, kf4[w].y, kf4[w].z, kf4[w].w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              t[sub][4 * w + e] = __builtin_fmaf(acc_s[sub][w >> 2][4 * (w & 3) + e], kk[e], -m_run[sub]);
          }
        }
        if (c <= NDT) pv_step(c, sub, vop, ev);
      }
      chunk_fence();
    }
#pragma unroll
    for (int sub = 0; sub < kSub; ++sub) {
      // (any lane over the bound triggers: no cross-half max needed here)
      const float mx = max32(t[sub]);
      lazy_rescale<NDT, LU, STAT>(mx, m_run[sub], acc_o[sub], acc_l[sub], acc_g[sub], t[sub]);
    }

    // (2) the score products of tile it + 1 (past the last tile they read a
    // stale stage and are unused), interleaved with P' of tile it; one
    // sub-tile after the other, so that few scores and products are live
    {
      v8i kop[2][NSTEP];
      load_kop(stage_of(r + 1), kop);
#pragma unroll
      for (int sub = 0; sub < kSub; ++sub) {
        load_c(stage_of(r + 1), acc_s[sub]);
#pragma unroll
        for (int c = 0; c < 4 || c < 2 * NSTEP; ++c) {
          if (c < 4) probs_quarter<PLO>(c, t[sub], pop[sub], plo[sub]);
          if (c < 2 * NSTEP) qk_step(c, sub, kop, acc_s[sub]);
          chunk_fence();
        }
        // keep the exponentials here rather than sunk past the staging
        // branches towards their use in the next iteration
        asm volatile("" ::"v"(pop[sub]));
        if constexpr (PLO) asm volatile("" ::"v"(plo[sub]));
        if constexpr (MASK) mask_scores(it + 1, acc_s[sub]);
      }
    }

    __syncthreads();
  };
  for (int it0 = 0; it0 < n_it; it0 += kStages) {
#pragma unroll
    for (int r = 0; r < kStages; ++r)
      if (it0 + r < n_it) tile_step(it0 + r, r);
  }
  {
    v8i vop[NDT + 1];
    load_v(stage_of(n_it - 1), vop);
    const int ev = __builtin_amdgcn_readfirstlane(((const int*)(stage_of(n_it - 1) + SM::KF_OFF))[128]);
#pragma unroll
    for (int sub = 0; sub < kSub; ++sub)
#pragma unroll
      for (int j = 0; j <= NDT; ++j) pv_step(j, sub, vop, ev);
  }

  // ---- epilogue ----------------------------------------------------------------
#pragma unroll
  for (int sub = 0; sub < kSub; ++sub) {
    // row sum: rows 0 and 1 of L (registers 0 and 1 of the lanes hh = 0; the
    // same registers of the lanes hh = 1 hold the zero rows 4 and 5)
    const float l_tot = xhalf_sum(acc_l[sub][0] + acc_l[sub][1]);
    const float g = STAT ? gram_diag(acc_g[sub], li, hh) : 0.0f;
    write_result<D, LU>(a, acc_o[sub], l_tot, m_run[sub], g, part, wave * kQPW + sub * 32 + li, q_rows[sub], head,
                        hh);
    if constexpr (STAT)
      if (part < 0 && __any(g > kPeakedGram * l_tot * l_tot) && lane == 0) flag_unit(a, unit);
  }
}

// ---- head dim 128: scores by v_mfma_f32_16x16x128_f8f6f4 -------------------
// The computation of attend_kernel (which serves head dim 64), with the score
// products taken 16 keys x 16 queries at a time over the whole head dimension.  Lane (q4 =
// lane / 16, i = lane % 16) then holds, for each of the tile's four 16-key
// blocks kb and the wave's two 16-query blocks qb, the scores of keys
// key16(kb, 4 q4 + e) (e = 0..3) for query 16 qb + i: 16 keys x 2 queries,
// against 32 keys x 1 query with the 32x32x64 product, so that a lane reads
// half as many per-key factors (kf, C) from LDS.  One v_permlane16_swap per
// pair of P' dwords (query blocks 0 and 1 of one key block) then gives every
// lane the 32 codes of one query in the B-operand order of the PV product:
// key16 maps (block, row) to keys so that code byte p of a lane holds the key
// that the transposed V rows keep at position p.  The running max is kept per
// query block; its rare updates reduce over the four lanes of a query.
__device__ __forceinline__ int key16(int kb, int r) { return vt_key(16 * (r >> 2) + 4 * kb + (r & 3)); }

// max over the four lanes i, i + 16, i + 32, i + 48 (the lanes of one query)
__device__ __forceinline__ float quad_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// max of the 16 scores of one query block
__device__ __forceinline__ float max16(const float (&t)[4][4]) {
  float a[6];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int j = 3 * i;
    a[i] = __builtin_fmaxf(__builtin_fmaxf(t[j >> 2][j & 3], t[(j + 1) >> 2][(j + 1) & 3]), t[(j + 2) >> 2][(j + 2) & 3]);
  }
  a[5] = t[3][3];
  return __builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(a[0], a[1]), a[2]),
                         __builtin_fmaxf(__builtin_fmaxf(a[3], a[4]), a[5]));
}

template <bool MASK, bool QLO, bool PLO, bool STAT>
__global__ __launch_bounds__(kThreads, RTV_ATTEND_WG_PER_CU) void attend16_kernel(AttendArgs a) {
  static_assert(kSub == 1, "one 32-query sub-tile per wave");
  static_assert(!(STAT && PLO), "the peaked-row check serves the one-code kernels");
  constexpr int D = 128;
  if (a.redo && a.flags[a.n_work] == 0u) return;      // no unit flagged
  if (a.dstate && !attend_derive(a)) return;
  using SM = Smem<D>;
  using LU = LogUnits<PLO>;
  constexpr int NDT = D / 32;               // 32-row d sub-tiles of O^T
  constexpr int P = D / 4;                  // RoPE pairs per lane
  __shared__ __attribute__((aligned(16))) uint8_t smem[kStages * SM::STAGE];

  int unit, part;
  if (!work_item(a, unit, part)) return;
  if (a.redo && a.flags[unit] == 0u) return;
  const int head = unit / a.n_qtiles;
  const int qtile = unit % a.n_qtiles;
  const int kvh = head / a.group;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int hh = lane >> 5;
  const int li = lane & 31;
  const int q4 = lane >> 4;
  const int i16 = lane & 15;

  const int64_t Sp = a.slots_padded;
  const uint8_t* kc = a.kc + (int64_t)kvh * Sp * D;
  const uint8_t* vc = a.vc + (int64_t)kvh * Sp * D;
  const uint8_t* frec = (const uint8_t*)a.fac_l + (int64_t)kvh * a.ring_tiles * 1024;
  const uint8_t* fu = a.fac_u + (int64_t)kvh * a.ring_tiles * 128;
  const int side = kStageJobs == 1 ? (__builtin_amdgcn_readfirstlane(tid) >= 256 ? 1 : 0) : -1;
  const int k_off = k_code_off<D>(tid & 255), v_off = v_code_off<D>(tid & 255);
  const int xk_off = (tid & 63) * 16, xv_off = (tid & 7) * 16;

  // ---- Q prologue: RoPE, each query's power-of-two scale (over the four
  // lanes that hold it) and e4m3 codes in the 16x16x128 B-operand layout:
  // lane (q4, i), query block qb: query 16 qb + i, byte b <-> d = 32 q4 + b
  // (q4 & 1 selects the RoPE pair block, q4 >> 1 the half of the pair)
  const int wrow = qtile * kQPB + wave * kQPW;  // first query row of the wave
  v8i qop[2], qlo[2];
  int qexp[2];                              // E8M0 scale of the lane's query of block qb
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = wrow + 16 * qb + i16;
    const int src_row = row < a.n_tokens ? row : a.n_tokens - 1;
    const int pb = q4 & 1;
    const bool upper = q4 >= 2;
    const uint16_t* q_src = a.q + (int64_t)src_row * a.ldq + (int64_t)head * D;
    const float* q_cs = a.rope + ((int64_t)src_row * (D / 2) + P * pb) * 2;
    float v[P];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < P; j += 8) {
      const uint4 w0 = *(const uint4*)(q_src + P * pb + j);
      const uint4 w1 = *(const uint4*)(q_src + D / 2 + P * pb + j);
      const uint32_t x0w[4] = {w0.x, w0.y, w0.z, w0.w};
      const uint32_t x1w[4] = {w1.x, w1.y, w1.z, w1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x0 = (e & 1) ? bf16_hi(x0w[e >> 1]) : bf16_lo(x0w[e >> 1]);
        const float x1 = (e & 1) ? bf16_hi(x1w[e >> 1]) : bf16_lo(x1w[e >> 1]);
        const float2 c = *(const float2*)(q_cs + 2 * (j + e));
        const float r0 = x0 * c.x - x1 * c.y;
        const float r1 = x1 * c.x + x0 * c.y;
        v[j + e] = upper ? r1 : r0;
        amax = __builtin_fmaxf(amax, fabsf(v[j + e]));
      }
    }
    const int e = query_exp(quad_max(amax));
    qexp[qb] = 127 + e;
#pragma unroll
    for (int j = 0; j < P; ++j) v[j] = __builtin_amdgcn_ldexpf(v[j], -e);   // exact
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      uint32_t c = 0, lo = 0;
      if constexpr (QLO) {
        split_fp8x2<false>(v[4 * w], v[4 * w + 1], c, lo);
        split_fp8x2<true>(v[4 * w + 2], v[4 * w + 3], c, lo);
      } else {
        c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[4 * w], v[4 * w + 1], 0, false);
        c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[4 * w + 2], v[4 * w + 3], (int)c, true);
      }
      qop[qb][w] = (int)c;
      qlo[qb][w] = (int)lo;
    }
  }

  // ---- tile schedule over the segments -------------------------------------
  const int lo0 = (int)a.seg_lo[0], hi0 = (int)a.seg_hi[0];
  const int lo1 = a.n_segments > 1 ? (int)a.seg_lo[1] : 0;
  const int hi1 = a.n_segments > 1 ? (int)a.seg_hi[1] : 0;
  const int t_first0 = (int)(lo0 / 64);
  const int t_count0 = hi0 > lo0 ? (int)((hi0 - 1) / 64) - t_first0 + 1 : 0;
  const int t_first1 = (int)(lo1 / 64);
  const int t_count1 = hi1 > lo1 ? (int)((hi1 - 1) / 64) - t_first1 + 1 : 0;
  const int n_all = t_count0 + t_count1;
  const int pidx = part < 0 ? 0 : part % a.parts_per_unit;
  const int pcount = part < 0 ? 1 : a.parts_per_unit;
  const int it_begin = (int)((int64_t)n_all * pidx / pcount);
  const int n_it = (int)((int64_t)n_all * (pidx + 1) / pcount) - it_begin;
  auto tref = [&](int it) {
    return tile_of(it_begin + it, t_count0, t_first0, t_first1, lo0, hi0, lo1, hi1);
  };
  auto clamp_it = [&](int it) { return it < n_it ? it : n_it - 1; };
  auto stage_of = [&](int it) { return smem + (it & (kStages - 1)) * SM::STAGE; };

  // Key rows of the lane's A operands: key16(kb, i) = row16 + 8 kb; factor
  // records of the lane's keys key16(kb, 4 q4 + e) = frow + 8 kb + e.  (A
  // quarter wave reads rows {8 kb + j} and {32 + 8 kb + j}, two to a bank
  // group in the padded rows; swizzling the upper rows apart measured no
  // faster.)
  const int row16 = key16(0, i16);          // = 32 ((i16 >> 2) & 1) + 4 (i16 >> 3) + (i16 & 3)
  const int frow = key16(0, 4 * q4);        // = 32 (q4 & 1) + 4 (q4 >> 1)
  auto load_kop = [&](const uint8_t* st, v8i (&kop)[4]) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const uint8_t* krow = st + (row16 + 8 * kb) * SM::KROW + 32 * q4;
      const uint4 k0 = *(const uint4*)(krow);
      const uint4 k1 = *(const uint4*)(krow + 16);
      kop[kb] = v8i{(int)k0.x, (int)k0.y, (int)k0.z, (int)k0.w, (int)k1.x, (int)k1.y, (int)k1.z, (int)k1.w};
    }
  };
  auto load_c = [&](const uint8_t* st, v4f (&cin)[4]) {
    const float* cp = (const float*)(st + SM::KF_OFF) + 64 + frow;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const float4 c4 = *(const float4*)(cp + 8 * kb);
      cin[kb] = v4f{c4.x, c4.y, c4.z, c4.w};
    }
  };
  // S = K . Q^T + C of key block kb for both query blocks
  auto qk_step = [&](int kb, const v8i (&kop)[4], const v4f (&cin)[4], v4f (&acc)[4][2]) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      acc[kb][qb] = mfma16_fp8_bscaled(kop[kb], qop[qb], cin[kb], qexp[qb]);
      if constexpr (QLO) acc[kb][qb] = mfma16_fp8_bscaled(kop[kb], qlo[qb], acc[kb][qb], qexp[qb] - kLoShift);
    }
  };
  // keys of tile it outside its segment: add -448 * 448 to their raw scores
  // (A: -448 at k = 0 of a masked key row, B: 448 at k = 0 of every query)
  auto mask_scores = [&](int it, v4f (&acc)[4][2]) {
    const TileRef tr = tref(it);
    const int base = tr.tile * 64;
    if (tr.lo > base || tr.hi < base + 64) {
      const v8i ones = v8i{q4 == 0 ? 0x7E : 0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int slot = base + row16 + 8 * kb;
        const bool masked = !(slot >= tr.lo && slot < tr.hi);
        const v8i bias = v8i{(q4 == 0 && masked) ? 0xFE : 0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) acc[kb][qb] = mfma16_fp8(bias, ones, acc[kb][qb]);
      }
    }
  };
  // O^T += V^T . P'^T as in attend_kernel.  The row sum is one 16x16x128
  // product with the same B operand read in that product's layout: lane
  // (q4, i) holds the codes of query 16 (q4 & 1) + i for the keys of half
  // q4 >> 1, so column i sums queries i (k-blocks 0, 2) and 16 + i (k-blocks
  // 1, 3).  A rows 0 / 2 carry U_hi / U_lo on k-blocks 0 and 2, rows 1 / 3 on
  // k-blocks 1 and 3 (every other lane reads the zero row), and lane (0, i)
  // accumulates (L_hi(i), L_hi(16 + i), L_lo(i), L_lo(16 + i)).
  v16f acc_o[NDT];
  v4f acc_l = v4f{};
  v16f acc_g = v16f{};                      // P' P'^T (peaked-row check)
#pragma unroll
  for (int d = 0; d < NDT; ++d) acc_o[d] = v16f{};
  const int u_off = SM::U_OFF + ((i16 < 4 && (i16 & 1) == (q4 & 1)) ? (i16 >> 1) : 2) * SM::VROW + 32 * (q4 >> 1);
  auto load_v = [&](const uint8_t* st, v8i (&vop)[NDT + 1]) {
#pragma unroll
    for (int d = 0; d <= NDT; ++d) {
      const uint8_t* vrow = d < NDT ? st + SM::K_BYTES + (32 * d + li) * SM::VROW + 32 * hh : st + u_off;
      const uint4 v0 = *(const uint4*)(vrow);
      const uint4 v1 = *(const uint4*)(vrow + 16);
      vop[d] = v8i{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w, (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
    }
  };
  v8i pop = v8i{}, plo = v8i{};
  auto pv_step = [&](int j, const v8i (&vop)[NDT + 1], int ev) {
    if (j < NDT) {
      acc_o[j] = mfma_fp8_scaled(vop[j], pop, acc_o[j], 127, ev);
      if constexpr (PLO) acc_o[j] = mfma_fp8_scaled(vop[j], plo, acc_o[j], 127, ev - kLoShift);
    } else {
      acc_l = mfma16_fp8_scaled(vop[NDT], pop, acc_l, 127 + 2, 127);
      if constexpr (PLO) acc_l = mfma16_fp8_scaled(vop[NDT], plo, acc_l, 127 + 2, 127 - kLoShift);
      if constexpr (STAT) acc_g = mfma_fp8(pop, pop, acc_g);
    }
  };
  // P' of key block kb (chunk kb of the second half): codes of both query
  // blocks, then the swap into the PV operand (dwords kb and 4 + kb)
  auto probs_block = [&](int kb, const float (&t)[2][4][4]) {
    uint32_t hi2[2], lo2[2] = {0u, 0u};
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      if constexpr (PLO) {
        float pp[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pp[e] = __builtin_amdgcn_exp2f(t[qb][kb][e]);
        uint32_t h = 0, l = 0;
        split_fp8x2<false>(pp[0], pp[1], h, l);
        split_fp8x2<true>(pp[2], pp[3], h, l);
        hi2[qb] = h;
        lo2[qb] = l;
      } else {
        uint32_t x = __builtin_amdgcn_cvt_pk_u8_f32(t[qb][kb][0], 0, __float_as_uint(t[qb][kb][0]));
        x = __builtin_amdgcn_cvt_pk_u8_f32(t[qb][kb][1], 1, x);
        x = __builtin_amdgcn_cvt_pk_u8_f32(t[qb][kb][2], 2, x);
        x = __builtin_amdgcn_cvt_pk_u8_f32(t[qb][kb][3], 3, x);
        hi2[qb] = x;
      }
    }
    const auto s = __builtin_amdgcn_permlane16_swap(hi2[0], hi2[1], false, false);
    pop[kb] = (int)s[0];
    pop[4 + kb] = (int)s[1];
    if constexpr (PLO) {
      const auto sl = __builtin_amdgcn_permlane16_swap(lo2[0], lo2[1], false, false);
      plo[kb] = (int)sl[0];
      plo[4 + kb] = (int)sl[1];
    }
  };

  // ---- prologue: as in attend_kernel ----------------------------------------
  TileRegs regs;
  if (n_it > 0) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      load_tile<D>(regs, tref(clamp_it(p)), kc, vc, frec, fu, side, k_off, v_off, xk_off, xv_off);
      store_tile<D, MASK>(regs, tref(clamp_it(p)), stage_of(p), LU::kUnit, tid);
    }
    load_tile<D>(regs, tref(clamp_it(2)), kc, vc, frec, fu, side, k_off, v_off, xk_off, xv_off);
  }
  for (int i = tid; i < SM::V_BYTES / 16; i += kThreads)
    ((uint4*)(stage_of(-1) + SM::K_BYTES))[i] = make_uint4(0, 0, 0, 0);
  if (tid == 0) ((int*)(stage_of(-1) + SM::KF_OFF))[128] = 127;
  if (tid < (kStages - 1) * (SM::VROW / 16))
    ((uint4*)(smem + (tid / (SM::VROW / 16)) * SM::STAGE + SM::U_OFF + 2 * SM::VROW))[tid % (SM::VROW / 16)] =
        make_uint4(0, 0, 0, 0);
  __syncthreads();

  v4f acc_s[4][2];
  float m_run[2];
  {
    v8i kop[4];
    v4f cin[4];
    load_kop(stage_of(0), kop);
    load_c(stage_of(0), cin);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) qk_step(kb, kop, cin, acc_s);
    if constexpr (MASK) mask_scores(0, acc_s);
    const float* kf = (const float*)(stage_of(0) + SM::KF_OFF) + frow;
    float t0[2][4][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const float4 k4 = *(const float4*)(kf + 8 * kb);
      const float kk[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int e = 0; e < 4; ++e) t0[qb][kb][e] = acc_s[kb][qb][e] * kk[e];
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) m_run[qb] = quad_max(max16(t0[qb])) - LU::kReset;
  }

  auto tile_step = [&](const int it, const int r) __attribute__((always_inline)) {
    // (0) staging of tile it + 2 and the loads of tile it + 3 (as in attend_kernel)
    store_tile<D, MASK>(regs, tref(clamp_it(it + 2)), stage_of(r + 2), LU::kUnit, tid);
    load_tile<D>(regs, tref(clamp_it(it + 3)), kc, vc, frec, fu, side, k_off, v_off, xk_off, xv_off);

    // (1) the PV and row-sum products of tile it - 1, interleaved with the
    // scores of tile it: t = fma(S, kf, -m), one key block (8 scores) per product
    const float* kf = (const float*)(stage_of(r) + SM::KF_OFF) + frow;
    float4 kf4[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) kf4[kb] = *(const float4*)(kf + 8 * kb);
    v8i vop[NDT + 1];
    load_v(stage_of(r + 3), vop);
    const int ev = __builtin_amdgcn_readfirstlane(((const int*)(stage_of(r + 3) + SM::KF_OFF))[128]);
    float t[2][4][4];
#pragma unroll
    for (int c = 0; c <= NDT; ++c) {
      if (c < 4) {
        const float kk[4] = {kf4[c].x, kf4[c].y, kf4[c].z, kf4[c].w};
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int e = 0; e < 4; ++e) t[qb][c][e] = __builtin_fmaf(acc_s[c][qb][e], kk[e], -m_run[qb]);
      }
      pv_step(c, vop, ev);
      chunk_fence();
    }
    {
      // lazy running max (rare): per query block, from the four lanes of each query
      float mx = 0.0f;
      {
        float flat[32];
#pragma unroll
        for (int j = 0; j < 32; ++j) flat[j] = t[j >> 4][(j >> 2) & 3][j & 3];
        mx = max32(flat);
      }
      if (__builtin_expect(__any(mx > LU::kTop), 0)) {
        float alpha[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const float raw = quad_max(max16(t[qb])) + m_run[qb];
          const float m_new = __builtin_fmaxf(m_run[qb], raw - LU::kReset);
          const float shift = m_run[qb] - m_new;
          alpha[qb] = exp2f(shift * (1.0f / LU::kUnit));
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e) t[qb][kb][e] += shift;
          m_run[qb] = m_new;
        }
        // the PV accumulators hold query 16 (q4 & 1) + i in lane (q4, i)
        const float al = (q4 & 1) ? alpha[1] : alpha[0];
#pragma unroll
        for (int d = 0; d < NDT; ++d) acc_o[d] *= al;
        acc_l *= v4f{alpha[0], alpha[1], alpha[0], alpha[1]};
        if constexpr (STAT) acc_g *= al * al;
      }
    }

    // (2) the score products of tile it + 1, interleaved with P' of tile it
    {
      v8i kop[4];
      v4f cin[4];
      load_kop(stage_of(r + 1), kop);
      load_c(stage_of(r + 1), cin);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        probs_block(c, t);
        qk_step(c, kop, cin, acc_s);
        chunk_fence();
      }
      asm volatile("" ::"v"(pop));
      if constexpr (PLO) asm volatile("" ::"v"(plo));
      if constexpr (MASK) mask_scores(it + 1, acc_s);
    }

    __syncthreads();
  };
  for (int it0 = 0; it0 < n_it; it0 += kStages) {
#pragma unroll
    for (int r = 0; r < kStages; ++r)
      if (it0 + r < n_it) tile_step(it0 + r, r);
  }
  {
    v8i vop[NDT + 1];
    load_v(stage_of(n_it - 1), vop);
    const int ev = __builtin_amdgcn_readfirstlane(((const int*)(stage_of(n_it - 1) + SM::KF_OFF))[128]);
#pragma unroll
    for (int j = 0; j <= NDT; ++j) pv_step(j, vop, ev);
  }

  // ---- epilogue (PV layout: lane (hh, li) holds query li, the query block q4 & 1)
  const float l_x = __shfl(acc_l[0] + acc_l[2], i16), l_y = __shfl(acc_l[1] + acc_l[3], i16);
  const float l_tot = li < 16 ? l_x : l_y;
  const float g = STAT ? gram_diag(acc_g, li, hh) : 0.0f;
  write_result<D, LU>(a, acc_o, l_tot, (q4 & 1) ? m_run[1] : m_run[0], g, part, wave * kQPW + li, wrow + li, head,
                      hh);
  if constexpr (STAT)
    if (part < 0 && __any(g > kPeakedGram * l_tot * l_tot) && lane == 0) flag_unit(a, unit);
}

// Merge the key-range parts of the split units: for each query,
// M = max_p m_p, w_p = 2^(m_p - M), O = sum_p w_p O_p / sum_p w_p l_p.
// With the peaked-row check the merged G = sum_p w_p^2 g_p against L^2 flags
// the unit.  One workgroup = kCombineQ queries of one split unit (blockIdx.x:
// the unit, blockIdx.y: the query group), kCombineT threads per query with D
// / kCombineT dimensions each: a query's partial rows are read as contiguous
// runs and the whole device takes part.
constexpr int kCombineQ = 16;
constexpr int kCombineT = 16;
template <int D>
__global__ __launch_bounds__(kCombineQ * kCombineT) void combine_kernel(AttendArgs a) {
  if (a.redo && a.flags[a.n_work] == 0u) return;      // no unit flagged
  if (a.dstate && !attend_derive(a)) return;
  constexpr int DT = D / kCombineT;               // dimensions per thread
  const int r = blockIdx.x;                       // split unit r
  if (a.n_full + r >= a.n_work) return;           // (device-state grids cover the most split units)
  const int unit = a.n_full + r;
  if (a.redo && a.flags[unit] == 0u) return;
  const int head = unit / a.n_qtiles;
  const int qtile = unit % a.n_qtiles;
  const int S = a.parts_per_unit;
  const int q = blockIdx.y * kCombineQ + (int)threadIdx.x / kCombineT;
  const int d0 = ((int)threadIdx.x % kCombineT) * DT;
  const int row = qtile * kQPB + q;
  if (row >= a.n_tokens) return;
  const int j0 = r * S;
  float M = -INFINITY;
  for (int p = 0; p < S; ++p) M = fmaxf(M, a.ws_ml[((int64_t)(j0 + p) * kQPB + q) * 4]);
  float L = 0.0f, G = 0.0f;
  float acc[DT];
#pragma unroll
  for (int d = 0; d < DT; ++d) acc[d] = 0.0f;
  for (int p = 0; p < S; ++p) {
    const float4 ml = *(const float4*)(a.ws_ml + ((int64_t)(j0 + p) * kQPB + q) * 4);
    const float w = exp2f(ml.x - M);
    L += w * ml.y;
    G += w * w * ml.z;
    const float* po = a.ws_o + ((int64_t)(j0 + p) * kQPB + q) * D + d0;
#pragma unroll
    for (int d = 0; d < DT; d += 4) {
      const float4 o = *(const float4*)(po + d);
      acc[d] += w * o.x; acc[d + 1] += w * o.y; acc[d + 2] += w * o.z; acc[d + 3] += w * o.w;
    }
  }
  if (a.check_peaked && !a.redo && d0 == 0 && G > kPeakedGram * L * L) flag_unit(a, unit);
  const float inv = 1.0f / L;
  uint16_t* dst = a.out + (int64_t)row * a.ldo + (int64_t)head * D + d0;
#pragma unroll
  for (int d = 0; d < DT; d += 4) {
    uint2 w;
    w.x = pack_bf16x2(acc[d] * inv, acc[d + 1] * inv);
    w.y = pack_bf16x2(acc[d + 2] * inv, acc[d + 3] * inv);
    *(uint2*)(dst + d) = w;
  }
}

}  // namespace

int attend_queries_per_block() { return kQPB; }

int attend_max_parts() { return kMaxParts; }
static size_t align256(size_t x) { return (x + 255) / 256 * 256; }
static size_t partials_bytes(int head_dim) {
  return align256((size_t)kMaxParts * kQPB * ((size_t)head_dim + 4) * sizeof(float));
}
size_t attend_workspace_bytes(int head_dim, int n_kv_heads, int64_t slots_padded, int64_t n_units) {
  const size_t tiles = (size_t)n_kv_heads * (size_t)(slots_padded / 64);
  return partials_bytes(head_dim) + align256(tiles * 64 * 16) + align256(tiles * 128) +
         align256(((size_t)n_units + 1) * sizeof(uint32_t));
}
void attend_set_workspace(AttendArgs& a, void* ws, int head_dim, int n_kv_heads, int64_t slots_padded,
                          int64_t n_units) {
  (void)n_units;
  uint8_t* p = static_cast<uint8_t*>(ws);
  const size_t tiles = (size_t)n_kv_heads * (size_t)(slots_padded / 64);
  a.ws_o = reinterpret_cast<float*>(p);
  a.ws_ml = a.ws_o + (size_t)kMaxParts * kQPB * head_dim;
  p += partials_bytes(head_dim);
  a.fac_l = reinterpret_cast<float*>(p);
  p += align256(tiles * 64 * 16);
  a.fac_u = p;
  p += align256(tiles * 128);
  a.flags = reinterpret_cast<uint32_t*>(p);
  a.n_kv_heads = n_kv_heads;
  a.ring_tiles = (int32_t)(slots_padded / 64);
}

hipError_t attend_capacity(int* workgroups) {
  int dev = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  hipDeviceProp_t prop;
  if (e == hipSuccess) e = hipGetDeviceProperties(&prop, dev);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attend16_kernel<false, false, false, true>, kThreads,
                                                     0);
  if (e != hipSuccess) return e;
  *workgroups = (per_cu > 0 ? per_cu : 1) * prop.multiProcessorCount;
  return hipSuccess;
}

namespace {

template <int D, bool MASK, bool QL, bool PL, bool ST>
void launch_one(const dim3& g, const dim3& b, const AttendArgs& a, hipStream_t s) {
  if constexpr (D == 128)
    hipLaunchKernelGGL((attend16_kernel<MASK, QL, PL, ST>), g, b, 0, s, a);
  else
    hipLaunchKernelGGL((attend_kernel<D, MASK, QL, PL, ST>), g, b, 0, s, a);
}

// the attention kernel variant: two-term Q and P' (precise), two-term Q with
// one-code P', or one-term Q with one-code P'; the one-code variants with or
// without the peaked-row check
template <int D, bool MASK>
void launch_variant(bool precise, bool two_term_q, bool check, const dim3& g, const dim3& b, const AttendArgs& a,
                    hipStream_t s) {
  if (precise)
    launch_one<D, MASK, true, true, false>(g, b, a, s);
  else if (two_term_q)
    check ? launch_one<D, MASK, true, false, true>(g, b, a, s) : launch_one<D, MASK, true, false, false>(g, b, a, s);
  else
    check ? launch_one<D, MASK, false, false, true>(g, b, a, s) : launch_one<D, MASK, false, false, false>(g, b, a, s);
}

template <int D>
hipError_t launch_attend_d(const AttendArgs& args_in, hipStream_t stream) {
  AttendArgs args = args_in;
  bool aligned = true, short_window = false;
  int n_tiles = 0, grid_per_xcd = 0, rem = 0;
  if (!args.dstate) {
    int64_t keys = 0;
    for (int s = 0; s < args.n_segments; ++s) {
      aligned = aligned && args.seg_lo[s] % 64 == 0 && args.seg_hi[s] % 64 == 0;
      keys += args.seg_hi[s] - args.seg_lo[s];
    }
    n_tiles = attend_window_tiles(args);
    short_window = keys < kPreciseKeys;
    attend_schedule(args, n_tiles, kMaxParts);
    grid_per_xcd = args.full_per_xcd + args.parts_per_xcd;
    rem = args.n_work - args.n_full;
  } else {
    // Device-state mode: the kernels derive the window and the schedule, so
    // the variant and the grids are fixed by the ring's shape.  Every window
    // holds at least one chunk and starts on a chunk boundary when the cap
    // is a multiple of the chunk; the grids cover the largest window.  With
    // unchecked one-code weights the variant follows the shortest window (one
    // chunk): a ring whose chunk is under 8192 keys takes the two-term kernel
    // on every window.
    const RingShape& sh = args.shape;
    const int64_t chunk = (int64_t)sh.chunk_frames * sh.tokens_per_frame;
    aligned = chunk % 64 == 0 && sh.max_window_frames % sh.chunk_frames == 0;
    short_window = chunk < kPreciseKeys;
    n_tiles = (int)(((int64_t)sh.capacity_frames * sh.tokens_per_frame + 63) / 64) + 1;
    AttendArgs whole = args, most = args;
    attend_schedule(whole, 1, kMaxParts);
    attend_schedule(most, n_tiles, kMaxParts);
    const int g1 = whole.full_per_xcd + whole.parts_per_xcd, g2 = most.full_per_xcd + most.parts_per_xcd;
    grid_per_xcd = g1 > g2 ? g1 : g2;
    rem = most.n_work - most.n_full;
  }
  // prob_terms 2: two terms everywhere; 0 (checked): the one-code kernel and
  // its check on every window, in both modes alike (short windows are usually
  // flagged and recomputed); 1 (unchecked): two terms below 8192 keys
  const bool check = args.check_peaked && !args.two_term_p;
  const bool precise = args.two_term_p || (!check && short_window);
  const bool two_term_q = precise || args.two_term_q;
  args.check_peaked = check ? 1 : 0;
  args.redo = 0;
  {
    const int waves = n_tiles * args.n_kv_heads;
    if (waves > 0) hipLaunchKernelGGL(factors_kernel<D>, dim3((waves + 3) / 4), dim3(256), 0, stream, args);
  }
  const dim3 g(8 * grid_per_xcd), b(kThreads);
  if (aligned)
    launch_variant<D, false>(precise, two_term_q, check, g, b, args, stream);
  else
    launch_variant<D, true>(precise, two_term_q, check, g, b, args, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 cg(rem, kQPB / kCombineQ), cb(kCombineQ * kCombineT);
  if (rem > 0) {
    hipLaunchKernelGGL(combine_kernel<D>, cg, cb, 0, stream, args);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (!check) return hipSuccess;
  // recompute the units flagged as peaked with two-term Q and P' (every
  // workgroup of these launches exits at once when none is flagged)
  AttendArgs redo = args;
  redo.redo = 1;
  if (aligned)
    launch_one<D, false, true, true, false>(g, b, redo, stream);
  else
    launch_one<D, true, true, true, false>(g, b, redo, stream);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (rem > 0) {
    hipLaunchKernelGGL(combine_kernel<D>, cg, cb, 0, stream, redo);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

hipError_t launch_attend(const AttendArgs& args, int head_dim, hipStream_t stream) {
  return head_dim == 128 ? launch_attend_d<128>(args, stream) : launch_attend_d<64>(args, stream);
}

}  // namespace rtv
