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
// window's (at most two) slot segments through a 3-stage LDS ring with one
// barrier per tile; waves 0-3 stage the K rows and waves 4-7 the V rows of
// tile t+2 while tile t is computed.
//
// Per wave, tile and sub-tile, with v_mfma_f32_32x32x64_f8f6f4 (e4m3, f32 acc):
//   S^T[key][query] = K . Q^T            2 key halves x D/64 k-steps
//   lane (hh, i) holds query i and 32 of the 64 keys: the softmax row is
//   per lane plus one v_permlane32_swap with lane i^32;
//   P' = p * w_key, w_key = sv_key * c, converted to e4m3, is the B operand of
//   O^T[d][query] += V^T . P'^T          D/32 d sub-tiles.
// Scores: the queries of a workgroup share one e4m3 scale s_q, so the whole
// per-score scale folds into a per-key factor kf = sk * s_q * log2(e)/sqrt(D)
// and t - m = fma(S_raw, kf, -m) is one instruction.  The running max m is
// lazy: it moves only when a tile's max exceeds it by more than kTau (log2
// units), so p <= 2^kTau, and c = kPmax / (2^kTau * max sv over the window)
// keeps P' below 448 with one constant for the whole window.
// Output O = acc / (c * l), rounded to bf16.
#include "device_common.hpp"
#include "kernels.hpp"

namespace rtv {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

#ifndef RTV_ATTEND_WAVES
#define RTV_ATTEND_WAVES 8
#endif
#ifndef RTV_ATTEND_SCHED
#define RTV_ATTEND_SCHED 0
#endif
#ifndef RTV_ATTEND_WG_PER_CU
#define RTV_ATTEND_WG_PER_CU 1
#endif
constexpr int kWaves = RTV_ATTEND_WAVES;
constexpr int kThreads = kWaves * kWave;
constexpr int kQPW = 32;                    // queries per wave
constexpr int kQPB = kWaves * kQPW;         // queries per workgroup
constexpr int kStages = 4;                  // LDS ring: tiles it - 1 .. it + 2
constexpr float kTau = 3.0f;
constexpr float kPmax = 440.0f;             // bound on P' (below the e4m3 max 448)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kMaskFactor = 1e30f;        // kf of a key outside the window segment

__device__ __forceinline__ v16f mfma_fp8(const v8i& a, const v8i& b, const v16f& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// the same with the B operand scaled by 2^(e - 127) (E8M0 exponent e):
// adds the low-order e4m3 part of a two-term operand
__device__ __forceinline__ v16f mfma_fp8_bscaled(const v8i& a, const v8i& b, const v16f& c, int e) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, e);
}

// two-term e4m3 of two values: hi = e4m3(x), lo = e4m3((x - hi) * 2^kLoShift)
// (|x - hi| <= 2^-4 |x|, so the scaled residual stays in range)
constexpr int kLoShift = 4;
// windows shorter than this many keys also carry P' as two terms (PLO)
constexpr int64_t kPreciseKeys = 8192;
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
  static constexpr int V_BYTES = D * VROW;
  static constexpr int STAGE = K_BYTES + V_BYTES + 2 * 64 * 4;   // + kf, wf
};

// Staged tile: with 512 threads, threads 0..255 (waves 0-3) move the K rows
// and kf, threads 256..511 (waves 4-7) the transposed V rows and wf; with
// 256 threads every thread moves a K piece and a V piece.  D/4 bytes each.
constexpr int kStageJobs = kThreads >= 512 ? 1 : 2;
struct TileRegs {
  uint4 c[kStageJobs][2];
  float s[kStageJobs];
};

struct TileRef {
  int tile;
  int lo, hi;         // the segment the tile belongs to (slot indices fit in int32)
};

template <int D>
__device__ __forceinline__ void load_tile(TileRegs& r, const TileRef& t, const uint8_t* kc,
                                          const uint8_t* vc, const float* ks, const float* vs,
                                          int tid) {
  constexpr int LD_BYTES = D / 4;
  const int gt = tid & 255;
#pragma unroll
  for (int j = 0; j < kStageJobs; ++j) {
    const bool isv = kStageJobs == 1 ? tid >= 256 : j == 1;
    const uint8_t* src = (isv ? vc : kc) + (int64_t)t.tile * 64 * D + gt * LD_BYTES;
    r.c[j][0] = *(const uint4*)(src);
    if constexpr (LD_BYTES == 32) r.c[j][1] = *(const uint4*)(src + 16);
    // every thread loads a scale (only 64 per job are used): no lane branch
    r.s[j] = (isv ? vs : ks)[(int64_t)t.tile * 64 + (gt & 63)];
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

// kscale = s_q * log2(e) / sqrt(D); wscale = c.  Branch-free apart from the
// masking of partial tiles: K and V pieces differ only in their address, and
// every thread writes the kf or wf entry of key (thread & 63); the threads
// that share a key hold the same scale and write the same value.
template <int D, bool MASK>
__device__ __forceinline__ void store_tile(const TileRegs& r, const TileRef& t, uint8_t* st,
                                           float kscale, float wscale, int tid) {
  using SM = Smem<D>;
  constexpr int LD_BYTES = D / 4;
  const int gt = tid & 255;
  const int base = t.tile * 64;
  const bool partial = MASK && (t.lo > base || t.hi < base + 64);
  const int b = gt * LD_BYTES;
  float* kf = (float*)(st + SM::K_BYTES + SM::V_BYTES);
  const int key = gt & 63;
  const bool ok = !MASK || (base + key >= t.lo && base + key < t.hi);
#pragma unroll
  for (int j = 0; j < kStageJobs; ++j) {
    const bool isv = kStageJobs == 1 ? tid >= 256 : j == 1;
#pragma unroll
    for (int h = 0; h < LD_BYTES / 16; ++h) {
      const int bb = b + 16 * h;
      uint4 q = r.c[j][h];
      if (partial) q = isv ? mask_v_piece(q, bb, base, t.lo, t.hi) : mask_k_piece<D>(q, bb, base, t.lo, t.hi);
      *(uint4*)(st + (isv ? v_piece_at<D>(bb) : k_piece_at<D>(bb))) = q;
    }
    // a key outside the segment gets kf = kMaskFactor: its raw score is the
    // bias -448*448 added by the masking MFMA, so t ~ -2e35 and p = 0
    const float kv = ok ? r.s[j] * kscale : kMaskFactor;
    const float wv = ok ? r.s[j] * wscale : 0.0f;
    kf[(isv ? 64 : 0) + key] = isv ? wv : kv;
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

// Softmax of one 32-query tile over one 64-key tile, first half: t = score - m
// for the lane's 32 keys, with the lazy running-max update (rare: rescales l
// and the O accumulator).
template <int NDT>
__device__ __forceinline__ void softmax_scores(const v16f (&s)[2], const float* kf, int hh, float& m,
                                               float& l, v16f (&o)[NDT], float (&t)[32]) {
  scores(s, kf, hh, m, t);
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < 32; j += 2) mx = __builtin_fmaxf(mx, __builtin_fmaxf(t[j], t[j + 1]));
  mx = xhalf_max(mx);
  // lazy rescale: only when the tile max exceeds the reference by > kTau
  // (always on the first tile, where m = -inf makes every t = +inf)
  if (__builtin_expect(__any(mx > kTau), 0)) {
    scores(s, kf, hh, 0.0f, t);   // raw scaled scores
    float raw = -INFINITY;
#pragma unroll
    for (int j = 0; j < 32; ++j) raw = __builtin_fmaxf(raw, t[j]);
    raw = xhalf_max(raw);
    const float m_new = __builtin_fmaxf(m, raw);
    const float alpha = exp2f(m - m_new);           // 0 on the first tile (m = -inf)
    l *= alpha;
#pragma unroll
    for (int d = 0; d < NDT; ++d) o[d] *= alpha;
#pragma unroll
    for (int j = 0; j < 32; ++j) t[j] -= m_new;
    m = m_new;
  }
}

// Second half: p = 2^t, l += p, and the e4m3 P' = p * w_key, the B operand of
// the PV product (PRECISE: as two terms).
template <bool PRECISE>
__device__ __forceinline__ v8i softmax_probs(const float (&t)[32], const float* wf, int hh, float& l,
                                             v8i& plo) {
  v8i pop;
  uint32_t prev = 0;
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int key0 = 32 * kh + 8 * g + 4 * hh;
      const float4 w4 = *(const float4*)(wf + key0);
      const float ww[4] = {w4.x, w4.y, w4.z, w4.w};
      float pp[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = __builtin_amdgcn_exp2f(t[16 * kh + 4 * g + e]);
        l += p;
        pp[e] = p * ww[e];
      }
      if constexpr (PRECISE) {
        uint32_t c = 0, lo = 0;
        split_fp8x2<false>(pp[0], pp[1], c, lo);
        split_fp8x2<true>(pp[2], pp[3], c, lo);
        pop[4 * kh + g] = (int)c;
        plo[4 * kh + g] = (int)lo;
      } else {
        uint32_t c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(pp[0], pp[1], (int)prev, false);
        c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(pp[2], pp[3], (int)c, true);
        pop[4 * kh + g] = (int)c;
        prev = c;
      }
    }
  return pop;
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
template <int D, bool MASK, bool QLO, bool PLO>
__global__ __launch_bounds__(kThreads, RTV_ATTEND_WG_PER_CU) void attend_kernel(AttendArgs a) {
  using SM = Smem<D>;
  constexpr int NSTEP = D / 64;             // MFMA k-steps for K.Q^T
  constexpr int NDT = D / 32;               // 32-row d sub-tiles of O^T
  constexpr int P = D / 4;                  // RoPE pairs per lane
  __shared__ __attribute__((aligned(16))) uint8_t smem[kStages * SM::STAGE];
  __shared__ float red[2 * kWaves];

  // work item: a whole unit (query tile x head) or one key-range part of one
  const int xcd = blockIdx.x & 7;
  const int local = blockIdx.x >> 3;
  int unit, part;
  if (local < a.full_per_xcd) {
    unit = xcd * a.full_per_xcd + local;
    if (unit >= a.n_full) return;
    part = -1;
  } else {
    const int j = xcd * a.parts_per_xcd + (local - a.full_per_xcd);
    if (j >= a.n_parts) return;
    unit = a.n_full + j / a.parts_per_unit;
    part = j;
  }
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
  const float* ks = a.ks + (int64_t)kvh * Sp;
  const float* vs = a.vs + (int64_t)kvh * Sp;

  // ---- window-wide max of the V scales -> P' scale constant c -------------
  float svmax = 0.0f;
  for (int64_t slot = a.seg_lo[0] + tid; slot < a.seg_hi[0]; slot += kThreads)
    svmax = __builtin_fmaxf(svmax, vs[slot]);
  if (a.n_segments > 1)
    for (int64_t slot = a.seg_lo[1] + tid; slot < a.seg_hi[1]; slot += kThreads)
      svmax = __builtin_fmaxf(svmax, vs[slot]);

  // ---- Q prologue pass 1: RoPE and the workgroup's max |q| ----------------
  const int q_row = qtile * kQPB + wave * kQPW + li;
  const int src_row = q_row < a.n_tokens ? q_row : a.n_tokens - 1;
  const uint16_t* q_src = a.q + (int64_t)src_row * a.ldq + (int64_t)head * D;
  const float* q_cs = a.rope + ((int64_t)src_row * (D / 2) + P * hh) * 2;
  float qamax = 0.0f;
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
      const float r0 = x0 * c.x - x1 * c.y;
      const float r1 = x1 * c.x + x0 * c.y;
      qamax = __builtin_fmaxf(qamax, __builtin_fmaxf(fabsf(r0), fabsf(r1)));
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    qamax = __builtin_fmaxf(qamax, __shfl_xor(qamax, o));
    svmax = __builtin_fmaxf(svmax, __shfl_xor(svmax, o));
  }
  if (lane == 0) {
    red[wave] = qamax;
    red[kWaves + wave] = svmax;
  }
  __syncthreads();
  qamax = 0.0f;
  svmax = 0.0f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    qamax = __builtin_fmaxf(qamax, red[w]);
    svmax = __builtin_fmaxf(svmax, red[kWaves + w]);
  }
  const float q_inv = qamax > 0.0f ? kFp8Max / qamax : 0.0f;
  const float kscale = (qamax / kFp8Max) * (kLog2e / sqrtf((float)D));
  const float cP = svmax > 0.0f ? kPmax / (exp2f(kTau) * svmax) : 1.0f;

  // ---- Q prologue pass 2: e4m3 codes in the B-operand layout ---------------
  // operand step s, byte b <-> d: D=128: d = 64 s + 32 hh + b; D=64: byte b < 16
  // -> d = 16 hh + b, b >= 16 -> d = 32 + 16 hh + b - 16 (RoPE pairs stay in-lane)
  v8i qop[NSTEP];
  v8i qlo[NSTEP];
  {
    float r0[P], r1[P];
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
        r0[j + e] = (x0 * c.x - x1 * c.y) * q_inv;
        r1[j + e] = (x1 * c.x + x0 * c.y) * q_inv;
      }
    }
#pragma unroll
    for (int w = 0; w < NSTEP * 8; ++w) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int b = 4 * w + e;
        if constexpr (D == 128) v[e] = (b < 32) ? r0[b] : r1[b - 32];
        else v[e] = (b < 16) ? r0[b] : r1[b - 16];
      }
      uint32_t c = 0, lo = 0;
      if constexpr (QLO) {
        split_fp8x2<false>(v[0], v[1], c, lo);
        split_fp8x2<true>(v[2], v[3], c, lo);
      } else {
        c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
        c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], (int)c, true);
      }
      qop[w / 8][w % 8] = (int)c;
      qlo[w / 8][w % 8] = (int)lo;
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

  // S^T = K . Q^T of the tile in stage st (raw integer-code products)
  auto qk = [&](const uint8_t* st, v16f (&acc)[2]) {
    v8i kop[2][NSTEP];
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
    acc[0] = v16f{};
    acc[1] = v16f{};
#pragma unroll
    for (int s = 0; s < NSTEP; ++s)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) acc[kh] = mfma_fp8(kop[kh][s], qop[s], acc[kh]);
    if constexpr (QLO)
#pragma unroll
      for (int s = 0; s < NSTEP; ++s)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) acc[kh] = mfma_fp8_bscaled(kop[kh][s], qlo[s], acc[kh], 127 - kLoShift);
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
  // O^T += V^T . P'^T with the V tile in stage st
  v16f acc_o[NDT];
#pragma unroll
  for (int d = 0; d < NDT; ++d) acc_o[d] = v16f{};
  auto pv = [&](const uint8_t* st, const v8i& pop, const v8i& plo) {
#pragma unroll
    for (int d = 0; d < NDT; ++d) {
      const uint8_t* vrow = st + SM::K_BYTES + (32 * d + li) * SM::VROW + 32 * hh;
      const uint4 v0 = *(const uint4*)(vrow);
      const uint4 v1 = *(const uint4*)(vrow + 16);
      const v8i vop = v8i{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w,
                          (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
      acc_o[d] = mfma_fp8(vop, pop, acc_o[d]);
      if constexpr (PLO) acc_o[d] = mfma_fp8_bscaled(vop, plo, acc_o[d], 127 - kLoShift);
    }
  };

  // ---- prologue: tiles 0 and 1 staged, tile 2 in registers, and the V rows
  // of the stage of tile -1 zeroed (the first iteration's product of the
  // previous tile then adds nothing); scores of tile 0
  TileRegs regs;
  if (n_it > 0) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      load_tile<D>(regs, tref(clamp_it(p)), kc, vc, ks, vs, tid);
      store_tile<D, MASK>(regs, tref(clamp_it(p)), stage_of(p), kscale, cP, tid);
    }
    load_tile<D>(regs, tref(clamp_it(2)), kc, vc, ks, vs, tid);
  }
  for (int i = tid; i < SM::V_BYTES / 16; i += kThreads)
    ((uint4*)(stage_of(-1) + SM::K_BYTES))[i] = make_uint4(0, 0, 0, 0);
  __syncthreads();

  float m_run = -INFINITY, l_run = 0.0f;
  v16f acc_s[2];
  qk(stage_of(0), acc_s);
  if constexpr (MASK) mask_scores(0, acc_s);
  v8i pop = v8i{}, plo = v8i{};

  // ---- main loop: iteration it computes the softmax of tile it while the
  // matrix cores take the PV product of tile it - 1 and the scores of tile
  // it + 1; the ring holds tiles it - 1 .. it + 2
  for (int it = 0; it < n_it; ++it) {
    const float* kf = (const float*)(stage_of(it) + SM::K_BYTES + SM::V_BYTES);
    const float* wf = kf + 64;
    pv(stage_of(it - 1), pop, plo);
    float t[32];
    softmax_scores<NDT>(acc_s, kf, hh, m_run, l_run, acc_o, t);
    // past the last tile these products read a stale stage and are unused
    qk(stage_of(it + 1), acc_s);
    if constexpr (MASK) mask_scores(it + 1, acc_s);
    pop = softmax_probs<PLO>(t, wf, hh, l_run, plo);

    // staging of tile it + 2 (stored into the stage tile it - 2 held) and it + 3
    // (loaded), unconditional with the tile index clamped (past the end the
    // copy lands in a stage nobody reads again)
    store_tile<D, MASK>(regs, tref(clamp_it(it + 2)), stage_of(it + 2), kscale, cP, tid);
    load_tile<D>(regs, tref(clamp_it(it + 3)), kc, vc, ks, vs, tid);
#if RTV_ATTEND_SCHED > 0
    // spread the score products of tile it + 1 over the exponentials
#pragma unroll
    for (int i = 0; i < 2 * NSTEP * (QLO ? 2 : 1); ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, RTV_ATTEND_SCHED, 0);
    }
#endif
    __syncthreads();
  }
  pv(stage_of(n_it - 1), pop, plo);

  // ---- epilogue ----------------------------------------------------------------
  const float l_tot = xhalf_sum(l_run);
  if (part >= 0) {
    // partial result of a key range: O / c unnormalized, with (m, l)
    const int q = wave * kQPW + li;
    float* po = a.ws_o + ((int64_t)part * kQPB + q) * D;
    const float inv_c = 1.0f / cP;
#pragma unroll
    for (int d = 0; d < NDT; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * d + 8 * g + 4 * hh;
        *(float4*)(po + d0) = make_float4(acc_o[d][4 * g + 0] * inv_c, acc_o[d][4 * g + 1] * inv_c,
                                          acc_o[d][4 * g + 2] * inv_c, acc_o[d][4 * g + 3] * inv_c);
      }
    if (hh == 0) *(float2*)(a.ws_ml + ((int64_t)part * kQPB + q) * 2) = make_float2(m_run, l_tot);
    return;
  }
  const float scale = 1.0f / (cP * l_tot);
  if (q_row < a.n_tokens) {
    uint16_t* dst = a.out + (int64_t)q_row * a.ldo + (int64_t)head * D;
#pragma unroll
    for (int d = 0; d < NDT; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * d + 8 * g + 4 * hh;
        uint2 w;
        w.x = pack_bf16x2(acc_o[d][4 * g + 0] * scale, acc_o[d][4 * g + 1] * scale);
        w.y = pack_bf16x2(acc_o[d][4 * g + 2] * scale, acc_o[d][4 * g + 3] * scale);
        *(uint2*)(dst + d0) = w;
      }
  }
}

// Merge the key-range parts of the split units: for each query,
// M = max_p m_p, w_p = 2^(m_p - M), O = sum_p w_p O_p / sum_p w_p l_p.
template <int D>
__global__ __launch_bounds__(2 * kQPB) void combine_kernel(AttendArgs a) {
  const int r = blockIdx.x;                       // split unit r
  const int unit = a.n_full + r;
  const int head = unit / a.n_qtiles;
  const int qtile = unit % a.n_qtiles;
  const int S = a.parts_per_unit;
  const int q = threadIdx.x >> 1;                 // 2 threads per query
  const int dh = (threadIdx.x & 1) * (D / 2);
  const int row = qtile * kQPB + q;
  if (q >= kQPB || row >= a.n_tokens) return;
  const int j0 = r * S;
  float M = -INFINITY;
  for (int p = 0; p < S; ++p) M = fmaxf(M, a.ws_ml[((int64_t)(j0 + p) * kQPB + q) * 2]);
  float L = 0.0f;
  float acc[D / 2];
#pragma unroll
  for (int d = 0; d < D / 2; ++d) acc[d] = 0.0f;
  for (int p = 0; p < S; ++p) {
    const float2 ml = *(const float2*)(a.ws_ml + ((int64_t)(j0 + p) * kQPB + q) * 2);
    const float w = exp2f(ml.x - M);
    L += w * ml.y;
    const float* po = a.ws_o + ((int64_t)(j0 + p) * kQPB + q) * D + dh;
#pragma unroll
    for (int d = 0; d < D / 2; d += 4) {
      const float4 o = *(const float4*)(po + d);
      acc[d] += w * o.x; acc[d + 1] += w * o.y; acc[d + 2] += w * o.z; acc[d + 3] += w * o.w;
    }
  }
  const float inv = 1.0f / L;
  uint16_t* dst = a.out + (int64_t)row * a.ldo + (int64_t)head * D + dh;
#pragma unroll
  for (int d = 0; d < D / 2; d += 8) {
    uint4 w;
    w.x = pack_bf16x2(acc[d] * inv, acc[d + 1] * inv);
    w.y = pack_bf16x2(acc[d + 2] * inv, acc[d + 3] * inv);
    w.z = pack_bf16x2(acc[d + 4] * inv, acc[d + 5] * inv);
    w.w = pack_bf16x2(acc[d + 6] * inv, acc[d + 7] * inv);
    *(uint4*)(dst + d) = w;
  }
}

}  // namespace

int attend_queries_per_block() { return kQPB; }

// parts are bounded so that the workspace has a fixed size
constexpr int kMaxParts = 512;
int attend_max_parts() { return kMaxParts; }
size_t attend_workspace_bytes(int head_dim) {
  return (size_t)kMaxParts * kQPB * ((size_t)head_dim + 2) * sizeof(float);
}

hipError_t attend_capacity(int* workgroups) {
  int dev = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  hipDeviceProp_t prop;
  if (e == hipSuccess) e = hipGetDeviceProperties(&prop, dev);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attend_kernel<128, false, false, false>, kThreads, 0);
  if (e != hipSuccess) return e;
  *workgroups = (per_cu > 0 ? per_cu : 1) * prop.multiProcessorCount;
  return hipSuccess;
}

hipError_t launch_attend(const AttendArgs& args_in, int head_dim, hipStream_t stream) {
  AttendArgs args = args_in;
  bool aligned = true;
  int64_t keys = 0;
  int n_tiles = 0;
  for (int s = 0; s < args.n_segments; ++s) {
    aligned = aligned && args.seg_lo[s] % 64 == 0 && args.seg_hi[s] % 64 == 0;
    keys += args.seg_hi[s] - args.seg_lo[s];
    if (args.seg_hi[s] > args.seg_lo[s])
      n_tiles += (int)((args.seg_hi[s] - 1) / 64 - args.seg_lo[s] / 64 + 1);
  }
  const bool short_window = keys < kPreciseKeys;
  const bool two_term_q = short_window || args.two_term_q;

  // Schedule: whole rounds of the device's concurrent workgroups run whole
  // windows; the remainder, which would leave most of the device idle in a
  // last round, is split along the keys so that it fills one short round.
  const int cap = args.capacity;
  const int U = args.n_work;
  int rem = cap > 0 ? U % cap : 0;
  int S = rem > 0 ? cap / rem : 1;
  if (S > n_tiles) S = n_tiles;
  if ((int64_t)rem * S > kMaxParts) S = kMaxParts / (rem > 0 ? rem : 1);
  if (S < 2 || !args.ws_o) { S = 1; rem = 0; }
  args.n_full = U - rem;
  args.parts_per_unit = S;
  args.n_parts = rem * S;
  args.full_per_xcd = (args.n_full + 7) / 8;
  args.parts_per_xcd = (args.n_parts + 7) / 8;
  const dim3 g(8 * (args.full_per_xcd + args.parts_per_xcd)), b(kThreads);
#define RTV_LAUNCH(DIM, MASK, QL, PL) \
  hipLaunchKernelGGL((attend_kernel<DIM, MASK, QL, PL>), g, b, 0, stream, args)
#define RTV_DISPATCH_MASK(DIM, QL, PL) \
  if (aligned) RTV_LAUNCH(DIM, false, QL, PL); else RTV_LAUNCH(DIM, true, QL, PL);
#define RTV_DISPATCH(DIM)                                 \
  if (short_window) {                                     \
    RTV_DISPATCH_MASK(DIM, true, true)                    \
  } else if (two_term_q) {                                \
    RTV_DISPATCH_MASK(DIM, true, false)                   \
  } else {                                                \
    RTV_DISPATCH_MASK(DIM, false, false)                  \
  }
  if (head_dim == 128) {
    RTV_DISPATCH(128)
  } else {
    RTV_DISPATCH(64)
  }
#undef RTV_DISPATCH
#undef RTV_DISPATCH_MASK
#undef RTV_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || rem == 0) return e;
  if (head_dim == 128)
    hipLaunchKernelGGL(combine_kernel<128>, dim3(rem), dim3(2 * kQPB), 0, stream, args);
  else
    hipLaunchKernelGGL(combine_kernel<64>, dim3(rem), dim3(2 * kQPB), 0, stream, args);
  return hipGetLastError();
}

}  // namespace rtv
