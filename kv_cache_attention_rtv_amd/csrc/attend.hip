// Chunk attention over the FP8 ring window (gfx950 matrix cores).
//
// The chunk's queries attend to every key of the valid window, the chunk
// itself included (240 such calls per diffusion step: page "Runway: Πώς ένα
// AI 57 δισ. παραμέτρων παράγει βίντεο στα 24 fps", section "Από οκτώ H100 σε
// τέσσερις"; the cache holds RoPE-rotated e4m3 K and e4m3 V, page "Runway
// explains how it serves a 57B video model in real time", fourth paragraph).
//
// Work decomposition: one workgroup = 128 queries of one query head (4 waves
// x 32 queries), iterating over 64-key tiles of the window's (at most two)
// slot segments.  Tiles are staged in LDS, double buffered: K rows [64][D],
// transposed V [D][64] (key order permuted in the ring so that each lane's
// 32 operand bytes are contiguous), and the per-key scales.
//
// Per wave and tile, with v_mfma_f32_32x32x64_f8f6f4 (e4m3 x e4m3 -> f32):
//   S^T[key][query] = K . Q^T       (2 key sub-tiles x D/64 k-steps)
//   lane (hh, i) of the result holds query i and 32 keys, so the softmax
//   row is per lane plus one exchange with lane i^32;
//   P'[query][key] = p * sv_key * c is converted to e4m3 and fed as the
//   B operand of O^T[d][query] += V^T . P'^T   (D/32 d sub-tiles).
// Scores: t = S_raw * sk_key * (sq_query * log2(e) / sqrt(D)); p = exp2(t - m).
// The running max m is lazy: it moves only when a tile's max exceeds it by
// more than kTau (log2 units), so p <= 2^kTau, and c = 448 / (2^kTau * max sv)
// keeps every P' inside the e4m3 range with one constant for the whole window.
// Output: O = acc / (c * l), rounded to bf16.
#include "device_common.hpp"
#include "kernels.hpp"

namespace rtv {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kQPW = 32;                   // queries per wave
constexpr int kQPB = kWaves * kQPW;        // queries per workgroup
constexpr float kTau = 3.0f;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ v16f mfma_fp8(const v8i& a, const v8i& b, const v16f& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// key index held by byte p of a transposed V tile row
__device__ __forceinline__ int vt_key(int p) {
  const int h = p >> 5, b = p & 31;
  return 32 * (b >> 4) + 8 * ((b >> 2) & 3) + 4 * h + (b & 3);
}

template <int D>
struct Smem {
  static constexpr int KROW = D + 16;      // padded K row (bytes): conflict-free 16 B reads
  static constexpr int VROW = 64 + 16;     // padded transposed-V row
  static constexpr int K_BYTES = 64 * KROW;
  static constexpr int V_BYTES = D * VROW;
  static constexpr int STAGE = K_BYTES + V_BYTES + 2 * 64 * 4;
};


// staged tile: D/4 bytes of K and of V per thread (two 16 B pieces for D=128)
struct TileRegs {
  uint4 k0, k1, v0, v1;
  float s;
};

struct TileRef {
  int tile;
  int64_t lo, hi;     // the segment the tile belongs to
};

__device__ __forceinline__ TileRef tile_of(int it, int t_count0, int t_first0, int t_first1,
                                           int64_t lo0, int64_t hi0, int64_t lo1, int64_t hi1) {
  const bool second = it >= t_count0;
  TileRef r;
  r.lo = second ? lo1 : lo0;
  r.hi = second ? hi1 : hi0;
  r.tile = second ? t_first1 + (it - t_count0) : t_first0 + it;
  return r;
}

template <int D>
__device__ __forceinline__ void load_tile(TileRegs& r, const TileRef& t, const uint8_t* kc,
                                          const uint8_t* vc, const float* ks, const float* vs,
                                          int tid) {
  constexpr int LD_BYTES = D / 4;
  const uint8_t* kt = kc + (int64_t)t.tile * 64 * D;
  const uint8_t* vt = vc + (int64_t)t.tile * 64 * D;
  r.k0 = *(const uint4*)(kt + tid * LD_BYTES);
  r.v0 = *(const uint4*)(vt + tid * LD_BYTES);
  if constexpr (LD_BYTES == 32) {
    r.k1 = *(const uint4*)(kt + tid * LD_BYTES + 16);
    r.v1 = *(const uint4*)(vt + tid * LD_BYTES + 16);
  }
  const float* src = tid < 64 ? ks : vs;
  r.s = tid < 128 ? src[(int64_t)t.tile * 64 + (tid & 63)] : 0.0f;
}

template <int D>
__device__ __forceinline__ void store_piece(uint4 kq, uint4 v, int b, uint8_t* st, bool partial,
                                            int64_t base, int64_t lo, int64_t hi) {
  using SM = Smem<D>;
  *(uint4*)(st + (b / D) * SM::KROW + (b % D)) = kq;
  const int row = b / 64, col = b % 64;
  if (partial) {
    // zero the codes of keys outside the segment (they may hold anything)
    uint32_t m[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      m[w] = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t slot = base + vt_key(col + 4 * w + e);
        if (slot >= lo && slot < hi) m[w] |= 0xFFu << (8 * e);
      }
    }
    v.x &= m[0]; v.y &= m[1]; v.z &= m[2]; v.w &= m[3];
  }
  *(uint4*)(st + SM::K_BYTES + row * SM::VROW + col) = v;
}

template <int D>
__device__ __forceinline__ void store_tile(const TileRegs& r, const TileRef& t, uint8_t* st,
                                           float cP, int tid) {
  using SM = Smem<D>;
  constexpr int LD_BYTES = D / 4;
  const int64_t base = (int64_t)t.tile * 64;
  const bool partial = t.lo > base || t.hi < base + 64;
  store_piece<D>(r.k0, r.v0, tid * LD_BYTES, st, partial, base, t.lo, t.hi);
  if constexpr (LD_BYTES == 32)
    store_piece<D>(r.k1, r.v1, tid * LD_BYTES + 16, st, partial, base, t.lo, t.hi);
  float* sk_s = (float*)(st + SM::K_BYTES + SM::V_BYTES);
  float* sw_s = sk_s + 64;
  if (tid < 128) {
    const int key = tid & 63;
    const int64_t slot = base + key;
    const bool ok = slot >= t.lo && slot < t.hi;
    if (tid < 64) sk_s[key] = ok ? r.s : 0.0f;
    else sw_s[key] = ok ? r.s * cP : 0.0f;
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attend_kernel(AttendArgs a) {
  using SM = Smem<D>;
  constexpr int NSTEP = D / 64;            // MFMA k-steps for K.Q^T
  constexpr int NDT = D / 32;              // 32-row d sub-tiles of O^T
  constexpr int P = D / 4;                 // RoPE pairs per lane
  constexpr int LD_BYTES = D / 4;          // bytes per thread per matrix per tile
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * SM::STAGE];
  __shared__ float red[kWaves];

  const int u = xcd_remap(blockIdx.x, a.n_work);
  if (u < 0) return;
  const int head = u / a.n_qtiles;
  const int qtile = u % a.n_qtiles;
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
    svmax = fmaxf(svmax, vs[slot]);
  if (a.n_segments > 1)
    for (int64_t slot = a.seg_lo[1] + tid; slot < a.seg_hi[1]; slot += kThreads)
      svmax = fmaxf(svmax, vs[slot]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) svmax = fmaxf(svmax, __shfl_xor(svmax, o));
  if (lane == 0) red[wave] = svmax;
  __syncthreads();
  svmax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float cP = svmax > 0.0f ? kFp8Max / (exp2f(kTau) * svmax) : 1.0f;

  // ---- Q prologue: RoPE, per-row e4m3, B-operand layout ------------------
  const int q_row = qtile * kQPB + wave * kQPW + li;
  const bool q_valid = q_row < a.n_tokens;
  const int q_src = q_valid ? q_row : a.n_tokens - 1;
  v8i qop[NSTEP];
  float a_i;
  {
    const uint16_t* src = a.q + (int64_t)q_src * a.ldq + (int64_t)head * D;
    const float* cs = a.rope + ((int64_t)q_src * (D / 2) + P * hh) * 2;
    float r0[P], r1[P];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < P; j += 8) {
      const uint4 w0 = *(const uint4*)(src + P * hh + j);
      const uint4 w1 = *(const uint4*)(src + D / 2 + P * hh + j);
      const uint32_t x0w[4] = {w0.x, w0.y, w0.z, w0.w};
      const uint32_t x1w[4] = {w1.x, w1.y, w1.z, w1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x0 = (e & 1) ? bf16_hi(x0w[e >> 1]) : bf16_lo(x0w[e >> 1]);
        const float x1 = (e & 1) ? bf16_hi(x1w[e >> 1]) : bf16_lo(x1w[e >> 1]);
        const float2 c = *(const float2*)(cs + 2 * (j + e));
        r0[j + e] = x0 * c.x - x1 * c.y;
        r1[j + e] = x1 * c.x + x0 * c.y;
        amax = fmaxf(amax, fmaxf(fabsf(r0[j + e]), fabsf(r1[j + e])));
      }
    }
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    const float inv = amax > 0.0f ? kFp8Max / amax : 0.0f;
    const float sq = amax / kFp8Max;
    // an all-zero query row gets a tiny positive factor instead of 0, so that
    // masked keys (-inf) still give p = 0 and the valid keys uniform weights
    a_i = fmaxf(sq * (kLog2e / sqrtf((float)D)), 1e-30f);
    // codes: operand step s holds bytes of r0 (s = 0) and r1 (s = 1) for D=128;
    // for D=64 one step holds r0[0..15] then r1[0..15].
    uint32_t words[NSTEP * 8];
#pragma unroll
    for (int w = 0; w < NSTEP * 8; ++w) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int b = 4 * w + e;           // operand byte over all steps
        float x;
        if constexpr (D == 128) x = (b < 32) ? r0[b] : r1[b - 32];
        else x = (b < 16) ? r0[b] : r1[b - 16];
        v[e] = x * inv;
      }
      const uint32_t signs = sign_bytes4(v[0], v[1], v[2], v[3]);
      uint32_t c = cvt_fp8x2<false>(fabsf(v[0]), fabsf(v[1]), 0u);
      c = cvt_fp8x2<true>(fabsf(v[2]), fabsf(v[3]), c);
      words[w] = c | signs;
    }
#pragma unroll
    for (int s = 0; s < NSTEP; ++s)
#pragma unroll
      for (int w = 0; w < 8; ++w) qop[s][w] = (int)words[8 * s + w];
  }

  // ---- tile schedule over the segments -------------------------------------
  // 64-slot tiles overlapping segment s: [t_first_s, t_first_s + t_count_s)
  const int64_t lo0 = a.seg_lo[0], hi0 = a.seg_hi[0];
  const int64_t lo1 = a.n_segments > 1 ? a.seg_lo[1] : 0;
  const int64_t hi1 = a.n_segments > 1 ? a.seg_hi[1] : 0;
  const int t_first0 = (int)(lo0 / 64);
  const int t_count0 = hi0 > lo0 ? (int)((hi0 - 1) / 64) - t_first0 + 1 : 0;
  const int t_first1 = (int)(lo1 / 64);
  const int t_count1 = hi1 > lo1 ? (int)((hi1 - 1) / 64) - t_first1 + 1 : 0;
  const int n_it = t_count0 + t_count1;

  // global -> register staging of one tile
  TileRegs regs;
  // ---- main loop -------------------------------------------------------------
  v16f acc_o[NDT];
#pragma unroll
  for (int d = 0; d < NDT; ++d) acc_o[d] = v16f{};
  float m_run = -INFINITY;
  float l_run = 0.0f;

  auto tref = [&](int it) {
    return tile_of(it, t_count0, t_first0, t_first1, lo0, hi0, lo1, hi1);
  };
  if (n_it > 0) {
    load_tile<D>(regs, tref(0), kc, vc, ks, vs, tid);
    store_tile<D>(regs, tref(0), smem, cP, tid);
  }
  __syncthreads();
  for (int it = 0; it < n_it; ++it) {
    const int stage = it & 1;
    if (it + 1 < n_it) load_tile<D>(regs, tref(it + 1), kc, vc, ks, vs, tid);

    const uint8_t* st = smem + stage * SM::STAGE;
    const float* sk_s = (const float*)(st + SM::K_BYTES + SM::V_BYTES);
    const float* sw_s = sk_s + 64;
    const TileRef tr = tref(it);
    const int64_t lo = tr.lo, hi = tr.hi;
    const int64_t base = (int64_t)tr.tile * 64;
    const bool partial = lo > base || hi < base + 64;

    // S^T = K . Q^T for the two 32-key sub-tiles
    v16f acc_s[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      acc_s[sub] = v16f{};
      const uint8_t* krow = st + (32 * sub + li) * SM::KROW;
#pragma unroll
      for (int s = 0; s < NSTEP; ++s) {
        v8i kop;
        uint4 k0, k1;
        if constexpr (D == 128) {
          k0 = *(const uint4*)(krow + 64 * s + 32 * hh);
          k1 = *(const uint4*)(krow + 64 * s + 32 * hh + 16);
        } else {
          k0 = *(const uint4*)(krow + 16 * hh);
          k1 = *(const uint4*)(krow + 32 + 16 * hh);
        }
        kop[0] = k0.x; kop[1] = k0.y; kop[2] = k0.z; kop[3] = k0.w;
        kop[4] = k1.x; kop[5] = k1.y; kop[6] = k1.z; kop[7] = k1.w;
        acc_s[sub] = mfma_fp8(kop, qop[s], acc_s[sub]);
      }
    }

    // scale by the key scales; tile max
    float uval[32];
    float mx = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int key0 = 32 * sub + 8 * g4 + 4 * hh;
        const float4 skv = *(const float4*)(sk_s + key0);
        const float sk4[4] = {skv.x, skv.y, skv.z, skv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x = acc_s[sub][4 * g4 + e] * sk4[e];
          if (partial) {
            const int64_t slot = base + key0 + e;
            if (!(slot >= lo && slot < hi)) x = -INFINITY;
          }
          uval[16 * sub + 4 * g4 + e] = x;
          mx = fmaxf(mx, x);
        }
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float cand = mx * a_i;            // mx is finite: every tile has a valid key
    const bool need = cand > m_run + kTau;
    if (__any(need)) {
      const float m_new = fmaxf(m_run, cand);
      const float alpha = exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < NDT; ++d) acc_o[d] *= alpha;
      m_run = m_new;
    }

    // probabilities, row sum, P' codes
    v8i pop;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int key0 = 32 * sub + 8 * g4 + 4 * hh;
        const float4 swv = *(const float4*)(sw_s + key0);
        const float sw4[4] = {swv.x, swv.y, swv.z, swv.w};
        float pp[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(uval[16 * sub + 4 * g4 + e], a_i, -m_run));
          l_run += p;
          pp[e] = p * sw4[e];
        }
        uint32_t c = cvt_fp8x2<false>(pp[0], pp[1], 0u);
        c = cvt_fp8x2<true>(pp[2], pp[3], c);
        pop[4 * sub + g4] = (int)c;
      }

    // O^T += V^T . P'^T
#pragma unroll
    for (int d = 0; d < NDT; ++d) {
      const uint8_t* vrow = st + SM::K_BYTES + (32 * d + li) * SM::VROW + 32 * hh;
      const uint4 v0 = *(const uint4*)(vrow);
      const uint4 v1 = *(const uint4*)(vrow + 16);
      v8i vop;
      vop[0] = v0.x; vop[1] = v0.y; vop[2] = v0.z; vop[3] = v0.w;
      vop[4] = v1.x; vop[5] = v1.y; vop[6] = v1.z; vop[7] = v1.w;
      acc_o[d] = mfma_fp8(vop, pop, acc_o[d]);
    }

    if (it + 1 < n_it) store_tile<D>(regs, tref(it + 1), smem + (stage ^ 1) * SM::STAGE, cP, tid);
    __syncthreads();
  }

  // ---- epilogue ----------------------------------------------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float scale = 1.0f / (cP * l_tot);
  if (q_valid) {
    uint16_t* dst = a.out + (int64_t)q_row * a.ldo + (int64_t)head * D;
#pragma unroll
    for (int d = 0; d < NDT; ++d)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * d + 8 * g4 + 4 * hh;
        uint2 w;
        w.x = pack_bf16x2(acc_o[d][4 * g4 + 0] * scale, acc_o[d][4 * g4 + 1] * scale);
        w.y = pack_bf16x2(acc_o[d][4 * g4 + 2] * scale, acc_o[d][4 * g4 + 3] * scale);
        *(uint2*)(dst + d0) = w;
      }
  }
}

}  // namespace

int attend_queries_per_block() { return kQPB; }

hipError_t launch_attend(const AttendArgs& args, int head_dim, hipStream_t stream) {
  const int blocks = ((args.n_work + 7) / 8) * 8;
  if (head_dim == 128)
    hipLaunchKernelGGL(attend_kernel<128>, dim3(blocks), dim3(kThreads), 0, stream, args);
  else
    hipLaunchKernelGGL(attend_kernel<64>, dim3(blocks), dim3(kThreads), 0, stream, args);
  return hipGetLastError();
}

}  // namespace rtv
