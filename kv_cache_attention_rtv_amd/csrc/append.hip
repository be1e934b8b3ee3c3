// Cache upkeep: RoPE on the chunk's K, per-(token, head) e4m3 quantization of
// K and V, and the write into the ring slots of the current chunk.
//
// The pages put RoPE and FP8 quantization at the moment a frame's K/V enter
// the cache, once, and keep the cache in a circular buffer that advances by a
// head index (page "Runway explains how it serves a 57B video model in real
// time", fourth paragraph; page "Runway: Πώς ένα AI 57 δισ. παραμέτρων
// παράγει βίντεο στα 24 fps", section "Από οκτώ H100 σε τέσσερις").
//
// One workgroup = one 64-slot tile of the ring x three KV heads (512 threads,
// 8 lanes per slot).  The RoPE (cos, sin) of a slot is loaded once and
// applied to the K rows of all three heads; the heads' K/V pieces are loaded
// two heads ahead of the arithmetic.  Eight lanes share a token row: lane g of
// the row holds the element groups
// [g*E, g*E+E) and [D/2+g*E, D/2+g*E+E), E = D/16, i.e. both halves of its
// RoPE pairs, so the rotation needs no lane exchange and every bf16 load is
// 8 lanes x 16 B = 128 B contiguous.  The row amax is an 8-lane DPP max.
// K codes go straight to their row, 16 bytes per lane; V codes go through
// LDS and are written transposed per tile ([d][64 slots], key order of the
// attention kernel's matrix-core operand), 16 bytes per lane.  The bf16
// inputs are read with non-temporal loads.
//
// Arithmetic is fixed bit for bit: RoPE products and the sum/difference are
// rounded separately (no contraction: this file is built with
// -ffp-contract=off), scale = RN(amax/448), x/scale is the correctly rounded
// quotient, and the e4m3 conversion rounds to nearest even.  Rows with a
// normal scale (all of them in practice) take the short form of these steps
// (quant_row); the others the general one.
#include "device_common.hpp"
#include "kernels.hpp"
#include "ring.hpp"

namespace rtv {
namespace {

constexpr int kAppendThreads = 512;   // 8 lanes per slot of a 64-slot tile
constexpr int kAppendHeads = 3;       // KV heads per workgroup (share the RoPE loads)
// (six waves per SIMD, at most 80 VGPRs: three workgroups per CU, the step
// chunk's 748 in one round)

__device__ __forceinline__ float dpp_max8(float x) {
  // max over the 8 lanes of each row group: quad xor 1, quad xor 2, then the
  // half-row mirror (lane i <-> 7-i within 8) pairs the two quads.
  float y;
  y = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
  x = fmaxf(x, y);
  y = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
  x = fmaxf(x, y);
  y = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
  return fmaxf(x, y);
}

// first key of the 4 consecutive positions 4*p4 .. 4*p4+3
__device__ __forceinline__ int vt_key_of_pos4(int p4) {
  const int h = p4 >> 3;
  const int b = (p4 & 7) << 2;
  return 32 * (b >> 4) + 8 * ((b >> 2) & 3) + 4 * h;
}

// bf16 pieces of one lane: E elements at d0 and E at D/2 + d0
template <int E>
struct RowPiece {
  uint32_t w0[E / 2], w1[E / 2];
};

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// K and V are read once per call: the loads are non-temporal, so that the
// chunk's 74 MB of bf16 input streams past the caches instead of evicting the
// RoPE rows, which the append of every layer reads again.
template <int D>
__device__ __forceinline__ RowPiece<D / 16> load_piece(const uint16_t* row, int g, bool valid) {
  constexpr int E = D / 16;
  RowPiece<E> r;
  if constexpr (E == 8) {
    u32x4_t p0 = {0, 0, 0, 0}, p1 = p0;
    if (valid) {
      p0 = __builtin_nontemporal_load((const u32x4_t*)(row + g * E));
      p1 = __builtin_nontemporal_load((const u32x4_t*)(row + D / 2 + g * E));
    }
    r.w0[0] = p0.x; r.w0[1] = p0.y; r.w0[2] = p0.z; r.w0[3] = p0.w;
    r.w1[0] = p1.x; r.w1[1] = p1.y; r.w1[2] = p1.z; r.w1[3] = p1.w;
  } else {
    u32x2_t p0 = {0, 0}, p1 = p0;
    if (valid) {
      p0 = __builtin_nontemporal_load((const u32x2_t*)(row + g * E));
      p1 = __builtin_nontemporal_load((const u32x2_t*)(row + D / 2 + g * E));
    }
    r.w0[0] = p0.x; r.w0[1] = p0.y;
    r.w1[0] = p1.x; r.w1[1] = p1.y;
  }
  return r;
}

// Device-state mode: the chunk's first slot and RoPE rows from the layer's
// ring state (the host computes the same from its copy in host-state mode).
// False, with the state's error set, when the chunk would run past the RoPE
// table: the kernel then writes nothing.
template <int D>
__device__ __forceinline__ bool append_derive(AppendArgs& a, int groups) {
  const RingShape& g = a.shape;
  const int64_t next = a.dstate->next_global_frame;
  RingWindow w;
  if (next + g.chunk_frames > g.max_global_frames ||
      ring_window(next, a.dstate->committed, g.tokens_per_frame, g.chunk_frames, g.capacity_frames, 0, &w) !=
          kRingOk) {
    if (blockIdx.x == 0 && threadIdx.x == 0) a.dstate->error = 1;
    return false;
  }
  a.write_slot = w.write_slot;
  a.rope = a.rope_table + next * g.tokens_per_frame * D;
  a.first_tile = (int32_t)(w.write_slot / kTileKeys);
  const int64_t last_tile = (w.write_slot + a.n_tokens - 1) / kTileKeys;
  a.n_work = (int32_t)(last_tile - a.first_tile + 1) * groups;
  return true;
}

template <int D, int HPW>
__global__ __launch_bounds__(kAppendThreads) __attribute__((amdgpu_waves_per_eu(6))) void append_rope_quant_kernel(AppendArgs a) {
  constexpr int E = D / 16;          // elements per lane per half
  constexpr int HALF = D / 2;
  constexpr int LDS_STRIDE = D + 4;  // bytes per V row in LDS
  static_assert(kAppendThreads == 8 * kTileKeys, "one lane octet per slot of the tile");
  __shared__ uint32_t vrow[HPW][kTileKeys * LDS_STRIDE / 4];

  const int groups = (a.n_heads + HPW - 1) / HPW;
  if (a.dstate && !append_derive<D>(a, groups)) return;
  const int u = xcd_remap(blockIdx.x, a.n_work);
  if (u < 0) return;
  const int st = a.first_tile + u / groups;
  const int h0 = (u % groups) * HPW;
  const int64_t tile_lo = (int64_t)st * kTileKeys;
  const int64_t lo = tile_lo > a.write_slot ? tile_lo : a.write_slot;
  const int64_t end = a.write_slot + a.n_tokens;
  const int64_t hi = (tile_lo + kTileKeys) < end ? (tile_lo + kTileKeys) : end;

  const int tid = threadIdx.x;
  const int g = tid & 7;
  const int r = tid >> 3;                        // key row within the tile
  const int64_t slot = tile_lo + r;
  const bool valid = slot >= lo && slot < hi;
  const int64_t t = valid ? slot - a.write_slot : 0;   // token in the chunk

  // ---- global loads ahead of the arithmetic: the K and V pieces of the first
  // two heads and, once for all heads, the row's RoPE (cos, sin); the pieces
  // of head j + 2 are loaded once head j is done, so at most two heads' pieces
  // are live (80 VGPRs, three workgroups per CU, the whole chunk in one round;
  // only the general quantization path of rows with a subnormal scale spills)
  RowPiece<E> kp[HPW], vp[HPW];
  auto load_head = [&](int j) {
    const bool hv = h0 + j < a.n_heads;
    kp[j] = load_piece<D>(a.k + t * a.ldk + (int64_t)(h0 + j) * D, g, valid && hv);
    vp[j] = load_piece<D>(a.v + t * a.ldv + (int64_t)(h0 + j) * D, g, valid && hv);
  };
#pragma unroll
  for (int j = 0; j < (HPW < 2 ? HPW : 2); ++j) load_head(j);
  float4 cs[E / 2];
  {
    const float4* tab = (const float4*)(a.rope + (t * HALF + g * E) * 2);
#pragma unroll
    for (int i = 0; i < E / 2; ++i) cs[i] = valid ? tab[i] : make_float4(1.f, 0.f, 1.f, 0.f);
  }

#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    const int h = h0 + j;
    if (h >= a.n_heads) break;                   // uniform over the workgroup
    // ---- K: rotate, quantize, store ------------------------------------
    // (each part takes the short form when every valid row of the wave has a
    // normal scale: one uniform choice per part)
    {
      float r0[E], r1[E];
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < E / 2; ++i) {
        const float4 c = cs[i];                  // (cos, sin) of two pairs
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int e = 2 * i + q;
          const float co = q ? c.z : c.x;
          const float si = q ? c.w : c.y;
          const float x0 = (e & 1) ? bf16_hi(kp[j].w0[e >> 1]) : bf16_lo(kp[j].w0[e >> 1]);
          const float x1 = (e & 1) ? bf16_hi(kp[j].w1[e >> 1]) : bf16_lo(kp[j].w1[e >> 1]);
          const float a0 = x0 * co;
          const float b0 = x1 * si;
          const float a1 = x1 * co;
          const float b1 = x0 * si;
          r0[e] = a0 - b0;
          r1[e] = a1 + b1;
          amax = fmaxf(fmaxf(amax, fabsf(r0[e])), fabsf(r1[e]));
        }
      }
      amax = dpp_max8(amax);
      uint32_t c0[E / 4], c1[E / 4];
      const float ks = quant_row<E>(r0, r1, c0, c1, amax, __all(!valid || fast_amax(amax)));
      // (D = 128: adjacent lanes swap halves, so that each lane stores 16
      // contiguous bytes: the even lane both first-half pieces, the odd lane
      // both second-half pieces)
      uint32_t x0 = 0, x1 = 0;
      const bool odd = g & 1;
      if constexpr (E == 8) {
        x0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)(odd ? c0[0] : c1[0]), 0xB1, 0xF, 0xF, false);
        x1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)(odd ? c0[1] : c1[1]), 0xB1, 0xF, 0xF, false);
      }
      if (valid) {
        uint8_t* dst = a.kc + ((int64_t)h * a.slots_padded + slot) * D;
        if constexpr (E == 8) {
          uint8_t* p = dst + (odd ? HALF + (g - 1) * E : g * E);
          *(uint4*)p = odd ? make_uint4(x0, x1, c1[0], c1[1]) : make_uint4(c0[0], c0[1], x0, x1);
        } else {
          *(uint32_t*)(dst + g * E) = c0[0];
          *(uint32_t*)(dst + HALF + g * E) = c1[0];
        }
        if (g == 0) a.ks[(int64_t)h * a.slots_padded + slot] = ks;
      }
    }
    // ---- V: quantize, stage row-major in LDS ----------------------------
    {
      float x0[E], x1[E];
      float amax = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        x0[e] = (e & 1) ? bf16_hi(vp[j].w0[e >> 1]) : bf16_lo(vp[j].w0[e >> 1]);
        x1[e] = (e & 1) ? bf16_hi(vp[j].w1[e >> 1]) : bf16_lo(vp[j].w1[e >> 1]);
        amax = fmaxf(fmaxf(amax, fabsf(x0[e])), fabsf(x1[e]));
      }
      amax = dpp_max8(amax);
      uint32_t c0[E / 4], c1[E / 4];
      const float vs = quant_row<E>(x0, x1, c0, c1, amax, __all(!valid || fast_amax(amax)));
      uint32_t* row = vrow[j] + r * (LDS_STRIDE / 4);
#pragma unroll
      for (int i = 0; i < E / 4; ++i) {
        row[(g * E) / 4 + i] = c0[i];
        row[(HALF + g * E) / 4 + i] = c1[i];
      }
      if (valid && g == 0) a.vs[(int64_t)h * a.slots_padded + slot] = vs;
    }
    if (j + 2 < HPW) load_head(j + 2);
  }
  __syncthreads();

  // ---- V: transposed write of each head's tile ----------------------------
  // Thread (q, dq) of a head: positions 16q..16q+15 (four runs of 4
  // consecutive keys) x d = 4dq..4dq+3; four 4x4 byte transposes turn the
  // 16 key rows into 4 d rows of 16 bytes, one 16-byte store each.
  const bool full = (lo == tile_lo) && (hi == tile_lo + kTileKeys);
  constexpr int kBlocks = 4 * (D / 4);   // per head
  const int n_here = (a.n_heads - h0) < HPW ? (a.n_heads - h0) : HPW;
  for (int id = tid; id < n_here * kBlocks; id += kAppendThreads) {
    const int j = id / kBlocks;
    const int h = h0 + j;
    const int w = id - j * kBlocks;
    const int q = w & 3;
    const int dq = w >> 2;
    uint8_t* vt = a.vc + (((int64_t)h * (a.slots_padded / kTileKeys) + st) * D) * kTileKeys;
    uint32_t o[4][4];
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      const int key0 = vt_key_of_pos4(4 * q + sub);
      const uint32_t* base = vrow[j] + key0 * (LDS_STRIDE / 4) + dq;
      const uint32_t a0 = base[0];
      const uint32_t a1 = base[LDS_STRIDE / 4];
      const uint32_t a2 = base[2 * (LDS_STRIDE / 4)];
      const uint32_t a3 = base[3 * (LDS_STRIDE / 4)];
      const uint32_t lo01 = __builtin_amdgcn_perm(a1, a0, 0x05010400u);
      const uint32_t hi01 = __builtin_amdgcn_perm(a1, a0, 0x07030602u);
      const uint32_t lo23 = __builtin_amdgcn_perm(a3, a2, 0x05010400u);
      const uint32_t hi23 = __builtin_amdgcn_perm(a3, a2, 0x07030602u);
      o[0][sub] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
      o[1][sub] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
      o[2][sub] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
      o[3][sub] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
    }
    if (full) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *(uint4*)(vt + (int64_t)(4 * dq + e) * kTileKeys + 16 * q) = make_uint4(o[e][0], o[e][1], o[e][2], o[e][3]);
    } else {
      // partial tile (chunk not aligned to 64 slots): write only this chunk's keys
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) {
        const int key0 = vt_key_of_pos4(4 * q + sub);
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int64_t sl = tile_lo + key0 + c;
            if (sl >= lo && sl < hi)
              vt[(int64_t)(4 * dq + e) * kTileKeys + 16 * q + 4 * sub + c] = (uint8_t)(o[e][sub] >> (8 * c));
          }
      }
    }
  }
}

__global__ void encode_e4m3_kernel(const float* __restrict__ x, uint8_t* __restrict__ out, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i + 3 < n) {
    const float4 v = *(const float4*)(x + i);
    const uint32_t signs = sign_bytes4(v.x, v.y, v.z, v.w);
    uint32_t w = cvt_fp8x2<false>(fabsf(v.x), fabsf(v.y), 0u);
    w = cvt_fp8x2<true>(fabsf(v.z), fabsf(v.w), w);
    *(uint32_t*)(out + i) = w | signs;
  } else {
    for (int64_t j = i; j < n; ++j) {
      const float v = x[j];
      const uint32_t w = cvt_fp8x2<false>(fabsf(v), 0.0f, 0u);
      out[j] = (uint8_t)((w & 0x7F) | ((__float_as_uint(v) >> 31) << 7));
    }
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& args_in, int head_dim, hipStream_t stream) {
  // work items: (tile, group of kAppendHeads heads); args_in.n_work counts (tile, head)
  AppendArgs args = args_in;
  const int tiles = args.n_work / args.n_heads;
  args.n_work = tiles * ((args.n_heads + kAppendHeads - 1) / kAppendHeads);
  const int blocks = ((args.n_work + 7) / 8) * 8;
  if (head_dim == 128)
    hipLaunchKernelGGL((append_rope_quant_kernel<128, kAppendHeads>), dim3(blocks), dim3(kAppendThreads), 0,
                       stream, args);
  else
    hipLaunchKernelGGL((append_rope_quant_kernel<64, kAppendHeads>), dim3(blocks), dim3(kAppendThreads), 0,
                       stream, args);
  return hipGetLastError();
}

__global__ __launch_bounds__(64) void advance_kernel(DevRingState* s, int n, int chunk_frames, int capacity_frames) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    s[i].next_global_frame += chunk_frames;
    const int c = s[i].committed + chunk_frames;
    s[i].committed = c < capacity_frames ? c : capacity_frames;
  }
}

hipError_t launch_advance(DevRingState* s, int n, int chunk_frames, int capacity_frames, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(advance_kernel, dim3((n + 63) / 64), dim3(64), 0, stream, s, n, chunk_frames, capacity_frames);
  return hipGetLastError();
}

hipError_t launch_encode_e4m3(const float* x, uint8_t* out, int64_t n, hipStream_t stream) {
  const int64_t threads = (n + 3) / 4;
  const int64_t blocks = (threads + 255) / 256;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(encode_e4m3_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, out, n);
  return hipGetLastError();
}

}  // namespace rtv
