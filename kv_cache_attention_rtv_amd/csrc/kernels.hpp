// Launch interfaces between the host library and the kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rtv {

// Ring state of one layer in device memory (device-state mode): the calls
// read it in their kernels and the advance kernel moves it, so that a
// captured sequence of calls replays correctly step after step.
struct DevRingState {
  int64_t next_global_frame;
  int32_t committed;
  int32_t error;          // set (and kept) when a call finds the state unusable,
                          // e.g. the chunk past the end of the RoPE table; the
                          // call's kernels then write nothing
};

// Fixed shape of the ring, for the device-state mode.
struct RingShape {
  int32_t tokens_per_frame;
  int32_t chunk_frames;
  int32_t capacity_frames;
  int32_t max_global_frames;
  int32_t max_window_frames;  // attend only (0 = all valid)
  int32_t head_dim;
};

struct AppendArgs {
  const uint16_t* k;      // [n][H][D] bf16, row stride ldk elements
  const uint16_t* v;
  int64_t ldk, ldv;
  const float* rope;      // (cos, sin) pairs of the chunk's first position: [n][D/2][2]
  uint8_t* kc;            // layer K codes  [H][Sp][D]
  uint8_t* vc;            // layer V codes  [H][Sp/64][D][64]
  float* ks;              // layer K scales [H][Sp]
  float* vs;
  int64_t slots_padded;   // Sp
  int64_t write_slot;     // first slot of the chunk
  int32_t n_tokens;
  int32_t n_heads;        // KV heads
  int32_t first_tile;     // write_slot / 64
  int32_t n_work;         // (#64-slot tiles touched) * n_heads
  // device-state mode (dstate != nullptr): rope, write_slot, first_tile and
  // n_work are derived in the kernel from *dstate; the grid covers the most
  // tiles a chunk can touch
  DevRingState* dstate;
  const float* rope_table;  // position 0 of the RoPE table
  RingShape shape;
};

struct AttendArgs {
  const uint16_t* q;      // [n][Hq][D] bf16, row stride ldq
  uint16_t* out;          // [n][Hq][D] bf16, row stride ldo
  int64_t ldq, ldo;
  const float* rope;      // (cos, sin) pairs of the chunk's first position
  const uint8_t* kc;      // layer ring (see AppendArgs)
  const uint8_t* vc;
  const float* ks;
  const float* vs;
  int64_t slots_padded;
  int64_t seg_lo[2];      // window segments in slot space [lo, hi)
  int64_t seg_hi[2];
  int32_t n_segments;
  int32_t n_tokens;
  int32_t n_q_heads;
  int32_t group;          // n_q_heads / n_kv_heads
  int32_t n_qtiles;       // ceil(n_tokens / queries per workgroup)
  int32_t n_work;         // n_qtiles * n_q_heads (units of work)
  int32_t capacity;       // workgroups the device runs concurrently (0 = never split)
  int32_t two_term_q;     // queries as two e4m3 terms on every window
  int32_t two_term_p;     // P' (and queries) as two e4m3 terms on every window
  int32_t check_peaked;   // one-code P' windows are checked for peaked rows and
                          // the flagged units recomputed with two-term Q and P'
  int32_t redo;           // this launch recomputes only the units flagged in `flags`
  // schedule (filled by launch_attend): units [0, n_full) run whole windows; units [n_full, n_work) are
  // split into parts_per_unit key ranges whose partial (O, m, l) go to the
  // workspace and are merged by the combine kernel
  int32_t n_full;
  int32_t parts_per_unit;
  int32_t full_per_xcd;
  int32_t parts_per_xcd;
  int32_t n_parts;
  float* ws_o;            // [n_parts][queries per workgroup][D] f32, sum p V
  float* ws_ml;           // [n_parts][queries per workgroup][4] f32 (m, sum p, sum p'^2, 0)
  uint32_t* flags;        // [n_work] 1 = unit flagged as peaked, then [n_work] = flagged count
  // per-window key factors (written by the factors kernel of the same call):
  float* fac_l;           // [n_kv_heads][ring tiles][64] float4 records (kf, log2(55 rho) / kf, 127 + e, 0),
                          // kf = max(sk, 2^-60) log2(e) / sqrt(D)
  uint8_t* fac_u;         // [n_kv_heads][ring tiles][2][64] e4m3 rows of 2^-2 / rho
  int32_t n_kv_heads;
  int32_t ring_tiles;     // slots_padded / 64
  // device-state mode (dstate != nullptr): rope, the segments and the
  // schedule are derived in the kernels from *dstate; the grids cover the
  // largest window
  DevRingState* dstate;
  const float* rope_table;
  RingShape shape;
};

// Split schedule of an attention call over n_tiles window tiles, shared by
// the host (host-state mode) and the kernels (device-state mode): whole
// rounds of the device's concurrent workgroups run whole windows; the
// remainder, which would leave most of the device idle in a last round, is
// split along the keys into parts (at most max_parts) so that it fills one
// short round.
__host__ __device__ inline void attend_schedule(AttendArgs& a, int n_tiles, int max_parts) {
  const int cap = a.capacity;
  const int U = a.n_work;
  int rem = cap > 0 ? U % cap : 0;
  int S = rem > 0 ? cap / rem : 1;
  if (S > n_tiles) S = n_tiles;
  if ((int64_t)rem * S > max_parts) S = max_parts / (rem > 0 ? rem : 1);
  if (S < 2 || !a.ws_o) { S = 1; rem = 0; }
  a.n_full = U - rem;
  a.parts_per_unit = S;
  a.n_parts = rem * S;
  a.full_per_xcd = (a.n_full + 7) / 8;
  a.parts_per_xcd = (a.n_parts + 7) / 8;
}

// number of 64-slot tiles the window segments of a touch
__host__ __device__ inline int attend_segment_tiles(int64_t lo, int64_t hi) {
  return hi > lo ? (int)((hi - 1) / 64 - lo / 64 + 1) : 0;
}
__host__ __device__ inline int attend_window_tiles(const AttendArgs& a) {
  // (constant indices only: the device copy of the arguments stays in registers)
  return (a.n_segments > 0 ? attend_segment_tiles(a.seg_lo[0], a.seg_hi[0]) : 0) +
         (a.n_segments > 1 ? attend_segment_tiles(a.seg_lo[1], a.seg_hi[1]) : 0);
}

// concurrent workgroups per device and workspace bound of the attention kernel
int attend_max_parts();
// workspace of rtv_attend: split-key-range partials and the per-window key
// factors; attend_set_workspace points the arguments into it
size_t attend_workspace_bytes(int head_dim, int n_kv_heads, int64_t slots_padded, int64_t n_units);
void attend_set_workspace(AttendArgs& a, void* ws, int head_dim, int n_kv_heads, int64_t slots_padded,
                          int64_t n_units);
hipError_t attend_capacity(int* workgroups);

hipError_t launch_append(const AppendArgs& args, int head_dim, hipStream_t stream);
hipError_t launch_attend(const AttendArgs& args, int head_dim, hipStream_t stream);
hipError_t launch_encode_e4m3(const float* x, uint8_t* out, int64_t n, hipStream_t stream);
int attend_queries_per_block();

// per-tensor e4m3 quantization (partial: quant_max_partials() u32 of workspace)
int quant_max_partials();
hipError_t launch_quant_fp8(const uint16_t* x, int64_t n, uint8_t* codes, float* scale,
                            uint32_t* partial, hipStream_t stream);
// the same with the partials in the library's static device array (no allocation)
hipError_t launch_quant_fp8_static(const uint16_t* x, int64_t n, uint8_t* codes, float* scale,
                                   hipStream_t stream);
int quant_scratch_words();
// FP8 QKV GEMM whose epilogue writes Q as bf16 and K, V (RoPE on K, e4m3 per
// (token, head)) straight into the ring slots of the chunk
struct QkvAppendArgs {
  const uint8_t* x;       // [M][K] e4m3
  const float* sx;
  const uint8_t* wt;      // [N][K] e4m3, N = q_cols + 2 * n_kv_heads * head_dim
  const float* sw;
  uint16_t* q_out;        // [M][ldq] bf16 (columns [0, q_cols))
  int64_t ldq;
  int32_t M, K, q_cols, n_kv_heads, head_dim;
  const float* rope;      // (cos, sin) pairs of the chunk's first position
  uint8_t* kc;
  uint8_t* vc;
  float* ks;
  float* vs;
  int64_t slots_padded;
  int64_t write_slot;     // multiple of 64
};
hipError_t launch_qkv_gemm_append(const QkvAppendArgs& q, hipStream_t stream);
// device-state mode: advance n layers' states by one chunk
hipError_t launch_advance(DevRingState* s, int n, int chunk_frames, int capacity_frames, hipStream_t stream);
hipError_t launch_gemm_fp8(const uint8_t* a, const float* sa, const uint8_t* bt, const float* sb,
                           uint16_t* c, int M, int N, int K, int64_t ldc, hipStream_t stream);

}  // namespace rtv
