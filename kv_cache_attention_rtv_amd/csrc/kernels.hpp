// Launch interfaces between the host library and the kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rtv {

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
  // schedule (filled by launch_attend): units [0, n_full) run whole windows; units [n_full, n_work) are
  // split into parts_per_unit key ranges whose partial (O, m, l) go to the
  // workspace and are merged by the combine kernel
  int32_t n_full;
  int32_t parts_per_unit;
  int32_t full_per_xcd;
  int32_t parts_per_xcd;
  int32_t n_parts;
  float* ws_o;            // [n_parts][queries per workgroup][D] f32, sum p V
  float* ws_ml;           // [n_parts][queries per workgroup][2] f32 (m, sum p)
  // per-window key factors (written by the factors kernel of the same call):
  float* fac_l;           // [n_kv_heads][ring tiles][64] float4 records (sk', log2(55 rho) / sk', 127 + e, 0)
  uint8_t* fac_u;         // [n_kv_heads][ring tiles][2][64] e4m3 rows of 2^-2 / rho
  int32_t n_kv_heads;
  int32_t ring_tiles;     // slots_padded / 64
};

// concurrent workgroups per device and workspace bound of the attention kernel
int attend_max_parts();
// workspace of rtv_attend: split-key-range partials and the per-window key
// factors; attend_set_workspace points the arguments into it
size_t attend_workspace_bytes(int head_dim, int n_kv_heads, int64_t slots_padded);
void attend_set_workspace(AttendArgs& a, void* ws, int head_dim, int n_kv_heads, int64_t slots_padded);
hipError_t attend_capacity(int* workgroups);

hipError_t launch_append(const AppendArgs& args, int head_dim, hipStream_t stream);
hipError_t launch_attend(const AttendArgs& args, int head_dim, hipStream_t stream);
hipError_t launch_encode_e4m3(const float* x, uint8_t* out, int64_t n, hipStream_t stream);
int attend_queries_per_block();

// per-tensor e4m3 quantization (partial: quant_max_partials() u32 of workspace)
int quant_max_partials();
hipError_t launch_quant_fp8(const uint16_t* x, int64_t n, uint8_t* codes, float* scale,
                            uint32_t* partial, hipStream_t stream);
hipError_t launch_gemm_fp8(const uint8_t* a, const float* sa, const uint8_t* bt, const float* sb,
                           uint16_t* c, int M, int N, int K, int64_t ldc, hipStream_t stream);

}  // namespace rtv
