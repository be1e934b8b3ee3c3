// Host side of the C ABI declared in include/rtv.h: validation, the device
// arena layout, per-layer ring state, the RoPE table, and kernel launches.
//
// Ring state lives on the host and every transition is driven by a host call,
// so the hot path never reads device memory back (a single host read-back per
// step is reported to have raised the step time from 168.5 ms to 278 ms: page
// "Runway explains how it serves a 57B video model in real time", fifth
// paragraph).  For graph capture (the forward pass is captured in a CUDA
// graph: page "Runway partage la construction de Runway Characters", fourth
// paragraph) the state can instead live in the arena between
// rtv_device_state_begin and rtv_device_state_end: the kernels then read it
// and the advance is a kernel, so the enqueued work does not depend on host
// values that a captured graph would freeze.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <thread>
#include <vector>

#include "../../include/rtv.h"
#include "kernels.hpp"
#include "ring.hpp"

namespace {

constexpr size_t kAlign = 256;
constexpr int64_t kTile = 64;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct LayerState {
  uint8_t* kc = nullptr;
  uint8_t* vc = nullptr;
  float* ks = nullptr;
  float* vs = nullptr;
  int64_t next_global_frame = 0;
  int32_t committed = 0;
  int32_t appended = 0;
};

struct Plan {
  int64_t slots = 0, slots_padded = 0;
  size_t rope_bytes = 0, ws_bytes = 0, state_bytes = 0, codes_bytes = 0, scales_bytes = 0, layer_bytes = 0,
         total = 0;
};

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

rtv_status check_config(const rtv_config* c) {
  if (!c) return RTV_ERR_INVALID_ARG;
  if (c->n_layers < 1 || c->n_kv_heads < 1 || c->n_q_heads < 1) return RTV_ERR_INVALID_ARG;
  if (c->n_q_heads % c->n_kv_heads != 0) return RTV_ERR_INVALID_ARG;
  if (c->head_dim < 2 || c->head_dim % 2) return RTV_ERR_INVALID_ARG;
  if (c->head_dim != 64 && c->head_dim != 128) return RTV_ERR_UNSUPPORTED;
  if (c->tokens_per_frame < 1 || c->chunk_frames < 1) return RTV_ERR_INVALID_ARG;
  if (c->capacity_frames < c->chunk_frames || c->capacity_frames % c->chunk_frames) return RTV_ERR_INVALID_ARG;
  if (c->max_global_frames < c->chunk_frames) return RTV_ERR_INVALID_ARG;
  if (!(c->rope_base > 0.0) || !std::isfinite(c->rope_base)) return RTV_ERR_INVALID_ARG;
  if (c->query_terms < 0 || c->query_terms > 2) return RTV_ERR_INVALID_ARG;
  if (c->prob_terms < 0 || c->prob_terms > 2) return RTV_ERR_INVALID_ARG;
  int64_t chunk;
  if (!mul_ok(c->chunk_frames, c->tokens_per_frame, &chunk) || chunk > INT32_MAX) return RTV_ERR_INVALID_ARG;
  return RTV_OK;
}

// units of attention work per call: query tiles x query heads
int64_t attend_units(const rtv_config& c) {
  const int64_t n = (int64_t)c.chunk_frames * c.tokens_per_frame;
  const int64_t qpb = rtv::attend_queries_per_block();
  return (n + qpb - 1) / qpb * c.n_q_heads;
}

rtv_status make_plan(const rtv_config* c, Plan* p) {
  rtv_status st = check_config(c);
  if (st != RTV_OK) return st;
  int64_t S, Sp, tmp, rope_elems;
  if (!mul_ok(c->capacity_frames, c->tokens_per_frame, &S)) return RTV_ERR_INVALID_ARG;
  Sp = (S + kTile - 1) / kTile * kTile;
  if (Sp > INT32_MAX) return RTV_ERR_INVALID_ARG;   // slot indices are int32 in kernels
  p->slots = S;
  p->slots_padded = Sp;
  if (!mul_ok((int64_t)c->max_global_frames, c->tokens_per_frame, &tmp)) return RTV_ERR_INVALID_ARG;
  if (!mul_ok(tmp, c->head_dim, &rope_elems)) return RTV_ERR_INVALID_ARG;   // (D/2) * 2 floats
  if (!mul_ok(rope_elems, 4, &tmp)) return RTV_ERR_INVALID_ARG;
  p->rope_bytes = align_up((size_t)tmp);
  // attention workspace (partial results of split key ranges, key factors,
  // peaked-unit flags), shared by all layers
  p->ws_bytes = align_up(rtv::attend_workspace_bytes(c->head_dim, c->n_kv_heads, Sp, attend_units(*c)));
  // per-layer ring state for the device-state mode
  p->state_bytes = align_up((size_t)c->n_layers * sizeof(rtv::DevRingState));
  if (!mul_ok((int64_t)c->n_kv_heads * c->head_dim, Sp, &tmp)) return RTV_ERR_INVALID_ARG;
  p->codes_bytes = align_up((size_t)tmp);
  p->scales_bytes = align_up((size_t)c->n_kv_heads * (size_t)Sp * 4);
  p->layer_bytes = 2 * p->codes_bytes + 2 * p->scales_bytes;
  int64_t layers_total;
  if (!mul_ok((int64_t)p->layer_bytes, c->n_layers, &layers_total)) return RTV_ERR_INVALID_ARG;
  p->total = p->rope_bytes + p->ws_bytes + p->state_bytes + (size_t)layers_total;
  return RTV_OK;
}

void fill_rope(int32_t D, double base, int64_t pos0, int64_t npos, float* out) {
  const int half = D / 2;
  std::vector<double> theta(half);
  for (int i = 0; i < half; ++i) theta[i] = std::pow(base, -2.0 * i / D);
  auto work = [&](int64_t a, int64_t b) {
    for (int64_t r = a; r < b; ++r) {
      const double p = (double)(pos0 + r);
      float* row = out + r * half * 2;
      for (int i = 0; i < half; ++i) {
        const double ang = p * theta[i];
        row[2 * i] = (float)std::cos(ang);
        row[2 * i + 1] = (float)std::sin(ang);
      }
    }
  };
  const int64_t per_thread = 1 << 14;
  unsigned nt = std::thread::hardware_concurrency();
  nt = std::max(1u, std::min(nt, 16u));
  if (npos < per_thread || nt == 1) {
    work(0, npos);
    return;
  }
  std::vector<std::thread> pool;
  const int64_t chunk = (npos + nt - 1) / nt;
  for (unsigned t = 0; t < nt; ++t) {
    const int64_t a = (int64_t)t * chunk, b = std::min(npos, a + chunk);
    if (a < b) pool.emplace_back(work, a, b);
  }
  for (auto& th : pool) th.join();
}

rtv::RingShape ring_shape(const rtv_config& cfg, int32_t max_window_frames) {
  rtv::RingShape s;
  s.tokens_per_frame = cfg.tokens_per_frame;
  s.chunk_frames = cfg.chunk_frames;
  s.capacity_frames = cfg.capacity_frames;
  s.max_global_frames = cfg.max_global_frames;
  s.max_window_frames = max_window_frames;
  s.head_dim = cfg.head_dim;
  return s;
}

}  // namespace

struct rtv_cache {
  rtv_config cfg;
  Plan plan;
  uint8_t* base = nullptr;
  float* rope = nullptr;
  float* ws = nullptr;          // attention workspace
  rtv::DevRingState* dstate = nullptr;  // per-layer ring state in the arena
  bool device_state = false;    // between rtv_device_state_begin and _end
  int capacity = 0;             // concurrent attention workgroups on the device
  std::vector<LayerState> layers;
};

extern "C" {

const char* rtv_status_string(rtv_status s) {
  switch (s) {
    case RTV_OK: return "ok";
    case RTV_ERR_INVALID_ARG: return "invalid argument";
    case RTV_ERR_BUFFER: return "device buffer too small or misaligned";
    case RTV_ERR_HIP: return "HIP runtime error";
    case RTV_ERR_STATE: return "call out of order or RoPE table exhausted";
    case RTV_ERR_UNSUPPORTED: return "unsupported shape";
    default: return "unknown status";
  }
}

rtv_status rtv_cache_bytes(const rtv_config* cfg, size_t* bytes) {
  if (!bytes) return RTV_ERR_INVALID_ARG;
  Plan p;
  rtv_status st = make_plan(cfg, &p);
  if (st != RTV_OK) return st;
  *bytes = p.total;
  return RTV_OK;
}

rtv_status rtv_rope_fill_host(int32_t head_dim, double rope_base, int64_t pos0, int64_t npos,
                              float* out) {
  if (!out || head_dim < 2 || head_dim % 2 || pos0 < 0 || npos < 0) return RTV_ERR_INVALID_ARG;
  if (!(rope_base > 0.0) || !std::isfinite(rope_base)) return RTV_ERR_INVALID_ARG;
  fill_rope(head_dim, rope_base, pos0, npos, out);
  return RTV_OK;
}

rtv_status rtv_ring_window(int64_t next_global_frame, int32_t committed_frames,
                           int32_t tokens_per_frame, int32_t chunk_frames,
                           int32_t capacity_frames, int32_t max_window_frames, rtv_window* out) {
  if (!out) return RTV_ERR_INVALID_ARG;
  rtv::RingWindow w;
  if (rtv::ring_window(next_global_frame, committed_frames, tokens_per_frame, chunk_frames,
                       capacity_frames, max_window_frames, &w) != rtv::kRingOk)
    return RTV_ERR_INVALID_ARG;
  out->window_frames = w.window_frames;
  out->n_segments = w.n_segments;
  for (int i = 0; i < 2; ++i) {
    out->seg_start[i] = w.seg_start[i];
    out->seg_len[i] = w.seg_len[i];
  }
  out->write_slot = w.write_slot;
  return RTV_OK;
}

rtv_status rtv_cache_create(const rtv_config* cfg, void* dev_buf, size_t bytes, void* stream,
                            rtv_cache** out) {
  if (!out) return RTV_ERR_INVALID_ARG;
  *out = nullptr;
  Plan p;
  rtv_status st = make_plan(cfg, &p);
  if (st != RTV_OK) return st;
  if (!dev_buf || (reinterpret_cast<uintptr_t>(dev_buf) % kAlign) != 0 || bytes < p.total)
    return RTV_ERR_BUFFER;
  hipStream_t s = static_cast<hipStream_t>(stream);

  rtv_cache* c = new (std::nothrow) rtv_cache();
  if (!c) return RTV_ERR_INVALID_ARG;
  c->cfg = *cfg;
  c->plan = p;
  c->base = static_cast<uint8_t*>(dev_buf);
  c->rope = reinterpret_cast<float*>(c->base);
  c->ws = reinterpret_cast<float*>(c->base + p.rope_bytes);
  c->dstate = reinterpret_cast<rtv::DevRingState*>(c->base + p.rope_bytes + p.ws_bytes);
  c->layers.resize(cfg->n_layers);
  uint8_t* cur = c->base + p.rope_bytes + p.ws_bytes + p.state_bytes;
  for (auto& L : c->layers) {
    L.kc = cur; cur += p.codes_bytes;
    L.vc = cur; cur += p.codes_bytes;
    L.ks = reinterpret_cast<float*>(cur); cur += p.scales_bytes;
    L.vs = reinterpret_cast<float*>(cur); cur += p.scales_bytes;
  }

  const int64_t npos = (int64_t)cfg->max_global_frames * cfg->tokens_per_frame;
  const size_t table_floats = (size_t)npos * cfg->head_dim;
  std::vector<float> table;
  const float* src = cfg->rope_cos_sin_host;
  if (!src) {
    try {
      table.resize(table_floats);
    } catch (...) {
      delete c;
      return RTV_ERR_INVALID_ARG;
    }
    fill_rope(cfg->head_dim, cfg->rope_base, 0, npos, table.data());
    src = table.data();
  }
  hipError_t e = hipMemcpyAsync(c->rope, src, table_floats * sizeof(float), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemsetAsync(c->base + p.rope_bytes, 0, p.total - p.rope_bytes, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = rtv::attend_capacity(&c->capacity);
  if (e != hipSuccess) {
    delete c;
    return RTV_ERR_HIP;
  }
  *out = c;
  return RTV_OK;
}

rtv_status rtv_destroy(rtv_cache* c) {
  if (!c) return RTV_ERR_INVALID_ARG;
  delete c;
  return RTV_OK;
}

rtv_status rtv_cache_layout(const rtv_cache* c, int32_t layer, rtv_layout* out) {
  if (!c || !out || layer < 0 || layer >= c->cfg.n_layers) return RTV_ERR_INVALID_ARG;
  const LayerState& L = c->layers[layer];
  out->k_codes = L.kc;
  out->v_codes = L.vc;
  out->k_scales = L.ks;
  out->v_scales = L.vs;
  out->slots = c->plan.slots;
  out->slots_padded = c->plan.slots_padded;
  out->next_global_frame = L.next_global_frame;
  out->head_frame = (int32_t)(L.next_global_frame % c->cfg.capacity_frames);
  out->committed_frames = L.committed;
  out->appended = L.appended;
  out->reserved = 0;
  return RTV_OK;
}

rtv_status rtv_cache_peaked_units(const rtv_cache* c, int32_t* units, void* stream) {
  if (!c || !units) return RTV_ERR_INVALID_ARG;
  rtv::AttendArgs a;
  rtv::attend_set_workspace(a, c->ws, c->cfg.head_dim, c->cfg.n_kv_heads, c->plan.slots_padded,
                            attend_units(c->cfg));
  uint32_t n = 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(&n, a.flags + attend_units(c->cfg), sizeof(n), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return RTV_ERR_HIP;
  *units = (int32_t)n;
  return RTV_OK;
}

rtv_status rtv_cache_window(const rtv_cache* c, int32_t layer, int32_t max_window_frames,
                            rtv_window* out) {
  if (!c || !out || layer < 0 || layer >= c->cfg.n_layers) return RTV_ERR_INVALID_ARG;
  const LayerState& L = c->layers[layer];
  return rtv_ring_window(L.next_global_frame, L.committed, c->cfg.tokens_per_frame,
                         c->cfg.chunk_frames, c->cfg.capacity_frames, max_window_frames, out);
}

rtv_status rtv_append_rope_quant(rtv_cache* c, int32_t layer, const void* k_bf16,
                                 int64_t k_tok_stride, const void* v_bf16, int64_t v_tok_stride,
                                 int32_t n_tokens, void* stream) {
  if (!c || layer < 0 || layer >= c->cfg.n_layers) return RTV_ERR_INVALID_ARG;
  const rtv_config& cfg = c->cfg;
  const int64_t chunk = (int64_t)cfg.chunk_frames * cfg.tokens_per_frame;
  const int64_t row = (int64_t)cfg.n_kv_heads * cfg.head_dim;
  if (n_tokens != chunk) return RTV_ERR_INVALID_ARG;
  if (!k_bf16 || !v_bf16) return RTV_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(k_bf16) | reinterpret_cast<uintptr_t>(v_bf16)) % 16)
    return RTV_ERR_INVALID_ARG;
  if (k_tok_stride < row || v_tok_stride < row || k_tok_stride % 8 || v_tok_stride % 8)
    return RTV_ERR_INVALID_ARG;
  LayerState& L = c->layers[layer];
  rtv::AppendArgs a;
  a.dstate = nullptr;
  a.rope_table = c->rope;
  a.shape = ring_shape(cfg, 0);
  rtv::RingWindow w;
  if (c->device_state) {
    // the kernel derives the slots and RoPE rows from the state in the arena;
    // the grid covers the most 64-slot tiles a chunk can touch
    a.dstate = c->dstate + layer;
    w.write_slot = 0;
    a.write_slot = 0;
    a.first_tile = 0;
    a.rope = c->rope;
  } else {
    if (L.next_global_frame + cfg.chunk_frames > cfg.max_global_frames) return RTV_ERR_STATE;
    if (rtv::ring_window(L.next_global_frame, L.committed, cfg.tokens_per_frame, cfg.chunk_frames,
                         cfg.capacity_frames, 0, &w) != rtv::kRingOk)
      return RTV_ERR_STATE;
  }
  a.k = static_cast<const uint16_t*>(k_bf16);
  a.v = static_cast<const uint16_t*>(v_bf16);
  a.ldk = k_tok_stride;
  a.ldv = v_tok_stride;
  a.kc = L.kc;
  a.vc = L.vc;
  a.ks = L.ks;
  a.vs = L.vs;
  a.slots_padded = c->plan.slots_padded;
  a.n_tokens = n_tokens;
  a.n_heads = cfg.n_kv_heads;
  int64_t n_work;
  if (c->device_state) {
    n_work = ((int64_t)n_tokens + kTile - 1) / kTile + 1;
    n_work *= cfg.n_kv_heads;
  } else {
    a.rope = c->rope + L.next_global_frame * cfg.tokens_per_frame * cfg.head_dim;
    a.write_slot = w.write_slot;
    a.first_tile = (int32_t)(w.write_slot / kTile);
    const int64_t last_tile = (w.write_slot + n_tokens - 1) / kTile;
    n_work = (last_tile - a.first_tile + 1) * cfg.n_kv_heads;
  }
  if (n_work > INT32_MAX / 2) return RTV_ERR_UNSUPPORTED;
  a.n_work = (int32_t)n_work;
  if (rtv::launch_append(a, cfg.head_dim, static_cast<hipStream_t>(stream)) != hipSuccess)
    return RTV_ERR_HIP;
  L.appended = 1;
  return RTV_OK;
}

rtv_status rtv_attend(rtv_cache* c, int32_t layer, const void* q_bf16, int64_t q_tok_stride,
                      void* out_bf16, int64_t out_tok_stride, int32_t max_window_frames,
                      void* stream) {
  if (!c || layer < 0 || layer >= c->cfg.n_layers) return RTV_ERR_INVALID_ARG;
  const rtv_config& cfg = c->cfg;
  const int64_t row = (int64_t)cfg.n_q_heads * cfg.head_dim;
  if (!q_bf16 || !out_bf16) return RTV_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(q_bf16) | reinterpret_cast<uintptr_t>(out_bf16)) % 16)
    return RTV_ERR_INVALID_ARG;
  if (q_tok_stride < row || out_tok_stride < row || q_tok_stride % 8 || out_tok_stride % 8)
    return RTV_ERR_INVALID_ARG;
  if (max_window_frames < 0 || (max_window_frames > 0 && max_window_frames < cfg.chunk_frames))
    return RTV_ERR_INVALID_ARG;
  LayerState& L = c->layers[layer];
  if (!L.appended) return RTV_ERR_STATE;
  rtv::RingWindow w;
  if (c->device_state) {
    // the kernels derive the window, the RoPE rows and the schedule
    w.n_segments = 0;
    for (int i = 0; i < 2; ++i) w.seg_start[i] = w.seg_len[i] = 0;
  } else if (rtv::ring_window(L.next_global_frame, L.committed, cfg.tokens_per_frame, cfg.chunk_frames,
                              cfg.capacity_frames, max_window_frames, &w) != rtv::kRingOk) {
    return RTV_ERR_STATE;
  }
  const int32_t n_tokens = cfg.chunk_frames * cfg.tokens_per_frame;
  rtv::AttendArgs a;
  a.dstate = c->device_state ? c->dstate + layer : nullptr;
  a.rope_table = c->rope;
  a.shape = ring_shape(cfg, max_window_frames);
  a.q = static_cast<const uint16_t*>(q_bf16);
  a.out = static_cast<uint16_t*>(out_bf16);
  a.ldq = q_tok_stride;
  a.ldo = out_tok_stride;
  a.rope = c->device_state ? c->rope : c->rope + L.next_global_frame * cfg.tokens_per_frame * cfg.head_dim;
  a.kc = L.kc;
  a.vc = L.vc;
  a.ks = L.ks;
  a.vs = L.vs;
  a.slots_padded = c->plan.slots_padded;
  a.n_segments = w.n_segments;
  for (int i = 0; i < 2; ++i) {
    a.seg_lo[i] = w.seg_start[i];
    a.seg_hi[i] = w.seg_start[i] + w.seg_len[i];
  }
  a.n_tokens = n_tokens;
  a.n_q_heads = cfg.n_q_heads;
  a.group = cfg.n_q_heads / cfg.n_kv_heads;
  const int qpb = rtv::attend_queries_per_block();
  a.n_qtiles = (n_tokens + qpb - 1) / qpb;
  a.n_work = a.n_qtiles * cfg.n_q_heads;
  a.capacity = c->capacity;
  a.two_term_q = cfg.query_terms == 2;
  a.two_term_p = cfg.prob_terms == 2;
  a.check_peaked = cfg.prob_terms == 0;
  a.redo = 0;
  rtv::attend_set_workspace(a, c->ws, cfg.head_dim, cfg.n_kv_heads, c->plan.slots_padded, attend_units(cfg));
  if (rtv::launch_attend(a, cfg.head_dim, static_cast<hipStream_t>(stream)) != hipSuccess)
    return RTV_ERR_HIP;
  return RTV_OK;
}

rtv_status rtv_advance(rtv_cache* c, int32_t layer, void* stream) {
  if (!c || layer < -1 || layer >= c->cfg.n_layers) return RTV_ERR_INVALID_ARG;
  const int lo = layer < 0 ? 0 : layer;
  const int hi = layer < 0 ? c->cfg.n_layers : layer + 1;
  for (int l = lo; l < hi; ++l)
    if (!c->layers[l].appended) return RTV_ERR_STATE;
  if (c->device_state) {
    if (rtv::launch_advance(c->dstate + lo, hi - lo, c->cfg.chunk_frames, c->cfg.capacity_frames,
                            static_cast<hipStream_t>(stream)) != hipSuccess)
      return RTV_ERR_HIP;
    for (int l = lo; l < hi; ++l) c->layers[l].appended = 0;
    return RTV_OK;
  }
  for (int l = lo; l < hi; ++l) {
    LayerState& L = c->layers[l];
    L.next_global_frame += c->cfg.chunk_frames;
    L.committed = std::min(L.committed + c->cfg.chunk_frames, c->cfg.capacity_frames);
    L.appended = 0;
  }
  return RTV_OK;
}

rtv_status rtv_qkv_gemm_append(rtv_cache* c, int32_t layer, const uint8_t* x_codes, const float* sx_dev,
                               const uint8_t* wt_codes, const float* sw_dev, int32_t n_tokens, int32_t k_dim,
                               int32_t q_cols, void* q_bf16, int64_t q_tok_stride, void* stream) {
  if (!c || layer < 0 || layer >= c->cfg.n_layers) return RTV_ERR_INVALID_ARG;
  const rtv_config& cfg = c->cfg;
  const int64_t chunk = (int64_t)cfg.chunk_frames * cfg.tokens_per_frame;
  if (n_tokens != chunk || k_dim <= 0 || k_dim % 64 != 0) return RTV_ERR_INVALID_ARG;
  if (q_cols < 0 || q_cols % cfg.head_dim != 0) return RTV_ERR_INVALID_ARG;
  if (!x_codes || !wt_codes || !sx_dev || !sw_dev || (q_cols > 0 && !q_bf16)) return RTV_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(x_codes) | reinterpret_cast<uintptr_t>(wt_codes) |
       reinterpret_cast<uintptr_t>(q_bf16)) % 16 ||
      (reinterpret_cast<uintptr_t>(sx_dev) | reinterpret_cast<uintptr_t>(sw_dev)) % 4)
    return RTV_ERR_INVALID_ARG;
  if (q_cols > 0 && (q_tok_stride < q_cols || q_tok_stride % 8 != 0)) return RTV_ERR_INVALID_ARG;
  const int64_t n_cols = (int64_t)q_cols + 2 * (int64_t)cfg.n_kv_heads * cfg.head_dim;
  if (n_cols > INT32_MAX) return RTV_ERR_INVALID_ARG;
  // the epilogue writes whole 64-slot tiles; the host-state ring gives the slots
  if (chunk % kTile != 0 || c->device_state) return RTV_ERR_UNSUPPORTED;
  LayerState& L = c->layers[layer];
  if (L.next_global_frame + cfg.chunk_frames > cfg.max_global_frames) return RTV_ERR_STATE;
  rtv::RingWindow w;
  if (rtv::ring_window(L.next_global_frame, L.committed, cfg.tokens_per_frame, cfg.chunk_frames,
                       cfg.capacity_frames, 0, &w) != rtv::kRingOk)
    return RTV_ERR_STATE;
  rtv::QkvAppendArgs q;
  q.x = x_codes; q.sx = sx_dev; q.wt = wt_codes; q.sw = sw_dev;
  q.q_out = static_cast<uint16_t*>(q_bf16);
  q.ldq = q_cols > 0 ? q_tok_stride : 0;
  q.M = n_tokens; q.K = k_dim; q.q_cols = q_cols;
  q.n_kv_heads = cfg.n_kv_heads; q.head_dim = cfg.head_dim;
  q.rope = c->rope + L.next_global_frame * cfg.tokens_per_frame * cfg.head_dim;
  q.kc = L.kc; q.vc = L.vc; q.ks = L.ks; q.vs = L.vs;
  q.slots_padded = c->plan.slots_padded;
  q.write_slot = w.write_slot;
  if (rtv::launch_qkv_gemm_append(q, static_cast<hipStream_t>(stream)) != hipSuccess) return RTV_ERR_HIP;
  L.appended = 1;
  return RTV_OK;
}

rtv_status rtv_device_state_begin(rtv_cache* c, void* stream) {
  if (!c) return RTV_ERR_INVALID_ARG;
  if (c->device_state) return RTV_ERR_STATE;
  std::vector<rtv::DevRingState> st(c->layers.size());
  for (size_t l = 0; l < st.size(); ++l) {
    st[l].next_global_frame = c->layers[l].next_global_frame;
    st[l].committed = c->layers[l].committed;
    st[l].error = 0;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(c->dstate, st.data(), st.size() * sizeof(rtv::DevRingState),
                                hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return RTV_ERR_HIP;
  c->device_state = true;
  return RTV_OK;
}

rtv_status rtv_device_state_end(rtv_cache* c, void* stream) {
  if (!c) return RTV_ERR_INVALID_ARG;
  if (!c->device_state) return RTV_ERR_STATE;
  std::vector<rtv::DevRingState> st(c->layers.size());
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(st.data(), c->dstate, st.size() * sizeof(rtv::DevRingState),
                                hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return RTV_ERR_HIP;
  bool error = false;
  for (size_t l = 0; l < st.size(); ++l) {
    c->layers[l].next_global_frame = st[l].next_global_frame;
    c->layers[l].committed = st[l].committed;
    error = error || st[l].error != 0;
  }
  c->device_state = false;
  return error ? RTV_ERR_STATE : RTV_OK;
}

rtv_status rtv_encode_e4m3(const float* x_dev, uint8_t* codes_dev, int64_t n, void* stream) {
  if (n < 0 || (n > 0 && (!x_dev || !codes_dev))) return RTV_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(x_dev) % 16 || reinterpret_cast<uintptr_t>(codes_dev) % 4)
    return RTV_ERR_INVALID_ARG;
  if (rtv::launch_encode_e4m3(x_dev, codes_dev, n, static_cast<hipStream_t>(stream)) != hipSuccess)
    return RTV_ERR_HIP;
  return RTV_OK;
}

size_t rtv_quant_workspace_bytes(int64_t n) {
  (void)n;
  return sizeof(uint32_t) * (size_t)rtv::quant_max_partials();
}

rtv_status rtv_quant_fp8_per_tensor(const void* x_bf16, int64_t n, uint8_t* codes_dev,
                                    float* scale_dev, void* workspace, void* stream) {
  if (n < 0 || !scale_dev || !workspace || (n > 0 && (!x_bf16 || !codes_dev))) return RTV_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(x_bf16) % 16 || reinterpret_cast<uintptr_t>(codes_dev) % 8 ||
      reinterpret_cast<uintptr_t>(scale_dev) % 4 || reinterpret_cast<uintptr_t>(workspace) % 4)
    return RTV_ERR_INVALID_ARG;
  if (rtv::launch_quant_fp8(static_cast<const uint16_t*>(x_bf16), n, codes_dev, scale_dev,
                            static_cast<uint32_t*>(workspace), static_cast<hipStream_t>(stream)) != hipSuccess)
    return RTV_ERR_HIP;
  return RTV_OK;
}

rtv_status rtv_quant_fp8_per_tensor_static(const void* x_bf16, int64_t n, uint8_t* codes_dev,
                                           float* scale_dev, void* stream) {
  if (n < 0 || !scale_dev || (n > 0 && (!x_bf16 || !codes_dev))) return RTV_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(x_bf16) % 16 || reinterpret_cast<uintptr_t>(codes_dev) % 8 ||
      reinterpret_cast<uintptr_t>(scale_dev) % 4)
    return RTV_ERR_INVALID_ARG;
  if (rtv::launch_quant_fp8_static(static_cast<const uint16_t*>(x_bf16), n, codes_dev, scale_dev,
                                   static_cast<hipStream_t>(stream)) != hipSuccess)
    return RTV_ERR_HIP;
  return RTV_OK;
}

rtv_status rtv_gemm_fp8(const uint8_t* a, const float* sa_dev, const uint8_t* bt,
                        const float* sb_dev, void* c_bf16, int32_t M, int32_t N, int32_t K,
                        int64_t ldc, void* stream) {
  if (M < 0 || N < 0 || K <= 0 || K % 64 != 0 || ldc < N) return RTV_ERR_INVALID_ARG;
  if (M == 0 || N == 0) return RTV_OK;
  if (!a || !bt || !sa_dev || !sb_dev || !c_bf16) return RTV_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(a) % 16 || reinterpret_cast<uintptr_t>(bt) % 16 ||
      reinterpret_cast<uintptr_t>(c_bf16) % 2 || reinterpret_cast<uintptr_t>(sa_dev) % 4 ||
      reinterpret_cast<uintptr_t>(sb_dev) % 4)
    return RTV_ERR_INVALID_ARG;
  if (rtv::launch_gemm_fp8(a, sa_dev, bt, sb_dev, static_cast<uint16_t*>(c_bf16), M, N, K, ldc,
                           static_cast<hipStream_t>(stream)) != hipSuccess)
    return RTV_ERR_HIP;
  return RTV_OK;
}

}  // extern "C"
