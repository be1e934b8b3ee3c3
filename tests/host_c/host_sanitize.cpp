// Host logic of librtv under AddressSanitizer and UndefinedBehaviorSanitizer
// (CPU only: the library's sources are built with the sanitizers on the host
// side, the device code as usual, and linked into this program; no call here
// reaches a GPU).
//
// It drives every part of the host code that runs without a device:
//   - the ring arithmetic (ring.hpp), exhaustively over small rings and at
//     frame indices near 2^40, through the inline function and the C entry;
//   - the split schedule of an attention call (kernels.hpp), over device
//     sizes, unit counts, window lengths and workspace bounds;
//   - the attention workspace: every region that attend_set_workspace hands
//     out lies inside attend_workspace_bytes;
//   - arena sizing on seeded random configurations, extreme fields included;
//   - the threaded RoPE fill into a buffer of exactly the requested size;
//   - argument validation of every entry point, and cache creation up to the
//     first device call (whose failure must free what the call allocated).
// Each group prints "<name> <failures>" and the program exits 1 on a failure;
// a sanitizer report aborts it before that.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "rtv.h"
#include "kernels.hpp"
#include "ring.hpp"

namespace {

int fails = 0;
#define CHECK(cond)                                                              \
  do {                                                                           \
    if (!(cond)) {                                                               \
      if (fails < 20) std::fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #cond); \
      ++fails;                                                                   \
    }                                                                            \
  } while (0)

// counter-based generator (splitmix64) for the random configurations
uint64_t mix(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

// invariants of one window: it holds wf frames ending with the chunk being
// written, as one slot range or two that wrap past the end of the ring
void check_window(const rtv::RingWindow& w, int64_t next, int32_t committed, int32_t T, int32_t F,
                  int32_t C, int32_t maxw) {
  int32_t want = committed + F < C ? committed + F : C;
  if (maxw > 0 && maxw < want) want = maxw;
  CHECK(w.window_frames == want);
  const int64_t S = (int64_t)C * T;
  CHECK(w.write_slot == (next % C) * T);
  CHECK(w.n_segments == 1 || w.n_segments == 2);
  int64_t total = 0;
  for (int i = 0; i < w.n_segments; ++i) {
    CHECK(w.seg_len[i] > 0);
    CHECK(w.seg_start[i] >= 0 && w.seg_start[i] + w.seg_len[i] <= S);
    total += w.seg_len[i];
  }
  CHECK(total == (int64_t)want * T);
  if (w.n_segments == 2) {
    CHECK(w.seg_start[0] + w.seg_len[0] == S);
    CHECK(w.seg_start[1] == 0);
  }
  // the window ends where the chunk being written ends
  const int64_t last = w.n_segments == 2 ? w.seg_start[1] + w.seg_len[1] : w.seg_start[0] + w.seg_len[0];
  CHECK(last % S == (w.write_slot + (int64_t)F * T) % S);
  // the first slot holds the oldest frame of the window
  CHECK(w.seg_start[0] == ((next + F - want) % C) * T);
}

void ring_group() {
  long windows = 0;
  const int32_t Ts[] = {1, 3, 64, 96};
  for (int32_t T : Ts)
    for (int32_t F = 1; F <= 4; ++F)
      for (int32_t C = F; C <= 24; C += F)
        for (int64_t next = 0; next <= 3 * C + F; next += F)
          for (int32_t committed = 0; committed <= C && committed <= next; ++committed)
            for (int32_t maxw = 0; maxw <= C; maxw = maxw == 0 ? F : maxw + 1) {
              rtv::RingWindow w;
              const int r = rtv::ring_window(next, committed, T, F, C, maxw, &w);
              CHECK(r == rtv::kRingOk);
              if (r != rtv::kRingOk) continue;
              check_window(w, next, committed, T, F, C, maxw);
              rtv_window o;
              CHECK(rtv_ring_window(next, committed, T, F, C, maxw, &o) == RTV_OK);
              CHECK(o.window_frames == w.window_frames && o.n_segments == w.n_segments &&
                    o.write_slot == w.write_slot && o.seg_start[0] == w.seg_start[0] &&
                    o.seg_len[0] == w.seg_len[0] && o.seg_start[1] == w.seg_start[1] &&
                    o.seg_len[1] == w.seg_len[1]);
              ++windows;
            }
  // far into a stream, and at the largest ring the library sizes
  for (int64_t next = (int64_t)1 << 40; next < ((int64_t)1 << 40) + 64; next += 4) {
    rtv::RingWindow w;
    CHECK(rtv::ring_window(next, 16, 2992, 4, 16, 0, &w) == rtv::kRingOk);
    check_window(w, next, 16, 2992, 4, 16, 0);
    CHECK(rtv::ring_window(next, 1 << 20, 1 << 10, 4, 1 << 20, 0, &w) == rtv::kRingOk);
    check_window(w, next, 1 << 20, 1 << 10, 4, 1 << 20, 0);
  }
  // rejected arguments leave the output untouched and never read past it
  rtv::RingWindow w;
  std::memset(&w, 0x5A, sizeof w);
  const int64_t bad[][6] = {
      {0, 0, 0, 4, 8, 0},   {0, 0, 96, 0, 8, 0},  {0, 0, 96, 4, 2, 0},  {0, 0, 96, 4, 6, 0},
      {2, 0, 96, 4, 8, 0},  {4, 8, 96, 4, 8, 0},  {0, -1, 96, 4, 8, 0}, {-4, 0, 96, 4, 8, 0},
      {0, 0, 96, 4, 8, -1}, {0, 0, 96, 4, 8, 2},  {8, 9, 96, 4, 8, 0},
  };
  for (const auto& b : bad) {
    CHECK(rtv::ring_window(b[0], (int32_t)b[1], (int32_t)b[2], (int32_t)b[3], (int32_t)b[4], (int32_t)b[5], &w) ==
          rtv::kRingBadArg);
    rtv_window o;
    CHECK(rtv_ring_window(b[0], (int32_t)b[1], (int32_t)b[2], (int32_t)b[3], (int32_t)b[4], (int32_t)b[5], &o) ==
          RTV_ERR_INVALID_ARG);
  }
  CHECK(rtv::ring_window(0, 0, 96, 4, 8, 0, nullptr) == rtv::kRingBadArg);
  CHECK(rtv_ring_window(0, 0, 96, 4, 8, 0, nullptr) == RTV_ERR_INVALID_ARG);
  unsigned char ref[sizeof w];
  std::memset(ref, 0x5A, sizeof ref);
  CHECK(std::memcmp(&w, ref, sizeof w) == 0);
  std::printf("ring_windows %ld\n", windows);
}

void schedule_group() {
  const int caps[] = {0, 1, 7, 256, 512, 748, 1024, 2048};
  const int tiles[] = {1, 2, 3, 5, 187, 748, 1496};
  const int maxp[] = {0, 1, 64, rtv::attend_max_parts()};
  float dummy;
  long cases = 0;
  for (int cap : caps)
    for (int U = 1; U <= 3000; U += (U < 64 ? 1 : 37))
      for (int n_tiles : tiles)
        for (int mp : maxp)
          for (int ws = 0; ws < 2; ++ws) {
            rtv::AttendArgs a;
            std::memset(&a, 0, sizeof a);
            a.capacity = cap;
            a.n_work = U;
            a.ws_o = ws ? &dummy : nullptr;
            rtv::attend_schedule(a, n_tiles, mp);
            const int S = a.parts_per_unit, rem = U - a.n_full;
            CHECK(S >= 1);
            CHECK(a.n_full >= 0 && a.n_full <= U);
            CHECK(S == 1 ? (rem == 0 && a.n_parts == 0) : (rem > 0 && a.n_parts == rem * S));
            CHECK(S <= n_tiles || S == 1);
            CHECK(a.n_parts <= (mp > 0 ? mp : 0) || a.n_parts == 0);
            if (!ws || cap == 0) CHECK(a.n_full == U);
            if (cap > 0 && S > 1) {
              CHECK(rem == U % cap);                          // whole rounds run whole windows
              CHECK((int64_t)rem * S <= cap);                 // the parts fit one round
            }
            // the eight per-XCD shares cover the units, with less than one unit per XCD to spare
            CHECK(a.full_per_xcd * 8 >= a.n_full && (a.full_per_xcd == 0 || (a.full_per_xcd - 1) * 8 < a.n_full));
            CHECK(a.parts_per_xcd * 8 >= a.n_parts && (a.parts_per_xcd == 0 || (a.parts_per_xcd - 1) * 8 < a.n_parts));
            ++cases;
          }
  std::printf("schedules %ld\n", cases);
}

void workspace_group() {
  const int qpb = rtv::attend_queries_per_block(), mp = rtv::attend_max_parts();
  long cases = 0;
  for (int D : {64, 128})
    for (int H : {1, 3, 12, 48})
      for (int64_t Sp : {64LL, 128LL, 47872LL, 95744LL, 1LL << 22})
        for (int64_t units : {1LL, 12LL, 2244LL, 1LL << 16}) {
          const size_t bytes = rtv::attend_workspace_bytes(D, H, Sp, units);
          std::vector<uint8_t> buf(bytes + 256);
          uint8_t* base = reinterpret_cast<uint8_t*>((reinterpret_cast<uintptr_t>(buf.data()) + 255) / 256 * 256);
          rtv::AttendArgs a;
          std::memset(&a, 0, sizeof a);
          rtv::attend_set_workspace(a, base, D, H, Sp, units);
          const size_t tiles = (size_t)H * (size_t)(Sp / 64);
          struct Region { const void* p; size_t n; } r[] = {
              {a.ws_o, (size_t)mp * qpb * D * sizeof(float)},
              {a.ws_ml, (size_t)mp * qpb * 4 * sizeof(float)},
              {a.fac_l, tiles * 64 * 16},
              {a.fac_u, tiles * 128},
              {a.flags, ((size_t)units + 1) * sizeof(uint32_t)},
          };
          for (int i = 0; i < 5; ++i) {
            const uint8_t* p = static_cast<const uint8_t*>(r[i].p);
            CHECK(p >= base && p + r[i].n <= base + bytes);
            CHECK(reinterpret_cast<uintptr_t>(p) % 16 == 0);
            for (int j = 0; j < i; ++j) {   // the regions do not overlap
              const uint8_t* q = static_cast<const uint8_t*>(r[j].p);
              CHECK(p + r[i].n <= q || q + r[j].n <= p);
            }
          }
          // touch the first and last byte of every region (ASan checks the bounds)
          for (auto& g : r) {
            uint8_t* p = const_cast<uint8_t*>(static_cast<const uint8_t*>(g.p));
            p[0] = 1;
            p[g.n - 1] = 1;
          }
          ++cases;
        }
  std::printf("workspaces %ld\n", cases);
}

int32_t pick(uint64_t& s, const int32_t* v, int n) { return v[(s = mix(s)) % n]; }

void sizing_group() {
  const int32_t small[] = {-1, 0, 1, 2, 3, 4, 12, 24, 60};
  const int32_t dims[] = {-2, 0, 1, 2, 32, 64, 96, 128, 256};
  const int32_t tpf[] = {-5, 0, 1, 7, 64, 2992, 65536, INT32_MAX};
  const int32_t frames[] = {-4, 0, 1, 2, 4, 8, 16, 24, 4096, 1 << 20, INT32_MAX};
  uint64_t s = 12345;
  long ok = 0, rejected = 0;
  for (int it = 0; it < 200000; ++it) {
    rtv_config c;
    std::memset(&c, 0, sizeof c);
    c.n_layers = pick(s, small, 9);
    c.n_q_heads = pick(s, small, 9);
    c.n_kv_heads = pick(s, small, 9);
    c.head_dim = pick(s, dims, 9);
    c.tokens_per_frame = pick(s, tpf, 8);
    c.chunk_frames = pick(s, frames, 11);
    c.capacity_frames = pick(s, frames, 11);
    c.max_global_frames = pick(s, frames, 11);
    const double bases[] = {10000.0, 0.0, -1.0, INFINITY, NAN, 1e-300};
    c.rope_base = bases[(s = mix(s)) % 6];
    c.query_terms = (int32_t)((s = mix(s)) % 4) - 1;
    c.prob_terms = (int32_t)((s = mix(s)) % 4) - 1;
    size_t bytes = 0;
    const rtv_status r = rtv_cache_bytes(&c, &bytes);
    CHECK(r == RTV_OK || r == RTV_ERR_INVALID_ARG || r == RTV_ERR_UNSUPPORTED);
    if (r != RTV_OK) {
      ++rejected;
      continue;
    }
    ++ok;
    // the arena holds at least the RoPE table and every layer's codes and scales
    const long double S = (long double)c.capacity_frames * c.tokens_per_frame;
    const long double need = (long double)c.max_global_frames * c.tokens_per_frame * c.head_dim * 4 +
                             (long double)c.n_layers * 2 * c.n_kv_heads * S * (c.head_dim + 4);
    CHECK((long double)bytes >= need);
    CHECK(bytes % 256 == 0);
  }
  size_t b;
  CHECK(rtv_cache_bytes(nullptr, &b) == RTV_ERR_INVALID_ARG);
  rtv_config c;
  std::memset(&c, 0, sizeof c);
  CHECK(rtv_cache_bytes(&c, nullptr) == RTV_ERR_INVALID_ARG);
  CHECK(ok > 100 && rejected > 100);
  std::printf("configs %ld %ld\n", ok, rejected);
}

void rope_group() {
  // threaded fill (the library splits long tables over threads)
  const int32_t D = 128;
  const int64_t pos0 = 7, npos = 40000;
  std::vector<float> out((size_t)npos * D);
  CHECK(rtv_rope_fill_host(D, 10000.0, pos0, npos, out.data()) == RTV_OK);
  double worst = 0;
  for (int64_t r = 0; r < npos; r += 97)
    for (int i = 0; i < D / 2; ++i) {
      const double cs = out[(size_t)r * D + 2 * i], sn = out[(size_t)r * D + 2 * i + 1];
      worst = std::fmax(worst, std::fabs(cs * cs + sn * sn - 1.0));
    }
  CHECK(worst < 1e-6);
  std::vector<float> zero(1);
  CHECK(rtv_rope_fill_host(D, 10000.0, 0, 0, zero.data()) == RTV_OK);
  CHECK(rtv_rope_fill_host(D, 10000.0, 0, 1, nullptr) == RTV_ERR_INVALID_ARG);
  CHECK(rtv_rope_fill_host(3, 10000.0, 0, 1, zero.data()) == RTV_ERR_INVALID_ARG);
  CHECK(rtv_rope_fill_host(D, -1.0, 0, 1, zero.data()) == RTV_ERR_INVALID_ARG);
  CHECK(rtv_rope_fill_host(D, NAN, 0, 1, zero.data()) == RTV_ERR_INVALID_ARG);
  CHECK(rtv_rope_fill_host(D, 10000.0, -1, 1, zero.data()) == RTV_ERR_INVALID_ARG);
  CHECK(rtv_rope_fill_host(D, 10000.0, 0, -1, zero.data()) == RTV_ERR_INVALID_ARG);
  std::printf("rope_rows %ld\n", (long)npos);
}

rtv_config small_config() {
  rtv_config c;
  std::memset(&c, 0, sizeof c);
  c.n_layers = 2;
  c.n_q_heads = 4;
  c.n_kv_heads = 2;
  c.head_dim = 64;
  c.tokens_per_frame = 96;
  c.chunk_frames = 4;
  c.capacity_frames = 8;
  c.max_global_frames = 64;
  c.rope_base = 10000.0;
  return c;
}

void validation_group() {
  rtv_config c = small_config();
  size_t bytes = 0;
  CHECK(rtv_cache_bytes(&c, &bytes) == RTV_OK);
  std::vector<uint8_t> host(bytes + 512);
  uint8_t* aligned = reinterpret_cast<uint8_t*>((reinterpret_cast<uintptr_t>(host.data()) + 255) / 256 * 256);
  rtv_cache* cache = reinterpret_cast<rtv_cache*>(0x1);
  CHECK(rtv_cache_create(&c, aligned, bytes, nullptr, nullptr) == RTV_ERR_INVALID_ARG);
  CHECK(rtv_cache_create(nullptr, aligned, bytes, nullptr, &cache) == RTV_ERR_INVALID_ARG && cache == nullptr);
  CHECK(rtv_cache_create(&c, nullptr, bytes, nullptr, &cache) == RTV_ERR_BUFFER && cache == nullptr);
  CHECK(rtv_cache_create(&c, aligned + 16, bytes, nullptr, &cache) == RTV_ERR_BUFFER && cache == nullptr);
  CHECK(rtv_cache_create(&c, aligned, bytes - 1, nullptr, &cache) == RTV_ERR_BUFFER && cache == nullptr);
  rtv_config bad = c;
  bad.head_dim = 96;
  CHECK(rtv_cache_create(&bad, aligned, bytes, nullptr, &cache) == RTV_ERR_UNSUPPORTED && cache == nullptr);
  bad = c;
  bad.capacity_frames = 6;
  CHECK(rtv_cache_create(&bad, aligned, bytes, nullptr, &cache) == RTV_ERR_INVALID_ARG && cache == nullptr);
  // with no device the first device call fails: the call frees what it
  // allocated (the leak checker sees it) and returns no cache
  int n_dev = 0;
  if (hipGetDeviceCount(&n_dev) != hipSuccess || n_dev == 0) {
    CHECK(rtv_cache_create(&c, aligned, bytes, nullptr, &cache) == RTV_ERR_HIP && cache == nullptr);
    std::printf("create_without_device 1\n");
  }
  // every call on no cache is rejected before it touches anything
  rtv_layout lay;
  rtv_window win;
  int32_t units;
  alignas(16) uint16_t q[16];
  CHECK(rtv_destroy(nullptr) == RTV_ERR_INVALID_ARG);
  CHECK(rtv_append_rope_quant(nullptr, 0, q, 8, q, 8, 384, nullptr) == RTV_ERR_INVALID_ARG);
  CHECK(rtv_attend(nullptr, 0, q, 8, q, 8, 0, nullptr) == RTV_ERR_INVALID_ARG);
  CHECK(rtv_advance(nullptr, -1, nullptr) == RTV_ERR_INVALID_ARG);
  CHECK(rtv_device_state_begin(nullptr, nullptr) == RTV_ERR_INVALID_ARG);
  CHECK(rtv_device_state_end(nullptr, nullptr) == RTV_ERR_INVALID_ARG);
  CHECK(rtv_cache_layout(nullptr, 0, &lay) == RTV_ERR_INVALID_ARG);
  CHECK(rtv_cache_peaked_units(nullptr, &units, nullptr) == RTV_ERR_INVALID_ARG);
  CHECK(rtv_cache_window(nullptr, 0, 0, &win) == RTV_ERR_INVALID_ARG);
  CHECK(rtv_qkv_gemm_append(nullptr, 0, nullptr, nullptr, nullptr, nullptr, 384, 64, 0, nullptr, 0, nullptr) ==
        RTV_ERR_INVALID_ARG);
  // the device-pointer entries reject their arguments before any launch
  float f[4];
  uint8_t codes[64];
  CHECK(rtv_encode_e4m3(nullptr, codes, 4, nullptr) == RTV_ERR_INVALID_ARG);
  CHECK(rtv_encode_e4m3(f, codes, -1, nullptr) == RTV_ERR_INVALID_ARG);
  CHECK(rtv_quant_fp8_per_tensor(q, 16, codes, nullptr, codes, nullptr) == RTV_ERR_INVALID_ARG);
  CHECK(rtv_quant_fp8_per_tensor(q, -1, codes, f, codes, nullptr) == RTV_ERR_INVALID_ARG);
  CHECK(rtv_quant_fp8_per_tensor_static(q, 16, codes, nullptr, nullptr) == RTV_ERR_INVALID_ARG);
  CHECK(rtv_quant_fp8_per_tensor_static(nullptr, 16, codes, f, nullptr) == RTV_ERR_INVALID_ARG);
  CHECK(rtv_gemm_fp8(codes, f, codes, f, q, 16, 16, 63, 16, nullptr) == RTV_ERR_INVALID_ARG);
  CHECK(rtv_gemm_fp8(codes, f, codes, f, q, 16, 16, 64, 8, nullptr) == RTV_ERR_INVALID_ARG);
  CHECK(rtv_gemm_fp8(codes, f, codes, f, q, -1, 16, 64, 16, nullptr) == RTV_ERR_INVALID_ARG);
  CHECK(rtv_gemm_fp8(nullptr, f, codes, f, q, 16, 16, 64, 16, nullptr) == RTV_ERR_INVALID_ARG);
  CHECK(rtv_gemm_fp8(nullptr, nullptr, nullptr, nullptr, nullptr, 0, 16, 64, 16, nullptr) == RTV_OK);
  for (int s = -7; s <= 1; ++s) CHECK(rtv_status_string((rtv_status)s) != nullptr);
  std::printf("validation 1\n");
}

}  // namespace

int main() {
  ring_group();
  std::printf("ring failures %d\n", fails);
  int before = fails;
  schedule_group();
  std::printf("schedule failures %d\n", fails - before);
  before = fails;
  workspace_group();
  std::printf("workspace failures %d\n", fails - before);
  before = fails;
  sizing_group();
  std::printf("sizing failures %d\n", fails - before);
  before = fails;
  rope_group();
  std::printf("rope failures %d\n", fails - before);
  before = fails;
  validation_group();
  std::printf("validation failures %d\n", fails - before);
  return fails ? 1 : 0;
}
