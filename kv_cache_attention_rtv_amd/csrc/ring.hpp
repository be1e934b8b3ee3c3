// Ring arithmetic of the frame-granular KV cache (header-only; host and
// device: the device-state mode derives the same windows in the kernels).
//
// The cache keeps the last C frames of a layer in a circular buffer and
// advances by moving a head index instead of copying (page "Runway explains
// how it serves a 57B video model in real time", fourth paragraph; page
// "Runway: Πώς ένα AI 57 δισ. παραμέτρων παράγει βίντεο στα 24 fps", section
// "Από οκτώ H100 σε τέσσερις", where it is called a circular buffer).
//
//   token t of global frame g      -> slot (g mod C) * T + t
//   the chunk being written        -> frames [next, next + F), slots from
//                                     (next mod C) * T, contiguous because
//                                     C is a multiple of F and next of F
//   window of an attend            -> the last W frames ending with that
//                                     chunk, W = min(committed + F, C, cap)
//   advance                        -> next += F, committed = min(committed + F, C)
//
// In slot space the window is one segment, or two when it wraps past slot
// C*T - 1.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rtv {

struct RingWindow {
  int32_t window_frames;
  int32_t n_segments;
  int64_t seg_start[2];
  int64_t seg_len[2];
  int64_t write_slot;
};

enum RingStatus { kRingOk = 0, kRingBadArg = -1 };

__host__ __device__ inline int ring_window(int64_t next_global_frame, int32_t committed, int32_t T, int32_t F,
                       int32_t C, int32_t max_window, RingWindow* w) {
  if (!w || T < 1 || F < 1 || C < F || C % F != 0) return kRingBadArg;
  if (committed < 0 || committed > C || next_global_frame < 0) return kRingBadArg;
  if (next_global_frame % F != 0 || committed > next_global_frame) return kRingBadArg;
  if (max_window < 0 || (max_window > 0 && max_window < F)) return kRingBadArg;
  int32_t wf = committed + F < C ? committed + F : C;
  if (max_window > 0 && max_window < wf) wf = max_window;
  const int64_t S = (int64_t)C * T;
  const int64_t head_frame = next_global_frame % C;
  const int64_t first = next_global_frame + F - wf;   // >= 0 since committed <= next
  const int64_t rf = first % C;
  const int64_t start = rf * T;
  const int64_t len = (int64_t)wf * T;
  w->window_frames = wf;
  w->write_slot = head_frame * T;
  if (start + len <= S) {
    w->n_segments = 1;
    w->seg_start[0] = start;
    w->seg_len[0] = len;
    w->seg_start[1] = 0;
    w->seg_len[1] = 0;
  } else {
    w->n_segments = 2;
    w->seg_start[0] = start;
    w->seg_len[0] = S - start;
    w->seg_start[1] = 0;
    w->seg_len[1] = start + len - S;
  }
  return kRingOk;
}

}  // namespace rtv
