"""CPU oracle for KV-cache upkeep and chunk attention — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The GPU library never
calls it, and this package never calls the GPU library.

What it computes (a plain, slow, obviously correct reading of the pages):

* RoPE and FP8 quantization are applied once, when a chunk's K/V enter the
  cache, and the cache then only grows by whole chunks
  (page "Runway explains how it serves a 57B video model in real time"
  (aidose.in), fourth paragraph; page "Runway: Πώς ένα AI 57 δισ. παραμέτρων
  παράγει βίντεο στα 24 fps" (pttl.gr), section "Από οκτώ H100 σε τέσσερις").
* The chunk's queries then attend over the valid cached window, including the
  chunk itself (same pages: 240 attention calls per step).

The oracle keeps NO ring: each layer holds an explicitly concatenated history
of committed chunks plus the current chunk, and the window is a slice of the
last W frames of that history.  Floating-point work that the method defines in
fp32 (RoPE, scale, x/scale) is done in numpy float32 with one rounding per
operation and no fused multiply-add; attention is evaluated in float64 on the
dequantized cache.

Modules
  e4m3       OCP FP8 E4M3FN encode/decode by table lookup (nearest, ties to even)
  rope       rotate-half RoPE and its cos/sin table (float64 angles, fp32 values)
  quant      per-(token, head) amax/448 scaling and e4m3 codes
  cache      concatenated-history KV cache: append / attend / advance
  attention  float64 softmax attention over dequantized K/V
  gemm       per-tensor e4m3 quantization and the float64 reference GEMM
  bf16       float32 <-> bfloat16 helpers used by the oracle itself

Pins: every function is checked by ``tests/test_oracle_*.py`` against values
that do not come from the oracle itself (format definitions, closed forms,
invariants, brute force, torch's CPU float8 cast).  One result has no such
pin and is marked "parity unpinned": the size of the attention error that FP8
queries and probabilities introduce (only the tolerance applies).
"""
