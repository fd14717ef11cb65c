"""The oracle: a plain, slow, fp64 CPU definition of the Mel-Band RoFormer core.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check in the graft entry point
and the CPU-baseline leg of the benchmark may import anything here.  The HIP
library never calls it, and it shares no code, tables or constants with the HIP
path: the two meet only on the seeded arrays that ``axial_band_split_amd.synth``
draws.

Modules
  mel     Slaney mel bands, binarised incidence, gather and inverse index tables
  model   weight inventory and the vectorised numpy forward (every step in fp64)
  brute   an independent scalar-loop forward for tiny shapes, used to pin ``model``
  attention  gated attention with q, k wider than v (the polar scheme's shape)
  pipeline   STFT, mask product, inverse STFT and the chunked overlap-add around the core

Every function cites the page passage it follows.  Pages:
  [P1] "Mel-Band RoFormer — architecture, inference hot path & RTX 3050 feasibility"
  [P3] "Vocal Separation Core (Mel-Band RoFormer) — ONNX / fp16 / WebGPU"
  [P4] "Mel-Band RoFormer (vocals), ONNX for the GPU (float16 weights)"
  [P5] "@audio/neural-separate 0.4.0 → 0.5.0" (its scripts/export-roformer.py and roformer.js)

Parity status: the band tables, the weight inventory and each step are pinned by
printed values, closed forms, invariants or the brute-force forward (see the
tests).  The RoPE base (10000) and the attention scale (1/sqrt(dh)) are not
printed on the pages: those two constants are "parity unpinned" against the real
model and pinned only by invariants.
"""
