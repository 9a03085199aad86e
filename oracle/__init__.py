"""Plain fp64 CPU oracle of the Streaming Sortformer / Nemotron-3-style
frame-classification forward and its speaker-cache update.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute this package: only the tests, the smoke check and the CPU-baseline
leg of the benchmark use it. It shares no code, table or constant generator
with the HIP library; the only common dependency is the seeded input
generator in ``synthetic`` (which holds none of the method's arithmetic).

Sources (cited by page title and section in every function):
* "Streaming Sortformer Diarizer" model card (ExecuTorch example), sections
  Pipeline, Streaming Architecture, Streaming Configurations, Model
  Parameters, Exported Methods, torch.export Fixes.
* Hugging Face Transformers docs, "Nemotron 3 Diarization": Overview,
  streaming usage, and the fixed-window section.
* NeMo Speaker Diarization API docs, SortformerEncLabelModel:
  forward_for_export, forward_streaming_step, SortformerStreamingState.
* ExecuTorch issue "Enable Nemotron-3-Diarization on MLX, CUDA, XNNPACK, and
  Vulkan": model-card summary and Progress.

Everything is computed in float64. bf16 configurations use bf16-rounded GEMM
weight matrices (upcast to float64) so that parity isolates the GPU's
arithmetic error. Readings of points the pages leave open are listed in the
repository's design notes and restated where they are used.

Parity status: every function here is pinned by a ``-m "not gpu"`` test to
something other than itself (closed forms, textbook routines, brute force,
page-given shapes and invariants), except the absolute probability values of
the full model, which no page prints (random weights): the GPU-vs-oracle
comparison is their only check.
"""
