"""CPU oracle of the batch-1 VLA forward pass — TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 NumPy implementation of what the policy computes,
written from the pages' descriptions and used only to check the HIP path.
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it. The product path (``vla_robot_policy_amd``) never
imports, calls or links anything here, and this package imports nothing from
it: the two share only the seeded input generators of ``synth``.

Sources (pages, by title and section):
  * "AI Infra如何优化VLA - 模型推理性能提升技术拆解" (RimBot report on StarVLA):
    section 整体方案 (model structure: ViT 24 L -> LLM 36 L with GQA 32/8 and
    SwiGLU 9728, prefill only -> 4-step flow-matching Euler DiT action head;
    the ten operator types), section 算子开发 (RMSNorm as the float chain
    mean(x^2) -> rsqrt -> *x -> *w; half-split RoPE on Q/K), section 算子融合
    (GELU MLP, SwiGLU MLP, fused QKV), section CUDA Graph (Vision graph
    PatchEmbed -> ViT blocks -> Merger; LLM graph 36 layers -> final RMSNorm;
    Action graph K denoise steps x 36 DiT layers).
  * "VLA-Perf: VLA 推理性能全景分析" section 2.3 (latency model), used by the
    roofline module of the product, not here.
  * "开源 APXInf 把 VLA 推理压到 26 毫秒" (FP8 weights on Jetson Thor).

Modules:
  ops     norms, RoPE, attention, activations, linear layers
  llm     pre-norm transformer block and the backbone prefill
  vit     patchify, ViT encoder, 2x2 merger
  dit     timestep embedding, DiT velocity field, Euler sampler
  policy  projector and the full policy step
  fp8     E4M3FN decoding and per-channel dequantisation
  io      float64 views of the stored seeded tensors

Every function is pinned by ``tests/test_oracle_*.py`` against closed forms,
invariants, library routines or brute force; parity of the whole-model
composition with a trained StarVLA / pi0.5 is unpinned (no trained weights
or printed reference outputs exist on the pages).
"""
