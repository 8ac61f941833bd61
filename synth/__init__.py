"""Seeded synthetic inputs for the batch-1 VLA forward pass.

This package is the only code shared by the CPU oracle (``oracle/``) and the
HIP path (``vla_robot_policy_amd/``). It holds shapes and seeded random
tensors and nothing of the method's arithmetic: no norm, no projection, no
attention, no sampler step. Weight values are drawn once, rounded to their
storage dtype, and the stored values *are* the tensors both sides consume.

Storage dtypes:
  * ``f32``  -> numpy float32
  * ``bf16`` -> numpy uint16 holding bfloat16 bit patterns (round to nearest
    even from a float32 draw)
  * ``fp8``  -> numpy uint8 holding OCP E4M3FN codes plus a float32 scale per
    output channel (row of the ``[N_out, K_in]`` weight); see ``synth.fp8``.
  * ``int8`` -> numpy int8 codes in [-127, 127] plus a float32 scale per
    output channel; see ``synth.int8``.
"""

from .configs import (  # noqa: F401
    BlockShape, ViTShape, DiTShape, Config, CONFIGS, get_config, small_config,
)
from .gen import (  # noqa: F401
    Tensor, TensorSet, make_weights, make_inputs, bf16_bits_to_f32, f32_to_bf16_bits,
)
