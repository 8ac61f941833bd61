"""Shapes of the five named workloads and of the reduced test shapes.

The named workloads are the ones the policy is measured on (get_config ids):

  1  one pre-norm transformer block, fp32, seq 64 (hidden 256, 4 q / 2 kv
     heads of 64, SwiGLU 688, RoPE base 1e4, RMSNorm eps 1e-6)
  2  36-layer VLM backbone prefill, bf16 weights, seq 256 (hidden 2560,
     GQA 32/8 x 128, SwiGLU 9728, RoPE base 1e6, final RMSNorm)
  3  DiT action expert in a 4-step flow-matching Euler loop, bf16
     (36 layers, hidden 1280, 16 heads, GELU MLP 5120, adaLN from a
     sinusoidal timestep embedding, 16x7 action chunk, 256 ctx tokens)
  4  full single-camera step: ViT (24 layers, hidden 1024, 16 heads,
     224x224 image in 14-px patches) -> 2x2 merger -> 64 visual + 40 text
     tokens through the 36-layer backbone at seq 104 -> projector -> the DiT
  5  two-camera long-context step: 560-token backbone (embeddings given) +
     DiT with a 50x32 chunk and 10 Euler steps, every Linear weight in fp8
     e4m3 with a float32 scale per output channel, activations bf16

Where the pages leave a shape open the plain reading is taken: the Q width
is heads*head_dim (4096 for the backbone, not the hidden size); the DiT
context width equals the DiT hidden size; the long-context sequence has no
vision encoder in front of it (its 560 embeddings are given).
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional


@dataclass(frozen=True)
class BlockShape:
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    rope_base: float
    eps: float = 1e-6
    qk_norm: bool = False   # per-head RMSNorm of Q and K before RoPE
    a8: str = ""            # W8A8: per-token activations into the block's Linears, "fp8" or "int8" ("": off)

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def qkv_dim(self) -> int:
        return self.q_dim + 2 * self.kv_dim


@dataclass(frozen=True)
class ViTShape:
    image: int = 224
    patch: int = 14
    channels: int = 3
    hidden: int = 1024
    heads: int = 16
    head_dim: int = 64
    mlp: int = 4096
    layers: int = 24
    merge: int = 2
    out_dim: int = 2560
    eps: float = 1e-6

    @property
    def grid(self) -> int:
        return self.image // self.patch

    @property
    def n_patches(self) -> int:
        return self.grid * self.grid

    @property
    def patch_dim(self) -> int:
        return self.channels * self.patch * self.patch

    @property
    def n_merged(self) -> int:
        return self.n_patches // (self.merge * self.merge)

    @property
    def merged_dim(self) -> int:
        return self.hidden * self.merge * self.merge


@dataclass(frozen=True)
class DiTShape:
    hidden: int = 1280
    heads: int = 16
    head_dim: int = 80
    mlp: int = 5120
    layers: int = 36
    tdim: int = 256
    ctx_dim: int = 1280
    chunk: int = 16
    action_dim: int = 7
    eps: float = 1e-6
    n_mod: int = 9          # shift/scale/gate for each of self-attn, cross-attn, MLP
    time_scale: float = 1000.0
    freq_base: float = 10000.0


@dataclass(frozen=True)
class Config:
    cid: int                 # seed root; 1..5 for the named workloads
    name: str
    kind: str                # 'block' | 'backbone' | 'dit' | 'step'
    wdtype: str              # 'f32' | 'bf16' | 'fp8' | 'int8'
    block: Optional[BlockShape] = None
    layers: int = 0          # backbone layers
    seq: int = 0             # backbone sequence length
    vit: Optional[ViTShape] = None
    n_images: int = 0
    n_text: int = 0          # embeddings given as input (rows after the visual tokens)
    dit: Optional[DiTShape] = None
    ctx_len: int = 0         # DiT context tokens
    steps: int = 0           # Euler steps K
    final_norm: bool = True  # backbone ends in an RMSNorm
    stress: bool = False     # wide norm gains / O(1) modulation for parity tests

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


LLM = BlockShape(hidden=2560, n_q_heads=32, n_kv_heads=8, head_dim=128,
                 intermediate=9728, rope_base=1e6, eps=1e-6)
SMALL_BLOCK = BlockShape(hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                         intermediate=688, rope_base=1e4, eps=1e-6)

CONFIGS = {
    1: Config(cid=1, name="block_fp32_s64", kind="block", wdtype="f32",
              block=SMALL_BLOCK, layers=1, seq=64, final_norm=False),
    2: Config(cid=2, name="backbone_bf16_s256", kind="backbone", wdtype="bf16",
              block=LLM, layers=36, seq=256),
    3: Config(cid=3, name="dit_bf16_k4", kind="dit", wdtype="bf16",
              dit=DiTShape(), ctx_len=256, steps=4),
    4: Config(cid=4, name="vla_step_bf16_1cam", kind="step", wdtype="bf16",
              block=LLM, layers=36, seq=104, vit=ViTShape(), n_images=1, n_text=40,
              dit=DiTShape(), ctx_len=104, steps=4),
    5: Config(cid=5, name="vla_step_fp8_s560", kind="step", wdtype="fp8",
              block=LLM, layers=36, seq=560, n_text=560,
              dit=DiTShape(chunk=50, action_dim=32), ctx_len=560, steps=10),
}


def get_config(cid: int) -> Config:
    return CONFIGS[cid]


def small_config(kind: str, wdtype: str = "bf16", seed: int = 1000, **kw) -> Config:
    """Reduced shapes that still span several kernel tiles and a ragged tail."""
    blk = kw.pop("block", SMALL_BLOCK)
    if kind == "block":
        base = Config(cid=seed, name=f"small_block_{wdtype}", kind="block", wdtype=wdtype,
                      block=blk, layers=1, seq=37, final_norm=False, stress=True)
    elif kind == "backbone":
        base = Config(cid=seed, name=f"small_backbone_{wdtype}", kind="backbone", wdtype=wdtype,
                      block=blk, layers=2, seq=45, stress=True)
    elif kind == "dit":
        base = Config(cid=seed, name=f"small_dit_{wdtype}", kind="dit", wdtype=wdtype,
                      dit=DiTShape(hidden=160, heads=2, head_dim=80, mlp=640, layers=2,
                                   ctx_dim=160, chunk=5, action_dim=7),
                      ctx_len=19, steps=3, stress=True)
    elif kind == "step":
        vit = ViTShape(image=56, patch=14, hidden=128, heads=2, head_dim=64, mlp=512,
                       layers=2, out_dim=blk.hidden)
        base = Config(cid=seed, name=f"small_step_{wdtype}", kind="step", wdtype=wdtype,
                      block=blk, layers=2, seq=vit.n_merged + 9, vit=vit, n_images=1, n_text=9,
                      dit=DiTShape(hidden=160, heads=2, head_dim=80, mlp=640, layers=2,
                                   ctx_dim=160, chunk=5, action_dim=7),
                      ctx_len=vit.n_merged + 9, steps=3, stress=True)
    else:
        raise ValueError(kind)
    return base.replace(**kw) if kw else base
