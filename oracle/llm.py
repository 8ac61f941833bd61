"""Pre-norm transformer block and the VLM backbone prefill (oracle side).

Page "AI Infra如何优化VLA - 模型推理性能提升技术拆解":
  * section 整体方案: the LLM is a 36-layer decoder with GQA (32 query / 8 KV
    heads) and a SwiGLU MLP with intermediate size 9728, run as a pure
    prefill (no autoregressive decode);
  * section 算子开发: RMSNorm is the pre-norm of each sublayer (72 pre-norm
    calls over 36 layers); RoPE rotates halves of Q and K in every layer;
  * section 算子融合: fused QKV (one projection producing Q, K and V) and the
    SwiGLU MLP;
  * section CUDA Graph: the LLM pass runs its layers and ends in a final
    RMSNorm.
Block (no biases, consistent with the decoder family the page names):
  h   = x + Attn(RoPE(Q), RoPE(K), V) W_o^T,   [Q|K|V] = RMSNorm(x, g1) W_qkv^T
  out = h + (SiLU(n W_g^T) * (n W_u^T)) W_d^T,  n = RMSNorm(h, g2)
With QK-norm (section 算子开发 counts RMSNorm calls on Q and K besides the
two pre-norms), every query and key head vector is RMS-normalised over the
head dimension with its own gain (q_norm, k_norm) before RoPE:
  Q_h <- RMSNorm(Q_h, q_norm),  K_g <- RMSNorm(K_g, k_norm).
With W8A8 (page "开源 APXInf 把 VLA 推理压到 26 毫秒": FP8 weights and
activations, INT8 where FP8 units are missing), the input rows of the four
Linears (n, the attention output, n2 and the SwiGLU product) are replaced by
their per-token FP8 (oracle/fp8.py) or INT8 (oracle/int8.py) values first.
"""

from __future__ import annotations

import numpy as np

from . import ops
from .fp8 import fake_quant_act_rows
from .int8 import fake_quant_act_rows as fake_quant_act_rows_int8


def block(x: np.ndarray, W, prefix: str, shape, pos0: int = 0) -> np.ndarray:
    """One pre-norm block on x [S, H]; ``pos0`` is the position of row 0."""
    x = np.asarray(x, dtype=np.float64)
    S, H = x.shape
    Hq, Hkv, D = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    # W8A8: every Linear of the block reads its input rows as per-token E4M3FN
    # codes times the row's scale (oracle/fp8.py)
    a8 = getattr(shape, "a8", "")
    act = {"fp8": fake_quant_act_rows, "int8": fake_quant_act_rows_int8}.get(a8, lambda t: t)
    n = act(ops.rmsnorm(x, W[prefix + "attn_norm"], shape.eps))
    q = ops.linear(n, W[prefix + "wq"]).reshape(S, Hq, D)
    k = ops.linear(n, W[prefix + "wk"]).reshape(S, Hkv, D)
    v = ops.linear(n, W[prefix + "wv"]).reshape(S, Hkv, D)
    if getattr(shape, "qk_norm", False):
        q = ops.rmsnorm(q, W[prefix + "q_norm"], shape.eps)
        k = ops.rmsnorm(k, W[prefix + "k_norm"], shape.eps)
    pos = np.arange(S) + pos0
    q = ops.rope(q, pos, shape.rope_base)
    k = ops.rope(k, pos, shape.rope_base)
    o = act(ops.attention(q, k, v, causal=True).reshape(S, Hq * D))
    h = x + ops.linear(o, W[prefix + "wo"])
    n2 = act(ops.rmsnorm(h, W[prefix + "mlp_norm"], shape.eps))
    a = act(ops.silu(ops.linear(n2, W[prefix + "wg"])) * ops.linear(n2, W[prefix + "wu"]))
    return h + ops.linear(a, W[prefix + "wd"])


def backbone(E: np.ndarray, W, cfg, layers=None) -> np.ndarray:
    """The layer stack over embeddings E [S, H], then the final RMSNorm when
    the config has one. Positions are 0..S-1 for every row (1-D RoPE)."""
    x = np.asarray(E, dtype=np.float64)
    n_layers = cfg.layers if layers is None else layers
    for l in range(n_layers):
        x = block(x, W, f"llm.{l}.", cfg.block)
    if cfg.final_norm:
        x = ops.rmsnorm(x, W["llm.final_norm"], cfg.block.eps)
    return x
