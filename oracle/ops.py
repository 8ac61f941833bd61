"""Operators of the VLA forward pass, float64, written from their definitions.

Page "AI Infra如何优化VLA - 模型推理性能提升技术拆解", section 整体方案 lists the
operator types of the whole model: RMSNorm, LayerNorm, RoPE, GELU, SiLU,
MatMul (QKV / MLP), SDPA, Sin/Cos, Embedding and element-wise. Embedding is
not on this path (token embeddings are an input).
"""

from __future__ import annotations

import numpy as np
from scipy.special import erf


def rmsnorm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """Section 算子开发: the float chain mean over the row of x*x, reciprocal
    square root (of mean + eps), times x, times the gain."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x * (1.0 / np.sqrt(ms + eps)) * gain


def layernorm(x: np.ndarray, gain, bias, eps: float) -> np.ndarray:
    """LayerNorm over the last axis with the biased variance; gain/bias may be
    None (the DiT's norms carry no affine terms)."""
    x = np.asarray(x, dtype=np.float64)
    mu = np.mean(x, axis=-1, keepdims=True)
    var = np.mean((x - mu) ** 2, axis=-1, keepdims=True)
    y = (x - mu) / np.sqrt(var + eps)
    if gain is not None:
        y = y * gain
    if bias is not None:
        y = y + bias
    return y


def rope_angles(positions: np.ndarray, head_dim: int, base: float) -> np.ndarray:
    """angle[p, i] = position_p * base^(-2i/D) for i < D/2."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / head_dim)
    return np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]


def rope(x: np.ndarray, positions: np.ndarray, base: float) -> np.ndarray:
    """Section 算子开发, RoPE: the two halves of each head (element i pairs with
    element i + D/2) are rotated by the position's angle. x is [S, heads, D]."""
    S, nh, D = x.shape
    half = D // 2
    ang = rope_angles(positions, D, base)[:, None, :]          # [S, 1, D/2]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def softmax(z: np.ndarray, axis: int = -1) -> np.ndarray:
    z = z - np.max(z, axis=axis, keepdims=True)
    e = np.exp(z)
    return e / np.sum(e, axis=axis, keepdims=True)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool) -> np.ndarray:
    """Scaled dot-product attention with grouped KV heads.

    q [Sq, Hq, D], k [Sk, Hkv, D], v [Sk, Hkv, Dv]. Query head h reads KV head
    h // (Hq / Hkv) (consecutive groups, GQA 32/8 in section 整体方案). Scores
    are scaled by 1/sqrt(D). With ``causal`` (requires Sq == Sk) query i sees
    keys j <= i. Returns [Sq, Hq, Dv].
    """
    Sq, Hq, D = q.shape
    Sk, Hkv, Dv = v.shape
    assert Hq % Hkv == 0
    group = Hq // Hkv
    out = np.empty((Sq, Hq, Dv), dtype=np.float64)
    if causal:
        assert Sq == Sk
        allowed = np.tril(np.ones((Sq, Sk), dtype=bool))
    for h in range(Hq):
        g = h // group
        s = (q[:, h, :] @ k[:, g, :].T) / np.sqrt(D)
        if causal:
            s = np.where(allowed, s, -np.inf)
        out[:, h, :] = softmax(s, axis=-1) @ v[:, g, :]
    return out


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def gelu(z: np.ndarray) -> np.ndarray:
    """Exact GELU: z * Phi(z), Phi the standard normal CDF (erf form)."""
    return 0.5 * z * (1.0 + erf(z / np.sqrt(2.0)))


def linear(x: np.ndarray, w: np.ndarray, b=None) -> np.ndarray:
    """PyTorch Linear convention: w is [N_out, K_in], y = x w^T (+ b)."""
    y = np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T
    if b is not None:
        y = y + b
    return y
