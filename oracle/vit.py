"""Vision encoder and 2x2 token merger (oracle side).

Page "AI Infra如何优化VLA - 模型推理性能提升技术拆解": section 整体方案 (a 24-layer
ViT vision encoder), section CUDA Graph (the vision pass is PatchEmbed -> the
ViT blocks -> Merger), section 算子融合 (GELU MLPs in the vision blocks and the
merger, merger width 4096). Plain readings where the page is silent: 14-px
patches flattened in (channel, row, column) order in raster patch order, a
learned absolute position table, pre-norm LayerNorm blocks with biased
projections, non-causal multi-head attention, exact (erf) GELU, no final
norm (the merger's LayerNorm plays that role), and the merger concatenating
each 2x2 group of neighbouring patches in raster order.
"""

from __future__ import annotations

import numpy as np

from . import ops


def patchify(img: np.ndarray, patch: int) -> np.ndarray:
    """img [C, H, W] -> [(H/p)*(W/p), C*p*p]; patch (r, c) is row r*(W/p)+c."""
    C, H, Wd = img.shape
    gr, gc = H // patch, Wd // patch
    out = np.empty((gr * gc, C * patch * patch), dtype=np.float64)
    for r in range(gr):
        for c in range(gc):
            out[r * gc + c] = img[:, r * patch:(r + 1) * patch, c * patch:(c + 1) * patch].reshape(-1)
    return out


def vit_layer(z: np.ndarray, W, p: str, v) -> np.ndarray:
    """One pre-norm encoder block on the patch rows z [S, D]: z + MHA(LN1(z)),
    then + MLP(LN2(.)), with biased projections and no mask."""
    S = z.shape[0]
    u = ops.layernorm(z, W[p + "ln1_g"], W[p + "ln1_b"], v.eps)
    q = ops.linear(u, W[p + "wq"], W[p + "bq"]).reshape(S, v.heads, v.head_dim)
    k = ops.linear(u, W[p + "wk"], W[p + "bk"]).reshape(S, v.heads, v.head_dim)
    vv = ops.linear(u, W[p + "wv"], W[p + "bv"]).reshape(S, v.heads, v.head_dim)
    o = ops.attention(q, k, vv, causal=False).reshape(S, v.heads * v.head_dim)
    z = z + ops.linear(o, W[p + "wo"], W[p + "bo"])
    u = ops.layernorm(z, W[p + "ln2_g"], W[p + "ln2_b"], v.eps)
    return z + ops.linear(ops.gelu(ops.linear(u, W[p + "w1"], W[p + "b1"])), W[p + "w2"], W[p + "b2"])


def vit(img: np.ndarray, W, v) -> np.ndarray:
    z = ops.linear(patchify(np.asarray(img, dtype=np.float64), v.patch), W["vit.pe_w"], W["vit.pe_b"])
    z = z + W["vit.pos"]
    for l in range(v.layers):
        z = vit_layer(z, W, f"vit.{l}.", v)
    return z


def merge_groups(u: np.ndarray, grid: int, m: int) -> np.ndarray:
    """[grid*grid, D] -> [(grid/m)^2, m*m*D]: merged token (R, C) concatenates
    patches (m*R + dy, m*C + dx) for dy, dx in raster order."""
    D = u.shape[1]
    g = grid // m
    out = np.empty((g * g, m * m * D), dtype=np.float64)
    for R in range(g):
        for C in range(g):
            parts = [u[(m * R + dy) * grid + (m * C + dx)] for dy in range(m) for dx in range(m)]
            out[R * g + C] = np.concatenate(parts)
    return out


def merger(z: np.ndarray, W, v) -> np.ndarray:
    u = ops.layernorm(z, W["mrg.ln_g"], W["mrg.ln_b"], v.eps)
    g = merge_groups(u, v.grid, v.merge)
    return ops.linear(ops.gelu(ops.linear(g, W["mrg.w1"], W["mrg.b1"])), W["mrg.w2"], W["mrg.b2"])
