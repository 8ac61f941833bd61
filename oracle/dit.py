"""DiT action expert and the flow-matching Euler sampler (oracle side).

Page "AI Infra如何优化VLA - 模型推理性能提升技术拆解", section 整体方案: the action
head is a 36-layer DiT run for 4 denoising steps by a flow-matching Euler
integrator starting from random noise; Sin/Cos is one of the operator types
(the timestep embedding). Section CUDA Graph: the action pass is the denoise
steps times the DiT layers.

Plain readings where the page is silent:
  * flow time runs from t = 0 (noise) upward, t_k = k / K, and the Euler step
    uses the velocity at the left end: a_{k+1} = a_k + v(a_k, t_k) / K;
  * phi(t) = [cos(1000 t w_i), sin(1000 t w_i)], w_i = 10000^(-i/(d/2)),
    i < d/2 with d = 256, then Linear -> SiLU -> Linear gives c;
  * each layer has 9 modulation vectors m = W_ada SiLU(c) + b_ada ordered
    [shift, scale, gate] x [self-attn, cross-attn, MLP]; a sublayer reads
    u = LN(x)(1 + scale) + shift (LN without affine) and adds gate * f(u);
  * self-attention over the action tokens has no mask and no positional
    term; cross-attention reads all context tokens; MLP is Linear -> exact
    GELU -> Linear; every Linear has a bias;
  * the final layer is modulated by 2 vectors [shift, scale] and projects to
    the action dimension.
"""

from __future__ import annotations

from typing import Callable, List, Optional

import numpy as np

from . import ops


def timestep_embedding(t: float, d) -> np.ndarray:
    half = d.tdim // 2
    i = np.arange(half, dtype=np.float64)
    w = d.freq_base ** (-i / half)
    arg = d.time_scale * float(t) * w
    return np.concatenate([np.cos(arg), np.sin(arg)])


def time_condition(t: float, W, d) -> np.ndarray:
    phi = timestep_embedding(t, d)
    return ops.linear(ops.silu(ops.linear(phi, W["dit.t1_w"], W["dit.t1_b"])), W["dit.t2_w"], W["dit.t2_b"])


def modulated(x: np.ndarray, shift: np.ndarray, scale: np.ndarray, eps: float) -> np.ndarray:
    return ops.layernorm(x, None, None, eps) * (1.0 + scale) + shift


def dit_layer(x: np.ndarray, sc: np.ndarray, ctx: np.ndarray, W, p: str, d) -> np.ndarray:
    n, D = x.shape
    hd, nh = d.head_dim, d.heads
    m = ops.linear(sc, W[p + "ada_w"], W[p + "ada_b"]).reshape(d.n_mod, D)
    sh_sa, sc_sa, g_sa, sh_ca, sc_ca, g_ca, sh_ml, sc_ml, g_ml = m
    u = modulated(x, sh_sa, sc_sa, d.eps)
    q = ops.linear(u, W[p + "sa_wq"], W[p + "sa_bq"]).reshape(n, nh, hd)
    k = ops.linear(u, W[p + "sa_wk"], W[p + "sa_bk"]).reshape(n, nh, hd)
    v = ops.linear(u, W[p + "sa_wv"], W[p + "sa_bv"]).reshape(n, nh, hd)
    o = ops.attention(q, k, v, causal=False).reshape(n, D)
    x = x + g_sa * ops.linear(o, W[p + "sa_wo"], W[p + "sa_bo"])
    u = modulated(x, sh_ca, sc_ca, d.eps)
    q = ops.linear(u, W[p + "ca_wq"], W[p + "ca_bq"]).reshape(n, nh, hd)
    L = ctx.shape[0]
    kc = ops.linear(ctx, W[p + "ca_wk"], W[p + "ca_bk"]).reshape(L, nh, hd)
    vc = ops.linear(ctx, W[p + "ca_wv"], W[p + "ca_bv"]).reshape(L, nh, hd)
    o = ops.attention(q, kc, vc, causal=False).reshape(n, D)
    x = x + g_ca * ops.linear(o, W[p + "ca_wo"], W[p + "ca_bo"])
    u = modulated(x, sh_ml, sc_ml, d.eps)
    hmid = ops.gelu(ops.linear(u, W[p + "mlp_w1"], W[p + "mlp_b1"]))
    return x + g_ml * ops.linear(hmid, W[p + "mlp_w2"], W[p + "mlp_b2"])


def dit_velocity(a: np.ndarray, t: float, ctx: np.ndarray, W, d) -> np.ndarray:
    """v_theta(a, t, ctx): action chunk a [chunk, A] -> velocity [chunk, A]."""
    x = ops.linear(np.asarray(a, dtype=np.float64), W["dit.in_w"], W["dit.in_b"])
    sc = ops.silu(time_condition(t, W, d))
    ctx = np.asarray(ctx, dtype=np.float64)
    for l in range(d.layers):
        x = dit_layer(x, sc, ctx, W, f"dit.{l}.", d)
    f = ops.linear(sc, W["dit.f_w"], W["dit.f_b"]).reshape(2, d.hidden)
    return ops.linear(modulated(x, f[0], f[1], d.eps), W["dit.out_w"], W["dit.out_b"])


def euler_sample(x0: np.ndarray, K: int, velocity: Callable[[np.ndarray, float], np.ndarray],
                 record: Optional[List[np.ndarray]] = None) -> np.ndarray:
    """x_{k+1} = x_k + (1/K) v(x_k, t_k), t_k = k/K, k = 0..K-1; returns x_K."""
    x = np.asarray(x0, dtype=np.float64)
    for k in range(K):
        v = velocity(x, k / K)
        if record is not None:
            record.append(v)
        x = x + v / K
    return x


def flow_sample(noise: np.ndarray, ctx: np.ndarray, W, d, K: int,
                record: Optional[List[np.ndarray]] = None) -> np.ndarray:
    return euler_sample(noise, K, lambda a, t: dit_velocity(a, t, ctx, W, d), record)


def flow_sample_stale(noise: np.ndarray, ctx_prev: np.ndarray, ctx_cur: np.ndarray, W, d, K: int, n_stale: int,
                      record: Optional[List[np.ndarray]] = None) -> np.ndarray:
    """The sampler of one control cycle under V-AEFusion (page "跨XPU平台表征视觉-
    语言-动作模型：机器人部署中的约束与加速", section 5.3 and Figure 9): the
    action expert starts denoising while the VLM still works on the current
    observation, so its first n_stale Euler steps (the stale steps) are
    conditioned on the previous cycle's context and the remaining K - n_stale
    steps on the current one. The time grid and the update are the plain
    sampler's; only the conditioning of each step changes."""
    if not 0 <= n_stale <= K:
        raise ValueError(f"n_stale {n_stale} outside [0, {K}]")
    conds = iter([ctx_prev] * n_stale + [ctx_cur] * (K - n_stale))
    return euler_sample(noise, K, lambda a, t: dit_velocity(a, t, next(conds), W, d), record)

