"""Roofline latency bound of a policy step (host-side model, no GPU needed).

Page "VLA-Perf: VLA 推理性能全景分析", section 2.3 (latency model): the latency
of a component is the sum over its operators, and one operator takes
max(FLOPs / peak FLOP/s, Bytes / memory bandwidth). Summing that over the
fused operator list of one step gives the bound a measured step is graded
against (bound / measured = fraction of roofline).

Bytes are algorithmic minimums: each weight is read once per use, and
activations are read and written once in bf16. Work that depends only on the
fixed timestep schedule or on the context (adaLN modulations for all K
steps, the cross-attention K/V of every layer) is counted once per step of
the policy, as the implementation hoists it out of the Euler loop.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List

# MI355X published peaks (dense; no structured sparsity).
MI355X = {
    "bf16": 2.5e15,
    "fp8": 5.0e15,
    "f32": 157.3e12,     # fp32 matrix / vector
    "f64": 78.6e12,
    "hbm": 8.0e12,       # bytes / s
}

ACT = 2  # bytes per activation element (bf16)


def ridge(peak_flops: float, bandwidth: float) -> float:
    """Arithmetic intensity (FLOP/byte) where the two roofs meet."""
    return peak_flops / bandwidth


@dataclass
class Op:
    name: str
    phase: str
    flops: float
    bytes: float
    count: int = 1
    compute: str = "bf16"   # which peak prices the FLOPs

    def time(self, peaks: Dict[str, float]) -> float:
        return self.count * max(self.flops / peaks[self.compute], self.bytes / peaks["hbm"])


def op_time(flops: float, nbytes: float, peak: float, bw: float) -> float:
    return max(flops / peak, nbytes / bw)


def _wbytes(wdtype: str, n: int, k: int) -> float:
    if wdtype == "f32":
        return 4.0 * n * k
    if wdtype == "bf16":
        return 2.0 * n * k
    if wdtype in ("fp8", "int8"):
        return 1.0 * n * k + 4.0 * n      # codes + one float32 scale per output channel
    raise ValueError(wdtype)


def _compute(wdtype: str) -> str:
    # 8-bit weights run on the bf16 matrix cores (their codes widen to bf16 exactly)
    return "f32" if wdtype == "f32" else "bf16"


def linear_op(name, phase, M, N, K, wdtype, count=1, bias=False, act_in=None, act_out=None, extra_bytes=0.0):
    a_in = ACT * M * K if act_in is None else act_in
    a_out = ACT * M * N if act_out is None else act_out
    b = _wbytes(wdtype, N, K) + a_in + a_out + (4.0 * N if bias else 0.0) + extra_bytes
    return Op(name, phase, 2.0 * M * N * K, b, count, _compute(wdtype))


def attn_op(name, phase, Sq, Sk, Hq, Hkv, D, causal, count=1, wdtype="bf16"):
    pairs = Sq * (Sq + 1) / 2.0 if causal else float(Sq * Sk)
    flops = 4.0 * Hq * D * pairs
    b = ACT * (Sq * Hq * D * 2 + Sk * Hkv * D * 2)
    return Op(name, phase, flops, b, count, _compute(wdtype))


def backbone_ops(cfg, S=None) -> List[Op]:
    b = cfg.block
    S = cfg.seq if S is None else S
    H, I, L, w = b.hidden, b.intermediate, cfg.layers, cfg.wdtype
    res = ACT * S * H
    ops = [
        linear_op("llm.qkv", "backbone", S, b.qkv_dim, H, w, L),
        attn_op("llm.attn", "backbone", S, S, b.n_q_heads, b.n_kv_heads, b.head_dim, True, L, w),
        linear_op("llm.o", "backbone", S, H, b.q_dim, w, L, extra_bytes=res),
        linear_op("llm.gate_up", "backbone", S, 2 * I, H, w, L, act_out=ACT * S * I),
        linear_op("llm.down", "backbone", S, H, I, w, L, extra_bytes=res),
    ]
    if cfg.final_norm:
        ops.append(Op("llm.final_norm", "backbone", 4.0 * S * H, 2.0 * res + 4.0 * H, 1, "f32"))
    return ops


def vit_ops(cfg) -> List[Op]:
    v = cfg.vit
    n = cfg.n_images
    S, D = v.n_patches, v.hidden
    w = "bf16" if cfg.wdtype in ("fp8", "int8") else cfg.wdtype
    ops = [linear_op("vit.patch_embed", "vit", S, D, v.patch_dim, w, n, bias=True,
                     extra_bytes=4.0 * S * D)]
    L = v.layers * n
    ops += [
        linear_op("vit.qkv", "vit", S, 3 * D, D, w, L, bias=True),
        attn_op("vit.attn", "vit", S, S, v.heads, v.heads, v.head_dim, False, L, w),
        linear_op("vit.o", "vit", S, D, D, w, L, bias=True, extra_bytes=ACT * S * D),
        linear_op("vit.up", "vit", S, v.mlp, D, w, L, bias=True),
        linear_op("vit.down", "vit", S, D, v.mlp, w, L, bias=True, extra_bytes=ACT * S * D),
        linear_op("mrg.fc1", "vit", v.n_merged, v.merged_dim, v.merged_dim, w, n, bias=True),
        linear_op("mrg.fc2", "vit", v.n_merged, v.out_dim, v.merged_dim, w, n, bias=True),
    ]
    return ops


def dit_ops(cfg) -> List[Op]:
    d = cfg.dit
    K, n, D, w, L = cfg.steps, d.chunk, d.hidden, cfg.wdtype, d.layers
    C = cfg.ctx_len
    ops = [
        # once per policy step (exact hoists: fixed t schedule, fixed context)
        linear_op("dit.time_fc1", "dit_once", K, D, d.tdim, w, 1, bias=True),
        linear_op("dit.time_fc2", "dit_once", K, D, D, w, 1, bias=True),
        linear_op("dit.adaln", "dit_once", K, L * d.n_mod * D, D, w, 1, bias=True),
        linear_op("dit.final_mod", "dit_once", K, 2 * D, D, w, 1, bias=True),
        linear_op("dit.cross_kv", "dit_once", C, L * 2 * D, d.ctx_dim, w, 1, bias=True),
        # per Euler step
        linear_op("dit.in_proj", "dit_step", n, D, d.action_dim, w, K, bias=True, act_in=4.0 * n * d.action_dim),
    ]
    LK = L * K
    res = ACT * n * D
    ops += [
        linear_op("dit.sa_qkv", "dit_step", n, 3 * D, D, w, LK, bias=True),
        attn_op("dit.sa_attn", "dit_step", n, n, d.heads, d.heads, d.head_dim, False, LK, w),
        linear_op("dit.sa_o", "dit_step", n, D, D, w, LK, bias=True, extra_bytes=res),
        linear_op("dit.ca_q", "dit_step", n, D, D, w, LK, bias=True),
        attn_op("dit.ca_attn", "dit_step", n, C, d.heads, d.heads, d.head_dim, False, LK, w),
        linear_op("dit.ca_o", "dit_step", n, D, D, w, LK, bias=True, extra_bytes=res),
        linear_op("dit.mlp_up", "dit_step", n, d.mlp, D, w, LK, bias=True),
        linear_op("dit.mlp_down", "dit_step", n, D, d.mlp, w, LK, bias=True, extra_bytes=res),
        linear_op("dit.out_proj", "dit_step", n, d.action_dim, D, w, K, bias=True, act_out=4.0 * n * d.action_dim),
    ]
    return ops


def fused_ops(cfg) -> Dict[str, Op]:
    """Operators of kernels that fuse several of the ops above, per launch.

    ``dit.layers`` is every DiT layer of one Euler step in a single launch:
    its algorithmic bytes are what must cross HBM once per launch (each
    layer's weights and biases, its context K/V, the residual stream in and
    out and its modulation vectors); intermediate activations stay on chip.
    Its FLOPs are those of the layers' GEMMs and attention.
    """
    out: Dict[str, Op] = {}
    if cfg.kind in ("dit", "step") and cfg.dit is not None:
        d = cfg.dit
        n, D, C, w = d.chunk, d.hidden, cfg.ctx_len, cfg.wdtype
        parts = {"dit.sa_qkv", "dit.sa_attn", "dit.sa_o", "dit.ca_q", "dit.ca_attn", "dit.ca_o", "dit.mlp_up", "dit.mlp_down"}
        flops = sum(o.flops for o in dit_ops(cfg) if o.name in parts)
        weights = (_wbytes(w, 3 * D, D) + 3 * _wbytes(w, D, D) + _wbytes(w, d.mlp, D) + _wbytes(w, D, d.mlp)
                   + 4.0 * (3 * D + 3 * D + d.mlp + D))
        nbytes = weights + ACT * C * 2 * D + 4.0 * n * D * 2 + 4.0 * 9 * D
        out["dit.layers"] = Op("dit.layers", "dit_step", d.layers * flops, d.layers * nbytes, cfg.steps, _compute(w))
    return out


def step_ops(cfg) -> List[Op]:
    if cfg.kind == "block":
        c = cfg.replace(final_norm=False, layers=1)
        return backbone_ops(c)
    if cfg.kind == "backbone":
        return backbone_ops(cfg)
    if cfg.kind == "dit":
        return dit_ops(cfg)
    if cfg.kind == "step":
        ops = vit_ops(cfg) if cfg.vit is not None else []
        ops += backbone_ops(cfg)
        ops.append(linear_op("proj", "projector", cfg.seq, cfg.dit.ctx_dim, cfg.block.hidden, cfg.wdtype, 1, bias=True))
        ops += dit_ops(cfg)
        return ops
    raise ValueError(cfg.kind)


@dataclass
class Bound:
    seconds: float
    flops: float
    bytes: float
    per_phase: Dict[str, float] = field(default_factory=dict)
    ops: List[Op] = field(default_factory=list)


def bound(cfg, peaks: Dict[str, float] = MI355X) -> Bound:
    ops = step_ops(cfg)
    per: Dict[str, float] = {}
    for o in ops:
        per[o.phase] = per.get(o.phase, 0.0) + o.time(peaks)
    return Bound(sum(per.values()), sum(o.flops * o.count for o in ops),
                 sum(o.bytes * o.count for o in ops), per, ops)
