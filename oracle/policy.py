"""The full policy step and its runners over seeded configs (oracle side).

Page "AI Infra如何优化VLA - 模型推理性能提升技术拆解", section 整体方案: vision
encoder -> LLM decoder (including projection layers) -> action head, run in
series. Plain readings: the token sequence is [visual tokens of each image in
order; text embeddings]; the backbone's final-normed output of every token is
projected by one biased Linear (backbone hidden -> DiT context width) and the
DiT cross-attends to all of it.
"""

from __future__ import annotations

from typing import Dict, List

import numpy as np

from . import dit, llm, vit
from .io import Weights, to_f64
from .ops import linear


def projector(h: np.ndarray, W) -> np.ndarray:
    return linear(h, W["proj.w"], W["proj.b"])


def vlm(image, text: np.ndarray, W, cfg) -> Dict[str, np.ndarray]:
    """Vision encoder, backbone and projector: the context the action head
    attends to ("ctx"), with the intermediate outputs that are graded."""
    out: Dict[str, np.ndarray] = {}
    rows: List[np.ndarray] = []
    if cfg.vit is not None:
        vis, mer = [], []
        for i in range(cfg.n_images):
            z = vit.vit(image[i], W, cfg.vit)
            vis.append(z)
            mer.append(vit.merger(z, W, cfg.vit))
        out["vit"] = np.stack(vis)
        out["merged"] = np.concatenate(mer)
        rows.append(out["merged"])
    rows.append(np.asarray(text, dtype=np.float64))
    E = np.concatenate(rows)
    out["hidden"] = llm.backbone(E, W, cfg)
    out["ctx"] = projector(out["hidden"], W)
    return out


def vla_step(image, text: np.ndarray, noise: np.ndarray, W, cfg) -> Dict[str, np.ndarray]:
    out = vlm(image, text, W, cfg)
    rec: List[np.ndarray] = []
    out["actions"] = dit.flow_sample(noise, out["ctx"], W, cfg.dit, cfg.steps, rec)
    out["velocities"] = np.stack(rec)
    return out


def vla_cycle_fused(image, text: np.ndarray, noise: np.ndarray, ctx_prev, W, cfg, n_stale: int) -> Dict[str, np.ndarray]:
    """One control cycle under V-AEFusion (page "跨XPU平台表征视觉-语言-动作模型：
    机器人部署中的约束与加速", section 5.3): the VLM of this cycle yields ctx
    as in vla_step; the action expert's first n_stale steps use ctx_prev, the
    context of the previous cycle, and the rest use ctx. With no previous
    cycle (ctx_prev None) every step uses ctx. Returns vla_step's outputs;
    "ctx" is what the next cycle receives as ctx_prev."""
    out = vlm(image, text, W, cfg)
    if ctx_prev is None:
        ctx_prev, n_stale = out["ctx"], 0
    rec: List[np.ndarray] = []
    out["actions"] = dit.flow_sample_stale(noise, ctx_prev, out["ctx"], W, cfg.dit, cfg.steps, n_stale, rec)
    out["velocities"] = np.stack(rec)
    return out


def run_config(cfg, weights, inputs) -> Dict[str, np.ndarray]:
    """Evaluate a config on its seeded tensors; returns the graded outputs."""
    W = weights if isinstance(weights, Weights) else Weights(weights)
    if cfg.kind == "block":
        return {"out": llm.block(to_f64(inputs["x"]), W, "llm.0.", cfg.block)}
    if cfg.kind == "backbone":
        return {"hidden": llm.backbone(to_f64(inputs["x"]), W, cfg)}
    if cfg.kind == "dit":
        rec: List[np.ndarray] = []
        a = dit.flow_sample(to_f64(inputs["noise"]), to_f64(inputs["ctx"]), W, cfg.dit, cfg.steps, rec)
        return {"actions": a, "velocities": np.stack(rec)}
    if cfg.kind == "step":
        img = to_f64(inputs["image"]) if cfg.vit is not None else None
        return vla_step(img, to_f64(inputs["text"]), to_f64(inputs["noise"]), W, cfg)
    raise ValueError(cfg.kind)
