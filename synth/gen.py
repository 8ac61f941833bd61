"""Seeded tensor generation for weights and inputs.

Every tensor is drawn independently with
``Generator(PCG64(SeedSequence([cfg.cid, kind, crc32(name)])))`` where kind is
0 for weights, 1 for inputs and 2 for the sampler's noise, so any tensor can be
regenerated on its own and generation can run in parallel threads.

Distributions (the configs fix "weights N(0, 0.02), inputs N(0, 1)"; the rest
is the plain reading): Linear weights N(0, 0.02); biases and additive tables
N(0, 0.02); norm gains 1 + N(0, 0.02). In ``stress`` configs (reduced parity
shapes) Linear weights are N(0, 1/fan_in) so every layer output stays O(1),
gains are U(0.5, 1.5) and the adaLN biases are N(0, 0.5), so a dropped or
misplaced term moves the result far outside any tolerance.

Matrices (Linear weights) are stored in the config's dtype; vectors and
additive tables (gains, biases, positional tables) are float32; inputs are
bf16 bits except in f32 configs; the noise is float32.
"""

from __future__ import annotations

import zlib
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Dict, Iterable, List, Optional, Tuple

import numpy as np

from .configs import Config
from . import fp8 as _fp8
from . import int8 as _int8

KIND_WEIGHTS, KIND_INPUTS, KIND_NOISE = 0, 1, 2


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest even) and return the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Spec:
    name: str
    shape: Tuple[int, ...]
    init: str        # 'w' | 'bias' | 'gain' | 'ada_bias' | 'normal'
    store: str       # 'f32' | 'bf16' | 'fp8' | 'int8'
    kind: int = KIND_WEIGHTS
    fan_in: int = 1


@dataclass
class Tensor:
    """A stored tensor. ``data`` is float32, uint16 bf16 bits or uint8 E4M3FN
    codes; ``scale`` is the float32 per-row scale of an fp8 matrix."""
    name: str
    dtype: str
    data: np.ndarray
    scale: Optional[np.ndarray] = None

    @property
    def shape(self):
        return self.data.shape

    @property
    def nbytes(self) -> int:
        return self.data.nbytes + (0 if self.scale is None else self.scale.nbytes)


def _draw(cfg: Config, spec: Spec) -> Tensor:
    ss = np.random.SeedSequence([cfg.cid, spec.kind, zlib.crc32(spec.name.encode())])
    g = np.random.Generator(np.random.PCG64(ss))
    n = int(np.prod(spec.shape))
    if spec.init == "gain" and cfg.stress:
        v = g.uniform(0.5, 1.5, size=n).astype(np.float32)
    else:
        v = g.standard_normal(n, dtype=np.float32)
        if spec.init == "w":
            std = (1.0 / np.sqrt(spec.fan_in)) if cfg.stress else 0.02
            v *= np.float32(std)
        elif spec.init == "bias":
            v *= np.float32(0.02)
        elif spec.init == "ada_bias":
            v *= np.float32(0.5 if cfg.stress else 0.02)
        elif spec.init == "gain":
            v = np.float32(1.0) + v * np.float32(0.02)
        elif spec.init == "normal":
            pass
        else:
            raise ValueError(spec.init)
    v = v.reshape(spec.shape)
    if spec.store == "f32":
        return Tensor(spec.name, "f32", v)
    if spec.store == "bf16":
        return Tensor(spec.name, "bf16", f32_to_bf16_bits(v))
    if spec.store == "fp8":
        codes, scale = _fp8.quantize_rows(v)
        return Tensor(spec.name, "fp8", codes, scale)
    if spec.store == "int8":
        codes, scale = _int8.quantize_rows(v)
        return Tensor(spec.name, "int8", codes, scale)
    raise ValueError(spec.store)


class TensorSet:
    """Lazily generated, optionally cached, named tensors of one config."""

    def __init__(self, cfg: Config, specs: List[Spec], cache: bool = True):
        self.cfg = cfg
        self.specs: Dict[str, Spec] = {s.name: s for s in specs}
        self.order = [s.name for s in specs]
        self.cache = cache
        self._store: Dict[str, Tensor] = {}

    def __contains__(self, name: str) -> bool:
        return name in self.specs

    def __getitem__(self, name: str) -> Tensor:
        t = self._store.get(name)
        if t is None:
            t = _draw(self.cfg, self.specs[name])
            if self.cache:
                self._store[name] = t
        return t

    def names(self) -> List[str]:
        return list(self.order)

    def generate_all(self, threads: int = 8, names: Optional[Iterable[str]] = None) -> "TensorSet":
        todo = [n for n in (names or self.order) if n not in self._store]
        if not self.cache:
            return self
        with ThreadPoolExecutor(max_workers=threads) as ex:
            for n, t in zip(todo, ex.map(lambda nm: _draw(self.cfg, self.specs[nm]), todo)):
                self._store[n] = t
        return self

    def drop(self, names: Iterable[str]) -> None:
        for n in names:
            self._store.pop(n, None)

    def stored_bytes(self) -> int:
        total = 0
        for s in self.specs.values():
            n = int(np.prod(s.shape))
            total += n * {"f32": 4, "bf16": 2, "fp8": 1, "int8": 1}[s.store] + (4 * s.shape[0] if s.store in ("fp8", "int8") else 0)
        return total


def _mat(cfg: Config) -> str:
    return cfg.wdtype


def _act(cfg: Config) -> str:
    return "f32" if cfg.wdtype == "f32" else "bf16"


def backbone_specs(cfg: Config) -> List[Spec]:
    b = cfg.block
    m = _mat(cfg)
    H = b.hidden
    out: List[Spec] = []
    for l in range(cfg.layers):
        p = f"llm.{l}."
        out += [
            Spec(p + "attn_norm", (H,), "gain", "f32"),
            Spec(p + "wq", (b.q_dim, H), "w", m, fan_in=H),
            Spec(p + "wk", (b.kv_dim, H), "w", m, fan_in=H),
            Spec(p + "wv", (b.kv_dim, H), "w", m, fan_in=H),
            Spec(p + "wo", (H, b.q_dim), "w", m, fan_in=b.q_dim),
            Spec(p + "mlp_norm", (H,), "gain", "f32"),
            Spec(p + "wg", (b.intermediate, H), "w", m, fan_in=H),
            Spec(p + "wu", (b.intermediate, H), "w", m, fan_in=H),
            Spec(p + "wd", (H, b.intermediate), "w", m, fan_in=b.intermediate),
        ]
        if b.qk_norm:
            out += [Spec(p + "q_norm", (b.head_dim,), "gain", "f32"), Spec(p + "k_norm", (b.head_dim,), "gain", "f32")]
    if cfg.final_norm:
        out.append(Spec("llm.final_norm", (H,), "gain", "f32"))
    return out


def vit_specs(cfg: Config) -> List[Spec]:
    v = cfg.vit
    m = "bf16" if cfg.wdtype in ("fp8", "int8") else _mat(cfg)
    D = v.hidden
    out = [
        Spec("vit.pe_w", (D, v.patch_dim), "w", m, fan_in=v.patch_dim),
        Spec("vit.pe_b", (D,), "bias", "f32"),
        Spec("vit.pos", (v.n_patches, D), "bias", "f32"),
    ]
    for l in range(v.layers):
        p = f"vit.{l}."
        out += [
            Spec(p + "ln1_g", (D,), "gain", "f32"), Spec(p + "ln1_b", (D,), "bias", "f32"),
            Spec(p + "wq", (D, D), "w", m, fan_in=D), Spec(p + "bq", (D,), "bias", "f32"),
            Spec(p + "wk", (D, D), "w", m, fan_in=D), Spec(p + "bk", (D,), "bias", "f32"),
            Spec(p + "wv", (D, D), "w", m, fan_in=D), Spec(p + "bv", (D,), "bias", "f32"),
            Spec(p + "wo", (D, D), "w", m, fan_in=D), Spec(p + "bo", (D,), "bias", "f32"),
            Spec(p + "ln2_g", (D,), "gain", "f32"), Spec(p + "ln2_b", (D,), "bias", "f32"),
            Spec(p + "w1", (v.mlp, D), "w", m, fan_in=D), Spec(p + "b1", (v.mlp,), "bias", "f32"),
            Spec(p + "w2", (D, v.mlp), "w", m, fan_in=v.mlp), Spec(p + "b2", (D,), "bias", "f32"),
        ]
    M = v.merged_dim
    out += [
        Spec("mrg.ln_g", (D,), "gain", "f32"), Spec("mrg.ln_b", (D,), "bias", "f32"),
        Spec("mrg.w1", (M, M), "w", m, fan_in=M), Spec("mrg.b1", (M,), "bias", "f32"),
        Spec("mrg.w2", (v.out_dim, M), "w", m, fan_in=M), Spec("mrg.b2", (v.out_dim,), "bias", "f32"),
    ]
    return out


def projector_specs(cfg: Config) -> List[Spec]:
    m = _mat(cfg)
    H, C = cfg.block.hidden, cfg.dit.ctx_dim
    return [Spec("proj.w", (C, H), "w", m, fan_in=H), Spec("proj.b", (C,), "bias", "f32")]


def dit_specs(cfg: Config) -> List[Spec]:
    d = cfg.dit
    m = _mat(cfg)
    D, A = d.hidden, d.action_dim
    out = [
        Spec("dit.in_w", (D, A), "w", m, fan_in=A), Spec("dit.in_b", (D,), "bias", "f32"),
        Spec("dit.t1_w", (D, d.tdim), "w", m, fan_in=d.tdim), Spec("dit.t1_b", (D,), "bias", "f32"),
        Spec("dit.t2_w", (D, D), "w", m, fan_in=D), Spec("dit.t2_b", (D,), "bias", "f32"),
    ]
    for l in range(d.layers):
        p = f"dit.{l}."
        out += [
            Spec(p + "ada_w", (d.n_mod * D, D), "w", m, fan_in=D),
            Spec(p + "ada_b", (d.n_mod * D,), "ada_bias", "f32"),
            Spec(p + "sa_wq", (D, D), "w", m, fan_in=D), Spec(p + "sa_bq", (D,), "bias", "f32"),
            Spec(p + "sa_wk", (D, D), "w", m, fan_in=D), Spec(p + "sa_bk", (D,), "bias", "f32"),
            Spec(p + "sa_wv", (D, D), "w", m, fan_in=D), Spec(p + "sa_bv", (D,), "bias", "f32"),
            Spec(p + "sa_wo", (D, D), "w", m, fan_in=D), Spec(p + "sa_bo", (D,), "bias", "f32"),
            Spec(p + "ca_wq", (D, D), "w", m, fan_in=D), Spec(p + "ca_bq", (D,), "bias", "f32"),
            Spec(p + "ca_wk", (D, d.ctx_dim), "w", m, fan_in=d.ctx_dim), Spec(p + "ca_bk", (D,), "bias", "f32"),
            Spec(p + "ca_wv", (D, d.ctx_dim), "w", m, fan_in=d.ctx_dim), Spec(p + "ca_bv", (D,), "bias", "f32"),
            Spec(p + "ca_wo", (D, D), "w", m, fan_in=D), Spec(p + "ca_bo", (D,), "bias", "f32"),
            Spec(p + "mlp_w1", (d.mlp, D), "w", m, fan_in=D), Spec(p + "mlp_b1", (d.mlp,), "bias", "f32"),
            Spec(p + "mlp_w2", (D, d.mlp), "w", m, fan_in=d.mlp), Spec(p + "mlp_b2", (D,), "bias", "f32"),
        ]
    out += [
        Spec("dit.f_w", (2 * D, D), "w", m, fan_in=D), Spec("dit.f_b", (2 * D,), "ada_bias", "f32"),
        Spec("dit.out_w", (A, D), "w", m, fan_in=D), Spec("dit.out_b", (A,), "bias", "f32"),
    ]
    return out


def weight_specs(cfg: Config) -> List[Spec]:
    if cfg.kind in ("block", "backbone"):
        return backbone_specs(cfg)
    if cfg.kind == "dit":
        return dit_specs(cfg)
    if cfg.kind == "step":
        out = []
        if cfg.vit is not None:
            out += vit_specs(cfg)
        out += backbone_specs(cfg) + projector_specs(cfg) + dit_specs(cfg)
        return out
    raise ValueError(cfg.kind)


def input_specs(cfg: Config) -> List[Spec]:
    a = _act(cfg)
    if cfg.kind in ("block", "backbone"):
        return [Spec("x", (cfg.seq, cfg.block.hidden), "normal", a, KIND_INPUTS)]
    if cfg.kind == "dit":
        d = cfg.dit
        return [Spec("ctx", (cfg.ctx_len, d.ctx_dim), "normal", a, KIND_INPUTS),
                Spec("noise", (d.chunk, d.action_dim), "normal", "f32", KIND_NOISE)]
    if cfg.kind == "step":
        d = cfg.dit
        out = []
        if cfg.vit is not None:
            v = cfg.vit
            out.append(Spec("image", (cfg.n_images, v.channels, v.image, v.image), "normal", a, KIND_INPUTS))
        out.append(Spec("text", (cfg.n_text, cfg.block.hidden), "normal", a, KIND_INPUTS))
        out.append(Spec("noise", (d.chunk, d.action_dim), "normal", "f32", KIND_NOISE))
        return out
    raise ValueError(cfg.kind)


def make_weights(cfg: Config, cache: bool = True) -> TensorSet:
    return TensorSet(cfg, weight_specs(cfg), cache=cache)


def make_inputs(cfg: Config) -> TensorSet:
    return TensorSet(cfg, input_specs(cfg), cache=True)
