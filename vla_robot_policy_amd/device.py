"""Upload seeded weights to the GPU and describe them to libvla.

Plumbing only: raw storage bytes (float32, bf16 bits, E4M3FN codes + scales)
are copied to device memory with torch, row blocks that libvla expects fused
(W_q|W_k|W_v, W_gate|W_up, the per-layer adaLN and cross-attention K/V
stacks) are concatenated on the host, and the ctypes structs of lib.py are
filled with the device addresses. Tensors stay referenced by the object so
the addresses remain valid for as long as it lives.
"""

from __future__ import annotations

import ctypes as C
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

from . import lib

_NP_RAW = {"f32": np.float32, "bf16": np.int16, "fp8": np.uint8, "int8": np.int8}


class DeviceWeights:
    def __init__(self, cfg, tensors, device: str = "cuda:0", threads: int = 8, keep_host: bool = True,
                 packed: bool = False):
        self.cfg = cfg
        # backbone Linears in the packed layout of vla_pack_weights (bf16 / 8-bit
        # weights with bf16 activations only)
        self.packed = packed
        self.keep_host = keep_host
        self.t = tensors
        self.device = torch.device(device)
        self.keep: List[torch.Tensor] = []
        self.threads = threads
        self.block_cfg = None
        self.backbone = None
        self.dit = None
        self.vit = None
        self.model = None
        self._structs = []

    # ------------------------------------------------------------ raw uploads
    def up_array(self, a: np.ndarray) -> torch.Tensor:
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        t = torch.from_numpy(a).to(self.device)
        self.keep.append(t)
        return t

    def up(self, name: str) -> int:
        return self.up_array(self.t[name].data).data_ptr()

    def up_rows(self, names: Sequence[str], pad_cols: int = 0):
        """Concatenate matrices along rows (and their 8-bit scales); returns (w, s)."""
        ts = [self.t[n] for n in names]
        data = np.concatenate([t.data for t in ts], axis=0)
        if pad_cols:
            data = np.pad(data, ((0, 0), (0, pad_cols)))
        w = self.up_array(data).data_ptr()
        s = None
        if ts[0].dtype in ("fp8", "int8"):
            s = self.up_array(np.concatenate([t.scale for t in ts])).data_ptr()
        return w, s

    def up_rows_packed(self, names: Sequence[str], code: int = None):
        """up_rows, then the matrix repacked on the device by vla_pack_weights
        (the row-major upload is dropped once the packing kernel has run);
        code: the weights' dtype (default: the model's)."""
        w, s = self.up_rows(names)
        src = next(t for t in reversed(self.keep) if t.data_ptr() == w)
        n = sum(self.t[x].data.shape[0] for x in names)
        k = self.t[names[0]].data.shape[1]
        code = lib.DTYPE_CODE[self.cfg.wdtype] if code is None else code
        out = torch.empty(lib.vla_packed_bytes(code, n, k), dtype=torch.uint8, device=self.device)
        lib.check(lib.vla_pack_weights(code, src, n, k, k, out, torch.cuda.current_stream(self.device).cuda_stream))
        torch.cuda.synchronize(self.device)
        self.keep = [t for t in self.keep if t is not src]
        self.keep.append(out)
        return out.data_ptr(), s

    def up_vec(self, names: Sequence[str]) -> int:
        return self.up_array(np.concatenate([self.t[n].data for n in names]).astype(np.float32)).data_ptr()

    def prefetch(self, names: Sequence[str]) -> None:
        if not self.keep_host:
            self.release()
        self._pending = list(names)
        self.t.generate_all(threads=self.threads, names=list(names))

    def release(self) -> None:
        """Drop the host copies of the last prefetched group (keep_host=False)."""
        if getattr(self, "_pending", None):
            self.t.drop(self._pending)
            self._pending = []

    # ------------------------------------------------------------ components
    def build_backbone(self) -> lib.Backbone:
        cfg = self.cfg
        b = cfg.block
        bc = lib.BlockCfg(hidden=b.hidden, n_q_heads=b.n_q_heads, n_kv_heads=b.n_kv_heads, head_dim=b.head_dim,
                          intermediate=b.intermediate, rope_base=b.rope_base, eps=b.eps,
                          wdtype=lib.DTYPE_CODE[cfg.wdtype], adtype=lib.VLA_F32 if cfg.wdtype == "f32" else lib.VLA_BF16,
                          flags=(lib.VLA_BLOCK_QK_NORM if b.qk_norm else 0) | (lib.VLA_BLOCK_A8 if b.a8 else 0)
                          | (lib.VLA_BLOCK_PACKED if self.packed else 0))
        rows = self.up_rows_packed if self.packed else self.up_rows
        layers = (lib.BlockWeights * cfg.layers)()
        for l in range(cfg.layers):
            p = f"llm.{l}."
            extra = ("q_norm", "k_norm") if b.qk_norm else ()
            self.prefetch([p + n for n in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "wg", "wu", "wd") + extra])
            L = layers[l]
            L.attn_norm = self.up(p + "attn_norm")
            L.w_qkv, L.s_qkv = rows([p + "wq", p + "wk", p + "wv"])
            L.w_o, L.s_o = rows([p + "wo"])
            L.mlp_norm = self.up(p + "mlp_norm")
            L.w_gate_up, L.s_gate_up = rows([p + "wg", p + "wu"])
            L.w_down, L.s_down = rows([p + "wd"])
            if b.qk_norm:
                L.q_norm = self.up(p + "q_norm")
                L.k_norm = self.up(p + "k_norm")
        final = self.up("llm.final_norm") if cfg.final_norm else None
        self.block_cfg = bc
        self._bb_layers = layers
        self.backbone = lib.Backbone(cfg=bc, n_layers=cfg.layers, layers=layers, final_norm=final)
        return self.backbone

    def build_dit(self) -> lib.Dit:
        cfg = self.cfg
        d = cfg.dit
        dc = lib.DitCfg(hidden=d.hidden, heads=d.heads, head_dim=d.head_dim, mlp=d.mlp, layers=d.layers, tdim=d.tdim,
                        ctx_dim=d.ctx_dim, eps=d.eps, time_scale=d.time_scale, freq_base=d.freq_base,
                        wdtype=lib.DTYPE_CODE[cfg.wdtype], flags=0)
        layers = (lib.DitLayer * d.layers)()
        ada_w, ada_b, ckv_w, ckv_b = [], [], [], []
        for l in range(d.layers):
            p = f"dit.{l}."
            stacked = ("ada_w", "ada_b", "ca_wk", "ca_wv", "ca_bk", "ca_bv")
            self.prefetch([n for n in self.t.names() if n.startswith(p) and n[len(p):] not in stacked])
            L = layers[l]
            L.w_qkv, L.s_qkv = self.up_rows([p + "sa_wq", p + "sa_wk", p + "sa_wv"])
            L.b_qkv = self.up_vec([p + "sa_bq", p + "sa_bk", p + "sa_bv"])
            L.w_o, L.s_o = self.up_rows([p + "sa_wo"])
            L.b_o = self.up_vec([p + "sa_bo"])
            L.w_cq, L.s_cq = self.up_rows([p + "ca_wq"])
            L.b_cq = self.up_vec([p + "ca_bq"])
            L.w_co, L.s_co = self.up_rows([p + "ca_wo"])
            L.b_co = self.up_vec([p + "ca_bo"])
            L.w_up, L.s_up = self.up_rows([p + "mlp_w1"])
            L.b_up = self.up_vec([p + "mlp_b1"])
            L.w_down, L.s_down = self.up_rows([p + "mlp_w2"])
            L.b_down = self.up_vec([p + "mlp_b2"])
            ada_w.append(p + "ada_w"); ada_b.append(p + "ada_b")
            ckv_w += [p + "ca_wk", p + "ca_wv"]; ckv_b += [p + "ca_bk", p + "ca_bv"]
        D = lib.Dit(cfg=dc, layers=layers)
        self.prefetch(ada_w + ada_b + ckv_w + ckv_b)
        D.w_ada, D.s_ada = self.up_rows(ada_w)
        D.b_ada = self.up_vec(ada_b)
        D.w_ckv, D.s_ckv = self.up_rows(ckv_w)
        D.b_ckv = self.up_vec(ckv_b)
        self.prefetch([n for n in self.t.names() if n.startswith("dit.") and n.split(".")[1] in
                       ("t1_w", "t1_b", "t2_w", "t2_b", "f_w", "f_b", "in_w", "in_b", "out_w", "out_b")])
        D.w_t1, D.s_t1 = self.up_rows(["dit.t1_w"]); D.b_t1 = self.up_vec(["dit.t1_b"])
        D.w_t2, D.s_t2 = self.up_rows(["dit.t2_w"]); D.b_t2 = self.up_vec(["dit.t2_b"])
        D.w_f, D.s_f = self.up_rows(["dit.f_w"]); D.b_f = self.up_vec(["dit.f_b"])
        D.w_in, D.s_in = self.up_rows(["dit.in_w"]); D.b_in = self.up_vec(["dit.in_b"])
        D.w_out, D.s_out = self.up_rows(["dit.out_w"]); D.b_out = self.up_vec(["dit.out_b"])
        self._dit_layers = layers
        self.dit = D
        return D

    def build_vit(self) -> lib.Vit:
        cfg = self.cfg
        v = cfg.vit
        vc = lib.VitCfg(image=v.image, patch=v.patch, channels=v.channels, hidden=v.hidden, heads=v.heads,
                        head_dim=v.head_dim, mlp=v.mlp, layers=v.layers, merge=v.merge, out_dim=v.out_dim, eps=v.eps,
                        wdtype=lib.VLA_BF16, flags=lib.VLA_BLOCK_PACKED if self.packed else 0)
        # the encoder's weights are bf16 whatever the backbone's
        rows = (lambda names: self.up_rows_packed(names, lib.VLA_BF16)) if self.packed else self.up_rows
        layers = (lib.VitLayer * v.layers)()
        for l in range(v.layers):
            p = f"vit.{l}."
            self.prefetch([n for n in self.t.names() if n.startswith(p)])
            L = layers[l]
            L.ln1_g, L.ln1_b = self.up(p + "ln1_g"), self.up(p + "ln1_b")
            L.w_qkv, _ = rows([p + "wq", p + "wk", p + "wv"])
            L.b_qkv = self.up_vec([p + "bq", p + "bk", p + "bv"])
            L.w_o, _ = rows([p + "wo"]); L.b_o = self.up_vec([p + "bo"])
            L.ln2_g, L.ln2_b = self.up(p + "ln2_g"), self.up(p + "ln2_b")
            L.w_up, _ = rows([p + "w1"]); L.b_up = self.up_vec([p + "b1"])
            L.w_down, _ = rows([p + "w2"]); L.b_down = self.up_vec([p + "b2"])
        V = lib.Vit(cfg=vc, layers=layers)
        pad = (-v.patch_dim) % 8
        V.w_pe, _ = self.up_rows(["vit.pe_w"], pad_cols=pad)
        V.b_pe = self.up("vit.pe_b")
        V.pos = self.up("vit.pos")
        V.mln_g, V.mln_b = self.up("mrg.ln_g"), self.up("mrg.ln_b")
        V.w_m1, _ = self.up_rows(["mrg.w1"]); V.b_m1 = self.up_vec(["mrg.b1"])
        V.w_m2, _ = self.up_rows(["mrg.w2"]); V.b_m2 = self.up_vec(["mrg.b2"])
        self._vit_layers = layers
        self.vit = V
        return V

    def build_model(self) -> lib.Model:
        cfg = self.cfg
        if cfg.vit is not None:
            self.build_vit()
        self.build_backbone()
        self.build_dit()
        M = lib.Model()
        M.vit = C.pointer(self.vit) if self.vit is not None else None
        M.backbone = C.pointer(self.backbone)
        M.w_proj, M.s_proj = self.up_rows(["proj.w"])
        M.b_proj = self.up_vec(["proj.b"])
        M.dit = C.pointer(self.dit)
        self.model = M
        if not self.keep_host:
            self.release()
            self.t.drop(self.t.names())
        return M


def upload_input(t, device="cuda:0") -> torch.Tensor:
    """Raw upload of a seeded input tensor (bf16 bits stay bits)."""
    a = np.ascontiguousarray(t.data)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(torch.device(device))


def workspace(nbytes: int, device="cuda:0") -> torch.Tensor:
    """A 256-byte aligned device workspace of at least nbytes."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=torch.device(device))


def bf16_bits_to_float(t: torch.Tensor) -> np.ndarray:
    """Device bf16 bits (int16 tensor) -> host float32 values."""
    a = t.detach().cpu().numpy().view(np.uint16).astype(np.uint32) << np.uint32(16)
    return a.view(np.float32)
