"""ctypes binding of libvla (include/vla.h): argument marshalling only.

Every function here has the name of the C entry point it calls and does no
arithmetic of the method; all of the forward pass runs in libvla's HIP
kernels. Loading fails loudly when libvla.so has not been built.
"""

from __future__ import annotations

import ctypes as C
import os
import re
from ctypes import POINTER, c_float, c_int32, c_size_t, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
# VLA_LIB_PATH selects another build of the same library (the host-side
# AddressSanitizer build of build_asan.py); the default is the in-tree one
LIB_PATH = os.environ.get("VLA_LIB_PATH") or os.path.join(HERE, "libvla.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "vla.h")

VLA_OK, VLA_ERR_INVALID_ARG, VLA_ERR_SHAPE, VLA_ERR_UNSUPPORTED, VLA_ERR_WORKSPACE, VLA_ERR_HIP, VLA_ERR_STATE = (
    0, -1, -2, -3, -4, -5, -6)
VLA_ERR_TIMEOUT = -7
VLA_F32, VLA_BF16, VLA_FP8_E4M3, VLA_INT8 = 0, 1, 2, 3
DTYPE_CODE = {"f32": VLA_F32, "bf16": VLA_BF16, "fp8": VLA_FP8_E4M3, "int8": VLA_INT8}
VLA_BLOCK_QK_NORM = 1
VLA_BLOCK_A8 = 2
VLA_BLOCK_PACKED = 4
VLA_STEP_GRAPH_CACHE = 8


class VlaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libvla status {status}: {msg}")
        self.status = status


class BlockCfg(C.Structure):
    _fields_ = [("hidden", c_int32), ("n_q_heads", c_int32), ("n_kv_heads", c_int32), ("head_dim", c_int32),
                ("intermediate", c_int32), ("rope_base", c_float), ("eps", c_float), ("wdtype", c_int32),
                ("adtype", c_int32), ("flags", c_int32)]


class BlockWeights(C.Structure):
    _fields_ = [(n, c_void_p) for n in ("attn_norm", "w_qkv", "s_qkv", "w_o", "s_o", "mlp_norm", "w_gate_up",
                                         "s_gate_up", "w_down", "s_down", "q_norm", "k_norm")]


class Backbone(C.Structure):
    _fields_ = [("cfg", BlockCfg), ("n_layers", c_int32), ("layers", POINTER(BlockWeights)), ("final_norm", c_void_p)]


class DitCfg(C.Structure):
    _fields_ = [(n, c_int32) for n in ("hidden", "heads", "head_dim", "mlp", "layers", "tdim", "ctx_dim")] + \
               [(n, c_float) for n in ("eps", "time_scale", "freq_base")] + [("wdtype", c_int32), ("flags", c_int32)]


_DIT_LAYER = ["qkv", "o", "cq", "co", "up", "down"]
_DIT_TOP = ["ada", "ckv", "t1", "t2", "f", "in", "out"]


class DitLayer(C.Structure):
    _fields_ = [(f"{p}_{n}", c_void_p) for n in _DIT_LAYER for p in ("w", "s", "b")]


class Dit(C.Structure):
    _fields_ = [("cfg", DitCfg), ("layers", POINTER(DitLayer))] + \
               [(f"{p}_{n}", c_void_p) for n in _DIT_TOP for p in ("w", "s", "b")]


class VitCfg(C.Structure):
    _fields_ = [(n, c_int32) for n in ("image", "patch", "channels", "hidden", "heads", "head_dim", "mlp", "layers",
                                         "merge", "out_dim")] + [("eps", c_float), ("wdtype", c_int32), ("flags", c_int32)]


class VitLayer(C.Structure):
    _fields_ = [(n, c_void_p) for n in ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_o", "b_o", "ln2_g", "ln2_b", "w_up",
                                         "b_up", "w_down", "b_down")]


class Vit(C.Structure):
    _fields_ = [("cfg", VitCfg), ("layers", POINTER(VitLayer))] + \
               [(n, c_void_p) for n in ("w_pe", "b_pe", "pos", "mln_g", "mln_b", "w_m1", "b_m1", "w_m2", "b_m2")]


class Model(C.Structure):
    _fields_ = [("vit", POINTER(Vit)), ("backbone", POINTER(Backbone)), ("w_proj", c_void_p), ("s_proj", c_void_p),
                ("b_proj", c_void_p), ("dit", POINTER(Dit))]


class StepShape(C.Structure):
    _fields_ = [(n, c_int32) for n in ("n_images", "n_text", "chunk", "action_dim", "steps")]


class StepIO(C.Structure):
    _fields_ = [(n, c_void_p) for n in ("images", "text", "noise", "actions", "hidden_out", "velocities")]


class StepCacheStats(C.Structure):
    _fields_ = [(n, c_int32) for n in ("entries", "hits", "misses", "evictions")]


_lib = None


def load() -> C.CDLL:
    """Load libvla.so (built by vla_robot_policy_amd.build); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libvla.so not built at {LIB_PATH}; run vla_robot_policy_amd/build.py "
                           "(or __graft_entry__.build()) first")
    lib = C.CDLL(LIB_PATH)
    S = c_int32
    sig = {
        "vla_block_forward": (S, [POINTER(BlockCfg), POINTER(BlockWeights), c_void_p, c_void_p, c_int32, c_void_p, c_size_t, c_void_p]),
        "vla_block_workspace_bytes": (c_size_t, [POINTER(BlockCfg), c_int32]),
        "vla_block_forward_static": (S, [POINTER(BlockCfg), POINTER(BlockWeights), c_void_p, c_void_p, c_int32, c_void_p]),
        "vla_packed_bytes": (c_size_t, [c_int32, c_int32, c_int32]),
        "vla_pack_weights": (S, [c_int32, c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p]),
        "vla_backbone_prefill": (S, [POINTER(Backbone), c_void_p, c_int32, c_void_p, c_void_p, c_size_t, c_void_p]),
        "vla_backbone_workspace_bytes": (c_size_t, [POINTER(Backbone), c_int32]),
        "vla_flow_euler_sample": (S, [POINTER(Dit), c_void_p, c_int32, c_void_p, c_int32, c_int32, c_int32, c_void_p,
                                      c_void_p, c_void_p, c_size_t, c_void_p]),
        "vla_dit_workspace_bytes": (c_size_t, [POINTER(Dit), c_int32, c_int32, c_int32, c_int32]),
        "vla_vit_encode": (S, [POINTER(Vit), c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
        "vla_vit_workspace_bytes": (c_size_t, [POINTER(Vit), c_int32]),
        "vla_step_workspace_bytes": (c_size_t, [POINTER(Model), POINTER(StepShape)]),
        "vla_step_plan_create": (S, [POINTER(Model), POINTER(StepShape), POINTER(StepIO), c_void_p, c_size_t,
                                     POINTER(c_void_p)]),
        "vla_step_run": (S, [c_void_p, c_void_p]),
        "vla_step_capture": (S, [c_void_p, c_void_p]),
        "vla_step_replay": (S, [c_void_p, c_void_p]),
        "vla_step_graph_nodes": (c_int32, [c_void_p]),
        "vla_step_kernel_label": (C.c_char_p, [c_void_p, c_int32]),
        "vla_step_launch_kernel": (S, [c_void_p, c_int32, c_void_p]),
        "vla_quantize_rows": (S, [c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p, c_int32, c_void_p, c_void_p]),
        "vla_step_run_shape": (S, [c_void_p, POINTER(StepShape), c_void_p]),
        "vla_step_fused_workspace_bytes": (c_size_t, [POINTER(Model), POINTER(StepShape)]),
        "vla_step_plan_create_fused": (S, [POINTER(Model), POINTER(StepShape), POINTER(StepIO), c_int32, c_void_p,
                                           c_size_t, POINTER(c_void_p)]),
        "vla_step_cycles": (C.c_int64, [c_void_p]),
        "vla_step_cache_info": (S, [c_void_p, POINTER(StepCacheStats)]),
        "vla_step_plan_destroy": (None, [c_void_p]),
        "vla_workspace_status": (S, [c_void_p, c_void_p]),
        "vla_step_status": (S, [c_void_p, c_void_p]),
        "vla_last_error": (C.c_char_p, []),
        "vla_abi_version": (c_int32, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def header_symbols() -> list:
    """Entry points declared in include/vla.h."""
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(vla_\w+)\s*\(", txt, flags=re.M)))


def check(status: int) -> None:
    if status != VLA_OK:
        raise VlaError(status, load().vla_last_error().decode())


def _p(t) -> int:
    """Device address of a torch tensor (or None / int passthrough)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


# ---------------------------------------------------------------- entry points (same names as the C ABI)

def vla_abi_version() -> int:
    return load().vla_abi_version()


def vla_last_error() -> str:
    return load().vla_last_error().decode()


def vla_block_workspace_bytes(cfg: BlockCfg, seq: int) -> int:
    return load().vla_block_workspace_bytes(C.byref(cfg), seq)


def vla_block_forward(cfg: BlockCfg, w: BlockWeights, x_in, x_out, seq: int, ws, ws_bytes: int, stream: int = 0) -> int:
    return load().vla_block_forward(C.byref(cfg), C.byref(w), _p(x_in), _p(x_out), seq, _p(ws), ws_bytes, stream)


VLA_STATIC_SCRATCH_BYTES = 64 << 20


def vla_block_forward_static(cfg: BlockCfg, w: BlockWeights, x_in, x_out, seq: int, stream: int = 0) -> int:
    return load().vla_block_forward_static(C.byref(cfg), C.byref(w), _p(x_in), _p(x_out), seq, stream)


def vla_packed_bytes(wdtype: int, n: int, k: int) -> int:
    return load().vla_packed_bytes(wdtype, n, k)


def vla_pack_weights(wdtype: int, w, n: int, k: int, ldw: int, packed, stream: int = 0) -> int:
    return load().vla_pack_weights(wdtype, _p(w), n, k, ldw, _p(packed), stream)


def vla_backbone_workspace_bytes(bb: Backbone, seq: int) -> int:
    return load().vla_backbone_workspace_bytes(C.byref(bb), seq)


def vla_backbone_prefill(bb: Backbone, embeds, seq: int, hidden_out, ws, ws_bytes: int, stream: int = 0) -> int:
    return load().vla_backbone_prefill(C.byref(bb), _p(embeds), seq, _p(hidden_out), _p(ws), ws_bytes, stream)


def vla_dit_workspace_bytes(dit: Dit, ctx_len: int, chunk: int, action_dim: int, K: int) -> int:
    return load().vla_dit_workspace_bytes(C.byref(dit), ctx_len, chunk, action_dim, K)


def vla_flow_euler_sample(dit: Dit, ctx, ctx_len: int, x0, chunk: int, action_dim: int, K: int, actions_out,
                          velocities_out, ws, ws_bytes: int, stream: int = 0) -> int:
    return load().vla_flow_euler_sample(C.byref(dit), _p(ctx), ctx_len, _p(x0), chunk, action_dim, K, _p(actions_out),
                                        _p(velocities_out), _p(ws), ws_bytes, stream)


def vla_vit_workspace_bytes(vit: Vit, n_images: int) -> int:
    return load().vla_vit_workspace_bytes(C.byref(vit), n_images)


def vla_vit_encode(vit: Vit, images, n_images: int, tokens_out, vit_out, ws, ws_bytes: int, stream: int = 0) -> int:
    return load().vla_vit_encode(C.byref(vit), _p(images), n_images, _p(tokens_out), _p(vit_out), _p(ws), ws_bytes, stream)


def vla_step_workspace_bytes(model: Model, shape: StepShape) -> int:
    return load().vla_step_workspace_bytes(C.byref(model), C.byref(shape))


def vla_step_plan_create(model: Model, shape: StepShape, io: StepIO, ws, ws_bytes: int):
    out = c_void_p()
    st = load().vla_step_plan_create(C.byref(model), C.byref(shape), C.byref(io), _p(ws), ws_bytes, C.byref(out))
    return st, out.value


def vla_step_run(plan, stream: int = 0) -> int:
    return load().vla_step_run(plan, stream)


def vla_step_capture(plan, stream: int = 0) -> int:
    return load().vla_step_capture(plan, stream)


def vla_step_replay(plan, stream: int = 0) -> int:
    return load().vla_step_replay(plan, stream)


def vla_step_graph_nodes(plan) -> int:
    return load().vla_step_graph_nodes(plan)


def vla_step_kernel_label(plan, index: int):
    r = load().vla_step_kernel_label(plan, index)
    return None if r is None else r.decode()


def vla_step_launch_kernel(plan, index: int, stream: int = 0) -> int:
    return load().vla_step_launch_kernel(plan, index, stream)


def vla_quantize_rows(x, x_dtype: int, code_dtype: int, rows: int, K: int, ldx: int, codes, ldc: int, scales,
                      stream: int = 0) -> int:
    return load().vla_quantize_rows(_p(x), x_dtype, code_dtype, rows, K, ldx, _p(codes), ldc, _p(scales), stream)


def vla_step_fused_workspace_bytes(model: Model, shape: StepShape) -> int:
    return load().vla_step_fused_workspace_bytes(C.byref(model), C.byref(shape))


def vla_step_plan_create_fused(model: Model, shape: StepShape, io: StepIO, n_stale: int, ws, ws_bytes: int):
    out = c_void_p()
    st = load().vla_step_plan_create_fused(C.byref(model), C.byref(shape), C.byref(io), n_stale, _p(ws), ws_bytes,
                                           C.byref(out))
    return st, out.value


def vla_step_cycles(plan) -> int:
    return load().vla_step_cycles(plan)


def vla_step_run_shape(plan, shape: StepShape, stream: int = 0) -> int:
    return load().vla_step_run_shape(plan, C.byref(shape), stream)


def vla_step_cache_info(plan):
    out = StepCacheStats()
    st = load().vla_step_cache_info(plan, C.byref(out))
    return st, out


def vla_workspace_status(ws, stream: int = 0) -> int:
    return load().vla_workspace_status(_p(ws), stream)


def vla_step_status(plan, stream: int = 0) -> int:
    return load().vla_step_status(plan, stream)


def vla_step_plan_destroy(plan) -> None:
    load().vla_step_plan_destroy(plan)
