"""Workspace plans against the launches that really run, without a GPU.

Every entry point sizes its workspace in a planning pass, then runs the same
schedule on the caller's memory; split-K GEMM partials and key-split
attention partials share one scratch buffer sized by the plan, with the
tile counters right after it. tests/shim/launch_shim.cpp stands in for
hipLaunchKernel in a child process (loaded before the library, so the
library's launches resolve to it): the schedule runs on host buffers, no
kernel executes, and every launch whose partials would reach past the
counters is reported. A plan that took another branch than the run (as
when a buffer's presence decided the path and the planning pass had none)
shows up here as an overflow."""

import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CHILD = r"""
import ctypes, json, sys
import numpy as np
ctypes.CDLL(sys.argv[1], mode=ctypes.RTLD_GLOBAL)
sys.path.insert(0, sys.argv[2])
from vla_robot_policy_amd import lib
a = json.loads(sys.argv[3])
keep = []
def buf(nbytes):
    b = np.zeros(int(nbytes) + 512, np.uint8)
    keep.append(b)
    return (b.ctypes.data + 255) // 256 * 256
wd = {"bf16": lib.VLA_BF16, "fp8": lib.VLA_FP8_E4M3, "int8": lib.VLA_INT8}[a["w"]]
esz = 2 if a["w"] == "bf16" else 1
out = {}
if a["kind"] == "dit":
    D, H, hd, mlp, L, td, cd, A, K, C, n = 160, 2, 80, 640, 2, 256, 160, 7, 2, a["ctx"], a["chunk"]
    cfg = lib.DitCfg(hidden=D, heads=H, head_dim=hd, mlp=mlp, layers=L, tdim=td, ctx_dim=cd, eps=1e-6,
                     time_scale=1000.0, freq_base=10000.0, wdtype=wd, flags=0)
    layers = (lib.DitLayer * L)()
    shp = {"qkv": (3 * D, D), "o": (D, D), "cq": (D, D), "co": (D, D), "up": (mlp, D), "down": (D, mlp)}
    for ly in layers:
        for k, (r, c) in shp.items():
            setattr(ly, "w_" + k, buf(r * c * esz)); setattr(ly, "b_" + k, buf(r * 4))
            if esz == 1: setattr(ly, "s_" + k, buf(r * 4))
    d = lib.Dit(cfg=cfg, layers=layers)
    top = {"ada": (L * 9 * D, D), "ckv": (L * 2 * D, cd), "t1": (D, td), "t2": (D, D), "f": (2 * D, D), "in": (D, A),
           "out": (A, D)}
    for k, (r, c) in top.items():
        setattr(d, "w_" + k, buf(r * c * esz)); setattr(d, "b_" + k, buf(r * 4))
        if esz == 1: setattr(d, "s_" + k, buf(r * 4))
    need = lib.vla_dit_workspace_bytes(d, C, n, A, K)
    out["need"] = need
    out["status"] = lib.vla_flow_euler_sample(d, buf(C * cd * 2), C, buf(n * A * 4), n, A, K, buf(n * A * 4),
                                              buf(K * n * A * 4), buf(need), need) if need else -99
elif a["kind"] == "vit":
    img, pt, D, mlp, L, od = a["image"], 14, 128, 512, 2, 256
    cfg = lib.VitCfg(image=img, patch=pt, channels=3, hidden=D, heads=2, head_dim=64, mlp=mlp, layers=L, merge=2,
                     out_dim=od, eps=1e-6, wdtype=lib.VLA_BF16, flags=0)
    layers = (lib.VitLayer * L)()
    for ly in layers:
        ly.ln1_g = buf(D * 4); ly.ln1_b = buf(D * 4); ly.ln2_g = buf(D * 4); ly.ln2_b = buf(D * 4)
        ly.w_qkv = buf(3 * D * D * 2); ly.b_qkv = buf(3 * D * 4); ly.w_o = buf(D * D * 2); ly.b_o = buf(D * 4)
        ly.w_up = buf(mlp * D * 2); ly.b_up = buf(mlp * 4); ly.w_down = buf(D * mlp * 2); ly.b_down = buf(D * 4)
    g = img // pt
    v = lib.Vit(cfg=cfg, layers=layers, w_pe=buf(D * 3 * pt * pt * 2), b_pe=buf(D * 4), pos=buf(g * g * D * 4),
                mln_g=buf(D * 4), mln_b=buf(D * 4), w_m1=buf(16 * D * D * 2), b_m1=buf(4 * D * 4), w_m2=buf(od * 4 * D * 2),
                b_m2=buf(od * 4))
    n = a["n_images"]
    need = lib.vla_vit_workspace_bytes(v, n)
    out["need"] = need
    out["status"] = lib.vla_vit_encode(v, buf(n * 3 * img * img * 2), n, buf(n * (g * g // 4) * od * 4), None, buf(need),
                                       need) if need else -99
else:
    Hd, I, S = 256, 688, a["seq"]
    cfg = lib.BlockCfg(hidden=Hd, n_q_heads=4, n_kv_heads=2, head_dim=64, intermediate=I, rope_base=1e4, eps=1e-6,
                       wdtype=wd, adtype=lib.VLA_BF16, flags=0)
    layers = (lib.BlockWeights * 2)()
    for ly in layers:
        ly.attn_norm = buf(Hd * 4); ly.mlp_norm = buf(Hd * 4)
        ly.w_qkv = buf(512 * Hd * esz); ly.w_o = buf(Hd * 256 * esz); ly.w_gate_up = buf(2 * I * Hd * esz)
        ly.w_down = buf(Hd * I * esz)
        if esz == 1:
            ly.s_qkv = buf(512 * 4); ly.s_o = buf(Hd * 4); ly.s_gate_up = buf(2 * I * 4); ly.s_down = buf(Hd * 4)
    bb = lib.Backbone(cfg=cfg, n_layers=2, layers=layers, final_norm=buf(Hd * 4))
    need = lib.vla_backbone_workspace_bytes(bb, S)
    out["need"] = need
    out["status"] = lib.vla_backbone_prefill(bb, buf(S * Hd * 2), S, buf(S * Hd * 2), buf(need), need) if need else -99
print(json.dumps(out), flush=True)
"""


@pytest.fixture(scope="module")
def shim(tmp_path_factory):
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    so = str(tmp_path_factory.mktemp("shim") / "launch_shim.so")
    cmd = [HIPCC, "-std=c++17", "-O1", "-fPIC", "-shared", "-x", "hip", "--offload-arch=gfx950",
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "vla_robot_policy_amd", "csrc"),
           os.path.join(ROOT, "tests", "shim", "launch_shim.cpp"), "-o", so, "-ldl"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    return so


def run_child(shim, **case):
    r = subprocess.run([sys.executable, "-c", CHILD, shim, ROOT, json.dumps(case)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    res = json.loads(r.stdout.strip().splitlines()[-1])
    launches = [int(l.split()[1]) for l in r.stderr.splitlines() if l.startswith("launches ")]
    overflows = [l for l in r.stderr.splitlines() if l.startswith("OVERFLOW")]
    return res, (launches[0] if launches else 0), overflows


# the launch-per-operation sampler (chunks above 16 rows) with context rows
# on both sides of 64 (above 64 the cross K/V GEMM does not split, so the
# MLP up-projection's partials size the scratch), and the layer kernel
@pytest.mark.parametrize("chunk,ctx,w", [(50, 530, "bf16"), (37, 70, "fp8"), (64, 19, "int8"), (17, 40, "bf16"),
                                         (16, 400, "bf16"), (5, 70, "fp8")])
def test_dit_plan_covers_launches(shim, chunk, ctx, w):
    res, n, over = run_child(shim, kind="dit", chunk=chunk, ctx=ctx, w=w)
    assert res["status"] == 0 and res["need"] > 0, res
    assert n > 10
    assert not over, over


@pytest.mark.parametrize("seq,w", [(37, "bf16"), (104, "bf16"), (200, "bf16"), (400, "fp8"), (130, "int8")])
def test_backbone_plan_covers_launches(shim, seq, w):
    res, n, over = run_child(shim, kind="backbone", seq=seq, w=w)
    assert res["status"] == 0 and res["need"] > 0, res
    assert n > 10
    assert not over, over


# the vision encoder and merger: one and two images of 8 x 8 and 16 x 16 patches
@pytest.mark.parametrize("image,n_images", [(112, 1), (224, 1), (224, 2)])
def test_vit_plan_covers_launches(shim, image, n_images):
    res, n, over = run_child(shim, kind="vit", image=image, n_images=n_images, w="bf16")
    assert res["status"] == 0 and res["need"] > 0, res
    assert n > 10
    assert not over, over
