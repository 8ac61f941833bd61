"""Benchmark of the batch-1 VLA policy step on one MI355X.

Workload (default): the full single-camera step — ViT (24 layers, 224x224
image, 14-px patches) -> 2x2 merger -> 36-layer GQA backbone at 104 tokens ->
projector -> 36-layer DiT in a 4-step flow-matching Euler loop — captured
once as a hipGraph by libvla and replayed; seeded synthetic weights and
inputs of that architecture, bf16. One JSON line on stdout.

  python bench.py [--steps K] [--warmup W] [--config 4] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import json
import re
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ms per VLA step at batch 1 (36L backbone + K-step DiT) + % of MFMA/HBM roofline"
WORKLOADS = {
    1: "one pre-norm decoder block, seq 64, fp32 (hidden 256, GQA 4/2 x 64, SwiGLU 688)",
    2: "36-layer backbone prefill, seq 256, bf16 (hidden 2560, GQA 32/8 x 128, SwiGLU 9728), final RMSNorm",
    3: "DiT flow-matching sampler, bf16: 36 layers x 4 Euler steps, chunk 16x7, 256 context tokens",
    4: ("full single-camera VLA step, bf16: ViT 24L (224x224, 14-px patches) -> 2x2 merger -> 36L backbone "
        "at seq 104 (64 visual + 40 text) -> projector -> DiT 36L x 4 Euler steps; one hipGraph"),
    5: ("two-camera long-context step, fp8 e4m3 weights (per-channel scales), bf16 activations: 36L backbone "
        "at seq 560 -> projector -> DiT 36L x 10 Euler steps, chunk 50x32; one hipGraph"),
}

# backbone Linears in the packed layout of vla_pack_weights (--row-major: as
# uploaded); the results are bitwise the same
PACKED = True

_CODE_TOKENS = re.compile(r'"(?:\\.|[^"\\\n])*"|//[^\n]*|/\*.*?\*/', re.S)


def _strip_comments(text: str) -> str:
    """C/C++ source without comments, trailing blanks or empty lines."""
    code = _CODE_TOKENS.sub(lambda m: m.group(0) if m.group(0).startswith('"') else "", text)
    return "\n".join(ln.rstrip() for ln in code.splitlines() if ln.strip())


def kernel_source_sha() -> str:
    """Hash of the HIP sources' code (the counters of a profile hold for this
    code only; comments do not enter the hash)."""
    import hashlib
    h = hashlib.sha256()
    src = os.path.join(ROOT, "vla_robot_policy_amd", "csrc")
    for name in sorted(os.listdir(src)):
        if name.endswith((".h", ".hip", ".cpp")):
            with open(os.path.join(src, name), encoding="utf-8") as f:
                h.update(name.encode() + b"\0" + _strip_comments(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(label: str, config: int):
    """HBM bytes per launch of `label` from the committed counter summary
    (FETCH_SIZE and WRITE_SIZE passes scaled by a plain copy of known size),
    or None when there is none, it was taken on another workload, or the
    kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    v = t.get("labels", {}).get(label)
    if v is None or t.get("config") != config or t.get("kernel_source_sha") != kernel_source_sha():
        return None
    return float(v["fetch_bytes_per_launch"]) + float(v["write_bytes_per_launch"])


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def copy_probe(nbytes: int, reps: int):
    """A plain device-to-device copy of known size: the reference that turns
    the HBM byte counters of a profiled run into bytes."""
    import torch
    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copied {n * 4} bytes x {reps}")


def shape_cache_bench(cfg, texts, steps, warmup):
    """Step latency per text length from one plan sized for the longest
    (vla_step_run_shape: the first call of a length runs eagerly and
    captures it, later calls replay its graph). Prints its own JSON line."""
    import numpy as np
    import torch
    from synth import make_inputs, make_weights
    from vla_robot_policy_amd import lib
    from vla_robot_policy_amd.device import DeviceWeights, upload_input, workspace

    n_vis = cfg.seq - cfg.n_text
    top = cfg.replace(n_text=max(texts), seq=n_vis + max(texts), ctx_len=n_vis + max(texts))
    W, I = make_weights(top), make_inputs(top)
    dw = DeviceWeights(top, W, keep_host=False, threads=16, packed=PACKED and not top.block.a8)
    model = dw.build_model()
    d = top.dit
    dev = torch.device("cuda:0")
    images = upload_input(I["image"]) if top.vit is not None else None
    text, noise = upload_input(I["text"]), upload_input(I["noise"])
    actions = torch.empty((d.chunk, d.action_dim), dtype=torch.float32, device=dev)

    def shape(nt):
        return lib.StepShape(n_images=top.n_images, n_text=nt, chunk=d.chunk, action_dim=d.action_dim, steps=top.steps)

    io = lib.StepIO(images=None if images is None else images.data_ptr(), text=text.data_ptr(),
                    noise=noise.data_ptr(), actions=actions.data_ptr(), hidden_out=None, velocities=None)
    need = lib.vla_step_workspace_bytes(model, shape(max(texts)))
    ws = workspace(need)
    st, plan = lib.vla_step_plan_create(model, shape(max(texts)), io, ws, need)
    lib.check(st)
    stream = torch.cuda.current_stream().cuda_stream
    rows = []
    try:
        for nt in texts:
            torch.cuda.synchronize()
            t = time.time()
            lib.check(lib.vla_step_run_shape(plan, shape(nt), stream))
            torch.cuda.synchronize()
            miss = (time.time() - t) * 1e3
            for _ in range(warmup):
                lib.check(lib.vla_step_run_shape(plan, shape(nt), stream))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(steps):
                lib.check(lib.vla_step_run_shape(plan, shape(nt), stream))
            e1.record()
            torch.cuda.synchronize()
            rows.append({"n_text": nt, "seq": n_vis + nt, "first_call_ms": round(miss, 2),
                         "replay_ms": round(e0.elapsed_time(e1) / steps, 4)})
            log(f"n_text {nt}: first call {miss:.1f} ms (eager + capture), replay {rows[-1]['replay_ms']:.3f} ms")
        # every call switches to another length: each replay starts with the
        # counter-clearing fill of its layout
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(steps):
            lib.check(lib.vla_step_run_shape(plan, shape(texts[i % len(texts)]), stream))
        e1.record()
        torch.cuda.synchronize()
        switch = e0.elapsed_time(e1) / steps
        st, info = lib.vla_step_cache_info(plan)
        lib.check(st)
    finally:
        lib.vla_step_plan_destroy(plan)
    line = {"metric": "ms per VLA step by text length, one plan with shape-keyed graphs", "unit": "ms",
            "higher_is_better": False, "steps": steps, "warmup": warmup, "data": "synthetic",
            "dtype": cfg.wdtype if cfg.wdtype in ("fp8", "int8") else "bf16",
            "config": {"workload": f"{n_vis} visual tokens + text lengths {texts}; plan sized for n_text {max(texts)}",
                       "global_batch": 1, "euler_steps": top.steps},
            "shapes": rows, "alternating_replay_ms": round(switch, 4),
            "cache": {"entries": info.entries, "hits": info.hits, "misses": info.misses, "evictions": info.evictions}}
    print(json.dumps(line), flush=True)


def fused_bench(cfg, n_stale, steps, warmup):
    """Cycle time of V-AEFusion (the action expert's first n_stale Euler steps
    on the previous cycle's context, alongside the VLM) against the plain
    step, both captured and replayed; prints its own JSON line."""
    import numpy as np
    import torch
    from synth import make_inputs, make_weights
    from vla_robot_policy_amd import lib
    from vla_robot_policy_amd.device import DeviceWeights, upload_input, workspace

    W, I = make_weights(cfg), make_inputs(cfg)
    dw = DeviceWeights(cfg, W, keep_host=False, threads=16, packed=PACKED and not cfg.block.a8)
    model = dw.build_model()
    d = cfg.dit
    dev = torch.device("cuda:0")
    images = upload_input(I["image"]) if cfg.vit is not None else None
    text, noise = upload_input(I["text"]), upload_input(I["noise"])
    actions = torch.empty((d.chunk, d.action_dim), dtype=torch.float32, device=dev)
    shape = lib.StepShape(n_images=cfg.n_images, n_text=cfg.n_text, chunk=d.chunk, action_dim=d.action_dim,
                          steps=cfg.steps)
    io = lib.StepIO(images=None if images is None else images.data_ptr(), text=text.data_ptr(),
                    noise=noise.data_ptr(), actions=actions.data_ptr(), hidden_out=None, velocities=None)
    stream = torch.cuda.current_stream().cuda_stream

    def timed(fused):
        if fused:
            need = lib.vla_step_fused_workspace_bytes(model, shape)
            ws = workspace(need)
            st, plan = lib.vla_step_plan_create_fused(model, shape, io, n_stale, ws, need)
        else:
            need = lib.vla_step_workspace_bytes(model, shape)
            ws = workspace(need)
            st, plan = lib.vla_step_plan_create(model, shape, io, ws, need)
        lib.check(st)
        try:
            lib.check(lib.vla_step_capture(plan, stream))
            for _ in range(warmup):
                lib.check(lib.vla_step_replay(plan, stream))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(steps):
                lib.check(lib.vla_step_replay(plan, stream))
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / steps, lib.vla_step_graph_nodes(plan)
        finally:
            lib.vla_step_plan_destroy(plan)

    plain_ms, plain_nodes = timed(False)
    log(f"plain step {plain_ms:.3f} ms ({plain_nodes} nodes)")
    fused_ms, fused_nodes = timed(True)
    log(f"fused cycle {fused_ms:.3f} ms ({fused_nodes} nodes), {n_stale} of {cfg.steps} steps stale")
    line = {"metric": "ms per control cycle, V-AEFusion (stale action-expert steps alongside the VLM)", "unit": "ms",
            "value": round(fused_ms, 4), "higher_is_better": False, "steps": steps, "warmup": warmup,
            "data": "synthetic", "dtype": cfg.wdtype if cfg.wdtype in ("fp8", "int8") else "bf16",
            "config": {"workload": f"{cfg.name}: {n_stale} of {cfg.steps} Euler steps stale", "global_batch": 1,
                       "seq_len": cfg.seq, "euler_steps": cfg.steps},
            "plain_step_ms": round(plain_ms, 4), "speedup": round(plain_ms / fused_ms, 4),
            "graph_nodes": {"plain": plain_nodes, "fused": fused_nodes}}
    print(json.dumps(line), flush=True)


def phase_of(label: str) -> str:
    """Roofline phase of a kernel label (the phases of roofline.bound)."""
    if label.startswith(("vit.", "mrg.")):
        return "vit"
    if label.startswith("llm."):
        return "backbone"
    if label == "proj":
        return "projector"
    if label in ("dit.time_embed", "dit.time_fc1", "dit.time_fc2", "dit.adaln", "dit.final_mod", "dit.cross_kv",
                 "dit.cross_vt", "dit.clear"):
        return "dit_once"
    if label.startswith("dit."):
        return "dit_step"
    return "other"


def phase_fractions(kernels, bound):
    """Measured time per phase (sum of each label's per-launch duration x
    launches per step) against the phase's roofline bound."""
    meas = {}
    for lb, v in kernels.items():
        ph = phase_of(lb)
        meas[ph] = meas.get(ph, 0.0) + v["avg_us"] * v["count"] * 1e-3
    out = {}
    for ph in sorted(set(meas) | set(bound.per_phase)):
        m, b = meas.get(ph, 0.0), bound.per_phase.get(ph, 0.0) * 1e3
        out[ph] = {"ms": round(m, 4), "bound_ms": round(b, 4), "frac": round(b / m, 4) if m else None}
    return out


def component_bench(cfg, steps, warmup):
    """One block (vla_block_forward), the backbone prefill alone
    (vla_backbone_prefill) or the flow sampler alone (vla_flow_euler_sample),
    launched eagerly back to back on one stream; returns (ms per call, p50,
    p90)."""
    import numpy as np
    import torch
    from synth import make_inputs, make_weights
    from vla_robot_policy_amd import lib
    from vla_robot_policy_amd.device import DeviceWeights, upload_input, workspace

    t0 = time.time()
    W, I = make_weights(cfg), make_inputs(cfg)
    dw = DeviceWeights(cfg, W, keep_host=False, threads=16,
                       packed=PACKED and cfg.kind in ("block", "backbone") and cfg.wdtype != "f32" and not cfg.block.a8)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    if cfg.kind == "block":
        bb = dw.build_backbone()
        x = upload_input(I["x"])
        out = torch.empty((cfg.seq, cfg.block.hidden), dtype=torch.float32 if cfg.wdtype == "f32" else torch.int16,
                          device=dev)
        need = lib.vla_block_workspace_bytes(dw.block_cfg, cfg.seq)
        ws = workspace(need)

        def call():
            lib.check(lib.vla_block_forward(dw.block_cfg, bb.layers[0], x, out, cfg.seq, ws, need, stream))
    elif cfg.kind == "backbone":
        bb = dw.build_backbone()
        x = upload_input(I["x"])
        out = torch.empty((cfg.seq, cfg.block.hidden), dtype=torch.int16, device=dev)
        need = lib.vla_backbone_workspace_bytes(bb, cfg.seq)
        ws = workspace(need)

        def call():
            lib.check(lib.vla_backbone_prefill(bb, x, cfg.seq, out, ws, need, stream))
    else:
        dit = dw.build_dit()
        d = cfg.dit
        ctx, noise = upload_input(I["ctx"]), upload_input(I["noise"])
        acts = torch.empty((d.chunk, d.action_dim), dtype=torch.float32, device=dev)
        need = lib.vla_dit_workspace_bytes(dit, cfg.ctx_len, d.chunk, d.action_dim, cfg.steps)
        ws = workspace(need)

        def call():
            lib.check(lib.vla_flow_euler_sample(dit, ctx, cfg.ctx_len, noise, d.chunk, d.action_dim, cfg.steps, acts,
                                                None, ws, need, stream))
    log(f"weights generated and uploaded in {time.time() - t0:.1f}s")
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for i in range(steps):
        call()
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(steps)])
    ms = evs[0].elapsed_time(evs[steps]) / steps
    log(f"{steps} calls: mean {ms:.3f} ms, p50 {np.median(per):.3f} ms")
    return ms, float(np.median(per)), float(np.percentile(per, 90))


def gpu_step_bench(cfg, steps, warmup, kernel_reps, only_label=None):
    import numpy as np
    import torch
    from synth import make_inputs, make_weights
    from vla_robot_policy_amd import lib
    from vla_robot_policy_amd.device import DeviceWeights, upload_input, workspace

    t0 = time.time()
    W, I = make_weights(cfg), make_inputs(cfg)
    dw = DeviceWeights(cfg, W, keep_host=False, threads=16, packed=PACKED and not cfg.block.a8)
    if cfg.kind == "step":
        model = dw.build_model()
    log(f"weights generated and uploaded in {time.time() - t0:.1f}s")
    d = cfg.dit
    dev = torch.device("cuda:0")
    images = upload_input(I["image"]) if cfg.vit is not None else None
    text = upload_input(I["text"])
    noise = upload_input(I["noise"])
    actions = torch.empty((d.chunk, d.action_dim), dtype=torch.float32, device=dev)
    shape = lib.StepShape(n_images=cfg.n_images, n_text=cfg.n_text, chunk=d.chunk, action_dim=d.action_dim,
                          steps=cfg.steps)
    io = lib.StepIO(images=None if images is None else images.data_ptr(), text=text.data_ptr(),
                    noise=noise.data_ptr(), actions=actions.data_ptr(), hidden_out=None, velocities=None)
    need = lib.vla_step_workspace_bytes(model, shape)
    ws = workspace(need)
    st, plan = lib.vla_step_plan_create(model, shape, io, ws, need)
    lib.check(st)
    stream = torch.cuda.current_stream().cuda_stream
    lib.check(lib.vla_step_capture(plan, stream))
    nodes = lib.vla_step_graph_nodes(plan)
    log(f"captured {nodes} kernel nodes")
    labels = [lib.vla_step_kernel_label(plan, i) for i in range(nodes)]
    if only_label is not None:
        # the kernels of the named labels alone, each label's launches
        # relaunched in graph order, label after label: the run a
        # hardware-counter pass profiles. The launch sequence goes to stderr
        # as one JSON line, so the profiler's dispatches (the last ones of the
        # process) can be attributed to labels.
        names = sorted(set(labels)) if only_label == "all" else only_label.split(",")
        seq = []
        torch.cuda.synchronize()
        for lb in names:
            idx = [i for i, x in enumerate(labels) if x == lb]
            for _ in range(kernel_reps):
                for i in idx:
                    lib.check(lib.vla_step_launch_kernel(plan, i, stream))
            torch.cuda.synchronize()
            seq.append({"label": lb, "launches": len(idx) * kernel_reps, "per_step": len(idx)})
        lib.vla_step_plan_destroy(plan)
        print("[bench] launch sequence " + json.dumps(seq), file=sys.stderr, flush=True)
        log(f"launched {sum(s['launches'] for s in seq)} kernels of {len(seq)} labels")
        return None
    for _ in range(warmup):
        lib.check(lib.vla_step_replay(plan, stream))
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(steps):
        lib.check(lib.vla_step_replay(plan, stream))
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(steps)])
    total_ms = evs[0].elapsed_time(evs[steps])
    log(f"{steps} replays: mean {total_ms / steps:.3f} ms, p50 {np.median(per):.3f} ms")
    # per-kernel durations: every captured launch of a label is relaunched in
    # graph order, back to back on the launch stream between two events, as
    # in a step (each launch reads its own weights, so they arrive from HBM
    # unless one launch's set is small); a 512 MiB read first evicts the
    # 256 MiB last-level cache with clean lines
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    sink = torch.empty(1, dtype=torch.float32, device=dev)
    where, count = {}, {}
    for i, lb in enumerate(labels):
        where.setdefault(lb, []).append(i)
        count[lb] = count.get(lb, 0) + 1
    kern = {}
    for lb, idx in where.items():
        reps = max(1, kernel_reps // len(idx))
        torch.sum(flush, dim=0, out=sink[0])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            for i in idx:
                lib.check(lib.vla_step_launch_kernel(plan, i, stream))
        e1.record()
        torch.cuda.synchronize()
        kern[lb] = {"avg_us": e0.elapsed_time(e1) * 1e3 / (reps * len(idx)), "count": count[lb]}
    del flush
    lib.check(lib.vla_step_replay(plan, stream))   # restore a consistent state
    torch.cuda.synchronize()
    lib.vla_step_plan_destroy(plan)
    return {"ms": total_ms / steps, "p50": float(np.median(per)), "p90": float(np.percentile(per, 90)),
            "nodes": nodes, "kernels": kern}


def cpu_baseline(cfg, reps: int = 3):
    """Oracle (float64 NumPy, as it stands) on a bounded sample of the step:
    `reps` layers of each repeated block type at the workload's shapes, the
    median per layer scaled by the number of such layers in one step."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from synth import make_weights
    from oracle import dit as odit, llm as ollm, vit as ovit
    from oracle.io import Weights

    rng = np.random.default_rng(0)
    W = Weights(make_weights(cfg), keep=True)
    parts = {}

    def clock(key, n_per_step, fn):
        ts = []
        for l in range(reps):
            t = time.time()
            fn(l)
            ts.append(time.time() - t)
        parts[key] = (float(np.median(ts)), n_per_step)

    x = rng.standard_normal((cfg.seq, cfg.block.hidden))
    for l in range(reps):          # converts each sampled layer's weights once, untimed
        ollm.block(x[:4], W, f"llm.{l}.", cfg.block)
    clock("llm_layer", cfg.layers, lambda l: ollm.block(x, W, f"llm.{l}.", cfg.block))
    if cfg.vit is not None:
        v = cfg.vit
        z = rng.standard_normal((v.n_patches, v.hidden))
        for l in range(reps):
            ovit.vit_layer(z[:4], W, f"vit.{l}.", v)
        clock("vit_layer", v.layers * cfg.n_images, lambda l: ovit.vit_layer(z, W, f"vit.{l}.", v))
    d = cfg.dit
    xa = rng.standard_normal((d.chunk, d.hidden))
    sc = rng.standard_normal(d.hidden)
    ctx = rng.standard_normal((cfg.ctx_len, d.ctx_dim))
    for l in range(reps):
        odit.dit_layer(xa, sc, ctx, W, f"dit.{l}.", d)
    clock("dit_layer_step", d.layers * cfg.steps, lambda l: odit.dit_layer(xa, sc, ctx, W, f"dit.{l}.", d))
    est = sum(s * n for s, n in parts.values())
    blas = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": round(est * 1e3, 1), "unit": "ms per step (extrapolated)", "cores": len(os.sched_getaffinity(0)),
            "blas_threads": int(blas), "kind": "oracle",
            "sample": (f"float64 oracle (oracle.llm.block, oracle.vit.vit_layer, oracle.dit.dit_layer), median over "
                       f"{reps} layers of each repeated block at the workload's shapes: "
                       + ", ".join(f"{k} {s * 1e3:.1f} ms x {n}" for k, (s, n) in parts.items())
                       + "; once-per-step parts (patch embed, merger, projector, time MLP, heads) omitted")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--kernel-reps", type=int, default=40,
                    help="launches per label for the per-kernel durations (at least one pass over its launches)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-label", default=None,
                    help="relaunch only the kernel with this label --kernel-reps times (for counter passes)")
    ap.add_argument("--euler-steps", type=int, default=None,
                    help="Euler steps of the sampler (1 = one-step generation); not the default workload")
    ap.add_argument("--a8", action="store_true",
                    help="W8A8: per-token fp8 activations into the backbone's Linears (fp8 workload); not the default")
    ap.add_argument("--int8", action="store_true",
                    help="the fp8 workload with int8 weights and per-token int8 activations in the backbone (W8A8 integer)")
    ap.add_argument("--qk-norm", action="store_true",
                    help="backbone blocks with QK-norm (per-head RMSNorm of Q and K before RoPE); not the default workload")
    ap.add_argument("--shape-cache", default=None,
                    help="comma-separated text lengths: time each from one plan sized for the longest "
                         "(shape-keyed graphs) and print that line instead of the headline")
    ap.add_argument("--fused", type=int, default=None, metavar="N_STALE",
                    help="time V-AEFusion cycles with N_STALE stale Euler steps against the plain step "
                         "and print that line instead of the headline")
    ap.add_argument("--row-major", action="store_true",
                    help="backbone weights as row-major matrices instead of the packed layout of vla_pack_weights")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="run only a device copy of this many bytes --kernel-reps times (counter calibration)")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {a.gpus}); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if a.copy_bytes:
        copy_probe(a.copy_bytes, a.kernel_reps)
        return
    global PACKED
    PACKED = not a.row_major
    from synth import get_config
    from vla_robot_policy_amd import roofline
    cfg = get_config(a.config)
    if a.qk_norm:
        import dataclasses
        cfg = cfg.replace(block=dataclasses.replace(cfg.block, qk_norm=True))
    variant = "; backbone with QK-norm" if a.qk_norm else ""
    if a.a8 or a.int8:
        if cfg.wdtype != "fp8":
            raise SystemExit("--a8 / --int8 need the fp8 workload (--config 5)")
        import dataclasses
        fmt = "int8" if a.int8 else "fp8"
        cfg = cfg.replace(wdtype=fmt, block=dataclasses.replace(cfg.block, a8=fmt))
        variant += (f"; W8A8 {fmt}: {fmt} weights, per-token {fmt} activations into the backbone's Linears "
                    "(codes widened to bf16 for exact products)")
    if a.euler_steps is not None:
        if not 1 <= a.euler_steps <= 64:
            raise SystemExit("--euler-steps must be in [1, 64]")
        cfg = cfg.replace(steps=a.euler_steps)
        variant += f"; sampler run for {a.euler_steps} Euler step{'s' if a.euler_steps > 1 else ''} instead of the workload's"
    if cfg.kind in ("block", "backbone", "dit"):
        if a.only_label or a.fused is not None or a.shape_cache:
            raise SystemExit("--only-label, --fused and --shape-cache need a policy step (--config 4 or 5)")
        ms, p50, p90 = component_bench(cfg, a.steps, a.warmup)
        b = roofline.bound(cfg)
        what = {"block": "decoder block", "backbone": "36-layer backbone prefill", "dit": "flow-matching action sampler"}[cfg.kind]
        print(json.dumps({
            "metric": f"ms per {what} at batch 1 + % of MFMA/HBM roofline", "value": round(ms, 4), "unit": "ms",
            "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 4), "higher_is_better": False,
            "scaling": "weak", "vs_baseline": None, "dtype": cfg.wdtype if cfg.wdtype in ("fp8", "int8", "f32") else "bf16",
            "data": "synthetic",
            "config": {"workload": WORKLOADS[a.config] + variant, "global_batch": 1, "seq_len": cfg.seq if cfg.kind != "dit" else None,
                       "euler_steps": cfg.steps if cfg.kind == "dit" else None, "parallelism": "single GPU"},
            "p50_ms": round(p50, 4), "p90_ms": round(p90, 4),
            "roofline_bound_ms": round(b.seconds * 1e3, 4), "roofline_frac": round(b.seconds * 1e3 / ms, 4),
            "launch": "eager (one entry-point call per step, kernels queued back to back)"}), flush=True)
        return
    if cfg.kind != "step":
        raise SystemExit("bench.py times policy steps (--config 4 or 5), a block (1), the backbone (2) or the sampler (3)")
    if a.fused is not None:
        fused_bench(cfg, a.fused, a.steps, a.warmup)
        return
    if a.shape_cache:
        shape_cache_bench(cfg, [int(t) for t in a.shape_cache.split(",")], a.steps, a.warmup)
        return
    r = gpu_step_bench(cfg, a.steps, a.warmup, a.kernel_reps, a.only_label)
    if r is None:
        return
    b = roofline.bound(cfg)
    ops = {o.name: o for o in b.ops}
    ops.update(roofline.fused_ops(cfg))
    # dominant kernel: largest (per-launch duration x launches per step)
    dom = max(r["kernels"].items(), key=lambda kv: kv[1]["avg_us"] * kv[1]["count"])
    name, kd = dom
    roof = None
    if name in ops:
        o = ops[name]
        peaks = roofline.MI355X
        hbm_bound = o.bytes / peaks["hbm"] >= o.flops / peaks[o.compute]
        dur = kd["avg_us"] * 1e-6
        if hbm_bound:
            ach, peak, unit = o.bytes / dur / 1e9, peaks["hbm"] / 1e9, "GB/s"
        else:
            ach, peak, unit = o.flops / dur / 1e12, peaks[o.compute] / 1e12, "TFLOP/s"
        roof = {"kernel": name, "bound": "hbm" if hbm_bound else "mfma", "achieved": round(ach, 1), "peak": peak,
                "unit": unit, "frac": round(ach / peak, 4), "traffic": measured_traffic(name, a.config),
                "avg_launch_us": round(kd["avg_us"], 2), "launches_per_step": kd["count"],
                "algorithmic_bytes_per_launch": o.bytes, "flops_per_launch": o.flops}
    cpu = None
    if not a.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(cfg)
    ms = r["ms"]
    line = {
        "metric": METRIC, "value": round(ms, 4), "unit": "ms", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.wdtype if cfg.wdtype in ("fp8", "int8") else "bf16", "data": "synthetic",
        "config": {"workload": WORKLOADS[a.config] + variant,
                   "global_batch": 1, "seq_len": cfg.seq,
                   "euler_steps": cfg.steps, "parallelism": "single GPU"},
        "hz": round(1000.0 / ms, 2), "p50_ms": round(r["p50"], 4), "p90_ms": round(r["p90"], 4),
        "tokens_per_s": round(cfg.seq / (ms * 1e-3), 1),
        "roofline_bound_ms": round(b.seconds * 1e3, 4), "roofline_frac_step": round(b.seconds * 1e3 / ms, 4),
        "phases": phase_fractions(r["kernels"], b),
        "graph_nodes": r["nodes"],
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels_us": {k: {"avg_us": round(v["avg_us"], 2), "count": v["count"]} for k, v in sorted(r["kernels"].items())},
        "pages_context": {"starvla_rtx4090_ms": 32.0, "pi05_rtx4090_bf16_ms": 31.38, "pi05_thor_fp8_ms": 26.32},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
