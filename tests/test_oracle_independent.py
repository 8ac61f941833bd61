"""Independent pins of the oracle's vision encoder, merger, time conditioning
and DiT cross-attention branch.

Each pin compares an oracle function with a second implementation built
from library routines (torch float64: ``TransformerEncoderLayer``,
``conv2d``, ``layer_norm``, ``scaled_dot_product_attention``, ``Linear``),
or with a closed form. Every pin is then run against planted mistakes: a
mutant is the oracle function's own source with one plausible slip edited
in (a causal mask, a gain taken from the wrong norm, a dropped bias, K/V
taken from the wrong operand, ...), executed in the oracle module's
namespace. A pin that a mutant passes would not be a pin, so each test
asserts that the real function passes and every mutant fails.

Sources: page "AI Infra如何优化VLA - 模型推理性能提升技术拆解", section 整体方案
(ViT encoder, DiT action head, Sin/Cos timestep operator) and section CUDA
Graph (PatchEmbed -> ViT blocks -> Merger).
"""

import inspect
import textwrap

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import dit, ops, vit
from oracle.io import Weights
from synth import make_weights, small_config
from synth.configs import DiTShape, ViTShape


def mutant(fn, old: str, new: str):
    """fn with `old` replaced by `new` in its source, compiled in fn's module."""
    src = textwrap.dedent(inspect.getsource(fn))
    assert old in src, f"mutation site not found in {fn.__name__}: {old!r}"
    ns = dict(fn.__globals__)
    exec(compile(src.replace(old, new), f"<mutant of {fn.__name__}>", "exec"), ns)
    return ns[fn.__name__]


def T(a):
    return torch.as_tensor(np.asarray(a, dtype=np.float64))


def rel(a, b) -> float:
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


class DictW(dict):
    pass


def _weights(cfg, prefix):
    Wt = make_weights(cfg)
    W = Weights(Wt)
    return DictW({n: W[n] for n in Wt.names() if n.startswith(prefix)})


# ---------------------------------------------------------------- ViT layer

VIT = ViTShape(image=56, patch=14, hidden=128, heads=2, head_dim=64, mlp=512, layers=2, out_dim=256)


def _vit_weights():
    cfg = small_config("step", "bf16").replace(vit=VIT)
    return _weights(cfg, "vit.") | _weights(cfg, "mrg.")


def _torch_encoder_layer(W, p, v):
    """torch's pre-norm encoder layer (exact-erf GELU, no dropout) carrying
    the block's weights."""
    D = v.hidden
    m = torch.nn.TransformerEncoderLayer(D, v.heads, dim_feedforward=v.mlp, dropout=0.0, activation="gelu",
                                         layer_norm_eps=v.eps, batch_first=True, norm_first=True,
                                         dtype=torch.float64)
    with torch.no_grad():
        m.self_attn.in_proj_weight.copy_(T(np.concatenate([W[p + "wq"], W[p + "wk"], W[p + "wv"]])))
        m.self_attn.in_proj_bias.copy_(T(np.concatenate([W[p + "bq"], W[p + "bk"], W[p + "bv"]])))
        m.self_attn.out_proj.weight.copy_(T(W[p + "wo"]))
        m.self_attn.out_proj.bias.copy_(T(W[p + "bo"]))
        m.linear1.weight.copy_(T(W[p + "w1"]))
        m.linear1.bias.copy_(T(W[p + "b1"]))
        m.linear2.weight.copy_(T(W[p + "w2"]))
        m.linear2.bias.copy_(T(W[p + "b2"]))
        m.norm1.weight.copy_(T(W[p + "ln1_g"]))
        m.norm1.bias.copy_(T(W[p + "ln1_b"]))
        m.norm2.weight.copy_(T(W[p + "ln2_g"]))
        m.norm2.bias.copy_(T(W[p + "ln2_b"]))
    m.train()   # dropout is 0; training mode keeps torch off its fused inference path
    return m


def _vit_layer_error(layer_fn, W, z):
    want = _torch_encoder_layer(W, "vit.0.", VIT)(T(z)[None])[0].detach().numpy()
    return rel(layer_fn(z, W, "vit.0.", VIT), want)


def test_vit_layer_matches_torch_encoder_layer():
    W = _vit_weights()
    z = np.random.default_rng(3).standard_normal((VIT.n_patches, VIT.hidden))
    assert _vit_layer_error(vit.vit_layer, W, z) < 1e-13
    mutants = {
        "causal mask": mutant(vit.vit_layer, "causal=False", "causal=True"),
        "LN1 gain in the MLP branch": mutant(vit.vit_layer, 'ops.layernorm(z, W[p + "ln2_g"]', 'ops.layernorm(z, W[p + "ln1_g"]'),
        "query bias dropped": mutant(vit.vit_layer, 'W[p + "wq"], W[p + "bq"]', 'W[p + "wq"], None'),
        "post-norm residual": mutant(vit.vit_layer, "return z + ops.linear(", "return ops.linear("),
        "attention output bias dropped": mutant(vit.vit_layer, 'W[p + "wo"], W[p + "bo"]', 'W[p + "wo"], None'),
    }
    for name, fn in mutants.items():
        assert _vit_layer_error(fn, W, z) > 1e-6, f"planted mistake not caught: {name}"


def test_vit_equal_patch_rows_attend_to_their_value_row():
    """All patch rows equal => every attention row is uniform and returns the
    common value row: the block equals its two residual branches evaluated
    on that single row."""
    W = _vit_weights()
    p = "vit.0."
    row = np.random.default_rng(5).standard_normal(VIT.hidden)
    z = np.tile(row, (VIT.n_patches, 1))
    u = F.layer_norm(T(row), (VIT.hidden,), T(W[p + "ln1_g"]), T(W[p + "ln1_b"]), VIT.eps)
    vrow = F.linear(u, T(W[p + "wv"]), T(W[p + "bv"]))
    h = T(row) + F.linear(vrow, T(W[p + "wo"]), T(W[p + "bo"]))
    u2 = F.layer_norm(h, (VIT.hidden,), T(W[p + "ln2_g"]), T(W[p + "ln2_b"]), VIT.eps)
    want = h + F.linear(F.gelu(F.linear(u2, T(W[p + "w1"]), T(W[p + "b1"]))), T(W[p + "w2"]), T(W[p + "b2"]))
    got = vit.vit_layer(z, W, p, VIT)
    np.testing.assert_allclose(got, np.tile(want.numpy(), (VIT.n_patches, 1)), rtol=1e-12, atol=1e-12)


def test_vit_encoder_matches_conv_patch_embedding_and_torch_layers():
    """Whole encoder: a stride-14 conv2d with the embedding weight seen as
    [D, C, 14, 14] (flatten order channel, row, column), raster order of the
    output grid, the position table, then torch's encoder layers."""
    W = _vit_weights()
    img = np.random.default_rng(7).standard_normal((3, VIT.image, VIT.image))
    D, P = VIT.hidden, VIT.patch
    z = F.conv2d(T(img)[None], T(W["vit.pe_w"]).reshape(D, 3, P, P), T(W["vit.pe_b"]), stride=P)
    z = z.flatten(2).transpose(1, 2) + T(W["vit.pos"])[None]
    for l in range(VIT.layers):
        z = _torch_encoder_layer(W, f"vit.{l}.", VIT)(z)
    assert rel(vit.vit(img, W, VIT), z[0].detach().numpy()) < 1e-13


# ---------------------------------------------------------------- merger

def _torch_merger(W, z, v):
    u = F.layer_norm(T(z), (v.hidden,), T(W["mrg.ln_g"]), T(W["mrg.ln_b"]), v.eps)
    g, m = v.grid, v.merge
    u = u.reshape(g // m, m, g // m, m, v.hidden).permute(0, 2, 1, 3, 4).reshape(-1, m * m * v.hidden)
    h = F.gelu(F.linear(u, T(W["mrg.w1"]), T(W["mrg.b1"])))
    return F.linear(h, T(W["mrg.w2"]), T(W["mrg.b2"])).numpy()


def test_merger_matches_torch_reshape_permute():
    """LayerNorm per patch, then each 2x2 group concatenated in raster order
    (torch reshape to [g/2, 2, g/2, 2, D] and permute), then the GELU MLP."""
    W = _vit_weights()
    z = np.random.default_rng(11).standard_normal((VIT.n_patches, VIT.hidden)) * 3 + 0.5
    want = _torch_merger(W, z, VIT)
    assert rel(vit.merger(z, W, VIT), want) < 1e-13
    post_ln = mutant(vit.merger,
                     'u = ops.layernorm(z, W["mrg.ln_g"], W["mrg.ln_b"], v.eps)\n    g = merge_groups(u, v.grid, v.merge)',
                     'g = merge_groups(z, v.grid, v.merge)\n'
                     '    g = ops.layernorm(g, np.tile(W["mrg.ln_g"], v.merge * v.merge), '
                     'np.tile(W["mrg.ln_b"], v.merge * v.merge), v.eps)')
    no_gelu = mutant(vit.merger, "ops.gelu(ops.linear(g,", "(ops.linear(g,")
    for name, fn in {"LayerNorm after the merge": post_ln, "GELU dropped": no_gelu}.items():
        assert rel(fn(z, W, VIT), want) > 1e-6, f"planted mistake not caught: {name}"


def test_merger_segments_are_normalised_patches(monkeypatch):
    """Every D-wide segment of every merged row is one LayerNorm-ed patch:
    with the affine terms removed, zero mean and variance s2 / (s2 + eps)."""
    W = _vit_weights()
    z = np.random.default_rng(13).standard_normal((VIT.n_patches, VIT.hidden)) * 2 + 1.0
    seen = {}
    real = vit.merge_groups

    def spy(u, grid, m):
        out = real(u, grid, m)
        seen["g"] = out
        return out

    monkeypatch.setattr(vit, "merge_groups", spy)
    vit.merger(z, W, VIT)
    seg = (seen["g"].reshape(-1, VIT.merge * VIT.merge, VIT.hidden) - W["mrg.ln_b"]) / W["mrg.ln_g"]
    np.testing.assert_allclose(seg.mean(-1), 0.0, atol=1e-12)
    s2 = z.var(-1)
    want_var = np.sort(s2 / (s2 + VIT.eps))
    np.testing.assert_allclose(np.sort(seg.var(-1).ravel()), want_var, rtol=1e-10)


# ---------------------------------------------------------------- time conditioning

def _dit_cfg():
    return small_config("dit", "bf16")


def _torch_time_condition(W, d, t):
    half = d.tdim // 2
    w = d.freq_base ** (-torch.arange(half, dtype=torch.float64) / half)
    phi = torch.cat([torch.cos(d.time_scale * t * w), torch.sin(d.time_scale * t * w)])
    f64 = torch.float64
    mlp = torch.nn.Sequential(torch.nn.Linear(d.tdim, d.hidden, dtype=f64), torch.nn.SiLU(),
                              torch.nn.Linear(d.hidden, d.hidden, dtype=f64))
    with torch.no_grad():
        mlp[0].weight.copy_(T(W["dit.t1_w"]))
        mlp[0].bias.copy_(T(W["dit.t1_b"]))
        mlp[2].weight.copy_(T(W["dit.t2_w"]))
        mlp[2].bias.copy_(T(W["dit.t2_b"]))
        return mlp(phi).numpy()


def test_time_condition_matches_torch_mlp():
    cfg = _dit_cfg()
    W = _weights(cfg, "dit.")
    d = cfg.dit
    ts = (0.0, 0.25, 0.5, 0.75, 0.1)
    for t in ts:
        assert rel(dit.time_condition(t, W, d), _torch_time_condition(W, d, t)) < 1e-13
    mutants = {
        "GELU instead of SiLU": mutant(dit.time_condition, "ops.silu(", "ops.gelu("),
        "first bias dropped": mutant(dit.time_condition, 'W["dit.t1_w"], W["dit.t1_b"]', 'W["dit.t1_w"], None'),
        "second layer skipped": mutant(dit.time_condition,
                                       'return ops.linear(ops.silu(ops.linear(phi, W["dit.t1_w"], W["dit.t1_b"])), W["dit.t2_w"], W["dit.t2_b"])',
                                       'return ops.silu(ops.linear(phi, W["dit.t1_w"], W["dit.t1_b"]))'),
    }
    for name, fn in mutants.items():
        worst = max(rel(fn(t, W, d), _torch_time_condition(W, d, t)) for t in ts)
        assert worst > 1e-6, f"planted mistake not caught: {name}"


# ---------------------------------------------------------------- DiT cross-attention branch

def _ca_only_weights(rng, d):
    """Layer 0 of the small DiT with its modulation fixed by the bias alone:
    the self-attention and MLP gates are zero, so the layer adds only the
    gated cross-attention branch; shifts and scales are random."""
    W = _weights(_dit_cfg(), "dit.")
    D = d.hidden
    W["dit.0.ada_w"] = np.zeros_like(W["dit.0.ada_w"])
    b = rng.standard_normal((9, D)) * 0.3
    b[2] = 0.0   # self-attention gate
    b[8] = 0.0   # MLP gate
    b[5] = rng.uniform(0.5, 1.5, D)   # cross-attention gate
    W["dit.0.ada_b"] = b.reshape(-1)
    return W, b


def _branch(layer_fn, W, x, ctx, d):
    return layer_fn(x, np.zeros(d.hidden), ctx, W, "dit.0.", d) - x


def _torch_ca_branch(W, b, x, ctx, d):
    """gate_ca * O(SDPA(q, K_c, V_c)), q from the modulated LayerNorm of x,
    K_c and V_c from the context, all through torch routines."""
    p = "dit.0."
    n, D = x.shape
    u = F.layer_norm(T(x), (D,), eps=d.eps) * (1 + T(b[4])) + T(b[3])
    q = F.linear(u, T(W[p + "ca_wq"]), T(W[p + "ca_bq"])).reshape(n, d.heads, d.head_dim).transpose(0, 1)
    k = F.linear(T(ctx), T(W[p + "ca_wk"]), T(W[p + "ca_bk"])).reshape(-1, d.heads, d.head_dim).transpose(0, 1)
    v = F.linear(T(ctx), T(W[p + "ca_wv"]), T(W[p + "ca_bv"])).reshape(-1, d.heads, d.head_dim).transpose(0, 1)
    o = F.scaled_dot_product_attention(q[None], k[None], v[None])[0].transpose(0, 1).reshape(n, D)
    return (T(b[5]) * F.linear(o, T(W[p + "ca_wo"]), T(W[p + "ca_bo"]))).numpy()


CA_MUTANTS = {
    "K/V from the modulated rows instead of the context": [
        ('ops.linear(ctx, W[p + "ca_wk"]', 'ops.linear(u, W[p + "ca_wk"]'),
        ('ops.linear(ctx, W[p + "ca_wv"]', 'ops.linear(u, W[p + "ca_wv"]'),
        ("L = ctx.shape[0]", "L = u.shape[0]")],
    "K and V weights swapped": [
        ('ops.linear(ctx, W[p + "ca_wk"], W[p + "ca_bk"])', "KSLOT"),
        ('ops.linear(ctx, W[p + "ca_wv"], W[p + "ca_bv"])', 'ops.linear(ctx, W[p + "ca_wk"], W[p + "ca_bk"])'),
        ("KSLOT", 'ops.linear(ctx, W[p + "ca_wv"], W[p + "ca_bv"])')],
    "query from the unmodulated stream": [
        ('q = ops.linear(u, W[p + "ca_wq"]', 'q = ops.linear(x, W[p + "ca_wq"]')],
    "value bias dropped": [('W[p + "ca_wv"], W[p + "ca_bv"]', 'W[p + "ca_wv"], None')],
}


def _ca_mutants():
    out = {}
    for name, edits in CA_MUTANTS.items():
        src = textwrap.dedent(inspect.getsource(dit.dit_layer))
        for old, new in edits:
            assert old in src, (name, old)
            src = src.replace(old, new)
        ns = dict(dit.dit_layer.__globals__)
        exec(compile(src, f"<mutant: {name}>", "exec"), ns)
        out[name] = ns["dit_layer"]
    return out


def _pins(layer_fn, rng, d):
    """Worst violation over the three cross-attention pins (0 = all hold)."""
    W, b = _ca_only_weights(rng, d)
    D = d.hidden
    x = rng.standard_normal((d.chunk, D)) * 1.5
    worst = 0.0
    # (1) one context token: softmax over one key is 1, so the branch is
    # gate * ((c W_v^T + b_v) W_o^T + b_o) for every row, whatever the query
    c1 = rng.standard_normal((1, d.ctx_dim))
    vrow = c1 @ W["dit.0.ca_wv"].T + W["dit.0.ca_bv"]
    want1 = np.tile(b[5] * (vrow @ W["dit.0.ca_wo"].T + W["dit.0.ca_bo"]), (d.chunk, 1))
    worst = max(worst, rel(_branch(layer_fn, W, x, c1, d), want1))
    # (2) zero query weights and bias: uniform attention, the mean V_c row
    ctx = rng.standard_normal((7, d.ctx_dim))
    W0 = DictW(W)
    W0["dit.0.ca_wq"] = np.zeros_like(W["dit.0.ca_wq"])
    W0["dit.0.ca_bq"] = np.zeros_like(W["dit.0.ca_bq"])
    vmean = (ctx @ W["dit.0.ca_wv"].T + W["dit.0.ca_bv"]).mean(0)
    want2 = np.tile(b[5] * (vmean @ W["dit.0.ca_wo"].T + W["dit.0.ca_bo"]), (d.chunk, 1))
    worst = max(worst, rel(_branch(layer_fn, W0, x, ctx, d), want2))
    # (3) the general branch against torch's SDPA on the same operands
    worst = max(worst, rel(_branch(layer_fn, W, x, ctx, d), _torch_ca_branch(W, b, x, ctx, d)))
    return worst


def test_dit_cross_attention_branch_closed_forms_and_sdpa():
    d = _dit_cfg().dit
    assert _pins(dit.dit_layer, np.random.default_rng(17), d) < 1e-12
    for name, fn in _ca_mutants().items():
        assert _pins(fn, np.random.default_rng(17), d) > 1e-6, f"planted mistake not caught: {name}"


def test_dit_velocity_depends_on_the_context():
    cfg = _dit_cfg()
    d = cfg.dit
    W = _weights(cfg, "dit.")
    rng = np.random.default_rng(19)
    a = rng.standard_normal((d.chunk, d.action_dim))
    ctx = rng.standard_normal((cfg.ctx_len, d.ctx_dim))
    ctx2 = ctx.copy()
    ctx2[3] += rng.standard_normal(d.ctx_dim)
    v1, v2 = dit.dit_velocity(a, 0.25, ctx, W, d), dit.dit_velocity(a, 0.25, ctx2, W, d)
    assert rel(v2, v1) > 1e-4
