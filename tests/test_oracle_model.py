"""Pins of the oracle's composed model (block, backbone, ViT, merger, DiT,
Euler sampler, policy step) against invariants and exact special cases."""

import math

import numpy as np
import pytest

from oracle import dit, llm, ops, policy, vit
from oracle.io import Weights
from synth import small_config, make_weights, make_inputs
from synth.configs import SMALL_BLOCK, DiTShape, ViTShape


class DictW(dict):
    """Plain name -> float64 weights for hand-built cases."""


def block_weights(rng, shape, scale=None, zero=False):
    H, I = shape.hidden, shape.intermediate
    s = (lambda k: 1.0 / math.sqrt(k)) if scale is None else (lambda k: scale)
    mk = (lambda *sh: np.zeros(sh)) if zero else (lambda *sh: rng.standard_normal(sh) * s(sh[1]))
    return DictW({
        "l.attn_norm": rng.uniform(0.5, 1.5, H), "l.mlp_norm": rng.uniform(0.5, 1.5, H),
        "l.wq": mk(shape.q_dim, H), "l.wk": mk(shape.kv_dim, H), "l.wv": mk(shape.kv_dim, H),
        "l.wo": mk(H, shape.q_dim), "l.wg": mk(I, H), "l.wu": mk(I, H), "l.wd": mk(H, I),
    })


def qk_block_weights(rng, shape):
    W = block_weights(rng, shape)
    W["l.q_norm"] = rng.uniform(0.5, 1.5, shape.head_dim)
    W["l.k_norm"] = rng.uniform(0.5, 1.5, shape.head_dim)
    return W


@pytest.mark.parametrize("which, head", [("l.wq", 1), ("l.wk", 0)])
def test_block_qk_norm_removes_each_head_scale(rng, which, head):
    """QK-norm normalises every query / key head vector: scaling one head's
    rows of W_q (or W_k) leaves the block output unchanged up to the eps
    term, while without QK-norm the same scaling changes the attention."""
    import dataclasses
    qk = dataclasses.replace(SMALL_BLOCK, qk_norm=True)
    W = qk_block_weights(rng, qk)
    x = rng.standard_normal((11, qk.hidden))
    D = qk.head_dim
    Ws = DictW(W)
    Ws[which] = W[which].copy()
    Ws[which][head * D:(head + 1) * D] *= 7.0
    y, ys = llm.block(x, W, "l.", qk), llm.block(x, Ws, "l.", qk)
    assert np.max(np.abs(ys - y)) / np.max(np.abs(y)) < 1e-6
    y0, y0s = llm.block(x, W, "l.", SMALL_BLOCK), llm.block(x, Ws, "l.", SMALL_BLOCK)
    assert np.max(np.abs(y0s - y0)) / np.max(np.abs(y0)) > 1e-3


def test_block_qk_norm_unit_gains_give_unit_rms_heads(rng, monkeypatch):
    """With unit gains each head vector reaching RoPE has mean square
    ms / (ms + eps) of its pre-norm value (RMSNorm's closed form), and the
    gains multiply it per dimension."""
    import dataclasses
    qk = dataclasses.replace(SMALL_BLOCK, qk_norm=True)
    W = qk_block_weights(rng, qk)
    W["l.q_norm"] = np.ones(qk.head_dim)
    seen = {}
    real_rope = ops.rope

    def spy(t, pos, base):
        seen.setdefault("q", t)    # first call: the queries
        return real_rope(t, pos, base)

    monkeypatch.setattr(ops, "rope", spy)
    x = rng.standard_normal((6, qk.hidden))
    llm.block(x, W, "l.", qk)
    n = ops.rmsnorm(x, W["l.attn_norm"], qk.eps)
    q_raw = (n @ W["l.wq"].T).reshape(6, qk.n_q_heads, qk.head_dim)
    ms = np.mean(q_raw * q_raw, axis=-1)
    np.testing.assert_allclose(np.mean(seen["q"] ** 2, axis=-1), ms / (ms + qk.eps), rtol=1e-12)


def test_block_zero_weights_is_identity(rng):
    W = block_weights(rng, SMALL_BLOCK, zero=True)
    x = rng.standard_normal((9, SMALL_BLOCK.hidden))
    np.testing.assert_array_equal(llm.block(x, W, "l.", SMALL_BLOCK), x)


def test_block_is_causal(rng):
    W = block_weights(rng, SMALL_BLOCK)
    x = rng.standard_normal((12, SMALL_BLOCK.hidden))
    y = llm.block(x, W, "l.", SMALL_BLOCK)
    x2 = x.copy()
    x2[7] += rng.standard_normal(SMALL_BLOCK.hidden)
    y2 = llm.block(x2, W, "l.", SMALL_BLOCK)
    np.testing.assert_array_equal(y2[:7], y[:7])
    assert np.max(np.abs(y2[7:] - y[7:])) > 1e-3


def test_block_gqa_equals_mha_with_replicated_kv_rows(rng):
    W = block_weights(rng, SMALL_BLOCK)
    mha_shape = SMALL_BLOCK.__class__(**{**SMALL_BLOCK.__dict__, "n_kv_heads": SMALL_BLOCK.n_q_heads})
    D, g = SMALL_BLOCK.head_dim, SMALL_BLOCK.n_q_heads // SMALL_BLOCK.n_kv_heads
    Wm = DictW(W)
    for nm in ("l.wk", "l.wv"):
        heads = W[nm].reshape(SMALL_BLOCK.n_kv_heads, D, -1)
        Wm[nm] = np.repeat(heads, g, axis=0).reshape(mha_shape.kv_dim, -1)
    x = rng.standard_normal((10, SMALL_BLOCK.hidden))
    np.testing.assert_allclose(llm.block(x, W, "l.", SMALL_BLOCK), llm.block(x, Wm, "l.", mha_shape),
                               rtol=1e-12, atol=1e-12)


def test_block_rope_relative_positions(rng, monkeypatch):
    # Scores depend only on position differences: shifting every position by
    # the same offset leaves the block output unchanged (RoPE on Q *and* K).
    W = block_weights(rng, SMALL_BLOCK)
    x = rng.standard_normal((8, SMALL_BLOCK.hidden))
    np.testing.assert_allclose(llm.block(x, W, "l.", SMALL_BLOCK, pos0=0),
                               llm.block(x, W, "l.", SMALL_BLOCK, pos0=37), rtol=1e-10, atol=1e-10)
    # ... while removing the rotation from K alone changes it
    y = llm.block(x, W, "l.", SMALL_BLOCK)
    saved = ops.rope
    calls = []

    def rope_q_only(t, pos, base):
        calls.append(1)
        return saved(t, pos, base) if len(calls) == 1 else t
    monkeypatch.setattr(ops, "rope", rope_q_only)
    y_bad = llm.block(x, W, "l.", SMALL_BLOCK)
    assert np.max(np.abs(y_bad - y)) > 1e-3


def test_swiglu_gate_takes_silu_hand_case():
    # hidden 2, intermediate 1, one token, no attention contribution.
    shape = SMALL_BLOCK.__class__(hidden=2, n_q_heads=1, n_kv_heads=1, head_dim=2, intermediate=1,
                                  rope_base=1e4, eps=0.0)
    W = DictW({"l.attn_norm": np.ones(2), "l.mlp_norm": np.ones(2),
               "l.wq": np.zeros((2, 2)), "l.wk": np.zeros((2, 2)), "l.wv": np.zeros((2, 2)),
               "l.wo": np.zeros((2, 2)),
               "l.wg": np.array([[1.0, 0.0]]), "l.wu": np.array([[0.0, 1.0]]), "l.wd": np.array([[1.0], [0.0]])})
    x = np.array([[3.0, 4.0]])
    # rmsnorm: rms = sqrt((9+16)/2) -> n = [3, 4]/sqrt(12.5); gate = n0, up = n1
    n0, n1 = 3 / math.sqrt(12.5), 4 / math.sqrt(12.5)
    want = x + np.array([[n0 / (1 + math.exp(-n0)) * n1, 0.0]])
    np.testing.assert_allclose(llm.block(x, W, "l.", shape), want, rtol=1e-14)


def test_backbone_counts_and_final_norm(monkeypatch):
    cfg = small_config("backbone", "bf16", layers=3, seq=9)
    Wt = make_weights(cfg)
    W = Weights(Wt)
    calls = []
    real = ops.rmsnorm
    monkeypatch.setattr(ops, "rmsnorm", lambda *a: calls.append(1) or real(*a))
    x = np.random.default_rng(0).standard_normal((9, cfg.block.hidden))
    y = llm.backbone(x, W, cfg)
    # two pre-norms per layer (72 over 36 layers on the page) + the final norm
    assert len(calls) == 2 * 3 + 1
    g = W["llm.final_norm"]
    np.testing.assert_allclose(np.sqrt(np.mean((y / g) ** 2, axis=-1)), 1.0, rtol=1e-5)


# ---------------------------------------------------------------- ViT / merger

def test_patchify_order():
    v = ViTShape(image=28, patch=14, channels=3)
    img = np.arange(3 * 28 * 28, dtype=np.float64).reshape(3, 28, 28)
    P = vit.patchify(img, 14)
    assert P.shape == (4, 588)
    # patch (r=1, c=0) is row 2; element (ch=2, ky=3, kx=5) is at 2*196 + 3*14 + 5
    assert P[2, 2 * 196 + 3 * 14 + 5] == img[2, 14 + 3, 0 + 5]
    assert P[1, 0] == img[0, 0, 14]


def test_merge_groups_raster_order():
    grid, m, D = 4, 2, 3
    u = np.arange(grid * grid)[:, None] * 10 + np.arange(D)[None, :]
    g = vit.merge_groups(u.astype(float), grid, m)
    assert g.shape == (4, 12)
    # merged token (R=1, C=0) = patches (2,0), (2,1), (3,0), (3,1) = rows 8, 9, 12, 13
    np.testing.assert_array_equal(g[2].reshape(4, D)[:, 0], [80, 90, 120, 130])


def test_vit_zero_blocks_keep_embedding(rng):
    cfg = small_config("step", "bf16")
    v = cfg.vit
    Wt = Weights(make_weights(cfg))
    W = DictW({n: Wt[n] for n in make_weights(cfg).names() if n.startswith("vit.")})
    for l in range(v.layers):
        for nm in ("wo", "bo", "w2", "b2"):
            W[f"vit.{l}.{nm}"] = np.zeros_like(W[f"vit.{l}.{nm}"])
    img = rng.standard_normal((3, v.image, v.image))
    z = vit.vit(img, W, v)
    np.testing.assert_allclose(z, vit.patchify(img, v.patch) @ W["vit.pe_w"].T + W["vit.pe_b"] + W["vit.pos"],
                               rtol=1e-13)


# ---------------------------------------------------------------- DiT / Euler

def test_timestep_embedding_closed_form():
    d = DiTShape()
    e0 = dit.timestep_embedding(0.0, d)
    np.testing.assert_array_equal(e0, np.r_[np.ones(128), np.zeros(128)])
    e = dit.timestep_embedding(0.25, d)
    for i in (0, 1, 64, 127):
        w = 10000.0 ** (-i / 128)
        assert abs(e[i] - math.cos(250.0 * w)) < 1e-12
        assert abs(e[128 + i] - math.sin(250.0 * w)) < 1e-12


def test_euler_exact_cases(rng):
    x0 = rng.standard_normal((4, 3))
    c = rng.standard_normal((4, 3))
    for K in (1, 4, 10):
        # K fp64 additions of c/K: rounding at most ~K eps (|x0| + |c|) per element
        got = dit.euler_sample(x0, K, lambda x, t: c)
        assert np.all(np.abs(got - (x0 + c)) <= 2 * K * np.finfo(float).eps * (np.abs(x0) + np.abs(c)))
        a = 0.7
        np.testing.assert_allclose(dit.euler_sample(x0, K, lambda x, t: a * x), (1 + a / K) ** K * x0, rtol=1e-13)
        f = lambda t: np.sin(3 * t) + t * t
        want = x0 + sum(f(k / K) for k in range(K)) / K
        np.testing.assert_allclose(dit.euler_sample(x0, K, lambda x, t: f(t) * np.ones_like(x)), want, rtol=1e-13)
    ts = []
    dit.euler_sample(x0, 4, lambda x, t: ts.append(t) or 0 * x)
    assert ts == [0.0, 0.25, 0.5, 0.75]


def _dit_weights(cfg):
    Wt = make_weights(cfg)
    W = Weights(Wt)
    return DictW({n: W[n] for n in Wt.names()})


def test_dit_only_output_bias_gives_constant_velocity(rng):
    cfg = small_config("dit", "bf16")
    W = _dit_weights(cfg)
    for n in W:
        if n != "dit.out_b":
            W[n] = np.zeros_like(W[n])
    a0 = rng.standard_normal((cfg.dit.chunk, cfg.dit.action_dim))
    ctx = rng.standard_normal((cfg.ctx_len, cfg.dit.ctx_dim))
    v = dit.dit_velocity(a0, 0.3, ctx, W, cfg.dit)
    np.testing.assert_array_equal(v, np.broadcast_to(W["dit.out_b"], v.shape))
    np.testing.assert_allclose(dit.flow_sample(a0, ctx, W, cfg.dit, 4), a0 + W["dit.out_b"], rtol=1e-14)


def test_dit_zero_gates_skip_every_sublayer(rng):
    cfg = small_config("dit", "bf16")
    d = cfg.dit
    W = _dit_weights(cfg)
    D = d.hidden
    for l in range(d.layers):
        W[f"dit.{l}.ada_w"] = np.zeros_like(W[f"dit.{l}.ada_w"])
        b = W[f"dit.{l}.ada_b"].reshape(9, D).copy()
        b[[2, 5, 8]] = 0.0              # gates
        W[f"dit.{l}.ada_b"] = b.reshape(-1)
    a = rng.standard_normal((d.chunk, d.action_dim))
    ctx = rng.standard_normal((cfg.ctx_len, d.ctx_dim))
    x = ops.linear(a, W["dit.in_w"], W["dit.in_b"])
    sc = ops.silu(dit.time_condition(0.5, W, d))
    f = ops.linear(sc, W["dit.f_w"], W["dit.f_b"]).reshape(2, D)
    want = ops.linear(ops.layernorm(x, None, None, d.eps) * (1 + f[1]) + f[0], W["dit.out_w"], W["dit.out_b"])
    np.testing.assert_allclose(dit.dit_velocity(a, 0.5, ctx, W, d), want, rtol=1e-12, atol=1e-12)


def test_dit_permutation_equivariance(rng):
    cfg = small_config("dit", "bf16")
    W = _dit_weights(cfg)
    d = cfg.dit
    a = rng.standard_normal((d.chunk, d.action_dim))
    ctx = rng.standard_normal((cfg.ctx_len, d.ctx_dim))
    perm = rng.permutation(d.chunk)
    v = dit.dit_velocity(a, 0.25, ctx, W, d)
    np.testing.assert_allclose(dit.dit_velocity(a[perm], 0.25, ctx, W, d), v[perm], rtol=1e-11, atol=1e-11)
    # and invariance to the order of the context tokens
    cperm = rng.permutation(cfg.ctx_len)
    np.testing.assert_allclose(dit.dit_velocity(a, 0.25, ctx[cperm], W, d), v, rtol=1e-11, atol=1e-11)


# ---------------------------------------------------------------- policy step

def test_small_step_composition():
    cfg = small_config("step", "bf16")
    Wt, It = make_weights(cfg), make_inputs(cfg)
    out = policy.run_config(cfg, Wt, It)
    assert out["merged"].shape == (cfg.vit.n_merged, cfg.block.hidden)
    assert out["hidden"].shape == (cfg.seq, cfg.block.hidden)
    assert out["actions"].shape == (cfg.dit.chunk, cfg.dit.action_dim)
    W = Weights(Wt)
    np.testing.assert_allclose(out["ctx"], out["hidden"] @ W["proj.w"].T + W["proj.b"], rtol=1e-13)
    # the actions are the Euler sum of the recorded velocities
    from oracle.io import to_f64
    np.testing.assert_allclose(out["actions"], to_f64(It["noise"]) + out["velocities"].sum(0) / cfg.steps,
                               rtol=1e-12, atol=1e-12)


def test_dit_modulation_order_shift_scale_gate(rng):
    # With scale = -1 and shift = 0 in every sublayer, u = LN(x)(1 + scale) + shift
    # is zero, so each sublayer adds the same row to every token. Any other order
    # of the 9 vectors ([shift, scale, gate] x [SA, CA, MLP]) breaks that.
    cfg = small_config("dit", "bf16")
    d = cfg.dit
    W = _dit_weights(cfg)
    D = d.hidden
    W["dit.0.ada_w"] = np.zeros_like(W["dit.0.ada_w"])
    b = np.zeros((9, D))
    b[[1, 4, 7]] = -1.0
    b[[2, 5, 8]] = rng.uniform(0.5, 1.5, (3, D))
    W["dit.0.ada_b"] = b.reshape(-1)
    x = rng.standard_normal((d.chunk, D))
    ctx = rng.standard_normal((cfg.ctx_len, d.ctx_dim))
    sc = rng.standard_normal(D)
    dx = dit.dit_layer(x, sc, ctx, W, "dit.0.", d) - x
    np.testing.assert_allclose(dx, np.broadcast_to(dx[0], dx.shape), rtol=1e-12, atol=1e-12)
    assert np.max(np.abs(dx)) > 1e-2
