"""Pins of the oracle's operators against closed forms, invariants and library
routines (torch CPU in float64, scipy, math) — none of them re-types the
oracle's own code."""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import ops


def t64(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))


# ---------------------------------------------------------------- RMSNorm / LN

def test_rmsnorm_matches_torch(rng):
    x = rng.standard_normal((7, 33)) * 3 + 0.5
    g = rng.uniform(0.5, 1.5, 33)
    ref = F.rms_norm(t64(x), (33,), weight=t64(g), eps=1e-6).numpy()
    np.testing.assert_allclose(ops.rmsnorm(x, g, 1e-6), ref, rtol=1e-13, atol=1e-13)


def test_rmsnorm_closed_forms(rng):
    x = rng.standard_normal((5, 64))
    eps = 0.25
    y = ops.rmsnorm(x, np.ones(64), eps)
    ms = np.mean(x * x, axis=-1)
    # rms of the output is sqrt(ms / (ms + eps)) when the gain is 1
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), np.sqrt(ms / (ms + eps)), rtol=1e-13)
    # scale invariance as eps -> 0
    np.testing.assert_allclose(ops.rmsnorm(7.0 * x, np.ones(64), 0.0), ops.rmsnorm(x, np.ones(64), 0.0), rtol=1e-13)
    # the gain multiplies after normalising (not before the statistics)
    g = np.full(64, 3.0)
    np.testing.assert_allclose(ops.rmsnorm(x, g, 1e-6), 3.0 * ops.rmsnorm(x, np.ones(64), 1e-6), rtol=1e-13)


def test_layernorm_matches_torch_and_moments(rng):
    x = rng.standard_normal((6, 40)) * 2 + 4.0
    g, b = rng.uniform(0.5, 1.5, 40), rng.standard_normal(40)
    ref = F.layer_norm(t64(x), (40,), t64(g), t64(b), eps=1e-6).numpy()
    np.testing.assert_allclose(ops.layernorm(x, g, b, 1e-6), ref, rtol=1e-12, atol=1e-12)
    eps = 0.5
    y = ops.layernorm(x, None, None, eps)
    var = np.var(x, axis=-1)
    np.testing.assert_allclose(np.mean(y, axis=-1), 0.0, atol=1e-13)
    np.testing.assert_allclose(np.var(y, axis=-1), var / (var + eps), rtol=1e-12)


# ---------------------------------------------------------------- RoPE

def test_rope_half_split_hand_case():
    # D = 4: theta_0 = 1, theta_1 = base^(-1/2). Element 0 pairs with element 2.
    base, p = 100.0, 3
    x = np.zeros((4, 1, 4))
    x[p, 0, 0] = 1.0
    y = ops.rope(x, np.arange(4), base)
    np.testing.assert_allclose(y[p, 0], [math.cos(p), 0.0, math.sin(p), 0.0], atol=1e-15)
    x = np.zeros((4, 1, 4))
    x[p, 0, 1] = 1.0
    th = base ** -0.5
    y = ops.rope(x, np.arange(4), base)
    np.testing.assert_allclose(y[p, 0], [0.0, math.cos(p * th), 0.0, math.sin(p * th)], atol=1e-15)


def test_rope_invariants(rng):
    S, nh, D, base = 9, 3, 16, 1e4
    x = rng.standard_normal((S, nh, D))
    y = ops.rope(x, np.arange(S), base)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    np.testing.assert_allclose(y[0], x[0], atol=0)                        # R_0 = I
    # <R_m q, R_n k> = <R_{m-n} q, k>
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    for m, n in [(5, 2), (7, 7), (3, 8)]:
        lhs = ops.rope(q[None, None], [m], base)[0, 0] @ ops.rope(k[None, None], [n], base)[0, 0]
        rhs = ops.rope(q[None, None], [m - n], base)[0, 0] @ k
        assert abs(lhs - rhs) < 1e-12


# ---------------------------------------------------------------- attention

def _sdpa(q, k, v, causal):
    # torch CPU float64 SDPA, with KV heads expanded to the query heads
    group = q.shape[1] // k.shape[1]
    kk = np.repeat(k, group, axis=1)
    vv = np.repeat(v, group, axis=1)
    o = F.scaled_dot_product_attention(t64(q).transpose(0, 1), t64(kk).transpose(0, 1),
                                       t64(vv).transpose(0, 1), is_causal=causal)
    return o.transpose(0, 1).numpy()


@pytest.mark.parametrize("causal", [True, False])
def test_attention_matches_torch_sdpa(rng, causal):
    q = rng.standard_normal((11, 8, 16))
    k = rng.standard_normal((11, 2, 16))
    v = rng.standard_normal((11, 2, 12))
    np.testing.assert_allclose(ops.attention(q, k, v, causal), _sdpa(q, k, v, causal), rtol=1e-12, atol=1e-12)


def test_attention_cross_lengths_match_torch(rng):
    q = rng.standard_normal((5, 4, 8))
    k = rng.standard_normal((13, 4, 8))
    v = rng.standard_normal((13, 4, 8))
    np.testing.assert_allclose(ops.attention(q, k, v, False), _sdpa(q, k, v, False), rtol=1e-12, atol=1e-12)


def test_attention_brute_force_loops(rng):
    # explicit scalar loops with math.exp on a tiny case
    S, Hq, Hkv, D = 4, 4, 2, 3
    q, k, v = rng.standard_normal((S, Hq, D)), rng.standard_normal((S, Hkv, D)), rng.standard_normal((S, Hkv, D))
    out = ops.attention(q, k, v, True)
    for h in range(Hq):
        g = h // 2
        for i in range(S):
            w = [math.exp(sum(q[i, h, d] * k[j, g, d] for d in range(D)) / math.sqrt(D)) for j in range(i + 1)]
            z = sum(w)
            for d in range(D):
                assert abs(out[i, h, d] - sum(w[j] * v[j, g, d] for j in range(i + 1)) / z) < 1e-12


def test_gqa_equals_mha_with_replicated_kv(rng):
    q = rng.standard_normal((10, 8, 16))
    k, v = rng.standard_normal((10, 2, 16)), rng.standard_normal((10, 2, 16))
    mha = ops.attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), True)
    np.testing.assert_allclose(ops.attention(q, k, v, True), mha, rtol=1e-14, atol=1e-14)
    # the mapping is consecutive (head h reads kv head h // 4), not modular
    wrong = ops.attention(q, np.tile(k, (1, 4, 1)), np.tile(v, (1, 4, 1)), True)
    assert np.max(np.abs(wrong - mha)) > 1e-3


def test_attention_special_cases(rng):
    S, D = 6, 8
    q = rng.standard_normal((S, 1, D))
    k = np.tile(rng.standard_normal((1, 1, D)), (S, 1, 1))      # all keys equal
    v = rng.standard_normal((S, 1, D))
    out = ops.attention(q, k, v, True)
    for i in range(S):
        np.testing.assert_allclose(out[i, 0], v[: i + 1, 0].mean(axis=0), rtol=1e-13)
    np.testing.assert_allclose(ops.attention(q, rng.standard_normal((S, 1, D)), v, True)[0, 0], v[0, 0], rtol=1e-14)


# ---------------------------------------------------------------- activations / linear

def test_activations_match_library(rng):
    z = rng.standard_normal(200) * 4
    np.testing.assert_allclose(ops.silu(z), F.silu(t64(z)).numpy(), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(ops.gelu(z), F.gelu(t64(z), approximate="none").numpy(), rtol=1e-13, atol=1e-15)
    for zi in z[:20]:
        assert abs(ops.gelu(np.array([zi]))[0] - 0.5 * zi * (1 + math.erf(zi / math.sqrt(2)))) < 1e-14
    assert ops.silu(np.array([0.0]))[0] == 0.0


def test_linear_convention(rng):
    x, w, b = rng.standard_normal((3, 5)), rng.standard_normal((4, 5)), rng.standard_normal(4)
    y = ops.linear(x, w, b)
    for i in range(3):
        for n in range(4):
            assert abs(y[i, n] - (sum(x[i, k] * w[n, k] for k in range(5)) + b[n])) < 1e-13
