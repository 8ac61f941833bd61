"""Packed weights (vla_pack_weights, VLA_BLOCK_PACKED) on the GPU.

The packed layout is checked byte for byte against its definition written
out here with numpy (blocks of 16 rows x 32 k, ordered [row block][k block],
lane l holding 8 consecutive k of row l % 16 from k 8 (l / 16), zeros
beyond N and K). A block and a backbone on packed weights must give the
same bits as on the row-major weights (the same products in the same
order), and stay within the oracle's bar."""

import dataclasses

import numpy as np
import pytest

from oracle import llm as ollm
from oracle.io import Weights, to_f64
from synth import make_inputs, make_weights, small_config

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import gpu_util
    return gpu_util


def packed_layout(w: np.ndarray, K: int) -> np.ndarray:
    """The packed copy of w[:, :K] (one element per entry, any dtype)."""
    N = w.shape[0]
    NB, KB = -(-N // 16), -(-K // 32)
    pad = np.zeros((NB * 16, KB * 32), dtype=w.dtype)
    pad[:N, :K] = w[:, :K]
    out = np.zeros((NB, KB, 64, 8), dtype=w.dtype)
    for l in range(64):
        r, k0 = l % 16, 8 * (l // 16)
        for kb in range(KB):
            out[:, kb, l, :] = pad[r::16, kb * 32 + k0: kb * 32 + k0 + 8]
    return out.reshape(-1)


@pytest.mark.parametrize("wdtype", ["bf16", "fp8", "int8"])
@pytest.mark.parametrize("N,K,ldw", [(37, 70, 80), (16, 32, 32), (1, 1, 8), (130, 688, 688)])
def test_pack_layout(gu, wdtype, N, K, ldw):
    import torch
    from vla_robot_policy_amd import lib
    rng = np.random.default_rng(N * 1000 + K)
    dt = np.uint16 if wdtype == "bf16" else np.uint8
    w = rng.integers(1, np.iinfo(dt).max, size=(N, ldw), dtype=dt)
    code = lib.DTYPE_CODE[wdtype]
    nbytes = lib.vla_packed_bytes(code, N, K)
    src = torch.from_numpy(w.view(np.int16) if dt == np.uint16 else w).cuda()
    out = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device="cuda")
    lib.check(lib.vla_pack_weights(code, src, N, K, ldw, out))
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(dt)
    want = packed_layout(w, K)
    assert got.shape == want.shape
    np.testing.assert_array_equal(got, want)


def _pair(gu, cfg, W):
    return gu.DeviceWeights(cfg, W), gu.DeviceWeights(cfg, W, packed=True)


@pytest.mark.parametrize("wdtype", ["bf16", "fp8", "int8"])
@pytest.mark.parametrize("seq", [1, 37, 104, 130, 200, 400])
def test_block_packed(gu, wdtype, seq):
    cfg = small_config("block", wdtype, seq=seq)
    W, I = make_weights(cfg), make_inputs(cfg)
    plain, packed = _pair(gu, cfg, W)
    x = gu.upload_input(I["x"])
    got = gu.run_block(cfg, packed, x, seq)
    ref = gu.run_block(cfg, plain, x, seq)
    want = ollm.block(to_f64(I["x"]), Weights(W), "llm.0.", cfg.block)
    gu.relerr(got, want, gu.TOL[wdtype], f"packed block {wdtype} seq {seq}")
    np.testing.assert_array_equal(got, ref)


def test_block_packed_qk_norm(gu):
    from synth.configs import SMALL_BLOCK
    cfg = small_config("block", "bf16", seq=130, block=dataclasses.replace(SMALL_BLOCK, qk_norm=True))
    W, I = make_weights(cfg), make_inputs(cfg)
    plain, packed = _pair(gu, cfg, W)
    x = gu.upload_input(I["x"])
    got = gu.run_block(cfg, packed, x, 130)
    want = ollm.block(to_f64(I["x"]), Weights(W), "llm.0.", cfg.block)
    gu.relerr(got, want, gu.TOL["bf16"], "packed block qk-norm bf16 seq 130")
    np.testing.assert_array_equal(got, gu.run_block(cfg, plain, x, 130))


@pytest.mark.parametrize("wdtype", ["bf16", "fp8"])
def test_backbone_packed(gu, wdtype):
    cfg = small_config("backbone", wdtype, seq=104)
    W, I = make_weights(cfg), make_inputs(cfg)
    plain, packed = _pair(gu, cfg, W)
    e = gu.upload_input(I["x"])
    got = gu.run_backbone(cfg, packed, e, cfg.seq)
    np.testing.assert_array_equal(got, gu.run_backbone(cfg, plain, e, cfg.seq))


def test_vit_packed(gu):
    """The vision encoder with its layers' four Linears packed: the same bits
    as with row-major weights, and within the bf16 bar of the oracle."""
    import torch
    from oracle import vit as ovit
    from vla_robot_policy_amd import lib
    cfg = small_config("step", "bf16")
    v = cfg.vit
    W, I = make_weights(cfg), make_inputs(cfg)
    outs = []
    for dw in _pair(gu, cfg, W):
        V = dw.build_vit()
        toks = torch.empty((v.n_merged, v.out_dim), dtype=torch.float32, device=gu.DEV)
        z = torch.empty((v.n_patches, v.hidden), dtype=torch.float32, device=gu.DEV)
        need = lib.vla_vit_workspace_bytes(V, 1)
        ws = gu.workspace(need)
        lib.check(lib.vla_vit_encode(V, gu.upload_input(I["image"]), 1, toks, z, ws, need))
        torch.cuda.synchronize()
        outs.append((z.cpu().numpy(), toks.cpu().numpy()))
    (z0, t0), (z1, t1) = outs
    zr = ovit.vit(to_f64(I["image"])[0], Weights(W), v)
    gu.relerr(z1, zr, gu.TOL["bf16"], "packed vit encoder")
    gu.relerr(t1, ovit.merger(zr, Weights(W), v), gu.TOL["bf16"], "packed vit merged")
    np.testing.assert_array_equal(z1, z0)
    np.testing.assert_array_equal(t1, t0)
