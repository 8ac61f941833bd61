"""vla_block_forward_static (scratch in the library's static device array,
no allocation) against vla_block_forward (the caller's workspace) through
the C ABI: two calls in a row on each block shape, the second with a
smaller input, must give the workspace entry point's results bit for bit
(same kernels, same tiles, same arithmetic), and both meet the oracle's bar."""

import numpy as np
import pytest

from oracle import llm as ollm
from oracle.io import Weights, to_f64
from synth import make_inputs, make_weights, small_config
from synth.configs import LLM

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import gpu_util
    return gpu_util


@pytest.mark.parametrize("wdtype, block, seqs", [("bf16", None, (130, 37)), ("f32", None, (64, 1)),
                                                  ("fp8", None, (45, 9)), ("bf16", LLM, (104, 40))],
                         ids=["bf16_small", "f32_small", "fp8_small", "bf16_2560"])
def test_static_block_matches_workspace_block(gu, wdtype, block, seqs):
    import torch
    from vla_robot_policy_amd import lib
    kw = {"block": block} if block is not None else {}
    cfg = small_config("block", wdtype, seq=seqs[0], **kw)
    W, I = make_weights(cfg), make_inputs(cfg)
    dw = gu.DeviceWeights(cfg, W)
    bb = dw.build_backbone()
    x_all = gu.upload_input(I["x"])
    for seq in seqs:                    # the second call is smaller than the first
        x = x_all[:seq].contiguous()
        want = gu.run_block(cfg, dw, x, seq)
        out = gu.act_empty(cfg, (seq, cfg.block.hidden))
        lib.check(lib.vla_block_forward_static(dw.block_cfg, bb.layers[0], x, out, seq))
        torch.cuda.synchronize()
        got = gu.to_host(out, gu.act_dtype(cfg))
        gu.say(f"static block {wdtype} hidden {cfg.block.hidden} seq {seq}: bitwise equal {np.array_equal(got, want)}")
        assert np.array_equal(got, want)
        ref = ollm.block(to_f64(I["x"])[:seq], Weights(W), "llm.0.", cfg.block)
        gu.relerr(got, ref, gu.TOL[wdtype], f"static block {wdtype} seq {seq}")
