"""The W8A8 activation quantiser on the GPU (vla_quantize_rows, E4M3FN and
int8 codes) against the oracle's (oracle/fp8.py, oracle/int8.py), bit for bit: both take their decisions from
the same float32 values (bf16 inputs are exact in float32), so every code
and every scale must agree. Rows cover a zero row, codes in the E4M3FN
subnormal range, exact ties (a row maximum of 448 makes the multiplier 1),
saturation at the row maximum, and magnitudes from 1e-3 to 1e3."""

import numpy as np
import pytest

from oracle import fp8 as ofp8
from oracle import int8 as oint8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import gpu_util
    return gpu_util


def _bf16_bits(x32):
    """Round float32 to bfloat16 (nearest, ties to even) and return the bits."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _rows(rng, K):
    x = rng.standard_normal((40, K)).astype(np.float32)
    x *= np.logspace(-3, 3, 40, dtype=np.float32)[:, None]
    x[0] = 0.0                                                  # zero row
    x[1] = rng.uniform(-1e-5, 1e-5, K)                          # everything but the maximum lands in fp8 subnormals
    x[1, 7] = 1.0
    # ties: with max|row| = 448 the multiplier is exactly 1, so these values
    # are their own E4M3FN inputs: midpoints between neighbouring codes
    ties = np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 5.0 * 2.0 ** -10, 9.0, 11.0, -13.0, 208.0, 432.0],
                    dtype=np.float32)
    x[2] = 0.5
    x[2, :ties.size] = ties
    x[2, -1] = 448.0
    x[3] = -x[2]
    return x


@pytest.mark.parametrize("K", [264, 4096, 9728])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_quantize_rows_bitwise(gu, K, dtype, fmt):
    import torch
    from vla_robot_policy_amd import lib
    rng = np.random.default_rng(11)
    x = _rows(rng, K)
    if dtype == "bf16":
        bits = _bf16_bits(x)
        x32 = (bits.astype(np.uint32) << 16).view(np.float32)  # the exact values the GPU reads
        xd = torch.from_numpy(bits.view(np.int16)).to(gu.DEV)
        code = lib.VLA_BF16
    else:
        x32 = x
        xd = torch.from_numpy(x32).to(gu.DEV)
        code = lib.VLA_F32
    R = x32.shape[0]
    codes = torch.empty((R, K), dtype=torch.uint8, device=gu.DEV)
    scales = torch.empty(R, dtype=torch.float32, device=gu.DEV)
    cd = lib.VLA_FP8_E4M3 if fmt == "fp8" else lib.VLA_INT8
    lib.check(lib.vla_quantize_rows(xd, code, cd, R, K, K, codes, K, scales))
    torch.cuda.synchronize()
    want_c, want_s = (ofp8 if fmt == "fp8" else oint8).quantize_act_rows(x32)
    want_c = want_c.view(np.uint8)
    got_c, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    bad = np.argwhere(got_c != want_c)
    if bad.size:
        r, k = bad[0]
        gu.say(f"first mismatch row {r} col {k}: x {x32[r, k]!r} gpu 0x{got_c[r, k]:02x} oracle 0x{want_c[r, k]:02x} "
               f"({bad.shape[0]} of {got_c.size})")
    assert bad.size == 0
    assert np.array_equal(got_s, want_s)
