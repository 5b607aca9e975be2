"""Exact-tie parity: the hardware E2M1 convert's tie rule and sign handling, enforced.

The inputs (tests/exact_inputs.py) make the float32 rotation exact and land elements exactly
on every E2M1 midpoint, next to them, on small negative values and on -0, for MXFP4 and NVFP4.
Parity is then demanded with no allowance: codes, scales and s_t bit-exact, flagged or not.
Ties must go to the even code and the sign bit must follow the input (round-to-nearest onto
E2M1: "Bridging the Gap Between Promise and Performance for Microscaling FP4 Quantization",
gist.science, German edition, Technische Zusammenfassung §2 "Theoretische Analyse der
Fehler"; the E2M1 codebook of "TORQ", gist.science, German edition, 1. Problemstellung).
"""
import numpy as np
import pytest
import torch

from microscaling_fp4_quantized_amd import binding as B
from exact_inputs import E4M3_TIES, build_input, check_tie_codes, mx_rows, nv_e4m3_tie_rows, nv_rows
from oracle import fp4_oracle as O
from parity import assert_quant_parity, compare_quant, dev_bf16, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load_library()


@pytest.mark.parametrize("block", (16, 64))
def test_mx_exact_ties(block):
    rows = mx_rows(block)
    bits, U = build_input(rows, block)
    say(f"case exact ties MXFP4 block {block}: X {bits.shape}")
    out = B.fp4_rotate_quantize(dev_bf16(bits), block, "mxfp4")
    torch.cuda.synchronize()
    res = compare_quant(out, bits, block, "mxfp4")
    assert_quant_parity(res, f"exact ties mx b{block}", exact=True)
    assert res["flagged"] > 50  # the ties are there and are flagged
    scale = np.ldexp(1.0, out[1].cpu().numpy().astype(np.int64) - 127)
    scale[out[1].cpu().numpy() == 0] = 0.0
    n = check_tie_codes(out[0].cpu().numpy(), U, scale, 32)
    say(f"  {n} elements exactly on an E2M1 midpoint")
    assert n > 50


@pytest.mark.parametrize("k", (-3, 10))
def test_nv_exact_ties(k):
    rows = nv_rows(k)
    bits, U = build_input(rows, 16)
    say(f"case exact ties NVFP4 block 16, s_t = 2^{k}: X {bits.shape}")
    out = B.fp4_rotate_quantize(dev_bf16(bits), 16, "nvfp4")
    torch.cuda.synchronize()
    res = compare_quant(out, bits, 16, "nvfp4")
    assert_quant_parity(res, f"exact ties nv s_t=2^{k}", exact=True)
    assert res["tensor_scale"] == 2.0 ** k
    assert res["flagged"] > 50
    d = O.e4m3_value(out[1].cpu().numpy())
    n = check_tie_codes(out[0].cpu().numpy(), U, d * 2.0 ** k, 16)
    say(f"  {n} elements exactly on an E2M1 midpoint")
    assert n > 50
    # the same with the tensor scale given instead of computed (one pass over X)
    given = torch.tensor([2.0 ** k], dtype=torch.float32, device="cuda")
    out2 = B.fp4_rotate_quantize(dev_bf16(bits), 16, "nvfp4", tensor_scale=given)
    torch.cuda.synchronize()
    assert torch.equal(out2[0], out[0]) and torch.equal(out2[1], out[1])


@pytest.mark.parametrize("k", (-12, 0, 9))
def test_nv_e4m3_scale_ties(k):
    # group maxima exactly on E4M3 rounding midpoints (and one bf16 step away): the group scale
    # code must be the even neighbour, as the oracle decides it exactly
    rows = nv_e4m3_tie_rows(k)
    bits, U = build_input(rows, 16)
    say(f"case E4M3 scale ties, s_t = 2^{k}: X {bits.shape}")
    for given in (None, torch.tensor([2.0 ** k], dtype=torch.float32, device="cuda")):
        out = B.fp4_rotate_quantize(dev_bf16(bits), 16, "nvfp4", tensor_scale=given)
        torch.cuda.synchronize()
        res = compare_quant(out, bits, 16, "nvfp4")
        assert_quant_parity(res, f"E4M3 ties s_t=2^{k}", exact=True)
        assert res["tensor_scale"] == 2.0 ** k
        sc = out[1].cpu().numpy().reshape(-1)
        amax = np.abs(U).reshape(-1, 16).max(axis=1)
        for m, want in E4M3_TIES:
            at = amax == 6 * m * 2.0 ** k
            assert at.sum() == 3 and np.all(sc[at] == want), (m, sc[at])


def test_negative_zero_block():
    # an all -0 block rotates to -0 at position 0 and +0 elsewhere; both formats keep those signs
    bits = np.full((2, 64), 0x8000, np.uint16)
    bits[1, :] = 0
    for fmt in ("mxfp4", "nvfp4"):
        say(f"case signed zeros {fmt}")
        out = B.fp4_rotate_quantize(dev_bf16(bits), 16, fmt)
        torch.cuda.synchronize()
        assert_quant_parity(compare_quant(out, bits, 16, fmt), f"signed zeros {fmt}", exact=True)
        y = O.rotate_fwht_f32(O.widen_bf16(bits), 16)
        codes = O.unpack_nibbles(out[0].cpu().numpy())
        assert np.array_equal(codes, np.signbit(y).astype(np.uint8) * 8)
