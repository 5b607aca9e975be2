"""GPU parity of fp4_rotate_quantize / fp4_quantize_weights against the oracle.

Codes, scales and the NVFP4 tensor scale must be bit-exact (near-boundary
elements are counted and reported). Sizes span several workgroups and ragged
tails; the stress workload runs at its full size (16384 x 8192) with sampled
rows checked against the oracle.
"""
import numpy as np
import pytest
import torch

from microscaling_fp4_quantized_amd import binding as B
from microscaling_fp4_quantized_amd import workloads as WL
from oracle import fp4_oracle as O
from parity import assert_quant_parity, compare_quant, dev_bf16, say

pytestmark = pytest.mark.gpu

FMTS = ("mxfp4", "nvfp4")
BLOCKS = (16, 32, 64, 128)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load_library()


def run(x_bits, block, fmt, ldx_pad=0, weights=False):
    M, K = x_bits.shape
    if ldx_pad:
        big = np.zeros((M, K + ldx_pad), dtype=np.uint16)
        big[:, :K] = x_bits
        big[:, K:] = 0x7F7F  # junk beyond K must be ignored
        xd = dev_bf16(big)[:, :K]
    else:
        xd = dev_bf16(x_bits)
    fn = B.fp4_quantize_weights if weights else B.fp4_rotate_quantize
    out = fn(xd, block, fmt)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("block", BLOCKS)
def test_tiny_workload(block, fmt):
    x = WL.draw_x(WL.WORKLOADS["tiny"])
    say(f"case tiny X {x.shape} block {block} {fmt}")
    assert_quant_parity(compare_quant(run(x, block, fmt), x, block, fmt), f"tiny b{block} {fmt}")
    w = WL.draw_w(WL.WORKLOADS["tiny"])
    assert_quant_parity(compare_quant(run(w, block, fmt, weights=True), w, block, fmt), f"tiny W b{block} {fmt}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("block,M,K,pad", [(32, 37, 384, 40), (128, 37, 384, 0), (64, 1, 64, 8),
                                           (16, 1000, 96, 0), (128, 3, 128, 64), (32, 257, 8192, 0)])
def test_ragged_and_strided(block, M, K, pad, fmt):
    x = WL.draw_normal_bf16((M, K), 3.0, seed=M + K + block)
    say(f"case ragged M {M} K {K} ldx {K + pad} block {block} {fmt}")
    assert_quant_parity(compare_quant(run(x, block, fmt, ldx_pad=pad), x, block, fmt), f"ragged {M}x{K}")


def edge_matrix():
    rng = np.random.default_rng(77)
    rows = []
    K = 256
    rows.append(np.zeros(K, np.float32))                        # all zero
    r = np.zeros(K, np.float32); r[5] = 3.0; rows.append(r)      # one spike
    rows.append(np.full(K, -2.5, np.float32))                    # constant
    for _ in range(20):                                          # small integers: exact ties after rotation
        rows.append(rng.integers(-8, 9, K).astype(np.float32))
    rows.append(rng.integers(-3, 4, K).astype(np.float32) * np.float32(2.0 ** -60))
    rows.append(rng.standard_normal(K).astype(np.float32) * np.float32(1e25))
    r = rng.standard_normal(K).astype(np.float32); r[::7] *= 1000; rows.append(r)
    x = WL.bf16_bits_from_f32(np.stack(rows))
    x[0, 1::2] = 0x8000  # negative zeros
    x[2, :8] = 0x0001    # bf16 subnormals
    return x


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("block", BLOCKS)
def test_edge_values(block, fmt):
    x = edge_matrix()
    say(f"case edge values {x.shape} block {block} {fmt}")
    assert_quant_parity(compare_quant(run(x, block, fmt), x, block, fmt), f"edge b{block} {fmt}")


@pytest.mark.parametrize("block", (16, 128))
def test_nv_zero_tensor_and_tiny_tensor(block):
    z = np.zeros((4, 128), np.uint16)
    z[1, 3] = 0x8000
    codes, scales, ts = run(z, block, "nvfp4")
    assert float(ts.item()) == 0.0
    assert int(scales.to(torch.int64).sum().item()) == 0
    assert_quant_parity(compare_quant((codes, scales, ts), z, block, "nvfp4"), "nv zero")
    t = WL.bf16_bits_from_f32(np.linspace(-1, 1, 4 * 128, dtype=np.float32).reshape(4, 128) * np.float32(2.0 ** -110))
    assert_quant_parity(compare_quant(run(t, block, "nvfp4"), t, block, "nvfp4"), "nv tiny tensor")


@pytest.mark.parametrize("name", ["stress_mx32", "stress_mx128", "stress_nv32", "stress_nv128"])
def test_stress_full_size_sampled(name):
    w = WL.WORKLOADS[name]
    x = WL.draw_x(w)
    say(f"case {name} X {x.shape} block {w.block} {w.fmt} (sampled rows)")
    out = run(x, w.block, w.fmt)
    rows = np.unique(np.concatenate([[0, 1, x.shape[0] - 1],
                                     np.random.default_rng(5).choice(x.shape[0], 200, replace=False)]))
    assert_quant_parity(compare_quant(out, x, w.block, w.fmt, rows=rows), name)


def test_outputs_stay_within_their_buffers():
    # guard bytes around codes/scales must stay untouched
    x = WL.draw_normal_bf16((33, 256), 1.0, seed=3)
    xd = dev_bf16(x)
    for fmt in FMTS:
        g = 32 if fmt == "mxfp4" else 16
        cbuf = torch.full((33 * 128 + 64,), 0xAB, dtype=torch.uint8, device="cuda")
        sbuf = torch.full((33 * 256 // g + 64,), 0xCD, dtype=torch.uint8, device="cuda")
        codes = cbuf[:33 * 128].view(33, 128)
        scales = sbuf[:33 * 256 // g].view(33, 256 // g)
        ts = torch.zeros(1, dtype=torch.float32, device="cuda") if fmt == "nvfp4" else None
        B.fp4_rotate_quantize(xd, 32, fmt, out=(codes, scales, ts))
        torch.cuda.synchronize()
        assert bool((cbuf[33 * 128:] == 0xAB).all()) and bool((sbuf[33 * 256 // g:] == 0xCD).all())
        assert_quant_parity(compare_quant((codes, scales, ts), x, 32, fmt), f"guard {fmt}")


def test_errors_raise():
    x = dev_bf16(WL.draw_normal_bf16((4, 64), 1.0, seed=9))
    with pytest.raises(B.Fp4Error):
        B.fp4_rotate_quantize(x, 8, "mxfp4")
    with pytest.raises(B.Fp4Error):
        B.fp4_rotate_quantize(x[:, 4:36], 32, "mxfp4")  # start 8 bytes past 16-byte alignment
    with pytest.raises(B.Fp4Error):
        B.fp4_rotate_quantize(x, 128, "mxfp4")  # K % block
