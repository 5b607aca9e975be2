"""GPU parity of the quantizer variants (fp4_rotate_quantize_ex / fp4_quantize_weights_ex):
the OCP floor and overflow-aware MXFP4 scale rules, data-free scale fitting (both formats) and
the randomized block Hadamard (sign vector), against the oracle on the same seeded inputs.

Both sides compute the rotation in the same float32 order and take every scale decision in
the same precision, so codes and scales must match bit for bit (no near-boundary allowance).
"""
import numpy as np
import pytest
import torch

from microscaling_fp4_quantized_amd import binding as B
from microscaling_fp4_quantized_amd import workloads as WL
from oracle import fp4_oracle as O
from parity import (GEMM_REL_FRO_TOL, assert_quant_parity, compare_quant, dev_bf16, gemm_reference, host, rel_fro,
                    say, tensor_amax)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load_library()


def dev_signs(s):
    return torch.from_numpy(np.ascontiguousarray(s, dtype=np.int8)).cuda()


MX_RULES = ("ocp_floor", "oas", "fit")


@pytest.mark.parametrize("rule", MX_RULES)
@pytest.mark.parametrize("block", [32, 64, 128])
def test_mx_rules_tiny_and_ragged(rule, block):
    # the tiny workload (outlier channels) plus a ragged row count and a strided input
    w = WL.WORKLOADS["tiny"]
    for x in (WL.draw_x(w), WL.draw_normal_bf16((37, 384), 3.0, seed=block)):
        say(f"case MX rule {rule} b{block} X {x.shape}")
        q = B.fp4_rotate_quantize(dev_bf16(x), block, "mxfp4", rule=rule)
        torch.cuda.synchronize()
        assert_quant_parity(compare_quant(q, x, block, "mxfp4", rule=rule), f"mx {rule} b{block}", exact=True)
    xs = WL.draw_normal_bf16((20, 640), 1.0, seed=7)
    wide = torch.zeros((20, 648), dtype=torch.bfloat16, device="cuda")
    wide[:, :640] = dev_bf16(xs)
    q = B.fp4_rotate_quantize(wide[:, :640], block, "mxfp4", rule=rule)
    torch.cuda.synchronize()
    assert_quant_parity(compare_quant(q, xs, block, "mxfp4", rule=rule), f"mx {rule} strided", exact=True)


@pytest.mark.parametrize("rule", MX_RULES)
def test_mx_rules_stress_sampled(rule):
    w = WL.WORKLOADS["stress_mx32"]
    x = WL.draw_x(w)
    say(f"case MX rule {rule} stress {x.shape} (sampled rows)")
    q = B.fp4_rotate_quantize(dev_bf16(x), w.block, "mxfp4", rule=rule)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, w.M - 1], np.random.default_rng(5).choice(w.M, 24, replace=False)]))
    assert_quant_parity(compare_quant(q, x, w.block, "mxfp4", rows=rows, rule=rule), f"mx {rule} stress", exact=True)


def test_mx_scale_edges_all_rules():
    # group maxima at and around the rule thresholds, zeros, tiny and huge magnitudes
    r = np.random.default_rng(8)
    K = 256
    base = r.standard_normal((24, K)).astype(np.float32) * 0.1
    peaks = np.array([3.0, 3.5, 3.25, 4.0, 6.0, 7.0, 3.5000002, 3.4999998, 2.0**-130, 1e-30, 2.0**90, 0.0],
                     np.float32)
    for i, p in enumerate(peaks):
        base[2 * i, 0] = p * 32 ** 0.5  # chunk 0 of the row: after the block-32 rotation the peak spreads
        base[2 * i + 1, :32] = p
    base[5] = 0.0
    x = WL.bf16_bits_from_f32(base)
    for rule in ("standard",) + MX_RULES:
        for block in (32, 128):
            q = B.fp4_rotate_quantize(dev_bf16(x), block, "mxfp4", rule=rule)
            torch.cuda.synchronize()
            assert_quant_parity(compare_quant(q, x, block, "mxfp4", rule=rule), f"edges {rule} b{block}", exact=True)


@pytest.mark.parametrize("block", [16, 32, 128])
def test_nv_fit(block):
    w = WL.WORKLOADS["tiny"]
    for x in (WL.draw_x(w), WL.draw_normal_bf16((29, 512), 0.05, seed=block + 1)):
        say(f"case NV fit b{block} X {x.shape}")
        q = B.fp4_rotate_quantize(dev_bf16(x), block, "nvfp4", rule="fit")
        torch.cuda.synchronize()
        assert_quant_parity(compare_quant(q, x, block, "nvfp4", rule="fit"), f"nv fit b{block}", exact=True)


def test_nv_fit_stress_sampled():
    w = WL.WORKLOADS["stress_nv32"]
    x = WL.draw_x(w)
    q = B.fp4_rotate_quantize(dev_bf16(x), w.block, "nvfp4", rule="fit")
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, w.M - 1], np.random.default_rng(6).choice(w.M, 16, replace=False)]))
    amax = tensor_amax(x, w.block)
    assert_quant_parity(compare_quant(q, x, w.block, "nvfp4", rows=rows, t_amax=amax, rule="fit"), "nv fit stress",
                        exact=True)


@pytest.mark.parametrize("fmt,block,rule", [("mxfp4", 32, "standard"), ("mxfp4", 128, "standard"),
                                            ("mxfp4", 64, "fit"), ("mxfp4", 32, "oas"), ("nvfp4", 16, "standard"),
                                            ("nvfp4", 32, "fit")])
def test_random_signs(fmt, block, rule):
    x = WL.draw_normal_bf16((33, 768), 1.0, seed=block)
    s = WL.draw_signs(768, block)
    say(f"case signs {fmt} b{block} {rule}")
    q = B.fp4_rotate_quantize(dev_bf16(x), block, fmt, rule=rule, signs=dev_signs(s))
    torch.cuda.synchronize()
    assert_quant_parity(compare_quant(q, x, block, fmt, rule=rule, signs=s), f"signs {fmt} b{block} {rule}",
                        exact=True)
    # strided input: the sign of channel k follows the column, not the flat chunk index
    wide = torch.zeros((33, 776), dtype=torch.bfloat16, device="cuda")
    wide[:, :768] = dev_bf16(x)
    q = B.fp4_rotate_quantize(wide[:, :768], block, fmt, rule=rule, signs=dev_signs(s))
    torch.cuda.synchronize()
    assert_quant_parity(compare_quant(q, x, block, fmt, rule=rule, signs=s), "signs strided", exact=True)


@pytest.mark.parametrize("fmt,block", [("mxfp4", 32), ("nvfp4", 16)])
def test_randomized_hadamard_linear_end_to_end(fmt, block):
    # X online and W offline rotated with the same signs, W scale-fitted: the product still
    # approximates X W^T, and equals the oracle's product of the same quantized operands
    w = WL.WORKLOADS["tiny"]
    x, wt = WL.draw_x(w), WL.draw_w(w)
    s = WL.draw_signs(w.K, 11)
    xq = B.fp4_rotate_quantize(dev_bf16(x), block, fmt, signs=dev_signs(s))
    wq = B.fp4_quantize_weights(dev_bf16(wt), block, fmt, rule="fit", signs=dev_signs(s))
    torch.cuda.synchronize()
    assert_quant_parity(compare_quant(wq, wt, block, fmt, rule="fit", signs=s), "W fit+signs", exact=True)
    y = B.fp4_linear(xq[0], xq[1], wq[0], wq[1], fmt, x_ts=xq[2], w_ts=wq[2])
    ref = gemm_reference(x, wt, block, fmt, np.arange(w.M), np.arange(w.N), w_rule="fit", signs=s)
    r = rel_fro(host(y), ref)
    say(f"randomized Hadamard linear {fmt}: rel fro {r:.3e}")
    assert r <= GEMM_REL_FRO_TOL
    exact = O.widen_bf16(x).astype(np.float64) @ O.widen_bf16(wt).astype(np.float64).T
    assert rel_fro(ref, exact) < 0.25  # still a 4-bit approximation of X W^T


def test_ex_standard_equals_plain():
    x = WL.draw_normal_bf16((40, 512), 1.0, seed=3)
    for fmt, block in (("mxfp4", 32), ("nvfp4", 16)):
        a = B.fp4_rotate_quantize(dev_bf16(x), block, fmt)
        b = B.fp4_rotate_quantize(dev_bf16(x), block, fmt, rule="standard")
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
        if fmt == "nvfp4":
            assert torch.equal(a[2], b[2])


def test_ex_errors_raise():
    x = dev_bf16(WL.draw_normal_bf16((4, 64), 1.0, seed=1))
    with pytest.raises(B.Fp4Error):
        B.fp4_rotate_quantize(x, 32, "nvfp4", rule="oas")
    with pytest.raises(ValueError):
        B.fp4_rotate_quantize(x, 32, "mxfp4", signs=torch.ones(63, dtype=torch.int8, device="cuda"))


@pytest.mark.parametrize("block", [16, 32])
@pytest.mark.parametrize("rule", ["standard", "fit"])
def test_nv_given_tensor_scale(block, rule):
    # s_t supplied by the caller: the computed one, 1/8 of it (heavy clipping) and 3x it
    w = WL.WORKLOADS["tiny"]
    for x in (WL.draw_x(w), WL.draw_normal_bf16((45, 640), 0.3, seed=block)):
        s_dyn = O.rotate_quantize(x, block, "nvfp4")[2]
        for factor in (1.0, 0.125, 3.0):
            st = np.float32(s_dyn * np.float32(factor))
            ts = torch.tensor([float(st)], dtype=torch.float32, device="cuda")
            say(f"case NV given s_t x{factor} b{block} {rule} X {x.shape}")
            q = B.fp4_rotate_quantize(dev_bf16(x), block, "nvfp4", rule=rule, tensor_scale=ts)
            torch.cuda.synchronize()
            assert q[2].data_ptr() == ts.data_ptr() and float(ts.item()) == float(st)  # read, not written
            assert_quant_parity(compare_quant(q, x, block, "nvfp4", rule=rule, tensor_scale=st),
                                f"nv given x{factor}", exact=True)


def test_nv_given_tensor_scale_stress_sampled():
    w = WL.WORKLOADS["stress_nv32"]
    x = WL.draw_x(w)
    st = np.float32(tensor_amax(x, w.block) / np.float32(2688.0) / np.float32(4.0))
    ts = torch.tensor([float(st)], dtype=torch.float32, device="cuda")
    q = B.fp4_rotate_quantize(dev_bf16(x), w.block, "nvfp4", tensor_scale=ts)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, w.M - 1], np.random.default_rng(9).choice(w.M, 16, replace=False)]))
    assert_quant_parity(compare_quant(q, x, w.block, "nvfp4", rows=rows, tensor_scale=st), "nv given stress",
                        exact=True)


def test_binding_refuses_mismatched_buffers():
    # the kernels trust the sizes that the pointers imply; the binding refuses a mismatch before any launch
    x = dev_bf16(WL.draw_normal_bf16((8, 256), 1.0, seed=2))
    w = dev_bf16(WL.draw_normal_bf16((64, 256), 0.02, seed=3))
    xq, xs, _ = B.fp4_rotate_quantize(x, 32, "mxfp4")
    wq, ws, _ = B.fp4_quantize_weights(w, 32, "mxfp4")
    bad_linear = [
        dict(xs=xs[:, :4].contiguous()),                       # Xs too narrow
        dict(ws=ws[:32].contiguous()),                         # Ws too short
        dict(wq=wq[:, :64].contiguous()),                      # K disagrees
        dict(out=torch.empty((8, 63), device="cuda")),         # Y too small
        dict(out=torch.empty((8, 64), device="cuda", dtype=torch.bfloat16)),  # Y of the wrong dtype
        dict(x_ts=torch.ones(1, device="cuda")),               # MXFP4 has no tensor scale
        dict(xs=xs.cpu()),                                     # host memory
    ]
    for bad in bad_linear:
        args = dict(xq=xq, xs=xs, wq=wq, ws=ws)
        kw = {k: v for k, v in bad.items() if k not in args}
        args.update({k: v for k, v in bad.items() if k in args})
        with pytest.raises(ValueError):
            B.fp4_linear(args["xq"], args["xs"], args["wq"], args["ws"], "mxfp4", **kw)
    nq, ns, nts = B.fp4_rotate_quantize(x, 16, "nvfp4")
    mq, ms, mts = B.fp4_quantize_weights(w, 16, "nvfp4")
    with pytest.raises(ValueError):
        B.fp4_linear(nq, ns, mq, ms, "nvfp4", x_ts=nts)                       # w_ts missing
    with pytest.raises(ValueError):
        B.fp4_linear(nq, ns, mq, ms[:, :8].contiguous(), "nvfp4", x_ts=nts, w_ts=mts)
    with pytest.raises(ValueError):
        B.fp4_rotate_quantize(x, 32, "mxfp4", out=(xq, xs[:, :7].contiguous(), None))
    with pytest.raises(ValueError):
        B.fp4_rotate_quantize(x, 32, "mxfp4", out=(xq[:4].contiguous(), xs, None))
    with pytest.raises(ValueError):
        B.fp4_rotate_quantize(x, 16, "nvfp4", out=(nq, ns, None))              # NVFP4 needs its scale word
    with pytest.raises(ValueError):
        B.fp4_rotate_quantize_linear(x, wq, ws[:, :4].contiguous(), 32)
    with pytest.raises(ValueError):
        B.fp4_rotate_quantize_linear(x, wq, ws, 32, out=torch.empty((8, 32), device="cuda"))
    # the same buffers, well formed, still run and agree with the two-call path
    y = B.fp4_linear(xq, xs, wq, ws, "mxfp4", out=torch.empty((8, 64), device="cuda"))
    assert torch.equal(y, B.fp4_linear(xq, xs, wq, ws, "mxfp4"))
