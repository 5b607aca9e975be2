"""Seeded sweep over random shapes and options: GPU against the oracle, element by element.

Small shapes the oracle checks in full, drawn so that every kernel route is taken: row counts
that leave ragged workgroups, K from 32 up, all Hadamard blocks, both formats, every scale
rule, random signs, padded leading dimensions and given tensor scales for the quantizer;
general, large-tile, decode and NVFP4 routes for the product.
"""
import numpy as np
import pytest
import torch

from microscaling_fp4_quantized_amd import binding as B
from microscaling_fp4_quantized_amd import workloads as WL
from oracle import fp4_oracle as O
from parity import GEMM_REL_FRO_TOL, assert_quant_parity, compare_quant, dev_bf16, gemm_reference, host, rel_fro, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load_library()


def _quant_cases(n, seed):
    r = np.random.default_rng(seed)
    out = []
    for i in range(n):
        fmt = ["mxfp4", "nvfp4"][i % 2]
        block = int(r.choice([16, 32, 64, 128]))
        K = int(block * r.integers(1, 6)) if block >= 32 else int(32 * r.integers(1, 12))
        K = max(K, 32)
        M = int(r.integers(1, 90))
        pad = int(8 * r.integers(0, 4))
        rules = ["standard", "fit"] + (["ocp_floor", "oas"] if fmt == "mxfp4" else [])
        rule = rules[int(r.integers(0, len(rules)))]
        signs = bool(r.integers(0, 2))
        given = fmt == "nvfp4" and bool(r.integers(0, 3) == 0)
        scale = float(10.0 ** r.uniform(-3, 3))
        out.append((i, fmt, block, M, K, pad, rule, signs, given, scale))
    return out


@pytest.mark.parametrize("case", _quant_cases(150, 2024), ids=lambda c: f"q{c[0]}")
def test_quantizer_sweep(case):
    i, fmt, block, M, K, pad, rule, use_signs, given, scale = case
    say(f"case sweep q{i}: {fmt} b{block} M {M} K {K} pad {pad} rule {rule} signs {use_signs} given {given}")
    x = WL.draw_normal_bf16((M, K), scale, seed=7000 + i)
    wide = torch.zeros((M, K + pad), dtype=torch.bfloat16, device="cuda")
    wide[:, :K] = dev_bf16(x)
    signs = WL.draw_signs(K, 100 + i) if use_signs else None
    sdev = torch.from_numpy(signs).cuda() if use_signs else None
    ts_given = None
    ts_np = None
    if given:
        ts_np = np.float32(O.rotate_quantize(x, block, "nvfp4", signs=signs)[2] * np.float32(0.5))
        ts_given = torch.tensor([float(ts_np)], dtype=torch.float32, device="cuda")
    q = B.fp4_rotate_quantize(wide[:, :K], block, fmt, rule=rule, signs=sdev, tensor_scale=ts_given)
    torch.cuda.synchronize()
    res = compare_quant(q, x, block, fmt, rule=rule, signs=signs, tensor_scale=ts_np)
    assert_quant_parity(res, f"sweep q{i}", exact=True)


def _linear_cases():
    r = np.random.default_rng(77)
    out = []
    shapes = [(int(r.integers(1, 17)), int(r.integers(1, 700)), 512 * int(r.integers(1, 5))) for _ in range(8)]  # decode
    shapes += [(int(r.integers(17, 300)), int(r.integers(1, 300)), 128 * int(r.integers(1, 9))) for _ in range(8)]  # general
    shapes += [(int(r.integers(256, 700)), int(r.integers(256, 700)), 512 * int(r.integers(1, 4))) for _ in range(8)]  # large
    for j, (M, N, K) in enumerate(shapes):
        out.append((j, "mxfp4", 32 if j % 2 == 0 else 128, M, N, K))
    nv = [(int(r.integers(1, 300)), int(r.integers(1, 300)), 128 * int(r.integers(1, 6))) for _ in range(6)]
    nv += [(int(r.integers(256, 600)), int(r.integers(256, 600)), 128 * int(r.integers(1, 6))) for _ in range(6)]
    for j, (M, N, K) in enumerate(nv):
        out.append((100 + j, "nvfp4", 16 if j % 2 == 0 else 32, M, N, K))
    return out


@pytest.mark.parametrize("case", _linear_cases(), ids=lambda c: f"l{c[0]}")
def test_linear_sweep(case):
    j, fmt, block, M, N, K = case
    say(f"case sweep l{j}: {fmt} b{block} M {M} N {N} K {K}")
    x = WL.draw_normal_bf16((M, K), 1.0, seed=9000 + j)
    w = WL.draw_normal_bf16((N, K), 0.02, seed=9500 + j)
    xq = B.fp4_rotate_quantize(dev_bf16(x), block, fmt)
    wq = B.fp4_quantize_weights(dev_bf16(w), block, fmt)
    for out_dtype in (torch.float32, torch.bfloat16):
        y = B.fp4_linear(xq[0], xq[1], wq[0], wq[1], fmt, x_ts=xq[2], w_ts=wq[2], out_dtype=out_dtype)
        torch.cuda.synchronize()
        ref = gemm_reference(x, w, block, fmt, np.arange(M), np.arange(N))
        if out_dtype == torch.bfloat16:
            ref = O.bf16_rne_f64(ref)
        got = host(y.float() if out_dtype == torch.bfloat16 else y).astype(np.float64)
        r = rel_fro(got, ref)
        say(f"sweep l{j} {out_dtype}: rel fro {r:.3e}")
        assert r <= GEMM_REL_FRO_TOL


def _quant_cases_extreme(n, seed):
    """Like _quant_cases, with input scales from 1e-35 to 1e35: tensor scales near the ends of
    the float32 range, E8M0 codes near 0 and 254, and the E4M3 decision's float64 fallback."""
    r = np.random.default_rng(seed)
    out = []
    for i in range(n):
        fmt = ["mxfp4", "nvfp4"][i % 2]
        block = int(r.choice([16, 32, 64, 128]))
        K = max(32, int(block * r.integers(1, 6)) if block >= 32 else int(32 * r.integers(1, 12)))
        M = int(r.integers(1, 60))
        rules = ["standard", "fit"] + (["ocp_floor", "oas"] if fmt == "mxfp4" else [])
        rule = rules[int(r.integers(0, len(rules)))]
        scale = float(10.0 ** r.uniform(-35, 35))
        out.append((i, fmt, block, M, K, rule, scale))
    return out


@pytest.mark.parametrize("case", _quant_cases_extreme(100, 2026), ids=lambda c: f"qx{c[0]}")
def test_quantizer_sweep_extreme_scales(case):
    i, fmt, block, M, K, rule, scale = case
    say(f"case sweep qx{i}: {fmt} b{block} M {M} K {K} rule {rule} scale {scale:.3g}")
    x = WL.draw_normal_bf16((M, K), scale, seed=12000 + i)
    q = B.fp4_rotate_quantize(dev_bf16(x), block, fmt, rule=rule)
    torch.cuda.synchronize()
    res = compare_quant(q, x, block, fmt, rule=rule)
    assert_quant_parity(res, f"sweep qx{i}", exact=True)


def _code_cases(n, seed):
    """Random codes and scales for fp4_linear over every kernel route: unit scales (every
    product and sum exact, so Y must equal the float64 product bit for bit) or random ones."""
    r = np.random.default_rng(seed)
    out = []
    for i in range(n):
        fmt = "mxfp4" if i % 5 < 3 else "nvfp4"
        route = i % 3
        if route == 0:
            M, N, K = int(r.integers(1, 17)), int(r.integers(1, 900)), 512 * int(r.integers(1, 9))
        elif route == 1:
            M, N, K = int(r.integers(17, 400)), int(r.integers(1, 400)), 128 * int(r.integers(1, 20))
        else:
            M, N, K = int(r.integers(256, 800)), int(r.integers(256, 800)), 512 * int(r.integers(1, 5))
        out.append((i, fmt, M, N, K, bool(i % 2), int(r.integers(0, 2**31))))
    return out


@pytest.mark.parametrize("case", _code_cases(60, 77077), ids=lambda c: f"lc{c[0]}")
def test_linear_random_codes(case):
    i, fmt, M, N, K, unit, seed = case
    say(f"case sweep lc{i}: {fmt} M {M} N {N} K {K} unit scales {unit}")
    r = np.random.default_rng(seed)
    g = 32 if fmt == "mxfp4" else 16
    xq = O.pack_nibbles(r.integers(0, 16, (M, K), dtype=np.uint8))
    wq = O.pack_nibbles(r.integers(0, 16, (N, K), dtype=np.uint8))
    one, lo, hi = (127, 118, 136) if fmt == "mxfp4" else (0x38, 0x20, 0x60)  # E8M0 / E4M3 codes of 1.0
    xs = np.full((M, K // g), one, np.uint8) if unit else r.integers(lo, hi, (M, K // g), dtype=np.uint8)
    ws = np.full((N, K // g), one, np.uint8) if unit else r.integers(lo, hi, (N, K // g), dtype=np.uint8)
    xt = wt = None
    kw = {}
    if fmt == "nvfp4":
        xt = np.float32(1.0) if unit else np.float32(r.uniform(0.01, 3.0))
        wt = np.float32(1.0) if unit else np.float32(r.uniform(0.01, 3.0))
        kw = dict(x_ts=torch.tensor([float(xt)], device="cuda"), w_ts=torch.tensor([float(wt)], device="cuda"))
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    ref = O.linear_f64(xq, xs, wq, ws, fmt, xt, wt)
    for out_dtype in (torch.float32, torch.bfloat16):
        y = B.fp4_linear(t(xq), t(xs), t(wq), t(ws), fmt, out_dtype=out_dtype, **kw)
        torch.cuda.synchronize()
        got = host(y.float() if out_dtype == torch.bfloat16 else y).astype(np.float64)
        want = O.bf16_rne_f64(ref) if out_dtype == torch.bfloat16 else ref.astype(np.float32).astype(np.float64)
        if unit:
            assert np.array_equal(got, want), f"lc{i} {out_dtype}: max |diff| {np.abs(got - want).max()}"
        else:
            r_err = rel_fro(got, want)
            say(f"sweep lc{i} {out_dtype}: rel fro {r_err:.3e}")
            assert r_err <= GEMM_REL_FRO_TOL
