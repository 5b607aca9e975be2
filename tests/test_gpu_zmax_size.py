"""The largest inputs the quantizer and the GEMM accept, checked on sampled rows against the oracle.

fp4_rotate_quantize takes up to 2^31 - 1 chunks of 32 elements (rows * K / 32 must fit in
31 bits). The first test runs an input just under that limit (X of 128 GiB, byte offsets far
beyond 2^32) for MXFP4, and for NVFP4 with a given tensor scale. The second runs the NVFP4
tensor-maximum pass over an 8 GiB input whose maximum is planted in a known row, so the
sampled rows determine T exactly. The GEMM tests take an operand beyond 4 GiB (MXFP4 and
NVFP4), and K at the large-tile MXFP4 kernel's 32-bit offset limit and one step past it. Inputs come from torch's seeded
generator on the device; only the sampled rows are copied to the host for the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from microscaling_fp4_quantized_amd import binding as B
from oracle import fp4_oracle as O
from parity import GEMM_REL_FRO_TOL, assert_quant_parity, compare_quant, gemm_reference, rel_fro, say

pytestmark = pytest.mark.gpu

GIB = 1 << 30


def _free_bytes() -> int:
    torch.cuda.empty_cache()
    return torch.cuda.mem_get_info()[0]


def _rows_bits(x: torch.Tensor, rows: np.ndarray) -> np.ndarray:
    sel = x[torch.from_numpy(rows).to(x.device)]
    return sel.view(torch.int16).cpu().numpy().view(np.uint16)


def _rows_out(out, rows: np.ndarray):
    idx = torch.from_numpy(rows).to(out[0].device)
    return out[0][idx], out[1][idx], out[2]


def test_max_chunk_count():
    K = 8192
    M = (2**31 - 1) // (K // 32)  # 8 388 607 rows: 2^31 - 256 chunks
    need = M * K * 2 + M * K // 2 + M * K // 16 + 2 * GIB
    if _free_bytes() < need:
        pytest.skip(f"needs {need / GIB:.0f} GiB of free device memory")
    say(f"case max chunk count: X {M}x{K} bf16 ({M * K * 2 / GIB:.0f} GiB), MXFP4 b32, then NVFP4 b32 given s_t")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20250531)
    x = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    x.normal_(generator=gen)
    rows = np.array([0, 1, 4097, M // 2, M - 2, M - 1])
    xb = _rows_bits(x, rows)

    out = B.fp4_rotate_quantize(x, 32, "mxfp4")
    torch.cuda.synchronize()
    got = _rows_out(out, rows)
    del out
    assert_quant_parity(compare_quant(got, xb, 32, "mxfp4"), "max chunk count mxfp4")

    s_t = np.float32(14.0 / 2688.0)  # clips only |y| > 14, far beyond this N(0, 1) input
    ts = torch.tensor([s_t], dtype=torch.float32, device="cuda")
    out = B.fp4_rotate_quantize(x, 32, "nvfp4", tensor_scale=ts)
    torch.cuda.synchronize()
    got = _rows_out(out, rows)
    del out, x
    assert_quant_parity(compare_quant(got, xb, 32, "nvfp4", tensor_scale=s_t), "max chunk count nvfp4 given s_t")
    torch.cuda.empty_cache()


def test_nv_tensor_maximum_beyond_4gib():
    K = 8192
    M = 524288  # X of 8 GiB
    need = M * K * 2 + M * K // 2 + M * K // 16 + GIB
    if _free_bytes() < need:
        pytest.skip(f"needs {need / GIB:.0f} GiB of free device memory")
    say(f"case NVFP4 tensor maximum: X {M}x{K} bf16 ({M * K * 2 / GIB:.0f} GiB), b32, planted maximum")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    x = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    x.normal_(generator=gen)
    r0, c0 = M - 3, 5000
    # rotated, this value dominates its block (|y| ~ 1000 / sqrt(32) ~ 177 against ~7 elsewhere),
    # so T over the sampled rows, which include r0, is T over the tensor
    x[r0, c0] = 1000.0
    rows = np.array([0, M // 3, r0, M - 1])
    xb = _rows_bits(x, rows)
    out = B.fp4_rotate_quantize(x, 32, "nvfp4")
    torch.cuda.synchronize()
    got = _rows_out(out, rows)
    del out, x
    res = compare_quant(got, xb, 32, "nvfp4")
    assert_quant_parity(res, "nvfp4 tensor maximum beyond 4 GiB")
    assert res["tensor_scale"] > 170.0 / 2688.0
    torch.cuda.empty_cache()


def test_gemm_operand_beyond_4gib():
    # Xq of 131072 x 32768 bytes: the large-tile kernel's row offsets into it pass 2^32 bytes
    M, K, N = 131072, 65536, 512
    need = M * K * 2 + M * K // 2 + M * K // 32 + M * N * 4 + GIB
    if _free_bytes() < need:
        pytest.skip(f"needs {need / GIB:.0f} GiB of free device memory")
    say(f"case GEMM operand beyond 4 GiB: M {M} K {K} N {N}, MXFP4 b32, Xq {M * K // 2 / GIB:.0f} GiB")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    x = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    x.normal_(generator=gen)
    w = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    w.normal_(mean=0.0, std=0.02, generator=gen)
    rows = np.array([0, 255, 256, M // 2 + 17, M - 1])
    cols = np.array([0, 1, 255, 256, N - 1])
    xb, wb = _rows_bits(x, rows), _rows_bits(w, cols)
    xq, xs, _ = B.fp4_rotate_quantize(x, 32, "mxfp4")
    del x
    wq, ws, _ = B.fp4_quantize_weights(w, 32, "mxfp4")
    y = B.fp4_linear(xq, xs, wq, ws, "mxfp4")
    torch.cuda.synchronize()
    got = y[torch.from_numpy(rows).to(y.device)][:, torch.from_numpy(cols).to(y.device)].cpu().numpy()
    del xq, xs, wq, ws, y, w
    ref = gemm_reference(xb, wb, 32, "mxfp4", np.arange(len(rows)), np.arange(len(cols)))
    assert np.linalg.norm(ref) > 0 and np.count_nonzero(ref) == ref.size
    r = rel_fro(got, ref)
    say(f"GEMM beyond 4 GiB sampled rel fro {r:.3e} (|ref| {np.linalg.norm(ref):.3e})")
    assert r <= GEMM_REL_FRO_TOL
    torch.cuda.empty_cache()


@pytest.mark.parametrize("K", [2**25 - 512, 2**25])
def test_gemm_k_at_the_offset_limit(K):
    # The large-tile MXFP4 kernel addresses a tile's operand rows from the tile's first row with
    # 32-bit offsets, so it takes K < 2^25 (256 rows x K/2 bytes < 2^32). K = 2^25 - 512 is the
    # largest K it runs, with offsets just below 4 GiB; K = 2^25 goes to the general kernel.
    M = N = 256
    need = 2 * M * K * 2 + 2 * (M * K // 2 + M * K // 32) + M * N * 4 + 2 * GIB
    if _free_bytes() < need:
        pytest.skip(f"needs {need / GIB:.0f} GiB of free device memory")
    say(f"case GEMM K at the 32-bit offset limit: M {M} N {N} K {K}, MXFP4 b32")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(K % 1000 + 5)
    x = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    x.normal_(generator=gen)
    w = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    w.normal_(mean=0.0, std=0.02, generator=gen)
    rows, cols = np.array([0, M - 1]), np.array([3, N - 2])
    xb, wb = _rows_bits(x, rows), _rows_bits(w, cols)
    xq, xs, _ = B.fp4_rotate_quantize(x, 32, "mxfp4")
    del x
    wq, ws, _ = B.fp4_quantize_weights(w, 32, "mxfp4")
    del w
    y = B.fp4_linear(xq, xs, wq, ws, "mxfp4")
    torch.cuda.synchronize()
    got = y[torch.from_numpy(rows).to(y.device)][:, torch.from_numpy(cols).to(y.device)].cpu().numpy()
    del xq, xs, wq, ws, y
    torch.cuda.empty_cache()
    ref = gemm_reference(xb, wb, 32, "mxfp4", np.arange(len(rows)), np.arange(len(cols)))
    assert np.count_nonzero(ref) == ref.size
    r = rel_fro(got, ref)
    say(f"GEMM K={K} sampled rel fro {r:.3e}")
    assert r <= GEMM_REL_FRO_TOL


def test_nv_gemm_operand_beyond_4gib():
    # NVFP4: Xq of 131072 x 32768 bytes; the large-tile kernel's row offsets pass 2^32 bytes.
    # A dominant value is planted in a sampled row of X and of W (as in the tensor-maximum test
    # above), so the oracle's T over the sampled rows is T over each whole tensor.
    M, K, N = 131072, 65536, 512
    need = M * K * 2 + M * K // 2 + M * K // 16 + M * N * 4 + GIB
    if _free_bytes() < need:
        pytest.skip(f"needs {need / GIB:.0f} GiB of free device memory")
    say(f"case NVFP4 GEMM operand beyond 4 GiB: M {M} K {K} N {N}, b16, Xq {M * K // 2 / GIB:.0f} GiB")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(13)
    x = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    x.normal_(generator=gen)
    w = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    w.normal_(mean=0.0, std=0.02, generator=gen)
    rows = np.array([0, 255, 256, M // 2 + 17, M - 1])
    cols = np.array([0, 1, 255, 256, N - 1])
    # rotated by H16 / 4 these give |y| = 250 and 5, against about 7 and 0.15 elsewhere
    x[int(rows[3]), 40000] = 1000.0
    w[int(cols[2]), 123] = 20.0
    xb, wb = _rows_bits(x, rows), _rows_bits(w, cols)
    xq, xs, xts = B.fp4_rotate_quantize(x, 16, "nvfp4")
    del x
    wq, ws, wts = B.fp4_quantize_weights(w, 16, "nvfp4")
    del w
    y = B.fp4_linear(xq, xs, wq, ws, "nvfp4", x_ts=xts, w_ts=wts)
    torch.cuda.synchronize()
    got = y[torch.from_numpy(rows).to(y.device)][:, torch.from_numpy(cols).to(y.device)].cpu().numpy()
    s_x, s_w = np.float32(xts.cpu()[0]), np.float32(wts.cpu()[0])
    del xq, xs, wq, ws, y
    torch.cuda.empty_cache()
    ref = gemm_reference(xb, wb, 16, "nvfp4", np.arange(len(rows)), np.arange(len(cols)))
    # the tensor scales: the oracle's, over the sampled rows, equal the GPU's bit for bit
    _, _, ox = O.rotate_quantize(xb, 16, "nvfp4")
    _, _, ow = O.rotate_quantize(wb, 16, "nvfp4")
    assert np.float32(ox).view(np.uint32) == s_x.view(np.uint32), (ox, s_x)
    assert np.float32(ow).view(np.uint32) == s_w.view(np.uint32), (ow, s_w)
    assert np.count_nonzero(ref) == ref.size
    r = rel_fro(got, ref)
    say(f"NVFP4 GEMM beyond 4 GiB sampled rel fro {r:.3e} (|ref| {np.linalg.norm(ref):.3e}), s_x {s_x:.6e} s_w {s_w:.6e}")
    assert r <= GEMM_REL_FRO_TOL
