"""GPU parity of fp4_linear (W4A4 GEMM) against the float64 oracle product.

The reference is always built from oracle-quantized operands. Small cases are
compared in full; the prefill and large workloads run at their full sizes and
are compared on sampled rows and columns of Y.
"""
import numpy as np
import pytest
import torch

from microscaling_fp4_quantized_amd import binding as B
from microscaling_fp4_quantized_amd import workloads as WL
from oracle import fp4_oracle as O
from parity import (GEMM_REL_FRO_TOL, assert_quant_parity, compare_quant, dev_bf16, gemm_reference, host,
                    rel_fro, say, tensor_amax)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load_library()


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


@pytest.mark.parametrize("M,N,K", [(64, 80, 512), (37, 200, 384), (1, 16, 128), (130, 129, 256)])
def test_unit_scales_bit_exact(M, N, K):
    # all scales 2^0: every partial sum is a multiple of 1/4 below 2^24 -> exact in any order
    rng = np.random.default_rng(M * N + K)
    c = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    d = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    xs = np.full((M, K // 32), 127, np.uint8)
    ws = np.full((N, K // 32), 127, np.uint8)
    ref = O.linear_f64(O.pack_nibbles(c), xs, O.pack_nibbles(d), ws, "mxfp4")
    say(f"case unit-scale exact M {M} N {N} K {K}")
    y = B.fp4_linear(dev_u8(O.pack_nibbles(c)), dev_u8(xs), dev_u8(O.pack_nibbles(d)), dev_u8(ws), "mxfp4")
    assert np.array_equal(host(y).astype(np.float64), ref)
    yb = B.fp4_linear(dev_u8(O.pack_nibbles(c)), dev_u8(xs), dev_u8(O.pack_nibbles(d)), dev_u8(ws), "mxfp4",
                      out_dtype=torch.bfloat16)
    yb = host(yb.float()).astype(np.float64)
    assert np.array_equal(yb, O.bf16_rne_f64(ref))


@pytest.mark.parametrize("M,N,K", [(1, 77, 512), (5, 300, 1536), (16, 4096, 4096), (3, 130, 8192), (16, 18, 2560),
                                   (9, 12300, 1024), (16, 12289, 4608), (8, 14336, 4096), (4, 200, 12288),
                                   (2, 33, 9216)])
def test_decode_kernel_unit_scales_exact(M, N, K):
    # M <= 16 with K % 512 == 0 runs the weight-streaming decode kernel: 8 waves, each fetching
    # its own 512-wide K slices into LDS (K = 8192: two slices per wave; K = 512, 1536, 2560 leave
    # some waves idle), LDS reduction; N % 16 != 0 leaves ragged weight rows; M >= 8 with
    # N >= 3 * 16 * 256 puts two 16-row tiles in a workgroup (12300, 12289: the last workgroup's
    # second tile is partly or wholly past N). Longer K takes the chunked variant: W staged
    # through LDS in chunks of at most 4096 K (4608 with two tiles: three chunks of 1536; 12288:
    # three of 4096; 9216: three of 3072).
    rng = np.random.default_rng(3 * M + N + K)
    c = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    d = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    xs = np.full((M, K // 32), 127, np.uint8)
    ws = np.full((N, K // 32), 127, np.uint8)
    ref = O.linear_f64(O.pack_nibbles(c), xs, O.pack_nibbles(d), ws, "mxfp4")
    say(f"case decode-kernel unit-scale exact M {M} N {N} K {K}")
    args = (dev_u8(O.pack_nibbles(c)), dev_u8(xs), dev_u8(O.pack_nibbles(d)), dev_u8(ws), "mxfp4")
    y = B.fp4_linear(*args)
    assert np.array_equal(host(y).astype(np.float64), ref)
    yb = B.fp4_linear(*args, out_dtype=torch.bfloat16)
    assert np.array_equal(host(yb.float()).astype(np.float64), O.bf16_rne_f64(ref))


@pytest.mark.parametrize("M,N,K", [(17, 300, 512), (32, 4096, 4096), (32, 12300, 1024), (33, 8000, 1024),
                                   (48, 777, 8192), (64, 8191, 4096), (63, 4100, 8192), (64, 16, 2560),
                                   (40, 20, 1536), (65, 300, 1024)])
def test_decode_kernel_up_to_64_tokens_unit_scales_exact(M, N, K):
    # 16 < M <= 64 with K % 512 == 0 and K <= 8192 runs the decode kernel with ceil(M / 16) column
    # fragments of X per W fragment (17, 33: one row into the last fragment; 48, 63, 64: three and
    # four fragments), except 33-64 rows against N >= 8192, which take the 128-row ring tiles;
    # N >= 3 * 16 * 256 with K <= 4096 puts two tiles in a workgroup (32 x 12300: ragged last
    # workgroup), K = 8192 gives each wave two slices with one tile, K = 512 and 2560 leave waves
    # idle. M = 65 takes the general kernel.
    rng = np.random.default_rng(5 * M + N + K)
    c = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    d = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    xs = np.full((M, K // 32), 127, np.uint8)
    ws = np.full((N, K // 32), 127, np.uint8)
    ref = O.linear_f64(O.pack_nibbles(c), xs, O.pack_nibbles(d), ws, "mxfp4")
    say(f"case decode-kernel (<= 64 tokens) unit-scale exact M {M} N {N} K {K}")
    args = (dev_u8(O.pack_nibbles(c)), dev_u8(xs), dev_u8(O.pack_nibbles(d)), dev_u8(ws), "mxfp4")
    y = B.fp4_linear(*args)
    assert np.array_equal(host(y).astype(np.float64), ref)
    yb = B.fp4_linear(*args, out_dtype=torch.bfloat16)
    assert np.array_equal(host(yb.float()).astype(np.float64), O.bf16_rne_f64(ref))


@pytest.mark.parametrize("M,N,K", [(50, 1000, 2048), (64, 8000, 4096), (32, 12300, 4096)])
def test_decode_kernel_up_to_64_tokens_random_scales(M, N, K):
    rng = np.random.default_rng(M + N)
    c = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    d = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    xs = rng.integers(110, 140, size=(M, K // 32)).astype(np.uint8)
    ws = rng.integers(110, 140, size=(N, K // 32)).astype(np.uint8)
    ref = O.linear_f64(O.pack_nibbles(c), xs, O.pack_nibbles(d), ws, "mxfp4")
    say(f"case decode-kernel (<= 64 tokens) random scales M {M} N {N} K {K}")
    y = B.fp4_linear(dev_u8(O.pack_nibbles(c)), dev_u8(xs), dev_u8(O.pack_nibbles(d)), dev_u8(ws), "mxfp4")
    r = rel_fro(host(y), ref)
    say(f"rel fro {r:.3e}")
    assert r <= 1e-6


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("M,N,K", [(65, 1024, 512), (100, 1100, 1536), (128, 2048, 512), (200, 3000, 4096),
                                   (255, 14336, 1024), (129, 1030, 8192), (33, 12300, 1024), (64, 12289, 4096),
                                   (48, 8192, 8192), (160, 8300, 1536), (129, 8192, 1024)])
def test_skinny_tiles_unit_scales_exact(fmt, M, N, K):
    # 64 < M < 256 with N >= 1024 (and K % 512 == 0 for MXFP4, K % 256 == 0 for NVFP4) runs the
    # large-tile kernels on one row tile of 64-column tiles, 128 rows up to M = 128 and 256 above,
    # whose rows past M repeat row M - 1 (N = 1100, 3000, 1030, 12300, 12289: a ragged last column
    # tile); for MXFP4 so do 33-64 rows against N >= 8192 (for NVFP4 those take the decode
    # kernel), and above 128 rows both take two 128-row tiles per column where the 256-row grid
    # would fill at most half the CUs (N <= 8192 on 256 CUs; 8300 and 14336 keep 256-row tiles).
    # Unit scales make every sum exact.
    rng = np.random.default_rng(3 * M + N + K)
    c = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    d = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    g, one = (32, 127) if fmt == "mxfp4" else (16, 0x38)
    xs = np.full((M, K // g), one, np.uint8)
    ws = np.full((N, K // g), one, np.uint8)
    ts = {} if fmt == "mxfp4" else {"x_ts": dev_f32(1.0), "w_ts": dev_f32(1.0)}
    ref = O.linear_f64(O.pack_nibbles(c), xs, O.pack_nibbles(d), ws, fmt, *(() if fmt == "mxfp4" else (1.0, 1.0)))
    say(f"case skinny-tile unit-scale exact {fmt} M {M} N {N} K {K}")
    args = (dev_u8(O.pack_nibbles(c)), dev_u8(xs), dev_u8(O.pack_nibbles(d)), dev_u8(ws), fmt)
    y = B.fp4_linear(*args, **ts)
    assert np.array_equal(host(y).astype(np.float64), ref)
    yb = B.fp4_linear(*args, **ts, out_dtype=torch.bfloat16)
    assert np.array_equal(host(yb.float()).astype(np.float64), O.bf16_rne_f64(ref))


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("M,N,K", [(150, 2100, 2048), (100, 1100, 4096), (128, 3000, 8192), (97, 1024, 1536),
                                   (40, 8200, 4096), (200, 9000, 2048)])
def test_skinny_tiles_random_scales(fmt, M, N, K):
    # random scales catch a stage multiplied with another stage's scale bytes, which unit scales
    # hide: the MXFP4 tiles keep three stages in flight (K = 1536: six stages in all); 40 rows
    # against N = 8200 take the 128-row MXFP4 tiles and the NVFP4 decode kernel; 150 x 2100 two
    # 128-row tiles per column, 200 x 9000 one 256-row tile
    rng = np.random.default_rng((21 if fmt == "mxfp4" else 22) + M + K)
    c = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    d = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    if fmt == "mxfp4":
        xs = rng.integers(110, 140, size=(M, K // 32)).astype(np.uint8)
        ws = rng.integers(110, 140, size=(N, K // 32)).astype(np.uint8)
        ref = O.linear_f64(O.pack_nibbles(c), xs, O.pack_nibbles(d), ws, "mxfp4")
        ts = {}
    else:
        xs = rng.integers(0, 0x7F, size=(M, K // 16)).astype(np.uint8)
        ws = rng.integers(0, 0x7F, size=(N, K // 16)).astype(np.uint8)
        ref = O.linear_f64(O.pack_nibbles(c), xs, O.pack_nibbles(d), ws, "nvfp4", np.float32(0.0123), np.float32(3.5e-3))
        ts = {"x_ts": dev_f32(0.0123), "w_ts": dev_f32(3.5e-3)}
    say(f"case skinny-tile random scales {fmt} M {M} N {N} K {K}")
    y = B.fp4_linear(dev_u8(O.pack_nibbles(c)), dev_u8(xs), dev_u8(O.pack_nibbles(d)), dev_u8(ws), fmt, **ts)
    r = rel_fro(host(y), ref)
    say(f"rel fro {r:.3e}")
    assert r <= 1e-6


def test_decode_kernel_random_scales():
    rng = np.random.default_rng(99)
    M, N, K = 7, 520, 3072
    c = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    d = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    xs = rng.integers(110, 140, size=(M, K // 32)).astype(np.uint8)
    ws = rng.integers(110, 140, size=(N, K // 32)).astype(np.uint8)
    ref = O.linear_f64(O.pack_nibbles(c), xs, O.pack_nibbles(d), ws, "mxfp4")
    y = B.fp4_linear(dev_u8(O.pack_nibbles(c)), dev_u8(xs), dev_u8(O.pack_nibbles(d)), dev_u8(ws), "mxfp4")
    r = rel_fro(host(y), ref)
    say(f"decode kernel random scales rel fro {r:.3e}")
    assert r <= 1e-6


@pytest.mark.parametrize("M,N,K", [(512, 512, 1024), (300, 520, 512), (256, 261, 512), (512, 772, 512),
                                   (777, 1000, 1536), (2048, 8192, 512), (2048, 12544, 512),
                                   (4000, 14272, 512)])
def test_large_tile_kernel_unit_scales_exact(M, N, K):
    # shapes routed to the large-tile kernel (K % 512 == 0, M, N >= 256), ragged edges included.
    # On 256 CUs the column plan is: one round of 256x256 tiles for 2048 x 8192; 256x256 tiles
    # then 256x192 tiles for 2048 x 12544; 256x192 tiles alone for the small shapes; for
    # 4000 x 14272, 32 panels of 256 then 32 of 192 (the last one 128 columns wide) over 16 row
    # tiles, the last one 160 rows. The bf16 output takes 16-byte pieces when N % 8 == 0, two
    # 8-byte halves when N % 8 == 4 (772), and single elements otherwise (261).
    rng = np.random.default_rng(M + N + K)
    c = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    d = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    xs = np.full((M, K // 32), 127, np.uint8)
    ws = np.full((N, K // 32), 127, np.uint8)
    ref = O.linear_f64(O.pack_nibbles(c), xs, O.pack_nibbles(d), ws, "mxfp4")
    say(f"case large-tile unit-scale exact M {M} N {N} K {K}")
    args = (dev_u8(O.pack_nibbles(c)), dev_u8(xs), dev_u8(O.pack_nibbles(d)), dev_u8(ws), "mxfp4")
    y = B.fp4_linear(*args)
    assert np.array_equal(host(y).astype(np.float64), ref)
    yb = B.fp4_linear(*args, out_dtype=torch.bfloat16)
    assert np.array_equal(host(yb.float()).astype(np.float64), O.bf16_rne_f64(ref))


@pytest.mark.parametrize("M,N,K", [(512, 768, 2048), (259, 300, 512), (2048, 12544, 1024)])
def test_large_tile_kernel_random_scales(M, N, K):
    rng = np.random.default_rng(7 * M + N)
    c = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    d = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    xs = rng.integers(110, 140, size=(M, K // 32)).astype(np.uint8)
    ws = rng.integers(110, 140, size=(N, K // 32)).astype(np.uint8)
    ref = O.linear_f64(O.pack_nibbles(c), xs, O.pack_nibbles(d), ws, "mxfp4")
    y = B.fp4_linear(dev_u8(O.pack_nibbles(c)), dev_u8(xs), dev_u8(O.pack_nibbles(d)), dev_u8(ws), "mxfp4")
    r = rel_fro(host(y), ref)
    say(f"large-tile random scales M {M} N {N} K {K}: rel fro {r:.3e}")
    assert r <= 1e-6


def offset_u8(a, off):
    """A contiguous device copy of a whose data pointer sits `off` bytes past a 256-byte boundary."""
    a = np.ascontiguousarray(a, dtype=np.uint8)
    buf = torch.zeros(a.size + 256, dtype=torch.uint8, device="cuda")
    v = buf[off:off + a.size].view(a.shape)
    v.copy_(torch.from_numpy(a))
    assert v.data_ptr() % 16 == off % 16
    return v


@pytest.mark.parametrize("M,N,K", [(4, 300, 1024), (300, 520, 512)])
def test_scales_only_4byte_aligned(M, N, K):
    # Xs / Ws 4 bytes past a 16-byte boundary (allowed by the contract): the decode and large-tile
    # kernels read 16 scale bytes at once, so these shapes must take the general kernel and stay exact
    rng = np.random.default_rng(5 * M + N)
    c = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    d = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    xs = np.full((M, K // 32), 127, np.uint8)
    ws = np.full((N, K // 32), 127, np.uint8)
    ref = O.linear_f64(O.pack_nibbles(c), xs, O.pack_nibbles(d), ws, "mxfp4")
    for ox, ow in ((4, 0), (0, 4), (12, 8)):
        say(f"case scales at byte offsets {ox}/{ow} M {M} N {N} K {K}")
        y = B.fp4_linear(dev_u8(O.pack_nibbles(c)), offset_u8(xs, ox), dev_u8(O.pack_nibbles(d)), offset_u8(ws, ow),
                         "mxfp4")
        assert np.array_equal(host(y).astype(np.float64), ref)


def test_fused_decode_refuses_unaligned_weight_scales():
    K, N = 512, 64
    x = dev_bf16(WL.draw_normal_bf16((2, K), 1.0, seed=4))
    wq = torch.zeros((N, K // 2), dtype=torch.uint8, device="cuda")
    with pytest.raises(B.Fp4Error):
        B.fp4_rotate_quantize_linear(x, wq, offset_u8(np.full((N, K // 32), 127, np.uint8), 4), 32)


def test_scale_byte_extremes_exact():
    # per-group scales spread over a wide exponent range, still exact in float32
    rng = np.random.default_rng(3)
    M, N, K = 48, 64, 1024
    c = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    d = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    xs = rng.integers(120, 135, size=(M, K // 32)).astype(np.uint8)
    ws = rng.integers(120, 135, size=(N, K // 32)).astype(np.uint8)
    ref = O.linear_f64(O.pack_nibbles(c), xs, O.pack_nibbles(d), ws, "mxfp4")
    y = B.fp4_linear(dev_u8(O.pack_nibbles(c)), dev_u8(xs), dev_u8(O.pack_nibbles(d)), dev_u8(ws), "mxfp4")
    r = rel_fro(host(y), ref)
    say(f"scale extremes rel fro {r:.3e}")
    assert r <= 1e-6


def dev_f32(v):
    return torch.tensor([v], dtype=torch.float32).cuda()


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (512, 768, 1024), (300, 520, 768), (777, 1000, 1536),
                                   (2048, 8192, 256), (2048, 12544, 256), (4000, 14272, 256), (256, 256, 128),
                                   (300, 520, 384)])
def test_nv_large_tile_kernel_unit_scales_exact(M, N, K):
    # NVFP4 shapes routed to the large-tile kernel (M, N >= 256, K % 256 == 0; K = 128 and 384 take
    # the general kernel): group scales 1.0 (E4M3 code 0x38) and tensor scales 1.0 make every
    # product a multiple of 1/4 and every sum exact.
    # Column plans on 256 CUs: one round of 256x256 tiles for 2048 x 8192, 256x256 then 256x192
    # tiles for 2048 x 12544 and for 4000 x 14272 (ragged in both: a last row tile of 160 rows,
    # a last 192-wide panel of 128 columns), 256x192 tiles alone for the small shapes.
    rng = np.random.default_rng(5 * M + N + K)
    c = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    d = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    xs = np.full((M, K // 16), 0x38, np.uint8)
    ws = np.full((N, K // 16), 0x38, np.uint8)
    ref = O.linear_f64(O.pack_nibbles(c), xs, O.pack_nibbles(d), ws, "nvfp4", 1.0, 1.0)
    say(f"case NV large-tile unit-scale exact M {M} N {N} K {K}")
    args = (dev_u8(O.pack_nibbles(c)), dev_u8(xs), dev_u8(O.pack_nibbles(d)), dev_u8(ws), "nvfp4")
    y = B.fp4_linear(*args, x_ts=dev_f32(1.0), w_ts=dev_f32(1.0))
    assert np.array_equal(host(y).astype(np.float64), ref)
    yb = B.fp4_linear(*args, x_ts=dev_f32(1.0), w_ts=dev_f32(1.0), out_dtype=torch.bfloat16)
    assert np.array_equal(host(yb.float()).astype(np.float64), O.bf16_rne_f64(ref))


@pytest.mark.parametrize("M,N,K", [(1, 77, 512), (5, 300, 1536), (16, 4096, 4096), (3, 130, 8192), (16, 18, 2560),
                                   (9, 12300, 1024), (16, 12289, 4096), (8, 14336, 4096), (2, 33, 8192),
                                   (4, 200, 9216), (16, 64, 640), (17, 300, 512), (33, 12300, 1024),
                                   (48, 777, 8192), (64, 12289, 4096), (64, 16, 2560), (65, 300, 1024)])
def test_nv_decode_kernel_unit_scales_exact(M, N, K):
    # NVFP4 with M <= 64, K % 512 == 0 and K <= 8192 runs the weight-streaming decode kernel: 8 waves
    # each dequantize their own 512-wide K slices of W (from LDS) and X (from L2) to fp16 (K = 8192:
    # two slices per wave; 512, 1536, 2560 leave waves idle); N >= 3 * 16 * 256 with K <= 4096 puts
    # two 16-row tiles in a workgroup (12300, 12289: ragged last workgroup); above 16 rows every W
    # fragment meets ceil(M / 16) X fragments. K = 9216 and 640, and M = 65, take the general
    # kernel. Unit group and tensor scales make every sum exact.
    rng = np.random.default_rng(7 * M + N + K)
    c = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    d = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    xs = np.full((M, K // 16), 0x38, np.uint8)
    ws = np.full((N, K // 16), 0x38, np.uint8)
    ref = O.linear_f64(O.pack_nibbles(c), xs, O.pack_nibbles(d), ws, "nvfp4", 1.0, 1.0)
    say(f"case NV decode-kernel unit-scale exact M {M} N {N} K {K}")
    args = (dev_u8(O.pack_nibbles(c)), dev_u8(xs), dev_u8(O.pack_nibbles(d)), dev_u8(ws), "nvfp4")
    y = B.fp4_linear(*args, x_ts=dev_f32(1.0), w_ts=dev_f32(1.0))
    assert np.array_equal(host(y).astype(np.float64), ref)
    yb = B.fp4_linear(*args, x_ts=dev_f32(1.0), w_ts=dev_f32(1.0), out_dtype=torch.bfloat16)
    assert np.array_equal(host(yb.float()).astype(np.float64), O.bf16_rne_f64(ref))


@pytest.mark.parametrize("M,N,K", [(7, 520, 3072), (16, 12300, 4096), (1, 300, 8192), (50, 1000, 2048),
                                   (64, 12300, 4096)])
def test_nv_decode_kernel_random_scales(M, N, K):
    rng = np.random.default_rng(13 * M + N)
    c = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    d = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    xs = rng.integers(0, 0x7F, size=(M, K // 16)).astype(np.uint8)  # every finite E4M3 code, subnormals included
    ws = rng.integers(0, 0x7F, size=(N, K // 16)).astype(np.uint8)
    xt, wt = 0.0123, 3.5e-3
    ref = O.linear_f64(O.pack_nibbles(c), xs, O.pack_nibbles(d), ws, "nvfp4", np.float32(xt), np.float32(wt))
    say(f"case NV decode-kernel random scales M {M} N {N} K {K}")
    y = B.fp4_linear(dev_u8(O.pack_nibbles(c)), dev_u8(xs), dev_u8(O.pack_nibbles(d)), dev_u8(ws), "nvfp4",
                     x_ts=dev_f32(xt), w_ts=dev_f32(wt))
    r = rel_fro(host(y), ref)
    say(f"rel fro {r:.3e}")
    assert r <= 1e-6


@pytest.mark.parametrize("M,N,K", [(512, 768, 2048), (259, 300, 512), (2048, 12544, 768)])
def test_nv_large_tile_kernel_random_scales(M, N, K):
    rng = np.random.default_rng(11 * M + N)
    c = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    d = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    xs = rng.integers(0, 0x7F, size=(M, K // 16)).astype(np.uint8)  # every finite E4M3 code, subnormals included
    ws = rng.integers(0, 0x7F, size=(N, K // 16)).astype(np.uint8)
    xt, wt = 0.0123, 3.5e-3
    ref = O.linear_f64(O.pack_nibbles(c), xs, O.pack_nibbles(d), ws, "nvfp4", np.float32(xt), np.float32(wt))
    y = B.fp4_linear(dev_u8(O.pack_nibbles(c)), dev_u8(xs), dev_u8(O.pack_nibbles(d)), dev_u8(ws), "nvfp4",
                     x_ts=dev_f32(xt), w_ts=dev_f32(wt))
    r = rel_fro(host(y), ref)
    say(f"NV large-tile random scales M {M} N {N} K {K}: rel fro {r:.3e}")
    assert r <= 1e-6


def quantize_both(x, w, block, fmt):
    xq = B.fp4_rotate_quantize(dev_bf16(x), block, fmt)
    wq = B.fp4_quantize_weights(dev_bf16(w), block, fmt)
    torch.cuda.synchronize()
    return xq, wq


def linear_of(xq, wq, fmt, out_dtype):
    y = B.fp4_linear(xq[0], xq[1], wq[0], wq[1], fmt, x_ts=xq[2], w_ts=wq[2], out_dtype=out_dtype)
    torch.cuda.synchronize()
    return host(y.float() if out_dtype == torch.bfloat16 else y).astype(np.float64)


@pytest.mark.parametrize("fmt,block", [("mxfp4", 32), ("mxfp4", 128), ("nvfp4", 16), ("nvfp4", 32)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_tiny_end_to_end(fmt, block, out_dtype):
    w = WL.WORKLOADS["tiny"]
    x, wt = WL.draw_x(w), WL.draw_w(w)
    say(f"case tiny linear {fmt} b{block} {out_dtype}")
    xq, wq = quantize_both(x, wt, block, fmt)
    assert_quant_parity(compare_quant(xq, x, block, fmt), "tiny X")
    assert_quant_parity(compare_quant(wq, wt, block, fmt), "tiny W")
    y = linear_of(xq, wq, fmt, out_dtype)
    ref = gemm_reference(x, wt, block, fmt, np.arange(x.shape[0]), np.arange(wt.shape[0]))
    if out_dtype == torch.bfloat16:
        ref = O.bf16_rne_f64(ref)
    r = rel_fro(y, ref)
    say(f"tiny {fmt} b{block} rel fro {r:.3e}")
    assert r <= GEMM_REL_FRO_TOL


@pytest.mark.parametrize("fmt,block", [("mxfp4", 32), ("nvfp4", 16)])
@pytest.mark.parametrize("M,N,K", [(37, 200, 384), (129, 77, 640), (1, 300, 128)])
def test_ragged_shapes(fmt, block, M, N, K):
    x = WL.draw_normal_bf16((M, K), 1.0, seed=M + 1)
    wt = WL.draw_normal_bf16((N, K), 0.02, seed=N + 2)
    say(f"case ragged linear {fmt} M {M} N {N} K {K}")
    xq, wq = quantize_both(x, wt, block, fmt)
    y = linear_of(xq, wq, fmt, torch.float32)
    ref = gemm_reference(x, wt, block, fmt, np.arange(M), np.arange(N))
    r = rel_fro(y, ref)
    say(f"ragged rel fro {r:.3e}")
    assert r <= GEMM_REL_FRO_TOL


@pytest.mark.parametrize("name", ["decode1", "decode4", "decode16", "decode_wide1", "decode_wide16", "decode_wide32",
                                  "decode_wide64", "decode_wide128", "decode_nv_wide1", "decode_nv_wide16",
                                  "decode_nv_wide64", "decode_nv_wide128"])
def test_decode_full(name):
    w = WL.WORKLOADS[name]
    x, wt = WL.draw_x(w), WL.draw_w(w)
    say(f"case {name} M {w.M} N {w.N} K {w.K}")
    xq, wq = quantize_both(x, wt, w.block, w.fmt)
    assert_quant_parity(compare_quant(xq, x, w.block, w.fmt), name + " X")
    y = linear_of(xq, wq, w.fmt, torch.float32)
    ref = gemm_reference(x, wt, w.block, w.fmt, np.arange(w.M), np.arange(w.N))
    r = rel_fro(y, ref)
    say(f"{name} rel fro {r:.3e}")
    assert r <= GEMM_REL_FRO_TOL


@pytest.mark.parametrize("name", ["prefill_mx", "prefill_mx_m4096", "prefill_nv", "large"])
def test_full_size_sampled(name):
    w = WL.WORKLOADS[name]
    x, wt = WL.draw_x(w), WL.draw_w(w)
    say(f"case {name} M {w.M} N {w.N} K {w.K} b{w.block} {w.fmt} out {w.out_dtype} (sampled)")
    out_dtype = torch.bfloat16 if w.out_dtype == "bf16" else torch.float32
    xq, wq = quantize_both(x, wt, w.block, w.fmt)
    y = linear_of(xq, wq, w.fmt, out_dtype)
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([[0, w.M - 1], rng.choice(w.M, 48, replace=False)]))
    cols = np.unique(np.concatenate([[0, w.N - 1], rng.choice(w.N, 384, replace=False)]))
    xa = wa = None
    if w.fmt == "nvfp4":
        xa, wa = tensor_amax(x, w.block), tensor_amax(wt, w.block)
    assert_quant_parity(compare_quant(xq, x, w.block, w.fmt, rows=rows, t_amax=xa), name + " X")
    assert_quant_parity(compare_quant(wq, wt, w.block, w.fmt, rows=cols, t_amax=wa), name + " W")
    ref = gemm_reference(x, wt, w.block, w.fmt, rows, cols, xa, wa)
    if out_dtype == torch.bfloat16:
        ref = O.bf16_rne_f64(ref)
    r = rel_fro(y[np.ix_(rows, cols)], ref)
    say(f"{name} sampled rel fro {r:.3e}")
    assert r <= GEMM_REL_FRO_TOL


@pytest.mark.parametrize("M,N,K,block", [(1, 4096, 4096, 32), (4, 300, 512, 128), (16, 4096, 4096, 32),
                                         (7, 77, 2048, 16), (16, 520, 1536, 64), (3, 64, 8192, 128),
                                         (2, 14336, 4096, 32), (5, 12300, 4096, 64), (2, 100, 9216, 32)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_fused_decode_equals_two_calls(M, N, K, block, out_dtype):
    # the one-launch decode step gives the same bits as fp4_rotate_quantize + fp4_linear, and
    # both match the oracle's product of the oracle-quantized operands
    x = WL.draw_normal_bf16((M, K), 1.0, seed=M + K)
    x[:, ::97] = WL.bf16_bits_from_f32(np.full((M, len(range(0, K, 97))), 40.0, np.float32))  # outlier channels
    wt = WL.draw_normal_bf16((N, K), 0.02, seed=N + 1)
    say(f"case fused decode M {M} N {N} K {K} b{block} {out_dtype}")
    wq = B.fp4_quantize_weights(dev_bf16(wt), block, "mxfp4")
    xd = dev_bf16(x)
    xq = B.fp4_rotate_quantize(xd, block, "mxfp4")
    y2 = B.fp4_linear(xq[0], xq[1], wq[0], wq[1], "mxfp4", out_dtype=out_dtype)
    y1 = B.fp4_rotate_quantize_linear(xd, wq[0], wq[1], block, out_dtype=out_dtype)  # may take two launches
    y0 = B.fp4_rotate_quantize_linear(xd, wq[0], wq[1], block, out_dtype=out_dtype, workspace=None)  # one launch
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(y0, y2)
    ref = gemm_reference(x, wt, block, "mxfp4", np.arange(M), np.arange(N))
    if out_dtype == torch.bfloat16:
        ref = O.bf16_rne_f64(ref)
    r = rel_fro(host(y1.float() if out_dtype == torch.bfloat16 else y1).astype(np.float64), ref)
    say(f"fused decode rel fro {r:.3e}")
    assert r <= GEMM_REL_FRO_TOL


@pytest.mark.parametrize("M,N", [(5, 256), (16, 4096)])  # one launch; two launches through the workspace
def test_fused_decode_strided_x(M, N):
    K = 1024
    x = WL.draw_normal_bf16((M, K), 1.0, seed=3)
    wt = WL.draw_normal_bf16((N, K), 0.02, seed=4)
    wide = torch.zeros((M, K + 64), dtype=torch.bfloat16, device="cuda")
    wide[:, :K] = dev_bf16(x)
    wq = B.fp4_quantize_weights(dev_bf16(wt), 32, "mxfp4")
    y1 = B.fp4_rotate_quantize_linear(wide[:, :K], wq[0], wq[1], 32)
    xq = B.fp4_rotate_quantize(dev_bf16(x), 32, "mxfp4")
    y2 = B.fp4_linear(xq[0], xq[1], wq[0], wq[1], "mxfp4")
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
