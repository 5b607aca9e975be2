"""The library's calls captured in a HIP graph (torch.cuda.graph) replay correctly.

Every kernel the calls launch is an ordinary kernel and none of them uses a memset (the NVFP4
tensor scale is written whole by its reduction kernel), so a captured step can be replayed. Each graph is
replayed several times with eager work on the same buffers in between, and every replay is
compared bit for bit with the eager result.
"""
import numpy as np
import pytest
import torch

from microscaling_fp4_quantized_amd import binding as B
from microscaling_fp4_quantized_amd import workloads as WL
from parity import dev_bf16, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load_library()


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # first-use setup (kernel attributes) happens outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


# 2048 x 12544 plans 256x256 then 256x192 tiles in one launch (on 256 CUs), for both formats
@pytest.mark.parametrize("fmt,block,M,N,K", [("mxfp4", 32, 512, 768, 1024), ("nvfp4", 16, 300, 520, 512),
                                             ("mxfp4", 128, 4, 4096, 4096), ("mxfp4", 32, 2048, 12544, 512),
                                             ("nvfp4", 16, 2048, 12544, 512)])
def test_step_graph_replays_match_eager(fmt, block, M, N, K):
    x = dev_bf16(WL.draw_normal_bf16((M, K), 1.0, seed=M))
    x2 = dev_bf16(WL.draw_normal_bf16((M, K), 2.0, seed=M + 1))
    w = dev_bf16(WL.draw_normal_bf16((N, K), 0.02, seed=N))
    wq = B.fp4_quantize_weights(w, block, fmt)
    g_ = 32 if fmt == "mxfp4" else 16
    xq = (torch.empty((M, K // 2), dtype=torch.uint8, device="cuda"),
          torch.empty((M, K // g_), dtype=torch.uint8, device="cuda"),
          torch.empty((1,), dtype=torch.float32, device="cuda") if fmt == "nvfp4" else None)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def step():
        B.fp4_rotate_quantize(x, block, fmt, out=xq)
        B.fp4_linear(xq[0], xq[1], wq[0], wq[1], fmt, x_ts=xq[2], w_ts=wq[2], out_dtype=torch.bfloat16, out=y)

    step()
    torch.cuda.synchronize()
    ref = (xq[0].clone(), xq[1].clone(), None if xq[2] is None else xq[2].clone(), y.clone())
    g = _capture(step)
    say(f"case graph {fmt} b{block} M {M} N {N} K {K}")
    for rep in range(5):
        # eager work on the same buffers between replays: a different X through the same outputs
        B.fp4_rotate_quantize(x2, block, fmt, out=xq)
        B.fp4_linear(xq[0], xq[1], wq[0], wq[1], fmt, x_ts=xq[2], w_ts=wq[2], out_dtype=torch.bfloat16, out=y)
        torch.cuda.synchronize()
        assert not torch.equal(y, ref[3])
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(xq[0], ref[0]) and torch.equal(xq[1], ref[1]), rep
        if xq[2] is not None:
            assert torch.equal(xq[2], ref[2]), rep
        assert torch.equal(y, ref[3]), rep


def test_fused_decode_graph_replays_match_eager():
    M, N, K = 2, 1024, 2048
    x = dev_bf16(WL.draw_normal_bf16((M, K), 1.0, seed=5))
    x2 = dev_bf16(WL.draw_normal_bf16((M, K), 1.0, seed=6))
    wq = B.fp4_quantize_weights(dev_bf16(WL.draw_normal_bf16((N, K), 0.02, seed=7)), 32, "mxfp4")
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    B.fp4_rotate_quantize_linear(x, wq[0], wq[1], 32, out=y)
    torch.cuda.synchronize()
    ref = y.clone()
    g = _capture(lambda: B.fp4_rotate_quantize_linear(x, wq[0], wq[1], 32, out=y))
    for rep in range(5):
        B.fp4_rotate_quantize_linear(x2, wq[0], wq[1], 32, out=y)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), rep
