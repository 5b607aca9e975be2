"""The allocation-free decode step gives the bits of the workspace call.

fp4_rotate_quantize_linear_noalloc is called through the C ABI (ctypes, raw device pointers) on
shapes where the decode step takes two launches, so the library's per-GPU array stands in for
the workspace, twice in a row, the second time with a smaller input; each result must equal that
of fp4_rotate_quantize_linear with a caller-allocated workspace bit for bit.
"""
import ctypes

import numpy as np
import pytest
import torch

from microscaling_fp4_quantized_amd import binding as B
from microscaling_fp4_quantized_amd import workloads as WL
from parity import dev_bf16, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return B.load_library()


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def test_noalloc_equals_workspace_call_twice(lib):
    for M, N, K, block, seed in ((16, 4096, 4096, 32, 5), (16, 4096, 1024, 64, 6)):
        say(f"case no-alloc decode step M {M} N {N} K {K} b{block}")
        x = dev_bf16(WL.draw_normal_bf16((M, K), 1.0, seed=seed))
        wq, ws, _ = B.fp4_quantize_weights(dev_bf16(WL.draw_normal_bf16((N, K), 0.02, seed=seed + 10)), block, "mxfp4")
        work = torch.empty(B.linear_workspace_bytes(M, K), dtype=torch.uint8, device="cuda")
        y_ws = torch.full((M, N), np.nan, dtype=torch.float32, device="cuda")
        y_na = torch.full((M, N), np.nan, dtype=torch.float32, device="cuda")
        st = lib.fp4_rotate_quantize_linear(_p(x), M, K, K, block, _p(wq), _p(ws), N, _p(y_ws), 0, _p(work),
                                            work.numel(), _stream())
        assert st == 0, lib.fp4_last_error()
        st = lib.fp4_rotate_quantize_linear_noalloc(_p(x), M, K, K, block, _p(wq), _p(ws), N, _p(y_na), 0, _stream())
        assert st == 0, lib.fp4_last_error()
        torch.cuda.synchronize()
        assert not torch.isnan(y_na).any()
        assert torch.equal(y_na, y_ws)
        # the same through the two calls, so the workspace call itself is the reference
        xq = B.fp4_rotate_quantize(x, block, "mxfp4")
        assert torch.equal(B.fp4_linear(xq[0], xq[1], wq, ws, "mxfp4"), y_ws)
