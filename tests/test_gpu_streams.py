"""Calls issued on two streams at once give the results of the same calls issued one after another.

Every entry point runs its kernels on the caller's current stream, keeps its temporaries (the
NVFP4 max pass's per-workgroup maxima, the decode step's workspace) in buffers of that call, and
shares nothing between calls except per-device launch settings. So calls on different streams
may overlap on the device in any way and still produce bit-identical outputs. Each case runs
four independent problems serially on the current stream, then three times spread over two
side streams without synchronisation between the calls, and compares every output bit for bit.
(The serial results themselves are checked against the oracle by the parity tests.)
"""
import pytest
import torch

from microscaling_fp4_quantized_amd import binding as B
from parity import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load_library()


def _inputs(seed, M, N, K):
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn(M, K, generator=g) * 2.0).to(torch.bfloat16)
    w = (torch.randn(N, K, generator=g) * 0.05).to(torch.bfloat16)
    return x.cuda(), w.cuda()


def _run(x, w, fmt, block):
    xq, xs, xt = B.fp4_rotate_quantize(x, block, fmt)
    wq, ws, wt = B.fp4_quantize_weights(w, block, fmt)
    y = B.fp4_linear(xq, xs, wq, ws, fmt, x_ts=xt, w_ts=wt, out_dtype=torch.bfloat16)
    outs = [xq, xs, wq, ws, y] + ([xt, wt] if fmt == "nvfp4" else [])
    if fmt == "mxfp4" and x.shape[0] <= 16:  # the fused decode step, both of its launch forms
        outs.append(B.fp4_rotate_quantize_linear(x, wq, ws, block, out_dtype=torch.float32))
        outs.append(B.fp4_rotate_quantize_linear(x, wq, ws, block, out_dtype=torch.float32, workspace=None))
    return outs


# 2048 x 12544 plans 256x256 then 256x192 tiles in one launch (on 256 CUs); 600 x 1300 takes the
# large-tile kernels with ragged edges; M < 256 the general kernels; M = 8 the decode path
CASES = [
    ("mxfp4", 32, 2048, 12544, 512),
    ("mxfp4", 32, 1024, 2048, 1024),
    ("mxfp4", 128, 200, 520, 640),
    ("mxfp4", 32, 8, 4096, 2048),
    ("nvfp4", 16, 2048, 12544, 512),
    ("nvfp4", 16, 600, 1300, 768),
    ("nvfp4", 64, 100, 300, 384),
]


@pytest.mark.parametrize("fmt,block,M,N,K", CASES)
def test_two_streams_match_serial(fmt, block, M, N, K):
    say(f"[streams] {fmt} b{block} M={M} N={N} K={K}")
    ins = [_inputs(100 + i, M, N, K) for i in range(4)]
    serial = [_run(x, w, fmt, block) for x, w in ins]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        for s in streams:
            s.wait_stream(torch.cuda.current_stream())
        par = []
        for i, (x, w) in enumerate(ins):
            with torch.cuda.stream(streams[i % 2]):
                par.append(_run(x, w, fmt, block))
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(serial, par)):
            for j, (ta, tb) in enumerate(zip(a, b)):
                assert torch.equal(ta, tb), f"problem {i}, output {j}, repetition {rep}"
