"""The C-ABI library loads and exports every symbol include/fp4.h declares, and
argument validation rejects bad calls before anything touches the GPU."""
import ctypes
import os
import re
import subprocess

import pytest

from microscaling_fp4_quantized_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4.h")


def declared_symbols():
    with open(HEADER) as f:
        text = f.read()
    return re.findall(r"FP4_API\s+[\w\s\*]+?\b(fp4_\w+)\s*\(", text)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.library_path()):
        pytest.skip("libfp4.so not built")
    return binding.load_library()


def test_header_declares_the_three_calls():
    syms = declared_symbols()
    for s in ("fp4_rotate_quantize", "fp4_quantize_weights", "fp4_linear", "fp4_last_error"):
        assert s in syms


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for s in declared_symbols():
        assert s in exported, s
        assert hasattr(lib, s)
    # nothing else with C linkage leaks out
    assert {s for s in exported if s.startswith("fp4_")} == set(declared_symbols())
    assert lib.fp4_abi_version() == 130


A16 = 0x10000  # a 16-byte aligned fake address: never dereferenced, validation fails first


def q(lib, X=A16, M=4, K=64, ldx=64, block=32, fmt=0, codes=A16, scales=A16, ts=None):
    return lib.fp4_rotate_quantize(X, M, K, ldx, block, fmt, codes, scales, ts, None)


def test_rotate_quantize_validation(lib):
    assert q(lib, fmt=2, X=None) == -4
    assert q(lib, block=8) == -3
    assert q(lib, block=256) == -3
    assert q(lib, X=None) == -1
    assert q(lib, codes=None) == -1
    assert q(lib, fmt=1, ts=None) == -1            # NVFP4 needs the tensor-scale buffer
    assert q(lib, fmt=0, ts=A16, X=None) == -1
    assert q(lib, ts=A16) == -1                    # MXFP4 forbids it
    assert q(lib, M=0, X=None, codes=None) == -1   # pointer checks come first
    assert q(lib, M=0) == -2
    assert q(lib, K=48, block=16) == -2            # K % 32
    assert q(lib, K=96, block=64) == -2            # K % block
    assert q(lib, ldx=32) == -2
    assert q(lib, X=A16 + 2) == -5
    assert q(lib, ldx=68) == -5
    assert q(lib, codes=A16 + 8) == -5
    assert q(lib, fmt=1, ts=A16, scales=A16 + 1) == -5
    assert b"multiple of 32" in lib.fp4_last_error() or lib.fp4_last_error()
    assert lib.fp4_quantize_weights(None, 4, 64, 64, 32, 0, A16, A16, None, None) == -1
    assert b"fp4_quantize_weights" in lib.fp4_last_error()


def qx(lib, rule=0, signs=None, fmt=0, ts=None, X=A16, M=4, K=64, ldx=64, block=32, codes=A16, scales=A16):
    return lib.fp4_rotate_quantize_ex(X, M, K, ldx, block, fmt, rule, signs, codes, scales, ts, None)


def test_rotate_quantize_ex_validation(lib):
    assert qx(lib, rule=4) == -4
    assert qx(lib, rule=-1) == -4
    assert qx(lib, rule=1, fmt=1, ts=A16) == -4    # the OCP floor rule is MXFP4 only
    assert qx(lib, rule=2, fmt=1, ts=A16) == -4    # so is OAS
    assert qx(lib, rule=3, signs=A16 + 8) == -5    # signs 16-byte aligned
    assert qx(lib, rule=0x10) == -4                # a given tensor scale is NVFP4 only
    assert qx(lib, rule=0x11, fmt=1, ts=A16) == -4  # OCP floor stays MXFP4 only with the flag
    assert qx(lib, rule=0x20) == -4                # unknown flag
    assert qx(lib, rule=0, X=None) == -1           # the checks shared with fp4_rotate_quantize come first
    assert qx(lib, rule=9, block=8) == -3
    assert b"fp4_rotate_quantize_ex" in lib.fp4_last_error()
    assert lib.fp4_quantize_weights_ex(None, 4, 64, 64, 32, 0, 3, None, A16, A16, None, None) == -1
    assert b"fp4_quantize_weights_ex" in lib.fp4_last_error()


def test_size_limits(lib):
    # rows * K / 32 must fit in 31 bits (chunk indices); rejected before anything is launched
    assert q(lib, M=1 << 26, K=1024, ldx=1024) == -2
    assert q(lib, M=(1 << 26) - 1, K=1024, ldx=1 << 41) == -2   # leading dimension out of range
    # rows * K / 32 beyond 64 bits must not wrap around into an accepted size
    assert q(lib, M=(1 << 40) + 1, K=1 << 30, ldx=1 << 30) == -2
    assert q(lib, M=(1 << 62), K=1 << 12, ldx=1 << 12) == -2
    assert lib.fp4_linear(A16, A16, None, A16, A16, None, 1 << 31, 4, 128, 0, A16, 0, None) == -2
    assert lib.fp4_linear(A16, A16, None, A16, A16, None, 4, 1 << 31, 128, 0, A16, 0, None) == -2


def fused(lib, X=A16, M=4, K=512, ldx=512, block=32, Wq=A16, Ws=A16, N=64, Y=A16, ydt=0, ws=None, wsb=0):
    return lib.fp4_rotate_quantize_linear(X, M, K, ldx, block, Wq, Ws, N, Y, ydt, ws, wsb, None)


def test_fused_decode_validation(lib):
    assert fused(lib, block=8) == -3
    assert fused(lib, ydt=2) == -4
    assert fused(lib, Ws=None) == -1
    assert fused(lib, M=17) == -2                      # a few tokens only
    assert fused(lib, M=0) == -2
    assert fused(lib, K=640, ldx=640) == -2            # K % 512
    assert fused(lib, M=16, K=1 << 15, ldx=1 << 15) == -2   # too large for on-chip memory
    assert fused(lib, ldx=256) == -2
    assert fused(lib, X=A16 + 2) == -5
    assert fused(lib, Y=A16 + 4) == -5
    assert fused(lib, Ws=A16 + 4) == -5                # 16 scale bytes are read at once
    assert b"fp4_rotate_quantize_linear" in lib.fp4_last_error()
    # workspace: FP4_LINEAR_WORKSPACE_BYTES(4, 512) = 1024 codes + 64 scale bytes
    assert binding.linear_workspace_bytes(4, 512) == 1088
    assert binding.linear_workspace_bytes(3, 512) == 768 + 48
    assert fused(lib, ws=A16, wsb=1087) == -2
    assert b"workspace" in lib.fp4_last_error()
    assert fused(lib, ws=A16 + 8, wsb=4096) == -5


def fused_na(lib, X=A16, M=4, K=512, ldx=512, block=32, Wq=A16, Ws=A16, N=64, Y=A16, ydt=0):
    return lib.fp4_rotate_quantize_linear_noalloc(X, M, K, ldx, block, Wq, Ws, N, Y, ydt, None)


def test_noalloc_decode_validation(lib):
    # the same argument checks as the workspace call, before anything is launched
    assert fused_na(lib, block=8) == -3
    assert fused_na(lib, ydt=2) == -4
    assert fused_na(lib, X=None) == -1
    assert fused_na(lib, M=17) == -2
    assert fused_na(lib, K=640, ldx=640) == -2
    assert fused_na(lib, M=16, K=1 << 15, ldx=1 << 15) == -2
    assert fused_na(lib, Y=A16 + 4) == -5
    assert b"fp4_rotate_quantize_linear_noalloc" in lib.fp4_last_error()
    # every workspace the decode step can need fits the library's array
    for M in (1, 16):
        K = 512
        while M * (K // 2 + 16 + K // 32) <= 160 * 1024:
            assert binding.linear_workspace_bytes(M, K) <= 160 * 1024 + 256
            K += 512


def lin(lib, Xq=A16, Xs=A16, xts=None, Wq=A16, Ws=A16, wts=None, M=4, N=4, K=128, fmt=0, Y=A16, ydt=0):
    return lib.fp4_linear(Xq, Xs, xts, Wq, Ws, wts, M, N, K, fmt, Y, ydt, None)


def test_linear_validation(lib):
    assert lin(lib, fmt=3) == -4
    assert lin(lib, ydt=5) == -4
    assert lin(lib, Y=None) == -1
    assert lin(lib, Ws=None) == -1
    assert lin(lib, fmt=1) == -1                   # NVFP4 needs both tensor scales
    assert lin(lib, fmt=1, xts=A16) == -1
    assert lin(lib, xts=A16) == -1                 # MXFP4 forbids them
    assert lin(lib, K=64) == -2
    assert lin(lib, K=192) == -2
    assert lin(lib, M=0) == -2
    assert lin(lib, Xq=A16 + 4) == -5
    assert lin(lib, Xs=A16 + 2) == -5
    assert lin(lib, Y=A16 + 8) == -5
    assert lin(lib, fmt=1, xts=A16 + 2, wts=A16) == -5   # tensor scales are float words
    assert lin(lib, fmt=1, xts=A16, wts=A16 + 1) == -5
    assert b"fp4_linear" in lib.fp4_last_error()
