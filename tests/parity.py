"""Parity helpers: compare the HIP path's outputs with the CPU oracle.

Rule (codes and scales): bit equality. Elements whose float32 rotated value lies
within 1e-6 (relative) of a rounding boundary are counted and reported; a
difference there is reported as "flagged", anywhere else as "unflagged". The
tolerance of the method's statement allows flagged differences; since the kernels
and the oracle take every float decision in the same float32 sequence, the tests
demand zero differences of either kind (exact=True, the default), and a flagged
difference would fail them too.
GEMM rule: relative Frobenius error <= 1e-3 against the float64 product of the
oracle's dequantized operands (for bf16 output: against that product rounded to
bf16).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import fp4_oracle as O

GEMM_REL_FRO_TOL = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def tensor_amax(x_bits: np.ndarray, block: int, chunk_rows: int = 2048, signs=None) -> np.float32:
    """max |rotated x| over the whole tensor (oracle rotation), in row chunks."""
    m = np.float32(0)
    for r in range(0, x_bits.shape[0], chunk_rows):
        y = O.rotate_fwht_f32(O.apply_signs(O.widen_bf16(x_bits[r:r + chunk_rows]), signs), block)
        m = max(m, np.float32(np.max(np.abs(y))))
    return np.float32(m)


def compare_quant(gpu, x_bits: np.ndarray, block: int, fmt: str, rows=None, t_amax=None, rule="standard",
                  signs=None, tensor_scale=None):
    """gpu = (codes, scales, ts) torch tensors for all rows; rows = sampled row indices.

    rule / signs: the quantizer variant both sides ran (the flags below are those of the
    standard rule; the variant tests demand zero mismatches of either kind)."""
    g_codes, g_scales, g_ts = gpu
    if rows is None:
        rows = np.arange(x_bits.shape[0])
    xr = x_bits[rows]
    if fmt == "nvfp4" and t_amax is None and tensor_scale is None:
        t_amax = tensor_amax(x_bits, block, signs=signs)
    o_packed, o_scales, o_ts = O.rotate_quantize(xr, block, fmt, tensor_amax=t_amax, rule=rule, signs=signs,
                                                 tensor_scale=tensor_scale)
    gc = host(g_codes)[rows]
    gs = host(g_scales)[rows]
    y32 = O.rotate_fwht_f32(O.apply_signs(O.widen_bf16(xr), signs), block)
    flags = O.near_boundary_flags(y32, o_scales, fmt, o_ts)
    oc, gcu = O.unpack_nibbles(o_packed), O.unpack_nibbles(gc)
    diff = oc != gcu
    g = 32 if fmt == "mxfp4" else 16
    sdiff = o_scales != gs
    gflags = flags.reshape(flags.shape[0], -1, g).any(axis=2)
    res = {
        "elements": int(oc.size),
        "flagged": int(flags.sum()),
        "code_mismatch_flagged": int((diff & flags).sum()),
        "code_mismatch_unflagged": int((diff & ~flags).sum()),
        "scale_mismatch_flagged": int((sdiff & gflags).sum()),
        "scale_mismatch_unflagged": int((sdiff & ~gflags).sum()),
    }
    if fmt == "nvfp4":
        gts = np.float32(host(g_ts)[0])
        res["tensor_scale_equal"] = bool(gts == np.float32(o_ts))
        res["tensor_scale"] = float(gts)
    return res


def assert_quant_parity(res, label="", exact=True):
    say(f"parity {label}: {res}")
    assert res["code_mismatch_unflagged"] == 0, res
    assert res["scale_mismatch_unflagged"] == 0, res
    if exact:
        assert res["code_mismatch_flagged"] == 0 and res["scale_mismatch_flagged"] == 0, res
    if "tensor_scale_equal" in res:
        assert res["tensor_scale_equal"], res


def rel_fro(y: np.ndarray, ref: np.ndarray) -> float:
    y = np.asarray(y, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(y - ref) / (den if den > 0 else 1.0))


def gemm_reference(x_bits, w_bits, block, fmt, xrows, wrows, x_amax=None, w_amax=None, x_rule="standard",
                   w_rule="standard", signs=None):
    """Oracle Y64[xrows][:, wrows] from oracle-quantized operands (never the GPU's)."""
    xq, xs, xt = O.rotate_quantize(x_bits[xrows], block, fmt, tensor_amax=x_amax, rule=x_rule, signs=signs)
    wq, ws, wt = O.rotate_quantize(w_bits[wrows], block, fmt, tensor_amax=w_amax, rule=w_rule, signs=signs)
    return O.linear_f64(xq, xs, wq, ws, fmt, xt, wt)
