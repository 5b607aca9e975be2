"""CPU oracle of the online MR-GPTQ-style FP4 path.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module. The
product (the HIP library and its Python binding) never does. The oracle and
the HIP path share no code; only the seeded input generators feed both.

It is plain, slow and written to be checked against the pages by eye: NumPy
only, float64 wherever the pages leave the precision open, and float32 where
a float decides an integer result (a code, a scale choice) and the pages fix no
precision: the rotation (R3), the NVFP4 element step (R6) and scale fitting
(R14) take that decision in float32, the precision of the rotated values.

Pages (cited by title and section):

* [BRIDGE-de]  "Bridging the Gap Between Promise and Performance for
  Microscaling FP4 Quantization" (gist.science, German),
  "Technische Zusammenfassung": §1 Problemstellung; §2 Methodik und Analyse
  ("Theoretische Analyse der Fehler", "Einführung von MR-GPTQ",
  "GPU-Kernel-Unterstützung (QuTLASS)").
* [BRIDGE-en]  the same paper on chatpaper.ai, English abstract.
* [BRIDGE-es]  the same paper (gist.science, Spanish), "Resumen técnico":
  §2 Metodología (A. Análisis de Error, B. MR-GPTQ, C. QuTLASS).
* [UNVEIL-nl]  "Unveiling the Potential of Quantization with MXFP4:
  Strategies for Quantization Error Reduction" (gist.science, Dutch),
  "Technische samenvatting": Probleemstelling; Methodologie
  (1. Overflow-Aware Scaling).
* [TORQ-de]    "TORQ: Two-Level Orthogonal Rotation for MXFP4 Quantization"
  (gist.science, German), "Technische Zusammenfassung": 1. Problemstellung.

What the method computes, step by step (the online path):

1. widen bf16 X to float32 (exact);
2. rotate each row by a block-diagonal Hadamard matrix, blocks of ``b``
   along K, applied to weights and activations alike ([BRIDGE-de] §2
   "Einführung von MR-GPTQ", item 1; [BRIDGE-es] §2.B item 1);
3. per group of 32 (MXFP4) or 16 (NVFP4) elements take the absolute maximum
   and derive the shared scale ([BRIDGE-de] §1; [UNVEIL-nl] Probleemstelling);
4. round every element to nearest onto the E2M1 grid (RTN, [BRIDGE-de] §2
   "Theoretische Analyse der Fehler"; E2M1 codebook [TORQ-de] 1.);
5. pack two 4-bit codes per byte;
6. multiply the dequantized operands: Y = dq(Xq) dq(Wq)^T ([BRIDGE-de] §2
   "GPU-Kernel-Unterstützung (QuTLASS)", 4-bit matmul).

Readings taken where the pages are silent:

R1  Blocks and groups are contiguous and aligned from k = 0; the Hadamard
    block b and the scale group g are independent (b in {16,32,64,128}).
R2  The Hadamard matrix is the plain Sylvester one, H[i,j] = (-1)^popcount(i&j),
    normalised by 1/sqrt(b) so that the rotation is orthogonal.
R3  The rotation is computed in float32 as the fast Walsh-Hadamard transform in
    ascending stride order (h = 1, 2, 4, ..., b/2; pair (i, i+h) with bit h of i
    clear -> (x_i + x_{i+h}, x_i - x_{i+h})), then one float32 multiply by
    c_b = fl32(1/sqrt(b)). Fixing this order makes the float32 result unique.
R4  MXFP4 scale: the smallest power of two 2^e with alpha_max <= 6 * 2^e, so
    that the block maximum lands in (3, 6] ([UNVEIL-nl] Methodologie, 1. OAS,
    which describes this mapping as the standard MXFP4 one). E8M0 code e + 127,
    e clamped to [-127, 127]; an all-zero group gets code 0.
R5  NVFP4 tensor scale s_t = fl32(T / (6 * 448)) with T the absolute maximum of
    the whole rotated tensor, recomputed on every call ([BRIDGE-es] §2.B item 2
    speaks of group and tensor scales). The E4M3 group code is the nearest
    E4M3FN value to alpha_max / (6 s_t) (ties to even, saturating at 448),
    decided exactly. s_t == 0 makes the whole tensor zero.
R6  NVFP4 element step. The pages give no precision for dividing an element by its
    two scales, and here a float decides an integer code, so one float32 sequence is
    fixed, in the precision of the rotated values (R3) and of the float32 tensor scale
    (R5): the group's dequantization scale is the float32 number S = fl32(d * s_t)
    (the two stored scales multiplied once), and a per-group scale is applied to the
    group's elements through its float32 reciprocal, R = fl32(1 / S), u = fl32(y * R).
    Three roundings separate u from the exact quotient y / (d s_t) (relative distance
    below 2^-22), so the code differs from the one the exact quotient gives only for
    elements that near_boundary_flags marks (a test checks this against the exact
    quotient). A group with S < 2^-126 (including d == 0) is all signed zeros.
R7  E2M1 rounding is round-to-nearest, ties to the even code, saturating at
    +-6, keeping the sign of the input (so -0 and small negatives give 0x8).
    Codes: bit 3 = sign, bits 2..0 index {0, .5, 1, 1.5, 2, 3, 4, 6}.
R8  Packing: byte j of a row holds element 2j in its low nibble and element
    2j+1 in its high nibble; scales are row-major [rows, K/g].
R9  The GEMM reference is the exact product of the dequantized operands,
    formed in float64: Y64 = dq(Xq) @ dq(Wq)^T, no bias.

Variants (each is a flag of the same step; the standard path above is unchanged):

R12 OCP floor rule (MXFP4): e = floor(log2 alpha_max) - 2, so the group maximum lands in
    [4, 8) and elements above 6 saturate. The pages call the (3, 6] mapping standard; this
    is the other common reading of an MX scale and is offered for comparison.
R13 Overflow-aware scaling (MXFP4, [UNVEIL-nl] Methodologie, 1. OAS): start from the
    standard exponent; when alpha_max / 2^e lies in (3, 3.5] use e - 1, so the maximum
    lands in (6, 7] and saturates to 6 while every smaller element gets twice the
    resolution. "Doubling the scale factor" in the page is read as doubling the scaled
    values, which is what moves (3, 3.5] to (6, 7].
R14 Scale fitting ([BRIDGE-de] §2 "Einführung von MR-GPTQ", item 2: MXFP4 scales fitted to
    the data range, NVFP4 scales optimised for E4M3 precision). The pages give no
    procedure; the reading taken is a data-free per-group search: among the standard
    scale and its two neighbours (MXFP4: e - 1, e + 1; NVFP4: the adjacent E4M3 codes,
    tensor scale unchanged) keep the one with the least squared error of the group.
    The pages give no precision either, and the choice is an integer decided by floats,
    so the error is formed in float32, the precision of the rotated values, summed in
    element order: d_i = fl32(y_i - deq_i), acc = fl32(acc + fl32(d_i * d_i)), with
    deq_i = e2m1 * 2^e (MX, exact) or fl32(e2m1 * S), S = fl32(d * s_t) (NV, as R6).
    Candidates are tried in the order standard, smaller, larger and replace the current
    one only when strictly better. The chosen scale is within float32 rounding of the
    exact least-squares choice (a test checks it with exact rationals). Meant for
    weights (offline), where the extra work is paid once.
R16 Given tensor scale (NVFP4, optional): s_t is supplied by the caller instead of being
    computed from this tensor (a calibrated static activation scale; [BRIDGE-es] §2.B treats
    the tensor scale as a quantity to optimise). Every step after the tensor maximum is the
    same; group maxima above 2688 s_t saturate at E4M3 448 and elements at E2M1 6. s_t = 0
    gives signed zeros, as in the computed case.
R15 Randomized block Hadamard (the QuaRot lineage the pages cite, [BRIDGE-de] §2
    "Theoretische Analyse der Fehler"): each input channel k is multiplied by a sign
    s_k in {+1, -1} before the rotation, i.e. R = D H with D = diag(s). The product is
    unchanged when W is rotated with the same signs.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "E2M1_MAGNITUDES",
    "E4M3_MAX",
    "NV_TENSOR_DIVISOR",
    "widen_bf16",
    "sylvester_hadamard",
    "hadamard_constant",
    "rotate_fwht_f32",
    "rotate_exact_f64",
    "e2m1_rne",
    "e2m1_value",
    "e4m3_value",
    "e4m3_rne_sat",
    "mx_shared_exponent",
    "mx_exponent_ocp_floor",
    "mx_exponent_oas",
    "sse_f32",
    "SCALE_RULES",
    "quantize_mxfp4",
    "quantize_nvfp4",
    "pack_nibbles",
    "unpack_nibbles",
    "rotate_quantize",
    "apply_signs",
    "dequantize",
    "linear_f64",
    "bf16_rne_f64",
    "near_boundary_flags",
]

# E2M1 magnitudes indexed by the 3 low bits of a code ([TORQ-de] 1.: the
# geometrically progressive e2m1 codebook; [UNVEIL-nl] OAS: formal limit 6.0).
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
_E2M1_MIDPOINTS = (E2M1_MAGNITUDES[:-1] + E2M1_MAGNITUDES[1:]) / 2.0  # 7 rounding boundaries

E2M1_MAX = 6.0
E4M3_MAX = 448.0
NV_TENSOR_DIVISOR = E2M1_MAX * E4M3_MAX  # 2688: maps T onto the largest (E4M3 x E2M1) product

MX_GROUP = 32  # [BRIDGE-de] §1: 32 elements share one scale in MXFP4
NV_GROUP = 16  # [BRIDGE-de] §1: 16 elements share one scale in NVFP4


# --------------------------------------------------------------------------
# step 1: bf16 -> float32
# --------------------------------------------------------------------------
def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32, exactly (bf16 is the top half)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
    return (b << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# step 2: block-wise Hadamard rotation ([BRIDGE-de] §2 MR-GPTQ item 1)
# --------------------------------------------------------------------------
def sylvester_hadamard(b: int) -> np.ndarray:
    """H_b[i, j] = (-1)^popcount(i & j) (reading R2), as int64 +-1."""
    if b < 1 or b & (b - 1):
        raise ValueError("Hadamard size must be a power of two")
    i = np.arange(b)
    pc = np.zeros((b, b), dtype=np.int64)
    a = i[:, None] & i[None, :]
    while np.any(a):
        pc += a & 1
        a = a >> 1
    return np.where(pc % 2 == 0, 1, -1).astype(np.int64)


def hadamard_constant(b: int) -> np.float32:
    """c_b = fl32(1/sqrt(b)) (reading R3)."""
    return np.float32(1.0 / np.sqrt(np.float64(b)))


def rotate_fwht_f32(x32: np.ndarray, b: int) -> np.ndarray:
    """Rotate rows by blocks of b along the last axis, in float32 (reading R3).

    x32: float32 [..., K] with K % b == 0. Returns a new float32 array.
    """
    x32 = np.asarray(x32, dtype=np.float32)
    K = x32.shape[-1]
    if K % b:
        raise ValueError("K must be a multiple of the Hadamard block")
    v = np.array(x32, dtype=np.float32, copy=True).reshape(-1, b)
    h = 1
    while h < b:
        w = v.reshape(v.shape[0], b // (2 * h), 2, h)
        lo = w[:, :, 0, :].copy()  # x_i, bit h of i clear
        hi = w[:, :, 1, :].copy()  # x_{i+h}
        w[:, :, 0, :] = lo + hi
        w[:, :, 1, :] = lo - hi
        h *= 2
    v = v * hadamard_constant(b)
    return v.reshape(x32.shape)


def rotate_exact_f64(x: np.ndarray, b: int) -> np.ndarray:
    """The same rotation as a dense product in float64: y = (H_b x) / sqrt(b) per block."""
    x = np.asarray(x, dtype=np.float64)
    H = sylvester_hadamard(b).astype(np.float64)
    v = x.reshape(-1, b) @ H.T / np.sqrt(np.float64(b))
    return v.reshape(x.shape)


# --------------------------------------------------------------------------
# element formats
# --------------------------------------------------------------------------
def e2m1_rne(u: np.ndarray) -> np.ndarray:
    """Round to the nearest E2M1 value, ties to the even code, saturate (reading R7).

    u: float array (the element already divided by its scale). Returns uint8
    codes 0..15 (bit 3 = sign of u).
    """
    u = np.asarray(u, dtype=np.float64)
    mag = np.abs(u)
    i = np.searchsorted(_E2M1_MIDPOINTS, mag, side="left")  # midpoints strictly below mag
    at = np.minimum(i, len(_E2M1_MIDPOINTS) - 1)
    tie = (i < len(_E2M1_MIDPOINTS)) & (mag == _E2M1_MIDPOINTS[at])
    i = np.where(tie & (i % 2 == 1), i + 1, i)
    sign = np.signbit(u).astype(np.int64)
    return (i | (sign << 3)).astype(np.uint8)


def e2m1_value(codes: np.ndarray) -> np.ndarray:
    """Decode E2M1 codes (uint8 0..15) to float64."""
    c = np.asarray(codes, dtype=np.uint8)
    v = E2M1_MAGNITUDES[c & 7]
    return np.where(c & 8, -v, v)


def _e4m3_table() -> np.ndarray:
    """Values of the finite non-negative E4M3FN codes 0x00..0x7E ([UNVEIL-nl]
    Probleemstelling: 4 exponent bits, 3 mantissa bits; bias 7, subnormals,
    no infinity, 0x7F is NaN)."""
    vals = []
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals, dtype=np.float64)


_E4M3_VALUES = _e4m3_table()
_E4M3_MIDPOINTS = (_E4M3_VALUES[:-1] + _E4M3_VALUES[1:]) / 2.0  # exact in float64


def e4m3_value(codes: np.ndarray) -> np.ndarray:
    """Decode non-negative E4M3FN codes 0..126 to float64."""
    c = np.asarray(codes, dtype=np.int64)
    if np.any((c < 0) | (c > 0x7E)):
        raise ValueError("E4M3 scale code out of the non-negative finite range")
    return _E4M3_VALUES[c]


def e4m3_rne_sat(q: np.ndarray) -> np.ndarray:
    """Nearest non-negative E4M3FN code to q >= 0, ties to even, saturating at 448."""
    q = np.asarray(q, dtype=np.float64)
    if np.any(q < 0) or np.any(np.isnan(q)):
        raise ValueError("E4M3 scale input must be a non-negative number")
    i = np.searchsorted(_E4M3_MIDPOINTS, q, side="left")
    at = np.minimum(i, len(_E4M3_MIDPOINTS) - 1)
    tie = (i < len(_E4M3_MIDPOINTS)) & (q == _E4M3_MIDPOINTS[at])
    i = np.where(tie & (i % 2 == 1), i + 1, i)
    return np.minimum(i, 0x7E).astype(np.uint8)


# --------------------------------------------------------------------------
# step 3-4, MXFP4 ([BRIDGE-de] §1: 32 elements, E8M0 power-of-two scale)
# --------------------------------------------------------------------------
def mx_shared_exponent(alpha_max: np.ndarray) -> np.ndarray:
    """e = ceil(log2(alpha_max / 6)), clamped to [-127, 127]; 0 -> -127 (reading R4).

    Written via frexp: alpha_max = f * 2^E with f in [0.5, 1); then
    alpha_max / 2^(E-3) = 8f lies in [4, 6] when f <= 0.75, and
    alpha_max / 2^(E-2) = 4f lies in (3, 4) when f > 0.75.
    """
    a = np.asarray(alpha_max, dtype=np.float64)
    f, E = np.frexp(a)
    e = E.astype(np.int64) - 3 + (f > 0.75)
    e = np.where(a == 0, -127, e)
    return np.clip(e, -127, 127)


SCALE_RULES = ("standard", "ocp_floor", "oas", "fit")


def mx_exponent_ocp_floor(alpha_max: np.ndarray) -> np.ndarray:
    """e = floor(log2 alpha_max) - 2, clamped to [-127, 127]; 0 -> -127 (reading R12).

    With alpha_max = f * 2^E, f in [0.5, 1): floor(log2 alpha_max) = E - 1.
    """
    a = np.asarray(alpha_max, dtype=np.float64)
    f, E = np.frexp(a)
    e = E.astype(np.int64) - 3
    e = np.where(a == 0, -127, e)
    return np.clip(e, -127, 127)


def mx_exponent_oas(alpha_max: np.ndarray) -> np.ndarray:
    """Overflow-aware exponent (reading R13): the standard e, lowered by one when
    alpha_max / 2^e lies in (3, 3.5] ([UNVEIL-nl] Methodologie, 1. OAS)."""
    a = np.asarray(alpha_max, dtype=np.float64)
    e = mx_shared_exponent(a)
    ratio = a * np.ldexp(1.0, -e)  # exact
    lower = (a > 0) & (ratio <= 3.5) & (e > -127)
    return np.where(lower, e - 1, e)


def sse_f32(y: np.ndarray, deq: np.ndarray) -> np.ndarray:
    """Squared error of groups [..., G] in float32, accumulated in element order (reading R14).

    Groups whose errors exceed about 2^64 overflow to +inf for every candidate; no candidate
    is then strictly better and the standard scale stays, as float32 arithmetic dictates."""
    y = np.asarray(y, dtype=np.float32)
    deq = np.asarray(deq, dtype=np.float32)
    acc = np.zeros(y.shape[:-1], dtype=np.float32)
    with np.errstate(over="ignore"):
        for i in range(y.shape[-1]):
            d = (y[..., i] - deq[..., i]).astype(np.float32)
            acc = (acc + (d * d).astype(np.float32)).astype(np.float32)
    return acc


def _mx_codes(grp32: np.ndarray, e: np.ndarray):
    """E2M1 codes of groups [..., 32] under exponent e, and their exact dequantized values."""
    u = grp32.astype(np.float64) * np.ldexp(1.0, -e)[..., None]  # exact
    codes = e2m1_rne(u)
    deq = (e2m1_value(codes) * np.ldexp(1.0, e)[..., None]).astype(np.float32)  # exact
    return codes, deq


def quantize_mxfp4(y32: np.ndarray, rule: str = "standard"):
    """MXFP4 codes and E8M0 scale codes of rotated float32 rows y32 [rows, K]."""
    rows, K = y32.shape
    grp = np.asarray(y32, dtype=np.float32).reshape(rows, K // MX_GROUP, MX_GROUP)
    alpha_max = np.max(np.abs(grp), axis=2)  # exact
    if rule == "standard" or rule == "fit":
        e = mx_shared_exponent(alpha_max)
    elif rule == "ocp_floor":
        e = mx_exponent_ocp_floor(alpha_max)
    elif rule == "oas":
        e = mx_exponent_oas(alpha_max)
    else:
        raise ValueError(rule)
    codes, deq = _mx_codes(grp, e)
    if rule == "fit":
        best = sse_f32(grp, deq)
        for step in (-1, 1):  # tried after the standard exponent: smaller, then larger
            cand = e + step
            valid = (cand >= -127) & (cand <= 127)
            cand = np.clip(cand, -127, 127)
            c_codes, c_deq = _mx_codes(grp, cand)
            c_sse = sse_f32(grp, c_deq)
            better = valid & (c_sse < best)
            e = np.where(better, cand, e)
            best = np.where(better, c_sse, best)
            codes = np.where(better[..., None], c_codes, codes)
    scales = (e + 127).astype(np.uint8)
    return codes.reshape(rows, K), scales


# --------------------------------------------------------------------------
# step 3-4, NVFP4 ([BRIDGE-de] §1: 16 elements; [UNVEIL-nl] E4M3 scale;
# [BRIDGE-es] §2.B: group and tensor scales)
# --------------------------------------------------------------------------
def _nv_codes(grp32: np.ndarray, scales: np.ndarray, s_t: np.float32):
    """E2M1 codes of groups [..., 16] under E4M3 group codes `scales` and tensor scale s_t
    (reading R6), and their dequantized values fl32(e2m1 * S), S = fl32(d * s_t)."""
    d = e4m3_value(scales).astype(np.float32)
    S = (d * s_t).astype(np.float32)
    zero_group = S < np.float32(2.0 ** -126)
    S_safe = np.where(zero_group, np.float32(1.0), S)
    R = (1.0 / S_safe.astype(np.float64)).astype(np.float32)  # = fl32(1/S)
    u = (grp32 * R[..., None]).astype(np.float32)
    codes = e2m1_rne(u)
    codes = np.where(zero_group[..., None], np.signbit(grp32).astype(np.uint8) << 3, codes).astype(np.uint8)
    deq = (e2m1_value(codes).astype(np.float32) * S[..., None]).astype(np.float32)
    return codes, deq


def quantize_nvfp4(y32: np.ndarray, tensor_amax: np.float32 | None = None, rule: str = "standard",
                   tensor_scale=None):
    """NVFP4 codes, E4M3 scale codes and the float32 tensor scale (readings R5, R6; R14 for "fit").

    tensor_amax: the absolute maximum over the whole rotated tensor; computed
    from y32 when None (pass it in when y32 holds only some rows).
    tensor_scale: a given s_t (reading R16); tensor_amax is then not used.
    """
    if rule not in ("standard", "fit"):
        raise ValueError(f"NVFP4 takes the standard or the fit rule, not {rule}")
    rows, K = y32.shape
    y32 = np.asarray(y32, dtype=np.float32)
    if tensor_scale is not None:
        s_t = np.float32(tensor_scale)
        if not (np.isfinite(s_t) and s_t >= 0):
            raise ValueError("a given tensor scale must be finite and non-negative")
    else:
        T = np.float32(np.max(np.abs(y32))) if tensor_amax is None else np.float32(tensor_amax)
        s_t = np.float32(T / np.float32(NV_TENSOR_DIVISOR))  # float32 division, rounded once
    grp = y32.reshape(rows, K // NV_GROUP, NV_GROUP)
    alpha_max = np.max(np.abs(grp), axis=2)
    if s_t == 0:
        scales = np.zeros(alpha_max.shape, dtype=np.uint8)
        codes = (np.signbit(grp).astype(np.uint8) << 3).reshape(rows, K)
        return codes, scales, s_t
    q = alpha_max.astype(np.float64) / (6.0 * np.float64(s_t))  # decided exactly (see R5)
    scales = e4m3_rne_sat(q)
    codes, deq = _nv_codes(grp, scales, s_t)
    if rule == "fit":
        best = sse_f32(grp, deq)
        base = scales.astype(np.int64)
        for step in (-1, 1):  # tried after the standard code: smaller, then larger
            cand = base + step
            valid = (cand >= 0) & (cand <= 0x7E)
            cand = np.clip(cand, 0, 0x7E).astype(np.uint8)
            c_codes, c_deq = _nv_codes(grp, cand, s_t)
            c_sse = sse_f32(grp, c_deq)
            better = valid & (c_sse < best)
            scales = np.where(better, cand, scales).astype(np.uint8)
            best = np.where(better, c_sse, best)
            codes = np.where(better[..., None], c_codes, codes)
    return codes.reshape(rows, K).astype(np.uint8), scales, s_t


# --------------------------------------------------------------------------
# step 5: packing (reading R8)
# --------------------------------------------------------------------------
def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


# --------------------------------------------------------------------------
# the whole online step: rotate + quantize + pack
# --------------------------------------------------------------------------
def apply_signs(x32: np.ndarray, signs) -> np.ndarray:
    """x * s_k per input channel k (reading R15); exact in float32."""
    if signs is None:
        return x32
    s = np.asarray(signs)
    if s.shape != (x32.shape[-1],) or not np.all((s == 1) | (s == -1)):
        raise ValueError("signs must be K values in {+1, -1}")
    return (x32 * s.astype(np.float32)).astype(np.float32)


def rotate_quantize(x_bits: np.ndarray, block: int, fmt: str, tensor_amax=None, rule: str = "standard",
                    signs=None, tensor_scale=None):
    """bf16 X [rows, K] -> (packed codes [rows, K/2], scale codes [rows, K/g], s_t or None).

    rule: "standard" (R4 / R5), "ocp_floor" (R12, MXFP4), "oas" (R13, MXFP4) or "fit" (R14);
    signs: optional K values in {+1, -1} applied before the rotation (R15);
    tensor_scale: NVFP4 only, a given s_t (R16).
    """
    x32 = widen_bf16(x_bits)
    if x32.ndim != 2:
        raise ValueError("X must be 2-D")
    y32 = rotate_fwht_f32(apply_signs(x32, signs), block)
    if fmt == "mxfp4":
        codes, scales = quantize_mxfp4(y32, rule)
        return pack_nibbles(codes), scales, None
    if fmt == "nvfp4":
        codes, scales, s_t = quantize_nvfp4(y32, tensor_amax, rule, tensor_scale)
        return pack_nibbles(codes), scales, s_t
    raise ValueError(fmt)


# --------------------------------------------------------------------------
# step 6: dequantize and multiply (reading R9)
# --------------------------------------------------------------------------
def dequantize(packed: np.ndarray, scales: np.ndarray, fmt: str, s_t=None) -> np.ndarray:
    """Exact float64 values of a quantized tensor [rows, K]."""
    codes = unpack_nibbles(packed)
    rows, K = codes.shape
    vals = e2m1_value(codes)
    if fmt == "mxfp4":
        sc = np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127)
        return (vals.reshape(rows, K // MX_GROUP, MX_GROUP) * sc[..., None]).reshape(rows, K)
    if fmt == "nvfp4":
        sc = e4m3_value(scales) * np.float64(s_t)
        return (vals.reshape(rows, K // NV_GROUP, NV_GROUP) * sc[..., None]).reshape(rows, K)
    raise ValueError(fmt)


def linear_f64(xq, xs, wq, ws, fmt: str, x_ts=None, w_ts=None) -> np.ndarray:
    """Y64 = dq(Xq) @ dq(Wq)^T in float64 ([BRIDGE-de] §2 QuTLASS: the 4-bit matmul)."""
    a = dequantize(xq, xs, fmt, x_ts)
    b = dequantize(wq, ws, fmt, w_ts)
    return a @ b.T


def bf16_rne_f64(y: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 (nearest, ties to even, one rounding), returned as
    float64. Values beyond the largest finite bfloat16 are outside its domain.

    Used only to form the reference of a bf16-output GEMM: the output dtype
    fixes the reference.
    """
    y = np.asarray(y, dtype=np.float64)
    _, e = np.frexp(y)  # |y| in [2^(e-1), 2^e): bf16 keeps 8 significant bits, so the step is 2^(e-8)
    e = np.maximum(e, -125)  # below 2^-126 bf16 is subnormal: a fixed step of 2^-133
    q = np.ldexp(1.0, e - 8)
    return np.round(y / q) * q  # y / q and the product are exact; np.round rounds half to even


# --------------------------------------------------------------------------
# parity support: elements and groups next to a rounding boundary
# --------------------------------------------------------------------------
def near_boundary_flags(y32: np.ndarray, scales: np.ndarray, fmt: str, s_t=None, rel=1e-6):
    """Elements whose float32 rotated value lies within ``rel`` (relative) of a rounding
    boundary of its quantization.

    * Element boundary: |y| = t * S for an E2M1 midpoint t (0.25, 0.75, ... 5), with S the
      group's dequantization scale in float64 (2^e for MXFP4, d * s_t for NVFP4). A group
      whose scale is zero stores signed zeros and has no element boundary.
    * Group boundary (flags every element of the group): the group maximum within ``rel``
      of 6 * 2^k for an integer k (MXFP4: the shared exponent steps there), or alpha_max /
      (6 s_t) within ``rel`` of a midpoint between two adjacent E4M3 values (NVFP4: the
      group code changes there).

    Returns a bool array [rows, K]. The parity tests count differences at flagged
    elements apart from the others: the others must be zero, and the exact tests (inputs
    whose rotation is exact, or the fixed float32 order on both sides) require zero
    differences of both kinds.
    """
    rows, K = y32.shape
    g = MX_GROUP if fmt == "mxfp4" else NV_GROUP
    grp = np.abs(np.asarray(y32, dtype=np.float64)).reshape(rows, K // g, g)
    if fmt == "mxfp4":
        scale = np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127)
    else:
        scale = e4m3_value(scales) * np.float64(s_t)
    flags = np.zeros(grp.shape, dtype=bool)
    live = (scale > 0)[..., None]
    for t in _E2M1_MIDPOINTS:
        bnd = t * scale[..., None]
        flags |= live & (np.abs(grp - bnd) <= rel * bnd)
    amax = grp.max(axis=2)
    if fmt == "mxfp4":
        # exponent thresholds alpha_max = 6 * 2^k, k the nearest integer to log2(alpha_max / 6)
        with np.errstate(divide="ignore"):
            k = np.round(np.log2(np.where(amax > 0, amax, 1.0) / 6.0))
        thr = 6.0 * np.ldexp(1.0, k.astype(np.int64))
        gflag = (amax > 0) & (np.abs(amax - thr) <= rel * thr)
    else:
        if s_t == 0:
            gflag = np.zeros(amax.shape, dtype=bool)
        else:
            q = amax / (6.0 * np.float64(s_t))
            j = np.clip(np.searchsorted(_E4M3_MIDPOINTS, q), 0, len(_E4M3_MIDPOINTS) - 1)
            gflag = np.zeros(amax.shape, dtype=bool)
            for jj in (j - 1, j):  # the midpoints just below and just above q
                m = _E4M3_MIDPOINTS[np.clip(jj, 0, len(_E4M3_MIDPOINTS) - 1)]
                gflag |= np.abs(q - m) <= rel * m
    flags |= gflag[..., None]
    return flags.reshape(rows, K)
