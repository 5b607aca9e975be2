"""Inputs whose block-Hadamard rotation is exact and lands on chosen values.

With block 16 (c = 1/4) and block 64 (c = 1/8) the normalisation is a power of two. For a
block u with at most four non-zero entries, each a multiple of 2^(s-2) no larger than 6 * 2^s,
the input x = H u * c is a bf16 value and every butterfly sum of H x is exact in float32, so
the rotated block is y = u bit for bit. The rows below put rotated values exactly on every
E2M1 midpoint (0.25, 0.75, ..., 5 times the group scale), next to them and on small negative
values, for MXFP4 (scales 2^e) and NVFP4 (group scales d s_t that are powers of two, so the
element step fl32(y * fl32(1/S)) is exact too). build_input checks the exactness it relies on.
"""
import numpy as np

from microscaling_fp4_quantized_amd import workloads as WL
from oracle import fp4_oracle as O

TIES = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)
# the even neighbour of each tie, as an index into {0, .5, 1, 1.5, 2, 3, 4, 6}
TIE_CODE = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}


def bf16_neighbours(v):
    """The bf16 values just below and just above v (v itself a bf16 value, v > 0)."""
    b = int(WL.bf16_bits_from_f32(np.array([v], np.float32))[0])
    assert float(WL.f32_from_bf16_bits(np.array([b], np.uint16))[0]) == v
    return [float(WL.f32_from_bf16_bits(np.array([b + d], np.uint16))[0]) for d in (-1, 1)]


def build_input(rows_of_blocks, block):
    """rows_of_blocks: rows, each a list of blocks, each a list of up to four values placed at
    positions 0, 5, 10, 15 of the block (a dict {pos: value} is taken as it is). Returns the bf16
    bits of X with rotate(X) = U exactly, and U."""
    K = block * len(rows_of_blocks[0])
    U = np.zeros((len(rows_of_blocks), K), np.float64)
    for r, blocks in enumerate(rows_of_blocks):
        assert len(blocks) * block == K
        for j, vals in enumerate(blocks):
            items = vals.items() if isinstance(vals, dict) else zip((0, 5, 10, 15), vals)
            for p, v in items:
                U[r, j * block + p] = v
    H = O.sylvester_hadamard(block).astype(np.float64)
    c = {16: 0.25, 64: 0.125}[block]
    X = (U.reshape(-1, block) @ H.T * c).reshape(U.shape)  # H is symmetric and H H = b I
    x32 = X.astype(np.float32)
    bits = WL.bf16_bits_from_f32(x32)
    assert np.array_equal(WL.f32_from_bf16_bits(bits).astype(np.float64), X), "input not exact in bf16"
    y = O.rotate_fwht_f32(O.widen_bf16(bits), block)
    assert np.array_equal(y.astype(np.float64), U), "rotation not exact"
    return bits, U


def mx_rows(block):
    """MXFP4 rows of eight 32-element groups; each group has a maximum that fixes its scale 2^e
    and probe values. Block 16: a group is two Hadamard blocks, so a maximum can sit alone in
    one block and a probe one bf16 step from a tie alone in the other. Block 64: a block holds
    two groups, each with its maximum and one probe (four values per block)."""
    rows = []
    if block == 16:
        blocks = []
        for e in (-20, -3, 0, 1, 7, 30):
            s = 2.0 ** e
            blocks += [[4 * s, 0.25 * s, -0.75 * s, 1.25 * s], [-1.75 * s, 2.5 * s, -3.5 * s, 5 * s]]
            blocks += [[4 * s, -0.25 * s, 0.75 * s, -1.25 * s], [1.75 * s, -2.5 * s, 3.5 * s, -5 * s]]
            blocks += [[6 * s, -0.125 * s, 5.5 * s], [-0.25 * s, 0.125 * s, -5.5 * s]]
            for t in TIES:
                for v in bf16_neighbours(t):
                    blocks += [[4 * s], [v * s], [-4 * s], [-v * s]]
        blocks += [[], []]  # an all-zero group (scale code 0)
        while len(blocks) % 16:
            blocks.append([])
        return [blocks[i:i + 16] for i in range(0, len(blocks), 16)]
    groups = []
    for e in (-20, -3, 0, 1, 7, 30):
        s = 2.0 ** e
        for t in TIES:
            groups += [[4 * s, t * s], [-4 * s, -t * s], [6 * s, -t * s]]
        groups += [[6 * s, -0.125 * s], [4 * s, -0.25 * s], [4 * s, 5.5 * s]]
    groups.append([])
    while len(groups) % 8:
        groups.append([])
    blocks = []
    for i in range(0, len(groups), 2):
        d = {p: v for p, v in zip((0, 7), groups[i])}
        d.update({32 + p: v for p, v in zip((0, 7), groups[i + 1])})
        blocks.append(d)
    return [blocks[i:i + 4] for i in range(0, len(blocks), 4)]


def nv_rows(k):
    """NVFP4 rows (block 16 = one 16-element group): s_t = 2^k from a tensor maximum of
    2688 * 2^k; groups with maximum 6 d s_t for d = 2^j, so S = d s_t is a power of two."""
    st = 2.0 ** k
    blocks = [[2688 * st]]  # the tensor maximum: code 448, element 6
    for j in (-9, -7, -6, -2, 0, 3, 8):  # 2^-9 and 2^-7 are subnormal E4M3 values
        S = 2.0 ** j * st
        blocks.append([6 * S, 0.25 * S, -0.75 * S, 1.25 * S])
        blocks.append([6 * S, -1.75 * S, 2.5 * S, -3.5 * S])
        blocks.append([-6 * S, 5 * S, -0.25 * S, 0.75 * S])
        blocks.append([6 * S, -0.125 * S, -5 * S, 3.5 * S])
        for t in TIES:
            for dv in (-0.0625, 0.0625):  # the finest offset that keeps every input exact in bf16
                blocks.append([6 * S, (t + dv) * S])
                blocks.append([-6 * S, -(t + dv) * S])
    blocks.append([])  # an all-zero group
    width = 16
    while len(blocks) % width:
        blocks.append([])
    return [blocks[i:i + width] for i in range(0, len(blocks), width)]


# E4M3 rounding midpoints of a / (6 s_t), with the even code each rounds to: between the
# subnormal steps k * 2^-9, within a binade, across a binade (1.875 / 2) and at the top (416 / 448)
E4M3_TIES = ((0.5 * 2.0 ** -9, 0x00), (1.5 * 2.0 ** -9, 0x02), (7.5 * 2.0 ** -9, 0x08), (1.0625, 0x38),
             (1.1875, 0x3A), (1.9375, 0x40), (17.0, 0x58), (432.0, 0x7E))


def nv_e4m3_tie_rows(k):
    """NVFP4 rows (block 16) whose group maxima divided by 6 s_t (s_t = 2^k) lie exactly on
    every kind of E4M3 rounding midpoint, with either sign, and one bf16 step to either side."""
    st = 2.0 ** k
    blocks = [[2688 * st]]
    for m, _ in E4M3_TIES:
        a = 6 * m * st
        for v in [a] + bf16_neighbours(a):
            ulp = 2.0 ** (np.floor(np.log2(v)) - 7)  # one bf16 step at v
            blocks += [[v], [-v], [v, -ulp]]
    width = 16
    while len(blocks) % width:
        blocks.append([])
    return [blocks[i:i + width] for i in range(0, len(blocks), width)]


def check_tie_codes(packed, U, scale_of_group, g):
    """Every element of U exactly at t * scale must carry the even neighbour's code, with the
    sign of the element (hand table, independent of the oracle)."""
    codes = O.unpack_nibbles(np.asarray(packed))
    rows, K = U.shape
    S = np.repeat(scale_of_group, g, axis=1)
    n = 0
    for t, want in TIE_CODE.items():
        at = (np.abs(U) == t * S) & (S > 0)
        for sign in (0, 8):
            sel = at & ((np.signbit(U) * 8) == sign)
            assert np.all(codes[sel] == want | sign), (t, sign, np.unique(codes[sel]))
            n += int(sel.sum())
    small = (np.abs(U) < 0.25 * S) & np.signbit(U)
    assert np.all(codes[small] == 8)  # a negative value rounding to zero keeps its sign
    return n


