"""A plain CPU model of the gfx950 scaled MFMA with fp8 (E4M3) operands,
16 rows x 16 columns x 128 K values per instruction (AMD CDNA4 ISA,
V_MFMA_SCALE_F32_16X16X128_F8F6F4), used to pin the scale re-layout from the
consumer's side.  It is written from the instruction's operand order, not
from the re-layout code:

* A operand: lane 16q + i holds row i; its bytes 0..15 are K values
  16q .. 16q+15 and its bytes 16..31 are K values 64+16q .. 64+16q+15.  The B
  operand is the same with columns in place of rows.
* Scale operand: lane 16kb + i supplies, in one 32-bit register, the e8m0
  scale of row i (column i for B) for K values 32kb .. 32kb+31; op_sel picks
  which byte of the register the instruction uses.
* Result: lane l, element r holds C[4 * (l // 16) + r][l % 16].

The GPU consumer test runs the real instruction against this model.
"""
from __future__ import annotations

import numpy as np

import oracle


def hw_k(q: int, j: int) -> int:
    """K index of byte j of a lane in lane group q."""
    return 16 * q + j if j < 16 else 64 + 16 * q + (j - 16)


def mfma_scale_16x16x128(a_regs: np.ndarray, b_regs: np.ndarray, sa_regs: np.ndarray,
                         sb_regs: np.ndarray, op_sel: int) -> np.ndarray:
    """One instruction: a_regs / b_regs (64, 32) fp8 bytes per lane,
    sa_regs / sb_regs (64, 4) scale register bytes per lane.  Returns the
    16 x 16 product in float64 (the hardware accumulates in fp32)."""
    a = np.zeros((16, 128))
    b = np.zeros((16, 128))
    va = oracle.e4m3_decode(a_regs.reshape(-1)).reshape(64, 32)
    vb = oracle.e4m3_decode(b_regs.reshape(-1)).reshape(64, 32)
    for lane in range(64):
        q, i = divmod(lane, 16)
        for j in range(32):
            a[i, hw_k(q, j)] = va[lane, j]
            b[i, hw_k(q, j)] = vb[lane, j]
    for kb in range(4):
        ea = sa_regs[16 * kb:16 * kb + 16, op_sel].astype(np.float64) - 127
        eb = sb_regs[16 * kb:16 * kb + 16, op_sel].astype(np.float64) - 127
        a[:, 32 * kb:32 * kb + 32] *= np.exp2(ea)[:, None]
        b[:, 32 * kb:32 * kb + 32] *= np.exp2(eb)[:, None]
    return a @ b.T


def lane_data(qk: np.ndarray, r0: int, k0: int, end: int) -> np.ndarray:
    """The consumer's data load for one operand: (64, 32) bytes of rows
    r0 .. r0+15 of qk (rows x tokens, e4m3 bytes), K step starting at token
    k0, zero past token ``end`` or past the last row."""
    regs = np.zeros((64, 32), dtype=np.uint8)
    for lane in range(64):
        q, i = divmod(lane, 16)
        r = r0 + i
        if r >= qk.shape[0]:
            continue
        for j in range(32):
            t = k0 + hw_k(q, j)
            if t < end:
                regs[lane, j] = qk[r, t]
    return regs


def lane_scales(tiles: np.ndarray, tile: int) -> np.ndarray:
    """The consumer's scale load: one 4-byte register per lane of a tile."""
    return tiles[tile * 256:(tile + 1) * 256].reshape(64, 4)


def grouped_gemm(qa: np.ndarray, ta: np.ndarray, sa_starts: np.ndarray, qb: np.ndarray,
                 tb: np.ndarray, sb_starts: np.ndarray, offs) -> list[np.ndarray]:
    """Per-group C_g = A_g B_g^T as a wave of the consumer computes it: A is
    (rows, tokens) e4m3 bytes, B is (cols, tokens) e4m3 bytes, ta / tb their
    re-laid-out scales with tile starts.  K steps of 128 tokens, four steps
    per scale tile (op_sel = step mod 4)."""
    rows, cols = qa.shape[0], qb.shape[0]
    RA, RBn = (rows + 15) // 16, (cols + 15) // 16
    out = []
    lo = 0
    for g, hi in enumerate(int(v) for v in offs):
        n = max(hi - lo, 0)
        kt_a = (sa_starts[g + 1] - sa_starts[g]) // max(RA, 1)
        kt_b = (sb_starts[g + 1] - sb_starts[g]) // max(RBn, 1)
        assert kt_a == kt_b == (n + 511) // 512
        c = np.zeros((RA * 16, RBn * 16))
        for ra in range(RA):
            for rb in range(RBn):
                acc = np.zeros((16, 16))
                for step in range((n + 127) // 128):
                    k0 = lo + 128 * step
                    a_regs = lane_data(qa, 16 * ra, k0, hi)
                    b_regs = lane_data(qb, 16 * rb, k0, hi)
                    sa = lane_scales(ta, sa_starts[g] + ra * kt_a + step // 4)
                    sb = lane_scales(tb, sb_starts[g] + rb * kt_b + step // 4)
                    acc += mfma_scale_16x16x128(a_regs, b_regs, sa, sb, step % 4)
                c[16 * ra:16 * ra + 16, 16 * rb:16 * rb + 16] = acc
        out.append(c[:rows, :cols])
        lo = max(lo, hi)
    return out


def dequantized_gemm(qa, sa, qb, sb, offs) -> list[np.ndarray]:
    """The same products from the jagged MX definition: every token's e4m3
    value times 2^(e8m0 - 127) of its block (blocks restart at each group
    start, numbered group after group), summed in float64.  sa is (rows,
    blocks), sb is (cols, blocks)."""
    va = oracle.e4m3_decode(qa.reshape(-1)).reshape(qa.shape)
    vb = oracle.e4m3_decode(qb.reshape(-1)).reshape(qb.shape)
    out = []
    lo, b0 = 0, 0
    for hi in (int(v) for v in offs):
        n = max(hi - lo, 0)
        blk = b0 + np.arange(n) // 32
        ea = np.exp2(sa[:, blk].astype(np.float64) - 127)
        eb = np.exp2(sb[:, blk].astype(np.float64) - 127)
        out.append((va[:, lo:lo + n] * ea) @ (vb[:, lo:lo + n] * eb).T)
        b0 += (n + 31) // 32
        lo = max(lo, hi)
    return out
