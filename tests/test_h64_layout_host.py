"""Host-side check of the index arithmetic of the 4096-point transform that
runs on the matrix cores (h64_slice in tern_kernels.hip).

The kernel relies on three facts, each checked here on the CPU against
scipy.linalg.hadamard and the FP64 oracle, for every lane and operand slot:
- the 4096-point Sylvester matrix is the Kronecker square of the 64-point
  one, so a block viewed as a 64 x 64 matrix X transforms as H64 X H64;
- the +-1 operands that the kernel builds from lane bits (parity formulas,
  restated below in the kernel's own terms) equal the Hadamard entries at
  the rows and columns those operand slots stand for;
- contracting the second product in the order in which the first leaves
  Z in the lanes still covers every row of Z exactly once.

The MFMA (v_mfma_f32_16x16x32_bf16) lane layout used throughout: A operand
lane l holds row l & 15, k-slots 8 (l >> 4) + 0..7; B operand lane l holds
column l & 15, the same k-slots; the result lane l holds column l & 15,
rows 4 (l >> 4) + 0..3.  No GPU is used.
"""
import numpy as np
import scipy.linalg

import synth

H64 = scipy.linalg.hadamard(64).astype(np.int64)


def popc(v):
    return bin(v).count("1")


def h_first_b(jt, c, g, ks, e):
    """Sign bit of the B operand of the first product, slot e of lane
    (c, g), step ks, slice jt (kernel: pm1(...) ^ flip)."""
    pb = (g & 1) & (c >> 3)
    base = (popc(e & c & 7) & 1) ^ pb
    flip = (((g >> 1) & jt) ^ (ks & (jt >> 1))) & 1
    return base ^ flip


def h_second_a(ot, st, c, g, e):
    """Sign bit of the A operand of the second product, slot e of lane
    (c, g), step st, row tile ot (kernel: hbase ^ fa / fb)."""
    pl = popc((c >> 2) & g) & 1
    q = [0, c & 1, (c >> 1) & 1, popc(c & 3) & 1][e & 3]
    fa = (ot >> 1) & st
    fb = fa ^ (ot & 1)
    return q ^ pl ^ (fb if e >= 4 else fa)


def second_row(st, g, e):
    """Row of Z that k-slot e of lane group g stands for at step st."""
    return 32 * st + 16 * (e >> 2) + 4 * g + (e & 3)


def test_kronecker_square_matches_oracle(oracle_lib):
    x = synth.activations_f32(41, 1, 4096)[0].astype(np.float64)
    X = x.reshape(64, 64)
    sandwich = (H64 @ X @ H64).reshape(-1) / 64.0
    ref = oracle_lib.fwht(x[None, :], None, 4096)[0]
    assert np.allclose(sandwich, ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_first_product_operand_signs():
    # B[k][col] = H64[32 ks + k][16 jt + col] for every slot of every lane
    for jt in range(4):
        for ks in range(2):
            for lane in range(64):
                c, g = lane & 15, lane >> 4
                for e in range(8):
                    row, col = 32 * ks + 8 * g + e, 16 * jt + c
                    want = 1 if H64[row, col] < 0 else 0
                    assert h_first_b(jt, c, g, ks, e) == want, (jt, ks, lane, e)


def test_second_product_operand_signs_and_order():
    # the k-slots of one step cover 32 distinct rows of Z, the two steps all 64
    seen = set()
    for st in range(2):
        rows = {second_row(st, g, e) for g in range(4) for e in range(8)}
        assert len(rows) == 32
        seen |= rows
    assert seen == set(range(64))
    # a result lane (column c, rows 4 g + r of tile it) holds exactly the Z
    # values the B operand slots of the second product ask for
    for st in range(2):
        for g in range(4):
            for e in range(8):
                it, r = 2 * st + (e >> 2), e & 3
                assert 16 * it + 4 * g + r == second_row(st, g, e)
    # A[row][k] = H64[16 ot + row][second_row(k)]
    for ot in range(4):
        for st in range(2):
            for lane in range(64):
                c, g = lane & 15, lane >> 4
                for e in range(8):
                    want = 1 if H64[16 * ot + c, second_row(st, g, e)] < 0 else 0
                    assert h_second_a(ot, st, c, g, e) == want, (ot, st, lane, e)


def test_lane_level_emulation_matches_oracle(oracle_lib):
    """Both products assembled slot by slot from the formulas above, with
    the MFMA semantics C[row][col] += sum_k A[row][k] B[k][col]."""
    x = synth.activations_f32(43, 1, 4096)[0].astype(np.float64)
    X = x.reshape(64, 64)
    out = np.zeros((64, 64))
    for jt in range(4):
        # first product: Z[:, 16 jt + 0..15] tile by tile
        Z = np.zeros((64, 16))
        for it in range(4):
            for ks in range(2):
                A = X[16 * it:16 * it + 16, 32 * ks:32 * ks + 32]
                B = np.zeros((32, 16))
                for lane in range(64):
                    c, g = lane & 15, lane >> 4
                    for e in range(8):
                        B[8 * g + e, c] = -1.0 if h_first_b(jt, c, g, ks, e) else 1.0
                Z[16 * it:16 * it + 16] += A @ B
        # second product in the permuted contraction order
        for ot in range(4):
            C = np.zeros((16, 16))
            for st in range(2):
                A = np.zeros((16, 32))
                B = np.zeros((32, 16))
                for lane in range(64):
                    c, g = lane & 15, lane >> 4
                    for e in range(8):
                        k = 8 * g + e
                        A[c, k] = -1.0 if h_second_a(ot, st, c, g, e) else 1.0
                        B[k, c] = Z[second_row(st, g, e), c]
                C += A @ B
            out[16 * ot:16 * ot + 16, 16 * jt:16 * jt + 16] = C
    ref = oracle_lib.fwht(x[None, :], None, 4096)[0]
    assert np.allclose(out.reshape(-1) / 64.0, ref, rtol=0, atol=1e-12 * np.abs(ref).max())
