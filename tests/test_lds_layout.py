"""CPU checks of the direct-to-LDS kernel's LDS layouts (no GPU).

The kernel (gemm_f32_mfma_dma in gemm_f32.hip) chooses, through each lane's
global offset, which element a buffer-load-to-LDS deposits in which LDS slot,
and reads MFMA fragments back with its own address formulas.  These tests
restate both maps and check that every fragment read returns exactly the
element the MFMA operand pairing asks for, and that each layout is a
permutation.  Freedom from bank conflicts is a hardware property: the chunk
swizzles were chosen by measuring SQ_LDS_BANK_CONFLICT on MI355X (zero
conflict cycles for both), not from a bank model.
"""
import pytest

def swz_a(r, BK=16):
    return (r >> 2) & 3 if BK == 16 else (r ^ (r >> 3)) & 7 if BK == 32 else r & 15


def a_store(BM, BK=16):
    """LDS slot (row, float index) -> global (row, k) for one A panel."""
    m = {}
    for f in range(BM * BK):
        r, e = divmod(f, BK)
        m[(r, e)] = (r, 4 * ((e // 4) ^ swz_a(r, BK)) + e % 4)
    return m


def b_store(BN, BK=16):
    """LDS slot (k, column) -> global (k, column) for one B panel."""
    if BN == 32:      # 32-wide panels: slot row p holds B row p ^ (bit 2 of p)
        return {(p, c): (p ^ ((p >> 2) & 1), c) for p in range(BK) for c in range(BN)}
    return {(k, c): (k, c ^ (((k >> 2) & 1) * 32)) for k in range(BK) for c in range(BN)}


@pytest.mark.parametrize("BK", [16, 32, 64])
@pytest.mark.parametrize("BM,WM", [(256, 2), (256, 4), (128, 2), (128, 4), (64, 2), (32, 1)])
def test_a_fragments_read_the_paired_k(BM, WM, BK):
    store = a_store(BM, BK)
    for wm in range(WM):
        for lane in range(64):
            li, lh = lane % 32, lane // 32
            for i in range(BM // WM // 32):
                row = wm * (BM // WM) + 32 * i + li
                for q in range(BK // 8):
                    for s in range(4):
                        slot = 4 * ((2 * q + lh) ^ swz_a(row, BK)) + s
                        assert store[(row, slot)] == (row, 8 * q + 4 * lh + s)


@pytest.mark.parametrize("BK", [16, 32, 64])
@pytest.mark.parametrize("BN,WN", [(256, 4), (256, 2), (128, 2), (128, 4), (64, 2)])
def test_b_fragments_read_the_paired_k(BN, WN, BK):
    store = b_store(BN, BK)
    wave_n = BN // WN
    for wn in range(WN):
        for lane in range(64):
            li, lh = lane % 32, lane // 32
            for j in range(wave_n // 32):
                base = wave_n * wn + 32 * j
                col = (base ^ (32 * lh)) + li
                for q in range(BK // 8):
                    for s in range(4):
                        k = 8 * q + 4 * lh + s
                        assert store[(k, col)] == (k, base + li)


def test_layouts_are_permutations():
    for r in range(256):
        assert sorted(c ^ swz_a(r, 16) for c in range(4)) == [0, 1, 2, 3]
        assert sorted(c ^ swz_a(r, 32) for c in range(8)) == list(range(8))
        assert sorted(c ^ swz_a(r, 64) for c in range(16)) == list(range(16))
    for BN in (64, 128, 256):
        for k in range(64):
            assert sorted(c ^ (((k >> 2) & 1) * 32) for c in range(BN)) == list(range(BN))


@pytest.mark.parametrize("BK", [16, 32, 64])
def test_narrow_b_fragments_read_the_paired_k(BK):
    """32-wide B panels: lane half lh reads logical row 8q + 4*lh + s from
    slot row 8q + 4*lh + (s ^ lh), column li."""
    store = b_store(32, BK)
    for lane in range(64):
        li, lh = lane % 32, lane // 32
        for q in range(BK // 8):
            for s in range(4):
                slot_row = 8 * q + 4 * lh + (s ^ lh)
                assert store[(slot_row, li)] == (8 * q + 4 * lh + s, li)
    # a permutation of the panel's rows, and the two halves of every read
    # land in different 32-float halves of a 64-float bank window
    assert sorted(p ^ ((p >> 2) & 1) for p in range(BK)) == list(range(BK))
    for q in range(BK // 8):
        for s in range(4):
            rows = [8 * q + 4 * lh + (s ^ lh) for lh in (0, 1)]
            assert (rows[0] * 32 // 32) % 2 != (rows[1] * 32 // 32) % 2
