"""CPU checks of the direct-to-LDS kernel's LDS layouts (no GPU).

The kernel (gemm_f32_mfma_dma in gemm_f32.hip) chooses, through each lane's
global offset, which element a buffer-load-to-LDS deposits in which LDS slot,
and reads MFMA fragments back with its own address formulas.  These tests
restate both maps and check that (1) every fragment read returns exactly the
element the MFMA operand pairing asks for, and (2) fragment reads are free of
bank conflicts under either plausible LDS organisation (32 banks served 8
lanes per cycle for 128-bit reads, or 64 banks served 16 lanes per cycle).
"""
import pytest

def swz_a(r, BK=16):
    return ((r >> 1) ^ (r >> 3)) & 3 if BK == 16 else (r ^ (r >> 3)) & 7


def a_store(BM, BK=16):
    """LDS slot (row, float index) -> global (row, k) for one A panel."""
    m = {}
    for f in range(BM * BK):
        r, e = divmod(f, BK)
        m[(r, e)] = (r, 4 * ((e // 4) ^ swz_a(r, BK)) + e % 4)
    return m


def b_store(BN, BK=16):
    """LDS slot (k, column) -> global (k, column) for one B panel."""
    return {(k, c): (k, c ^ (((k >> 2) & 1) * 32)) for k in range(BK) for c in range(BN)}


def worst_conflict(byte_addrs, width, banks, group):
    worst = 1
    for g0 in range(0, len(byte_addrs), group):
        use = {}
        for a in byte_addrs[g0:g0 + group]:
            for w in range(width // 4):
                b = (a // 4 + w) % banks
                use[b] = use.get(b, 0) + 1
        worst = max(worst, max(use.values()))
    return worst


@pytest.mark.parametrize("BK", [16, 32])
@pytest.mark.parametrize("BM,WM", [(256, 2), (256, 4), (128, 2), (128, 4), (64, 2)])
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


@pytest.mark.parametrize("BK", [16, 32])
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
    for BN in (64, 128, 256):
        for k in range(32):
            assert sorted(c ^ (((k >> 2) & 1) * 32) for c in range(BN)) == list(range(BN))


@pytest.mark.parametrize("banks,g128,g32", [(32, 8, 32), (64, 16, 64)])
def test_fragment_reads_are_conflict_free(banks, g128, g32):
    for BK in (16, 32):
        for base in range(0, 256, 32):
            for q in range(BK // 8):
                addrs = [(base + l % 32) * 4 * BK + 16 * ((2 * q + l // 32) ^ swz_a(base + l % 32, BK))
                         for l in range(64)]
                assert worst_conflict(addrs, 16, banks, g128) == 1, (BK, base, q)
    for BN in (64, 128, 256):
        for c0 in range(0, BN, 32):
            for s in range(4):
                addrs = [((4 * (l // 32) + s) * BN + ((c0 ^ (32 * (l // 32))) + l % 32)) * 4 for l in range(64)]
                assert worst_conflict(addrs, 4, banks, g32) == 1


def test_unswizzled_a_would_conflict():
    """Without the chunk permutation 32 rows of 64 bytes hit the same banks."""
    addrs = [(l % 32) * 64 + 16 * (l // 32) for l in range(64)]
    assert worst_conflict(addrs, 16, 64, 16) == 4
