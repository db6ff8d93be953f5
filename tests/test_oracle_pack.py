"""Pins of the oracle's prepacked-B layout against positions worked out by
hand from its definition (slot p of block (R, t) holds row 16R + p/4, bytes
64t + 16((p mod 4) XOR ((p/16) mod 4)) .. +15), and against the properties
a packing must have: every byte of B lands exactly once, padding rows are
zero, and the packing read backwards (an independent gather) gives B back.
A slip -- a transposed row/chunk index, a missing XOR, the XOR on the wrong
bits, blocks ordered by stage first -- moves one of the hand-checked bytes."""
import numpy as np
import pytest


@pytest.fixture(scope="module")
def orc():
    import oracle
    return oracle


def _distinct(N, row):
    # every 16-byte piece tagged by (row, piece) so any misplacement shows
    B = np.zeros((N, row), np.uint8)
    for r in range(N):
        for c in range(row // 16):
            B[r, 16 * c:16 * c + 16] = (np.arange(16) + 7 * r + 13 * c) % 256
    return B


def test_hand_worked_positions(orc):
    N, row = 40, 256              # 3 groups (the last one 8 rows short), 4 blocks per group
    B = _distinct(N, row)
    Bp = orc.pack_b(B)
    assert Bp.size == 48 * 256
    piece = lambda i: Bp[16 * i:16 * i + 16]           # 16-byte slot i of the whole pack
    # block (0, 0): slot 0 -> row 0 chunk 0; slot 1 -> row 0 chunk 1; slot 3 -> row 0 chunk 3
    assert np.array_equal(piece(0), B[0, 0:16])
    assert np.array_equal(piece(1), B[0, 16:32])
    assert np.array_equal(piece(3), B[0, 48:64])
    # slot 4 -> row 1 chunk 0; slot 16 -> row 4, chunk 0 ^ 1 = 1; slot 17 -> row 4 chunk 0
    assert np.array_equal(piece(4), B[1, 0:16])
    assert np.array_equal(piece(16), B[4, 16:32])
    assert np.array_equal(piece(17), B[4, 0:16])
    # slot 35 -> row 8, chunk 3 ^ 2 = 1; slot 63 -> row 15, chunk 3 ^ 3 = 0
    assert np.array_equal(piece(35), B[8, 16:32])
    assert np.array_equal(piece(63), B[15, 0:16])
    # block (0, 1) is the next 1 KB: bytes 64..127 of rows 0..15; slot 64 + 18 -> row 4, chunk 2 ^ 1 = 3
    assert np.array_equal(piece(64), B[0, 64:80])
    assert np.array_equal(piece(64 + 18), B[4, 64 + 48:64 + 64])
    # group 1 starts after 4 blocks: slot 256 -> row 16 chunk 0; block (1, 3) slot 5 -> row 17, chunk 1
    assert np.array_equal(piece(256), B[16, 0:16])
    assert np.array_equal(piece(256 + 3 * 64 + 5), B[17, 192 + 16:192 + 32])
    # group 2 holds rows 32..39 and 8 rows of zeros (slots 32..63 of each block)
    g2 = Bp[2 * 4 * 1024:].reshape(4, 64, 16)
    assert (g2[:, 32:, :] == 0).all()
    assert np.array_equal(g2[0, 0], B[32, 0:16])


@pytest.mark.parametrize("N,row", [(1, 64), (16, 64), (17, 128), (256, 512), (300, 1024)])
def test_every_byte_once(orc, N, row):
    rng = np.random.default_rng(N + row)
    B = rng.integers(0, 256, (N, row), dtype=np.uint8)
    Bp = orc.pack_b(B)
    G = (N + 15) // 16
    assert Bp.size == G * 16 * row
    # undo the packing by the definition read backwards (a gather, not the oracle's loop)
    nst = row // 64
    p = np.arange(64)
    rows = p // 4
    chunks = (p % 4) ^ ((p // 16) % 4)
    blocks = Bp.reshape(G, nst, 64, 16)
    U = np.zeros((G * 16, row), np.uint8)
    for t in range(nst):
        U.reshape(G, 16, row)[:, rows[:, None], 64 * t + 16 * chunks[:, None] + np.arange(16)] = blocks[:, t]
    assert np.array_equal(U[:N], B)
    assert (U[N:] == 0).all()


# ------------------------------------------ e2m1 B under e4m3 A (32-byte rows)

def test_b32_hand_worked_positions(orc):
    """Slot p of block (R, t) holds row 32R + p/2, bytes 32t + 16((p mod 2)
    XOR ((p/16) mod 2)) .. +15."""
    N, row = 40, 128             # 2 groups (the second 24 rows short), 4 blocks per group
    B = _distinct(N, row)
    Bp = orc.pack_b32(B)
    assert Bp.size == 64 * 128
    piece = lambda i: Bp[16 * i:16 * i + 16]
    # block (0, 0): slot 0 -> row 0 chunk 0, slot 1 -> row 0 chunk 1, slot 2 -> row 1 chunk 0
    assert np.array_equal(piece(0), B[0, 0:16])
    assert np.array_equal(piece(1), B[0, 16:32])
    assert np.array_equal(piece(2), B[1, 0:16])
    # slot 16 -> row 8, chunk 0 ^ 1 = 1; slot 17 -> row 8 chunk 0; slot 33 -> row 16, chunk 1 ^ 0 = 1
    assert np.array_equal(piece(16), B[8, 16:32])
    assert np.array_equal(piece(17), B[8, 0:16])
    assert np.array_equal(piece(33), B[16, 16:32])
    # slot 63 -> row 31, chunk 1 ^ 1 = 0
    assert np.array_equal(piece(63), B[31, 0:16])
    # block (0, 2): bytes 64..95; slot 128 + 18 -> row 9, chunk 0 ^ 1 = 1 -> bytes 80..95
    assert np.array_equal(piece(128 + 18), B[9, 80:96])
    # group 1 after 4 blocks: slot 256 -> row 32 chunk 0; rows 40..63 are zeros (slots 16..63 of its blocks)
    assert np.array_equal(piece(256), B[32, 0:16])
    g1 = Bp[4 * 1024:].reshape(4, 64, 16)
    assert (g1[:, 16:, :] == 0).all()


@pytest.mark.parametrize("N,row", [(1, 32), (32, 32), (33, 64), (300, 256), (257, 1024)])
def test_b32_every_byte_once(orc, N, row):
    rng = np.random.default_rng(N * 3 + row)
    B = rng.integers(0, 256, (N, row), dtype=np.uint8)
    Bp = orc.pack_b32(B)
    G = (N + 31) // 32
    assert Bp.size == G * 32 * row
    nst = row // 32
    p = np.arange(64)
    rows = p // 2
    chunks = (p % 2) ^ ((p // 16) % 2)
    blocks = Bp.reshape(G, nst, 64, 16)
    U = np.zeros((G * 32, row), np.uint8)
    for t in range(nst):
        U.reshape(G, 32, row)[:, rows[:, None], 32 * t + 16 * chunks[:, None] + np.arange(16)] = blocks[:, t]
    assert np.array_equal(U[:N], B)
    assert (U[N:] == 0).all()
