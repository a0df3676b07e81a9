"""The dK/dV kernel keeps one LDS operand offset per read pattern and derives
the others with an XOR: offset(ks) = offset(0) ^ 32 ks for the row-wise
16-byte reads of step ks, and offset(db) = offset(0) ^ 64 db for the
transpose reads of head-dim block db.  This holds because the tile swizzle
only permutes the chunk bits that the row term of the offset never sets.
The test recomputes every offset from its definition (row-major tile of D
bf16 values, 16-byte chunks XOR-swizzled per row) for all 64 lanes."""
import pytest


def b_swz(D, row):
    """Chunk swizzle of a tile row read both row-wise and by transpose reads."""
    if D == 128:
        return ((row & 3) << 2) | ((row >> 2) & 3)
    return (((row >> 1) & 1) << 2) | ((row >> 2) & 3)


def byte_offset(D, row, col):
    """LDS byte offset of element (row, col) of the swizzled tile."""
    return (row * D + ((col // 8) ^ b_swz(D, row)) * 8 + col % 8) * 2


@pytest.mark.parametrize("D", [64, 128])
def test_swizzle_is_a_permutation_of_each_row(D):
    for row in range(64):
        offs = sorted(byte_offset(D, row, c) for c in range(0, D, 8))
        assert offs == [row * D * 2 + 16 * i for i in range(D // 8)]


@pytest.mark.parametrize("D", [64, 128])
def test_row_wise_offsets_are_one_xor_apart(D):
    for lane in range(64):
        n, h = lane & 31, lane >> 5
        # step ks reads 8 elements of row n at column 16 ks + 8 h
        offs = [byte_offset(D, n, 16 * ks + 8 * h) for ks in range(D // 16)]
        assert all(o == offs[0] ^ (32 * ks) for ks, o in enumerate(offs))


@pytest.mark.parametrize("D", [64, 128])
def test_transpose_offsets_are_one_xor_apart(D):
    for lane in range(64):
        h, gq, r4, c4 = lane >> 5, lane >> 4, (lane >> 2) & 3, lane & 3
        for r in (4 * h + r4, 8 + 4 * h + r4):
            # block db reads 4 elements of row r from column 32 db + 16 (gq & 1) + 4 c4
            offs = [byte_offset(D, r, 32 * db + 16 * (gq & 1) + 4 * c4) for db in range(D // 32)]
            assert all(o == offs[0] ^ (64 * db) for db, o in enumerate(offs))
