"""Pins of the oracle's base-3 packing (64 weights in 13 bytes, layout
B3T1024): hand-worked blocks, exhaustive digit round trips, the byte
position of every weight by an independent formula, whole-matrix round
trips."""
import numpy as np
import pytest

from conftest import read_golden
from oracle import base3 as b3


def _codes(spec: str) -> np.ndarray:
    if spec == "k%3":
        return np.arange(64) % 3
    v, n = spec.split("*")
    return np.full(int(n), int(v))


@pytest.mark.parametrize("row", read_golden("base3_blocks.txt"), ids=lambda r: r[0])
def test_worked_blocks(row):
    name, spec, want = row
    c = _codes(spec)
    got = b3.encode_block(c)
    assert got.tolist() == [int(v) for v in want.split()]
    assert b3.decode_block(got).tolist() == c.tolist()


def test_every_byte_value_round_trips():
    # a byte's five base-3 digits: columns 4j..4j+3 and 48+j of block byte j
    for v in range(243):
        c = np.ones(64, dtype=np.int64)
        c[0], c[1], c[2], c[3], c[48] = v % 3, v // 3 % 3, v // 9 % 3, v // 27 % 3, v // 81
        assert b3.encode_block(c)[0] == v
        assert b3.decode_block(b3.encode_block(c)).tolist() == c.tolist()
    for v in range(81):  # the last byte has four digits
        c = np.ones(64, dtype=np.int64)
        c[60:64] = [v % 3, v // 3 % 3, v // 9 % 3, v // 27 % 3]
        assert b3.encode_block(c)[12] == v


def test_density_is_1_625_bits():
    assert b3.packed_bytes(16, 1024) - 256 == 16 * 1024 * 13 // 64
    assert (b3.packed_bytes(8192, 28672) - 256) * 8 / (8192 * 28672) == 1.625


def test_weight_positions():
    # one weight of +1 in a field of zeros (codes 1): exactly one byte
    # differs from the all-zero encoding, at the offset the layout defines
    M, K = 32, 2048
    base = b3.pack(np.zeros((M, K), np.int8), 1.0)
    rng = np.random.default_rng(4)
    for m, k in [(0, 0), (31, 2047), (5, 48), (17, 1023), (16, 1024), (3, 700)] + \
            [tuple(x) for x in rng.integers(0, [M, K], size=(20, 2))]:
        w = np.zeros((M, K), np.int8)
        w[m, k] = 1
        diff = np.nonzero(b3.pack(w, 1.0) != base)[0]
        # independent formula: tile, lane, byte in the 52-byte run
        tile = (m // 16) * (K // 1024) + k // 1024
        lane = m % 16 + 16 * ((k % 1024) // 256)
        blk, col = (k % 256) // 64, k % 64
        j = col // 4 if col < 48 else (col - 48 if col < 60 else 12)
        if j < 12:   # word 3 blk + j // 4: chunk (3 blk + j // 4) // 4 of the lane
            word = 3 * blk + j // 4
            off = tile * 3328 + 16 * (64 * (word // 4) + lane) + 4 * (word % 4) + j % 4
        else:        # word 12, byte blk
            off = tile * 3328 + 3072 + 4 * lane + blk
        assert diff.tolist() == [off], (m, k)


def test_code_bytes_are_a_partition():
    # every byte of the code region belongs to exactly one lane's block byte
    M, K = 32, 2048
    offs = np.concatenate([np.asarray(o) for _, _, o in b3._lane_runs(M, K)])
    assert np.array_equal(np.sort(offs), np.arange(M * K * 13 // 64))


@pytest.mark.parametrize("M,K", [(16, 1024), (48, 2048), (32, 3072)])
def test_round_trip(M, K):
    rng = np.random.default_rng(M + K)
    w = rng.integers(-1, 2, size=(M, K), dtype=np.int8)
    buf = b3.pack(w, 0.0213)
    assert buf.size == b3.packed_bytes(M, K)
    back, s = b3.unpack(buf, M, K)
    assert np.array_equal(back, w) and s == np.float32(0.0213)
    assert not buf[M * K * 13 // 64 + 4:].any()  # zero tail
    rows = [3, 17, 40]
    part, _ = b3.unpack(buf, M, K, rows=rows) if M > 40 else (w[[]], s)
    if M > 40:
        assert np.array_equal(part, w[rows])


def test_bad_shapes_and_values():
    with pytest.raises(ValueError):
        b3.packed_bytes(16, 512)
    with pytest.raises(ValueError):
        b3.pack(np.full((16, 1024), 2, np.int8), 1.0)
