"""Pins of the oracle's I2_S layout and to_float: hand-worked bytes, the
page's shift formula element by element, agreement with the independently
written T16Q256 packer where the two layouts coincide, round trips and
bfloat16 rounding worked by hand."""
import numpy as np
import pytest

import oracle
from conftest import read_golden
from oracle import interop as io


@pytest.mark.parametrize("row", read_golden("i2s_examples.txt"), ids=lambda r: r[0])
def test_worked_examples(row):
    name, block, ws, scale, hexbytes = row
    w = np.array([[int(v) for v in ws.split()]], np.int8)
    got = io.i2s_pack(w, float(scale), int(block))
    assert got.tobytes().hex(" ") == hexbytes
    back, s, bad = io.i2s_unpack(got, 1, w.size, int(block))
    assert np.array_equal(back, w) and s == np.float32(float(scale)) and bad == 0


@pytest.mark.parametrize("block", [4, 8, 16, 64, 128, 256])
def test_each_weight_follows_the_shift_formula(block):
    # a single nonzero code at every position j of a block: its byte is
    # j % (block/4) and its value is code << (6 - 2 * group), group j // (block/4)
    q = block // 4
    for j in range(block):
        for v in (-1, 1):
            w = np.zeros((1, 2 * block), np.int8)
            w[0, block + j] = v  # in the second block
            b = io.i2s_pack(w, 1.0, block)[: 2 * block // 4]
            zero = (1 << 6) | (1 << 4) | (1 << 2) | 1  # four code-1 (0) values
            want = np.full(2 * q, zero, np.uint8)
            g, p = j // q, j % q
            want[q + p] = (zero & ~(3 << (6 - 2 * g))) | ((v + 1) << (6 - 2 * g))
            assert np.array_equal(b, want), (block, j, v)


def test_block16_runs_equal_the_t16q256_words():
    # With 16-weight blocks a block's 4 bytes put weight 4g + i at byte i,
    # group g -- the word of 16 columns in the T16Q256 layout, which the
    # C packer writes with its own code.
    rng = np.random.default_rng(3)
    M, K = 32, 512
    w = rng.integers(-1, 2, size=(M, K), dtype=np.int8)
    i2s = io.i2s_pack(w, 1.0, 16)[: M * K // 4].reshape(M, K // 16, 4)
    t16, _ = oracle.pack(w, 1.0)
    for m in (0, 5, 31):
        for k16 in range(K // 16):
            k = 16 * k16
            tile = (m // 16) * (K // 256) + k // 256
            slot = (m % 16) + 16 * ((k % 64) // 16)
            off = tile * 1024 + slot * 16 + 4 * ((k % 256) // 64)
            assert np.array_equal(t16[off: off + 4], i2s[m, k16]), (m, k)


@pytest.mark.parametrize("block", [4, 32, 128, 256])
def test_round_trip_and_invalid_codes(block):
    rng = np.random.default_rng(block)
    M, K = 16, 512
    w = rng.integers(-1, 2, size=(M, K), dtype=np.int8)
    buf = io.i2s_pack(w, 0.0213, block)
    assert buf.size == io.i2s_bytes(M, K)
    back, s, bad = io.i2s_unpack(buf, M, K, block)
    assert np.array_equal(back, w) and s == np.float32(0.0213) and bad == 0
    buf[7] |= 0xC0  # group 0 of byte 7 becomes code 3
    buf[9] = 0xFF   # four code-3 values
    back, _, bad = io.i2s_unpack(buf, M, K, block)
    assert bad == 5
    assert back.max() == 1


def test_bad_blocks():
    w = np.zeros((1, 24), np.int8)
    for block in (0, 6, 16, 48):  # not a multiple of 4, or not dividing 24
        with pytest.raises(ValueError):
            io.i2s_pack(w, 1.0, block)


def test_to_float():
    w = np.array([[-1, 0, 1, 1]], np.int8)
    assert io.to_float(w, 0.75).tolist() == [[-0.75, 0.0, 0.75, 0.75]]
    # bfloat16 keeps 8 significant bits.  1 + 2**-8 is halfway between 1 and
    # 1 + 2**-7: even -> 1 (0x3f80); 1 + 3 * 2**-8 is halfway between
    # 1 + 2**-7 and 1 + 2**-6: even -> 1 + 2**-6 (0x3f82); 1 + 2**-8 + 2**-20
    # is above halfway -> 1 + 2**-7 (0x3f81)
    for s, bits in ((1 + 2.0**-8, 0x3F80), (1 + 3 * 2.0**-8, 0x3F82),
                    (1 + 2.0**-8 + 2.0**-20, 0x3F81)):
        got = io.to_float(w, s, "bf16")[0]
        assert got.tolist() == [bits | 0x8000, 0, bits, bits], (s, got)
