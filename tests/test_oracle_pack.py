"""Pins of the oracle's packing against what the pages and the layout fix.

Nothing here recomputes the oracle's byte formula: positions come from the
hand-worked golden table, values from the code map and shift of the pages.
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from conftest import read_golden


def _shapes():
    return st.tuples(st.integers(1, 4).map(lambda a: 16 * a),
                     st.integers(1, 3).map(lambda b: 256 * b))


@pytest.mark.parametrize("value,byte", [(-1, 0x00), (0, 0x55), (1, 0xAA)])
def test_constant_matrices(value, byte):
    # code = w + 1 in every 2-bit field: 00 00 00 00, 01 01 01 01, 10 10 10 10
    M, K = 48, 768
    p, bad = oracle.pack(np.full((M, K), value, np.int8), 0.5)
    assert bad == 0
    assert p.size == M * K // 4 + 256
    assert np.all(p[:M * K // 4] == byte)


def test_single_weight_positions():
    M, K = 32, 512
    for m, k, byte, g, plus, minus in read_golden("pack_single.txt"):
        m, k, byte, g = int(m), int(k), int(byte), int(g)
        for v, expect in ((1, int(plus, 16)), (-1, int(minus, 16))):
            w = np.zeros((M, K), np.int8)
            w[m, k] = v
            p, _ = oracle.pack(w, 1.0)
            data = p[:M * K // 4]
            assert data[byte] == expect, (m, k, v)
            others = np.delete(data, byte)
            assert np.all(others == 0x55), (m, k, v)


def test_tail_holds_scale_then_zeros():
    M, K = 16, 256
    for scale, hexbytes in read_golden("pack_tail.txt"):
        p, _ = oracle.pack(np.zeros((M, K), np.int8), float(scale))
        tail = p[M * K // 4:]
        assert tail.size == 256
        assert bytes(tail[:4]).hex(" ") == hexbytes
        assert np.all(tail[4:] == 0)
        assert oracle.scale_of(p, M, K) == np.float32(float(scale))


@settings(max_examples=25, deadline=None)
@given(_shapes(), st.integers(0, 2**31 - 1))
def test_round_trip_lossless(shape, seed):
    # "lossless" packing: unpack(pack(W)) == W for every ternary W
    M, K = shape
    w = np.random.default_rng(seed).integers(-1, 2, (M, K)).astype(np.int8)
    p, bad = oracle.pack(w, 0.25)
    assert bad == 0
    np.testing.assert_array_equal(oracle.unpack(p, M, K), w)


@settings(max_examples=10, deadline=None)
@given(_shapes(), st.integers(0, 2**31 - 1))
def test_no_code_three(shape, seed):
    M, K = shape
    w = np.random.default_rng(seed).integers(-1, 2, (M, K)).astype(np.int8)
    p, _ = oracle.pack(w, 1.0)
    data = p[:M * K // 4]
    for s in (0, 2, 4, 6):
        assert np.all(((data >> s) & 3) != 3)


def test_every_position_is_a_distinct_field():
    # A bijection between the M*K weights and the M*K 2-bit fields: setting
    # one weight to +1 changes exactly one field, and no two weights share it.
    M, K = 16, 256
    seen = set()
    base = oracle.pack(np.zeros((M, K), np.int8), 1.0)[0][:M * K // 4]
    for m in range(M):
        for k in range(0, K, 3):
            w = np.zeros((M, K), np.int8)
            w[m, k] = 1
            d = oracle.pack(w, 1.0)[0][:M * K // 4]
            diff = np.nonzero(d != base)[0]
            assert diff.size == 1
            b = int(diff[0])
            x = int(d[b] ^ base[b])
            assert x in (0xC0, 0x30, 0x0C, 0x03)
            key = (b, x)
            assert key not in seen
            seen.add(key)


def test_tile_is_one_contiguous_kilobyte():
    # A 16 x 256 tile of weights lives in exactly 1024 consecutive bytes,
    # tiles in row-tile-major order.
    M, K = 48, 768
    rng = np.random.default_rng(7)
    base_w = np.zeros((M, K), np.int8)
    base = oracle.pack(base_w, 1.0)[0][:M * K // 4]
    for mt in range(M // 16):
        for q in range(K // 256):
            w = base_w.copy()
            w[16 * mt:16 * mt + 16, 256 * q:256 * q + 256] = rng.integers(
                -1, 2, (16, 256))
            d = oracle.pack(w, 1.0)[0][:M * K // 4]
            changed = np.nonzero(d != base)[0]
            lo = (mt * (K // 256) + q) * 1024
            assert changed.min() >= lo and changed.max() < lo + 1024


def test_invalid_values_clamped_and_counted():
    M, K = 16, 256
    w = np.zeros((M, K), np.int8)
    w[0, 0] = 5
    w[3, 7] = -100
    w[15, 255] = 2
    p, bad = oracle.pack(w, 1.0)
    assert bad == 3
    u = oracle.unpack(p, M, K)
    assert u[0, 0] == 1 and u[3, 7] == -1 and u[15, 255] == 1
    assert np.count_nonzero(u) == 3


def test_shape_rules():
    with pytest.raises(ValueError):
        oracle.pack(np.zeros((15, 256), np.int8), 1.0)
    with pytest.raises(ValueError):
        oracle.pack(np.zeros((16, 200), np.int8), 1.0)
