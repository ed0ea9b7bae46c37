"""Pins for the oracle's counter-based generator: its Philox4x64-10 blocks
equal numpy's independent implementation of the same published generator
(numpy.random.Philox), element offsets are consistent, and the keep rate
matches ceil(65536 p) / 65536 statistically."""
import numpy as np
import pytest

from oracle import philox as OP


@pytest.mark.parametrize("key", [(0, 0), (123, 456), (2**64 - 1, 2**63 + 5)])
def test_blocks_equal_numpy_philox(key):
    """numpy's Philox advances its counter before each block, so starting it
    at c - 1 yields block c first; the four words come out in order."""
    for start in (0, 1, 2**32 - 1, 2**64 - 9):
        n = 6
        bg = np.random.Philox(counter=np.array([start, 0, 0, 0], dtype=np.uint64),
                              key=np.array(key, dtype=np.uint64))
        raw = bg.random_raw(4 * n).reshape(n, 4)
        ctr = np.zeros((n, 4), dtype=np.uint64)
        ctr[:, 0] = (np.arange(1, n + 1, dtype=np.uint64) + np.uint64(start)) if start < 2**64 - n else \
            np.array([(start + i + 1) % 2**64 for i in range(n)], dtype=np.uint64)
        got = OP.philox4x64_10(ctr, key)
        assert np.array_equal(got, raw), (key, start)


def test_offsets_are_a_window_of_one_stream():
    whole = OP.chunks16(99, 0, 16 * 50 + 7)
    for off, cnt in ((16, 100), (32, 1), (0, 5), (48, 16 * 40 + 7)):
        assert np.array_equal(OP.chunks16(99, off, cnt), whole[off: off + cnt])
    # unaligned start inside a block
    assert np.array_equal(OP.chunks16(99, 5, 30), whole[5:35])


def test_chunk_order_within_a_block():
    w = OP.philox4x64_10(np.array([[3, 0, 0, 0]], dtype=np.uint64), (7, 0))[0]
    ch = OP.chunks16(7, 48, 16)
    for j in range(16):
        assert int(ch[j]) == (int(w[j // 4]) >> (16 * (j % 4))) & 0xFFFF


@pytest.mark.parametrize("p", [0.05, 0.1, 0.5])
def test_keep_rate(p):
    n = 1 << 20
    keep = OP.keep_mask(2024, 0, n, p)
    rate = 1.0 - np.ceil(65536 * np.float32(p)) / 65536
    se = np.sqrt(rate * (1 - rate) / n)
    assert abs(keep.mean() - rate) <= 5 * se


def test_p_zero_keeps_everything():
    assert OP.keep_mask(1, 0, 4096, 0.0).all()
