"""Pins for the oracle's dense bit-packing (CPU only).

Checked against hand-worked vectors (tests/golden/pack_vectors.json) and an
independent big-integer construction of each row's little-endian bitstream.
"""
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pack_vectors.json")


def _codes(case):
    c = case["codes"]
    if isinstance(c, list):
        return np.array(c, np.uint8)
    if c.startswith("j mod 8"):
        return (np.arange(32) % 8).astype(np.uint8)
    if c.startswith("j mod 4"):
        return (np.arange(16) % 4).astype(np.uint8)
    raise ValueError(c)


def test_hand_worked_vectors(orc):
    cases = json.load(open(GOLDEN))["cases"]
    for case in cases:
        b = case["bits"]
        codes = _codes(case)
        # pad the row to one 128-code group with zeros (zeros add no bits)
        row = np.zeros(128, np.uint8)
        row[: len(codes)] = codes
        words = orc.pack(row[None, :], b)[0]
        want = [int(h, 16) for h in case["words"]]
        assert [int(x) for x in words[: len(want)]] == want, case
        assert (words[len(want):] == 0).all()


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_matches_big_integer_bitstream(orc, bits):
    g = np.random.Generator(np.random.PCG64(bits))
    n, k = 3, 256
    q = g.integers(0, 1 << bits, size=(n, k)).astype(np.uint8)
    words = orc.pack(q, bits)
    assert words.shape == (n, k * bits // 32)
    assert words.nbytes == n * k * bits // 8
    for r in range(n):
        stream = 0
        for j in range(k):
            stream |= int(q[r, j]) << (j * bits)
        want = [(stream >> (32 * i)) & 0xFFFFFFFF for i in range(k * bits // 32)]
        assert [int(x) for x in words[r]] == want


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_unpack_inverts_pack_and_groups_start_at_4b_words(orc, bits):
    g = np.random.Generator(np.random.PCG64(100 + bits))
    n, k = 5, 640
    q = g.integers(0, 1 << bits, size=(n, k)).astype(np.uint8)
    words = orc.pack(q, bits)
    assert (orc.unpack(words, k, bits) == q).all()
    # a change inside group 3 touches only words [4b*3, 4b*4) of its row
    q2 = q.copy()
    q2[1, 3 * 128: 4 * 128] ^= 1
    w2 = orc.pack(q2, bits)
    changed = np.nonzero((w2 != words).any(axis=0))[0]
    assert changed.min() >= 4 * bits * 3 and changed.max() < 4 * bits * 4
    assert (w2[[0, 2, 3, 4]] == words[[0, 2, 3, 4]]).all()


def test_eight_bit_bytes_are_codes(orc):
    g = np.random.Generator(np.random.PCG64(8))
    q = g.integers(0, 256, size=(2, 256)).astype(np.uint8)
    words = orc.pack(q, 8)
    assert (words.view(np.uint8).reshape(2, 256) == q).all()
