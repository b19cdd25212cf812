"""Pins of the cache-management oracle against facts fixed outside it: the E4M3 format's
closed-form codes and round trips, rounding midpoints, saturation; FNV-1a's published test
vectors; and the block-hash chain's defining properties."""

import struct

import numpy as np
import pytest

import oracle
from oracle import cache_management as cm


def q1(x):
    return int(cm.quantize_e4m3(np.float32(x)))


def test_e4m3_closed_form_codes():
    # 1.0 = 2^0: exponent field 7, mantissa 0
    assert q1(1.0) == 0x38
    assert q1(-1.0) == 0xB8
    assert q1(448.0) == 0x7E                       # largest finite: 1.75 * 2^8
    assert q1(2.0 ** -9) == 0x01                   # smallest subnormal
    assert q1(2.0 ** -6) == 0x08                   # smallest normal
    assert q1(0.875 * 2.0 ** -6) == 0x07           # largest subnormal
    assert q1(0.0) == 0x00 and q1(-0.0) == 0x80
    assert q1(1.5) == 0x3C and q1(0.25) == 0x28 and q1(-3.5) == 0xC6


def test_e4m3_ties_go_to_the_even_code():
    assert q1(1.0625) == 0x38                      # between 1.0 (0x38) and 1.125 (0x39)
    assert q1(1.1875) == 0x3A                      # between 1.125 (0x39) and 1.25 (0x3A)
    assert q1(2.0 ** -10) == 0x00                  # half the smallest subnormal
    assert q1(3 * 2.0 ** -10) == 0x02              # between 1 and 2 quanta of 2^-9
    assert q1(-1.0625) == 0xB8


def test_e4m3_saturation_and_nan():
    for x in (448.0, 449.0, 464.0, 500.0, 1e6, np.inf):
        assert q1(x) == 0x7E and q1(-x) == 0xFE
    assert q1(np.nan) & 0x7F == 0x7F


def test_e4m3_round_trip_and_midpoints():
    table = oracle.fp8_e4m3fn_table()
    for c in range(256):
        if c & 0x7F == 0x7F:
            continue
        assert q1(table[c]) == c, hex(c)
    # each midpoint of two neighbouring non-negative codes goes to the even one; just
    # inside the midpoint goes to the nearer one
    for c in range(126):
        lo, hi = table[c], table[c + 1]
        m = (lo + hi) / 2                            # exact in binary32 (5 significant bits)
        assert np.float32(m) == m
        assert q1(m) == (c if c % 2 == 0 else c + 1)
        assert q1(np.nextafter(np.float32(m), np.float32(0))) == c
        assert q1(np.nextafter(np.float32(m), np.float32(1e9))) == c + 1


def test_quantizing_append_uses_the_fp32_quotient():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 2, 16)).astype(np.float32) * 40
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)          # truncated to bf16
    scale = np.array([0.37, 1.9], np.float32)
    pool = np.zeros((4, 2, 8, 16), np.uint8)
    slots = np.array([5, -1, 17])
    out = cm.kv_append_fp8(pool, bits, scale, slots, 8)
    xb = (bits.astype(np.uint32) << 16).view(np.float32)
    for i, slot in ((0, 5), (2, 17)):
        for h in range(2):
            want = [q1(np.float32(v) / scale[h]) for v in xb[i, h]]
            assert out[slot // 8, h, slot % 8].tolist() == want
    assert out.sum() == out[0, :, 5].sum() + out[2, :, 1].sum()  # slot -1 skipped
    # decoding the codes stays within half a quantum (relative 2^-4) of x / scale
    dec = oracle.fp8_e4m3fn_table()[out[0, :, 5]] * scale[:, None]
    assert np.all(np.abs(dec - xb[0]) <= np.abs(xb[0]) / 16 + 2.0 ** -10 * scale[:, None])


def test_copy_blocks():
    pool = np.arange(5 * 2 * 4 * 3, dtype=np.uint16).reshape(5, 2, 4, 3)
    out = cm.copy_blocks(pool, [1, 3, 9], [4, 0, 2])
    assert np.array_equal(out[4], pool[1]) and np.array_equal(out[0], pool[3])
    assert np.array_equal(out[[1, 2, 3]], pool[[1, 2, 3]])     # id 9 out of range: skipped


def test_fnv1a64_published_vectors():
    assert cm.fnv1a64(b"") == 0xCBF29CE484222325
    assert cm.fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert cm.fnv1a64(b"foobar") == 0x85944171F73967E8


def test_block_hash_chain_properties():
    rng = np.random.default_rng(7)
    toks = rng.integers(0, 50000, 70).tolist()
    h = cm.block_hashes(toks, 16)
    assert len(h) == 4                                            # 64 of 70 tokens
    # block 0 by the definition written out with struct
    data = struct.pack("<Q", 0) + struct.pack("<16i", *toks[:16])
    assert h[0] == cm.fnv1a64(data)
    # same prefix -> same hashes; one changed token changes its block and all later ones
    other = list(toks)
    other[40] += 1
    h2 = cm.block_hashes(other, 16)
    assert h2[:2] == h[:2] and all(a != b for a, b in zip(h2[2:], h[2:]))
    # a chain can be continued from the hash of the block before
    assert cm.block_hashes(toks[32:], 16, parent=h[1]) == h[2:]
    assert len(set(h)) == 4
    with pytest.raises(Exception):
        cm.block_hashes(toks, 0)
