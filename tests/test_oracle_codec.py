"""Pins of the oracle's codec (unpack codes / zero points, dequantize).

The oracle is checked against hand-decoded bytes (tests/golden), against an
independent decoder built on ``numpy.unpackbits(bitorder="little")`` and
against the invariants the method fixes (round trip, codes equal to the zero
point dequantize to zero, ragged tails are ignored).
"""
import numpy as np
import pytest

import oracle


def np_decode_fields(byte_rows, bits):
    """Independent decoder: split every byte into bits, least-significant bit
    first, and regroup them into consecutive ``bits``-wide unsigned fields."""
    b = np.unpackbits(np.asarray(byte_rows, np.uint8)[..., None], axis=-1, bitorder="little")
    b = b.reshape(*byte_rows.shape[:-1], -1, bits)
    return (b * (1 << np.arange(bits))).sum(-1).astype(np.int64)


def np_codes(B, K, bits):
    """Codes [N, K]: fields of each row's bytes, blocks laid end to end."""
    N, kb, blob = B.shape
    bs = blob * 8 // bits
    f = np_decode_fields(B.reshape(N, kb * blob), bits)  # [N, kb*bs]
    assert f.shape[1] == kb * bs
    return f[:, :K]


def np_zero_points(zp, N, kb, bits):
    if zp is None:
        return np.full((N, kb), 1 << (bits - 1), np.int64)
    return np_decode_fields(zp, bits)[:, :kb]


def test_golden_code_bytes(golden):
    for bits, byte, *codes in golden("codec_bytes.txt"):
        bits, byte, codes = int(bits), int(byte, 16), [int(c) for c in codes]
        bs = 16
        blob = bs * bits // 8
        B = np.zeros((1, 1, blob), np.uint8)
        B[0, 0, 0] = byte
        got = oracle.unpack_codes(B, 1, bs, bs, bits)[0, :len(codes)]
        assert list(got) == codes, (bits, hex(byte))


def test_golden_zero_point_bytes(golden):
    for bits, byte, *zps in golden("zero_point_bytes.txt"):
        bits, byte, zps = int(bits), int(byte, 16), [int(c) for c in zps]
        kb = len(zps)
        zp = np.zeros((1, -(-kb * bits // 8)), np.uint8)
        zp[0, 0] = byte
        got = oracle.unpack_zero_points(zp, 1, kb, bits)[0]
        assert list(got) == zps, (bits, hex(byte))


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_default_zero_point(bits):
    got = oracle.unpack_zero_points(None, 3, 5, bits)
    assert (got == (1 << (bits - 1))).all()


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("bs", [16, 32, 128])
def test_roundtrip_pack_unpack(bits, bs):
    rng = np.random.default_rng(bits * 1000 + bs)
    N, kb = 5, 4
    K = kb * bs
    B = rng.integers(0, 256, size=(N, kb, bs * bits // 8), dtype=np.uint8)
    codes = oracle.unpack_codes(B, N, K, bs, bits)
    assert (oracle.pack_codes(codes, bs, bits) == B).all()
    zp = rng.integers(0, 256, size=(N, kb * bits // 8), dtype=np.uint8)
    zps = oracle.unpack_zero_points(zp, N, kb, bits)
    assert (oracle.pack_zero_points(zps, bits) == zp).all()


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("K,bs", [(16, 16), (33, 16), (100, 32), (256, 64), (70, 128)])
def test_codes_match_independent_decoder(bits, K, bs):
    rng = np.random.default_rng(K * 7 + bits)
    N = 6
    kb = -(-K // bs)
    B = rng.integers(0, 256, size=(N, kb, bs * bits // 8), dtype=np.uint8)
    zp = rng.integers(0, 256, size=(N, -(-kb * bits // 8)), dtype=np.uint8)
    assert (oracle.unpack_codes(B, N, K, bs, bits) == np_codes(B, K, bits)).all()
    assert (oracle.unpack_zero_points(zp, N, kb, bits) == np_zero_points(zp, N, kb, bits)).all()


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_ragged_tail_is_ignored(bits):
    """Bits past K in the last block never reach a code or a weight."""
    rng = np.random.default_rng(bits)
    N, K, bs = 4, 45, 32
    kb = 2
    B = rng.integers(0, 256, size=(N, kb, bs * bits // 8), dtype=np.uint8)
    B2 = B.copy()
    tail_bit = (K - bs) * bits            # first unused bit of the last block
    B2[:, 1, (tail_bit + 7) // 8:] ^= 0xFF
    if tail_bit % 8:
        B2[:, 1, tail_bit // 8] ^= np.uint8((0xFF << (tail_bit % 8)) & 0xFF)
    s = rng.uniform(0.5, 1.0, size=(N, kb))
    assert (oracle.unpack_codes(B, N, K, bs, bits) == oracle.unpack_codes(B2, N, K, bs, bits)).all()
    assert (oracle.dequantize(B, s, None, N, K, bs, bits) ==
            oracle.dequantize(B2, s, None, N, K, bs, bits)).all()


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_codes_equal_zero_point_dequantize_to_zero(bits):
    rng = np.random.default_rng(11 + bits)
    N, K, bs = 7, 96, 32
    kb = 3
    zps = rng.integers(0, 1 << bits, size=(N, kb), dtype=np.uint8)
    codes = np.repeat(zps, bs, axis=1)[:, :K]
    B = oracle.pack_codes(codes, bs, bits)
    zp = oracle.pack_zero_points(zps, bits)
    W = oracle.dequantize(B, rng.uniform(0.1, 2.0, (N, kb)), zp, N, K, bs, bits)
    assert (W == 0).all()
    # Without zero points, codes equal to 2^(bits-1) do the same.
    B0 = oracle.pack_codes(np.full((N, K), 1 << (bits - 1), np.uint8), bs, bits)
    assert (oracle.dequantize(B0, np.ones((N, kb)), None, N, K, bs, bits) == 0).all()


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_dequantize_matches_independent_formula(bits):
    rng = np.random.default_rng(21 + bits)
    N, K, bs = 5, 80, 16
    kb = 5
    B = rng.integers(0, 256, size=(N, kb, bs * bits // 8), dtype=np.uint8)
    zp = rng.integers(0, 256, size=(N, -(-kb * bits // 8)), dtype=np.uint8)
    s = rng.uniform(-1, 1, size=(N, kb))
    expect = (np_codes(B, K, bits) - np.repeat(np_zero_points(zp, N, kb, bits), bs, 1)[:, :K]) \
        * np.repeat(s, bs, 1)[:, :K]
    assert np.array_equal(oracle.dequantize(B, s, zp, N, K, bs, bits), expect)
